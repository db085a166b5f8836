"""Calls on several streams at once: each stream has its own workspace, so its calls'
workgroups hand words to one another only inside that workspace.  The results of calls
running concurrently must equal those of the same calls run one at a time.

Workloads: a sampling verification (bf16, aligned rows), a top-k verification (f32,
ragged rows, the one-pass threshold's select and merge launches before k_verify) and the
batched sampler, which shares the second stream's workspace (calls ordered on one stream
may share one).  The serial results are held to the oracle as well.
"""
import numpy as np
import pytest

import oracle
import parity
from rejection_sampling_verify_02_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_02_amd as sv
    sv.load_library()
    return torch.device("cuda:0")


def _verify_inputs(raw, T, k, dev):
    tokens = parity.prepare(raw, T, k)
    return (parity.to_device(raw.target, dev), parity.to_device(raw.draft, dev), parity.to_device(tokens, dev),
            parity.to_device(raw.u_accept, dev), parity.to_device(raw.u_sample, dev)), tokens


def test_concurrent_streams_match_serial(dev):
    import torch
    import rejection_sampling_verify_02_amd as sv

    T1, k1 = 1.0, 0
    raw1 = wl.make_random(24, 4, 50000, "bf16", seed=7101)
    in1, tok1 = _verify_inputs(raw1, T1, k1, dev)
    T2, k2 = 0.8, 40
    raw2 = wl.make_random(16, 3, 70001, "f32", seed=7102)
    in2, tok2 = _verify_inputs(raw2, T2, k2, dev)
    z3, u3 = wl.make_sample(40, 90001, "bf16", seed=7103)
    in3 = (parity.to_device(z3, dev), parity.to_device(u3, dev))

    def v1(ws, stream):
        return sv.spec_verify(*in1, T1, k1, workspace=ws, stream=stream)

    def v2(ws, stream):
        return sv.spec_verify(*in2, T2, k2, workspace=ws, stream=stream)

    def s3(ws, stream):
        return sv.spec_sample(*in3, 0.9, 0, workspace=ws, stream=stream)

    # one at a time on the current stream
    cur = torch.cuda.current_stream(dev)
    ws0 = sv.Workspace()
    ref = [tuple(t.cpu() for t in f(ws0, cur.cuda_stream)) for f in (v1, v2, s3)]
    torch.cuda.synchronize(dev)
    for raw, tok, T, r in ((raw1, tok1, T1, ref[0]), (raw2, tok2, T2, ref[1])):
        k = k1 if raw is raw1 else k2
        acc_r, out_r, diag = oracle.spec_verify_ref(raw.target, raw.draft, tok, raw.u_accept,
                                                    raw.u_sample, T, k, with_diagnostics=True)
        res = parity.compare(tok, raw.V, T, r[0].numpy(), r[1].numpy(), acc_r, out_r, diag)
        assert not res.failures, res.failures[:3]

    # two streams at once, 30 rounds; the second alternates the top-k verification and the
    # sampler in one workspace
    s_a, s_b = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    s_a.wait_stream(cur)
    s_b.wait_stream(cur)
    ws_a, ws_b = sv.Workspace(), sv.Workspace()
    got = []
    for it in range(30):
        with torch.cuda.stream(s_a):
            ga = v1(ws_a, s_a.cuda_stream)
        with torch.cuda.stream(s_b):
            gb = v2(ws_b, s_b.cuda_stream) if it % 2 == 0 else s3(ws_b, s_b.cuda_stream)
        got.append((ga, gb, it % 2))
    torch.cuda.synchronize(dev)
    for it, (ga, gb, odd) in enumerate(got):
        for a, b in zip(ga, ref[0]):
            assert torch.equal(a.cpu(), b), f"stream A, round {it}"
        rb = ref[2] if odd else ref[1]
        for a, b in zip(gb, rb):
            assert torch.equal(a.cpu(), b), f"stream B, round {it} ({'sampler' if odd else 'top-k'})"
    assert np.all(ref[0][0].numpy() >= 0) and np.all(ref[2][1].numpy() == 0)

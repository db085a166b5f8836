"""GPU parity of the per-position overlap ``spec_overlap`` against the oracle's ``overlap``.

All calls go through the C ABI.  Pair statuses must match exactly.  beta and tv must
match the oracle's fp64 values within TOL: the kernels form every term in fp32 from a
once-rounded log2(e)/T and fp64 log-partitions -- the normalisers from one v_exp_f32 per
logit, min(p_v, q_v) as one v_exp_f32 of the smaller of the two exponents, the draft
side's exponent shifted by a per-chunk constant rounded to fp32 once (at most ~7e-7
relative on q_v), and a chunk's tv term as p's chunk mass less the chunk's sum of the
minima, both summed in the same order.  The per-element relative errors (argument
rounding, exp, the temperature rounding seen as a perturbed T) stay below ~1e-6 on the
mass-carrying terms, and the fp32 vector sums add about 1e-6 relative, so both sums are
within ~3e-6 of exact, and TOL = 1e-5 leaves a margin of three.  Where p and q are
bitwise the same the kernels give tv = 0 exactly, and where their supports are disjoint
beta = 0 exactly.
"""
import numpy as np
import pytest

import oracle
from parity import to_device
from rejection_sampling_verify_02_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_02_amd as sv
    sv.load_library()
    return torch.device("cuda:0")


def run_both(target, draft, T, k, dev, label="", ws=None):
    import rejection_sampling_verify_02_amd as sv
    print(f"[overlap] {label} target={target.shape} T={T} k={k}", flush=True)
    beta, tv, st = sv.spec_overlap(to_device(target, dev), to_device(draft, dev), T, k, workspace=ws)
    g_b, g_t, g_s = beta.cpu().numpy(), tv.cpu().numpy(), st.cpu().numpy()
    o_b, o_t, o_s = oracle.overlap(target, draft, T, k)
    np.testing.assert_array_equal(g_s, o_s)
    ok = o_s == 0
    assert np.all(np.isnan(g_b[~ok])) and np.all(np.isnan(g_t[~ok]))
    eb = np.abs(g_b[ok] - o_b[ok]).max(initial=0.0)
    et = np.abs(g_t[ok] - o_t[ok]).max(initial=0.0)
    print(f"[overlap] {label}: pairs={int(ok.sum())} max|dbeta|={eb:.2e} max|dtv|={et:.2e}", flush=True)
    assert eb <= TOL and et <= TOL, (eb, et)
    return g_b, g_t, g_s


def test_overlap_b64_g4_v128256_full_size(dev):
    """B=64, G=4, V=128256 bf16, T=1, in the verification layout (target rows G+1)."""
    raw = wl.make_config(3)
    b, t, _ = run_both(raw.target, raw.draft, 1.0, 0, dev, "zipf_bf16_b64")
    assert 0.2 < float(np.mean(b)) < 0.99


def test_overlap_topk_workload_full_size(dev):
    """B=128, G=6, V=128256 bf16, T=0.8, top-k 50: identical rows, noisy rows and rows whose
    draft support avoids the target's (beta exactly 0)."""
    raw = wl.make_config(5)
    tau = oracle.topk_threshold_rows(raw.target[:, :raw.G], 50)
    zt = wl.bf16_to_f32(raw.target[:, :raw.G])
    wl.apply_disjoint_support(raw, zt >= tau[..., None])
    b, t, _ = run_both(raw.target, raw.draft, 0.8, 50, dev, "topk_stress")
    g1 = raw.B // 3 + (1 if raw.B % 3 else 0)
    assert np.all(t[:g1] == 0.0) and np.all(np.abs(b[:g1] - 1.0) <= TOL)
    assert np.all(b[raw.disjoint_rows] == 0.0)


SHAPES = [
    # B, G, V, dtype, T, k, target rows (G or G+1)
    (3, 2, 20001, "bf16", 1.0, 0, 3),     # odd V: element-wise path
    (5, 3, 32000, "f32", 0.7, 0, 3),      # pairs layout
    (2, 1, 1, "bf16", 1.0, 0, 2),         # a single token: beta 1, tv 0
    (4, 2, 64, "bf16", 1.0, 1, 3),        # top-1: beta 0 or 1
    (2, 2, 50000, "bf16", 0.05, 0, 3),    # very low temperature
    (2, 2, 50000, "bf16", 5.0, 50, 2),    # very high temperature with top-k
    (9, 5, 9003, "f32", 0.8, 7, 6),       # odd V, f32 top-k, lanes with two pairs
    (37, 3, 3000, "bf16", 1.0, 0, 4),     # many short pairs
    (1, 1, 300000, "bf16", 1.0, 0, 2),    # 19 chunks per row
    (2, 3, 152064, "bf16", 1.0, 0, 4),    # the greedy workload's vocabulary
]


@pytest.mark.parametrize("B,G,V,dtype,T,k,TR", SHAPES)
def test_overlap_shapes(dev, B, G, V, dtype, T, k, TR):
    raw = wl.make_random(B, G, V, dtype, seed=B * 131 + V)
    target = raw.target if TR == G + 1 else raw.target[:, :G].copy()
    run_both(target, raw.draft, T, k, dev, f"{B}x{G}x{V}")


def test_overlap_p_equals_q_and_single_token(dev):
    raw = wl.make_random(6, 3, 40000, "bf16", seed=61)
    b, t, _ = run_both(raw.target, raw.target[:, :3].copy(), 1.0, 0, dev, "p=q")
    assert np.all(t == 0.0)
    raw1 = wl.make_random(4, 2, 1, "f32", seed=62)
    b1, t1, _ = run_both(raw1.target, raw1.draft, 1.0, 0, dev, "V=1")
    assert np.all(t1 == 0.0) and np.all(np.abs(b1 - 1.0) <= TOL)


def test_overlap_row_codes(dev):
    raw = wl.make_random(6, 3, 20000, "f32", seed=63)
    t, d = raw.target.copy(), raw.draft.copy()
    t[0, 1, 123] = np.nan
    d[2, 0, 5] = np.inf
    d[3, 2, :] = -np.inf
    t[4, 3, 7] = np.nan  # the trailing target row is not read
    _, _, s = run_both(t, d, 1.0, 0, dev, "row codes")
    assert s[0, 1] == oracle.ERR_ROW and s[2, 0] == oracle.ERR_ROW and s[3, 2] == oracle.ERR_ROW
    assert int(np.sum(s != 0)) == 3


def test_overlap_empty_and_determinism(dev):
    import rejection_sampling_verify_02_amd as sv
    raw = wl.make_random(4, 0, 100, "bf16", seed=64)
    b, t, s = sv.spec_overlap(to_device(raw.target, dev), to_device(raw.draft, dev), 1.0)
    assert b.shape == (4, 0)
    raw = wl.make_random(8, 4, 70000, "bf16", seed=65)
    tt, dd = to_device(raw.target, dev), to_device(raw.draft, dev)
    r1 = [x.cpu().numpy() for x in sv.spec_overlap(tt, dd, 0.9, 20)]
    r2 = [x.cpu().numpy() for x in sv.spec_overlap(tt, dd, 0.9, 20)]
    for a, c in zip(r1, r2):
        np.testing.assert_array_equal(a, c)


def test_overlap_shares_workspace_with_verify(dev):
    """One workspace, alternating calls of both operations and shapes: results equal
    those of calls on fresh workspaces."""
    import rejection_sampling_verify_02_amd as sv
    from parity import prepare
    ws = sv.Workspace()
    raw_a = wl.make_random(16, 4, 30000, "bf16", seed=66)
    raw_b = wl.make_random(3, 2, 130000, "bf16", seed=67)
    tok_a = prepare(raw_a, 1.0, 0)
    ref_a = [x.cpu().numpy() for x in sv.spec_overlap(to_device(raw_a.target, dev), to_device(raw_a.draft, dev),
                                                       1.0, 0, workspace=sv.Workspace())]
    ref_v = [x.cpu().numpy() for x in sv.spec_verify(
        to_device(raw_a.target, dev), to_device(raw_a.draft, dev), to_device(tok_a, dev),
        to_device(raw_a.u_accept, dev), to_device(raw_a.u_sample, dev), 1.0, 0, workspace=sv.Workspace())]
    for rep in range(3):
        got_v = [x.cpu().numpy() for x in sv.spec_verify(
            to_device(raw_a.target, dev), to_device(raw_a.draft, dev), to_device(tok_a, dev),
            to_device(raw_a.u_accept, dev), to_device(raw_a.u_sample, dev), 1.0, 0, workspace=ws)]
        for a, c in zip(got_v, ref_v):
            np.testing.assert_array_equal(a, c)
        run_both(raw_b.target, raw_b.draft, 0.7, 30, dev, f"shared ws {rep}", ws=ws)
        got_a = [x.cpu().numpy() for x in sv.spec_overlap(to_device(raw_a.target, dev),
                                                           to_device(raw_a.draft, dev), 1.0, 0, workspace=ws)]
        for a, c in zip(got_a, ref_a):
            np.testing.assert_array_equal(a, c)

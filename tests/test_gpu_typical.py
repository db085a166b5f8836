"""GPU parity of typical acceptance ``spec_typical_verify`` against the oracle's ``typical_verify``.

All calls go through the C ABI.  Codes must match exactly; accepted lengths and tokens
must match, except for a sequence whose first differing decision the oracle places within
BAND_LOG of its threshold in log space (counted, at most 1% of sequences).  BAND_LOG comes
from the arithmetic.  The kernels form ln p(x) from a once-rounded log2(e)/T and an fp64
log-partition: error ~1e-6 of |z_x * k2| at worst, a few 1e-6 in nats.  The entropy comes
from chunk sums of e and e*t (each vector's terms a pairwise fp32 tree, vectors and chunks
in fp64), so each sum carries ~3 fp32 roundings (~2e-7 relative) on top of one rounding
of each e and t; with |log2 t| + |D| <= ~35 at V = 128256 that is at most ~7e-6 in nats.
2e-5 leaves a margin of about three.  The greedy next token is an integer argmax and must
match exactly.
"""
import numpy as np
import pytest

import oracle
from parity import to_device, prepare
from rejection_sampling_verify_02_amd import workloads as wl

pytestmark = pytest.mark.gpu

BAND_LOG = 2e-5


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_02_amd as sv
    sv.load_library()
    return torch.device("cuda:0")


def run_both(target, tok, T, eps, delta, k, dev, label):
    import torch
    import rejection_sampling_verify_02_amd as sv
    print(f"[typical] {label} target={target.shape} T={T} k={k} eps={eps} delta={delta}", flush=True)
    acc, out = sv.spec_typical_verify(to_device(target, dev), torch.from_numpy(np.ascontiguousarray(tok)).to(dev),
                                      T, eps, delta, k)
    g_acc, g_out = acc.cpu().numpy(), out.cpu().numpy()
    o_acc, o_out, d = oracle.typical_verify(target, tok, T, eps, delta, k, with_diagnostics=True)
    B = len(o_acc)
    exact = boundary = 0
    bad = []
    for b in range(B):
        if o_acc[b] < 0:
            assert g_acc[b] == o_acc[b] and np.all(g_out[b] == -1), (b, g_acc[b], o_acc[b])
            continue
        if g_acc[b] == o_acc[b] and np.array_equal(g_out[b], o_out[b]):
            exact += 1
            continue
        i = int(min(g_acc[b], o_acc[b]))  # the first position where the decisions differ
        if g_acc[b] != o_acc[b] and i < tok.shape[1] and abs(d["margin"][b, i]) < BAND_LOG:
            boundary += 1
        else:
            bad.append((b, int(g_acc[b]), int(o_acc[b]), g_out[b][:6].tolist(), o_out[b][:6].tolist()))
    print(f"[typical] {label}: seqs={B} exact={exact} boundary={boundary} codes={int(np.sum(o_acc < 0))} "
          f"mean accepted={float(np.mean(np.maximum(o_acc, 0))):.2f}", flush=True)
    assert not bad, bad[:4]
    assert boundary <= max(1, B // 100)
    return g_acc, g_out


def test_typical_b64_g4_v128256(dev):
    """B=64, G=4, V=128256 bf16, T=1, drafts drawn from q, eps = 0.1, delta = 0.3."""
    raw = wl.make_config(3)
    x = prepare(raw, 1.0, 0)
    acc, _ = run_both(raw.target, x, 1.0, 0.1, 0.3, 0, dev, "zipf_bf16_b64")
    assert 0.3 < float(np.mean(acc)) < 4.0


SHAPES = [
    # B, G, V, dtype, T, k, eps, delta
    (8, 5, 32000, "f32", 0.7, 0, 0.05, 0.2),
    (16, 4, 20001, "bf16", 1.0, 0, 0.1, 0.3),   # odd V: element-wise path
    (8, 6, 50000, "bf16", 0.05, 0, 0.3, 0.5),   # very low temperature
    (8, 6, 50000, "bf16", 5.0, 50, 0.01, 0.9),  # very high temperature with top-k
    (32, 3, 9003, "f32", 1.0, 7, 0.0, 0.3),     # eps = 0: the support
    (4, 64, 3000, "bf16", 1.0, 0, 0.002, 0.5),  # long drafts
    (3, 70, 3000, "bf16", 1.0, 0, 0.002, 0.5),  # positions past the first 64 (a second round of tests)
    (2, 63, 200000, "bf16", 1.0, 0, 0.1, 0.3),  # 64 rows x 13 chunks: more partials than LDS holds
    (5, 0, 1000, "bf16", 1.0, 0, 0.1, 0.3),     # no drafts: the greedy token
    (3, 2, 1, "f32", 1.0, 0, 0.5, 0.5),         # a single token
]


@pytest.mark.parametrize("B,G,V,dtype,T,k,eps,delta", SHAPES)
def test_typical_shapes(dev, B, G, V, dtype, T, k, eps, delta):
    raw = wl.make_random(B, G, V, dtype, seed=B * 53 + G * 7 + V)
    x = oracle.sample_rows(raw.draft, raw.u_draft, T, k).astype(np.int32) if G else np.zeros((B, 0), np.int32)
    run_both(raw.target, x, T, eps, delta, k, dev, f"{B}x{G}x{V}")


def test_typical_uniform_rows_exact(dev):
    """Uniform rows: p(x) = 1/K and H = ln K; thresholds a factor apart from p(x) (no
    boundary), so the GPU must reproduce the closed-form decisions."""
    V = 4096
    rows = []
    for K in (4, 8, 16, 2):
        z = np.full(V, -np.inf, np.float32)
        z[100:100 + K] = 1.5
        rows.append(z)
    t = np.stack(rows)[None]
    tok = np.array([[101, 105, 110]], np.int32)
    acc, out = run_both(t, tok, 1.0, 0.1, 2.0, 0, dev, "uniform rows")
    assert acc[0] == 2 and list(out[0]) == [101, 105, 100, -1]


def test_typical_near_one_hot_matches_greedy(dev):
    """At T = 1e-3 the rule reduces to greedy verification: the same results as spec_verify
    at T = 0 on the GPU."""
    import torch
    import rejection_sampling_verify_02_amd as sv
    raw = wl.make_random(48, 5, 30000, "bf16", seed=111)
    x = oracle.argmax_rows(raw.target[:, :5]).astype(np.int32)
    x[::2, 1] = (x[::2, 1] + 5) % 30000
    x[1::3, 3] = (x[1::3, 3] + 1) % 30000
    acc_t, out_t = run_both(raw.target, x, 1e-3, 0.4, 0.4, 0, dev, "near one-hot")
    acc_g, out_g = sv.spec_verify(to_device(raw.target, dev), None, torch.from_numpy(x).to(dev), None, None, 0.0)
    np.testing.assert_array_equal(acc_t, acc_g.cpu().numpy())
    np.testing.assert_array_equal(out_t, out_g.cpu().numpy())


def test_typical_codes(dev):
    raw = wl.make_random(8, 4, 5000, "f32", seed=112)
    t = raw.target.copy()
    x = oracle.sample_rows(raw.draft, raw.u_draft, 1.0).astype(np.int32)
    x[1, 2] = 5000         # -1
    t[2, 3, 7] = np.nan    # -3
    t[3, 4, 0] = np.inf    # -3 (the row of the next token)
    t[4, 0, :] = -np.inf   # -3 (nothing finite)
    t[5, 4, 4321] = np.nan  # -3 (the row of the next token, whose sums are not formed)
    t[6, 4, :] = -np.inf   # -3 (nothing finite in the row of the next token)
    g_acc, _ = run_both(t, x, 1.0, 0.1, 0.3, 0, dev, "codes")
    assert list(g_acc[1:7]) == [oracle.ERR_TOKEN, oracle.ERR_ROW, oracle.ERR_ROW, oracle.ERR_ROW,
                                oracle.ERR_ROW, oracle.ERR_ROW]
    assert g_acc[0] >= 0 and g_acc[7] >= 0

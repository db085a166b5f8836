"""The C-ABI library loads, exports every declared symbol, and validates host
arguments without touching a GPU (every status below is decided before any HIP call)."""
import ctypes
import re
from pathlib import Path

import pytest

import rejection_sampling_verify_02_amd as sv

ROOT = Path(__file__).resolve().parents[1]
HEADERS = sorted((ROOT / "include").glob("*.h"))


@pytest.fixture(scope="module")
def lib():
    if not sv.LIB_PATH.exists():
        from rejection_sampling_verify_02_amd import build
        build.build()
    return sv.load_library()


def declared_functions():
    text = "\n".join(h.read_text() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


def test_header_declares_expected_entry_points():
    assert set(declared_functions()) == set(sv.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = __import__("subprocess").run(["nm", "-D", "--defined-only", str(sv.LIB_PATH)],
                                      capture_output=True, text=True, check=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", nm, re.M), f"{name} not exported with C linkage"


def test_status_strings(lib):
    for code in range(10):
        s = sv.sv_status_string(code)
        assert s and s != "unknown status"
    assert sv.sv_status_string(99) == "unknown status"


def test_launch_plan(lib):
    assert sv.sv_launch_plan(64, 4, 128256, sv.SV_BF16, 1.0, 0) == ["k_verify"]
    assert sv.sv_launch_plan(256, 7, 152064, sv.SV_BF16, 0.0, 50) == ["k_argmax"]
    assert sv.sv_launch_plan(128, 6, 128256, sv.SV_BF16, 0.8, 50) == ["k_topk_select", "k_topk_merge", "k_topk_verify"]
    assert sv.sv_launch_plan(8, 5, 32000, sv.SV_F32, 0.7, 5) == ["k_topk_select", "k_topk_merge", "k_topk_verify"]
    # k above the one-pass select's limit: the radix digit passes (2 for bf16, 4 for f32)
    assert sv.sv_launch_plan(128, 6, 128256, sv.SV_BF16, 0.8, 257) == \
        ["k_topk_digit", "k_topk_digit", "k_verify"]
    assert len(sv.sv_launch_plan(8, 5, 32000, sv.SV_F32, 0.7, 1000)) == 5
    assert sv.sv_launch_plan(8, 5, 32000, sv.SV_F32, 0.7, 32000) == ["k_verify"]


def test_workspace_bytes(lib):
    small = sv.sv_workspace_bytes(1, 1, 32, sv.SV_F32, 1.0, 0)
    big = sv.sv_workspace_bytes(64, 4, 128256, sv.SV_BF16, 1.0, 0)
    topk = sv.sv_workspace_bytes(64, 4, 128256, sv.SV_BF16, 1.0, 50)
    assert 0 < small < big < topk
    assert big % 256 == 0
    # 576 rows x 8 chunks of (float + double) partials at least
    assert big >= 576 * 8 * 12


V_, I_, F_, Z_ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
FAKE = 1 << 20  # never dereferenced: argument checks reject before any launch


def call(lib, **kw):
    a = dict(target=FAKE, draft=FAKE, dt=sv.SV_BF16, tokens=FAKE, ua=FAKE, us=FAKE, B=4, G=3,
             V=1024, T=1.0, k=0, acc=FAKE, out=FAKE, stats=None, ws=FAKE, nbytes=1 << 30,
             stream=None)
    a.update(kw)
    return lib.spec_verify(V_(a["target"]), V_(a["draft"]), a["dt"], V_(a["tokens"]), V_(a["ua"]),
                           V_(a["us"]), a["B"], a["G"], a["V"], F_(a["T"]), a["k"], V_(a["acc"]),
                           V_(a["out"]), V_(a["stats"]), V_(a["ws"]), Z_(a["nbytes"]),
                           V_(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(G=-1), 2), (dict(V=0), 2),
    (dict(dt=7), 3),
    (dict(T=-1.0), 4), (dict(T=float("nan")), 4), (dict(T=float("inf")), 4),
    (dict(target=None), 1), (dict(acc=None), 1), (dict(out=None), 1), (dict(ws=None), 1),
    (dict(tokens=None), 1), (dict(draft=None), 1), (dict(ua=None), 1), (dict(us=None), 1),
    (dict(nbytes=100), 5), (dict(ws=FAKE + 64), 5),
    (dict(target=FAKE + 1), 6), (dict(draft=FAKE + 2, dt=sv.SV_F32), 6),
])
def test_host_argument_errors(lib, kw, status):
    assert call(lib, **kw) == status


@pytest.mark.parametrize("kw", [
    dict(T=0.0, draft=None, ua=None, us=None),   # greedy reads no draft logits or uniforms
    dict(G=0, tokens=None, draft=None, ua=None),  # no drafts: only u_sample is read
])
def test_optional_pointers_are_optional(lib, kw):
    # with a too-small workspace the call stops at the workspace check, after the
    # pointer checks have passed
    assert call(lib, nbytes=16, **kw) == 5


def test_zero_prefix(lib):
    for args in [(1, 1, 32, sv.SV_F32, 1.0, 0), (64, 4, 128256, sv.SV_BF16, 1.0, 0),
                 (256, 7, 152064, sv.SV_BF16, 0.0, 0), (128, 6, 128256, sv.SV_BF16, 0.8, 50)]:
        z, n = sv.sv_workspace_zero_bytes(*args), sv.sv_workspace_bytes(*args)
        assert 0 < z <= n and z % 256 == 0
    # top-k: the thresholds handed from kernel to kernel lie beyond the prefix
    assert sv.sv_workspace_zero_bytes(128, 6, 128256, sv.SV_BF16, 0.8, 50) < \
        sv.sv_workspace_bytes(128, 6, 128256, sv.SV_BF16, 0.8, 50)
    assert sv.sv_workspace_zero_bytes(0, 1, 32, sv.SV_F32, 1.0, 0) == 0
    # more rows need more counters
    assert sv.sv_workspace_zero_bytes(64, 4, 128256, sv.SV_BF16, 1.0, 0) > \
        sv.sv_workspace_zero_bytes(8, 5, 32000, sv.SV_F32, 0.7, 0)


def call_sample(lib, **kw):
    a = dict(logits=FAKE, dt=sv.SV_BF16, u=FAKE, B=4, V=1024, T=1.0, k=0, tok=FAKE, st=FAKE,
             ws=FAKE, nbytes=1 << 30, stream=None)
    a.update(kw)
    return lib.spec_sample(V_(a["logits"]), a["dt"], V_(a["u"]), a["B"], a["V"], F_(a["T"]), a["k"],
                           V_(a["tok"]), V_(a["st"]), V_(a["ws"]), Z_(a["nbytes"]), V_(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(V=0), 2), (dict(dt=9), 3), (dict(T=-0.5), 4),
    (dict(logits=None), 1), (dict(u=None), 1), (dict(tok=None), 1), (dict(st=None), 1),
    (dict(ws=None), 1), (dict(nbytes=16), 5), (dict(logits=FAKE + 1), 6),
])
def test_sample_host_argument_errors(lib, kw, status):
    assert call_sample(lib, **kw) == status


def test_sample_greedy_reads_no_uniform(lib):
    # stops at the workspace check, after the pointer checks passed without u
    assert call_sample(lib, T=0.0, u=None, nbytes=16) == 5
    assert sv.sv_launch_plan(256, 0, 128256, sv.SV_BF16, 1.0, 0) == ["k_verify"]


def call_overlap(lib, **kw):
    a = dict(t=FAKE, d=FAKE, dt=sv.SV_BF16, B=4, G=3, V=1024, TR=4, T=1.0, k=0, beta=FAKE, tv=FAKE,
             st=FAKE, ws=FAKE, nbytes=1 << 30, stream=None)
    a.update(kw)
    return lib.spec_overlap(V_(a["t"]), V_(a["d"]), a["dt"], a["B"], a["G"], a["V"], a["TR"], F_(a["T"]),
                            a["k"], V_(a["beta"]), V_(a["tv"]), V_(a["st"]), V_(a["ws"]), Z_(a["nbytes"]),
                            V_(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(V=0), 2), (dict(G=-1), 2), (dict(TR=2), 2), (dict(TR=5), 2), (dict(dt=9), 3),
    (dict(T=0.0), 4), (dict(T=-1.0), 4), (dict(T=float("nan")), 4), (dict(T=float("inf")), 4),
    (dict(t=None), 1), (dict(d=None), 1), (dict(beta=None), 1), (dict(tv=None), 1), (dict(st=None), 1),
    (dict(ws=None), 1), (dict(t=FAKE + 1), 6), (dict(d=FAKE + 1), 6), (dict(nbytes=16), 5),
    (dict(ws=FAKE + 8), 5),
])
def test_overlap_host_argument_errors(lib, kw, status):
    assert call_overlap(lib, **kw) == status


def test_overlap_layouts_and_empty(lib):
    # both target layouts pass the checks (stopped at the workspace check)
    assert call_overlap(lib, TR=3, nbytes=16) == 5
    assert call_overlap(lib, TR=4, nbytes=16) == 5
    # no drafted positions: nothing to compute, nothing enqueued, no pointer needed
    assert call_overlap(lib, G=0, TR=0, t=None, d=None, beta=None, tv=None, st=None, ws=None) == 0
    assert sv.sv_overlap_launch_plan(4, 0, 1024, sv.SV_BF16, 1.0, 0) == []


def test_overlap_plan_and_workspace(lib):
    assert sv.sv_overlap_launch_plan(64, 4, 128256, sv.SV_BF16, 1.0, 0) == ["k_overlap"]
    assert sv.sv_overlap_launch_plan(64, 4, 128256, sv.SV_BF16, 1.0, 50) == ["k_topk_select", "k_topk_merge", "k_overlap"]
    assert sv.sv_overlap_launch_plan(64, 4, 128256, sv.SV_BF16, 1.0, 300) == \
        ["k_topk_digit", "k_topk_digit", "k_overlap"]
    assert len(sv.sv_overlap_launch_plan(8, 5, 32000, sv.SV_F32, 0.7, 500)) == 5
    args = (64, 4, 128256, sv.SV_BF16, 1.0, 0)
    n, z = lib.sv_overlap_workspace_bytes(*args), lib.sv_overlap_workspace_zero_bytes(*args)
    assert 0 < z <= n and z % 256 == 0 and n % 256 == 0
    # per chunk of 512 rows: 3 partial words; per chunk of 256 pairs: 4 sum words
    assert z == 512 * 8 * 3 * 8 + 256 * 8 * 4 * 8
    a2 = (64, 4, 128256, sv.SV_BF16, 1.0, 50)
    assert lib.sv_overlap_workspace_zero_bytes(*a2) < lib.sv_overlap_workspace_bytes(*a2)
    assert lib.sv_overlap_workspace_zero_bytes(64, 4, 128256, sv.SV_BF16, 0.0, 0) == 0



def call_tree(lib, **kw):
    a = dict(t=FAKE, d=FAKE, dt=sv.SV_BF16, tok=FAKE, par=FAKE, ua=FAKE, us=FAKE, B=4, N=8, V=1024, S=3,
             T=1.0, k=0, acc=FAKE, out=FAKE, path=FAKE, ws=FAKE, nbytes=1 << 30, stream=None)
    a.update(kw)
    return lib.spec_tree_verify(V_(a["t"]), V_(a["d"]), a["dt"], V_(a["tok"]), V_(a["par"]), V_(a["ua"]),
                                V_(a["us"]), a["B"], a["N"], a["V"], a["S"], F_(a["T"]), a["k"], V_(a["acc"]),
                                V_(a["out"]), V_(a["path"]), V_(a["ws"]), Z_(a["nbytes"]), V_(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(N=0), 2), (dict(N=1025), 2), (dict(V=0), 2), (dict(S=-1), 2), (dict(S=8), 2),
    (dict(dt=9), 3), (dict(T=-1.0), 4), (dict(T=float("nan")), 4),
    (dict(t=None), 1), (dict(tok=None), 1), (dict(par=None), 1), (dict(acc=None), 1), (dict(out=None), 1),
    (dict(ws=None), 1), (dict(d=None), 1), (dict(ua=None), 1), (dict(us=None), 1),
    (dict(t=FAKE + 1), 6), (dict(d=FAKE + 1), 6), (dict(nbytes=16), 5),
])
def test_tree_host_argument_errors(lib, kw, status):
    assert call_tree(lib, **kw) == status


def test_tree_optional_pointers_and_plan(lib):
    # path is optional; greedy reads no draft and no uniforms (stops at the workspace check)
    assert call_tree(lib, path=None, nbytes=16) == 5
    assert call_tree(lib, T=0.0, d=None, ua=None, us=None, nbytes=16) == 5
    # the walk forms the residual masses it needs inside the draw's launch
    assert sv.sv_tree_launch_plan(16, 32, 128256, 4, sv.SV_BF16, 1.0, 0) == ["k_tree_rows", "k_tree_draw"]
    # nodes of two or more children need rows of at most 32 chunks (a tree's draw items wait
    # for one another); chains (max_children 1) and greedy trees have no such limit
    assert lib.sv_tree_workspace_bytes(3, 10, 600000, 3, sv.SV_BF16, 1.0, 0) == 256
    assert lib.sv_tree_workspace_bytes(3, 10, 524288, 3, sv.SV_BF16, 1.0, 0) > 256
    assert lib.sv_tree_workspace_bytes(3, 10, 600000, 1, sv.SV_BF16, 1.0, 0) > 256
    assert lib.sv_tree_workspace_bytes(3, 10, 600000, 3, sv.SV_BF16, 0.0, 0) > 256
    assert sv.sv_tree_launch_plan(16, 32, 128256, 1, sv.SV_BF16, 1.0, 0) == ["k_tree_rows", "k_tree_draw"]
    assert sv.sv_tree_launch_plan(16, 32, 128256, 4, sv.SV_BF16, 0.0, 0) == ["k_tree_rows", "k_tree_walk"]
    assert sv.sv_tree_launch_plan(16, 32, 128256, 4, sv.SV_F32, 0.7, 5)[:3] == ["k_topk_select", "k_topk_merge", "k_tree_rows"]
    assert sv.sv_tree_launch_plan(16, 32, 128256, 4, sv.SV_F32, 0.7, 300)[:4] == ["k_topk_digit"] * 4
    args = (16, 32, 128256, 4, sv.SV_BF16, 1.0, 0)
    n, z = lib.sv_tree_workspace_bytes(*args), lib.sv_tree_workspace_zero_bytes(*args)
    assert 0 < z < n and z % 256 == 0 and n % 256 == 0
    assert lib.sv_tree_workspace_zero_bytes(16, 32, 128256, 4, sv.SV_BF16, -1.0, 0) == 0


def call_typ(lib, **kw):
    a = dict(t=FAKE, dt=sv.SV_BF16, tok=FAKE, B=4, G=3, V=1024, T=1.0, k=0, eps=0.1, delta=0.3, acc=FAKE,
             out=FAKE, ws=FAKE, nbytes=1 << 30, stream=None)
    a.update(kw)
    return lib.spec_typical_verify(V_(a["t"]), a["dt"], V_(a["tok"]), a["B"], a["G"], a["V"], F_(a["T"]), a["k"],
                                   F_(a["eps"]), F_(a["delta"]), V_(a["acc"]), V_(a["out"]), V_(a["ws"]),
                                   Z_(a["nbytes"]), V_(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(G=-1), 2), (dict(G=257), 2), (dict(V=0), 2), (dict(dt=9), 3), (dict(T=0.0), 4),
    (dict(T=float("inf")), 4), (dict(eps=-0.1), 8), (dict(delta=float("nan")), 8), (dict(eps=float("inf")), 8),
    (dict(t=None), 1), (dict(tok=None), 1), (dict(acc=None), 1), (dict(out=None), 1), (dict(ws=None), 1),
    (dict(t=FAKE + 1), 6), (dict(nbytes=16), 5),
])
def test_typical_host_argument_errors(lib, kw, status):
    assert call_typ(lib, **kw) == status


def test_typical_plan_and_workspace(lib):
    assert call_typ(lib, G=0, tok=None, nbytes=16) == 5
    assert call_typ(lib, G=256, nbytes=16) == 5
    assert call_typ(lib, eps=0.0, delta=0.0, nbytes=16) == 5
    assert sv.sv_typical_launch_plan(64, 4, 128256, sv.SV_BF16, 1.0, 0) == ["k_typical"]
    assert sv.sv_typical_launch_plan(64, 4, 128256, sv.SV_BF16, 1.0, 50) == ["k_topk_select", "k_topk_merge", "k_typical"]
    assert sv.sv_typical_launch_plan(64, 4, 128256, sv.SV_BF16, 1.0, 300) == ["k_topk_digit"] * 2 + ["k_typical"]
    args = (64, 4, 128256, sv.SV_BF16, 1.0, 0)
    n, z = lib.sv_typical_workspace_bytes(*args), lib.sv_typical_workspace_zero_bytes(*args)
    assert z == n == 320 * 8 * 8 * 8  # 320 rows of 8 chunks, 8 words each
    assert lib.sv_typical_workspace_zero_bytes(64, 4, 128256, sv.SV_BF16, 0.0, 0) == 0


def test_tag_epoch_before_any_launch(lib):
    """No kernel has been launched in this process: the launch count's 2^31 epoch is 0."""
    assert sv.load_library().sv_tag_epoch() == 0


def test_read_probe_validates_arguments(lib):
    """The streaming-read probe refuses NULL pointers and sizes that are not whole 32 KiB
    chunks before any HIP call."""
    import ctypes
    V = ctypes.c_void_p
    f = sv.load_library().sv_read_probe
    assert f(None, 32768, V(256), None) == 1
    assert f(V(256), 32768, None, None) == 1
    assert f(V(256), 0, V(256), None) == 2
    assert f(V(256), 32768 + 16, V(256), None) == 2
    assert f(V(264), 32768, V(256), None) == 2


def test_noalloc_refuses_oversized_arguments(lib):
    """spec_verify_noalloc answers arguments whose workspace exceeds its scratch array with
    SV_ERR_SCRATCH, after the usual argument checks and before any HIP call."""
    import ctypes
    V = ctypes.c_void_p
    p = V(256)
    f = sv.load_library().spec_verify_noalloc
    big = (1024, 8, 256000, sv.SV_BF16, 1.0, 50)   # about 241 MiB of workspace
    assert sv.sv_workspace_bytes(*big) > sv.NOALLOC_SCRATCH_BYTES
    assert f(p, p, sv.SV_BF16, p, p, p, 1024, 8, 256000, 1.0, 50, p, p, None, None) == 9
    assert f(p, p, sv.SV_BF16, p, p, p, 0, 8, 256000, 1.0, 50, p, p, None, None) == 2
    assert f(None, p, sv.SV_BF16, p, p, p, 1024, 8, 256000, 1.0, 50, p, p, None, None) == 1
    small = (64, 4, 128256, sv.SV_BF16, 1.0, 0)
    assert sv.sv_workspace_bytes(*small) <= sv.NOALLOC_SCRATCH_BYTES
    assert sv.sv_status_string(9) != "unknown status"

"""fp64 CPU oracle for batched speculative-sampling verification.

TEST INFRASTRUCTURE ONLY.  This package is the checker, not the product: only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the HIP library in
``rejection_sampling_verify_02_amd`` and never calls it.

The arithmetic lives in ``spec_verify_ref.c`` (plain C, double precision,
sums in index order); this module only builds that file and marshals NumPy
arrays into it.  The functions and the passages they follow:

* ``spec_verify_ref`` -- chain verification with a correction or bonus draw
  ("Speculative Decoding 的朴素思想", sections "一次 sampling 怎么执行",
  "Correction 为什么用正残差", "从单个 token 接到一段 draft"; "推测解码：接受规则、
  状态与收益边界", section "两模型精确采样").
* ``policy_rows`` -- logits to distribution with temperature and top-k
  (first page, section "从 LM head 到 sampling distribution").
* ``invcdf`` / ``sample_rows`` -- the draw by cumulative intervals (first page,
  section "一次 sampling 怎么执行", step 1); ``sample_rows`` is also the oracle of the
  library's batched sampler ``spec_sample``.
* ``topk_threshold_rows`` / ``argmax_rows`` -- the top-k cut and greedy choice.
* ``tree_verify`` -- verification of a draft tree by multi-step rejection (first page,
  "Token Tree Verifier"; EAGLE page, section 6.2): siblings are tested in order against
  the current distribution, which each rejection replaces by norm([cur - q]_+).
* ``typical_verify`` -- Medusa's typical acceptance (first page, "Medusa-1 与 typical
  acceptance"): the longest prefix of drafted tokens with p(x) > min(eps, delta *
  exp(-H(p))), then the target's greedy token.
* ``overlap`` -- per drafted position, beta = sum min(p, q) (the acceptance
  probability, first page, section "为什么接受概率恰好是这个比值"; the overlap behind the
  LK loss and DSpark's c* on the second page) and tv = sum [p - q]_+.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against values
the pages print, closed forms, invariants and library routines, including the
fallback taken when a rejection's residual mass is exactly zero (rows that
differ only at a token whose mass is lost in double precision reach it).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "spec_verify_ref.c"
_LIB = _HERE / "libspec_verify_ref.so"

F32, BF16 = 0, 1

ERR_TOKEN, ERR_QZERO, ERR_ROW, ERR_UNIFORM, ERR_TREE = -1, -2, -3, -4, -6


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-o", str(tmp), str(_SRC), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _bind(lib):
    P = ctypes.c_void_p
    i32, f64 = ctypes.c_int, ctypes.c_double
    lib.ref_spec_verify.argtypes = [P, P, i32, P, P, P, i32, i32, i32, f64, i32,
                                    P, P, P, P, P, i32]
    lib.ref_spec_verify.restype = i32
    lib.ref_policy_rows.argtypes = [P, i32, i32, i32, f64, i32, P, P]
    lib.ref_policy_rows.restype = i32
    lib.ref_sample_rows.argtypes = [P, i32, i32, i32, f64, i32, P, P, P, P, i32]
    lib.ref_sample_rows.restype = i32
    lib.ref_topk_threshold_rows.argtypes = [P, i32, i32, i32, i32, P]
    lib.ref_topk_threshold_rows.restype = i32
    lib.ref_argmax_rows.argtypes = [P, i32, i32, i32, P]
    lib.ref_argmax_rows.restype = i32
    lib.ref_overlap.argtypes = [P, P, i32, i32, i32, i32, i32, f64, i32, P, P, P, i32]
    lib.ref_overlap.restype = i32
    lib.ref_tree_verify.argtypes = [P, P, i32, P, P, P, P, i32, i32, i32, f64, i32, P, P, P, P, P, i32]
    lib.ref_tree_verify.restype = i32
    lib.ref_typical_verify.argtypes = [P, i32, P, i32, i32, i32, f64, i32, f64, f64, P, P, P, P, i32]
    lib.ref_typical_verify.restype = i32
    lib.ref_invcdf.argtypes = [P, i32, f64, P]
    lib.ref_invcdf.restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build(force=False)
        _lib = _bind(ctypes.CDLL(str(_LIB)))
    return _lib


def _swap_library(path):
    """Route every call through another build of the oracle (mutation tests); returns the old one."""
    global _lib
    old = _lib
    _lib = None if path is None else _bind(ctypes.CDLL(str(path)))
    return old


def default_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits(a: np.ndarray) -> tuple[np.ndarray, int]:
    """float32 arrays are f32 logits; uint16 arrays hold bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


def spec_verify_ref(target, draft, draft_tokens, u_accept, u_sample, temperature, top_k=0,
                    *, with_diagnostics=False, nthreads=None):
    """Oracle verification of B sequences.

    target [B, G+1, V] and draft [B, G, V] logits (float32, or uint16 bf16 bits),
    draft_tokens [B, G] int32, u_accept [B, G] and u_sample [B] float32.  With
    temperature 0 the draft logits and uniforms may be None.

    Returns (accepted_len [B], out_tokens [B, G+1]) and, with diagnostics,
    a dict holding row_logz [B, 2G+1], accept_margin [B, G] and sample_margin [B].
    """
    lib = _load()
    target, dt = _logits(target)
    B, G1, V = target.shape
    G = G1 - 1
    greedy = temperature == 0
    if draft is None:
        draft = np.zeros((B, G, V), dtype=target.dtype)
    draft, dt2 = _logits(draft)
    assert dt2 == dt and draft.shape == (B, G, V)
    tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, G)
    ua = np.zeros((B, G), np.float32) if u_accept is None else np.ascontiguousarray(u_accept, np.float32)
    us = np.zeros((B,), np.float32) if u_sample is None else np.ascontiguousarray(u_sample, np.float32)
    assert ua.shape == (B, G) and us.shape == (B,)
    acc = np.empty((B,), np.int32)
    out = np.empty((B, G + 1), np.int32)
    logz = am = sm = None
    if with_diagnostics:
        logz = np.full((B, 2 * G + 1), np.nan)
        am = np.full((B, G), np.nan)
        sm = np.full((B,), np.nan)
    rc = lib.ref_spec_verify(_ptr(target), _ptr(draft), dt, _ptr(tokens), _ptr(ua), _ptr(us),
                             B, G, V, float(temperature), int(top_k), _ptr(acc), _ptr(out),
                             _ptr(logz), _ptr(am), _ptr(sm),
                             int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    if with_diagnostics:
        return acc, out, {"row_logz": logz, "accept_margin": am, "sample_margin": sm}
    return acc, out


def policy_rows(logits, temperature, top_k=0):
    """Probabilities [R, V] and log-partitions [R] of each row (rows flattened)."""
    lib = _load()
    z, dt = _logits(logits)
    V = z.shape[-1]
    R = z.size // V
    P = np.empty((R, V), np.float64)
    L = np.empty((R,), np.float64)
    lib.ref_policy_rows(_ptr(z), dt, R, V, float(temperature), int(top_k), _ptr(P), _ptr(L))
    return P.reshape(z.shape), L.reshape(z.shape[:-1])


def sample_rows(logits, u, temperature, top_k=0, nthreads=None, *, with_status=False):
    """One token per row drawn from the row's policy by inverse CDF with uniform u.

    With ``with_status`` also returns each row's status (0, -3 invalid row, -4 uniform
    outside [0,1)) and the draw's boundary distance."""
    lib = _load()
    z, dt = _logits(logits)
    V = z.shape[-1]
    R = z.size // V
    u = np.zeros((R,), np.float32) if u is None else np.ascontiguousarray(u, np.float32).reshape(R)
    tok = np.empty((R,), np.int32)
    st = np.empty((R,), np.int32)
    mg = np.empty((R,), np.float64)
    lib.ref_sample_rows(_ptr(z), dt, R, V, float(temperature), int(top_k), _ptr(u), _ptr(tok),
                        _ptr(st), _ptr(mg), int(nthreads or default_threads()))
    shp = z.shape[:-1]
    if with_status:
        return tok.reshape(shp), st.reshape(shp), mg.reshape(shp)
    return tok.reshape(shp)


def topk_threshold_rows(logits, top_k):
    lib = _load()
    z, dt = _logits(logits)
    V = z.shape[-1]
    R = z.size // V
    tau = np.empty((R,), np.float64)
    lib.ref_topk_threshold_rows(_ptr(z), dt, R, V, int(top_k), _ptr(tau))
    return tau.reshape(z.shape[:-1])


def argmax_rows(logits):
    lib = _load()
    z, dt = _logits(logits)
    V = z.shape[-1]
    R = z.size // V
    idx = np.empty((R,), np.int32)
    lib.ref_argmax_rows(_ptr(z), dt, R, V, _ptr(idx))
    return idx.reshape(z.shape[:-1])


def tree_verify(target, draft, tokens, parent, u_accept, u_sample, temperature, top_k=0, *,
                with_diagnostics=False, nthreads=None):
    """Oracle verification of B draft trees of N nodes.

    target [B, N, V] (p at every node) and draft [B, N, V] (q at every node; leaf rows
    unused; may be None at temperature 0) logits, float32 or uint16 bf16 bits; tokens
    and parent [B, N] int32 (parent[:, 0] = -1, parent[n] < n); u_accept [B, N] and
    u_sample [B] float32 (None at temperature 0).  Returns (accepted_len [B], out_tokens
    [B, N], path_nodes [B, N]) and, with diagnostics, a dict of accept_margin [B, N] and
    sample_margin [B]."""
    lib = _load()
    target, dt = _logits(target)
    B, N, V = target.shape
    if draft is None:
        draft = np.zeros_like(target)
    draft, dt2 = _logits(draft)
    assert dt2 == dt and draft.shape == (B, N, V)
    tok = np.ascontiguousarray(tokens, np.int32).reshape(B, N)
    par = np.ascontiguousarray(parent, np.int32).reshape(B, N)
    ua = np.zeros((B, N), np.float32) if u_accept is None else np.ascontiguousarray(u_accept, np.float32)
    us = np.zeros((B,), np.float32) if u_sample is None else np.ascontiguousarray(u_sample, np.float32)
    acc = np.empty((B,), np.int32)
    out = np.empty((B, N), np.int32)
    path = np.empty((B, N), np.int32)
    am = np.empty((B, N), np.float64)
    sm = np.empty((B,), np.float64)
    rc = lib.ref_tree_verify(_ptr(target), _ptr(draft), dt, _ptr(tok), _ptr(par), _ptr(ua), _ptr(us),
                             B, N, V, float(temperature), int(top_k), _ptr(acc), _ptr(out), _ptr(path),
                             _ptr(am), _ptr(sm), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    if with_diagnostics:
        return acc, out, path, {"accept_margin": am, "sample_margin": sm}
    return acc, out, path


def typical_verify(target, draft_tokens, temperature, epsilon, delta, top_k=0, *,
                   with_diagnostics=False, nthreads=None):
    """Oracle typical acceptance of B sequences: target [B, G+1, V] logits (float32 or
    uint16 bf16 bits), draft_tokens [B, G] int32, temperature > 0, epsilon, delta >= 0.
    Returns (accepted_len [B], out_tokens [B, G+1]) and, with diagnostics, a dict of
    margin [B, G] (log p(x) - log threshold) and entropy [B, G+1] (nats)."""
    lib = _load()
    target, dt = _logits(target)
    B, G1, V = target.shape
    G = G1 - 1
    tok = np.ascontiguousarray(draft_tokens, np.int32).reshape(B, G)
    acc = np.empty((B,), np.int32)
    out = np.empty((B, G + 1), np.int32)
    mg = np.empty((B, G), np.float64)
    ent = np.empty((B, G + 1), np.float64)
    rc = lib.ref_typical_verify(_ptr(target), dt, _ptr(tok), B, G, V, float(temperature), int(top_k),
                                float(epsilon), float(delta), _ptr(acc), _ptr(out), _ptr(mg), _ptr(ent),
                                int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (typical acceptance needs T > 0, eps, delta >= 0)")
    if with_diagnostics:
        return acc, out, {"margin": mg, "entropy": ent}
    return acc, out


def overlap(target, draft, temperature, top_k=0, *, nthreads=None):
    """beta [B, G], tv [B, G] and status [B, G] of every drafted position.

    target [B, TR, V] with TR = G or G + 1 rows per sequence (position i uses target row
    i; a trailing row G is not read), draft [B, G, V]; float32 or uint16 bf16 bits.
    temperature must be > 0.  Status is 0, or -3 when either row is unusable (beta and
    tv are then NaN)."""
    lib = _load()
    target, dt = _logits(target)
    draft, dt2 = _logits(draft)
    assert dt2 == dt and target.ndim == 3 and draft.ndim == 3
    B, G, V = draft.shape
    TR = target.shape[1]
    assert target.shape[0] == B and target.shape[2] == V and TR in (G, G + 1)
    beta = np.empty((B, G), np.float64)
    tv = np.empty((B, G), np.float64)
    st = np.empty((B, G), np.int32)
    rc = lib.ref_overlap(_ptr(target), _ptr(draft), dt, B, G, V, TR, float(temperature), int(top_k),
                         _ptr(beta), _ptr(tv), _ptr(st), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (overlap needs temperature > 0)")
    return beta, tv, st


def invcdf(w, u):
    """Index drawn from non-negative weights w by uniform u, and its boundary distance."""
    lib = _load()
    w = np.ascontiguousarray(w, np.float64)
    d = ctypes.c_double(0.0)
    v = lib.ref_invcdf(_ptr(w), w.size, float(u), ctypes.byref(d))
    return int(v), float(d.value)

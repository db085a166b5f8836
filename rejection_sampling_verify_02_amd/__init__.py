"""MI355X-native batched speculative-sampling verification.

Thin binding over the C ABI in ``include/spec_verify.h`` (library
``libspec_verify.so`` built in-tree by ``rejection_sampling_verify_02_amd.build``).
Every step of the verification runs in the library's HIP kernels; this module
only checks and marshals arguments.  PyTorch is used for device memory and the
current stream.  There is no CPU fallback: if the library is not built, every
call raises.

    acc, out = spec_verify(target_logits, draft_logits, draft_tokens,
                           u_accept, u_sample, temperature, top_k)
"""
from __future__ import annotations

import ctypes
from pathlib import Path

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libspec_verify.so"

SV_F32, SV_BF16 = 0, 1
ROW_BAD_TOKEN, ROW_Q_ZERO, ROW_BAD_LOGITS, ROW_BAD_UNIFORM, ROW_INTERNAL, ROW_BAD_TREE = -1, -2, -3, -4, -5, -6
MAX_LAUNCHES = 8

_STATUS = {0: "SV_OK", 1: "SV_ERR_NULL", 2: "SV_ERR_SHAPE", 3: "SV_ERR_DTYPE",
           4: "SV_ERR_TEMPERATURE", 5: "SV_ERR_WORKSPACE", 6: "SV_ERR_ALIGN", 7: "SV_ERR_LAUNCH",
           8: "SV_ERR_PARAM", 9: "SV_ERR_SCRATCH"}

EXPORTED = ("spec_verify", "spec_verify_timed", "sv_workspace_bytes", "sv_workspace_zero_bytes",
            "sv_status_string", "sv_launch_plan", "spec_sample", "spec_sample_timed",
            "spec_overlap", "spec_overlap_timed", "sv_overlap_workspace_bytes",
            "sv_overlap_workspace_zero_bytes", "sv_overlap_launch_plan",
            "spec_tree_verify", "spec_tree_verify_timed", "sv_tree_workspace_bytes",
            "sv_tree_workspace_zero_bytes", "sv_tree_launch_plan",
            "spec_typical_verify", "spec_typical_verify_timed", "sv_typical_workspace_bytes",
            "sv_typical_workspace_zero_bytes", "sv_typical_launch_plan", "sv_tag_epoch",
            "sv_read_probe", "spec_verify_noalloc", "sv_timeline_stamps")


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{_STATUS.get(status, status)}: {text}")
        self.status = status


_lib = None


def load_library(path: Path | str | None = None) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is not built; run `python -m rejection_sampling_verify_02_amd.build`")
    lib = ctypes.CDLL(str(p))
    V, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    common = [V, V, I32, V, V, V, I32, I32, I32, F32, I32, V, V, V, V, SZ, V]
    lib.spec_verify.argtypes = common
    lib.spec_verify.restype = I32
    lib.spec_verify_noalloc.argtypes = common[:14] + [V]
    lib.spec_verify_noalloc.restype = I32
    lib.spec_verify_timed.argtypes = common + [V, I32, V]
    lib.spec_verify_timed.restype = I32
    smp = [V, I32, V, I32, I32, F32, I32, V, V, V, SZ, V]
    lib.spec_sample.argtypes = smp
    lib.spec_sample.restype = I32
    lib.spec_sample_timed.argtypes = smp + [V, I32, V]
    lib.spec_sample_timed.restype = I32
    ovl = [V, V, I32, I32, I32, I32, I32, F32, I32, V, V, V, V, SZ, V]
    lib.spec_overlap.argtypes = ovl
    lib.spec_overlap.restype = I32
    lib.spec_overlap_timed.argtypes = ovl + [V, I32, V]
    lib.spec_overlap_timed.restype = I32
    for fn in (lib.sv_overlap_workspace_bytes, lib.sv_overlap_workspace_zero_bytes):
        fn.argtypes = [I32, I32, I32, I32, F32, I32]
        fn.restype = SZ
    lib.sv_overlap_launch_plan.argtypes = [I32, I32, I32, I32, F32, I32]
    lib.sv_overlap_launch_plan.restype = ctypes.c_char_p
    tree = [V, V, I32, V, V, V, V, I32, I32, I32, I32, F32, I32, V, V, V, V, SZ, V]
    lib.spec_tree_verify.argtypes = tree
    lib.spec_tree_verify.restype = I32
    lib.spec_tree_verify_timed.argtypes = tree + [V, I32, V]
    lib.spec_tree_verify_timed.restype = I32
    for fn in (lib.sv_tree_workspace_bytes, lib.sv_tree_workspace_zero_bytes):
        fn.argtypes = [I32, I32, I32, I32, I32, F32, I32]
        fn.restype = SZ
    lib.sv_tree_launch_plan.argtypes = [I32, I32, I32, I32, I32, F32, I32]
    lib.sv_tree_launch_plan.restype = ctypes.c_char_p
    typ = [V, I32, V, I32, I32, I32, F32, I32, F32, F32, V, V, V, SZ, V]
    lib.spec_typical_verify.argtypes = typ
    lib.spec_typical_verify.restype = I32
    lib.spec_typical_verify_timed.argtypes = typ + [V, I32, V]
    lib.spec_typical_verify_timed.restype = I32
    for fn in (lib.sv_typical_workspace_bytes, lib.sv_typical_workspace_zero_bytes):
        fn.argtypes = [I32, I32, I32, I32, F32, I32]
        fn.restype = SZ
    lib.sv_typical_launch_plan.argtypes = [I32, I32, I32, I32, F32, I32]
    lib.sv_typical_launch_plan.restype = ctypes.c_char_p
    lib.sv_workspace_bytes.argtypes = [I32, I32, I32, I32, F32, I32]
    lib.sv_workspace_bytes.restype = SZ
    lib.sv_workspace_zero_bytes.argtypes = [I32, I32, I32, I32, F32, I32]
    lib.sv_workspace_zero_bytes.restype = SZ
    lib.sv_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.sv_read_probe.restype = I32
    lib.sv_timeline_stamps.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.sv_timeline_stamps.restype = I32
    lib.sv_tag_epoch.argtypes = []
    lib.sv_tag_epoch.restype = ctypes.c_uint32
    lib.sv_status_string.argtypes = [I32]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_launch_plan.argtypes = [I32, I32, I32, I32, F32, I32]
    lib.sv_launch_plan.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def sv_status_string(status: int) -> str:
    return load_library().sv_status_string(int(status)).decode()


def sv_workspace_bytes(B: int, G: int, V: int, dtype: int, temperature: float, top_k: int = 0) -> int:
    return int(load_library().sv_workspace_bytes(B, G, V, dtype, float(temperature), int(top_k)))


def sv_workspace_zero_bytes(B: int, G: int, V: int, dtype: int, temperature: float,
                            top_k: int = 0) -> int:
    return int(load_library().sv_workspace_zero_bytes(B, G, V, dtype, float(temperature), int(top_k)))


def sv_launch_plan(B: int, G: int, V: int, dtype: int, temperature: float, top_k: int = 0) -> list[str]:
    s = load_library().sv_launch_plan(B, G, V, dtype, float(temperature), int(top_k)).decode()
    return s.split(";")


def sv_overlap_launch_plan(B: int, G: int, V: int, dtype: int, temperature: float,
                          top_k: int = 0) -> list[str]:
    s = load_library().sv_overlap_launch_plan(B, G, V, dtype, float(temperature), int(top_k)).decode()
    return s.split(";") if s else []


def sv_tree_launch_plan(B: int, N: int, V: int, max_children: int, dtype: int, temperature: float,
                       top_k: int = 0) -> list[str]:
    s = load_library().sv_tree_launch_plan(B, N, V, max_children, dtype, float(temperature), int(top_k)).decode()
    return s.split(";")


def sv_typical_launch_plan(B: int, G: int, V: int, dtype: int, temperature: float, top_k: int = 0) -> list[str]:
    return load_library().sv_typical_launch_plan(B, G, V, dtype, float(temperature), int(top_k)).decode().split(";")


# ------------------------------------------------------------------ workspace

class Workspace:
    """A device buffer for the library's scratch data, one per device, grown on demand.

    The library's workgroups hand results to one another as tagged words kept in the
    first ``sv_workspace_zero_bytes(...)`` bytes: those must hold zeros or words of
    completed calls when a call starts, and every call leaves them that way.  This class
    remembers how long a zeroed prefix the buffer has and, before a call that needs a
    longer one, zeroes it with a fill kernel on the call's stream.  Calls sharing a
    workspace must be ordered on one stream.
    """

    def __init__(self):
        self._buf = {}
        self._zero = {}
        self._used = {}   # the longest prefix any call has marked since the last full zeroing
        self._epoch = {}

    def get(self, nbytes: int, zero_bytes: int, device, stream: int):
        import torch
        key = torch.device(device).index
        buf = self._buf.get(key)
        epoch = int(load_library().sv_tag_epoch())
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            torch.cuda.synchronize(device)
            self._buf[key] = buf
            self._zero[key] = buf.numel()
            self._used[key] = 0
            self._epoch[key] = epoch
        if epoch != self._epoch[key]:
            # the launch count passed a multiple of 2^31: tags of calls made before it may
            # come back, so every word a call has marked is cleared
            n = max(self._used[key], zero_bytes)
            with torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device)):
                buf[:n].zero_()
            self._zero[key] = n
            self._used[key] = 0
            self._epoch[key] = epoch
        if zero_bytes > self._zero[key]:
            with torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device)):
                buf[:zero_bytes].zero_()
            self._zero[key] = zero_bytes
        return buf

    def called(self, device, zero_bytes: int) -> None:
        """Record that a call with this zero prefix was enqueued."""
        import torch
        key = torch.device(device).index
        self._zero[key] = zero_bytes
        self._used[key] = max(self._used.get(key, 0), zero_bytes)


_default_ws = Workspace()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def spec_verify(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature: float,
                top_k: int = 0, *, row_stats: bool = False, workspace: Workspace | None = None,
                stream=None, out=None, events=None):
    """Batched verification on the GPU (see include/spec_verify.h for the semantics).

    target_logits [B, G+1, V] and draft_logits [B, G, V] (bfloat16 or float32, same dtype),
    draft_tokens [B, G] int32, u_accept [B, G] and u_sample [B] float32; with
    temperature 0 the draft logits and uniforms may be None.

    Returns (accepted_len [B], out_tokens [B, G+1]) int32 tensors, plus row_stats
    [B, 2G+1, 2] float32 when requested.  ``out`` may supply preallocated output
    tensors (accepted_len, out_tokens[, row_stats]).  ``events`` (a list of raw
    hipEvent_t handles, two per kernel: start and stop of that dispatch) times each
    kernel; the number of kernels launched is then returned as the last element.
    """
    import torch
    lib = load_library()
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("target_logits must be a device tensor")
    dt = _dtype_code(target_logits)
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, G+1, V]")
    B, G1, V = target_logits.shape
    G = G1 - 1
    _check(target_logits, "target_logits", (B, G + 1, V), target_logits.dtype, dev)
    greedy = float(temperature) == 0.0
    if draft_tokens is not None and draft_tokens.dtype == torch.int64:
        draft_tokens = draft_tokens.to(torch.int32)
    if G > 0 or draft_tokens is not None:
        _check(draft_tokens, "draft_tokens", (B, G), torch.int32, dev)
    if not greedy:
        if G > 0 or draft_logits is not None:
            _check(draft_logits, "draft_logits", (B, G, V), target_logits.dtype, dev)
        if G > 0 or u_accept is not None:
            _check(u_accept, "u_accept", (B, G), torch.float32, dev)
        _check(u_sample, "u_sample", (B,), torch.float32, dev)
    else:
        draft_logits = u_accept = u_sample = None
    if out is not None:
        acc, toks = out[0], out[1]
        stats = out[2] if row_stats else None
    else:
        acc = torch.empty((B,), dtype=torch.int32, device=dev)
        toks = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
        stats = torch.empty((B, 2 * G + 1, 2), dtype=torch.float32, device=dev) if row_stats else None
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_workspace_bytes(B, G, V, dt, float(temperature), int(top_k)))
    zbytes = int(lib.sv_workspace_zero_bytes(B, G, V, dt, float(temperature), int(top_k)))
    wso = workspace or _default_ws
    ws = wso.get(nbytes, zbytes, dev, stream)
    args = [_ptr(target_logits), _ptr(draft_logits), dt, _ptr(draft_tokens), _ptr(u_accept),
            _ptr(u_sample), B, G, V, float(temperature), int(top_k), _ptr(acc), _ptr(toks),
            _ptr(stats), _ptr(ws), ws.numel(), ctypes.c_void_p(stream)]
    if events is None:
        st = lib.spec_verify(*args)
        nl = None
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        n = ctypes.c_int32(0)
        st = lib.spec_verify_timed(*args, arr, len(events), ctypes.byref(n))
        nl = n.value
    if st != 0:
        raise SpecVerifyError(st, sv_status_string(st))
    wso.called(dev, zbytes)
    res = (acc, toks) + ((stats,) if row_stats else ())
    return res + ((nl,) if events is not None else ())


def spec_sample(logits, u, temperature: float, top_k: int = 0, *, workspace: Workspace | None = None,
                stream=None, out=None, events=None):
    """Batched sampling on the GPU (see include/spec_verify.h): one token per row of
    logits [B, V] (bfloat16 or float32) drawn by inverse CDF with u [B] float32 (None at
    temperature 0).  Returns (tokens [B], row_status [B]) int32 tensors; ``out`` may supply
    them.  ``events`` as for spec_verify."""
    import torch
    lib = load_library()
    dev = logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be a device tensor")
    dt = _dtype_code(logits)
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V]")
    B, V = logits.shape
    _check(logits, "logits", (B, V), logits.dtype, dev)
    greedy = float(temperature) == 0.0
    if greedy:
        u = None
    else:
        _check(u, "u", (B,), torch.float32, dev)
    if out is not None:
        tok, st = out
    else:
        tok = torch.empty((B,), dtype=torch.int32, device=dev)
        st = torch.empty((B,), dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_workspace_bytes(B, 0, V, dt, float(temperature), int(top_k)))
    zbytes = int(lib.sv_workspace_zero_bytes(B, 0, V, dt, float(temperature), int(top_k)))
    wso = workspace or _default_ws
    ws = wso.get(nbytes, zbytes, dev, stream)
    args = [_ptr(logits), dt, _ptr(u), B, V, float(temperature), int(top_k), _ptr(tok), _ptr(st),
            _ptr(ws), ws.numel(), ctypes.c_void_p(stream)]
    if events is None:
        rc = lib.spec_sample(*args)
        nl = None
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        n = ctypes.c_int32(0)
        rc = lib.spec_sample_timed(*args, arr, len(events), ctypes.byref(n))
        nl = n.value
    if rc != 0:
        raise SpecVerifyError(rc, sv_status_string(rc))
    wso.called(dev, zbytes)
    return (tok, st) if events is None else (tok, st, nl)


def spec_overlap(target_logits, draft_logits, temperature: float, top_k: int = 0, *,
                 workspace: Workspace | None = None, stream=None, out=None, events=None):
    """Per-position overlap on the GPU (see include/spec_verify.h): for target [B, TR, V]
    (TR = G + 1, the verification layout, or G) and draft [B, G, V] logits (bfloat16 or
    float32), returns (beta, tv, status): beta = sum min(p, q) and tv = sum [p - q]_+ as
    [B, G] float64 tensors and the pair status [B, G] int32.  ``out`` may supply the three
    tensors; ``events`` as for spec_verify."""
    import torch
    lib = load_library()
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be device tensors")
    dt = _dtype_code(target_logits)
    if target_logits.dim() != 3 or draft_logits is None or draft_logits.dim() != 3:
        raise ValueError("target must be [B, TR, V] and draft [B, G, V]")
    B, G, V = draft_logits.shape
    TR = target_logits.shape[1]
    _check(target_logits, "target_logits", (B, TR, V), target_logits.dtype, dev)
    _check(draft_logits, "draft_logits", (B, G, V), target_logits.dtype, dev)
    if out is not None:
        beta, tv, st = out
    else:
        beta = torch.empty((B, G), dtype=torch.float64, device=dev)
        tv = torch.empty((B, G), dtype=torch.float64, device=dev)
        st = torch.empty((B, G), dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_overlap_workspace_bytes(B, G, V, dt, float(temperature), int(top_k)))
    zbytes = int(lib.sv_overlap_workspace_zero_bytes(B, G, V, dt, float(temperature), int(top_k)))
    wso = workspace or _default_ws
    ws = wso.get(nbytes, zbytes, dev, stream)
    args = [_ptr(target_logits), _ptr(draft_logits), dt, B, G, V, TR, float(temperature), int(top_k),
            _ptr(beta), _ptr(tv), _ptr(st), _ptr(ws), ws.numel(), ctypes.c_void_p(stream)]
    if events is None:
        rc = lib.spec_overlap(*args)
        nl = None
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        n = ctypes.c_int32(0)
        rc = lib.spec_overlap_timed(*args, arr, len(events), ctypes.byref(n))
        nl = n.value
    if rc != 0:
        raise SpecVerifyError(rc, sv_status_string(rc))
    wso.called(dev, zbytes)
    return (beta, tv, st) if events is None else (beta, tv, st, nl)


def spec_tree_verify(target_logits, draft_logits, tokens, parent, u_accept, u_sample, temperature: float,
                     top_k: int = 0, *, max_children: int | None = None, workspace: Workspace | None = None,
                     stream=None, out=None, events=None):
    """Tree verification on the GPU (see include/spec_verify.h): target and draft logits
    [B, N, V] (bfloat16 or float32; draft may be None at temperature 0), tokens and parent
    [B, N] int32, u_accept [B, N] and u_sample [B] float32 (None at temperature 0).
    max_children (the most children any node has) defaults to N - 1.  Returns
    (accepted_len [B], out_tokens [B, N], path_nodes [B, N]) int32 tensors; ``out`` may
    supply them; ``events`` as for spec_verify."""
    import torch
    lib = load_library()
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be device tensors")
    dt = _dtype_code(target_logits)
    if target_logits.dim() != 3:
        raise ValueError("target must be [B, N, V]")
    B, N, V = target_logits.shape
    greedy = float(temperature) == 0.0
    _check(target_logits, "target_logits", (B, N, V), target_logits.dtype, dev)
    _check(tokens, "tokens", (B, N), torch.int32, dev)
    _check(parent, "parent", (B, N), torch.int32, dev)
    if greedy:
        draft_logits = u_accept = u_sample = None
    else:
        _check(draft_logits, "draft_logits", (B, N, V), target_logits.dtype, dev)
        _check(u_accept, "u_accept", (B, N), torch.float32, dev)
        _check(u_sample, "u_sample", (B,), torch.float32, dev)
    S = (N - 1) if max_children is None else int(max_children)
    if out is not None:
        acc, toks, path = out
    else:
        acc = torch.empty((B,), dtype=torch.int32, device=dev)
        toks = torch.empty((B, N), dtype=torch.int32, device=dev)
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_tree_workspace_bytes(B, N, V, S, dt, float(temperature), int(top_k)))
    zbytes = int(lib.sv_tree_workspace_zero_bytes(B, N, V, S, dt, float(temperature), int(top_k)))
    wso = workspace or _default_ws
    ws = wso.get(nbytes, zbytes, dev, stream)
    args = [_ptr(target_logits), _ptr(draft_logits), dt, _ptr(tokens), _ptr(parent), _ptr(u_accept),
            _ptr(u_sample), B, N, V, S, float(temperature), int(top_k), _ptr(acc), _ptr(toks), _ptr(path),
            _ptr(ws), ws.numel(), ctypes.c_void_p(stream)]
    if events is None:
        rc = lib.spec_tree_verify(*args)
        nl = None
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        n = ctypes.c_int32(0)
        rc = lib.spec_tree_verify_timed(*args, arr, len(events), ctypes.byref(n))
        nl = n.value
    if rc != 0:
        raise SpecVerifyError(rc, sv_status_string(rc))
    wso.called(dev, zbytes)
    return (acc, toks, path) if events is None else (acc, toks, path, nl)


def spec_typical_verify(target_logits, draft_tokens, temperature: float, epsilon: float, delta: float,
                        top_k: int = 0, *, workspace: Workspace | None = None, stream=None, out=None,
                        events=None):
    """Typical acceptance on the GPU (see include/spec_verify.h): target logits [B, G+1, V]
    (bfloat16 or float32), draft_tokens [B, G] int32.  Returns (accepted_len [B],
    out_tokens [B, G+1]) int32 tensors; ``out`` may supply them; ``events`` as for
    spec_verify."""
    import torch
    lib = load_library()
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("logits must be device tensors")
    dt = _dtype_code(target_logits)
    if target_logits.dim() != 3:
        raise ValueError("target must be [B, G+1, V]")
    B, G1, V = target_logits.shape
    G = G1 - 1
    _check(target_logits, "target_logits", (B, G1, V), target_logits.dtype, dev)
    _check(draft_tokens, "draft_tokens", (B, G), torch.int32, dev)
    if out is not None:
        acc, toks = out
    else:
        acc = torch.empty((B,), dtype=torch.int32, device=dev)
        toks = torch.empty((B, G1), dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    nbytes = int(lib.sv_typical_workspace_bytes(B, G, V, dt, float(temperature), int(top_k)))
    zbytes = int(lib.sv_typical_workspace_zero_bytes(B, G, V, dt, float(temperature), int(top_k)))
    wso = workspace or _default_ws
    ws = wso.get(nbytes, zbytes, dev, stream)
    args = [_ptr(target_logits), dt, _ptr(draft_tokens), B, G, V, float(temperature), int(top_k), float(epsilon),
            float(delta), _ptr(acc), _ptr(toks), _ptr(ws), ws.numel(), ctypes.c_void_p(stream)]
    if events is None:
        rc = lib.spec_typical_verify(*args)
        nl = None
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        n = ctypes.c_int32(0)
        rc = lib.spec_typical_verify_timed(*args, arr, len(events), ctypes.byref(n))
        nl = n.value
    if rc != 0:
        raise SpecVerifyError(rc, sv_status_string(rc))
    wso.called(dev, zbytes)
    return (acc, toks) if events is None else (acc, toks, nl)


def read_probe(buf, out=None, *, stream: int | None = None):
    """The streaming-read probe (a measurement aid, not part of the method): reads every
    byte of the contiguous device tensor ``buf`` (a whole number of 32 KiB chunks) once and
    returns the per-chunk wrapping sums of its 32-bit words (uint32 values in an int32
    tensor of buf.nbytes // 32768 elements)."""
    import torch
    lib = load_library()
    n = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty((n // 32768,), dtype=torch.int32, device=buf.device)
    if stream is None:
        stream = torch.cuda.current_stream(buf.device).cuda_stream
    rc = lib.sv_read_probe(_ptr(buf), n, _ptr(out), ctypes.c_void_p(stream))
    if rc != 0:
        raise SpecVerifyError(rc, "sv_read_probe refused its arguments" if rc != 7 else "kernel launch failed")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature: float,
                        top_k: int = 0, *, out, row_stats=None, stream=None):
    """spec_verify through the allocation-free entry point (the library's per-GPU scratch
    array instead of a workspace).  ``out`` supplies the output tensors (accepted_len [B],
    out_tokens [B, G+1]) and ``row_stats`` optionally a [B, 2G+1, 2] float32 tensor, so that
    the call allocates nothing; calls that overlap on one GPU race (see the header)."""
    import torch
    lib = load_library()
    dev = target_logits.device
    dt = _dtype_code(target_logits)
    B, G1, V = target_logits.shape
    G = G1 - 1
    acc, toks = out
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    greedy = float(temperature) == 0.0
    args = [_ptr(target_logits), None if greedy else _ptr(draft_logits), dt, _ptr(draft_tokens),
            None if greedy else _ptr(u_accept), None if greedy else _ptr(u_sample), B, G, V,
            float(temperature), int(top_k), _ptr(acc), _ptr(toks), _ptr(row_stats), ctypes.c_void_p(stream)]
    st = lib.spec_verify_noalloc(*args)
    if st != 0:
        raise SpecVerifyError(st, sv_status_string(st))
    return acc, toks

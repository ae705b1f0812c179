"""ctypes binding of libdspark.so (the C ABI in include/dspark.h).

Argument marshalling only: shapes, dtypes and devices of torch tensors are checked, their
device pointers and the current HIP stream are handed to the library, and outputs and
workspaces are allocated with torch. Every step of the computation runs in the library's
kernels; there is no fallback, and loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdspark.so")

OK, ERR_INVALID_ARG, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP = range(5)
F32, BF16 = 0, 1
PATH_NAMES = {0: "sweep", 1: "mfma", 2: "resident", 3: "slab"}
GLOBAL, EARLY_STOP = 0, 1
DRAFT_PER_POSITION = 1
DRAFT_TEST_SPIN = 256
STS_NLL, STS_ECE = 0, 1

# every symbol include/dspark.h declares
EXPORTS = (
    "dspark_status_string", "dspark_last_error", "dspark_version",
    "dspark_markov_draft_path", "dspark_markov_draft_one_launch", "dspark_markov_draft_workspace_bytes",
    "dspark_markov_draft_plan", "dspark_noalloc_scratch_bytes", "dspark_markov_draft_noalloc",
    "dspark_rnn_draft_workspace_bytes", "dspark_rnn_draft_path", "dspark_rnn_draft",
    "dspark_markov_draft", "dspark_markov_draft_ex",
    "dspark_verify_workspace_bytes", "dspark_verify",
    "dspark_verify_tv_workspace_bytes", "dspark_verify_tv",
    "dspark_verify_markov_workspace_bytes", "dspark_verify_markov",
    "dspark_tv_labels_workspace_bytes", "dspark_tv_labels",
    "dspark_schedule_workspace_bytes", "dspark_schedule",
    "dspark_markov_draft_schedule_workspace_bytes", "dspark_markov_draft_schedule_fused",
    "dspark_markov_draft_schedule",
    "dspark_conf_ring_bytes", "dspark_conf_ring_init", "dspark_conf_ring_push", "dspark_schedule_lagged",
    "dspark_sts_fit_workspace_bytes", "dspark_sts_fit",
)

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t

_SIGS = {
    "dspark_status_string": (ctypes.c_char_p, [_I]),
    "dspark_last_error": (ctypes.c_char_p, []),
    "dspark_version": (_I, []),
    "dspark_markov_draft_path": (_I, [_I, _I, _I, _I, _P, _P]),
    "dspark_markov_draft_one_launch": (_I, [_I, _I, _I, _I, _P, _P, _I]),
    "dspark_markov_draft_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "dspark_markov_draft_plan": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P]),
    "dspark_noalloc_scratch_bytes": (_Z, []),
    "dspark_rnn_draft_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "dspark_rnn_draft_path": (_I, [_I, _I, _I, _P, _P, _P]),
    "dspark_rnn_draft": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "dspark_markov_draft_noalloc": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _I]),
    "dspark_markov_draft": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "dspark_markov_draft_ex": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _Z, _P, _I]),
    "dspark_verify_workspace_bytes": (_Z, [_I, _I, _I]),
    "dspark_verify": (_I, [_I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "dspark_verify_tv_workspace_bytes": (_Z, [_I, _I, _I]),
    "dspark_verify_tv": (_I, [_I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "dspark_verify_markov_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "dspark_verify_markov": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P,
                                  _P, _P, _P, _P, _P, _Z, _P]),
    "dspark_tv_labels_workspace_bytes": (_Z, [_I, _I, _I]),
    "dspark_tv_labels": (_I, [_I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "dspark_schedule_workspace_bytes": (_Z, [_I, _I, _I]),
    "dspark_schedule": (_I, [_I, _I, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "dspark_markov_draft_schedule_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I]),
    "dspark_markov_draft_schedule_fused": (_I, [_I, _I, _I, _I, _I, _P, _P, _I]),
    "dspark_markov_draft_schedule": (_I, [_I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P,
                                          _I, _P, _P, _Z, _P, _P, _I, _I, _P, _P, _P, _P, _P,
                                          _P, _Z, _P]),
    "dspark_conf_ring_bytes": (_Z, [_I, _I]),
    "dspark_conf_ring_init": (_I, [_I, _I, _P, _Z, _P]),
    "dspark_conf_ring_push": (_I, [_I, _I, _P, _Z, _P, _P]),
    "dspark_schedule_lagged": (_I, [_I, _I, _P, _Z, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "dspark_sts_fit_workspace_bytes": (_Z, [_I, _I, _I]),
    "dspark_sts_fit": (_I, [_I, _I, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
}

_lib = None
_lock = threading.Lock()


class DsparkError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


def load(path: str | None = None):
    """Load libdspark.so once; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            p = path or LIB_PATH
            if not os.path.exists(p):
                raise RuntimeError(f"{p} is missing: build it with "
                                   "`python -m draft_sampling_verification_head_amd.build`")
            lib = ctypes.CDLL(p)
            for name, (res, args) in _SIGS.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _check(status: int, where: str):
    if status != OK:
        lib = load()
        raise DsparkError(status, where, lib.dspark_last_error().decode())


# ----------------------------------------------------------------------------- torch helpers
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_ws_cache: dict = {}


def _stream_obj(stream=None):
    torch = _torch()
    return stream if stream is not None else torch.cuda.current_stream()


def workspace(nbytes: int, device, tag: str = "", stream=None, ws=None):
    """The workspace of one call: the caller's ``ws`` (a uint8 device tensor, checked for size
    and never replaced), or a cached buffer of at least nbytes per (device, stream, kind).
    Calls of one kind on one stream are stream-ordered, so they never overlap; calls on
    another stream get a buffer of their own. A cached buffer that must grow is replaced;
    the old one is freed only after the work queued on its stream (record_stream), but a
    graph captured over it would keep its address, so graph capture should pass ``ws``."""
    torch = _torch()
    if ws is not None:
        if ws.dtype != torch.uint8 or ws.device != torch.device(device) or ws.numel() < nbytes:
            raise ValueError(f"workspace must be a uint8 tensor on {device} of >= {nbytes} bytes")
        return ws
    s = _stream_obj(stream)
    key = (str(device), int(s.cuda_stream), tag)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(s):
            buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


# ----------------------------------------------------------------------------- entry points
def markov_draft_path(B: int, W1, W2) -> str:
    """Which kernel path markov_draft takes for B requests with these factors on the
    current device: "sweep", "slab", "mfma" or "resident" (see dspark_markov_draft_path)."""
    torch = _torch()
    V, r = W1.shape
    wdt = BF16 if W1.dtype == torch.bfloat16 else F32
    return PATH_NAMES[load().dspark_markov_draft_path(B, V, r, wdt, _ptr(W1), _ptr(W2))]


def markov_draft_one_launch(B: int, W1, W2, want_logits: bool = False) -> bool:
    """Whether markov_draft draws all positions in one launch (dspark_markov_draft_one_launch)."""
    torch = _torch()
    V, r = W1.shape
    wdt = BF16 if W1.dtype == torch.bfloat16 else F32
    return bool(load().dspark_markov_draft_one_launch(B, V, r, wdt, _ptr(W1), _ptr(W2), int(want_logits)))


def markov_draft_plan(U, W1, W2, Ld=None, per_position=False, test_spin=False):
    """dspark_markov_draft_plan: (path name, one launch, workspace bytes) of this exact call."""
    torch = _torch()
    B, G, V = U.shape
    r = W1.shape[1]
    wdt = BF16 if W1.dtype == torch.bfloat16 else F32
    opts = (DRAFT_PER_POSITION if per_position else 0) | (DRAFT_TEST_SPIN if test_spin else 0)
    path, one, nb = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    _check(load().dspark_markov_draft_plan(B, V, r, G, wdt, _ptr(W1), _ptr(W2), _ptr(U), _ptr(Ld), opts,
                                           ctypes.byref(path), ctypes.byref(one), ctypes.byref(nb)),
           "dspark_markov_draft_plan")
    return PATH_NAMES[path.value], bool(one.value), int(nb.value)


def draft_gave_up(ws) -> int:
    """The give-up count of the last one-launch draft call on workspace ``ws`` (bytes 0..3);
    synchronises with the device."""
    torch = _torch()
    return int(ws[:4].view(torch.int32).item())


def markov_draft(U, W1, W2, x0, u, *, want_q=True, want_lse=True, want_logits=False,
                 per_position=False, out=None, stream=None, ws=None, test_spin=False):
    """dspark_markov_draft (dspark_markov_draft_ex with DSPARK_DRAFT_PER_POSITION when
    per_position). U [B][gamma][V] fp32, W1 [V][r], W2 [r][V] (fp32 or bf16), x0 [B] int32,
    u [B][gamma] fp32. ``ws``: an explicit uint8 workspace (else a cached one); ``test_spin``:
    DSPARK_DRAFT_TEST_SPIN (failure injection). Returns dict x, q, lse, L (None when not
    asked)."""
    torch = _torch()
    lib = load()
    B, G, V = U.shape
    r = W1.shape[1]
    dev = U.device
    wdt = {torch.float32: F32, torch.bfloat16: BF16}.get(W1.dtype)
    if wdt is None:
        raise TypeError("W1/W2 must be float32 or bfloat16")
    _need(U, "U", torch.float32, (B, G, V), dev)
    _need(W1, "W1", W1.dtype, (V, r), dev)
    _need(W2, "W2", W1.dtype, (r, V), dev)
    _need(x0, "x0", torch.int32, (B,), dev)
    _need(u, "u", torch.float32, (B, G), dev)
    o = out or {}
    x = o.get("x") if o.get("x") is not None else torch.empty((B, G), dtype=torch.int32, device=dev)
    q = o.get("q") if o.get("q") is not None else (torch.empty((B, G), dtype=torch.float32, device=dev) if want_q else None)
    lse = o.get("lse") if o.get("lse") is not None else (torch.empty((B, G), dtype=torch.float32, device=dev) if want_lse else None)
    L = o.get("L") if o.get("L") is not None else (torch.empty((B, G, V), dtype=torch.float32, device=dev) if want_logits else None)
    opts = (DRAFT_PER_POSITION if per_position else 0) | (DRAFT_TEST_SPIN if test_spin else 0)
    _, _, nbytes = markov_draft_plan(U, W1, W2, L, per_position, test_spin)
    ws = workspace(nbytes, dev, "draft", stream, ws)
    st = lib.dspark_markov_draft_ex(B, V, r, G, _ptr(U), _ptr(W1), _ptr(W2), wdt, _ptr(x0), _ptr(u),
                                    _ptr(x), _ptr(q), _ptr(lse), _ptr(L), _ptr(ws), ws.numel(),
                                    _stream(stream), opts)
    _check(st, "dspark_markov_draft")
    return dict(x=x, q=q, lse=lse, L=L)


def rnn_draft_path(B: int, W1, W2, A) -> str:
    """dspark_rnn_draft_path: "resident" (one launch) or "mfma" (launches per position)."""
    V, r = W1.shape
    return PATH_NAMES[load().dspark_rnn_draft_path(B, V, r, _ptr(W1), _ptr(W2), _ptr(A))]


def rnn_draft(U, W1, W2, A, x0, u, *, want_q=True, want_lse=True, want_logits=False,
              want_state=False, stream=None, ws=None):
    """dspark_rnn_draft: the RNN-head draft (bf16 factors). U [B][gamma][V] fp32, W1 [V][r],
    W2 [r][V], A [r][r] bf16, x0 [B] int32, u [B][gamma] fp32. Returns dict x, q, lse, L, h."""
    torch = _torch()
    lib = load()
    B, G, V = U.shape
    r = W1.shape[1]
    dev = U.device
    if W1.dtype != torch.bfloat16:
        raise TypeError("rnn_draft needs bfloat16 factors")
    _need(U, "U", torch.float32, (B, G, V), dev)
    _need(W1, "W1", torch.bfloat16, (V, r), dev)
    _need(W2, "W2", torch.bfloat16, (r, V), dev)
    _need(A, "A", torch.bfloat16, (r, r), dev)
    _need(x0, "x0", torch.int32, (B,), dev)
    _need(u, "u", torch.float32, (B, G), dev)
    f32 = lambda shape: torch.empty(shape, dtype=torch.float32, device=dev)   # noqa: E731
    x = torch.empty((B, G), dtype=torch.int32, device=dev)
    q = f32((B, G)) if want_q else None
    lse = f32((B, G)) if want_lse else None
    L = f32((B, G, V)) if want_logits else None
    h = f32((B, G, r)) if want_state else None
    nbytes = lib.dspark_rnn_draft_workspace_bytes(B, V, r, G)
    ws = workspace(nbytes, dev, "rnn_draft", stream, ws)
    st = lib.dspark_rnn_draft(B, V, r, G, _ptr(U), _ptr(W1), _ptr(W2), _ptr(A), BF16, _ptr(x0), _ptr(u),
                              _ptr(x), _ptr(q), _ptr(lse), _ptr(L), _ptr(h), _ptr(ws), ws.numel(),
                              _stream(stream))
    _check(st, "dspark_rnn_draft")
    return dict(x=x, q=q, lse=lse, L=L, h=h)


def markov_draft_noalloc(U, W1, W2, x0, u, *, out, per_position=False, stream=None):
    """dspark_markov_draft_noalloc: the draft with the library's static scratch instead of a
    workspace. ``out`` holds the caller's output tensors (x required; q, lse, L optional);
    nothing is allocated here either. Returns ``out``."""
    torch = _torch()
    lib = load()
    B, G, V = U.shape
    r = W1.shape[1]
    dev = U.device
    wdt = {torch.float32: F32, torch.bfloat16: BF16}.get(W1.dtype)
    if wdt is None:
        raise TypeError("W1/W2 must be float32 or bfloat16")
    _need(U, "U", torch.float32, (B, G, V), dev)
    _need(W1, "W1", W1.dtype, (V, r), dev)
    _need(W2, "W2", W1.dtype, (r, V), dev)
    _need(x0, "x0", torch.int32, (B,), dev)
    _need(u, "u", torch.float32, (B, G), dev)
    _need(out["x"], "x", torch.int32, (B, G), dev)
    for k, shape in (("q", (B, G)), ("lse", (B, G)), ("L", (B, G, V))):
        if out.get(k) is not None:
            _need(out[k], k, torch.float32, shape, dev)
    st = lib.dspark_markov_draft_noalloc(B, V, r, G, _ptr(U), _ptr(W1), _ptr(W2), wdt, _ptr(x0),
                                         _ptr(u), _ptr(out["x"]), _ptr(out.get("q")),
                                         _ptr(out.get("lse")), _ptr(out.get("L")), _stream(stream),
                                         DRAFT_PER_POSITION if per_position else 0)
    _check(st, "dspark_markov_draft_noalloc")
    return out


def verify(Ld, Lt, x, u_acc, u_fin, *, t_off=None, length=None, ld_lse=None, want_lse=False,
           out=None, stream=None, with_tv=False, ws=None):
    """dspark_verify (dspark_verify_tv when with_tv). Ld [B][gamma][V], Lt [rows][V] fp32;
    x, u_acc [B][gamma]; u_fin [B]. Returns dict n [B], y [B][gamma+1] (and lse_d, lse_t when
    want_lse; cstar [B][gamma] when with_tv)."""
    torch = _torch()
    lib = load()
    B, G, V = Ld.shape
    dev = Ld.device
    _need(Ld, "Ld", torch.float32, (B, G, V), dev)
    if Lt.dim() != 2 or Lt.shape[1] != V:
        raise ValueError("Lt must be [rows][V]")
    _need(Lt, "Lt", torch.float32, tuple(Lt.shape), dev)
    _need(x, "x", torch.int32, (B, G), dev)
    _need(u_acc, "u_acc", torch.float32, (B, G), dev)
    _need(u_fin, "u_fin", torch.float32, (B,), dev)
    if t_off is not None:
        _need(t_off, "t_off", torch.int32, (B + 1,), dev)
    if length is not None:
        _need(length, "length", torch.int32, (B,), dev)
    if ld_lse is not None:
        _need(ld_lse, "ld_lse", torch.float32, (B, G), dev)
    o = out or {}
    n = o.get("n") if o.get("n") is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    y = o.get("y") if o.get("y") is not None else torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    lse_d, lse_t = o.get("lse_d"), o.get("lse_t")
    if want_lse and lse_d is None:
        lse_d = torch.empty((B, G), dtype=torch.float32, device=dev)
    if want_lse and lse_t is None:
        lse_t = torch.empty((B, G + 1), dtype=torch.float32, device=dev)
    if lse_d is not None:
        _need(lse_d, "lse_d", torch.float32, (B, G), dev)
    if lse_t is not None:
        _need(lse_t, "lse_t", torch.float32, (B, G + 1), dev)
    if with_tv:
        cstar = o.get("cstar") if o.get("cstar") is not None else torch.empty((B, G), dtype=torch.float32, device=dev)
        _need(cstar, "cstar", torch.float32, (B, G), dev)
        nbytes = lib.dspark_verify_tv_workspace_bytes(B, V, G)
        ws = workspace(nbytes, dev, "verify_tv", stream, ws)
        st = lib.dspark_verify_tv(B, V, G, _ptr(Ld), _ptr(Lt), int(Lt.shape[0]), _ptr(t_off),
                                  _ptr(length), _ptr(x), _ptr(ld_lse), _ptr(u_acc), _ptr(u_fin),
                                  _ptr(n), _ptr(y), _ptr(lse_d), _ptr(lse_t), _ptr(cstar),
                                  _ptr(ws), ws.numel(), _stream(stream))
        _check(st, "dspark_verify_tv")
        return dict(n=n, y=y, lse_d=lse_d, lse_t=lse_t, cstar=cstar)
    nbytes = lib.dspark_verify_workspace_bytes(B, V, G)
    ws = workspace(nbytes, dev, "verify", stream, ws)
    st = lib.dspark_verify(B, V, G, _ptr(Ld), _ptr(Lt), int(Lt.shape[0]), _ptr(t_off),
                           _ptr(length), _ptr(x), _ptr(ld_lse), _ptr(u_acc), _ptr(u_fin),
                           _ptr(n), _ptr(y), _ptr(lse_d), _ptr(lse_t), _ptr(ws), ws.numel(),
                           _stream(stream))
    _check(st, "dspark_verify")
    return dict(n=n, y=y, lse_d=lse_d, lse_t=lse_t)


def verify_markov(U, W1, W2, x0, x, ld_lse, Lt, u_acc, u_fin, *, t_off=None, length=None,
                  out=None, stream=None, ws=None):
    """dspark_verify_markov: verify + TV labels with the draft logits rebuilt from U, W1, W2
    (bf16 factors). U [B][gamma][V] fp32, x0 [B], x [B][gamma] int32, ld_lse [B][gamma] from the
    draft, Lt [rows][V] fp32, u_acc [B][gamma], u_fin [B]. Returns dict n, y, lse_t, cstar."""
    torch = _torch()
    lib = load()
    B, G, V = U.shape
    r = W1.shape[1]
    dev = U.device
    if W1.dtype != torch.bfloat16:
        raise TypeError("verify_markov needs bfloat16 factors")
    _need(U, "U", torch.float32, (B, G, V), dev)
    _need(W1, "W1", torch.bfloat16, (V, r), dev)
    _need(W2, "W2", torch.bfloat16, (r, V), dev)
    _need(x0, "x0", torch.int32, (B,), dev)
    _need(x, "x", torch.int32, (B, G), dev)
    _need(ld_lse, "ld_lse", torch.float32, (B, G), dev)
    if Lt.dim() != 2 or Lt.shape[1] != V:
        raise ValueError("Lt must be [rows][V]")
    _need(Lt, "Lt", torch.float32, tuple(Lt.shape), dev)
    _need(u_acc, "u_acc", torch.float32, (B, G), dev)
    _need(u_fin, "u_fin", torch.float32, (B,), dev)
    if t_off is not None:
        _need(t_off, "t_off", torch.int32, (B + 1,), dev)
    if length is not None:
        _need(length, "length", torch.int32, (B,), dev)
    o = out or {}
    n = o.get("n") if o.get("n") is not None else torch.empty((B,), dtype=torch.int32, device=dev)
    y = o.get("y") if o.get("y") is not None else torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    lse_t = o.get("lse_t") if o.get("lse_t") is not None else torch.empty((B, G + 1), dtype=torch.float32, device=dev)
    cstar = o.get("cstar") if o.get("cstar") is not None else torch.empty((B, G), dtype=torch.float32, device=dev)
    _need(lse_t, "lse_t", torch.float32, (B, G + 1), dev)
    _need(cstar, "cstar", torch.float32, (B, G), dev)
    nbytes = lib.dspark_verify_markov_workspace_bytes(B, V, r, G)
    ws = workspace(nbytes, dev, "verify_markov", stream, ws)
    st = lib.dspark_verify_markov(B, V, r, G, _ptr(U), _ptr(W1), _ptr(W2), BF16, _ptr(x0), _ptr(x),
                                  _ptr(ld_lse), _ptr(Lt), int(Lt.shape[0]), _ptr(t_off),
                                  _ptr(length), _ptr(u_acc), _ptr(u_fin), _ptr(n), _ptr(y),
                                  _ptr(lse_t), _ptr(cstar), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "dspark_verify_markov")
    return dict(n=n, y=y, lse_t=lse_t, cstar=cstar)


def tv_labels(Ld, Lt, *, t_off=None, length=None, lse_d=None, lse_t=None, out=None, stream=None,
              ws=None):
    """dspark_tv_labels. Returns c* [B][gamma] (NaN beyond each request's length)."""
    torch = _torch()
    lib = load()
    B, G, V = Ld.shape
    dev = Ld.device
    _need(Ld, "Ld", torch.float32, (B, G, V), dev)
    if Lt.dim() != 2 or Lt.shape[1] != V:
        raise ValueError("Lt must be [rows][V]")
    _need(Lt, "Lt", torch.float32, tuple(Lt.shape), dev)
    if t_off is not None:
        _need(t_off, "t_off", torch.int32, (B + 1,), dev)
    if length is not None:
        _need(length, "length", torch.int32, (B,), dev)
    if lse_d is not None:
        _need(lse_d, "lse_d", torch.float32, (B, G), dev)
    if lse_t is not None:
        _need(lse_t, "lse_t", torch.float32, (B, G + 1), dev)
    c = out if out is not None else torch.empty((B, G), dtype=torch.float32, device=dev)
    nbytes = lib.dspark_tv_labels_workspace_bytes(B, V, G)
    ws = workspace(nbytes, dev, "tv", stream, ws)
    st = lib.dspark_tv_labels(B, V, G, _ptr(Ld), _ptr(Lt), int(Lt.shape[0]), _ptr(t_off),
                              _ptr(length), _ptr(lse_d), _ptr(lse_t), _ptr(c), _ptr(ws),
                              ws.numel(), _stream(stream))
    _check(st, "dspark_tv_labels")
    return c


def _schedule_outputs(R, G, dev, out, want_a):
    torch = _torch()
    o = out or {}
    length = o.get("len") if o.get("len") is not None else torch.empty((R,), dtype=torch.int32, device=dev)
    t_off = o.get("t_off") if o.get("t_off") is not None else torch.empty((R + 1,), dtype=torch.int32, device=dev)
    K = o.get("K") if o.get("K") is not None else torch.empty((1,), dtype=torch.int32, device=dev)
    theta = o.get("theta") if o.get("theta") is not None else torch.empty((1,), dtype=torch.float32, device=dev)
    a = o.get("a") if o.get("a") is not None else (torch.empty((R, G), dtype=torch.float32, device=dev)
                                                   if want_a else None)
    return dict(len=length, t_off=t_off, K=K, theta=theta, a=a)


def schedule(conf, sps, Bmax, *, temp=None, mode=GLOBAL, want_a=False, out=None, stream=None,
             ws=None):
    """dspark_schedule. conf [R][gamma] fp32, sps [Bmax+1] fp32, temp [gamma] fp32 or None.
    Returns dict len [R], t_off [R+1], K [1], theta [1] (and a [R][gamma] when want_a)."""
    torch = _torch()
    lib = load()
    R, G = conf.shape
    dev = conf.device
    _need(conf, "conf", torch.float32, (R, G), dev)
    _need(sps, "sps", torch.float32, (Bmax + 1,), dev)
    if temp is not None:
        _need(temp, "temp", torch.float32, (G,), dev)
    o = _schedule_outputs(R, G, dev, out, want_a)
    ws = workspace(lib.dspark_schedule_workspace_bytes(R, G, int(Bmax)), dev, "schedule", stream, ws)
    st = lib.dspark_schedule(R, G, _ptr(conf), _ptr(temp), _ptr(sps), int(Bmax), int(mode),
                             _ptr(o["len"]), _ptr(o["t_off"]), _ptr(o["K"]), _ptr(o["theta"]),
                             _ptr(o["a"]), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "dspark_schedule")
    return o


def markov_draft_schedule_fused(B: int, W1, W2, R: int, gamma: int) -> bool:
    """dspark_markov_draft_schedule_fused: whether markov_draft_schedule runs the schedule in
    the draft's launch."""
    torch = _torch()
    V, r = W1.shape
    wdt = {torch.float32: F32, torch.bfloat16: BF16}[W1.dtype]
    return bool(load().dspark_markov_draft_schedule_fused(B, V, r, gamma, wdt, _ptr(W1), _ptr(W2), R))


def markov_draft_schedule(U, W1, W2, x0, u, sps, Bmax, *, conf=None, ring=None, temp=None,
                          mode=GLOBAL, want_q=True, want_lse=True, want_logits=False,
                          want_a=False, out=None, out_sched=None, stream=None, ws=None):
    """dspark_markov_draft_schedule: the draft of markov_draft and the schedule of schedule
    (conf [R][gamma]) or schedule_lagged (ring, a ConfRing) in one call. Returns (draft dict,
    schedule dict) as those two calls return them."""
    torch = _torch()
    lib = load()
    B, G, V = U.shape
    r = W1.shape[1]
    dev = U.device
    wdt = {torch.float32: F32, torch.bfloat16: BF16}.get(W1.dtype)
    if wdt is None:
        raise TypeError("W1/W2 must be float32 or bfloat16")
    _need(U, "U", torch.float32, (B, G, V), dev)
    _need(W1, "W1", W1.dtype, (V, r), dev)
    _need(W2, "W2", W1.dtype, (r, V), dev)
    _need(x0, "x0", torch.int32, (B,), dev)
    _need(u, "u", torch.float32, (B, G), dev)
    if (conf is None) == (ring is None):
        raise ValueError("give exactly one of conf and ring")
    if ring is not None:
        R = ring.R
        if ring.gamma != G:
            raise ValueError("the ring's gamma differs from the draft's")
    else:
        R = conf.shape[0]
        _need(conf, "conf", torch.float32, (R, G), dev)
    _need(sps, "sps", torch.float32, (Bmax + 1,), dev)
    if temp is not None:
        _need(temp, "temp", torch.float32, (G,), dev)
    o = out or {}
    x = o.get("x") if o.get("x") is not None else torch.empty((B, G), dtype=torch.int32, device=dev)
    q = o.get("q") if o.get("q") is not None else (torch.empty((B, G), dtype=torch.float32, device=dev) if want_q else None)
    lse = o.get("lse") if o.get("lse") is not None else (torch.empty((B, G), dtype=torch.float32, device=dev) if want_lse else None)
    L = o.get("L") if o.get("L") is not None else (torch.empty((B, G, V), dtype=torch.float32, device=dev) if want_logits else None)
    so = _schedule_outputs(R, G, dev, out_sched, want_a)
    nbytes = lib.dspark_markov_draft_schedule_workspace_bytes(B, V, r, G, R, int(Bmax))
    ws = workspace(nbytes, dev, "draft_schedule", stream, ws)
    st = lib.dspark_markov_draft_schedule(
        B, V, r, G, _ptr(U), _ptr(W1), _ptr(W2), wdt, _ptr(x0), _ptr(u), _ptr(x), _ptr(q),
        _ptr(lse), _ptr(L), R, _ptr(conf), _ptr(ring.buf if ring is not None else None),
        ring.nbytes if ring is not None else 0, _ptr(temp), _ptr(sps), int(Bmax), int(mode),
        _ptr(so["len"]), _ptr(so["t_off"]), _ptr(so["K"]), _ptr(so["theta"]), _ptr(so["a"]),
        _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "dspark_markov_draft_schedule")
    return dict(x=x, q=q, lse=lse, L=L), so


class ConfRing:
    """Two-step-lag confidence history (dspark_conf_ring_*): one device buffer holding a
    round counter and three [R][gamma] fp32 slots, initialised to "no history" (all 1.0)."""

    def __init__(self, R: int, gamma: int, device=None, stream=None):
        torch = _torch()
        self.R, self.gamma = int(R), int(gamma)
        self.nbytes = int(load().dspark_conf_ring_bytes(self.R, self.gamma))
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device or "cuda")
        self.reset(stream)

    def reset(self, stream=None):
        """dspark_conf_ring_init: counter 0, every slot 1.0."""
        _check(load().dspark_conf_ring_init(self.R, self.gamma, _ptr(self.buf), self.nbytes,
                                            _stream(stream)), "dspark_conf_ring_init")

    def push(self, conf, stream=None):
        """dspark_conf_ring_push: this round's confidences [R][gamma] fp32."""
        torch = _torch()
        _need(conf, "conf", torch.float32, (self.R, self.gamma), self.buf.device)
        _check(load().dspark_conf_ring_push(self.R, self.gamma, _ptr(self.buf), self.nbytes,
                                            _ptr(conf), _stream(stream)), "dspark_conf_ring_push")

    def rounds(self) -> int:
        """The device counter (pushes so far); synchronises with the device."""
        return int(self.buf[:8].view(_torch().int64).item())


def schedule_lagged(ring: ConfRing, sps, Bmax, *, temp=None, mode=GLOBAL, want_a=False, out=None,
                    stream=None, ws=None):
    """dspark_schedule_lagged: dspark_schedule on the confidences pushed two rounds ago."""
    torch = _torch()
    lib = load()
    R, G, dev = ring.R, ring.gamma, ring.buf.device
    _need(sps, "sps", torch.float32, (Bmax + 1,), dev)
    if temp is not None:
        _need(temp, "temp", torch.float32, (G,), dev)
    o = _schedule_outputs(R, G, dev, out, want_a)
    ws = workspace(lib.dspark_schedule_workspace_bytes(R, G, int(Bmax)), dev, "schedule", stream, ws)
    st = lib.dspark_schedule_lagged(R, G, _ptr(ring.buf), ring.nbytes, _ptr(temp), _ptr(sps),
                                    int(Bmax), int(mode), _ptr(o["len"]), _ptr(o["t_off"]),
                                    _ptr(o["K"]), _ptr(o["theta"]), _ptr(o["a"]), _ptr(ws),
                                    ws.numel(), _stream(stream))
    _check(st, "dspark_schedule_lagged")
    return o


def sts_fit(conf, n_acc, grid, *, length=None, bins=15, objective=STS_NLL, want_obj=False,
            stream=None, ws=None):
    """dspark_sts_fit. conf [N][gamma] fp32, n_acc [N] int32 (and length [N] int32) from
    verify, grid [n_grid] fp32. Returns dict T, ece_before, ece_after [gamma] (and obj
    [gamma][n_grid] when want_obj)."""
    torch = _torch()
    lib = load()
    N, G = conf.shape
    dev = conf.device
    _need(conf, "conf", torch.float32, (N, G), dev)
    _need(n_acc, "n_acc", torch.int32, (N,), dev)
    if length is not None:
        _need(length, "length", torch.int32, (N,), dev)
    nT = grid.shape[0]
    _need(grid, "grid", torch.float32, (nT,), dev)
    T = torch.empty(G, dtype=torch.float32, device=dev)
    eb = torch.empty(G, dtype=torch.float32, device=dev)
    ea = torch.empty(G, dtype=torch.float32, device=dev)
    obj = torch.empty((G, nT), dtype=torch.float32, device=dev) if want_obj else None
    nbytes = lib.dspark_sts_fit_workspace_bytes(N, G, nT)
    ws = workspace(nbytes, dev, "sts", stream, ws)
    st = lib.dspark_sts_fit(N, G, _ptr(conf), _ptr(n_acc), _ptr(length), _ptr(grid), nT, bins,
                            objective, _ptr(T), _ptr(eb), _ptr(ea), _ptr(obj), _ptr(ws),
                            ws.numel(), _stream(stream))
    _check(st, "dspark_sts_fit")
    return dict(T=T, ece_before=eb, ece_after=ea, obj=obj)

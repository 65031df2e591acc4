"""Python binding of libgq.so (C ABI in include/gq.h).

Argument marshalling only: torch tensors supply device memory and the HIP
stream; every step of the computation runs in the library's kernels.  Each
function has the name of the C entry point it calls.  A non-OK status raises
GQError(status, message).  If the built library is missing, loading raises.
GQ_LIBRARY=<path> loads another build of the same library instead (for instance the
host-sanitized libgq_asan.so, see build.py).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.environ.get("GQ_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "_lib", "libgq.so")

GQ_OK, GQ_EINVAL, GQ_ESHAPE, GQ_EDTYPE, GQ_ENOMEM, GQ_EHIP = 0, 1, 2, 3, 4, 5
GQ_ENOTPD, GQ_ENONFINITE, GQ_ENOTIMPL, GQ_ECHECK = 6, 7, 8, 9
GQ_F32, GQ_BF16 = 0, 1
GQ_INIT_QUANTILE, GQ_INIT_GIVEN, GQ_INIT_UNIFORM = 0, 1, 2
GQ_GRAM_AUTO, GQ_GRAM_DENSE = 0, 1
GQ_FISHER_CHECK_FINITE = 2
ABI_VERSION = 8
DEFAULT_BLOCK = 512

# every symbol include/gq.h declares
EXPORTS = (
    "gq_abi_version", "gq_last_error", "gq_lnq_options_default", "lnq_options_default",
    "gq_fisher_workspace_size", "gq_fisher_accumulate", "gq_lnq_workspace_size",
    "lnq_workspace_size", "lnq_codebook_update", "lnq_assign_sweep",
    "lnq_objective", "lnq_quantize", "lnq_quantize_static", "lnq_static_scratch_bytes",
    "grid_quantize", "lut_packed_row_words", "lut_pack_codes",
    "lut_gemv", "gq_fisher_stream_workspace_size", "gq_fisher_accumulate_host",
    "ganq_workspace_size", "ganq_quantize", "ganq_factor_damped",
    "gq_timing_enable", "gq_timing_read", "gq_stage_name",
)
STAGE_COUNT = 18


class GQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libgq status {status}: {message}")
        self.status = status
        self.message = message


class lnq_options(ctypes.Structure):
    """gq_lnq_options (block, ridge_rel, init, gram_update, ridge_abs, check_finite,
    check_residual)."""
    _fields_ = [("block", ctypes.c_int32), ("ridge_rel", ctypes.c_float),
                ("init", ctypes.c_int32), ("gram_update", ctypes.c_int32),
                ("ridge_abs", ctypes.c_float), ("check_finite", ctypes.c_int32),
                ("check_residual", ctypes.c_int32)]


_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float

_SIGS = {
    "gq_abi_version": (ctypes.c_int, []),
    "gq_last_error": (ctypes.c_char_p, []),
    "gq_lnq_options_default": (None, [ctypes.POINTER(lnq_options)]),
    "lnq_options_default": (None, [ctypes.POINTER(lnq_options)]),
    "gq_fisher_workspace_size": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "gq_fisher_accumulate": (ctypes.c_int, [_vp, _i32, _i64, _i64, _vp, _i32, _i64, _i32, _vp,
                                            _i32, _vp, _sz, _vp]),
    "gq_lnq_workspace_size": (_sz, [_i64, _i64, _i32, _i32, _i32]),
    "lnq_workspace_size": (_sz, [_i64, _i64, _i32, _i32, _i32]),
    "lnq_codebook_update": (ctypes.c_int, [_vp, _i32, _i64, _vp, _i32, _i64, _vp, _i32, _vp, _f32,
                                           _vp, _vp, _sz, _vp]),
    "lnq_assign_sweep": (ctypes.c_int, [_vp, _i32, _i64, _vp, _i32, _i64, _vp, _i32, _vp, _f32,
                                        _i32, _vp, _vp, _sz, _vp]),
    "lnq_objective": (ctypes.c_int, [_vp, _i32, _i64, _vp, _i32, _i64, _vp, _vp, _i32, _f32, _vp,
                                     _vp, _vp, _sz, _vp]),
    "lnq_quantize": (ctypes.c_int, [_vp, _i32, _i64, _i64, _vp, _i32, _i32, _i32,
                                    ctypes.POINTER(lnq_options), _vp, _vp, _vp, _vp, _vp, _sz,
                                    _vp]),
    "lnq_quantize_static": (ctypes.c_int, [_vp, _i32, _i64, _i64, _vp, _i32, _i32, _i32,
                                           ctypes.POINTER(lnq_options), _vp, _vp, _vp, _vp,
                                           _vp]),
    "lnq_static_scratch_bytes": (_sz, []),
    "grid_quantize": (ctypes.c_int, [_vp, _i32, _i64, _i64, _vp, _i32, _i32, _i32,
                                     ctypes.POINTER(lnq_options), _vp, _vp, _vp, _vp, _vp, _sz,
                                     _vp]),
    "lut_packed_row_words": (_i64, [_i64, _i32]),
    "lut_pack_codes": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "lut_gemv": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i32, _vp, _i32, _i32, _vp, _vp]),
    "gq_fisher_stream_workspace_size": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "gq_fisher_accumulate_host": (ctypes.c_int, [_vp, _i32, _i64, _i64, _vp, _i32, _i64, _i32,
                                                 _vp, _i32, _i64, _vp, _sz, _vp]),
    "ganq_workspace_size": (_sz, [_i64, _i64, _i32, _i32, _i32]),
    "ganq_quantize": (ctypes.c_int, [_vp, _i32, _i64, _i64, _vp, _i32, _i32, _i32,
                                     ctypes.POINTER(lnq_options), _vp, _vp, _vp, _vp, _vp, _vp,
                                     _sz, _vp]),
    "ganq_factor_damped": (ctypes.c_int, [_vp, _i32, _i64, _f32, _vp, _vp, _vp, _sz, _vp]),
    "gq_timing_enable": (None, [ctypes.c_int]),
    "gq_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "gq_stage_name": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


def library(path: str | None = None) -> ctypes.CDLL:
    """Load libgq.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise GQError(GQ_ENOTIMPL, f"{p} is missing: build it with "
                                   "`python -m post_weight_quantization_gq_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.gq_abi_version() != ABI_VERSION:
        raise GQError(GQ_ENOTIMPL, "libgq ABI version mismatch")
    _lib = lib
    return lib


def _check(status: int):
    if status != GQ_OK:
        raise GQError(status, library().gq_last_error().decode(errors="replace"))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GQ_F32
    if t.dtype == torch.bfloat16:
        return GQ_BF16
    raise GQError(GQ_EDTYPE, f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise GQError(GQ_EINVAL, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise GQError(GQ_EINVAL, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise GQError(GQ_EDTYPE, f"{name} must be {dtype}, got {t.dtype}")
    return t


def _shape(t, shape, name):
    """GQ_ESHAPE unless tensor t has exactly this shape (checked before any launch: the
    C ABI sees only pointers, so a mis-shaped buffer would be read or written out of
    bounds on the device)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise GQError(GQ_ESHAPE, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _counter(t, name, n=1):
    """Optional device counter: int64 with at least n elements (its device is checked
    with the other tensors)."""
    if t is None:
        return
    if t.dtype != torch.int64 or t.numel() < n:
        raise GQError(GQ_ESHAPE, f"{name} must be an int64 tensor of at least {n} element(s)")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise GQError(GQ_EINVAL, f"tensors on different devices: {sorted(map(str, devs))}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ws(nbytes: int, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ws_arg(ws):
    """(pointer, bytes) of a workspace tensor; ws=False passes NULL, which makes the
    library allocate its scratch stream-ordered (hipMallocAsync / hipFreeAsync)."""
    if ws is False or ws is None:
        return None, 0
    return _ptr(ws), ws.numel()


def abi_version() -> int:
    return library().gq_abi_version()


def options(block: int = DEFAULT_BLOCK, ridge_rel: float = 1e-6, init: int = GQ_INIT_QUANTILE,
            gram_update: int = GQ_GRAM_AUTO, ridge_abs: float = 0.0,
            check_finite: bool = False, check_residual: bool = False) -> lnq_options:
    o = lnq_options()
    library().gq_lnq_options_default(ctypes.byref(o))
    o.block, o.ridge_rel, o.init, o.gram_update = block, ridge_rel, init, gram_update
    o.ridge_abs, o.check_finite = ridge_abs, int(bool(check_finite))
    o.check_residual = int(bool(check_residual))
    return o


def fisher_workspace_size(n, d_in, d_out, groups, dtype=GQ_BF16) -> int:
    return int(library().gq_fisher_workspace_size(n, d_in, d_out, groups, dtype))


def lnq_workspace_size(d_out, d_in, groups, bits, w_dtype=GQ_BF16) -> int:
    return int(library().gq_lnq_workspace_size(d_out, d_in, groups, bits, w_dtype))


def gq_fisher_accumulate(X, G, groups: int, F=None, accumulate: bool = False, ws=None,
                         stream=None, check_finite: bool = False) -> torch.Tensor:
    """F[g] (=|+=) X^T diag(s_g) X; X [n][d_in], G [n][d_out] (float32 or bfloat16).
    check_finite: scan X and G for NaN / Inf first (GQError GQ_ENONFINITE, F untouched;
    the call then synchronises the stream)."""
    lib = library()
    if X.dim() != 2 or G.dim() != 2:
        raise GQError(GQ_ESHAPE, "X and G must be 2-D")
    n, d_in = X.shape
    d_out = G.shape[1]
    if G.shape[0] != n:
        raise GQError(GQ_ESHAPE, "X and G need the same number of tokens")
    _shape(F, (groups, d_in, d_in), "F")
    _dev(X, "X")
    _dev(G, "G")
    if F is None:
        F = torch.empty((groups, d_in, d_in), dtype=torch.float32, device=X.device)
        if accumulate:
            raise GQError(GQ_EINVAL, "accumulate needs an existing F")
    _dev(F, "F", torch.float32)
    _same_device(X, G, F, ws if isinstance(ws, torch.Tensor) else None)
    if ws is None:
        ws = _ws(fisher_workspace_size(n, d_in, d_out, groups, _dt(X)), X.device)
    wp, wn = _ws_arg(ws)
    flags = int(bool(accumulate)) | (GQ_FISHER_CHECK_FINITE if check_finite else 0)
    _check(lib.gq_fisher_accumulate(_ptr(X), _dt(X), n, d_in, _ptr(G), _dt(G), d_out, groups,
                                    _ptr(F), flags, wp, wn, _stream(stream)))
    return F


fisher = gq_fisher_accumulate


def _lnq_common(F, W, groups, bits=None, C=None, P=None):
    """Shapes first (no device needed), then device, dtype and contiguity."""
    if W.dim() != 2 or F.dim() != 3:
        raise GQError(GQ_ESHAPE, "W must be 2-D and F 3-D")
    d_out, d_in = W.shape
    _shape(F, (groups, d_in, d_in), "F")
    if bits is not None:
        _shape(C, (d_out, 1 << bits), "C")
        _shape(P, (d_out, d_in), "P")
    _dev(F, "F", torch.float32)
    _dev(W, "W")
    if C is not None:
        _dev(C, "C", torch.float32)
    if P is not None:
        _dev(P, "P", torch.uint8)
    _same_device(F, W, C, P)
    return d_out, d_in


def _lnq_ws(ws, d_out, d_in, groups, bits, W):
    if ws is None:
        ws = _ws(lnq_workspace_size(d_out, d_in, groups, bits, _dt(W)), W.device)
    elif ws is not False:
        _same_device(W, ws)
    return _ws_arg(ws)


def lnq_codebook_update(F, W, P, C, bits: int, ridge_rel: float = 1e-6, n_not_pd=None,
                        ws=None, stream=None) -> torch.Tensor:
    """One codebook step; C [d_out][2^bits] float32 is updated in place."""
    lib = library()
    groups = F.shape[0]
    _counter(n_not_pd, "n_not_pd")
    d_out, d_in = _lnq_common(F, W, groups, bits, C, P)
    if n_not_pd is not None:
        _dev(n_not_pd, "n_not_pd")
        _same_device(W, n_not_pd)
    wp, nb = _lnq_ws(ws, d_out, d_in, groups, bits, W)
    _check(lib.lnq_codebook_update(_ptr(F), groups, d_in, _ptr(W), _dt(W), d_out, _ptr(P), bits,
                                   _ptr(C), ridge_rel, _ptr(n_not_pd), wp, nb,
                                   _stream(stream)))
    return C


def lnq_assign_sweep(F, W, C, P, bits: int, ridge_rel: float = 1e-6,
                     block: int = DEFAULT_BLOCK, n_changed=None, ws=None,
                     stream=None) -> torch.Tensor:
    """One assignment pass; P [d_out][d_in] uint8 is updated in place."""
    lib = library()
    groups = F.shape[0]
    _counter(n_changed, "n_changed")
    d_out, d_in = _lnq_common(F, W, groups, bits, C, P)
    if n_changed is not None:
        _dev(n_changed, "n_changed")
        _same_device(W, n_changed)
    wp, nb = _lnq_ws(ws, d_out, d_in, groups, bits, W)
    _check(lib.lnq_assign_sweep(_ptr(F), groups, d_in, _ptr(W), _dt(W), d_out, _ptr(C), bits,
                                _ptr(P), ridge_rel, block, _ptr(n_changed), wp, nb,
                                _stream(stream)))
    return P


def lnq_objective(F, W, C, P, bits: int, ridge_rel: float = 1e-6, obj_total=None, ws=None,
                  stream=None) -> torch.Tensor:
    """Per-row objectives e_j^T F' e_j (float64 [d_out])."""
    lib = library()
    groups = F.shape[0]
    if obj_total is not None and (obj_total.dtype != torch.float64 or obj_total.numel() < 1):
        raise GQError(GQ_ESHAPE, "obj_total must be a float64 tensor of at least one element")
    d_out, d_in = _lnq_common(F, W, groups, bits, C, P)
    if obj_total is not None:
        _dev(obj_total, "obj_total")
        _same_device(W, obj_total)
    rows = torch.empty(d_out, dtype=torch.float64, device=W.device)
    wp, nb = _lnq_ws(ws, d_out, d_in, groups, bits, W)
    _check(lib.lnq_objective(_ptr(F), groups, d_in, _ptr(W), _dt(W), d_out, _ptr(C), _ptr(P),
                             bits, ridge_rel, _ptr(rows), _ptr(obj_total), wp, nb,
                             _stream(stream)))
    return rows


def _outputs(W, d_out, d_in, bits, C, P):
    m = 1 << bits
    if C is None:
        C = torch.empty((d_out, m), dtype=torch.float32, device=W.device)
    if P is None:
        P = torch.empty((d_out, d_in), dtype=torch.uint8, device=W.device)
    return C, P


def lnq_quantize(W, F, bits: int, iters: int, block: int = DEFAULT_BLOCK,
                 ridge_rel: float = 1e-6, C=None, P=None, init: int | None = None,
                 trace: bool = True, ws=None, stream=None, gram_update: int = GQ_GRAM_AUTO,
                 ridge_abs: float = 0.0, check_finite: bool = False,
                 check_residual: bool = False):
    """Whole LNQ on a layer.  Returns (C, P, obj_trace or None, n_changed).

    With C and P given and init unset, starts from them (GQ_INIT_GIVEN).
    ridge_abs: fixed ridge added to ridge_rel * mean(diag F_g).  check_finite: a checked
    call (GQ_ENONFINITE for NaN / Inf in W or F before anything is written, GQ_ENOTPD
    after the run if a codebook system was not positive definite).  ws=False lets the
    library allocate its scratch.  check_residual: the debug check of every assignment
    pass against a fresh F'(C[P] - W) (GQError GQ_ECHECK on a mismatch).
    """
    lib = library()
    groups = F.shape[0]
    if init is None:
        init = GQ_INIT_GIVEN if (C is not None and P is not None) else GQ_INIT_QUANTILE
    d_out, d_in = _lnq_common(F, W, groups, bits, C, P)
    C, P = _outputs(W, d_out, d_in, bits, C, P)
    tr = torch.empty(2 * iters + 1, dtype=torch.float64, device=W.device) if trace else None
    nch = torch.zeros(max(iters, 1), dtype=torch.int64, device=W.device)
    opt = options(block, ridge_rel, init, gram_update, ridge_abs, check_finite, check_residual)
    wp, nb = _lnq_ws(ws, d_out, d_in, groups, bits, W)
    _check(lib.lnq_quantize(_ptr(W), _dt(W), d_out, d_in, _ptr(F), groups, bits, iters,
                            ctypes.byref(opt), _ptr(C), _ptr(P), _ptr(tr), _ptr(nch), wp,
                            nb, _stream(stream)))
    return C, P, tr, nch[:iters]


def lnq_quantize_static(W, F, bits: int, iters: int, block: int = DEFAULT_BLOCK,
                        ridge_rel: float = 1e-6, C=None, P=None, init: int | None = None,
                        trace: bool = True, stream=None, gram_update: int = GQ_GRAM_AUTO,
                        ridge_abs: float = 0.0, check_finite: bool = False,
                        check_residual: bool = False):
    """lnq_quantize on the library's fixed per-device scratch (no workspace, nothing
    allocated by the library; the outputs are still the caller's).  Calls that overlap
    on one device race.  Returns (C, P, obj_trace or None, n_changed)."""
    lib = library()
    groups = F.shape[0]
    if init is None:
        init = GQ_INIT_GIVEN if (C is not None and P is not None) else GQ_INIT_QUANTILE
    d_out, d_in = _lnq_common(F, W, groups, bits, C, P)
    C, P = _outputs(W, d_out, d_in, bits, C, P)
    tr = torch.empty(2 * iters + 1, dtype=torch.float64, device=W.device) if trace else None
    nch = torch.zeros(max(iters, 1), dtype=torch.int64, device=W.device)
    opt = options(block, ridge_rel, init, gram_update, ridge_abs, check_finite, check_residual)
    _check(lib.lnq_quantize_static(_ptr(W), _dt(W), d_out, d_in, _ptr(F), groups, bits, iters,
                                   ctypes.byref(opt), _ptr(C), _ptr(P), _ptr(tr), _ptr(nch),
                                   _stream(stream)))
    return C, P, tr, nch[:iters]


def lnq_static_scratch_bytes() -> int:
    return int(library().lnq_static_scratch_bytes())


def grid_quantize(W, F, bits: int, iters: int, block: int = DEFAULT_BLOCK,
                  ridge_rel: float = 1e-6, C=None, P=None, init: int | None = None,
                  trace: bool = True, ws=None, stream=None, ridge_abs: float = 0.0,
                  check_finite: bool = False, check_residual: bool = False):
    """Fixed-grid backend: uniform grid per row, `iters` assignment passes.

    Returns (C, P, obj_trace [iters+1] or None, n_changed [iters]).  With C and P
    given and init unset, starts from them (GQ_INIT_GIVEN).
    """
    lib = library()
    groups = F.shape[0]
    if init is None:
        init = GQ_INIT_GIVEN if (C is not None and P is not None) else GQ_INIT_UNIFORM
    d_out, d_in = _lnq_common(F, W, groups, bits, C, P)
    C, P = _outputs(W, d_out, d_in, bits, C, P)
    tr = torch.empty(iters + 1, dtype=torch.float64, device=W.device) if trace else None
    nch = torch.zeros(max(iters, 1), dtype=torch.int64, device=W.device)
    opt = options(block, ridge_rel, init, GQ_GRAM_AUTO, ridge_abs, check_finite, check_residual)
    wp, nb = _lnq_ws(ws, d_out, d_in, groups, bits, W)
    _check(lib.grid_quantize(_ptr(W), _dt(W), d_out, d_in, _ptr(F), groups, bits, iters,
                             ctypes.byref(opt), _ptr(C), _ptr(P), _ptr(tr), _ptr(nch), wp,
                             nb, _stream(stream)))
    return C, P, tr, nch[:iters]


def fisher_stream_workspace_size(chunk_tokens, d_in, d_out, groups, dtype=GQ_BF16) -> int:
    return int(library().gq_fisher_stream_workspace_size(chunk_tokens, d_in, d_out, groups,
                                                          dtype))


def gq_fisher_accumulate_host(X, G, groups: int, F=None, accumulate: bool = False,
                              chunk_tokens: int = 16384, ws=None, stream=None,
                              device=None) -> torch.Tensor:
    """F[g] (=|+=) X^T diag(s_g) X with X [n][d_in], G [n][d_out] in HOST memory (CPU
    tensors, pinned for asynchronous copies), streamed to the GPU in chunks of tokens."""
    lib = library()
    for t, name in ((X, "X"), (G, "G")):
        if t.device.type != "cpu" or not t.is_contiguous():
            raise GQError(GQ_EINVAL, f"{name} must be a contiguous host (CPU) tensor")
    n, d_in = X.shape
    d_out = G.shape[1]
    if G.shape[0] != n:
        raise GQError(GQ_ESHAPE, "X and G need the same number of tokens")
    if X.dtype != G.dtype:
        raise GQError(GQ_EDTYPE, "X and G must share a dtype")
    _shape(F, (groups, d_in, d_in), "F")
    dev = F.device if F is not None else (device or torch.device("cuda", torch.cuda.current_device()))
    if F is None:
        F = torch.empty((groups, d_in, d_in), dtype=torch.float32, device=dev)
        if accumulate:
            F.zero_()
    _dev(F, "F", torch.float32)
    if ws is not None:
        _same_device(F, ws)
    if ws is None:
        nb = fisher_stream_workspace_size(min(chunk_tokens, n), d_in, d_out, groups, _dt(X))
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _check(lib.gq_fisher_accumulate_host(ctypes.c_void_p(X.data_ptr()), _dt(X), n, d_in,
                                         ctypes.c_void_p(G.data_ptr()), _dt(G), d_out, groups,
                                         _ptr(F), int(accumulate), chunk_tokens, _ptr(ws),
                                         ws.numel(), _stream(stream)))
    return F


def ganq_workspace_size(d_out, d_in, groups, bits, w_dtype=GQ_BF16) -> int:
    return int(library().ganq_workspace_size(d_out, d_in, groups, bits, w_dtype))


def ganq_quantize(W, F, bits: int, iters: int, ridge_rel: float = 1e-6, C=None, P=None,
                  init: int | None = None, trace: bool = True, ws=None, stream=None,
                  ridge_abs: float = 0.0, check_finite: bool = False):
    """GANQ-style alternation.  Returns (C, P, obj_trace [2 iters + 1] or None,
    n_changed [iters], not_pd [groups] int32)."""
    lib = library()
    groups = F.shape[0]
    if init is None:
        init = GQ_INIT_GIVEN if (C is not None and P is not None) else GQ_INIT_QUANTILE
    d_out, d_in = _lnq_common(F, W, groups, bits, C, P)
    C, P = _outputs(W, d_out, d_in, bits, C, P)
    tr = torch.empty(2 * iters + 1, dtype=torch.float64, device=W.device) if trace else None
    nch = torch.zeros(max(iters, 1), dtype=torch.int64, device=W.device)
    npd = torch.zeros(groups, dtype=torch.int32, device=W.device)
    opt = options(DEFAULT_BLOCK, ridge_rel, init, GQ_GRAM_AUTO, ridge_abs, check_finite)
    if ws is None:
        ws = torch.empty(max(ganq_workspace_size(d_out, d_in, groups, bits, _dt(W)), 1),
                         dtype=torch.uint8, device=W.device)
    wp, nb = _ws_arg(ws)
    _check(lib.ganq_quantize(_ptr(W), _dt(W), d_out, d_in, _ptr(F), groups, bits, iters,
                             ctypes.byref(opt), _ptr(C), _ptr(P), _ptr(tr), _ptr(nch), _ptr(npd),
                             wp, nb, _stream(stream)))
    return C, P, tr, nch[:iters], npd


def ganq_factor_damped(F, ridge_rel: float = 1e-6, ws=None, stream=None):
    """(L [groups][d][d] float32 lower, not_pd [groups] int32) of F' = F + lambda I."""
    lib = library()
    if F.dim() != 3 or F.shape[1] != F.shape[2]:
        raise GQError(GQ_ESHAPE, "F must be [groups][d_in][d_in]")
    _dev(F, "F", torch.float32)
    groups, d_in = F.shape[0], F.shape[1]
    L = torch.empty_like(F)
    npd = torch.zeros(groups, dtype=torch.int32, device=F.device)
    if ws is None:
        ws = torch.empty(max(ganq_workspace_size(groups, d_in, groups, 1), 1), dtype=torch.uint8,
                         device=F.device)
    _check(lib.ganq_factor_damped(_ptr(F), groups, d_in, ridge_rel, _ptr(L), _ptr(npd), _ptr(ws),
                                  ws.numel(), _stream(stream)))
    return L, npd


def lut_packed_row_words(d_in: int, bits: int) -> int:
    return int(library().lut_packed_row_words(d_in, bits))


def lut_pack_codes(P, bits: int, Q=None, stream=None) -> torch.Tensor:
    """P [d_out][d_in] uint8 -> packed codes Q [d_out][row words] (int32 storage of the
    uint32 words)."""
    lib = library()
    if P.dim() != 2:
        raise GQError(GQ_ESHAPE, "P must be [d_out][d_in]")
    d_out, d_in = P.shape
    rw = lut_packed_row_words(d_in, bits)
    _shape(Q, (d_out, max(rw, 1)), "Q")
    _dev(P, "P", torch.uint8)
    if Q is None:
        Q = torch.empty((d_out, max(rw, 1)), dtype=torch.int32, device=P.device)
    _dev(Q, "Q", torch.int32)
    _same_device(P, Q)
    _check(lib.lut_pack_codes(_ptr(P), d_out, d_in, bits, _ptr(Q), _stream(stream)))
    return Q


def lut_gemv(Q, C, x, bits: int, d_in: int | None = None, y=None, stream=None) -> torch.Tensor:
    """y [batch][d_out] = sum_i C[j][code_ji] x[b][i]; x [batch][d_in] or [d_in]
    (d_in, if given, must be x's last dimension)."""
    lib = library()
    if x.dim() not in (1, 2) or C.dim() != 2:
        raise GQError(GQ_ESHAPE, "x must be [batch][d_in] or [d_in] and C [d_out][2^bits]")
    xx = x if x.dim() == 2 else x.unsqueeze(0)
    batch, dx = xx.shape
    if d_in is not None and d_in != dx:
        raise GQError(GQ_ESHAPE, f"d_in={d_in} differs from the activations' {dx}")
    d_in = dx
    d_out = C.shape[0]
    _shape(C, (d_out, 1 << bits), "C")
    _shape(Q, (d_out, max(lut_packed_row_words(d_in, bits), 1)), "Q")
    _shape(y, (batch, d_out), "y")
    _dev(Q, "Q", torch.int32)
    _dev(C, "C", torch.float32)
    _dev(x, "x")
    if y is None:
        y = torch.empty((batch, d_out), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32)
    _same_device(Q, C, x, y)
    _check(lib.lut_gemv(_ptr(Q), _ptr(C), d_out, d_in, bits, _ptr(xx), _dt(xx), batch, _ptr(y),
                        _stream(stream)))
    return y if x.dim() == 2 else y[0]


STAGES = ("group_scale", "fisher_mfma", "fisher_finalize", "fisher_plain", "lnq_prepare",
          "lnq_resid", "lnq_init", "lnq_gram", "lnq_solve", "lnq_sweep", "lnq_small",
          "fisher_pack", "lnq_delta", "lut_pack", "lut_gemv", "fisher_h2d", "ganq_chol",
          "ganq_pass")


def gq_timing_enable(on=True) -> None:
    """Bracket later launch sequences with HIP events on their stream (diagnostics).

    on: True (every stage), False (off), a stage name, or an iterable of names.
    """
    if on is True:
        mask = -1
    elif on is False or on is None:
        mask = 0
    else:
        names = [on] if isinstance(on, str) else list(on)
        mask = 0
        for n in names:
            mask |= 1 << STAGES.index(n)
    library().gq_timing_enable(mask)


def gq_timing_read() -> dict:
    """{stage name: (milliseconds, launch sequences)} since the last read; clears."""
    lib = library()
    ms = (ctypes.c_double * STAGE_COUNT)()
    cnt = (_i64 * STAGE_COUNT)()
    _check(lib.gq_timing_read(ms, cnt))
    return {lib.gq_stage_name(i).decode(): (ms[i], cnt[i]) for i in range(STAGE_COUNT)}

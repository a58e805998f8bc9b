"""Python binding of libsvdq.so, the SVDQuant W4A4 linear layer for MI355X (gfx950).

Argument marshalling only: every computation runs in the library (host
packer in C++, forward in HIP kernels).  The functions carry the C ABI's
names and argument order (see include/svdq.h).  Host functions take numpy
arrays; device functions take torch tensors that already live on the GPU
(torch only supplies device memory and the current stream).

The library must be built first (``python bit_diffusion_model_svdq_amd/build.py``);
importing this package without it raises an ImportError.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SVDQ_LIBRARY names another build of the same library (the host-sanitizer build
# that the CPU tests can run against); by default the in-tree libsvdq.so.
LIB_PATH = os.environ.get("SVDQ_LIBRARY") or os.path.join(_HERE, "libsvdq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with python bit_diffusion_model_svdq_amd/build.py")

# torch ships its own HIP runtime under the same soname as the system one the
# library is linked against.  Whichever is loaded first serves the whole
# process, and a process that ends up with parts of both finds no device, so
# torch (which owns the device memory and streams) is loaded before the library.
try:
    import torch as _torch  # noqa: F401
except ImportError:  # host-only use (packer) without torch
    _torch = None

_lib = ctypes.CDLL(LIB_PATH)

SVDQ_OK = 0
STATUS_NAMES = {0: "SVDQ_OK", 1: "SVDQ_ERR_INVALID_ARG", 2: "SVDQ_ERR_UNSUPPORTED",
                3: "SVDQ_ERR_ALIGNMENT", 4: "SVDQ_ERR_WORKSPACE", 5: "SVDQ_ERR_NO_CONVERGENCE",
                6: "SVDQ_ERR_HIP"}

EXPORTS = [
    "svdq_act_absmax_update", "svdq_pack_weights", "svdq_quantize_residual", "svdq_append_lora",
    "svdq_forward_workspace_bytes", "svdq_linear_forward", "svdq_forward_quantize",
    "svdq_forward_gemm", "svdq_quantize_activations", "svdq_debug_group_partials",
    "svdq_status_string", "svdq_last_error",
    "svdq_quantize_residual_mxfp4", "svdq_forward_workspace_bytes_mxfp4", "svdq_linear_forward_mxfp4",
    "svdq_forward_quantize_mxfp4", "svdq_forward_gemm_mxfp4", "svdq_quantize_activations_mxfp4",
    "svdq_linear_forward_act", "svdq_forward_gemm_act", "svdq_linear_forward_act_mxfp4",
    "svdq_forward_gemm_act_mxfp4", "svdq_mxfp4_tiled_scale_bytes", "svdq_mxfp4_tile_scales",
    "svdq_act_absmax_update_device", "svdq_forward_workspace_layout",
    "svdq_forward_workspace_layout_mxfp4", "svdq_static_workspace_bytes", "svdq_linear_forward_noalloc",
    "svdq_forward_fused", "svdq_debug_fused_forward", "svdq_forward_fused_mxfp4",
    "svdq_debug_fused_forward_mxfp4",
]

# svdq_activation
SVDQ_ACT_NONE = 0
SVDQ_ACT_GELU_TANH = 1


class SvdqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.svdq_last_error().decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


class svdq_pack_params(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_float), ("rank", ctypes.c_int), ("group", ctypes.c_int),
                ("s_min", ctypes.c_float)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_sig = {
    "svdq_act_absmax_update": [_P, ctypes.c_int64, _I, _P],
    "svdq_pack_weights": [_P, _I, _I, _P, ctypes.POINTER(svdq_pack_params), _P, _P, _P, _P, _P, _P],
    "svdq_quantize_residual": [_P, _I, _I, _P, _P, _P, _I, _P, _P],
    "svdq_append_lora": [_P, _I, _I, _P, _P, _I, _P, _P, _I, _P, _P],
    "svdq_forward_workspace_bytes": [_I, _I, _I, _I],
    "svdq_linear_forward": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "svdq_forward_quantize": [_P, _I, _I, _I, _P, _P, _P, ctypes.c_size_t, _P],
    "svdq_forward_gemm": [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "svdq_quantize_activations": [_P, _I, _I, _P, _P, _I, _P, _P, _P, _P],
    "svdq_debug_group_partials": [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P],
    "svdq_act_absmax_update_device": [_P, ctypes.c_int64, _I, _P, _P],
    "svdq_forward_workspace_layout": [_I, _I, _I, _I, _P, _P, _P, _P],
    "svdq_static_workspace_bytes": [],
    "svdq_forward_fused": [_I, _I, _I, _I],
    "svdq_debug_fused_forward": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P],
    "svdq_forward_fused_mxfp4": [_I, _I, _I, _I],
    "svdq_debug_fused_forward_mxfp4": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P],
    "svdq_linear_forward_noalloc": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P],
    "svdq_forward_workspace_layout_mxfp4": [_I, _I, _I, _I, _P, _P, _P, _P, _P],
    "svdq_quantize_residual_mxfp4": [_P, _I, _I, _P, _P, _P, _I, _P, _P],
    "svdq_forward_workspace_bytes_mxfp4": [_I, _I, _I, _I],
    "svdq_linear_forward_mxfp4": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "svdq_forward_quantize_mxfp4": [_P, _I, _I, _I, _P, _P, _P, ctypes.c_size_t, _P],
    "svdq_forward_gemm_mxfp4": [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "svdq_quantize_activations_mxfp4": [_P, _I, _I, _P, _P, _I, _P, _P, _P, _P],
    "svdq_linear_forward_act": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, ctypes.c_size_t, _P],
    "svdq_forward_gemm_act": [_I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, ctypes.c_size_t, _P],
    "svdq_linear_forward_act_mxfp4": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, ctypes.c_size_t, _P],
    "svdq_forward_gemm_act_mxfp4": [_I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, ctypes.c_size_t, _P],
    "svdq_mxfp4_tiled_scale_bytes": [_I, _I],
    "svdq_mxfp4_tile_scales": [_P, _I, _I, _P],
    "svdq_status_string": [_I],
    "svdq_last_error": [],
}
for _name, _args in _sig.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _I
_lib.svdq_forward_workspace_bytes.restype = ctypes.c_size_t
_lib.svdq_static_workspace_bytes.restype = ctypes.c_size_t
_lib.svdq_forward_workspace_bytes_mxfp4.restype = ctypes.c_size_t
_lib.svdq_mxfp4_tiled_scale_bytes.restype = ctypes.c_size_t
_lib.svdq_status_string.restype = ctypes.c_char_p
_lib.svdq_last_error.restype = ctypes.c_char_p


def _check(st: int, where: str):
    if st != SVDQ_OK:
        raise SvdqError(st, where)


# ------------------------------------------------------------------ host side
def _host(a, dtype, shape=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=dtype)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _hp(a):
    return None if a is None else a.ctypes.data


def svdq_act_absmax_update(X_bf16: np.ndarray, amax: np.ndarray) -> np.ndarray:
    """Folds bf16 rows X [M, K] (uint16 bits) into the running abs-max amax [K] (float32, in place)."""
    X = _host(X_bf16, np.uint16)
    if amax.dtype != np.float32 or not amax.flags.c_contiguous or amax.shape != (X.shape[1],):
        raise ValueError("amax must be a contiguous float32 [K] array")
    _check(_lib.svdq_act_absmax_update(_hp(X), X.shape[0], X.shape[1], _hp(amax)), "svdq_act_absmax_update")
    return amax


def svdq_pack_weights(W: np.ndarray, act_absmax: np.ndarray, alpha: float = 0.5, rank: int = 32,
                      s_min: float = 1e-5, group: int = 64, want_sigma: bool = False):
    """Offline pack.  Returns dict(smooth, L1 [r,K] bf16 bits, L2 [N,r] bf16 bits, Wq, w_scales[, sigma])."""
    W = _host(W, np.float32)
    N, K = W.shape
    A = _host(act_absmax, np.float32, (K,))
    p = svdq_pack_params(alpha, rank, group, s_min)
    out = dict(smooth=np.empty(K, np.float32), L1=np.empty((rank, K), np.uint16),
               L2=np.empty((N, rank), np.uint16), Wq=np.empty((N, K // 2), np.uint8),
               w_scales=np.empty((N, max(K // 64, 0)), np.float32))
    sigma = np.empty(min(N, K), np.float64) if want_sigma else None
    st = _lib.svdq_pack_weights(_hp(W), N, K, _hp(A), ctypes.byref(p), _hp(out["smooth"]),
                                _hp(out["L1"]) if rank else None, _hp(out["L2"]) if rank else None,
                                _hp(out["Wq"]), _hp(out["w_scales"]), _hp(sigma))
    _check(st, "svdq_pack_weights")
    if want_sigma:
        out["sigma"] = sigma
    return out


def svdq_quantize_residual(W, smooth, L1, L2):
    """Wq [N, K/2] and w_scales [N, K/64] from W, s, L1 [r, K], L2 [N, r] (host arrays)."""
    W = _host(W, np.float32)
    N, K = W.shape
    s = _host(smooth, np.float32, (K,))
    L1 = _host(L1, np.uint16)
    L2 = _host(L2, np.uint16)
    r = L1.shape[0] if L1.ndim == 2 else 0
    Wq = np.empty((N, K // 2), np.uint8)
    ws = np.empty((N, K // 64), np.float32)
    st = _lib.svdq_quantize_residual(_hp(W), N, K, _hp(s), _hp(L1) if r else None,
                                     _hp(L2) if r else None, r, _hp(Wq), _hp(ws))
    _check(st, "svdq_quantize_residual")
    return Wq, ws


def svdq_append_lora(smooth, L1, L2, A, B):
    """(L1' [r + rl, K], L2' [N, r + rl]): the packed layer's low-rank factors with a
    LoRA (A [K, rl] down, B [rl, N] up, float32) appended; host arrays."""
    A = _host(A, np.float32)
    B = _host(B, np.float32)
    K, rl = A.shape
    N = B.shape[1]
    s = _host(smooth, np.float32, (K,))
    L1 = _host(L1, np.uint16)
    L2 = _host(L2, np.uint16)
    r = L1.shape[0] if (L1 is not None and L1.ndim == 2) else 0
    L1o = np.empty((r + rl, K), np.uint16)
    L2o = np.empty((N, r + rl), np.uint16)
    st = _lib.svdq_append_lora(_hp(s), K, N, _hp(L1) if r else None, _hp(L2) if r else None, r,
                               _hp(A), _hp(B), rl, _hp(L1o), _hp(L2o))
    _check(st, "svdq_append_lora")
    return L1o, L2o


# ---------------------------------------------------------------- device side
def _dp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# The C ABI sees only pointers, so a wrong tensor would be read or written out
# of bounds; every device wrapper checks its tensors against the shapes the
# library will assume before it calls in.
_BF16 = ("int16", "bfloat16")      # bf16 bit patterns: int16 views or torch.bfloat16


def _need(t, name, dtypes, shape=None, numel=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} must not be None")
    if not hasattr(t, "data_ptr") or not hasattr(t, "is_contiguous"):
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    dt = str(t.dtype).replace("torch.", "")
    if dtypes is not None and dt not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(dtypes)} (got {dt})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements (got {t.numel()})")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors live on different devices: {sorted(str(d) for d in devs)}")


def _rank_of(L1, L2=None, N=None):
    r = L1.shape[0] if L1 is not None else 0
    if (L2 is None) != (L1 is None) and r > 0:
        raise ValueError("L1 and L2 must both be given (or both None for r = 0)")
    return r


def _check_layer(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, Y, mx=False):
    """Shapes of one layer's device tensors, as include/svdq.h lays them out."""
    if X is not None:
        _need(X, "X", _BF16, (M, K))
    if smooth is not None or X is not None:
        _need(smooth, "smooth", ("float32",), (K,))
    if L1 is not None or (X is not None and r > 0):
        _need(L1, "L1", _BF16, (r, K), optional=r == 0)
    if Wq is not None:
        _need(L2, "L2", _BF16, (N, r), optional=r == 0)
        _need(Wq, "Wq", ("uint8",), (N, K // 2))
        if mx:
            _need(w_scales, "w_e8m0", ("uint8",), numel=svdq_mxfp4_tiled_scale_bytes(N, K))
        else:
            _need(w_scales, "w_scales", ("float32",), (N, K // 64))
        _need(bias, "bias", _BF16, (N,), optional=True)
        _need(Y, "Y", _BF16, (M, N))
    _same_device(X, smooth, L1, L2, Wq, w_scales, bias, Y)


def _check_ws(workspace, *others):
    _need(workspace, "workspace", None)
    _same_device(workspace, *others)


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def svdq_forward_workspace_bytes(M: int, K: int, N: int, r: int) -> int:
    return int(_lib.svdq_forward_workspace_bytes(M, K, N, r))


def svdq_forward_workspace_layout(M: int, K: int, N: int, r: int, mxfp4: bool = False) -> dict:
    """Byte offsets of qx, sx and the T slices inside the forward's workspace, the
    number of T slices and (MXFP4) the row count of the k-tiled activation scales."""
    qo, so, to = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    ts, rows = ctypes.c_int(), ctypes.c_int()
    if mxfp4:
        st = _lib.svdq_forward_workspace_layout_mxfp4(M, K, N, r, ctypes.byref(qo), ctypes.byref(so),
                                                      ctypes.byref(to), ctypes.byref(ts), ctypes.byref(rows))
    else:
        st = _lib.svdq_forward_workspace_layout(M, K, N, r, ctypes.byref(qo), ctypes.byref(so),
                                                ctypes.byref(to), ctypes.byref(ts))
    _check(st, "svdq_forward_workspace_layout")
    out = dict(qx=qo.value, sx=so.value, T=to.value, t_slices=ts.value)
    if mxfp4:
        out["sx_rows"] = rows.value
    return out


def svdq_linear_forward(X, smooth, L1, L2, Wq, w_scales, bias, Y, workspace, stream=None):
    """Y [M, N] (bf16 tensor, written) = SVDQuant linear of X [M, K] bf16.  All tensors on the GPU."""
    M, K = X.shape
    N = Wq.shape[0]
    r = _rank_of(L1, L2)
    _check_layer(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, Y)
    _check_ws(workspace, X)
    st = _lib.svdq_linear_forward(_dp(X), M, K, N, r, _dp(smooth), _dp(L1), _dp(L2), _dp(Wq),
                                  _dp(w_scales), _dp(bias), _dp(Y), _dp(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "svdq_linear_forward")
    return Y


def svdq_linear_forward_act(X, smooth, L1, L2, Wq, w_scales, bias, activation, Y, workspace,
                            stream=None):
    """svdq_linear_forward with an svdq_activation applied to Y (SVDQ_ACT_GELU_TANH: GELU, tanh form)."""
    M, K = X.shape
    N = Wq.shape[0]
    r = _rank_of(L1, L2)
    _check_layer(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, Y)
    _check_ws(workspace, X)
    st = _lib.svdq_linear_forward_act(_dp(X), M, K, N, r, _dp(smooth), _dp(L1), _dp(L2), _dp(Wq),
                                      _dp(w_scales), _dp(bias), int(activation), _dp(Y), _dp(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "svdq_linear_forward_act")
    return Y


def svdq_static_workspace_bytes() -> int:
    return int(_lib.svdq_static_workspace_bytes())


def svdq_linear_forward_noalloc(X, smooth, L1, L2, Wq, w_scales, bias, activation, Y, stream=None):
    """svdq_linear_forward_act without a workspace argument: the library's static device
    workspace serves instead (no allocation; calls that overlap on one GPU race)."""
    M, K = X.shape
    N = Wq.shape[0]
    r = _rank_of(L1, L2)
    _check_layer(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, Y)
    st = _lib.svdq_linear_forward_noalloc(_dp(X), M, K, N, r, _dp(smooth), _dp(L1), _dp(L2), _dp(Wq),
                                          _dp(w_scales), _dp(bias), int(activation), _dp(Y), _stream(stream))
    _check(st, "svdq_linear_forward_noalloc")
    return Y


def svdq_forward_quantize(X, smooth, L1, workspace, stream=None):
    M, K = X.shape
    r = L1.shape[0] if L1 is not None else 0
    _check_layer(X, M, K, 16, r, smooth, L1, None, None, None, None, None)
    _check_ws(workspace, X)
    st = _lib.svdq_forward_quantize(_dp(X), M, K, r, _dp(smooth), _dp(L1), _dp(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "svdq_forward_quantize")


def svdq_forward_gemm(M, K, L2, Wq, w_scales, bias, Y, workspace, r, stream=None):
    N = Wq.shape[0]
    _check_layer(None, M, K, N, r, None, None, L2, Wq, w_scales, bias, Y)
    _check_ws(workspace, Wq)
    st = _lib.svdq_forward_gemm(M, K, N, r, _dp(L2), _dp(Wq), _dp(w_scales), _dp(bias), _dp(Y),
                                _dp(workspace), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check(st, "svdq_forward_gemm")


def svdq_forward_gemm_act(M, K, L2, Wq, w_scales, bias, activation, Y, workspace, r, stream=None):
    N = Wq.shape[0]
    _check_layer(None, M, K, N, r, None, None, L2, Wq, w_scales, bias, Y)
    _check_ws(workspace, Wq)
    st = _lib.svdq_forward_gemm_act(M, K, N, r, _dp(L2), _dp(Wq), _dp(w_scales), _dp(bias),
                                    int(activation), _dp(Y), _dp(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "svdq_forward_gemm_act")


def svdq_quantize_activations(X, smooth, L1, qx, sx, T, stream=None):
    M, K = X.shape
    r = L1.shape[0] if L1 is not None else 0
    _check_layer(X, M, K, 16, r, smooth, L1, None, None, None, None, None)
    _need(qx, "qx", ("uint8",), (M, K // 2))
    _need(sx, "sx", ("float32",), (M, K // 64))
    _need(T, "T", ("float32",), (M, r), optional=r == 0)
    _same_device(X, qx, sx, T)
    st = _lib.svdq_quantize_activations(_dp(X), M, K, _dp(smooth), _dp(L1), r, _dp(qx), _dp(sx),
                                        _dp(T), _stream(stream))
    _check(st, "svdq_quantize_activations")


def svdq_act_absmax_update_device(X, amax, stream=None):
    """Folds bf16 rows X [M, K] (GPU tensor) into the running abs-max amax [K]
    (float32 GPU tensor holding values >= +0, updated in place)."""
    if X.dim() != 2:
        raise ValueError("X must be a [M, K] tensor")
    M, K = X.shape
    _need(X, "X", _BF16, (M, K))
    _need(amax, "amax", ("float32",), (K,))
    _same_device(X, amax)
    st = _lib.svdq_act_absmax_update_device(_dp(X), M, K, _dp(amax), _stream(stream))
    _check(st, "svdq_act_absmax_update_device")
    return amax


def svdq_forward_fused(M, K, N, r) -> bool:
    """Whether the int4 forward runs (M, K, N, r) as the single fused small-K kernel."""
    return bool(_lib.svdq_forward_fused(int(M), int(K), int(N), int(r)))


def svdq_debug_fused_forward(X, smooth, L1, L2, Wq, w_scales, bias, activation, Y, qx, sx, stream=None):
    """The fused small-K forward, also writing its activation codes qx [M, K/2] and scales sx [M, K/64]."""
    M, K = X.shape
    N = Wq.shape[0]
    r = _rank_of(L1, L2)
    _check_layer(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, Y)
    _need(qx, "qx", ("uint8",), (M, K // 2))
    _need(sx, "sx", ("float32",), (M, K // 64))
    _same_device(X, qx, sx)
    st = _lib.svdq_debug_fused_forward(_dp(X), M, K, N, r, _dp(smooth), _dp(L1), _dp(L2), _dp(Wq),
                                       _dp(w_scales), _dp(bias), int(activation), _dp(Y), _dp(qx), _dp(sx),
                                       _stream(stream))
    _check(st, "svdq_debug_fused_forward")
    return Y


def svdq_forward_fused_mxfp4(M, K, N, r) -> bool:
    """Whether the MXFP4 forward runs (M, K, N, r) as the single fused small-K kernel."""
    return bool(_lib.svdq_forward_fused_mxfp4(int(M), int(K), int(N), int(r)))


def svdq_debug_fused_forward_mxfp4(X, smooth, L1, L2, Wq, w_e8m0, bias, activation, Y, qx, sx_e8m0,
                                   stream=None):
    """The fused MXFP4 forward, also writing its codes qx [M, K/2] and E8M0 bytes sx_e8m0 [M, K/32]."""
    M, K = X.shape
    N = Wq.shape[0]
    r = _rank_of(L1, L2)
    _check_layer(X, M, K, N, r, smooth, L1, L2, Wq, w_e8m0, bias, Y, mx=True)
    _need(qx, "qx", ("uint8",), (M, K // 2))
    _need(sx_e8m0, "sx_e8m0", ("uint8",), (M, K // 32))
    _same_device(X, qx, sx_e8m0)
    st = _lib.svdq_debug_fused_forward_mxfp4(_dp(X), M, K, N, r, _dp(smooth), _dp(L1), _dp(L2), _dp(Wq),
                                             _dp(w_e8m0), _dp(bias), int(activation), _dp(Y), _dp(qx),
                                             _dp(sx_e8m0), _stream(stream))
    _check(st, "svdq_debug_fused_forward_mxfp4")
    return Y


def svdq_debug_group_partials(qx, Wq, m0, m1, n0, n1, P, stream=None):
    M = qx.shape[0]
    K = qx.shape[1] * 2
    N = Wq.shape[0]
    _need(qx, "qx", ("uint8",), (M, K // 2))
    _need(Wq, "Wq", ("uint8",), (N, K // 2))
    if not (0 <= m0 < m1 <= M and 0 <= n0 < n1 <= N):
        raise ValueError(f"block [{m0},{m1})x[{n0},{n1}) is outside [0,{M})x[0,{N})")
    _need(P, "P", ("int32",), (m1 - m0, n1 - n0, K // 64))
    _same_device(qx, Wq, P)
    st = _lib.svdq_debug_group_partials(_dp(qx), _dp(Wq), M, N, K, m0, m1, n0, n1, _dp(P),
                                        _stream(stream))
    _check(st, "svdq_debug_group_partials")


def svdq_status_string(status: int) -> str:
    return _lib.svdq_status_string(status).decode()


def svdq_last_error() -> str:
    return _lib.svdq_last_error().decode()


# ------------------------------------------------------------ MXFP4 variant
def svdq_quantize_residual_mxfp4(W, smooth, L1, L2):
    """Wq [N, K/2] (E2M1 codes) and row-major w_e8m0 [N, K/32] from W, s, L1 [r, K], L2 [N, r]
    (host arrays).  The forward takes the scales k-tiled (svdq_mxfp4_tile_scales)."""
    W = _host(W, np.float32)
    N, K = W.shape
    s = _host(smooth, np.float32, (K,))
    L1 = _host(L1, np.uint16)
    L2 = _host(L2, np.uint16)
    r = L1.shape[0] if (L1 is not None and L1.ndim == 2) else 0
    Wq = np.empty((N, K // 2), np.uint8)
    we = np.empty((N, K // 32), np.uint8)
    st = _lib.svdq_quantize_residual_mxfp4(_hp(W), N, K, _hp(s), _hp(L1) if r else None,
                                           _hp(L2) if r else None, r, _hp(Wq), _hp(we))
    _check(st, "svdq_quantize_residual_mxfp4")
    return Wq, we


def svdq_mxfp4_tiled_scale_bytes(rows: int, K: int) -> int:
    return int(_lib.svdq_mxfp4_tiled_scale_bytes(rows, K))


def svdq_mxfp4_tile_scales(scales):
    """Row-major E8M0 scales [rows, K/32] (host) -> the k-tiled layout [ceil(K/256), rows, 8]."""
    sc = _host(scales, np.uint8)
    rows, nb = sc.shape
    K = 32 * nb
    out = np.empty(((K + 255) // 256, rows, 8), np.uint8)
    _check(_lib.svdq_mxfp4_tile_scales(_hp(sc), rows, K, _hp(out)), "svdq_mxfp4_tile_scales")
    return out


def svdq_forward_workspace_bytes_mxfp4(M: int, K: int, N: int, r: int) -> int:
    return int(_lib.svdq_forward_workspace_bytes_mxfp4(M, K, N, r))


def svdq_linear_forward_mxfp4(X, smooth, L1, L2, Wq, w_e8m0, bias, Y, workspace, stream=None):
    M, K = X.shape
    N = Wq.shape[0]
    r = _rank_of(L1, L2)
    _check_layer(X, M, K, N, r, smooth, L1, L2, Wq, w_e8m0, bias, Y, mx=True)
    _check_ws(workspace, X)
    st = _lib.svdq_linear_forward_mxfp4(_dp(X), M, K, N, r, _dp(smooth), _dp(L1), _dp(L2), _dp(Wq),
                                        _dp(w_e8m0), _dp(bias), _dp(Y), _dp(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "svdq_linear_forward_mxfp4")
    return Y


def svdq_linear_forward_act_mxfp4(X, smooth, L1, L2, Wq, w_e8m0, bias, activation, Y, workspace,
                                  stream=None):
    M, K = X.shape
    N = Wq.shape[0]
    r = _rank_of(L1, L2)
    _check_layer(X, M, K, N, r, smooth, L1, L2, Wq, w_e8m0, bias, Y, mx=True)
    _check_ws(workspace, X)
    st = _lib.svdq_linear_forward_act_mxfp4(_dp(X), M, K, N, r, _dp(smooth), _dp(L1), _dp(L2),
                                            _dp(Wq), _dp(w_e8m0), _dp(bias), int(activation), _dp(Y),
                                            _dp(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream))
    _check(st, "svdq_linear_forward_act_mxfp4")
    return Y


def svdq_forward_quantize_mxfp4(X, smooth, L1, workspace, stream=None):
    M, K = X.shape
    r = L1.shape[0] if L1 is not None else 0
    _check_layer(X, M, K, 16, r, smooth, L1, None, None, None, None, None)
    _check_ws(workspace, X)
    st = _lib.svdq_forward_quantize_mxfp4(_dp(X), M, K, r, _dp(smooth), _dp(L1), _dp(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "svdq_forward_quantize_mxfp4")


def svdq_forward_gemm_mxfp4(M, K, L2, Wq, w_e8m0, bias, Y, workspace, r, stream=None):
    N = Wq.shape[0]
    _check_layer(None, M, K, N, r, None, None, L2, Wq, w_e8m0, bias, Y, mx=True)
    _check_ws(workspace, Wq)
    st = _lib.svdq_forward_gemm_mxfp4(M, K, N, r, _dp(L2), _dp(Wq), _dp(w_e8m0), _dp(bias), _dp(Y),
                                      _dp(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream))
    _check(st, "svdq_forward_gemm_mxfp4")


def svdq_forward_gemm_act_mxfp4(M, K, L2, Wq, w_e8m0, bias, activation, Y, workspace, r,
                                stream=None):
    N = Wq.shape[0]
    _check_layer(None, M, K, N, r, None, None, L2, Wq, w_e8m0, bias, Y, mx=True)
    _check_ws(workspace, Wq)
    st = _lib.svdq_forward_gemm_act_mxfp4(M, K, N, r, _dp(L2), _dp(Wq), _dp(w_e8m0), _dp(bias),
                                          int(activation), _dp(Y), _dp(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "svdq_forward_gemm_act_mxfp4")


def svdq_quantize_activations_mxfp4(X, smooth, L1, qx, sx_e8m0, T, stream=None):
    M, K = X.shape
    r = L1.shape[0] if L1 is not None else 0
    _check_layer(X, M, K, 16, r, smooth, L1, None, None, None, None, None)
    _need(qx, "qx", ("uint8",), (M, K // 2))
    _need(sx_e8m0, "sx_e8m0", ("uint8",), (M, K // 32))
    _need(T, "T", ("float32",), (M, r), optional=r == 0)
    _same_device(X, qx, sx_e8m0, T)
    st = _lib.svdq_quantize_activations_mxfp4(_dp(X), M, K, _dp(smooth), _dp(L1), r, _dp(qx),
                                              _dp(sx_e8m0), _dp(T), _stream(stream))
    _check(st, "svdq_quantize_activations_mxfp4")

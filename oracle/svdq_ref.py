"""ctypes front of the plain C oracle (oracle/svdq_ref.c).

TEST INFRASTRUCTURE, like the rest of this package: only the test suite, the
package smoke check and the CPU-baseline leg of the benchmark use it.  It
marshals numpy arrays to the C functions and back; every step of the method
runs in the C file.  Names and return values follow the numpy oracle
(oracle/svdq_oracle.py), so the two can be checked against each other and
against the same pins.

The shared object is built in-tree with gcc (``build()``), and built on first
use when it is missing or older than its source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "svdq_ref.c")
LIB = os.path.join(HERE, "libsvdq_ref.so")
CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]

F32, F64 = np.float32, np.float64
GROUP = 64
MX_BLOCK = 32

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle into oracle/libsvdq_ref.so (always recompiles)."""
    tmp = LIB + ".tmp"
    r = subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the C oracle failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = ctypes.CDLL(LIB)
        _lib.oref_bf16_from_double.restype = ctypes.c_uint16
        _lib.oref_bf16_from_double.argtypes = [ctypes.c_double]
        _lib.oref_gelu_tanh.restype = ctypes.c_double
        _lib.oref_gelu_tanh.argtypes = [ctypes.c_double]
        _lib.oref_e2m1_round.argtypes = [ctypes.c_double]
        _lib.oref_mx_shared_exponent.argtypes = [ctypes.c_double]
        _lib.oref_e2m1_value.restype = ctypes.c_double
        _lib.oref_e2m1_value.argtypes = [ctypes.c_int]
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _call(name, *args):
    fn = getattr(_load(), name)
    conv = []
    for a in args:
        if isinstance(a, np.ndarray) or a is None:
            conv.append(_p(a))
        elif isinstance(a, float):
            conv.append(ctypes.c_double(a))
        else:
            conv.append(ctypes.c_int(int(a)))
    rc = fn(*conv)
    if rc != 0:
        raise ValueError(f"{name}: arguments rejected")


def _bf16(a):
    return None if a is None else _c(a, np.uint16)


# ------------------------------------------------------------------ helpers
def bf16_from_f64(x) -> np.ndarray:
    x = np.asarray(x, dtype=F64)
    lib = _load()
    return np.array([lib.oref_bf16_from_double(float(v)) for v in x.ravel()],
                    dtype=np.uint16).reshape(x.shape)


def bf16_to_f32(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (the upper half of a float32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(F32)


def bf16_to_f64(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(F64)


def unpack_nibbles(b) -> np.ndarray:
    """Decode packed int4 codes [..., K/2] (even channel in the low nibble) to int8 [..., K]."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    lo, hi = b & 0xF, b >> 4
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out


def rel_fro(Y, Yref) -> float:
    Y, Yref = np.asarray(Y, dtype=F64), np.asarray(Yref, dtype=F64)
    return float(np.linalg.norm(Y - Yref) / max(np.linalg.norm(Yref), 1e-300))


def max_abs_ratio(Y, Yref) -> float:
    Y, Yref = np.asarray(Y, dtype=F64), np.asarray(Yref, dtype=F64)
    return float(np.max(np.abs(Y - Yref)) / max(np.max(np.abs(Yref)), 1e-300))


def forward_exact(X_bf16, W, bias_bf16=None):
    """Unquantized X W^T + b in float64 (what E4 approximates; for reporting error)."""
    Y = bf16_to_f64(X_bf16) @ np.asarray(W, dtype=F32).astype(F64).T
    if bias_bf16 is not None:
        Y = Y + bf16_to_f64(bias_bf16)[None, :]
    return Y


def gelu_tanh(x) -> np.ndarray:
    x = np.asarray(x, dtype=F64)
    lib = _load()
    return np.array([lib.oref_gelu_tanh(float(v)) for v in x.ravel()], F64).reshape(x.shape)


# ----------------------------------------------------------- stage one
def act_absmax(xcal_bf16) -> np.ndarray:
    X = _bf16(xcal_bf16)
    A = np.empty(X.shape[1], F32)
    _call("oref_act_absmax", X, X.shape[0], X.shape[1], A)
    return A


def weight_absmax(W) -> np.ndarray:
    W = _c(W, F32)
    out = np.empty(W.shape[1], F32)
    _call("oref_weight_absmax", W, W.shape[0], W.shape[1], out)
    return out


def smoothing_factors(A, Wsc, alpha: float = 0.5, s_min: float = 1e-5) -> np.ndarray:
    A, Wsc = _c(A, F32), _c(Wsc, F32)
    s = np.empty(A.shape[0], F32)
    _call("oref_smoothing_factors", A, Wsc, A.shape[0], float(alpha), float(s_min), s)
    return s


def smooth_weight(W, s) -> np.ndarray:
    W, s = _c(W, F32), _c(s, F32)
    out = np.empty(W.shape, F64)
    _call("oref_smooth_weight", W, W.shape[0], W.shape[1], s, out)
    return out


# ----------------------------------------------------------- stage two
def svd_sorted(What):
    """(U [N, p], sigma [p], V [K, p]) by one-sided Jacobi, sigma descending."""
    What = _c(What, F64)
    N, K = What.shape
    p = min(N, K)
    U, S, V = np.empty((N, p), F64), np.empty(p, F64), np.empty((K, p), F64)
    _call("oref_svd", What, N, K, U, S, V)
    return U, S, V


def lowrank_factors(U, S, V, r: int):
    U, S, V = _c(U, F64), _c(S, F64), _c(V, F64)
    N, p = U.shape
    K = V.shape[0]
    L1, L2 = np.empty((r, K), np.uint16), np.empty((N, r), np.uint16)
    _call("oref_lowrank_factors", U, S, V, N, K, p, r, L1, L2)
    return L1, L2


def residual(What, L1_bf16, L2_bf16) -> np.ndarray:
    What = _c(What, F64)
    N, K = What.shape
    L1 = _bf16(L1_bf16).reshape(-1, K)
    L2 = _bf16(L2_bf16).reshape(N, -1)
    R = np.empty((N, K), F32)
    _call("oref_residual", What, N, K, L1, L2, L1.shape[0], R)
    return R


# --------------------------------------------------------- stage three
def quantize_groups(v32, weight_scale: bool = False):
    v = _c(v32, F32)
    shape = v.shape
    v2 = v.reshape(-1, shape[-1])
    q = np.empty(v2.shape, np.int8)
    sc = np.empty((v2.shape[0], shape[-1] // GROUP), F32)
    _call("oref_quantize_groups", v2, v2.shape[0], v2.shape[1], int(weight_scale), q, sc)
    return q.reshape(shape), sc.reshape(shape[:-1] + (shape[-1] // GROUP,))


def pack_nibbles(q) -> np.ndarray:
    q = _c(q, np.int8)
    q2 = q.reshape(-1, q.shape[-1])
    out = np.empty((q2.shape[0], q2.shape[1] // 2), np.uint8)
    _call("oref_pack_nibbles", q2, q2.shape[0], q2.shape[1], out)
    return out.reshape(q.shape[:-1] + (q.shape[-1] // 2,))


def quantize_residual(W, s, L1, L2):
    W, s = _c(W, F32), _c(s, F32)
    N, K = W.shape
    L1 = _bf16(L1).reshape(-1, K)
    L2 = _bf16(L2).reshape(N, -1)
    Wq, ws = np.empty((N, K // 2), np.uint8), np.empty((N, K // GROUP), F32)
    _call("oref_quantize_residual", W, N, K, s, L1, L2, L1.shape[0], Wq, ws)
    return Wq, ws


def pack_weights(W, A, alpha: float = 0.5, rank: int = 32, s_min: float = 1e-5):
    W, A = _c(W, F32), _c(A, F32)
    N, K = W.shape
    s = np.empty(K, F32)
    L1, L2 = np.empty((rank, K), np.uint16), np.empty((N, rank), np.uint16)
    Wq, ws = np.empty((N, K // 2), np.uint8), np.empty((N, K // GROUP), F32)
    sigma = np.empty(min(N, K), F64)
    _call("oref_pack_weights", W, N, K, A, float(alpha), float(s_min), rank, s, L1, L2, Wq, ws,
          sigma)
    What = smooth_weight(W, s)
    return dict(s=s, L1=L1, L2=L2, Wq=Wq, w_scales=ws, sigma=sigma, What=What,
                R=residual(What, L1, L2))


# ------------------------------------------------------------- forward
def smooth_activations(X_bf16, s) -> np.ndarray:
    X, s = _bf16(X_bf16), _c(s, F32)
    out = np.empty(X.shape, F32)
    _call("oref_smooth_activations", X, X.shape[0], X.shape[1], s, out)
    return out


def quantize_activations(X_bf16, s, L1_bf16=None):
    """(qx packed [M, K/2], sx [M, K/64], T [M, r] float64, x_hat float32 [M, K])."""
    X, s = _bf16(X_bf16), _c(s, F32)
    M, K = X.shape
    L1 = None if L1_bf16 is None or np.asarray(L1_bf16).size == 0 else _bf16(L1_bf16).reshape(-1, K)
    r = 0 if L1 is None else L1.shape[0]
    qx, sx = np.empty((M, K // 2), np.uint8), np.empty((M, K // GROUP), F32)
    T = np.empty((M, r), F64)
    _call("oref_quantize_activations", X, M, K, s, L1, r, qx, sx, T)
    return qx, sx, T, smooth_activations(X, s)


def group_partials(qx_packed, wq_packed) -> np.ndarray:
    qx, wq = _c(qx_packed, np.uint8), _c(wq_packed, np.uint8)
    M, N, K = qx.shape[0], wq.shape[0], qx.shape[1] * 2
    P = np.empty((M, N, K // GROUP), np.int32)
    _call("oref_group_partials", qx, wq, M, N, K, P)
    return P


_ACT = {None: 0, "gelu_tanh": 1}


def _act(activation) -> int:
    if activation not in _ACT:
        raise ValueError(f"unknown activation {activation!r}")
    return _ACT[activation]


def forward(X_bf16, s, L1_bf16, L2_bf16, Wq, w_scales, bias_bf16=None, activation=None,
            rows=None):
    """Y [rows, N] in float64 (all rows, or rows = (m0, m1))."""
    X, s = _bf16(X_bf16), _c(s, F32)
    M, K = X.shape
    Wq, ws = _c(Wq, np.uint8), _c(w_scales, F32)
    N = Wq.shape[0]
    r = 0 if L1_bf16 is None else np.asarray(L1_bf16).size // K
    L1 = _bf16(L1_bf16).reshape(r, K) if r else None
    L2 = _bf16(L2_bf16).reshape(N, r) if r else None
    m0, m1 = (0, M) if rows is None else rows
    Y = np.empty((m1 - m0, N), F64)
    _call("oref_forward_rows", X, M, K, N, r, s, L1, L2, Wq, ws, _bf16(bias_bf16),
          _act(activation), m0, m1, Y)
    return Y


def append_lora(s, L1_bf16, L2_bf16, A, B):
    s, A, B = _c(s, F32), _c(A, F32), _c(B, F32)
    K, rl = A.shape
    N = B.shape[1]
    L1 = _bf16(L1_bf16).reshape(-1, K)
    r = L1.shape[0]
    L2 = _bf16(L2_bf16).reshape(N, r)
    L1o, L2o = np.empty((r + rl, K), np.uint16), np.empty((N, r + rl), np.uint16)
    _call("oref_append_lora", s, L1, L2, K, N, r, A, B, rl, L1o, L2o)
    return L1o, L2o


# --------------------------------------------------------------- MXFP4
E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(codes) -> np.ndarray:
    c = np.asarray(codes)
    lib = _load()
    return np.array([lib.oref_e2m1_value(int(v)) for v in c.ravel()], F64).reshape(c.shape)


def e2m1_round(y) -> np.ndarray:
    y = np.asarray(y, dtype=F64)
    lib = _load()
    return np.array([lib.oref_e2m1_round(float(v)) for v in y.ravel()], np.int64).reshape(y.shape)


def mx_shared_exponent(amax) -> np.ndarray:
    a = np.asarray(amax, dtype=F64)
    lib = _load()
    return np.array([lib.oref_mx_shared_exponent(float(v)) for v in a.ravel()],
                    np.int64).reshape(a.shape)


def quantize_residual_mx(W, s, L1, L2):
    """(Wq packed [N, K/2], w_e8m0 [N, K/32]) of R = W diag(s) - L2 L1."""
    W, s = _c(W, F32), _c(s, F32)
    N, K = W.shape
    L1 = _bf16(L1).reshape(-1, K)
    L2 = _bf16(L2).reshape(N, -1)
    Wq, we = np.empty((N, K // 2), np.uint8), np.empty((N, K // MX_BLOCK), np.uint8)
    _call("oref_quantize_residual_mx", W, N, K, s, L1, L2, L1.shape[0], Wq, we)
    return Wq, we


def quantize_activations_mx(X_bf16, s, L1_bf16=None):
    """(qx packed [M, K/2], sx_e8m0 [M, K/32], T [M, r], x_hat)."""
    X, s = _bf16(X_bf16), _c(s, F32)
    M, K = X.shape
    L1 = None if L1_bf16 is None or np.asarray(L1_bf16).size == 0 else _bf16(L1_bf16).reshape(-1, K)
    r = 0 if L1 is None else L1.shape[0]
    qx, se = np.empty((M, K // 2), np.uint8), np.empty((M, K // MX_BLOCK), np.uint8)
    T = np.empty((M, r), F64)
    _call("oref_quantize_activations_mx", X, M, K, s, L1, r, qx, se, T)
    return qx, se, T, smooth_activations(X, s)


def quantize_mx(v32):
    """(codes uint8 [R, K] 4-bit patterns, exponents int64 [R, K/32])."""
    v = _c(v32, F32)
    R, K = v.shape
    codes, e8 = np.empty((R, K), np.uint8), np.empty((R, K // MX_BLOCK), np.uint8)
    _call("oref_quantize_mx", v, R, K, codes, e8)
    return codes, e8.astype(np.int64) - 127


def forward_mx(X_bf16, s, L1_bf16, L2_bf16, Wq, w_e8m0, bias_bf16=None, activation=None,
               rows=None):
    X, s = _bf16(X_bf16), _c(s, F32)
    M, K = X.shape
    Wq, we = _c(Wq, np.uint8), _c(w_e8m0, np.uint8)
    N = Wq.shape[0]
    r = 0 if L1_bf16 is None else np.asarray(L1_bf16).size // K
    L1 = _bf16(L1_bf16).reshape(r, K) if r else None
    L2 = _bf16(L2_bf16).reshape(N, r) if r else None
    m0, m1 = (0, M) if rows is None else rows
    Y = np.empty((m1 - m0, N), F64)
    _call("oref_forward_mx_rows", X, M, K, N, r, s, L1, L2, Wq, we, _bf16(bias_bf16),
          _act(activation), m0, m1, Y)
    return Y

"""CPU oracle for the SVDQuant W4A4 linear layer with its low-rank branch.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it, and it shares no
code, tables or helpers with that path.

It is plain, slow and written to be checked by eye against the pages:
numpy in float64, except at the points where the method itself fixes a
float32 rounding (smoothing, quantization scales, codes), where numpy's
IEEE float32 arithmetic is used.  Citations name the page and the section
or equation:

  [Term] "SVDQuant Low-Rank Residual Quantization Algorithm Terminology
         Entry" (mindstudio docs), section 2.3 "Mathematical Description":
         (E1) outlier migration  Y = XW + b = (X diag(s)^-1)(diag(s) W) + b
         (E2) s = A_scale^alpha / W_scale^(1-alpha),  s >= s_min
         (E3) W ~ (U S) V^T,  R = W - (U S) V^T
         (E4) out = Q(X diag(s)^-1) Q(R) + (X diag(s)^-1 V)(U S)^T ~ XW + b
         (E5) Eckart-Young: the truncated SVD is the best rank-r approximation
         (E6) residual energy = sum of the squared tail singular values
         (E7) XW^T = X L_r^T + X R^T, low-bit only for R
  [Abs]  "SVDQuant: Absorbing Outliers by Low-Rank Components for 4-Bit
         Diffusion Models" (codewithpapers abstract): 4-bit weights and
         activations, high-precision low-rank branch.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  weights are stored [N, K] (out, in) and s indexes input channels k;
  W_scale is the per-input-channel absolute maximum;
  s_min = 1e-5 and both statistics are floored at 1e-5 before the power;
  the low-rank factors are L1 = V_r^T (lora_down, stored [r, K]) and
  L2 = U_r Sigma_r (lora_up, stored [N, r]), both rounded to bfloat16 --
  the page's V [in, rank] and (U S)^T [rank, out] kept in the same
  [out, in] storage order as W;
  R is formed from the rounded factors;
  Q is symmetric 4-bit, one float32 scale per 64 consecutive input channels,
  scale = fl32(amax / 7), codes = clamp(rne(fl32(v * fl32(7 / amax))), -7, 7),
  an all-zero group gets scale 0 and codes 0, and so does a group whose amax
  lies below 2^-100 (there fl32(7 / amax) would approach the float32 overflow
  at about 2^-125.5; such a group's values are below anything the layer's
  output resolves);
  a weight scale additionally has its two lowest significand bits cleared
  (rounded toward zero), so that 3 * scale is exact in float32;
  x_hat = fl32(X * fl32(1 / s));
  codes are packed two per byte, the even channel in the low nibble.

Parity status: every function below has at least one pin in
tests/test_oracle_pins.py that does not re-type its formula.

A second, plain C implementation of the same contract, written separately
from the pages, is svdq_ref.c beside this file; every pin runs on both.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 64
QMAX = 7
TINY_GROUP = 2.0 ** -100    # absmax below this: coded as a zero group
S_MIN = 1e-5
STAT_FLOOR = 1e-5

F32 = np.float32
F64 = np.float64


# ---------------------------------------------------------------- bfloat16
def bf16_from_f64(x) -> np.ndarray:
    """Round float64 values straight to bfloat16 (nearest, ties to even).

    Returns uint16 bit patterns.  Works on the exact binary value: the
    significand is cut to 8 bits with one rounding, no detour via float32.
    """
    x = np.asarray(x, dtype=F64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.ravel()
    flat_out = out.ravel()
    for i, v in enumerate(flat_in):
        flat_out[i] = _bf16_scalar(float(v))
    return out


def _bf16_scalar(v: float) -> int:
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    m, e = math.frexp(a)            # a = m * 2^e, m in [0.5, 1)
    # bfloat16 normal numbers: 8 significant bits, exponent of the leading bit >= -126
    lead = e - 1                    # a in [2^lead, 2^(lead+1))
    bits_exp = max(lead, -126)      # subnormal range keeps the -126 exponent grid
    ulp = math.ldexp(1.0, bits_exp - 7)
    q = a / ulp                     # exact: a power-of-two division
    r = math.floor(q)
    frac = q - r
    if frac > 0.5 or (frac == 0.5 and (r % 2 == 1)):
        r += 1
    val = r * ulp
    if val >= math.ldexp(1.0, 128):  # overflow to infinity
        return sign | 0x7F80
    # encode val (exactly a bfloat16) through float32 bits
    return sign | int(np.array(val, dtype=F32).view(np.uint32) >> 16)


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(F32).astype(F64)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(F32)


# ---------------------------------------------------- stage one: smoothing
def act_absmax(xcal_bf16) -> np.ndarray:
    """A_scale[k]: absolute maximum of each input channel over the calibration rows.

    [Term] 2.3, the definition of A_scale under (E2).  Exact (float32 max).
    """
    return np.max(np.abs(bf16_to_f32(xcal_bf16)), axis=0)


def weight_absmax(W) -> np.ndarray:
    """W_scale[k]: absolute maximum over output rows of input channel k.

    [Term] 2.3, W_scale under (E2) ("per-column maximum"; W is stored [N, K]
    here, so the column of the page's [in, out] W is our input channel).
    """
    return np.max(np.abs(np.asarray(W, dtype=F32)), axis=0)


def smoothing_factors(A, Wsc, alpha: float = 0.5, s_min: float = S_MIN) -> np.ndarray:
    """s[k] = max(A^alpha / W_scale^(1-alpha), s_min), evaluated in float64, stored float32.

    [Term] 2.3 (E2).  Plain per-element libm pow.
    """
    A = np.asarray(A, dtype=F64)
    Wsc = np.asarray(Wsc, dtype=F64)
    s = np.empty(A.shape, dtype=F64)
    for k in range(A.shape[0]):
        a = max(float(A[k]), STAT_FLOOR)
        w = max(float(Wsc[k]), STAT_FLOOR)
        s[k] = max(math.pow(a, alpha) / math.pow(w, 1.0 - alpha), s_min)
    return s.astype(F32)


def smooth_weight(W, s) -> np.ndarray:
    """W_hat = W diag(s) (each input channel k scaled by s[k]), exact in float64.

    [Term] 2.3 (E1): the weight side of the outlier migration.
    """
    return np.asarray(W, dtype=F32).astype(F64) * np.asarray(s, dtype=F32).astype(F64)[None, :]


# --------------------------------------------- stage two: low-rank branch
def svd_sorted(What):
    """Thin SVD W_hat = U diag(sigma) V^T, sigma descending.

    [Term] 2.2 and 2.3 (E3).  numpy's LAPACK SVD is the library step; the
    sign of each pair is fixed so that the largest-magnitude entry of v_i
    is positive (any sign is a valid SVD; this just makes runs repeatable).
    Returns U [N, p], sigma [p], V [K, p].
    """
    U, S, Vt = np.linalg.svd(np.asarray(What, dtype=F64), full_matrices=False)
    order = np.argsort(-S, kind="stable")
    U, S, V = U[:, order], S[order], Vt[order, :].T
    idx = np.argmax(np.abs(V), axis=0)
    sgn = np.sign(V[idx, np.arange(V.shape[1])])
    sgn[sgn == 0] = 1.0
    return U * sgn[None, :], S, V * sgn[None, :]


def lowrank_factors(U, S, V, r: int):
    """L1 = bf16(V_r^T) stored [r, K] (lora_down), L2 = bf16(U_r Sigma_r) stored [N, r] (lora_up).

    [Term] 2.3 (E4): the branch is (X diag(s)^-1 V)(U S)^T, so Sigma rides
    with U.  Returns uint16 bfloat16 bit patterns.
    """
    L1 = bf16_from_f64(V[:, :r].T)
    L2 = bf16_from_f64(U[:, :r] * S[None, :r])
    return L1, L2


def residual(What, L1_bf16, L2_bf16) -> np.ndarray:
    """R = fl32(W_hat - (U S) V^T) with R[n, k] = W_hat[n, k] - sum_j L2[n, j] L1[j, k].

    [Term] 2.3 (E3) with the stored (rounded) factors.  The inner sum runs
    over j in ascending order in float64 starting from 0, each product exact
    (bfloat16 x bfloat16), then one subtraction and one rounding to float32.
    """
    What = np.asarray(What, dtype=F64)
    L1 = bf16_to_f64(L1_bf16)
    L2 = bf16_to_f64(L2_bf16)
    r = L1.shape[0] if L1.ndim == 2 else 0
    acc = np.zeros(What.shape, dtype=F64)
    for j in range(r):
        acc += L2[:, j][:, None] * L1[j, :][None, :]
    return (What - acc).astype(F32)


# ------------------------------------------- stage three: quantization Q
def quantize_groups(v32, weight_scale: bool = False):
    """Q(.) over groups of 64 consecutive entries of the last axis.

    [Term] 2.3 (E4) names Q; [Abs] fixes 4 bits.  Symmetric, codes in
    [-7, 7]:  a = max|v|;  scale = fl32(a / 7);  inv = fl32(7 / a);
    q = clamp(rne(fl32(v * inv)), -7, 7).  a < 2^-100 (a == 0 included)
    gives scale 0, q 0.
    weight_scale=True clears the two lowest significand bits of the scale.
    Returns (codes int8 [..., K], scales float32 [..., K/64]).
    """
    v = np.asarray(v32, dtype=F32)
    K = v.shape[-1]
    assert K % GROUP == 0
    g = v.reshape(v.shape[:-1] + (K // GROUP, GROUP))
    a = np.max(np.abs(g), axis=-1)
    nz = a >= F32(TINY_GROUP)
    safe = np.where(nz, a, F32(1))
    scale = np.where(nz, safe / F32(QMAX), F32(0)).astype(F32)
    inv = np.where(nz, F32(QMAX) / safe, F32(0)).astype(F32)
    q = np.rint(g * inv[..., None])
    q = np.clip(q, -QMAX, QMAX).astype(np.int8)
    if weight_scale:
        scale = (scale.view(np.uint32) & np.uint32(0xFFFFFFFC)).view(F32)
    return q.reshape(v.shape), scale


def pack_nibbles(q) -> np.ndarray:
    """Two codes per byte: byte i = (q[2i] & 0xF) | (q[2i+1] & 0xF) << 4."""
    q = np.asarray(q, dtype=np.int8).astype(np.int16)
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(b) -> np.ndarray:
    """Inverse of pack_nibbles: uint8 [..., K/2] -> int8 codes [..., K]."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int16)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# --------------------------------------------------------- offline pack
def pack_weights(W, A, alpha: float = 0.5, rank: int = 32, s_min: float = S_MIN):
    """The whole offline pipeline: smoothing, truncated SVD, residual quantization.

    [Term] 2.1 (three stages in this order) and 2.3 (E1)-(E4).
    Returns a dict with s, L1, L2 (bf16 bits), Wq (packed), w_scales, sigma,
    and the float64 W_hat and float32 R for tests.
    """
    Wsc = weight_absmax(W)
    s = smoothing_factors(A, Wsc, alpha, s_min)
    What = smooth_weight(W, s)
    U, S, V = svd_sorted(What)
    L1, L2 = lowrank_factors(U, S, V, rank)
    R = residual(What, L1, L2)
    q, ws = quantize_groups(R, weight_scale=True)
    return dict(s=s, L1=L1, L2=L2, Wq=pack_nibbles(q), w_scales=ws, sigma=S,
                What=What, R=R, U=U, V=V)


def quantize_residual(W, s, L1, L2):
    """Wq and w_scales from given s, L1, L2 (the last two steps of pack_weights)."""
    R = residual(smooth_weight(W, s), L1, L2)
    q, ws = quantize_groups(R, weight_scale=True)
    return pack_nibbles(q), ws


# ------------------------------------------------------------- forward
def smooth_activations(X_bf16, s) -> np.ndarray:
    """x_hat = fl32(X * fl32(1 / s)), float32 [M, K].  [Term] 2.3 (E1), (E4)."""
    inv_s = (F32(1) / np.asarray(s, dtype=F32)).astype(F32)
    return (bf16_to_f32(X_bf16) * inv_s[None, :]).astype(F32)


def quantize_activations(X_bf16, s, L1_bf16=None):
    """First half of (E4): Q(X diag(s)^-1) and the lora_down product T = x_hat L1^T.

    Returns (qx packed uint8 [M, K/2], sx float32 [M, K/64], T float64 [M, r], x_hat).
    """
    xh = smooth_activations(X_bf16, s)
    q, sx = quantize_groups(xh)
    if L1_bf16 is None or np.asarray(L1_bf16).size == 0:
        T = np.zeros((xh.shape[0], 0), dtype=F64)
    else:
        T = xh.astype(F64) @ bf16_to_f64(L1_bf16).T
    return pack_nibbles(q), sx, T, xh


def group_partials(qx_packed, wq_packed) -> np.ndarray:
    """P[m, n, g] = sum over k in group g of qx[m, k] * qw[n, k], exact int32.

    [Term] 2.3 (E4) the product Q(.)Q(R), (E7) low-bit only for R.  The
    integer dot products are evaluated as float64 matrix products, which
    are exact here (every partial sum is an integer below 2^53).
    """
    qx = unpack_nibbles(qx_packed).astype(F64)
    qw = unpack_nibbles(wq_packed).astype(F64)
    M, K = qx.shape
    N = qw.shape[0]
    G = K // GROUP
    P = np.empty((M, N, G), dtype=np.int32)
    for g in range(G):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        P[:, :, g] = (qx[:, sl] @ qw[:, sl].T).astype(np.int32)
    return P


# ------------------------------------------------ MLP activation (DiT block)
# A DiT MLP puts GELU between its up and down projections.  GELU in its tanh
# form (Hendrycks and Gimpel, "Gaussian Error Linear Units", section 2):
#   gelu(x) = 0.5 x (1 + tanh(sqrt(2 / pi) (x + 0.044715 x^3))).
# The pages do not treat the MLP; the reading used here fuses the activation
# into the up projection's output: gelu of the float sum main + low + b,
# before the output's single rounding to bfloat16.
ACTIVATIONS = (None, "gelu_tanh")


def gelu_tanh(x) -> np.ndarray:
    """GELU, tanh form, in float64."""
    x = np.asarray(x, dtype=F64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def _activate(Y, activation):
    if activation is None:
        return Y
    if activation == "gelu_tanh":
        return gelu_tanh(Y)
    raise ValueError(f"unknown activation {activation!r}")


def forward(X_bf16, s, L1_bf16, L2_bf16, Wq, w_scales, bias_bf16=None, activation=None):
    """Y = Q(X diag(s)^-1) Q(R) + (X diag(s)^-1 L1^T) L2^T + b in float64.

    [Term] 2.3 (E4) and (E7); bias added once.  The low-bit term is
    sum_g sx[m, g] * sw[n, g] * P[m, n, g] with exact integer P.
    activation "gelu_tanh" applies gelu_tanh to the sum (the MLP's up
    projection).  Returns float64 [M, N].
    """
    qx, sx, T, _ = quantize_activations(X_bf16, s, L1_bf16)
    qxv = unpack_nibbles(qx).astype(F64)
    qwv = unpack_nibbles(Wq).astype(F64)
    sw = np.asarray(w_scales, dtype=F32).astype(F64)
    sxd = sx.astype(F64)
    M, K = qxv.shape
    N = qwv.shape[0]
    main = np.zeros((M, N), dtype=F64)
    for g in range(K // GROUP):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        Pg = qxv[:, sl] @ qwv[:, sl].T
        main += (sxd[:, g][:, None] * sw[:, g][None, :]) * Pg
    if T.shape[1] > 0:
        low = T @ bf16_to_f64(L2_bf16).T
    else:
        low = np.zeros((M, N), dtype=F64)
    Y = main + low
    if bias_bf16 is not None:
        Y = Y + bf16_to_f64(bias_bf16)[None, :]
    return _activate(Y, activation)


def append_lora(s, L1_bf16, L2_bf16, A, B):
    """Fold an off-the-shelf LoRA into the low-rank branch, leaving Q(R) as it is.

    [Abs]: the engine takes existing low-rank adapters without re-quantizing the
    4-bit weights.  A LoRA adds X A B to the output (A [K, rl] down, B [rl, N]
    up).  The branch of E4 sees x_hat = X diag(s)^-1, and x_hat (diag(s) A) B =
    X A B, so the adapter joins the branch as extra rank-rl factors:
      L1' = [L1 ; bf16((diag(s) A)^T)]   [r + rl, K]   (A[k, j] * s[k], exact in float64)
      L2' = [L2 | bf16(B^T)]             [N, r + rl]
    """
    s64 = np.asarray(s, dtype=F32).astype(F64)
    A64 = np.asarray(A, dtype=F32).astype(F64)
    B64 = np.asarray(B, dtype=F32).astype(F64)
    L1n = bf16_from_f64((A64 * s64[:, None]).T)
    L2n = bf16_from_f64(B64.T)
    L1 = np.asarray(L1_bf16, dtype=np.uint16).reshape(-1, A64.shape[0])
    L2 = np.asarray(L2_bf16, dtype=np.uint16).reshape(B64.shape[1], -1)
    return np.concatenate([L1, L1n], axis=0), np.concatenate([L2, L2n], axis=1)


def forward_exact(X_bf16, W, bias_bf16=None):
    """Unquantized reference X W^T + b in float64 (what E4 approximates)."""
    Y = bf16_to_f64(X_bf16) @ np.asarray(W, dtype=F32).astype(F64).T
    if bias_bf16 is not None:
        Y = Y + bf16_to_f64(bias_bf16)[None, :]
    return Y


# --------------------------------------------------------- comparisons
# ------------------------------------------------------------- MXFP4 variant
# The same three stages with Q(.) taken as the OCP microscaling format MXFP4:
# blocks of 32 consecutive input channels share one power-of-two scale (an
# E8M0 byte, 2^(byte - 127)) and each element is an FP4 E2M1 number.  The
# pages give only "the quantization operation" for Q ([Term] 2.3, E4); this
# variant is the MXFP4 reading of it, with the scale rule of the OCP MX v1.0
# specification: shared exponent = floor(log2(amax)) - 2, where 2 is the
# exponent of E2M1's largest value 6 = 1.5 * 2^2, and elements rounded to
# nearest (ties to even) with saturation at +-6.
MX_BLOCK = 32
E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E2M1_EMAX = 2


def e2m1_value(codes) -> np.ndarray:
    """Value of 4-bit E2M1 patterns: bit 3 is the sign, bits 0..2 index E2M1_MAG."""
    c = np.asarray(codes).astype(np.int64)
    mag = np.asarray(E2M1_MAG, dtype=F64)[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_round(y) -> np.ndarray:
    """Index (0..7) of the E2M1 magnitude nearest to y >= 0.

    Ties go to the even index (IEEE ties-to-even on E2M1's one significand
    bit); values beyond 6 land on 6 (saturation).
    """
    y = np.asarray(y, dtype=F64)
    mags = np.asarray(E2M1_MAG, dtype=F64)
    best = np.zeros(y.shape, dtype=np.int64)
    best_d = np.abs(y - mags[0])
    for i in range(1, 8):
        d = np.abs(y - mags[i])
        better = (d < best_d) | ((d == best_d) & (i % 2 == 0))
        best = np.where(better, i, best)
        best_d = np.where(better, d, best_d)
    return best


def mx_shared_exponent(amax) -> np.ndarray:
    """floor(log2(amax)) - E2M1_EMAX, clipped to the E8M0 range [-127, 127];
    an all-zero block gets -127."""
    amax = np.asarray(amax, dtype=F64)
    m, x = np.frexp(amax)                 # amax = m * 2^x, 0.5 <= m < 1, so floor(log2) = x - 1
    e = np.clip(x.astype(np.int64) - 1 - E2M1_EMAX, -127, 127)
    return np.where(amax > 0, e, -127)


def quantize_mx(v32):
    """MXFP4 of float32 rows [R, K] (K % 32 == 0).

    Returns (codes uint8 [R, K] of 4-bit patterns, exponents int64 [R, K/32]).
    The sign bit is the sign of the input (so a negative value that rounds to
    zero keeps it); scaling by 2^-e is exact.
    """
    v = np.asarray(v32, dtype=F32).astype(F64)
    R, K = v.shape
    blocks = v.reshape(R, K // MX_BLOCK, MX_BLOCK)
    e = mx_shared_exponent(np.max(np.abs(blocks), axis=2))
    y = np.abs(blocks) / np.exp2(e.astype(F64))[:, :, None]
    idx = e2m1_round(y)
    sign = np.signbit(blocks).astype(np.int64)
    codes = (idx | (sign << 3)).astype(np.uint8)
    return codes.reshape(R, K), e


def e8m0_bytes(e) -> np.ndarray:
    return (np.asarray(e, dtype=np.int64) + 127).astype(np.uint8)


def unpack_codes4(b) -> np.ndarray:
    """Raw 4-bit patterns [R, 2 * C] of packed bytes [R, C] (even index in the low nibble)."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], b.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def quantize_residual_mx(W, s, L1, L2):
    """Stage three with MXFP4: (Wq packed [N, K/2], w_e8m0 [N, K/32]) of R = W diag(s) - L2 L1."""
    R = residual(smooth_weight(W, s), L1, L2)
    codes, e = quantize_mx(R)
    return pack_nibbles(codes.astype(np.int64)), e8m0_bytes(e)


def quantize_activations_mx(X_bf16, s, L1_bf16=None):
    """(qx packed [M, K/2], sx_e8m0 [M, K/32], T [M, r], x_hat) with MXFP4 codes of x_hat."""
    xh = smooth_activations(X_bf16, s)
    codes, e = quantize_mx(xh)
    if L1_bf16 is not None and np.asarray(L1_bf16).size:
        T = xh.astype(F64) @ bf16_to_f64(L1_bf16).T
    else:
        T = np.zeros((xh.shape[0], 0), dtype=F64)
    return pack_nibbles(codes.astype(np.int64)), e8m0_bytes(e), T, xh


def forward_mx(X_bf16, s, L1_bf16, L2_bf16, Wq, w_e8m0, bias_bf16=None, activation=None):
    """Y = Q_mx(X diag(s)^-1) Q_mx(R) + (X diag(s)^-1 L1^T) L2^T + b in float64.

    The low-bit term is sum over blocks b of 2^(ea[m,b] + eb[n,b]) times the
    exact dot product of the two blocks' E2M1 values.
    """
    qx, sxe, T, _ = quantize_activations_mx(X_bf16, s, L1_bf16)
    a = e2m1_value(unpack_codes4(qx))
    w = e2m1_value(unpack_codes4(Wq))
    ea = sxe.astype(np.int64) - 127
    eb = np.asarray(w_e8m0).astype(np.int64) - 127
    M, K = a.shape
    N = w.shape[0]
    main = np.zeros((M, N), dtype=F64)
    for b in range(K // MX_BLOCK):
        sl = slice(b * MX_BLOCK, (b + 1) * MX_BLOCK)
        main += np.exp2((ea[:, b][:, None] + eb[:, b][None, :]).astype(F64)) * (a[:, sl] @ w[:, sl].T)
    low = T @ bf16_to_f64(L2_bf16).T if T.shape[1] > 0 else np.zeros((M, N), dtype=F64)
    Y = main + low
    if bias_bf16 is not None:
        Y = Y + bf16_to_f64(bias_bf16)[None, :]
    return _activate(Y, activation)


def rel_fro(Y, Yref) -> float:
    Y = np.asarray(Y, dtype=F64)
    Yref = np.asarray(Yref, dtype=F64)
    return float(np.linalg.norm(Y - Yref) / max(np.linalg.norm(Yref), 1e-300))


def max_abs_ratio(Y, Yref) -> float:
    Y = np.asarray(Y, dtype=F64)
    Yref = np.asarray(Yref, dtype=F64)
    return float(np.max(np.abs(Y - Yref)) / max(np.max(np.abs(Yref)), 1e-300))

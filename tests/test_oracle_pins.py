"""Pins for the CPU oracle, each one fixed by the pages or by mathematics, not by
re-typing the oracle's own formulas.

Citations: [Term] = the "SVDQuant Low-Rank Residual Quantization Algorithm
Terminology Entry", section 2.3 (equations E1-E7 as numbered in the oracle's
header); [Abs] = the SVDQuant abstract page.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import svdq_oracle as numpy_oracle
from oracle import svdq_ref as c_oracle
import synth

F32, F64 = np.float32, np.float64


@pytest.fixture(params=["numpy", "c"])
def O(request):
    """Every pin runs on both oracles: the numpy one and the plain C one (oracle/svdq_ref.c),
    two independent implementations of the same contract."""
    return numpy_oracle if request.param == "numpy" else c_oracle


def _bits(x):
    return np.asarray(x, dtype=F32).view(np.uint32)


# ------------------------------------------------------------ bfloat16 helper
def test_bf16_matches_torch_on_float32_inputs(O):
    g = np.random.Generator(np.random.PCG64(1))
    x = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000),
                        np.array([0.0, -0.0, 1.00390625, 1.01171875, 3.0e38, 1e-40, -1e-41])]).astype(F32)
    ours = O.bf16_from_f64(x.astype(F64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounds_float64_once(O):
    # 1 + 2^-8 + 2^-40 lies above the tie: one rounding gives 1 + 2^-7.
    # (Rounding to float32 first would land on the tie and then go to 1.0.)
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert O.bf16_to_f64(O.bf16_from_f64(np.array([v])))[0] == 1.0 + 2.0 ** -7
    # exact ties go to even
    assert O.bf16_to_f64(O.bf16_from_f64(np.array([1.0 + 2.0 ** -8])))[0] == 1.0
    assert O.bf16_to_f64(O.bf16_from_f64(np.array([1.0 + 3 * 2.0 ** -8])))[0] == 1.0 + 2.0 ** -6


# -------------------------------------------------------------- stage one (E1, E2)
def test_act_and_weight_absmax_by_hand(O):
    X = synth.f32_to_bf16_bits(np.array([[1.0, -3.0, 0.5], [-2.0, 2.0, -0.25]], dtype=F32))
    np.testing.assert_array_equal(O.act_absmax(X), np.array([2.0, 3.0, 0.5], dtype=F32))
    W = np.array([[0.5, -4.0], [-1.5, 1.0], [1.0, 0.25]], dtype=F32)  # [N=3, K=2]
    np.testing.assert_array_equal(O.weight_absmax(W), np.array([1.5, 4.0], dtype=F32))


def test_smoothing_closed_forms(O):
    A = np.array([4.0, 9.0, 0.5, 0.0], dtype=F32)
    Wsc = np.array([0.25, 0.5, 2.0, 0.0], dtype=F32)
    # alpha = 1: s = A (floored statistics)
    np.testing.assert_array_equal(O.smoothing_factors(A, Wsc, 1.0), np.array([4.0, 9.0, 0.5, 1e-5], dtype=F32))
    # alpha = 0: s = 1 / W_scale
    np.testing.assert_array_equal(O.smoothing_factors(A, Wsc, 0.0),
                                  np.array([4.0, 2.0, 0.5, 1e5], dtype=F32))
    # alpha = 1/2: s = sqrt(A / W_scale); A = 4, W_scale = 1/4 gives 4 exactly
    s = O.smoothing_factors(A, Wsc, 0.5)
    assert s[0] == 4.0 and s[2] == 0.5 and s[3] == 1.0
    assert abs(float(s[1]) - math.sqrt(9.0) / math.sqrt(0.5)) < 1e-6 * 4.3
    # s_min holds
    assert O.smoothing_factors(np.array([1e-9], F32), np.array([10.0], F32), 0.5, s_min=1e-2)[0] == F32(1e-2)


def test_smoothing_is_an_identity_E1(O):
    w = synth.WORKLOADS["tiny"]
    X = synth.activations(w)[:64]
    W = synth.weight(w)[:96]                      # N != K catches a transposed scaling
    s = O.smoothing_factors(O.act_absmax(X), O.weight_absmax(W), 0.5)
    ref = O.bf16_to_f64(X) @ W.astype(F64).T
    exact = (O.bf16_to_f64(X) / s.astype(F64)[None, :]) @ O.smooth_weight(W, s).T
    assert O.rel_fro(exact, ref) < 1e-13
    # the float32 smoothed activations the method quantizes keep the identity to float32 accuracy
    fl = O.smooth_activations(X, s).astype(F64) @ O.smooth_weight(W, s).T
    assert O.rel_fro(fl, ref) < 1e-6


# --------------------------------------------------------- stage two (E3, E5, E6)
def test_svd_special_cases(O):
    d = np.array([0.5, -3.0, 2.0, 0.0, 1.0])
    U, S, V = O.svd_sorted(np.diag(d))
    np.testing.assert_allclose(S, [3.0, 2.0, 1.0, 0.5, 0.0], atol=1e-15)
    u = np.array([1.0, 2.0, -2.0])
    v = np.array([3.0, 0.0, 4.0, 0.0])
    _, S, _ = O.svd_sorted(np.outer(u, v))
    assert abs(S[0] - 15.0) < 1e-13 and np.all(np.abs(S[1:]) < 1e-13)
    # 2x2 closed form: singular values of [[a, b], [0, c]]
    a, b, c = 3.0, 4.0, 2.0
    tr = a * a + b * b + c * c
    det = (a * c) ** 2
    s1 = math.sqrt((tr + math.sqrt(tr * tr - 4 * det)) / 2)
    s2 = math.sqrt((tr - math.sqrt(tr * tr - 4 * det)) / 2)
    _, S, _ = O.svd_sorted(np.array([[a, b], [0.0, c]]))
    np.testing.assert_allclose(S, [s1, s2], rtol=1e-14)


def test_svd_recovers_a_pure_spike(O):
    w = synth.WORKLOADS["tiny"]
    g = synth.rng_for("tiny", 1)
    U0, _ = np.linalg.qr(g.standard_normal((300, 8)))
    V0, _ = np.linalg.qr(g.standard_normal((200, 8)))
    sig = np.linspace(5, 1, 8)
    U, S, V = O.svd_sorted((U0 * sig) @ V0.T)
    np.testing.assert_allclose(S[:8], sig, rtol=1e-12)
    assert np.all(S[8:] < 1e-12)
    # sign convention: the largest-magnitude entry of each v_i is positive
    idx = np.argmax(np.abs(V[:, :8]), axis=0)
    assert np.all(V[idx, np.arange(8)] > 0)


@pytest.mark.parametrize("r", [0, 4, 16])
def test_eckart_young_and_orthogonality_E5_E6(O, r):
    w = synth.WORKLOADS["tiny"]
    W = synth.weight(w)[:160, :192]
    s = O.smoothing_factors(np.ones(192, F32), O.weight_absmax(W), 0.5)
    What = O.smooth_weight(W, s)
    U, S, V = O.svd_sorted(What)
    assert np.all(np.diff(S) <= 0)
    p = S.shape[0]
    np.testing.assert_allclose(U.T @ U, np.eye(p), atol=1e-12)
    np.testing.assert_allclose(V.T @ V, np.eye(p), atol=1e-12)
    fro2 = float(np.sum(What ** 2))
    assert abs(fro2 - float(np.sum(S ** 2))) < 1e-12 * fro2
    L = (U[:, :r] * S[:r]) @ V[:, :r].T
    tail = float(np.sum(S[r:] ** 2))
    assert abs(float(np.sum((What - L) ** 2)) - tail) < 1e-10 * fro2
    # optimality: random rank-r competitors built from perturbed subspaces do worse
    g = synth.rng_for("tiny", 2)
    for _ in range(3):
        if r == 0:
            break
        Q, _ = np.linalg.qr(V[:, :r] + 0.05 * g.standard_normal((192, r)))
        Lc = (What @ Q) @ Q.T                    # best approximation within that row space
        assert float(np.sum((What - Lc) ** 2)) > tail


def test_lowrank_factors_put_sigma_on_lora_up(O):
    w = synth.WORKLOADS["tiny"]
    W = synth.weight(w)[:128, :256]
    U, S, V = O.svd_sorted(W.astype(F64))
    L1, L2 = O.lowrank_factors(U, S, V, 8)
    assert L1.shape == (8, 256) and L2.shape == (128, 8)
    # lora_down rows are unit vectors (to bfloat16 accuracy); lora_up columns carry sigma
    np.testing.assert_allclose(np.linalg.norm(O.bf16_to_f64(L1), axis=1), 1.0, rtol=1e-2)
    np.testing.assert_allclose(np.linalg.norm(O.bf16_to_f64(L2), axis=0), S[:8], rtol=1e-2)
    # L2 L1 approximates W_r with the tail energy (E6) up to bfloat16 rounding
    Lr = O.bf16_to_f64(L2) @ O.bf16_to_f64(L1)
    err2 = float(np.sum((W.astype(F64) - Lr) ** 2))
    assert abs(err2 - float(np.sum(S[8:] ** 2))) < 2e-2 * float(np.sum(S[:8] ** 2)) ** 0.5 * 2 ** -6


def test_residual_of_an_exact_lowrank_weight_is_zero(O):
    """W_hat = L2 L1 exactly (dyadic factors, N != K): R = W_hat - L2 L1 must be exactly 0."""
    g = synth.rng_for("tiny", 3)
    K, N, r = 192, 128, 5
    L1v = g.integers(-16, 17, (r, K)) / 16.0
    L2v = g.integers(-16, 17, (N, r)) / 8.0
    L1 = O.bf16_from_f64(L1v)
    L2 = O.bf16_from_f64(L2v)
    What = L2v @ L1v
    R = O.residual(What, L1, L2)
    assert R.dtype == F32 and np.all(R == 0)
    q, sc = O.quantize_groups(R, weight_scale=True)
    assert np.all(q == 0) and np.all(sc == 0)
    # and a non-zero remainder survives exactly where it was put
    What2 = What.copy()
    What2[3, 70] += 0.75
    R2 = O.residual(What2, L1, L2)
    assert R2[3, 70] == F32(0.75) and np.count_nonzero(R2) == 1


# -------------------------------------------------------------------- Q (E4)
def test_quantizer_ties_go_to_even_by_hand(O):
    v = np.zeros(64, F32)
    v[:8] = [7.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -7.0]
    q, sc = O.quantize_groups(v[None, :])
    assert sc[0, 0] == 1.0
    np.testing.assert_array_equal(q[0, :8], [7, 2, 4, -2, 0, 2, 0, -7])
    # a = 3.5: scale = 0.5, inv = 2 -> 1.25 * 2 = 2.5 -> 2, 1.75 * 2 = 3.5 -> 4
    v = np.zeros(64, F32)
    v[:3] = [3.5, 1.25, -1.75]
    q, sc = O.quantize_groups(v[None, :])
    assert sc[0, 0] == 0.5
    np.testing.assert_array_equal(q[0, :3], [7, 2, -4])


def test_quantizer_zero_group_and_absmax_code(O):
    v = np.zeros((2, 128), F32)
    v[1, 64:] = np.linspace(-0.3, 0.9, 64, dtype=F32)
    q, sc = O.quantize_groups(v)
    assert sc[0, 0] == 0 and sc[0, 1] == 0 and sc[1, 0] == 0 and np.all(q[0] == 0)
    assert q[1, 127] == 7 and sc[1, 1] == F32(F32(0.9) / F32(7))


def test_quantizer_error_bound_and_range(O):
    g = synth.rng_for("tiny", 4)
    v = (g.standard_normal((64, 1024)) * np.exp(g.uniform(-8, 8, (64, 1)))).astype(F32)
    for wscale in (False, True):
        q, sc = O.quantize_groups(v, weight_scale=wscale)
        assert q.min() >= -7 and q.max() <= 7
        deq = q.reshape(64, 16, 64).astype(F64) * sc.astype(F64)[..., None]
        err = np.abs(v.reshape(64, 16, 64).astype(F64) - deq)
        assert np.all(err <= sc.astype(F64)[..., None] / 2 * (1 + 2.0 ** -16) + 1e-300)
        # the group's absmax element maps to +-7
        amax_idx = np.argmax(np.abs(v.reshape(64, 16, 64)), axis=-1)
        got = np.take_along_axis(np.abs(q.reshape(64, 16, 64)), amax_idx[..., None], -1)
        assert np.all(got == 7)
    # weight scales have the two low significand bits clear, so 3 * scale is exact in float32
    assert np.all((_bits(sc) & 3) == 0)
    assert np.all((F32(3) * sc).astype(F64) == 3.0 * sc.astype(F64))


def test_quantizer_tiny_groups(O):
    """The reading for groups far below float32's normal range: absmax < 2^-100 is a zero
    group (7/a would near the float32 overflow at about 2^-125.5, and 0 * inf would be NaN).
    At and above 2^-100 the codes are those of the same group scaled up by a power of two
    (equivariance holds exactly there, subnormal members included) and the scale is the
    scaled group's scale scaled back."""
    g = np.random.default_rng(77)
    base = np.clip(g.standard_normal((3, 64)) * 3, -4.9, 4.9).astype(F32)
    base[:, 0] = 5.0                                # a fixed absmax: scaled groups hit the threshold exactly
    base[1, 1:8] = 1e-30                            # members that go subnormal when scaled down
    q0, s0 = O.quantize_groups(base)
    at = (base.astype(F64) * 2.0 ** -100 / 5.0).astype(F32)     # absmax exactly 2^-100
    assert np.all(np.max(np.abs(at), axis=1) == F32(2.0 ** -100))
    q1, s1 = O.quantize_groups(at)
    scaled = (at.astype(F64) * 2.0 ** 100).astype(F32)
    q1s, s1s = O.quantize_groups(scaled)
    np.testing.assert_array_equal(q1, q1s)
    assert np.all(s1 == (s1s.astype(F64) * 2.0 ** -100).astype(F32))
    below = (at.astype(F64) / 2).astype(F32)        # absmax 2^-101, members deep in subnormals
    q2, s2 = O.quantize_groups(below)
    assert np.all(q2 == 0) and np.all(s2 == 0)
    sub = np.full((1, 64), F32(1e-40))              # an all-subnormal group
    sub[0, ::2] *= -1
    q3, s3 = O.quantize_groups(sub)
    assert np.all(q3 == 0) and np.all(s3 == 0)
    with np.errstate(all="raise"):                  # no overflow, no 0 * inf anywhere
        O.quantize_groups(np.concatenate([at, below, sub]))


def test_quantizer_power_of_two_equivariance(O):
    g = synth.rng_for("tiny", 5)
    v = g.standard_normal((8, 256)).astype(F32)
    q0, s0 = O.quantize_groups(v)
    for k in (-5, 3, 11):
        q1, s1 = O.quantize_groups((v * F32(2.0 ** k)).astype(F32))
        np.testing.assert_array_equal(q1, q0)
        np.testing.assert_array_equal(s1, s0 * F32(2.0 ** k))


def test_nibble_packing_by_hand(O):
    q = np.array([[1, -1, 7, -7, 0, 3] + [0] * 58], dtype=np.int8)
    b = O.pack_nibbles(q)
    assert b.shape == (1, 32)
    assert list(b[0, :3]) == [0xF1, 0x97, 0x30]
    np.testing.assert_array_equal(O.unpack_nibbles(b), q)


def test_group_partials_brute_force(O):
    g = synth.rng_for("tiny", 6)
    qx = g.integers(-7, 8, (3, 128)).astype(np.int8)
    qw = g.integers(-7, 8, (5, 128)).astype(np.int8)
    P = O.group_partials(O.pack_nibbles(qx), O.pack_nibbles(qw))
    assert P.shape == (3, 5, 2)
    for m in range(3):
        for n in range(5):
            for gg in range(2):
                acc = 0
                for k in range(64 * gg, 64 * gg + 64):
                    acc += int(qx[m, k]) * int(qw[n, k])
                assert P[m, n, gg] == acc
    # extreme codes: |P| reaches 64 * 49
    P = O.group_partials(O.pack_nibbles(np.full((1, 64), -7, np.int8)), O.pack_nibbles(np.full((1, 64), 7, np.int8)))
    assert P[0, 0, 0] == -3136


# --------------------------------------------------------------- forward (E4, E7)
def _lossless_problem(O, M=6, K=128, N=96, r=3, seed=7):
    """Inputs on which both quantizers are lossless, so E4 holds with equality:
    Y must equal X W^T + b up to float64 rounding."""
    g = synth.rng_for("tiny", seed)
    G = K // 64
    s = (2.0 ** g.integers(-2, 3, K)).astype(F32)
    # activations: x_hat = q * 2^e with each group's absmax code = 7
    qx = g.integers(-7, 8, (M, K))
    qx[:, ::64] = 7 * np.where(g.random((M, G)) < 0.5, 1, -1)
    ex = 2.0 ** g.integers(-3, 2, (M, G))
    xh = qx * np.repeat(ex, 64, axis=1)
    X = synth.f32_to_bf16_bits((xh * s[None, :]).astype(F32))
    assert np.all(O.bf16_to_f64(X) == xh * s[None, :])
    # residual: R = q * 2^f with each group's absmax code = 7
    qr = g.integers(-7, 8, (N, K))
    qr[:, 5::64] = 7
    ew = 2.0 ** g.integers(-6, -2, (N, G))
    R = qr * np.repeat(ew, 64, axis=1)
    L1v = g.integers(-8, 9, (r, K)) / 8.0
    L2v = g.integers(-8, 9, (N, r)) / 16.0
    What = R + L2v @ L1v
    W = (What / s[None, :].astype(F64)).astype(F32)
    assert np.all(W.astype(F64) * s[None, :] == What)
    b = synth.f32_to_bf16_bits(g.standard_normal(N).astype(F32))
    return X, W, s, O.bf16_from_f64(L1v), O.bf16_from_f64(L2v), b


def test_forward_equals_xw_plus_b_when_quantization_is_lossless(O):
    X, W, s, L1, L2, b = _lossless_problem(O)
    Wq, ws = O.quantize_residual(W, s, L1, L2)
    Y = O.forward(X, s, L1, L2, Wq, ws, b)
    Yx = O.forward_exact(X, W, b)
    assert O.rel_fro(Y, Yx) < 1e-14
    # dropping either branch or the bias breaks it
    Y0 = O.forward(X, s, np.zeros((0, W.shape[1]), np.uint16), np.zeros((W.shape[0], 0), np.uint16), Wq, ws, b)
    assert O.rel_fro(Y0, Yx) > 1e-3
    assert O.rel_fro(O.forward(X, s, L1, L2, Wq, ws, None), Yx) > 1e-3


def test_rank_zero_collapses_to_plain_w4a4(O):
    w = synth.WORKLOADS["tiny"]
    X = synth.activations(w)[:32]
    W = synth.weight(w)[:80]
    b = synth.bias(w)[:80]
    A = O.act_absmax(synth.calibration_activations(w))
    pk = O.pack_weights(W, A, 0.5, rank=0)
    assert np.all(pk["R"] == pk["What"].astype(F32))
    Y = O.forward(X, pk["s"], pk["L1"], pk["L2"], pk["Wq"], pk["w_scales"], b)
    # independent route: dequantize both operands, one float64 matrix product
    qx, sx, _, _ = O.quantize_activations(X, pk["s"])
    dx = O.unpack_nibbles(qx).astype(F64) * np.repeat(sx.astype(F64), 64, axis=1)
    dw = O.unpack_nibbles(pk["Wq"]).astype(F64) * np.repeat(pk["w_scales"].astype(F64), 64, axis=1)
    Yd = dx @ dw.T + O.bf16_to_f64(b)[None, :]
    assert O.rel_fro(Y, Yd) < 1e-13
    # s = 1 gives the naive W4A4 of the unsmoothed operands
    pk1 = O.pack_weights(W, O.weight_absmax(W), 0.5, rank=0)
    assert np.all(pk1["s"] == 1.0)


def test_svdquant_beats_smoothing_alone_beats_naive(O):
    """[Abs]: smoothing alone is insufficient at 4 bits; the low-rank branch absorbs the outliers."""
    w = synth.WORKLOADS["tiny"]
    X = synth.activations(w)
    W = synth.weight(w)[:256]          # the first 256 output rows; every input channel
    b = synth.bias(w)[:256]
    A = O.act_absmax(synth.calibration_activations(w))
    Yx = O.forward_exact(X, W, b)
    errs = {}
    for name, AA, r in (("svdq", A, 16), ("smooth", A, 0), ("naive", O.weight_absmax(W), 0)):
        pk = O.pack_weights(W, AA, 0.5, rank=r)
        Y = O.forward(X, pk["s"], pk["L1"], pk["L2"], pk["Wq"], pk["w_scales"], b)
        errs[name] = O.rel_fro(Y, Yx)
    assert errs["svdq"] < errs["smooth"] < errs["naive"], errs


def test_activation_codes_power_of_two_equivariance(O):
    w = synth.WORKLOADS["tiny"]
    X = synth.activations(w)[:16]
    s = O.smoothing_factors(O.act_absmax(X), np.full(w.K, 0.1, F32), 0.5)
    qx0, sx0, _, _ = O.quantize_activations(X, s)
    X4 = synth.f32_to_bf16_bits(O.bf16_to_f32(X) * F32(4))
    qx1, sx1, _, _ = O.quantize_activations(X4, s)
    np.testing.assert_array_equal(qx1, qx0)
    np.testing.assert_array_equal(sx1, sx0 * F32(4))


def test_quantizer_matches_exact_rational_evaluation(O):
    """Each rounding point of Q evaluated with exact rationals and one IEEE rounding each."""
    g = synth.rng_for("tiny", 8)
    v = (g.standard_normal(64) * 3).astype(F32)

    def rn32(fr):                      # round a Fraction to the nearest float32 (ties to even)
        f = F32(float(fr))             # float(Fraction) is correctly rounded to float64
        lo, hi = sorted([f, np.nextafter(f, F32(np.inf) if Fraction(float(f)) < fr else F32(-np.inf))])
        dlo, dhi = abs(Fraction(float(lo)) - fr), abs(Fraction(float(hi)) - fr)
        if dlo != dhi:
            return lo if dlo < dhi else hi
        return lo if (_bits(lo) & 1) == 0 else hi

    a = max(abs(Fraction(float(x))) for x in v)
    scale = rn32(a / 7)
    inv = rn32(7 / a)
    want = []
    for x in v:
        t = Fraction(float(rn32(Fraction(float(x)) * Fraction(float(inv)))))
        fl = math.floor(t)
        d = t - fl
        qi = fl + (1 if d > Fraction(1, 2) or (d == Fraction(1, 2) and fl % 2 == 1) else 0)
        want.append(max(-7, min(7, qi)))
    q, sc = O.quantize_groups(v[None, :])
    assert sc[0, 0] == scale
    np.testing.assert_array_equal(q[0], np.array(want, np.int8))


def _rn32(fr):
    """Round a Fraction to the nearest float32, ties to even (one IEEE rounding)."""
    f = F32(float(fr))
    lo, hi = sorted([f, np.nextafter(f, F32(np.inf) if Fraction(float(f)) < fr else F32(-np.inf))])
    dlo, dhi = abs(Fraction(float(lo)) - fr), abs(Fraction(float(hi)) - fr)
    if dlo != dhi:
        return lo if dlo < dhi else hi
    return lo if (_bits(lo) & 1) == 0 else hi


def _q_exact(vals, weight):
    """Q of one 64-group with exact rationals: scale fl32(a/7) (weights: two low
    significand bits cleared), inv fl32(7/a), q = clamp(rne(fl32(v inv)), -7, 7)."""
    a = max(abs(v) for v in vals)
    if a < Fraction(2) ** -100:          # a zero group, as the contract reads it
        return [0] * len(vals), Fraction(0)
    scale = _rn32(a / 7)
    if weight:
        scale = (np.asarray([scale], F32).view(np.uint32) & np.uint32(0xFFFFFFFC)).view(F32)[0]
    inv = Fraction(float(_rn32(7 / a)))
    q = []
    for v in vals:
        t = Fraction(float(_rn32(v * inv)))
        fl = math.floor(t)
        d = t - fl
        qi = fl + (1 if d > Fraction(1, 2) or (d == Fraction(1, 2) and fl % 2 == 1) else 0)
        q.append(max(-7, min(7, qi)))
    return q, Fraction(float(scale))


@pytest.mark.parametrize("K,r", [(64, 0), (64, 1), (128, 0), (128, 1)])
def test_forward_matches_exact_rationals(O, K, r):
    """Brute force with Fractions on tiny layers ([Term] 2.3, E1 and E4): smoothing,
    the residual R = W diag(s) - L2 L1, both quantizations, the exact group products,
    the low-rank branch and the bias, each rounding point taken once as the contract
    fixes it.  Dyadic X, W, L1, L2, b and power-of-two s keep the smoothing exact, so
    the oracle's codes, scales and P must match exactly and its float64 Y to 1e-15."""
    g = np.random.default_rng(100 + K + r)
    M, N = 2, 2
    X = synth.f32_to_bf16_bits((g.integers(-64, 64, (M, K)) / 16.0).astype(F32))
    s = np.ldexp(np.ones(K, F32), g.integers(-2, 3, K)).astype(F32)
    W = (g.integers(-64, 64, (N, K)) / 32.0).astype(F32)
    L1 = synth.f32_to_bf16_bits((g.integers(-8, 8, (r, K)) / 8.0).astype(F32))
    L2 = synth.f32_to_bf16_bits((g.integers(-8, 8, (N, r)) / 4.0).astype(F32))
    b = synth.f32_to_bf16_bits((g.integers(-8, 8, N) / 8.0).astype(F32))

    xv = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(X)]
    sv = [Fraction(float(v)) for v in s]
    l1 = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(L1)]
    l2 = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(L2)]
    xh = [[x * Fraction(float(_rn32(1 / sk))) for x, sk in zip(row, sv)] for row in xv]
    R = [[Fraction(float(_rn32(Fraction(float(W[n, k])) * sv[k] - sum(l2[n][j] * l1[j][k] for j in range(r)))))
          for k in range(K)] for n in range(N)]
    G = K // 64
    qx, sx = [[None] * G for _ in range(M)], [[None] * G for _ in range(M)]
    qw, sw = [[None] * G for _ in range(N)], [[None] * G for _ in range(N)]
    for gi in range(G):
        sl = slice(64 * gi, 64 * gi + 64)
        for m in range(M):
            qx[m][gi], sx[m][gi] = _q_exact(xh[m][sl], weight=False)
        for n in range(N):
            qw[n][gi], sw[n][gi] = _q_exact(R[n][sl], weight=True)
    T = [[sum(xh[m][k] * l1[j][k] for k in range(K)) for j in range(r)] for m in range(M)]

    pk = O.quantize_activations(X, s, L1)
    codes = O.unpack_nibbles(pk[0])
    Wq, wsc = O.quantize_residual(W, s, L1, L2)
    wcodes = O.unpack_nibbles(Wq)
    P = O.group_partials(pk[0], Wq)
    Y = O.forward(X, s, L1, L2, Wq, wsc, b)
    for gi in range(G):
        for m in range(M):
            assert list(codes[m, 64 * gi:64 * gi + 64]) == qx[m][gi]
            assert Fraction(float(pk[1][m, gi])) == sx[m][gi]
        for n in range(N):
            assert list(wcodes[n, 64 * gi:64 * gi + 64]) == qw[n][gi]
            assert Fraction(float(wsc[n, gi])) == sw[n][gi]
    bv = [Fraction(float(v)) for v in O.bf16_to_f64(b)]
    for m in range(M):
        for n in range(N):
            want = bv[n] + sum(T[m][j] * l2[n][j] for j in range(r))
            for gi in range(G):
                p_exact = sum(a * w for a, w in zip(qx[m][gi], qw[n][gi]))
                assert P[m, n, gi] == p_exact
                want += sx[m][gi] * sw[n][gi] * p_exact
            assert abs(Fraction(float(Y[m, n])) - want) <= abs(want) * Fraction(1, 10 ** 15)


def test_quantizer_golden_examples(O):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "quantizer_examples.txt")
    n = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        vals, scale, codes = [p.split() for p in line.split("|")]
        v = np.zeros(64, F32)
        v[:len(vals)] = [float(t) for t in vals]
        q, sc = O.quantize_groups(v[None, :])
        assert sc[0, 0] == F32(float(scale[0]))
        np.testing.assert_array_equal(q[0, :len(codes)], [int(c) for c in codes])
        n += 1
    assert n == 4


# ------------------------------------------------------- LoRA concatenation
def test_append_lora_adds_exactly_x_a_b(O):
    """[Abs] LoRAs attach without re-quantization.  With power-of-two smoothing
    factors and factors whose scaled values are bf16 numbers, every rounding on
    the branch is exact, so the adapter's rows of T equal X A exactly and the
    output grows by exactly (X A) B; Q(R) and the original rank are untouched."""
    g = np.random.default_rng(11)
    M, K, N, r, rl = 8, 128, 48, 16, 16
    s = (2.0 ** g.integers(-3, 4, size=K)).astype(F32)
    X = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(F32))
    W = (g.standard_normal((N, K)) * 0.1).astype(F32)
    A_scaled = O.bf16_to_f32(synth.f32_to_bf16_bits(g.standard_normal((K, rl)).astype(F32) * 0.05))
    A = (A_scaled / s[:, None]).astype(F32)              # A * s is a bf16 number, exactly
    B = O.bf16_to_f32(synth.f32_to_bf16_bits(g.standard_normal((rl, N)).astype(F32) * 0.05))
    L1 = synth.f32_to_bf16_bits(g.standard_normal((r, K)).astype(F32) * 0.1)
    L2 = synth.f32_to_bf16_bits(g.standard_normal((N, r)).astype(F32) * 0.1)
    Wq, ws = O.quantize_residual(W, s, L1, L2)
    L1n, L2n = O.append_lora(s, L1, L2, A, B)
    assert L1n.shape == (r + rl, K) and L2n.shape == (N, r + rl)
    np.testing.assert_array_equal(L1n[:r], L1)
    np.testing.assert_array_equal(L2n[:, :r], L2)
    _, _, T0, _ = O.quantize_activations(X, s, L1)
    _, _, T1, _ = O.quantize_activations(X, s, L1n)
    XA = O.bf16_to_f64(X) @ A.astype(F64)
    np.testing.assert_array_equal(T1[:, :r], T0)
    np.testing.assert_allclose(T1[:, r:], XA, rtol=1e-12, atol=1e-12 * np.abs(XA).max())
    d = O.forward(X, s, L1n, L2n, Wq, ws) - O.forward(X, s, L1, L2, Wq, ws)
    XAB = XA @ B.astype(F64)
    assert np.max(np.abs(d - XAB)) <= 1e-12 * np.max(np.abs(XAB))


def test_append_lora_transposes_and_scales_per_input_channel(O):
    """The adapter's down factor is scaled per input channel k (not per output):
    one nonzero A entry at (k, j) lands at L1'[r + j, k] as bf16(A[k, j] s[k])."""
    K, N, rl = 64, 16, 16
    s = np.ones(K, F32)
    s[5] = 4.0
    A = np.zeros((K, rl), F32)
    A[5, 3] = 0.75
    B = np.zeros((rl, N), F32)
    B[3, 9] = -1.5
    L1n, L2n = O.append_lora(s, np.zeros((0, K), np.uint16), np.zeros((N, 0), np.uint16), A, B)
    assert O.bf16_to_f64(L1n)[3, 5] == 3.0 and np.count_nonzero(L1n) == 1
    assert O.bf16_to_f64(L2n)[9, 3] == -1.5 and np.count_nonzero(L2n) == 1


# ------------------------------------------------------------------- MXFP4
def test_e2m1_decode_table(O):
    """All 16 E2M1 patterns: sign bit 3, then (exponent, significand) = bits 2..1, bit 0."""
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    got = O.e2m1_value(np.arange(16))
    np.testing.assert_array_equal(got, want)
    assert np.signbit(got[8])


def test_e2m1_round_ties_even_and_saturation(O):
    """Hand-derived: midpoints go to the even significand (0, 1, 1, 2, 2, 4, 4); past 5
    everything is 6, including values far beyond the largest E2M1 number."""
    y = [0.0, 0.2499, 0.25, 0.2501, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0,
         5.0001, 6.0, 7.0, 100.0]
    want_val = [0, 0, 0, 0.5, 0.5, 1, 1, 1, 1.5, 2, 2, 2, 3, 4, 4, 4, 6, 6, 6, 6]
    idx = O.e2m1_round(y)
    np.testing.assert_array_equal(np.asarray(O.E2M1_MAG)[idx], want_val)


def test_mx_shared_exponent_rule(O):
    """OCP MX v1.0 with E2M1 (largest value 1.5 * 2^2): e = floor(log2 amax) - 2."""
    amax = [1.0, 1.5, 3.999, 4.0, 6.0, 7.99, 8.0, 0.75, 2.0 ** -100, 0.0, 1e-45, 3e38]
    want = [-2, -2, -1, 0, 0, 0, 1, -3, -102, -127, -127, 125]
    np.testing.assert_array_equal(O.mx_shared_exponent(np.asarray(amax, F32)), want)


def test_mx_block_error_bound_and_range(O):
    """Every element lies within half a grid step of its code (the step is 0.5, 1 or 2
    times 2^e in [0, 2), [2, 4), [4, 6]), except saturated ones, which the scale rule
    keeps below 8 * 2^e, i.e. within 2 * 2^e of 6 * 2^e; codes are valid patterns."""
    g = np.random.default_rng(21)
    v = (g.standard_normal((64, 256)) * np.exp(g.uniform(-8, 8, (64, 1)))).astype(F32)
    v[:, :40] *= 30.0
    codes, e = O.quantize_mx(v)
    assert codes.max() <= 15
    scale = np.repeat(np.exp2(e.astype(F64)), 32, axis=1)
    q = O.e2m1_value(codes) * scale
    y = np.abs(v.astype(F64)) / scale
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    err = np.abs(v.astype(F64) - q)
    sat = y > 6
    assert np.all(err[~sat] <= 0.5 * step[~sat] * scale[~sat])
    assert np.all(y < 8) and np.all(err[sat] <= 2 * scale[sat])


def test_mx_power_of_two_equivariance(O):
    g = np.random.default_rng(22)
    v = g.standard_normal((8, 128)).astype(F32)
    c0, e0 = O.quantize_mx(v)
    c1, e1 = O.quantize_mx(v * F32(2.0 ** 7))
    np.testing.assert_array_equal(c1, c0)
    np.testing.assert_array_equal(e1, e0 + 7)


def _mx_exact_rows(O, g, rows, K):
    """Rows that MXFP4 represents exactly: E2M1 values times a power of two per block,
    with one +-4 or +-6 per block so that the scale rule picks that power."""
    codes = g.integers(0, 16, size=(rows, K))
    codes[:, ::32] = g.choice([6, 7, 14, 15], size=(rows, K // 32))
    e = g.integers(-4, 5, size=(rows, K // 32))
    return O.e2m1_value(codes) * np.repeat(np.exp2(e.astype(F64)), 32, axis=1)


def test_mx_forward_lossless_limit(O):
    """With X and W exactly representable in MXFP4, s = 1 and no low-rank branch, the
    MXFP4 forward is exactly X W^T + b: this pins the block pairing along K, the
    addition of the two block exponents and the packing order of the codes."""
    g = np.random.default_rng(23)
    M, N, K = 6, 5, 128
    X = synth.f32_to_bf16_bits(_mx_exact_rows(O, g, M, K).astype(F32))
    W = _mx_exact_rows(O, g, N, K).astype(F32)
    assert np.array_equal(O.bf16_to_f64(X), _mx_exact_rows(O, np.random.default_rng(23), M, K))
    s = np.ones(K, F32)
    b = synth.f32_to_bf16_bits(g.standard_normal(N).astype(F32))
    none1, none2 = np.zeros((0, K), np.uint16), np.zeros((N, 0), np.uint16)
    Wq, we = O.quantize_residual_mx(W, s, none1, none2)
    Y = O.forward_mx(X, s, none1, none2, Wq, we, b)
    np.testing.assert_array_equal(Y, O.forward_exact(X, W, b))


def test_mx_forward_matches_exact_rationals(O):
    """Brute force with Fractions on a tiny layer: the MXFP4 contract evaluated exactly
    (block exponents from each block's absmax, nearest E2M1 values, exact sums) equals
    the oracle's float64 forward (r = 0, s = 1, dyadic inputs: every sum is exact)."""
    from fractions import Fraction as Fr
    g = np.random.default_rng(24)
    M, N, K = 2, 3, 64
    X = synth.f32_to_bf16_bits((g.integers(-64, 64, (M, K)) / 16.0).astype(F32))
    W = (g.integers(-64, 64, (N, K)) / 32.0).astype(F32)
    s = np.ones(K, F32)
    none1, none2 = np.zeros((0, K), np.uint16), np.zeros((N, 0), np.uint16)
    Wq, we = O.quantize_residual_mx(W, s, none1, none2)
    Y = O.forward_mx(X, s, none1, none2, Wq, we)
    mags = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]

    def q_block(vals):
        vals = [Fr(float(v)) for v in vals]
        amax = max(abs(v) for v in vals)
        e = -127
        if amax:
            fl = 0
            while Fr(2) ** (fl + 1) <= amax:
                fl += 1
            while Fr(2) ** fl > amax:
                fl -= 1
            e = fl - 2
        out = []
        for v in vals:
            y = abs(v) / Fr(2) ** e
            d = [abs(y - m) for m in mags]
            best = min(range(8), key=lambda i: (d[i], i % 2))
            out.append((-1 if v < 0 else 1) * mags[best] * Fr(2) ** e)
        return out

    xv = O.bf16_to_f64(X)
    for m in range(M):
        for n in range(N):
            acc = Fr(0)
            for blk in range(K // 32):
                sl = slice(32 * blk, 32 * blk + 32)
                acc += sum(a * w for a, w in zip(q_block(xv[m, sl]), q_block(W[n, sl])))
            assert Fr(Y[m, n]) == acc


@pytest.mark.parametrize("K,r", [(64, 1), (128, 2)])
def test_mx_forward_with_lowrank_branch_matches_exact_rationals(O, K, r):
    """The MXFP4 forward with its low-rank branch and bias, brute force with Fractions
    ([Term] 2.3, E4: both terms): smoothing by power-of-two s, the residual
    R = W diag(s) - L2 L1 rounded once to float32, block exponents from each block's
    absmax, nearest E2M1 values, T = x_hat L1^T and T L2^T.  The exact T and the exact
    Y must equal the oracle's (dyadic inputs keep every float64 sum exact), so a
    transposed L2, T taken from X instead of x_hat, a dropped term or a residual of
    the wrong sign fails here."""
    from fractions import Fraction as Fr
    g = np.random.default_rng(300 + K + r)
    M, N = 2, 3
    X = synth.f32_to_bf16_bits((g.integers(-64, 64, (M, K)) / 16.0).astype(F32))
    s = np.ldexp(np.ones(K, F32), g.integers(-2, 3, K)).astype(F32)
    W = (g.integers(-64, 64, (N, K)) / 32.0).astype(F32)
    L1 = synth.f32_to_bf16_bits((g.integers(-8, 8, (r, K)) / 8.0).astype(F32))
    L2 = synth.f32_to_bf16_bits((g.integers(-8, 8, (N, r)) / 4.0).astype(F32))
    b = synth.f32_to_bf16_bits((g.integers(-8, 8, N) / 8.0).astype(F32))
    # the branch must matter: x_hat differs from X, and L2 is not symmetric in use
    assert np.any(s != 1)

    mags = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]

    def q_block(vals):
        amax = max(abs(v) for v in vals)
        e = -127
        if amax:
            fl = 0
            while Fr(2) ** (fl + 1) <= amax:
                fl += 1
            while Fr(2) ** fl > amax:
                fl -= 1
            e = fl - 2
        out = []
        for v in vals:
            y = abs(v) / Fr(2) ** e
            d = [abs(y - m) for m in mags]
            best = min(range(8), key=lambda i: (d[i], i % 2))
            out.append((-1 if v < 0 else 1) * mags[best] * Fr(2) ** e)
        return out, e

    xv = [[Fr(float(v)) for v in row] for row in O.bf16_to_f64(X)]
    sv = [Fr(float(v)) for v in s]
    l1 = [[Fr(float(v)) for v in row] for row in O.bf16_to_f64(L1)]
    l2 = [[Fr(float(v)) for v in row] for row in O.bf16_to_f64(L2)]
    bv = [Fr(float(v)) for v in O.bf16_to_f64(b)]
    xh = [[x * Fr(float(_rn32(1 / sk))) for x, sk in zip(row, sv)] for row in xv]
    R = [[Fr(float(_rn32(Fr(float(W[n, k])) * sv[k] - sum(l2[n][j] * l1[j][k] for j in range(r)))))
          for k in range(K)] for n in range(N)]
    T = [[sum(xh[m][k] * l1[j][k] for k in range(K)) for j in range(r)] for m in range(M)]

    qx, sxe, T_o, _ = O.quantize_activations_mx(X, s, L1)
    Wq, we = O.quantize_residual_mx(W, s, L1, L2)
    Y = O.forward_mx(X, s, L1, L2, Wq, we, b)
    assert T_o.shape == (M, r)
    for m in range(M):
        for j in range(r):
            assert Fr(T_o[m, j]) == T[m][j]
    for m in range(M):
        for n in range(N):
            acc = bv[n] + sum(T[m][j] * l2[n][j] for j in range(r))
            for blk in range(K // 32):
                sl = slice(32 * blk, 32 * blk + 32)
                qa, ea = q_block(xh[m][sl])
                qw, ew = q_block(R[n][sl])
                assert sxe[m, blk] == ea + 127 and we[n, blk] == ew + 127
                acc += sum(a * w for a, w in zip(qa, qw))
            assert abs(Fr(Y[m, n]) - acc) <= abs(acc) * Fr(1, 10 ** 15)


# ------------------------------------------------------------- GELU (tanh form)
def test_gelu_tanh_odd_part_is_identity(O):
    """0.5 x (1 + tanh u(x)) - 0.5 (-x) (1 + tanh u(-x)) = x because u is odd and tanh is odd:
    a dropped 1/2, a sign error inside u or a missing x fails this."""
    x = np.linspace(-9.0, 9.0, 3601)
    d = O.gelu_tanh(x) - O.gelu_tanh(-x)
    assert np.max(np.abs(d - x)) <= 1e-14 * 9.0


def test_gelu_tanh_against_erf_gelu(O):
    """The tanh form approximates x Phi(x) (Phi from math.erf, a library routine) to
    within 4.8e-4 everywhere; a wrong cubic coefficient (0.04 or 0.05) or a wrong
    sqrt(2/pi) (0.8) gives 6e-4 to 3e-3."""
    x = np.linspace(-8.0, 8.0, 16001)
    exact = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    err = np.abs(O.gelu_tanh(x) - exact)
    assert err.max() <= 4.8e-4
    assert err.max() >= 1e-4          # it is the tanh form, not the erf form
    assert np.abs(x[np.argmax(err)]) > 2.0 and np.abs(x[np.argmax(err)]) < 3.5


def test_gelu_tanh_limits_and_minimum(O):
    assert O.gelu_tanh(0.0) == 0.0
    assert abs(O.gelu_tanh(20.0) - 20.0) < 1e-12
    assert abs(O.gelu_tanh(-20.0)) < 1e-12
    # slope 1/2 at the origin
    h = 1e-6
    assert abs((O.gelu_tanh(h) - O.gelu_tanh(-h)) / (2 * h) - 0.5) < 1e-9
    # the minimum, about -0.17 near x = -0.75 (GELU's known shape)
    x = np.linspace(-3.0, 0.0, 30001)
    g = O.gelu_tanh(x)
    assert -0.171 < g.min() < -0.169 and -0.80 < x[np.argmin(g)] < -0.70


def test_forward_activation_is_applied_after_bias(O):
    """The fused point: gelu of main + low + b (bias included), unknown names rejected."""
    rng = np.random.default_rng(7)
    M, K, N, r = 4, 128, 16, 16
    X = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    s = np.ones(K, np.float32)
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    L1 = O.bf16_from_f64(rng.standard_normal((r, K)) * 0.05)
    L2 = O.bf16_from_f64(rng.standard_normal((N, r)) * 0.05)
    Wq, sw = O.quantize_residual(W, s, L1, L2)
    b = O.bf16_from_f64(rng.standard_normal(N))
    Y = O.forward(X, s, L1, L2, Wq, sw, b)
    Yg = O.forward(X, s, L1, L2, Wq, sw, b, activation="gelu_tanh")
    assert np.array_equal(O.gelu_tanh(Y), Yg)
    assert not np.allclose(Yg, O.gelu_tanh(Y - O.bf16_to_f64(b)[None, :]) + O.bf16_to_f64(b)[None, :])
    with pytest.raises(ValueError):
        O.forward(X, s, L1, L2, Wq, sw, b, activation="relu")

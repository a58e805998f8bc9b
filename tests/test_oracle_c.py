"""The plain C oracle (oracle/svdq_ref.c) beside the numpy oracle.

Every pin in test_oracle_pins.py runs on both oracles.  This file adds what is
particular to the C one: its Jacobi SVD against LAPACK (a library routine, the
survey's P-4 check), and the two independent implementations against each
other on the workloads' own data -- codes, scales, group partials, MXFP4 bytes
and the packed weights bit for bit, outputs to float64 rounding.

Citations: [Term] = the "SVDQuant Low-Rank Residual Quantization Algorithm
Terminology Entry", section 2.3 (E1-E7 in page order); [Abs] = the SVDQuant
abstract.
"""
import numpy as np
import pytest

import synth
from oracle import svdq_oracle as N_
from oracle import svdq_ref as C

F32, F64 = np.float32, np.float64


@pytest.mark.parametrize("shape", [(96, 160), (160, 96), (64, 64)])
def test_jacobi_svd_matches_lapack(shape):
    """[Term] E3/E5: singular values to 1e-12 of LAPACK's, singular subspaces equal
    (|U_c^T U_lapack| and |V_c^T V_lapack| are identities for distinct sigma), and
    U diag(sigma) V^T reproduces the matrix, for tall, wide and square inputs."""
    g = np.random.default_rng(sum(shape))
    A = g.standard_normal(shape) * np.exp(g.uniform(-2, 2, (1, shape[1])))
    U, S, V = C.svd_sorted(A)
    Sl = np.linalg.svd(A, compute_uv=False)
    np.testing.assert_allclose(S, Sl, rtol=1e-12, atol=1e-13 * Sl[0])
    Ul, _, Vlt = np.linalg.svd(A, full_matrices=False)
    p = min(shape)
    np.testing.assert_allclose(np.abs(U.T @ Ul), np.eye(p), atol=1e-8)
    np.testing.assert_allclose(np.abs(V.T @ Vlt.T), np.eye(p), atol=1e-8)
    np.testing.assert_allclose((U * S) @ V.T, A, atol=1e-12 * Sl[0])


def test_jacobi_svd_of_a_rank_deficient_matrix():
    """Rank 3 in 40 x 30: three singular values from the closed form of the Gram
    matrix, the rest zero, and the null directions still orthonormal."""
    g = np.random.default_rng(5)
    Q1, _ = np.linalg.qr(g.standard_normal((40, 3)))
    Q2, _ = np.linalg.qr(g.standard_normal((30, 3)))
    A = (Q1 * [4.0, 2.0, 0.5]) @ Q2.T
    U, S, V = C.svd_sorted(A)
    np.testing.assert_allclose(S[:3], [4.0, 2.0, 0.5], rtol=1e-13)
    assert np.all(S[3:] < 1e-13)
    np.testing.assert_allclose(V.T @ V, np.eye(30), atol=1e-12)


def test_the_c_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        C.quantize_groups(np.zeros((2, 96), F32))          # K not a multiple of 64
    with pytest.raises(ValueError):
        C.lowrank_factors(np.eye(4), np.ones(4), np.eye(4), 5)   # rank above min(N, K)


def _workload_slice(name, M, N, K):
    w = synth.WORKLOADS[name]
    X = np.ascontiguousarray(synth.activations(w, M)[:, :K])   # the first M rows of the draw
    W = np.ascontiguousarray(synth.weight(w)[:N, :K])
    b = synth.bias(w)[:N]
    A = N_.act_absmax(synth.calibration_activations(w)[:, :K])
    return w, X, W, b, A


@pytest.mark.parametrize("name,M,N,K", [("tiny", 64, 192, 256), ("smallk_640", 48, 128, 640),
                                        ("mlp_down", 16, 96, 1024)])
def test_pack_agrees_with_the_numpy_oracle(name, M, N, K):
    """The offline pack ([Term] 2.1, E1-E4) of both oracles on the workloads' own
    weights: s bit-exact, sigma to 1e-12, and -- where the two SVDs round the
    factors alike, which they do on these inputs -- L1, L2, Wq and the scales bit-exact."""
    w, X, W, b, A = _workload_slice(name, M, N, K)
    r = min(w.rank, 16)
    pc = C.pack_weights(W, A, w.alpha, r)
    pn = N_.pack_weights(W, A, w.alpha, r)
    np.testing.assert_array_equal(pc["s"], pn["s"])
    np.testing.assert_allclose(pc["sigma"], pn["sigma"], rtol=1e-12, atol=1e-12 * pn["sigma"][0])
    for key in ("L1", "L2", "Wq", "w_scales"):
        np.testing.assert_array_equal(pc[key], pn[key], err_msg=key)


@pytest.mark.parametrize("name,M,N,K,act", [("tiny", 64, 256, 1024, None),
                                            ("smallk_1280", 32, 160, 1280, None),
                                            ("mlp_down", 24, 64, 12288, None),
                                            ("tiny", 16, 128, 512, "gelu_tanh")])
def test_forward_agrees_with_the_numpy_oracle(name, M, N, K, act):
    """The forward ([Term] E1, E4, E7) of both oracles from the same packed layer:
    codes, scales and group partials bit-exact, T and Y to float64 rounding."""
    w, X, W, b, A = _workload_slice(name, M, N, K)
    pk = N_.pack_weights(W, A, w.alpha, min(w.rank, 32))
    qc, sc, Tc, xc = C.quantize_activations(X, pk["s"], pk["L1"])
    qn, sn, Tn, xn = N_.quantize_activations(X, pk["s"], pk["L1"])
    np.testing.assert_array_equal(qc, qn)
    np.testing.assert_array_equal(sc.view(np.uint32), sn.view(np.uint32))
    np.testing.assert_array_equal(xc.view(np.uint32), xn.view(np.uint32))
    assert N_.rel_fro(Tc, Tn) < 1e-13
    np.testing.assert_array_equal(C.group_partials(qc, pk["Wq"]), N_.group_partials(qn, pk["Wq"]))
    Yc = C.forward(X, pk["s"], pk["L1"], pk["L2"], pk["Wq"], pk["w_scales"], b, act)
    Yn = N_.forward(X, pk["s"], pk["L1"], pk["L2"], pk["Wq"], pk["w_scales"], b, act)
    assert N_.rel_fro(Yc, Yn) < 1e-13
    # a row window of the C forward is the same rows of the whole
    Yw = C.forward(X, pk["s"], pk["L1"], pk["L2"], pk["Wq"], pk["w_scales"], b, act, rows=(3, 7))
    np.testing.assert_array_equal(Yw, Yc[3:7])


@pytest.mark.parametrize("name,M,N,K", [("tiny", 32, 128, 1024), ("smallk_640", 32, 64, 640)])
def test_mxfp4_agrees_with_the_numpy_oracle(name, M, N, K):
    """The MXFP4 reading of Q in both oracles: weight and activation codes and E8M0
    bytes bit-exact, T and Y (with the low-rank branch and bias) to float64 rounding."""
    w, X, W, b, A = _workload_slice(name, M, N, K)
    pk = N_.pack_weights(W, A, w.alpha, min(w.rank, 32))
    Wc, ec = C.quantize_residual_mx(W, pk["s"], pk["L1"], pk["L2"])
    Wn, en = N_.quantize_residual_mx(W, pk["s"], pk["L1"], pk["L2"])
    np.testing.assert_array_equal(Wc, Wn)
    np.testing.assert_array_equal(ec, en)
    qc, sc, Tc, _ = C.quantize_activations_mx(X, pk["s"], pk["L1"])
    qn, sn, Tn, _ = N_.quantize_activations_mx(X, pk["s"], pk["L1"])
    np.testing.assert_array_equal(qc, qn)
    np.testing.assert_array_equal(sc, sn)
    assert N_.rel_fro(Tc, Tn) < 1e-13
    Yc = C.forward_mx(X, pk["s"], pk["L1"], pk["L2"], Wn, en, b)
    Yn = N_.forward_mx(X, pk["s"], pk["L1"], pk["L2"], Wn, en, b)
    assert N_.rel_fro(Yc, Yn) < 1e-13


def test_append_lora_agrees_with_the_numpy_oracle():
    """[Abs]: a LoRA joins the branch without re-quantization; both oracles fold the
    DiT block's seeded rank-16 adapter into the same bf16 factors."""
    w, X, W, b, A = _workload_slice("dit_qkv", 8, 96, 512)
    pk = N_.pack_weights(W, A, w.alpha, 32)
    La, Lb = synth.lora_factors(w)
    La, Lb = La[:512], Lb[:, :96]
    c = C.append_lora(pk["s"], pk["L1"], pk["L2"], La, Lb)
    n = N_.append_lora(pk["s"], pk["L1"], pk["L2"], La, Lb)
    np.testing.assert_array_equal(c[0], n[0])
    np.testing.assert_array_equal(c[1], n[1])

"""CPU tests of the C ABI: exported symbols, host-side packer parity with the oracle,
and the argument validation of every entry point (no GPU needed: validation
fails before anything is launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import svdq_oracle as O

S = pytest.importorskip("bit_diffusion_model_svdq_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
F32, F64 = np.float32, np.float64


def _header_functions():
    text = open(os.path.join(ROOT, "include", "svdq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svdq_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(S.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(S.EXPORTS)


def test_status_strings():
    for st in range(7):
        assert S.svdq_status_string(st) not in ("", "unknown status")
    assert S.svdq_status_string(99) == "unknown status"


# ------------------------------------------------------------------ packer
def test_act_absmax_is_exact():
    w = synth.WORKLOADS["tiny"]
    Xc = synth.calibration_activations(w)
    A = np.zeros(w.K, F32)
    S.svdq_act_absmax_update(Xc[:100], A)
    S.svdq_act_absmax_update(Xc[100:], A)     # streaming in two batches
    np.testing.assert_array_equal(A, O.act_absmax(Xc))


@pytest.mark.parametrize("N,K,r", [(1024, 1024, 16), (192, 320, 32), (320, 192, 16), (128, 256, 0)])
def test_quantize_residual_bit_exact(N, K, r):
    w = synth.WORKLOADS["tiny"]
    W = synth.weight(w)[:N, :K]
    A = O.act_absmax(synth.calibration_activations(w))[:K]
    po = O.pack_weights(W, A, 0.5, rank=r)
    Wq, ws = S.svdq_quantize_residual(W, po["s"], po["L1"], po["L2"])
    np.testing.assert_array_equal(Wq, po["Wq"])
    np.testing.assert_array_equal(ws.view(np.uint32), po["w_scales"].view(np.uint32))


@pytest.mark.parametrize("N,K,r", [(1024, 1024, 16), (192, 320, 32), (320, 192, 16)])
def test_pack_weights_matches_oracle(N, K, r):
    w = synth.WORKLOADS["tiny"]
    W = synth.weight(w)[:N, :K]
    A = O.act_absmax(synth.calibration_activations(w))[:K]
    pl = S.svdq_pack_weights(W, A, 0.5, r, want_sigma=True)
    po = O.pack_weights(W, A, 0.5, rank=r)
    np.testing.assert_array_equal(pl["smooth"], po["s"])
    p = min(N, K)
    # leading singular values to 1e-12 (the Gram route is accurate for sigma near sigma_1)
    np.testing.assert_allclose(pl["sigma"][:2 * r], po["sigma"][:2 * r], rtol=1e-12)
    np.testing.assert_allclose(pl["sigma"][:p], po["sigma"][:p], atol=1e-6 * po["sigma"][0])
    # factors are not unique; their product is (bf16 rounding aside)
    Ll = O.bf16_to_f64(pl["L2"]) @ O.bf16_to_f64(pl["L1"])
    Lo = O.bf16_to_f64(po["L2"]) @ O.bf16_to_f64(po["L1"])
    assert np.linalg.norm(Ll - Lo) <= 1e-3 * np.linalg.norm(Lo)
    # Eckart-Young (E6) with the library's own factors, up to bf16 rounding of the factors
    What = po["What"]
    tail = float(np.sum(po["sigma"][r:] ** 2))
    err2 = float(np.sum((What - Ll) ** 2))
    assert abs(err2 - tail) <= 2 ** -6 * np.sqrt(tail * float(np.sum(po["sigma"][:r] ** 2))) + 1e-9
    # lora_down rows orthonormal to bf16 accuracy
    L1 = O.bf16_to_f64(pl["L1"])
    np.testing.assert_allclose(L1 @ L1.T, np.eye(r), atol=2e-2)
    # with identical factors the quantized residual is bit-identical
    if np.array_equal(pl["L1"], po["L1"]) and np.array_equal(pl["L2"], po["L2"]):
        np.testing.assert_array_equal(pl["Wq"], po["Wq"])
        np.testing.assert_array_equal(pl["w_scales"], po["w_scales"])


def test_pack_exact_lowrank_weight_leaves_zero_residual():
    """W = L2 L1 with dyadic factors and s = 1: the library's own SVD must absorb all of it."""
    K, N, r = 256, 192, 16
    W = np.zeros((N, K), F32)
    g = synth.rng_for("tiny", 20)
    rows = g.choice(N, r, replace=False)
    cols = g.choice(K, r, replace=False)
    vals = 2.0 ** -np.arange(1, r + 1)
    W[rows, cols] = vals                           # a scaled partial permutation: sigma = vals
    A = O.weight_absmax(W)                         # A == W_scale -> s = 1 for alpha = 1/2
    pl = S.svdq_pack_weights(W, A, 0.5, r, want_sigma=True)
    np.testing.assert_array_equal(pl["smooth"], np.ones(K, F32))
    np.testing.assert_allclose(pl["sigma"][:r], vals, rtol=1e-12)
    assert np.all(pl["sigma"][r:] < 1e-6)
    # what is left is round-off of the floating-point eigenvectors, ~1e-40 against entries of 2^-16..2^-1
    assert float(np.max(pl["w_scales"])) < 1e-30


def _exact_spectrum_weight(N, K, sigma):
    """W = U diag(sigma) V^T with U, V columns of Sylvester-Hadamard matrices scaled to
    unit length (N, K powers of 4, so 1/sqrt is a power of two) and dyadic sigma: every
    entry is a short dyadic sum, exact in float32, so the float32 W has exactly these
    singular values, repeated ones included."""
    from scipy.linalg import hadamard
    p = len(sigma)
    U = hadamard(N)[:, 1:p + 1] / np.sqrt(N)
    V = hadamard(K)[:, 1:p + 1] / np.sqrt(K)
    W64 = (U * np.asarray(sigma)[None, :]) @ V.T
    W = W64.astype(F32)
    assert np.array_equal(W.astype(F64), W64)
    return W, U, V


@pytest.mark.parametrize("N,K", [(64, 256), (256, 64)])
def test_pack_degenerate_singular_values_at_the_rank_boundary(N, K):
    """sigma_r = sigma_(r+1) (and a repeated pair inside the kept rank): the rank-r
    subspace is not unique, so only invariants are checked ([Term] 2.3, E5 and E6):
    the library's singular values are the designed ones, their squares sum to
    ||W_hat||_F^2, the lora_down rows are orthonormal and span v_1..v_15 plus a unit
    vector of the degenerate plane (nothing outside v_1..v_17), and the residual energy
    ||W_hat - L2 L1||_F^2 is the tail sum up to the bf16 rounding of the factors.
    Exercises both Gram sides (N < K and K < N) and the re-orthogonalization of
    inverse iteration inside a cluster."""
    r = 16
    sigma = np.array([8, 7, 6, 6, 5.5, 5, 4.5, 4, 3.75, 3.5, 3.25, 3, 2.75, 2.5, 2.25, 2, 2,
                      1.75, 1.5, 1.25, 1, 0.75, 0.5, 0.25])
    assert sigma[r - 1] == sigma[r] and sigma[2] == sigma[3]
    W, U, V = _exact_spectrum_weight(N, K, sigma)
    A = O.weight_absmax(W)                         # A == W_scale -> s = 1 for alpha = 1/2
    pl = S.svdq_pack_weights(W, A, 0.5, r, want_sigma=True)
    np.testing.assert_array_equal(pl["smooth"], np.ones(K, F32))
    sg = pl["sigma"]
    np.testing.assert_allclose(sg[:len(sigma)], sigma, rtol=1e-12, atol=1e-12 * sigma[0])
    assert np.all(sg[len(sigma):] < 1e-6 * sigma[0])
    Wd = W.astype(F64)
    assert abs(np.sum(sg ** 2) - np.sum(Wd ** 2)) <= 1e-12 * np.sum(Wd ** 2)
    L1 = O.bf16_to_f64(pl["L1"])                   # [r, K]
    L2 = O.bf16_to_f64(pl["L2"])                   # [N, r]
    bf = 2.0 ** -8                                 # bf16 relative rounding, with margin
    assert np.max(np.abs(L1 @ L1.T - np.eye(r))) <= 4 * bf
    # nothing outside span(v_1 .. v_17)
    V17 = V[:, :r + 1]
    out = L1.T - V17 @ (V17.T @ L1.T)
    assert np.linalg.norm(out) <= 4 * bf * np.sqrt(r)
    # v_1 .. v_15 lie in the row space of L1
    V15 = V[:, :r - 1]
    Q, _ = np.linalg.qr(L1.T)
    miss = V15 - Q @ (Q.T @ V15)
    assert np.linalg.norm(miss) <= 4 * bf * np.sqrt(r)
    # residual energy: the tail sum of squares, up to the rounding of the factors
    tail = float(np.sum(sigma[r:] ** 2))
    res = float(np.sum((Wd - L2 @ L1) ** 2))
    assert abs(res - tail) <= 0.02 * tail
    # the residual the library quantized is that of its own rounded factors
    Wq, ws = S.svdq_quantize_residual(W, pl["smooth"], pl["L1"], pl["L2"])
    np.testing.assert_array_equal(Wq, pl["Wq"])
    np.testing.assert_array_equal(ws, pl["w_scales"])


@pytest.mark.slow
def test_pack_weights_dit_projection_shape():
    w = synth.WORKLOADS["dit_proj"]
    W = synth.weight(w)
    A = np.zeros(w.K, F32)
    S.svdq_act_absmax_update(synth.calibration_activations(w), A)
    pl = S.svdq_pack_weights(W, A, w.alpha, w.rank, want_sigma=True)
    po = O.pack_weights(W, O.act_absmax(synth.calibration_activations(w)), w.alpha, rank=w.rank)
    np.testing.assert_array_equal(pl["smooth"], po["s"])
    np.testing.assert_allclose(pl["sigma"][:64], po["sigma"][:64], rtol=1e-12)
    Ll = O.bf16_to_f64(pl["L2"]) @ O.bf16_to_f64(pl["L1"])
    Lo = O.bf16_to_f64(po["L2"]) @ O.bf16_to_f64(po["L1"])
    assert np.linalg.norm(Ll - Lo) <= 1e-3 * np.linalg.norm(Lo)
    Wq, ws = S.svdq_quantize_residual(W, po["s"], po["L1"], po["L2"])
    np.testing.assert_array_equal(Wq, po["Wq"])
    np.testing.assert_array_equal(ws.view(np.uint32), po["w_scales"].view(np.uint32))


# -------------------------------------------------------- validation errors
def _status(fn, *args):
    return getattr(S._lib, fn)(*args)


def test_pack_rejects_bad_arguments_and_writes_nothing():
    W = np.ones((64, 128), F32)
    A = np.ones(128, F32)
    outs = dict(s=np.full(128, 7, F32), L1=np.full((16, 128), 7, np.uint16), L2=np.full((64, 16), 7, np.uint16),
                Wq=np.full((64, 64), 7, np.uint8), ws=np.full((64, 2), 7, F32))

    def call(N=64, K=128, rank=16, group=64, alpha=0.5, smin=1e-5, Wp=True):
        p = S.svdq_pack_params(alpha, rank, group, smin)
        return S._lib.svdq_pack_weights(W.ctypes.data if Wp else None, N, K, A.ctypes.data, ctypes.byref(p),
                                        outs["s"].ctypes.data, outs["L1"].ctypes.data, outs["L2"].ctypes.data,
                                        outs["Wq"].ctypes.data, outs["ws"].ctypes.data, None)

    assert call(group=32) == 2                    # SVDQ_ERR_UNSUPPORTED
    assert call(K=100) == 1
    assert call(rank=17) == 1
    assert call(rank=144) == 1
    assert call(alpha=1.5) == 1
    assert call(smin=0.0) == 1
    assert call(Wp=False) == 1
    assert "NULL" in S.svdq_last_error()
    for a in outs.values():
        assert np.all(a == 7)
    with pytest.raises(S.SvdqError):
        S.svdq_quantize_residual(np.ones((8, 96), F32), np.ones(96, F32), np.zeros((0, 96), np.uint16),
                                 np.zeros((8, 0), np.uint16))


def test_workspace_bytes():
    """qx + sx + T; plus the GEMM's split partials when its 256 x 192 tiles leave a
    last partial wave (this container has no GPU: the library assumes 256 CUs)."""
    al = lambda x: (x + 255) // 256 * 256
    # T: one partial T per K-slice of the quantize kernel's launch plan (a cost
    # model over 16- or 32-row blocks and slices of at most 48 groups)
    M, K, N, r = 4096, 3072, 3072, 32          # 16 x 16 = 256 tiles: one full wave
    b = S.svdq_forward_workspace_bytes(M, K, N, r)
    assert b == al(M * K // 2) + al(M * K // 64 * 4) + al(2 * M * r * 4)   # 128 blocks x 2 slices
    M, K, N = 4608, 12288, 3072                # 18 x 16 = 288 tiles: 32 left, each cut 8 ways
    b = S.svdq_forward_workspace_bytes(M, K, N, r)
    assert b == al(M * K // 2) + al(M * K // 64 * 4) + al(5 * M * r * 4) + 32 * 8 * 256 * 192 * 4
    M, K, N, r = 256, 1024, 1024, 16           # 8 blocks of 32 rows, one slice
    b = S.svdq_forward_workspace_bytes(M, K, N, r)
    assert b == al(M * K // 2) + al(M * K // 64 * 4) + al(M * r * 4)
    M, K, N, r = 4608, 3072, 9216, 48          # 144 blocks, one slice (a second would cost the GEMM more)
    b = S.svdq_forward_workspace_bytes(M, K, N, r)
    assert b == al(M * K // 2) + al(M * K // 64 * 4) + al(M * r * 4)
    assert S.svdq_forward_workspace_bytes(M, 100, N, r) == 0
    assert S.svdq_forward_workspace_bytes(M, K, 40, r) == 0
    assert S.svdq_forward_workspace_bytes(M, K, N, 24) == 0


def test_workspace_layout_matches_the_workspace_size():
    """Offsets of qx, sx and the T slices: the parts in that order, 256-byte aligned,
    the T slices of the quantize kernel's plan (2 at the DiT projection, 5 at the MLP
    down projection, 1 where a second slice would cost the GEMM more)."""
    al = lambda x: (x + 255) // 256 * 256
    for (M, K, N, r, slices) in [(4096, 3072, 3072, 32, 2), (4608, 12288, 3072, 32, 5),
                                 (256, 1024, 1024, 16, 1), (4608, 3072, 9216, 48, 1), (77, 192, 48, 0, 0)]:
        lay = S.svdq_forward_workspace_layout(M, K, N, r)
        assert lay["qx"] == 0
        assert lay["sx"] == al(M * K // 2)
        assert lay["t_slices"] == slices
        if r:
            assert lay["T"] == al(M * K // 2) + al(M * K // 64 * 4)
            assert lay["T"] + slices * M * r * 4 <= S.svdq_forward_workspace_bytes(M, K, N, r)
        mx = S.svdq_forward_workspace_layout(M, K, N, r, mxfp4=True) if K % 128 == 0 else None
        if mx:
            assert mx["sx"] == al(M * K // 2) and mx["sx_rows"] == M + (M & 1)
            assert mx["t_slices"] == slices
    with pytest.raises(S.SvdqError):
        S.svdq_forward_workspace_layout(4096, 100, 3072, 32)
    with pytest.raises(S.SvdqError):
        S.svdq_forward_workspace_layout(64, 192, 64, 16, mxfp4=True)


def test_device_entry_points_validate_before_launching():
    """Each case fails validation, so nothing reaches the GPU runtime."""
    L = S._lib
    a = 1 << 20            # a fake 16-byte-aligned address; never dereferenced
    mis = a + 4
    ws = S.svdq_forward_workspace_bytes(256, 1024, 1024, 16)
    fwd = lambda X=a, M=256, K=1024, N=1024, r=16, L1=a, L2=a, bias=a, wsb=ws: L.svdq_linear_forward(
        X, M, K, N, r, a, L1, L2, a, a, bias, a, a, wsb, None)
    assert fwd(K=1000) == 1
    assert fwd(M=0) == 1
    assert fwd(N=1000) == 1
    assert fwd(r=24) == 1
    assert fwd(r=144) == 1
    assert fwd(L1=None) == 1
    assert fwd(X=mis) == 3
    assert fwd(bias=mis) == 3
    assert fwd(wsb=ws - 1) == 4
    assert "workspace" in S.svdq_last_error()
    assert L.svdq_forward_quantize(a, 256, 1000, 16, a, a, a, ws, None) == 1
    assert L.svdq_forward_gemm(256, 1024, 1000, 16, a, a, a, None, a, a, ws, None) == 1
    assert L.svdq_quantize_activations(a, 256, 1024, a, None, 16, a, a, a, None) == 1
    assert L.svdq_quantize_activations(a, 256, 1024, a, a, 16, a, a, None, None) == 1
    assert L.svdq_debug_group_partials(a, a, 256, 1024, 1024, 0, 300, 0, 16, a, None) == 1
    assert L.svdq_debug_group_partials(a, a, 256, 1024, 1024, 10, 10, 0, 16, a, None) == 1
    assert L.svdq_debug_group_partials(a, mis, 256, 1024, 1024, 0, 16, 0, 16, a, None) == 3
    # the canonical-layout quantize stages a whole row in LDS: K <= 12544, any rank
    for r_ in (0, 16, 128):
        assert L.svdq_quantize_activations(a, 16, 12608, a, a, r_, a, a, a, None) == 1
        assert "12544" in S.svdq_last_error()
        assert L.svdq_quantize_activations_mxfp4(a, 16, 12672, a, a, r_, a, a, a, None) == 1
    # the allocation-free forward: shapes checked, then its workspace need against the
    # static array, all before any HIP call (nothing here has a GPU)
    na = lambda M=256, K=1024, N=1024, r=16: L.svdq_linear_forward_noalloc(
        a, M, K, N, r, a, a, a, a, a, a, 0, a, None)
    assert S.svdq_static_workspace_bytes() == 64 << 20
    assert na(K=1000) == 1
    assert na(r=24) == 1
    assert S.svdq_forward_workspace_bytes(4608, 12288, 3072, 32) > 64 << 20
    assert na(M=4608, K=12288, N=3072, r=32) == 4
    assert "static workspace" in S.svdq_last_error()
    assert L.svdq_act_absmax_update_device(a, -1, 64, a, None) == 1
    assert L.svdq_act_absmax_update_device(a, 8, 0, a, None) == 1
    assert L.svdq_act_absmax_update_device(None, 8, 64, a, None) == 1
    assert L.svdq_act_absmax_update_device(a, 8, 64, None, None) == 1
    assert L.svdq_act_absmax_update_device(a + 1, 8, 64, a, None) == 3
    assert L.svdq_act_absmax_update_device(a, 8, 64, a + 2, None) == 3
    assert L.svdq_act_absmax_update_device(a, 0, 64, a, None) == 0   # empty batch: nothing to launch


def test_fused_plan_and_its_debug_entry_point_validate():
    """svdq_forward_fused (host only) takes small layers and refuses the rest; the fused
    debug launch rejects bad arguments before any HIP call (nothing here has a GPU).  The
    work bound assumes the MI355X's 256 compute units, which is also the count the library
    assumes where it cannot query a device."""
    L = S._lib
    fused = lambda M, K, N, r: S.svdq_forward_fused(M, K, N, r)
    assert fused(1024, 640, 640, 32)          # 100 blocks of 16 x 16 x 64 per compute unit
    assert fused(256, 1024, 1024, 16)
    assert fused(1, 64, 16, 16)
    assert fused(37, 1280, 2560, 32)
    assert not fused(4096, 640, 640, 32)      # 400 per compute unit: the two kernels
    assert not fused(1024, 1280, 1280, 32)
    assert not fused(256, 1344, 256, 16)      # K past 1280
    assert not fused(256, 640, 640, 48)       # r past 32
    assert not fused(256, 640, 2576, 16)      # N past 2560
    assert not fused(0, 640, 640, 16) and not fused(256, 600, 640, 16) and not fused(256, 640, 600, 16)
    a = 1 << 20
    dbg = lambda M=256, K=1024, N=1024, r=16, qx=a, sx=a, act=0, X=a: L.svdq_debug_fused_forward(
        X, M, K, N, r, a, a, a, a, a, a, act, a, qx, sx, None)
    assert dbg(M=4096, K=640, N=640, r=32) == 1
    assert "fused" in S.svdq_last_error()
    assert dbg(qx=None) == 1
    assert dbg(sx=None) == 1
    assert dbg(act=5) == 1
    assert dbg(X=a + 4) == 3
    assert dbg(qx=a + 8) == 3


def test_fused_mx_plan_and_its_debug_entry_point_validate():
    """svdq_forward_fused_mxfp4: the int4 range with K a multiple of 128, and up to 400
    blocks per compute unit where K <= 640; the MXFP4 fused debug launch rejects bad
    arguments before any HIP call."""
    L = S._lib
    fused = lambda M, K, N, r: S.svdq_forward_fused_mxfp4(M, K, N, r)
    assert fused(1024, 640, 640, 32) and fused(256, 1024, 1024, 16) and fused(1, 128, 16, 16)
    assert fused(37, 1280, 2560, 32) and fused(300, 1280, 1280, 0)
    assert not fused(1, 64, 16, 16)           # K must be a multiple of 128
    assert not fused(256, 320, 640, 16)
    assert fused(4096, 640, 640, 32)          # 400 blocks per compute unit at K = 640
    assert not fused(6144, 640, 640, 32)      # 600: the two kernels
    assert not fused(1024, 1280, 1280, 32)    # 400 at K = 1280: the two kernels
    assert not fused(256, 1408, 256, 16)      # K past 1280
    assert not fused(256, 640, 640, 48)       # r past 32
    assert not fused(256, 640, 2576, 16)      # N past 2560
    assert not fused(0, 640, 640, 16) and not fused(256, 640, 600, 16)
    a = 1 << 20
    dbg = lambda M=256, K=1024, N=1024, r=16, qx=a, sx=a, act=0, X=a: L.svdq_debug_fused_forward_mxfp4(
        X, M, K, N, r, a, a, a, a, a, a, act, a, qx, sx, None)
    assert dbg(M=6144, K=640, N=640, r=32) == 1
    assert "fused" in S.svdq_last_error()
    assert dbg(K=320) == 1                    # not a multiple of 128
    assert dbg(qx=None) == 1
    assert dbg(sx=None) == 1
    assert dbg(act=5) == 1
    assert dbg(X=a + 4) == 3
    assert dbg(sx=a + 8) == 3


def test_append_lora_bit_exact_with_oracle():
    """The library's LoRA concatenation gives the oracle's bytes (one rounding of
    A[k, j] s[k] and of B[j, n] to bf16)."""
    w = synth.WORKLOADS["tiny"]
    g = np.random.default_rng(5)
    K, N, r = w.K, w.N, 16
    s = np.exp(g.uniform(-3, 3, K)).astype(np.float32)
    L1 = synth.f32_to_bf16_bits(g.standard_normal((r, K)).astype(np.float32))
    L2 = synth.f32_to_bf16_bits(g.standard_normal((N, r)).astype(np.float32))
    A, B = synth.lora_factors(w)
    L1n, L2n = S.svdq_append_lora(s, L1, L2, A, B)
    L1o, L2o = O.append_lora(s, L1, L2, A, B)
    np.testing.assert_array_equal(L1n, L1o)
    np.testing.assert_array_equal(L2n, L2o)
    L1z, L2z = S.svdq_append_lora(s, None, None, A, B)          # r = 0: the adapter alone
    np.testing.assert_array_equal(L1z, L1o[r:])
    np.testing.assert_array_equal(L2z, L2o[:, r:])
    with pytest.raises(S.SvdqError):                           # r + rl > 128
        S.svdq_append_lora(s, np.zeros((128, K), np.uint16), np.zeros((N, 128), np.uint16), A, B)


@pytest.mark.parametrize("name,rank", [("tiny", 16), ("smallk_640", 32)])
def test_quantize_residual_mxfp4_bit_exact(name, rank):
    """The library's MXFP4 residual quantizer gives the oracle's codes and E8M0 bytes
    from the same s, L1, L2."""
    w = synth.WORKLOADS[name]
    W = synth.weight(w)
    g = np.random.default_rng(6)
    s = np.exp(g.uniform(-2, 2, w.K)).astype(np.float32)
    L1 = synth.f32_to_bf16_bits(g.standard_normal((rank, w.K)).astype(np.float32) * 0.05)
    L2 = synth.f32_to_bf16_bits(g.standard_normal((w.N, rank)).astype(np.float32) * 0.05)
    Wq, we = S.svdq_quantize_residual_mxfp4(W, s, L1, L2)
    Wq_o, we_o = O.quantize_residual_mx(W, s, L1, L2)
    np.testing.assert_array_equal(Wq, Wq_o)
    np.testing.assert_array_equal(we, we_o)


def test_workspace_bytes_mxfp4():
    """qx | activation scales k-tiled [ceil(K/256)][M rounded up to even][8] | T slices."""
    al = lambda x: (x + 255) // 256 * 256
    M, K, N, r = 4096, 3072, 3072, 32
    b = S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r)
    assert b == al(M * K // 2) + al(M * K // 32) + al(2 * M * r * 4)
    M, K = 77, 640                                                     # odd M, K % 256 == 128
    assert S.svdq_forward_workspace_bytes_mxfp4(M, K, 48, 0) == al(M * K // 2) + al(3 * 78 * 8)
    # 4608 tokens, N = 3072: 18 x 16 = 288 tiles of 256 x 192 on 256 CUs leave 32.  At
    # K = 3072 (24 steps) they are too short to split: no partials (a one-slice T at r = 48)
    M, K, N, r = 4608, 3072, 3072, 48
    assert S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r) == (
        al(M * K // 2) + al(M * K // 32) + al(M * r * 4))
    # at K = 12288 (96 steps) the 32 are cut into 8 K-shares of fp32 partial tiles; k1 runs
    # 5 K-slices of 39 groups, so T has 5 slices
    K = 12288
    assert S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r) == (
        al(M * K // 2) + al(M * K // 32) + al(5 * M * r * 4) + al(32 * 8 * 256 * 192 * 4))
    # the threshold: 56 steps split, 55 do not
    part = al(16 * 8 * 256 * 192 * 4)
    for K, split in ((7168, True), (7040, False)):
        base = S.svdq_forward_workspace_bytes_mxfp4(4300, K, N, 0)
        assert base == al(4300 * K // 2) + al((K + 255) // 256 * 4300 * 8) + (part if split else 0), K
    K = 3072
    assert S.svdq_forward_workspace_bytes_mxfp4(M, 64, N, r) == 0     # K must be a multiple of 128
    assert S.svdq_forward_workspace_bytes_mxfp4(M, K, 40, r) == 0


@pytest.mark.parametrize("rows,K", [(48, 3072), (7, 640), (1, 128), (16, 384)])
def test_mxfp4_tile_scales_layout(rows, K):
    """The k-tiled scale layout: byte (t * rows + n) * 8 + j holds block 8 t + j of row n, and
    the blocks past K/32 of the last tile are 127 -- a numpy re-indexing of the row-major bytes."""
    sc = np.random.default_rng(rows + K).integers(0, 256, (rows, K // 32), dtype=np.uint8)
    t = S.svdq_mxfp4_tile_scales(sc)
    nt = (K + 255) // 256
    assert t.shape == (nt, rows, 8)
    assert S.svdq_mxfp4_tiled_scale_bytes(rows, K) == t.nbytes
    padded = np.full((rows, 8 * nt), 127, np.uint8)
    padded[:, :K // 32] = sc
    np.testing.assert_array_equal(t, padded.reshape(rows, nt, 8).transpose(1, 0, 2))
    flat = t.reshape(-1)
    n, b = rows - 1, K // 32 - 1                                       # last row, last block
    assert flat[((b // 8) * rows + n) * 8 + b % 8] == sc[n, b]


def test_mxfp4_tile_scales_rejects():
    assert S.svdq_mxfp4_tiled_scale_bytes(0, 128) == 0
    assert S.svdq_mxfp4_tiled_scale_bytes(4, 64) == 0
    with pytest.raises(S.SvdqError):
        S.svdq_mxfp4_tile_scales(np.zeros((4, 3), np.uint8))          # K = 96

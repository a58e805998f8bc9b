"""GPU parity of the MXFP4 variant against the CPU oracle, through the C ABI.

Bit-exact: activation codes (E2M1 patterns) and E8M0 scale bytes, including
zero, negative-zero, tie, saturation, tiny and huge blocks.  Within tolerance:
T and the bf16 output Y (relative Frobenius error <= 5e-3 and max |error| <=
1e-2 max |Y_ref|), with the weights packed by the oracle.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import svdq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("bit_diffusion_model_svdq_amd")

F32, F64 = np.float32, np.float64
Y_REL_FRO = 5e-3
Y_MAX_ABS = 1e-2
T_REL_FRO = 1e-4

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


_CACHE = {}


def packed_mx(name, M=None, K=None, N=None, rank=None):
    key = (name, M, K, N, rank)
    if key in _CACHE:
        return _CACHE[key]
    w = synth.WORKLOADS[name]
    M, K, N = M or w.M, K or w.K, N or w.N
    r = w.rank if rank is None else rank
    X = np.ascontiguousarray(synth.activations(w, max(M, w.M))[:M, :K])
    W = np.ascontiguousarray(synth.weight(w)[:N, :K])
    b = synth.bias(w)[:N]
    A = O.act_absmax(synth.calibration_activations(w)[:, :K])
    pk = O.pack_weights(W, A, w.alpha, rank=r)
    Wq, we = O.quantize_residual_mx(W, pk["s"], pk["L1"], pk["L2"])
    # the oracle takes row-major scales, the forward k-tiled ones
    p = dict(X=X, b=b, M=M, K=K, N=N, r=r, s=pk["s"], L1=pk["L1"], L2=pk["L2"], Wq=Wq, we=we,
             we_tiled=S.svdq_mxfp4_tile_scales(we))
    _CACHE[key] = p
    return p


def run_k1(X, s, L1):
    M, K = X.shape
    r = L1.shape[0] if L1 is not None and L1.size else 0
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    sx = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    T = torch.empty((M, max(r, 1)), dtype=torch.float32, device=DEV)
    S.svdq_quantize_activations_mxfp4(dev(X), dev(s), dev(L1) if r else None, qx, sx, T if r else None)
    torch.cuda.synchronize()
    return qx.cpu().numpy(), sx.cpu().numpy(), T.cpu().numpy()[:, :r]


def run_forward(p):
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    Y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    ws = torch.empty(S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r), dtype=torch.uint8, device=DEV)
    S.svdq_linear_forward_mxfp4(dev(p["X"]), dev(p["s"]), dev(p["L1"]) if r else None,
                                dev(p["L2"]) if r else None, dev(p["Wq"]), dev(p["we_tiled"]), dev(p["b"]), Y, ws)
    torch.cuda.synchronize()
    return O.bf16_to_f64(Y.cpu().numpy().view(np.uint16))


def check_y(Yg, Yref, label):
    rf, ma = O.rel_fro(Yg, Yref), O.max_abs_ratio(Yg, Yref)
    say(f"{label}: rel_fro {rf:.3e} max_abs/max {ma:.3e}")
    assert rf <= Y_REL_FRO and ma <= Y_MAX_ABS


def test_k1_mx_edge_blocks_bit_exact():
    """Hand-built blocks (s = 1, so x_hat = X): zeros with a negative zero, every E2M1
    tie, a block whose absmax 7 saturates, a bf16-subnormal block (scale 2^-127), a huge
    block, then random blocks; 16 rows so each is a full MFMA row tile."""
    say("k1 mx edge blocks")
    M, K = 16, 512
    g = np.random.default_rng(31)
    X = (g.standard_normal((M, K)) * np.exp(g.uniform(-6, 6, (M, 1)))).astype(F32)
    X[:, 0:32] = 0.0
    X[:, 5] = -0.0
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.25, -2.5, 6.0, 0.5], F32)
    X[:, 32:64] = 0.0
    X[:, 32:32 + len(ties)] = ties
    X[:, 64:96] = np.linspace(-7, 7, 32, dtype=F32)
    X[:, 96:128] = np.linspace(-1, 1, 32, dtype=F32) * F32(1e-39)
    X[:, 128:160] = np.linspace(-1, 1, 32, dtype=F32) * F32(3e38)
    Xb = synth.f32_to_bf16_bits(X)
    s = np.ones(K, F32)
    qx, sx, _ = run_k1(Xb, s, None)
    qx_o, sx_o, _, _ = O.quantize_activations_mx(Xb, s)
    np.testing.assert_array_equal(sx, sx_o)
    np.testing.assert_array_equal(qx, qx_o)
    assert sx_o[0, 0] == 0 and sx_o[0, 3] == 0 and sx_o[0, 4] == 252


@pytest.mark.parametrize("name", ["tiny", "smallk_640", "smallk_1280", "dit_proj"])
def test_k1_mx_codes_scales_bit_exact_and_T(name):
    say(f"k1 mx {name}")
    p = packed_mx(name)
    qx, sx, T = run_k1(p["X"], p["s"], p["L1"])
    qx_o, sx_o, T_o, _ = O.quantize_activations_mx(p["X"], p["s"], p["L1"])
    np.testing.assert_array_equal(sx, sx_o)
    np.testing.assert_array_equal(qx, qx_o)
    assert O.rel_fro(T, T_o) <= T_REL_FRO


@pytest.mark.parametrize("name", ["tiny", "smallk_640", "smallk_1280"])
def test_forward_mx_full(name):
    say(f"forward mx {name}")
    p = packed_mx(name)
    Yg = run_forward(p)
    Yref = O.forward_mx(p["X"], p["s"], p["L1"], p["L2"], p["Wq"], p["we"], p["b"])
    check_y(Yg, Yref, f"mx {name}")


def test_forward_mx_dit_proj_sampled_rows():
    say("forward mx dit_proj")
    p = packed_mx("dit_proj")
    Yg = run_forward(p)
    rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(p["M"] - 16, p["M"]),
                                     synth.rng_for("dit_proj", 40).choice(p["M"], 224, replace=False)]))
    Yref = O.forward_mx(p["X"][rows], p["s"], p["L1"], p["L2"], p["Wq"], p["we"], p["b"])
    check_y(Yg[rows], Yref, "mx dit_proj sampled")
    Yx = O.forward_exact(p["X"][rows], synth.weight(synth.WORKLOADS["dit_proj"]), p["b"])
    say(f"dit_proj MXFP4 method error vs X W^T + b: gpu {O.rel_fro(Yg[rows], Yx):.4f} "
        f"oracle {O.rel_fro(Yref, Yx):.4f}")


def test_forward_mx_long_token_batch_sampled_rows():
    """65536 tokens through the DiT projection's MXFP4 layer (16 times the benchmarked
    batch): codes and scale bytes bit-exact, Y within tolerance, on sampled rows that
    include both ends."""
    say("forward mx long batch, 65536 tokens")
    M = 16 * synth.WORKLOADS["dit_proj"].M
    p = packed_mx("dit_proj", M=M)
    K, N, r = p["K"], p["N"], p["r"]
    rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(M - 16, M),
                                     synth.rng_for("dit_proj", 41).choice(M, 224, replace=False)]))
    ridx = torch.from_numpy(rows).to(DEV)
    Xd, sd, L1d = dev(p["X"]), dev(p["s"]), dev(p["L1"])
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    sx = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    S.svdq_quantize_activations_mxfp4(Xd, sd, L1d, qx, sx, T)
    Y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    ws = torch.empty(S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r), dtype=torch.uint8, device=DEV)
    S.svdq_linear_forward_mxfp4(Xd, sd, L1d, dev(p["L2"]), dev(p["Wq"]), dev(p["we_tiled"]), dev(p["b"]), Y, ws)
    torch.cuda.synchronize()
    qx_o, sx_o, T_o = O.quantize_activations_mx(p["X"][rows], p["s"], p["L1"])[:3]
    np.testing.assert_array_equal(qx[ridx].cpu().numpy(), qx_o)
    np.testing.assert_array_equal(sx[ridx].cpu().numpy(), sx_o)
    assert O.rel_fro(T[ridx].cpu().numpy(), T_o) <= T_REL_FRO
    Yg = O.bf16_to_f64(Y[ridx].cpu().numpy().view(np.uint16))
    Yref = O.forward_mx(p["X"][rows], p["s"], p["L1"], p["L2"], p["Wq"], p["we"], p["b"])
    check_y(Yg, Yref, "mx long batch sampled")


@pytest.mark.parametrize("M,K,N,r", [(200, 640, 208, 48), (1, 128, 16, 16), (77, 256, 48, 0),
                                     (250, 384, 144, 128)])
def test_forward_mx_ragged_shapes(M, K, N, r):
    """Partial row and column tiles, an odd number of 128-channel steps (K = 640, 384:
    the last pipeline stage has one step), r = 0, 48 and 128, M = 1."""
    say(f"forward mx ragged {M}x{K}x{N} r={r}")
    p = packed_mx("tiny", M=M, K=K, N=N, rank=r)
    qx, sx, _ = run_k1(p["X"], p["s"], p["L1"])
    qx_o, sx_o, _, _ = O.quantize_activations_mx(p["X"], p["s"], p["L1"])
    np.testing.assert_array_equal(qx, qx_o)
    np.testing.assert_array_equal(sx, sx_o)
    Yg = run_forward(p)
    Yref = O.forward_mx(p["X"], p["s"], p["L1"], p["L2"], p["Wq"], p["we"], p["b"])
    check_y(Yg, Yref, f"mx ragged {M}x{K}x{N} r={r}")


def forward_parts_mx(p):
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    d = dict(X=dev(p["X"]), s=dev(p["s"]), L1=dev(p["L1"]) if r else None, L2=dev(p["L2"]) if r else None,
             Wq=dev(p["Wq"]), we=dev(p["we_tiled"]), b=dev(p["b"]))
    ws = torch.empty(S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r), dtype=torch.uint8, device=DEV)
    return d, ws


@pytest.mark.parametrize("name", ["smallk_1280", "smallk_640"])
def test_forward_mx_stages_match_the_forward_call(name):
    """svdq_forward_quantize_mxfp4 then svdq_forward_gemm_mxfp4 (the workspace carries the
    k-tiled activation scales between them) against svdq_linear_forward_mxfp4.  Where the
    forward runs those two stages (1024 x 1280 -> 1280), the outputs are identical bit for
    bit.  Where it runs the fused small-K kernel (4096 x 640 -> 640), that kernel sums T in
    another order, so both results are held to the oracle instead (its codes and scale
    bytes are compared bit for bit by the fused kernel's own tests)."""
    say(f"mx stages vs forward {name}")
    p = packed_mx(name)
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    Yf = run_forward(p)
    d, ws = forward_parts_mx(p)
    Y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    S.svdq_forward_quantize_mxfp4(d["X"], d["s"], d["L1"], ws)
    S.svdq_forward_gemm_mxfp4(M, K, d["L2"], d["Wq"], d["we"], d["b"], Y, ws, r)
    torch.cuda.synchronize()
    Ys = O.bf16_to_f64(Y.cpu().numpy().view(np.uint16))
    if not S.svdq_forward_fused_mxfp4(M, K, N, r):
        np.testing.assert_array_equal(Ys, Yf)
    else:
        Yref = O.forward_mx(p["X"], p["s"], p["L1"], p["L2"], p["Wq"], p["we"], p["b"])
        check_y(Ys, Yref, f"mx {name} two stages")
        check_y(Yf, Yref, f"mx {name} fused forward")


def test_forward_mx_in_hip_graph_replays_match_eager():
    """The MXFP4 forward captured in a HIP graph: every replay, with eager work and
    synchronizations between replays, reproduces the eager output bit for bit."""
    say("mx graph replay smallk_1280")
    p = packed_mx("smallk_1280")
    M, N = p["M"], p["N"]
    Y_eager = run_forward(p)
    d, ws = forward_parts_mx(p)
    Yg = torch.empty((M, N), dtype=torch.int16, device=DEV)
    fwd = lambda: S.svdq_linear_forward_mxfp4(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["we"], d["b"], Yg, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for rep in range(3):
        Yg.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(O.bf16_to_f64(Yg.cpu().numpy().view(np.uint16)), Y_eager,
                                      err_msg=f"replay {rep}")
        run_forward(p)              # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M,K", [(77, 640), (256, 1024)])
def test_k1_mx_workspace_scales_k_tiled(M, K):
    """The forward's workspace: codes [M, K/2] first, then the E8M0 scales k-tiled
    [ceil(K/256)][M rounded up to even][8] -- bit-exact against the oracle's row-major
    bytes re-indexed (an odd M and K % 256 == 128 exercise the row pitch and the tail)."""
    say(f"k1 mx workspace layout {M}x{K}")
    p = packed_mx("tiny", M=M, K=K, N=64, rank=16)
    d, ws = forward_parts_mx(p)
    S.svdq_forward_quantize_mxfp4(d["X"], d["s"], d["L1"], ws)
    torch.cuda.synchronize()
    qx_o, sx_o, _, _ = O.quantize_activations_mx(p["X"], p["s"], p["L1"])
    w = ws.cpu().numpy()
    qbytes = (M * K // 2 + 255) // 256 * 256
    np.testing.assert_array_equal(w[:M * K // 2].reshape(M, K // 2), qx_o)
    rows, nt, nb = M + (M & 1), (K + 255) // 256, K // 32
    tiled = w[qbytes:qbytes + nt * rows * 8].reshape(nt, rows, 8)
    got = tiled[:, :M, :].transpose(1, 0, 2).reshape(M, nt * 8)[:, :nb]
    np.testing.assert_array_equal(got, sx_o)


def _mx_ragged_case(M, K, N, r, wname, tag):
    w = synth.WORKLOADS[wname]
    X = np.ascontiguousarray(synth.activations(w, M)[:, :K])
    W = np.ascontiguousarray(synth.weight(w)[:N, :K])
    b = synth.bias(w)[:N]
    A = O.act_absmax(synth.calibration_activations(w)[:, :K])
    pk = O.pack_weights(W, A, 0.5, rank=r)
    Wq, we = O.quantize_residual_mx(W, pk["s"], pk["L1"], pk["L2"])
    p = dict(X=X, b=b, M=M, K=K, N=N, r=r, s=pk["s"], L1=pk["L1"], L2=pk["L2"], Wq=Wq, we=we,
             we_tiled=S.svdq_mxfp4_tile_scales(we))
    Yg = run_forward(p)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(4090, 4110), np.arange(M - 40, M),
                                     synth.rng_for("dit_proj", 34).choice(M, 200, replace=False)]))
    Yref = O.forward_mx(X[rows], pk["s"], pk["L1"], pk["L2"], Wq, we, b)
    check_y(Yg[rows], Yref, tag)


def test_forward_mx_partial_wave_ragged():
    """4300 x 640 -> 3072, r = 48: 17 x 16 = 272 tiles of 256 x 192 on 256 CUs leave 16.
    With 5 steps of 128 channels, K is too short for the remainder split, so 128 x 192
    tiles at two workgroups per CU run the GEMM: 544 tiles, the last wave partly
    filled, the last token tile ragged."""
    say("forward mx partial wave 4300x640x3072 r=48")
    _mx_ragged_case(4300, 640, 3072, 48, "dit_proj", "mx partial wave")


def test_forward_mx_remainder_split_ragged():
    """4300 x 7168 -> 3072, r = 48: 272 tiles of 256 x 192 on 256 CUs leave 16
    (including the ragged last token tile). With 56 steps of 128 channels, each is cut
    along K into 8 shares, which the fixup pass sums before it adds the low-rank
    branch and the bias."""
    say("forward mx remainder split 4300x7168x3072 r=48")
    _mx_ragged_case(4300, 7168, 3072, 48, "mlp_down", "mx remainder split")

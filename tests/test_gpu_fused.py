"""GPU parity of the fused small-K forward (one kernel: quantize, lora_down,
W4A4 GEMM, lora_up, bias, activation), int4 and MXFP4, through the C ABI.

The forward takes this path for K <= 1280, r <= 32, N <= 2560 and at most
256 blocks of 16 x 16 outputs x 64 channels per compute unit
(svdq_forward_fused).  Bit-exact: the activation codes and scales the fused
kernel quantized (svdq_debug_fused_forward writes them out) against the
oracle's quantizer (Terminology Entry, section 2.3, E2-E3).  Within the Y
tolerance of the other forward tests: every output against the oracle's
forward, at both small-K UNet widths and at ragged and edge shapes.
"""
import numpy as np
import pytest

import synth
from oracle import svdq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("bit_diffusion_model_svdq_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from test_gpu_parity import DEV, check_y, dev, host, packed, say, to_device  # noqa: E402

GELU = S.SVDQ_ACT_GELU_TANH


def layer(M, K, N, r, seed, bias=True):
    """A seeded layer packed by the oracle (outlier channels as in the workloads)."""
    g = np.random.default_rng(seed)
    X = (g.standard_normal((M, K)) * 1.5).astype(np.float32)
    X[:, g.choice(K, max(1, K // 200), replace=False)] *= 40.0
    W = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    Xb = synth.f32_to_bf16_bits(X)
    pk = O.pack_weights(W, O.act_absmax(Xb), 0.5, rank=r)
    b = O.bf16_from_f64(g.standard_normal(N) * 0.3) if bias else None
    return dict(X=Xb, W=W, b=b, r=r, M=M, K=K, N=N, **{k: pk[k] for k in ("s", "L1", "L2", "Wq", "w_scales")})


def fused_run(p, act=S.SVDQ_ACT_NONE):
    """svdq_debug_fused_forward: Y and the codes/scales the kernel quantized."""
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    d = to_device(p) if p["b"] is not None else dict(to_device(dict(p, b=np.zeros(N, np.uint16))), b=None)
    Y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    sx = torch.empty((M, K // 64), dtype=torch.float32, device=DEV)
    S.svdq_debug_fused_forward(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], act, Y, qx, sx)
    torch.cuda.synchronize()
    return d, O.bf16_to_f64(host(Y, np.uint16)), qx.cpu().numpy(), sx.cpu().numpy()


def oracle_y(p, act=S.SVDQ_ACT_NONE):
    b = p["b"] if p["b"] is not None else np.zeros(p["N"], np.uint16)
    return O.forward(p["X"], p["s"], p["L1"], p["L2"], p["Wq"], p["w_scales"], b,
                     activation="gelu_tanh" if act == GELU else None)


def check_codes(p, qx, sx, label):
    qx_o, sx_o, _, _ = O.quantize_activations(p["X"], p["s"], p["L1"])
    np.testing.assert_array_equal(qx, qx_o, err_msg=f"{label}: codes")
    np.testing.assert_array_equal(sx.view(np.uint32), sx_o.view(np.uint32), err_msg=f"{label}: scales")


@pytest.mark.parametrize("name,M", [("smallk_640", 1024), ("smallk_1280", 256)])
def test_fused_smallk_workloads_codes_and_every_output(name, M):
    """The small-K UNet widths (640 -> 640 at 1024 tokens, 1280 -> 1280 at 256
    tokens, r = 32): codes and scales bit-exact, every output within tolerance,
    and the plain forward identical to the debug launch bit for bit."""
    p = packed(name, M=M)
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    say(f"fused {name} {M}x{K}x{N} r={r}")
    assert S.svdq_forward_fused(M, K, N, r)
    d, Yg, qx, sx = fused_run(p)
    check_codes(p, qx, sx, name)
    check_y(Yg, oracle_y(p), f"fused {name}")
    Y2 = torch.empty((M, N), dtype=torch.int16, device=DEV)
    ws = torch.empty(S.svdq_forward_workspace_bytes(M, K, N, r), dtype=torch.uint8, device=DEV)
    S.svdq_linear_forward(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], Y2, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(Y2, np.uint16), O.bf16_from_f64(Yg))


# (M, K, N, r, bias, act): ragged rows and columns, one group, the K, N and r
# limits, no low-rank branch, no bias, GELU
EDGES = [
    (200, 640, 208, 32, True, S.SVDQ_ACT_NONE),
    (1, 64, 16, 16, True, S.SVDQ_ACT_NONE),
    (37, 1280, 2560, 32, True, GELU),
    (300, 1280, 1280, 0, True, S.SVDQ_ACT_NONE),
    (129, 320, 400, 16, False, GELU),
    (1024, 640, 640, 16, True, GELU),
]


@pytest.mark.parametrize("M,K,N,r,bias,act", EDGES, ids=[f"{e[0]}x{e[1]}x{e[2]}r{e[3]}" for e in EDGES])
def test_fused_edges(M, K, N, r, bias, act):
    say(f"fused edge M={M} K={K} N={N} r={r} bias={bias} act={act}")
    assert S.svdq_forward_fused(M, K, N, r)
    p = layer(M, K, N, r, seed=M + 7 * K + 13 * N + r, bias=bias)
    _, Yg, qx, sx = fused_run(p, act)
    check_codes(p, qx, sx, f"{M}x{K}x{N}")
    check_y(Yg, oracle_y(p, act), f"fused {M}x{K}x{N} r={r}")


def test_fused_range_and_rejection():
    """Shapes past the fused range run the two-kernel forward; the debug entry
    point refuses them before launching anything."""
    assert not S.svdq_forward_fused(4096, 1344, 640, 32)     # K past 1280
    assert not S.svdq_forward_fused(4096, 640, 640, 48)      # r past 32 (the LoRA-widened rank)
    assert not S.svdq_forward_fused(4096, 640, 2576, 32)     # N past 2560
    assert not S.svdq_forward_fused(4096, 3072, 3072, 32)    # the DiT projection
    assert not S.svdq_forward_fused(4096, 640, 640, 32)      # 400 group-tiles per compute unit
    assert S.svdq_forward_fused(1024, 640, 640, 32)          # 100
    assert not S.svdq_forward_fused(0, 640, 640, 32)         # invalid shapes: 0
    p = layer(64, 1344, 64, 16, seed=5)
    d = to_device(p)
    Y = torch.empty((64, 64), dtype=torch.int16, device=DEV)
    qx = torch.empty((64, 1344 // 2), dtype=torch.uint8, device=DEV)
    sx = torch.empty((64, 1344 // 64), dtype=torch.float32, device=DEV)
    with pytest.raises(S.SvdqError) as e:
        S.svdq_debug_fused_forward(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"],
                                   S.SVDQ_ACT_NONE, Y, qx, sx)
    assert e.value.status == 1


# ---------------------------------------------------------------- MXFP4
# The same fused forward with Q taken as MXFP4 (svdq_forward_fused_mxfp4: the
# int4 range with K a multiple of 128, up to 400 blocks of 16 x 16 x 64 per
# compute unit where K <= 640): codes and E8M0 bytes bit-exact against
# the oracle's MXFP4 quantizer, every output within the MXFP4 forward tests'
# tolerance of the oracle's forward_mx.
from test_gpu_mxfp4 import check_y as check_y_mx  # noqa: E402
from test_gpu_mxfp4 import packed_mx  # noqa: E402


def mx_layer(M, K, N, r, seed, bias=True):
    """A seeded layer, MXFP4 residual packed by the oracle (outlier channels as in the workloads)."""
    g = np.random.default_rng(seed)
    X = (g.standard_normal((M, K)) * 1.5).astype(np.float32)
    X[:, g.choice(K, max(1, K // 200), replace=False)] *= 40.0
    W = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    Xb = synth.f32_to_bf16_bits(X)
    pk = O.pack_weights(W, O.act_absmax(Xb), 0.5, rank=r)
    Wq, we = O.quantize_residual_mx(W, pk["s"], pk["L1"], pk["L2"])
    b = O.bf16_from_f64(g.standard_normal(N) * 0.3) if bias else None
    return dict(X=Xb, b=b, r=r, M=M, K=K, N=N, s=pk["s"], L1=pk["L1"], L2=pk["L2"], Wq=Wq, we=we,
                we_tiled=S.svdq_mxfp4_tile_scales(we))


def mx_device(p):
    r = p["r"]
    return dict(X=dev(p["X"]), s=dev(p["s"]), L1=dev(p["L1"]) if r else None,
                L2=dev(p["L2"]) if r else None, Wq=dev(p["Wq"]), we=dev(p["we_tiled"]),
                b=dev(p["b"]) if p["b"] is not None else None)


def fused_run_mx(p, act=S.SVDQ_ACT_NONE):
    """svdq_debug_fused_forward_mxfp4: Y and the codes / E8M0 bytes the kernel quantized."""
    M, K, N = p["M"], p["K"], p["N"]
    d = mx_device(p)
    Y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    sx = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    S.svdq_debug_fused_forward_mxfp4(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["we"], d["b"], act, Y,
                                     qx, sx)
    torch.cuda.synchronize()
    return d, O.bf16_to_f64(host(Y, np.uint16)), qx.cpu().numpy(), sx.cpu().numpy()


def oracle_y_mx(p, act=S.SVDQ_ACT_NONE):
    b = p["b"] if p["b"] is not None else np.zeros(p["N"], np.uint16)
    return O.forward_mx(p["X"], p["s"], p["L1"], p["L2"], p["Wq"], p["we"], b,
                        activation="gelu_tanh" if act == GELU else None)


def check_codes_mx(p, qx, sx, label):
    qx_o, sx_o, _, _ = O.quantize_activations_mx(p["X"], p["s"], p["L1"])
    np.testing.assert_array_equal(qx, qx_o, err_msg=f"{label}: codes")
    np.testing.assert_array_equal(sx, sx_o, err_msg=f"{label}: E8M0 bytes")


@pytest.mark.parametrize("name,M", [("smallk_640", 1024), ("smallk_640", None), ("smallk_1280", 256)])
def test_fused_mx_smallk_workloads_codes_and_every_output(name, M):
    """The small-K UNet widths in MXFP4: codes and scale bytes bit-exact, every
    output within tolerance, the plain forward identical to the debug launch."""
    p = packed_mx(name, M=M)
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    say(f"fused mx {name} {M}x{K}x{N} r={r}")
    assert S.svdq_forward_fused_mxfp4(M, K, N, r)
    d, Yg, qx, sx = fused_run_mx(p)
    check_codes_mx(p, qx, sx, name)
    check_y_mx(Yg, oracle_y_mx(p), f"fused mx {name}")
    Y2 = torch.empty((M, N), dtype=torch.int16, device=DEV)
    ws = torch.empty(S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r), dtype=torch.uint8, device=DEV)
    S.svdq_linear_forward_mxfp4(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["we"], d["b"], Y2, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(Y2, np.uint16), O.bf16_from_f64(Yg))


# (M, K, N, r, bias, act): ragged rows and columns, one 128-channel step, the K,
# N and r limits, no low-rank branch, no bias, GELU, an odd number of steps
MX_EDGES = [
    (200, 640, 208, 32, True, S.SVDQ_ACT_NONE),
    (1, 128, 16, 16, True, S.SVDQ_ACT_NONE),
    (37, 1280, 2560, 32, True, GELU),
    (300, 1280, 1280, 0, True, S.SVDQ_ACT_NONE),
    (129, 384, 400, 16, False, GELU),
    (1024, 640, 640, 16, True, GELU),
]


@pytest.mark.parametrize("M,K,N,r,bias,act", MX_EDGES, ids=[f"{e[0]}x{e[1]}x{e[2]}r{e[3]}" for e in MX_EDGES])
def test_fused_mx_edges(M, K, N, r, bias, act):
    say(f"fused mx edge M={M} K={K} N={N} r={r} bias={bias} act={act}")
    assert S.svdq_forward_fused_mxfp4(M, K, N, r)
    p = mx_layer(M, K, N, r, seed=3 * M + 5 * K + 11 * N + r, bias=bias)
    _, Yg, qx, sx = fused_run_mx(p, act)
    check_codes_mx(p, qx, sx, f"{M}x{K}x{N}")
    check_y_mx(Yg, oracle_y_mx(p, act), f"fused mx {M}x{K}x{N} r={r}")


def test_fused_mx_range_and_rejection():
    """Shapes past the fused range run the two-kernel MXFP4 forward; the debug
    entry point refuses them before launching anything."""
    assert not S.svdq_forward_fused_mxfp4(1024, 704, 640, 32)     # K not a multiple of 128
    assert not S.svdq_forward_fused_mxfp4(1024, 1408, 640, 32)    # K past 1280
    assert not S.svdq_forward_fused_mxfp4(1024, 640, 640, 48)     # r past 32
    assert not S.svdq_forward_fused_mxfp4(1024, 640, 2576, 32)    # N past 2560
    assert not S.svdq_forward_fused_mxfp4(6144, 640, 640, 32)     # 600 group-tiles per compute unit
    assert not S.svdq_forward_fused_mxfp4(1024, 1280, 1280, 32)   # 400 at K = 1280
    assert S.svdq_forward_fused_mxfp4(4096, 640, 640, 32)         # 400 at K = 640
    assert S.svdq_forward_fused_mxfp4(1024, 640, 640, 32)
    p = mx_layer(64, 1408, 64, 16, seed=9)
    d = mx_device(p)
    Y = torch.empty((64, 64), dtype=torch.int16, device=DEV)
    qx = torch.empty((64, 1408 // 2), dtype=torch.uint8, device=DEV)
    sx = torch.empty((64, 1408 // 32), dtype=torch.uint8, device=DEV)
    with pytest.raises(S.SvdqError) as e:
        S.svdq_debug_fused_forward_mxfp4(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["we"], d["b"],
                                         S.SVDQ_ACT_NONE, Y, qx, sx)
    assert e.value.status == 1

"""GPU parity of the DiT block path: GELU (tanh form) fused into the GEMM
epilogue, the up -> down chain of the MLP fed straight from the fused output,
and the fused QKV width (N = 9216), each with the rank-32 branch widened by a
seeded rank-16 LoRA to r = 48 -- int4 and MXFP4, through the C ABI.

Every input and expected value is the oracle's: the oracle runs the same chain
on the sampled rows (its up projection, GELU, bf16 rounding, its down
projection), never on GPU output.
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

from test_gpu_parity import DEV, check_y, dev, host, packed, say  # noqa: E402

GELU = S.SVDQ_ACT_GELU_TANH


def with_lora(name, mx=False):
    """The workload's oracle pack with its seeded rank-16 LoRA appended (r = 48);
    for mx the residual is re-quantized to MXFP4 from the same s, L1, L2."""
    p = dict(packed(name))
    if mx:
        p["Wq"], p["w_scales"] = O.quantize_residual_mx(p["W"], p["s"], p["L1"], p["L2"])
    A, B = synth.lora_factors(synth.WORKLOADS[name])
    p["L1"], p["L2"] = O.append_lora(p["s"], p["L1"], p["L2"], A, B)
    p["r"] = p["L1"].shape[0]
    return p


def layer_to_device(p):
    """Device copies of a packed layer; MXFP4 weight scales (E8M0 bytes) go k-tiled, as the
    forward reads them."""
    ws = p["w_scales"]
    if ws.dtype == np.uint8:
        ws = S.svdq_mxfp4_tile_scales(ws)
    return dict(s=dev(p["s"]), L1=dev(p["L1"]), L2=dev(p["L2"]), Wq=dev(p["Wq"]), ws=dev(ws),
                b=dev(p["b"]))


def gpu_linear(Xd, d, M, K, N, r, act, mx):
    """One linear through the _act entry point; Xd is a bf16 (int16) device tensor [M, K]."""
    Y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    if mx:
        ws = torch.empty(S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r), dtype=torch.uint8, device=DEV)
        S.svdq_linear_forward_act_mxfp4(Xd, d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], act, Y, ws)
    else:
        ws = torch.empty(S.svdq_forward_workspace_bytes(M, K, N, r), dtype=torch.uint8, device=DEV)
        S.svdq_linear_forward_act(Xd, d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], act, Y, ws)
    return Y


def oracle_linear(X_bf16, p, act, mx):
    f = O.forward_mx if mx else O.forward
    return f(X_bf16, p["s"], p["L1"], p["L2"], p["Wq"], p["w_scales"], p["b"],
             activation="gelu_tanh" if act == GELU else None)


@pytest.mark.parametrize("mx", [False, True], ids=["int4", "mxfp4"])
def test_gelu_epilogue_tiny_full(mx):
    """The tiny layer with GELU fused: every output against the oracle."""
    say(f"gelu tiny {'mxfp4' if mx else 'int4'}")
    p = dict(packed("tiny"))
    if mx:
        p["Wq"], p["w_scales"] = O.quantize_residual_mx(p["W"], p["s"], p["L1"], p["L2"])
    d = layer_to_device(p)
    Y = gpu_linear(dev(p["X"]), d, p["M"], p["K"], p["N"], p["r"], GELU, mx)
    torch.cuda.synchronize()
    Yg = O.bf16_to_f64(host(Y, np.uint16))
    check_y(Yg, oracle_linear(p["X"], p, GELU, mx), f"gelu tiny {'mx' if mx else 'int4'}")
    assert Yg.min() >= -0.171   # GELU's floor survives the fusion


@pytest.mark.parametrize("mx", [False, True], ids=["int4", "mxfp4"])
def test_gelu_epilogue_ragged(mx):
    """Ragged tiles (M, N not multiples of the tile) with r = 48 and GELU."""
    M, K, N, r = 200, 640, 208, 48
    say(f"gelu ragged {M}x{K}x{N} r={r} {'mxfp4' if mx else 'int4'}")
    g = synth.rng_for("tiny", 41)
    X = synth.f32_to_bf16_bits((g.standard_normal((M, K)) * 2.0).astype(np.float32))
    W = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    s = np.exp(g.uniform(-1, 1, K)).astype(np.float32)
    L1 = O.bf16_from_f64(g.standard_normal((r, K)) * 0.05)
    L2 = O.bf16_from_f64(g.standard_normal((N, r)) * 0.05)
    b = O.bf16_from_f64(g.standard_normal(N) * 0.3)
    if mx:
        Wq, ws = O.quantize_residual_mx(W, s, L1, L2)
    else:
        Wq, ws = O.quantize_residual(W, s, L1, L2)
    p = dict(s=s, L1=L1, L2=L2, Wq=Wq, w_scales=ws, b=b)
    Y = gpu_linear(dev(X), layer_to_device(p), M, K, N, r, GELU, mx)
    torch.cuda.synchronize()
    check_y(O.bf16_to_f64(host(Y, np.uint16)), oracle_linear(X, p, GELU, mx), "gelu ragged")


def test_unknown_activation_rejected():
    p = dict(packed("tiny"))
    d = layer_to_device(p)
    with pytest.raises(S.SvdqError) as e:
        gpu_linear(dev(p["X"]), d, p["M"], p["K"], p["N"], p["r"], 7, False)
    assert e.value.status == 1
    pm = dict(p)
    pm["Wq"], pm["w_scales"] = O.quantize_residual_mx(p["W"], p["s"], p["L1"], p["L2"])
    with pytest.raises(S.SvdqError) as e:
        gpu_linear(dev(p["X"]), layer_to_device(pm), p["M"], p["K"], p["N"], p["r"], -1, True)
    assert e.value.status == 1


@pytest.mark.parametrize("mx", [False, True], ids=["int4", "mxfp4"])
def test_mlp_chain_full_size(mx):
    """The DiT MLP at full size (4608 tokens, 3072 -> 12288 -> 3072, r = 48 on both
    linears): the up projection with GELU fused writes H, which the down projection
    reads directly.  Sampled rows of H and of the block output against the oracle's
    own chain on those rows."""
    say(f"mlp chain {'mxfp4' if mx else 'int4'}")
    up, down = with_lora("mlp_up", mx), with_lora("mlp_down", mx)
    M, K, Nh = up["M"], up["K"], up["N"]
    assert down["K"] == Nh and down["M"] == M
    H = gpu_linear(dev(up["X"]), layer_to_device(up), M, K, Nh, up["r"], GELU, mx)
    Y = gpu_linear(H, layer_to_device(down), M, Nh, down["N"], down["r"], S.SVDQ_ACT_NONE, mx)
    torch.cuda.synchronize()
    g = synth.rng_for("mlp_up", 43)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(M - 8, M), g.choice(M, 48, replace=False)]))
    Hg = O.bf16_to_f64(host(H, np.uint16)[rows])
    Yg = O.bf16_to_f64(host(Y, np.uint16)[rows])
    H_ref = oracle_linear(up["X"][rows], up, GELU, mx)
    check_y(Hg, H_ref, "mlp up + GELU (sampled rows)")
    H_ref_bf16 = O.bf16_from_f64(H_ref)
    Y_ref = oracle_linear(H_ref_bf16, down, S.SVDQ_ACT_NONE, mx)
    check_y(Yg, Y_ref, "mlp up -> GELU -> down (sampled rows)")


@pytest.mark.parametrize("mx", [False, True], ids=["int4", "mxfp4"])
def test_dit_qkv_full_launch_sampled_rows(mx):
    """The fused QKV projection (3072 -> 9216, 4608 tokens, r = 48) at full size."""
    say(f"dit qkv {'mxfp4' if mx else 'int4'}")
    p = with_lora("dit_qkv", mx)
    M = p["M"]
    Y = gpu_linear(dev(p["X"]), layer_to_device(p), M, p["K"], p["N"], p["r"], S.SVDQ_ACT_NONE, mx)
    torch.cuda.synchronize()
    g = synth.rng_for("dit_qkv", 44)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(M - 8, M), g.choice(M, 48, replace=False)]))
    check_y(O.bf16_to_f64(host(Y, np.uint16)[rows]), oracle_linear(p["X"][rows], p, S.SVDQ_ACT_NONE, mx),
            "dit qkv (sampled rows)")

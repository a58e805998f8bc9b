"""Bit-exact checks on the forward's own launch plans, through the C ABI.

The forward picks its GEMM tile from the shape (256x192 one per CU, 128x192 two
per CU, 128x128, 64x64), cuts a last, nearly empty wave of tiles along K into
shares, and plans the quantize kernel as one or several K-slices.  The tests
here take their bit-exact values from exactly those launches:

- the exact int32 group partials P ([Term] 2.3, E4 and E7) of windows of each
  tile class and of the split shares, from svdq_debug_group_partials, which
  runs the forward's GEMM launch for the whole M x N x K layer;
- the int4 and MXFP4 activation codes and scales that svdq_forward_quantize
  leaves in the workspace under multi-slice plans (DiT projection: 2 slices,
  MLP down projection: 5 slices), with T summed over its slices;
- Y over the whole 4096 x 3072 headline matrix and over the DiT block's
  attention output projection (4608 x 3072 -> 3072, r = 48) in both formats.
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

from test_gpu_parity import DEV, T_REL_FRO, check_y, dev, host, packed, run_forward, say, to_device  # noqa: E402
from test_gpu_block import gpu_linear, layer_to_device, oracle_linear, with_lora  # noqa: E402

_CODES = {}


def random_codes(rows, K, seed):
    """Packed int4 codes in [-7, 7] with both extremes present in every row."""
    key = (rows, K, seed)
    if key not in _CODES:
        g = np.random.default_rng(seed)
        q = g.integers(-7, 8, size=(rows, K)).astype(np.int8)
        q[:, 0] = 7
        q[:, 1] = -7
        _CODES[key] = O.pack_nibbles(q)
    return _CODES[key]


# (label, M, K, N): the tile class each shape selects on 256 compute units
PLANS = [
    ("256x192 tiles, one wave", 4096, 3072, 3072),
    ("128x192 tiles, two per CU", 4608, 3072, 9216),
    ("128x192 tiles with the K-split remainder", 4608, 12288, 3072),
    ("128x128 tiles", 2048, 1024, 2048),
    ("64x64 tiles", 4096, 640, 640),
]
WINDOWS = {
    4096 * 3072: [(0, 300, 0, 200), (3968, 4096, 2880, 3072), (1000, 1001, 1500, 1501)],
    4608 * 9216: [(4500, 4608, 9000, 9216), (0, 130, 180, 200)],
    4608 * 3072: [(4090, 4160, 0, 200), (4500, 4608, 2900, 3072), (100, 140, 1000, 1010)],
    2048 * 2048: [(1900, 2048, 0, 300)],
    4096 * 640: [(0, 64, 0, 640), (4000, 4096, 600, 640)],
}


@pytest.mark.parametrize("label,M,K,N", PLANS, ids=[p[0] for p in PLANS])
def test_group_partials_from_the_forward_launch(label, M, K, N):
    qx = random_codes(M, K, seed=M + K)
    wq = random_codes(N, K, seed=N + 7 * K)
    qxd, wqd = dev(qx), dev(wq)
    G = K // 64
    for (m0, m1, n0, n1) in WINDOWS[M * N]:
        say(f"P {label} {M}x{K}x{N} window [{m0},{m1})x[{n0},{n1})")
        P = torch.empty((m1 - m0, n1 - n0, G), dtype=torch.int32, device=DEV)
        S.svdq_debug_group_partials(qxd, wqd, m0, m1, n0, n1, P)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(P.cpu().numpy(), O.group_partials(qx[m0:m1], wq[n0:n1]))


def _workspace_view(ws, off, nbytes):
    return ws[off:off + nbytes].cpu().numpy()


@pytest.mark.parametrize("name,slices", [("dit_proj", 2), ("mlp_down", 5)])
def test_forward_workspace_codes_bit_exact_int4(name, slices):
    """svdq_forward_quantize under the forward's own multi-slice plan: qx and sx in the
    workspace equal the oracle's bit for bit; the T slices, summed in order, equal T."""
    p = packed(name)
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    lay = S.svdq_forward_workspace_layout(M, K, N, r)
    say(f"workspace int4 {name}: {lay}")
    assert lay["t_slices"] == slices
    d = to_device(p)
    ws = torch.empty(S.svdq_forward_workspace_bytes(M, K, N, r), dtype=torch.uint8, device=DEV)
    S.svdq_forward_quantize(d["X"], d["s"], d["L1"], ws)
    torch.cuda.synchronize()
    qx = _workspace_view(ws, lay["qx"], M * K // 2).reshape(M, K // 2)
    sx = _workspace_view(ws, lay["sx"], M * K // 16).view(np.float32).reshape(M, K // 64)
    Ts = _workspace_view(ws, lay["T"], slices * M * r * 4).view(np.float32).reshape(slices, M, r)
    qx_o, sx_o, T_o, _ = O.quantize_activations(p["X"], p["s"], p["L1"])
    np.testing.assert_array_equal(qx, qx_o)
    np.testing.assert_array_equal(sx.view(np.uint32), sx_o.view(np.uint32))
    T = Ts[0].astype(np.float32)
    for i in range(1, slices):
        T = (T + Ts[i]).astype(np.float32)
    assert O.rel_fro(T, T_o) <= T_REL_FRO


def test_forward_workspace_codes_bit_exact_mxfp4_two_slices():
    """MXFP4 at the DiT projection (two K-slices): codes and the k-tiled E8M0 scales in the
    workspace, against the oracle's row-major bytes re-indexed."""
    p = dict(packed("dit_proj"))
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    lay = S.svdq_forward_workspace_layout(M, K, N, r, mxfp4=True)
    say(f"workspace mxfp4 dit_proj: {lay}")
    assert lay["t_slices"] == 2
    d = to_device(p)
    ws = torch.empty(S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r), dtype=torch.uint8, device=DEV)
    S.svdq_forward_quantize_mxfp4(d["X"], d["s"], d["L1"], ws)
    torch.cuda.synchronize()
    qx_o, sx_o, T_o, _ = O.quantize_activations_mx(p["X"], p["s"], p["L1"])
    qx = _workspace_view(ws, lay["qx"], M * K // 2).reshape(M, K // 2)
    np.testing.assert_array_equal(qx, qx_o)
    rows, nt, nb = lay["sx_rows"], (K + 255) // 256, K // 32
    tiled = _workspace_view(ws, lay["sx"], nt * rows * 8).reshape(nt, rows, 8)
    got = tiled[:, :M, :].transpose(1, 0, 2).reshape(M, nt * 8)[:, :nb]
    np.testing.assert_array_equal(got, sx_o)
    Ts = _workspace_view(ws, lay["T"], 2 * M * r * 4).view(np.float32).reshape(2, M, r)
    assert O.rel_fro((Ts[0] + Ts[1]).astype(np.float32), T_o) <= T_REL_FRO


def test_forward_headline_every_output():
    """The benchmarked launch (4096 x 3072 -> 3072, r = 32) against the oracle on all
    12.6 M outputs."""
    say("forward dit_proj, every output")
    p = packed("dit_proj")
    d = to_device(p)
    Yg = run_forward(p, d)
    Yref = O.forward(p["X"], p["s"], p["L1"], p["L2"], p["Wq"], p["w_scales"], p["b"])
    check_y(Yg, Yref, "dit_proj full")


@pytest.mark.parametrize("mx", [False, True], ids=["int4", "mxfp4"])
def test_dit_out_projection_at_its_shape(mx):
    """The DiT block's attention output projection at its own shape (4608 x 3072 -> 3072,
    rank 32 plus the seeded rank-16 LoRA, r = 48): every output against the oracle."""
    say(f"dit out projection {'mxfp4' if mx else 'int4'}")
    p = with_lora("dit_out", mx)
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    assert (M, K, N, r) == (4608, 3072, 3072, 48)
    Y = gpu_linear(dev(p["X"]), layer_to_device(p), M, K, N, r, S.SVDQ_ACT_NONE, mx)
    torch.cuda.synchronize()
    check_y(O.bf16_to_f64(host(Y, np.uint16)), oracle_linear(p["X"], p, S.SVDQ_ACT_NONE, mx),
            f"dit out {'mx' if mx else 'int4'}")


# The 256x192 and 128x128 tiles store their output wave by wave (each wave stages
# its share in LDS and writes its own row segments); the shapes below select those
# tiles with a partial last row tile and a partial last column tile.
WAVE_STORE = [("256x192 tiles, ragged", "dit_proj", 4000, 3072, 3056),
              ("128x128 tiles, ragged", "dit_qkv", 2000, 1024, 2032),
              ("256x192 tiles, one stage", "dit_proj", 4096, 128, 3072),
              ("256x192 tiles, two stages, the last one group", "dit_proj", 4096, 192, 3072)]


@pytest.mark.parametrize("act", [0, 1], ids=["none", "gelu"])
@pytest.mark.parametrize("label,name,M,K,N", WAVE_STORE, ids=[w[0] for w in WAVE_STORE])
def test_wave_store_tiles_ragged(label, name, M, K, N, act):
    """The per-wave store on ragged tiles, with and without the fused GELU: every
    output of the last 80 rows (the partial row tile) and of 64 rows spread over
    the rest, every column (the partial column tile included), against the oracle."""
    say(f"wave store {label} {M}x{K}x{N} act={act}")
    p = packed(name, M=M, K=K, N=N)
    d = to_device(p)
    Y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    ws = torch.empty(S.svdq_forward_workspace_bytes(M, K, N, p["r"]), dtype=torch.uint8, device=DEV)
    S.svdq_linear_forward_act(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], act, Y, ws)
    torch.cuda.synchronize()
    Yg = O.bf16_to_f64(host(Y, np.uint16))
    rows = np.unique(np.concatenate([np.linspace(0, M - 81, 64).astype(int), np.arange(M - 80, M)]))
    Yref = O.forward(p["X"][rows], p["s"], p["L1"], p["L2"], p["Wq"], p["w_scales"], p["b"],
                     activation="gelu_tanh" if act else None)
    check_y(Yg[rows], Yref, f"wave store {label} act={act}")


@pytest.mark.parametrize("act", [0, 1], ids=["none", "gelu"])
@pytest.mark.parametrize("M,K,N", [(4000, 3072, 3056), (4096, 128, 3072)], ids=["ragged", "one step"])
def test_wave_store_mxfp4_ragged(M, K, N, act):
    """The MXFP4 GEMM's per-wave store (256x192 tiles, four-buffer ring): the last 80
    rows and 64 spread rows, every column, against the oracle's MXFP4 forward."""
    say(f"wave store mxfp4 {M}x{K}x{N} act={act}")
    p = dict(packed("dit_proj", M=M, K=K, N=N))
    p["Wq"], p["w_scales"] = O.quantize_residual_mx(p["W"], p["s"], p["L1"], p["L2"])
    d = layer_to_device(p)
    Y = gpu_linear(dev(p["X"]), d, M, K, N, p["r"], act, True)
    torch.cuda.synchronize()
    Yg = O.bf16_to_f64(host(Y, np.uint16))
    rows = np.unique(np.concatenate([np.linspace(0, M - 81, 64).astype(int), np.arange(M - 80, M)]))
    Yref = O.forward_mx(p["X"][rows], p["s"], p["L1"], p["L2"], p["Wq"], p["w_scales"], p["b"],
                        activation="gelu_tanh" if act else None)
    check_y(Yg[rows], Yref, f"wave store mxfp4 {M}x{K}x{N} act={act}")

"""A seeded sweep of layer shapes through the forward, both formats, against the
oracle on sampled rows (through the C ABI).

The fixed-shape tests pin the benchmarked workloads and chosen edge cases; this
sweep draws M, K, N, r, bias and activation at random within the forward's
limits, so that many combinations of the launch plans meet the oracle: the
fused small-K kernel or the two kernels, each GEMM tile class, the K-split,
partial waves and ragged last tiles, k1's slice plans.  The low-rank factors
are drawn directly (the branch's arithmetic does not depend on where L1 and L2
come from) and the residual goes through the oracle's quantizer
(Terminology Entry, section 2.3, E2-E4), so no SVD is needed per shape.  Every
output row sampled is held to the tolerance of the other forward tests; the
codes and scales themselves are compared bit for bit by the k1 and fused tests.
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

DEV = torch.device("cuda:0")
Y_REL_FRO, Y_MAX_ABS = 5e-3, 1e-2
CASES = 24
ROWS = 24


def dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(DEV)


def draw(seed, mx):
    g = np.random.default_rng(seed)
    step = 128 if mx else 64
    K = int(g.choice([1, 2, 3, 5, 8, 10, 12, 16, 20, 24, 40, 48, 64])) * step // (2 if mx else 1)
    K = max(step, K // step * step)
    N = 16 * int(g.integers(1, 320))
    M = int(g.choice([1, 7, 64, 200, 513, 1024, 2047, 4096, 4608, int(g.integers(1, 6000))]))
    # keep the oracle's work (sampled rows x K x N) and the test's memory modest
    while K * N > (24 << 20):
        N = max(16, N // 2 // 16 * 16)
    r = int(g.choice([0, 16, 32, 48]))
    return M, K, N, r, bool(g.integers(0, 2)), int(g.integers(0, 2))


def case(seed, mx):
    M, K, N, r, has_bias, act = draw(seed, mx)
    g = np.random.default_rng(seed + 1)
    X = (g.standard_normal((M, K)) * 1.2).astype(np.float32)
    X[:, g.choice(K, max(1, K // 200), replace=False)] *= 30.0     # outlier channels
    Xb = synth.f32_to_bf16_bits(X)
    W = (g.standard_normal((N, K)) * 0.04).astype(np.float32)
    s = np.exp(g.uniform(-1.5, 1.5, K)).astype(np.float32)
    L1 = O.bf16_from_f64(g.standard_normal((r, K)) * 0.02)
    L2 = O.bf16_from_f64(g.standard_normal((N, r)) * 0.02)
    if mx:
        Wq, ws = O.quantize_residual_mx(W, s, L1, L2)
    else:
        Wq, ws = O.quantize_residual(W, s, L1, L2)
    b = O.bf16_from_f64(g.standard_normal(N) * 0.2) if has_bias else None
    return dict(M=M, K=K, N=N, r=r, act=act, X=Xb, s=s, L1=L1, L2=L2, Wq=Wq, ws=ws, b=b)


@pytest.mark.parametrize("mx", [False, True], ids=["int4", "mxfp4"])
@pytest.mark.parametrize("i", range(CASES))
def test_random_shape_against_oracle(i, mx):
    p = case(1000 * i + (7 if mx else 3), mx)
    M, K, N, r, act = p["M"], p["K"], p["N"], p["r"], p["act"]
    fused = (S.svdq_forward_fused_mxfp4 if mx else S.svdq_forward_fused)(M, K, N, r)
    print(f"sweep {'mxfp4' if mx else 'int4'} M={M} K={K} N={N} r={r} bias={p['b'] is not None} "
          f"act={act} fused={fused}", flush=True)
    Y = torch.full((M, N), 0x7FC0, dtype=torch.int16, device=DEV)
    ws_dev = dev(S.svdq_mxfp4_tile_scales(p["ws"]) if mx else p["ws"])
    nbytes = (S.svdq_forward_workspace_bytes_mxfp4 if mx else S.svdq_forward_workspace_bytes)(M, K, N, r)
    work = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    f = S.svdq_linear_forward_act_mxfp4 if mx else S.svdq_linear_forward_act
    f(dev(p["X"]), dev(p["s"]), dev(p["L1"]) if r else None, dev(p["L2"]) if r else None, dev(p["Wq"]),
      ws_dev, dev(p["b"]) if p["b"] is not None else None, act, Y, work)
    torch.cuda.synchronize()
    g = np.random.default_rng(i)
    rows = np.unique(np.concatenate([[0, M - 1], g.choice(M, min(M, ROWS), replace=False)]))
    Yg = O.bf16_to_f64(Y[torch.from_numpy(rows).to(DEV)].cpu().numpy().view(np.uint16))
    fwd = O.forward_mx if mx else O.forward
    Yref = fwd(p["X"][rows], p["s"], p["L1"] if r else None, p["L2"] if r else None, p["Wq"], p["ws"],
               p["b"], activation="gelu_tanh" if act else None)
    rf, ma = O.rel_fro(Yg, Yref), O.max_abs_ratio(Yg, Yref)
    print(f"  rel_fro {rf:.3e} max_abs/max {ma:.3e}", flush=True)
    assert np.isfinite(Yg).all()
    assert rf <= Y_REL_FRO and ma <= Y_MAX_ABS

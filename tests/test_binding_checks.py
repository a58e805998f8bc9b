"""The Python binding rejects tensors that do not match the shapes the C ABI
assumes, before it calls into the library (CPU only: the stand-in tensors below
claim a GPU device but are never passed to the library)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
S = pytest.importorskip("bit_diffusion_model_svdq_amd")


class OnGpu:
    """A host tensor that reports a GPU device: enough for the binding's checks."""

    def __init__(self, t, device="cuda:0"):
        self._t = t
        self.device = torch.device(device)

    def __getattr__(self, k):
        return getattr(self._t, k)

    def t(self):
        return OnGpu(self._t.t(), str(self.device))


def g(shape, dtype, device="cuda:0"):
    return OnGpu(torch.zeros(shape, dtype=dtype), device)


M, K, N, r = 32, 256, 64, 16


def layer(**over):
    d = dict(X=g((M, K), torch.int16), s=g((K,), torch.float32), L1=g((r, K), torch.int16),
             L2=g((N, r), torch.int16), Wq=g((N, K // 2), torch.uint8), ws=g((N, K // 64), torch.float32),
             b=g((N,), torch.int16), Y=g((M, N), torch.int16), work=g((1 << 20,), torch.uint8))
    d.update(over)
    return d


def fwd(d):
    S.svdq_linear_forward(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], d["Y"], d["work"])


@pytest.mark.parametrize("key,bad,msg", [
    ("Y", g((M, N - 16), torch.int16), "Y must have shape"),
    ("Y", g((M, N), torch.float32), "Y must have dtype"),
    ("ws", g((N, K // 32), torch.float32), "w_scales must have shape"),
    ("Wq", g((N, K), torch.uint8), "Wq must have shape"),
    ("L2", g((r, N), torch.int16), "L2 must have shape"),
    ("L1", g((K, r), torch.int16), "L1 must have shape"),
    ("s", g((K,), torch.float64), "smooth must have dtype"),
    ("b", g((N + 16,), torch.int16), "bias must have shape"),
    ("X", g((M, K), torch.int16, "cpu"), "must live on the GPU"),
    ("Y", g((M, N), torch.int16, "cuda:1"), "different devices"),
])
def test_forward_rejects_mismatched_tensors(key, bad, msg):
    with pytest.raises(ValueError, match=msg):
        fwd(layer(**{key: bad}))


def test_forward_rejects_a_transposed_view():
    d = layer(X=OnGpu(torch.zeros((K, M), dtype=torch.int16)).t())
    with pytest.raises(ValueError, match="X must be contiguous"):
        fwd(d)


def test_forward_rejects_half_a_low_rank_branch():
    with pytest.raises(ValueError, match="L1 and L2"):
        fwd(layer(L2=None))


def test_gemm_and_quantize_entry_points_check_their_tensors():
    d = layer()
    with pytest.raises(ValueError, match="w_scales must have shape"):
        S.svdq_forward_gemm(M, K, d["L2"], d["Wq"], g((N, 1), torch.float32), d["b"], d["Y"], d["work"], r)
    with pytest.raises(ValueError, match="Y must have shape"):
        S.svdq_forward_gemm_act(M, K, d["L2"], d["Wq"], d["ws"], d["b"], 0, g((M + 1, N), torch.int16),
                                d["work"], r)
    with pytest.raises(ValueError, match="smooth must have shape"):
        S.svdq_forward_quantize(d["X"], g((K + 64,), torch.float32), d["L1"], d["work"])
    with pytest.raises(ValueError, match="sx must have shape"):
        S.svdq_quantize_activations(d["X"], d["s"], d["L1"], g((M, K // 2), torch.uint8),
                                    g((M, K // 32), torch.float32), g((M, r), torch.float32))
    with pytest.raises(ValueError, match="T must have shape"):
        S.svdq_quantize_activations(d["X"], d["s"], d["L1"], g((M, K // 2), torch.uint8),
                                    g((M, K // 64), torch.float32), g((M, r + 16), torch.float32))
    with pytest.raises(ValueError, match="P must have shape"):
        S.svdq_debug_group_partials(g((M, K // 2), torch.uint8), d["Wq"], 0, 8, 0, 16,
                                    g((8, 16, K // 32), torch.int32))
    with pytest.raises(ValueError, match="outside"):
        S.svdq_debug_group_partials(g((M, K // 2), torch.uint8), d["Wq"], 0, M + 1, 0, 16,
                                    g((M + 1, 16, K // 64), torch.int32))


def test_mxfp4_entry_points_check_the_k_tiled_scales():
    Kx = 384                                      # 3 blocks of 128: k-tiled bytes exceed row-major ones
    d = dict(X=g((M, Kx), torch.int16), s=g((Kx,), torch.float32), L1=g((r, Kx), torch.int16),
             L2=g((N, r), torch.int16), Wq=g((N, Kx // 2), torch.uint8), b=g((N,), torch.int16),
             Y=g((M, N), torch.int16), work=g((1 << 20,), torch.uint8))
    wrong = g((N, Kx // 32), torch.uint8)         # row-major scales
    tiled = S.svdq_mxfp4_tiled_scale_bytes(N, Kx)
    assert wrong.numel() != tiled
    with pytest.raises(ValueError, match="w_e8m0 must hold"):
        S.svdq_linear_forward_mxfp4(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], wrong, d["b"], d["Y"], d["work"])
    with pytest.raises(ValueError, match="sx_e8m0 must have shape"):
        S.svdq_quantize_activations_mxfp4(d["X"], d["s"], d["L1"], g((M, Kx // 2), torch.uint8),
                                          g((M, Kx // 64), torch.uint8), g((M, r), torch.float32))


@pytest.mark.parametrize("key,bad,msg", [
    ("qx", g((M, K), torch.uint8), "qx must have shape"),
    ("sx", g((M, K // 32), torch.float32), "sx must have shape"),
    ("sx", g((M, K // 64), torch.float64), "sx must have dtype"),
    ("Y", g((M, N - 16), torch.int16), "Y must have shape"),
    ("qx", g((M, K // 2), torch.uint8, "cuda:1"), "different devices"),
])
def test_fused_debug_entry_rejects_mismatched_tensors(key, bad, msg):
    d = layer(qx=g((M, K // 2), torch.uint8), sx=g((M, K // 64), torch.float32))
    d[key] = bad
    with pytest.raises(ValueError, match=msg):
        S.svdq_debug_fused_forward(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"],
                                   S.SVDQ_ACT_NONE, d["Y"], d["qx"], d["sx"])


def mx_layer(**over):
    d = layer(Wq=g((N, K // 2), torch.uint8), ws=g((S.svdq_mxfp4_tiled_scale_bytes(N, K),), torch.uint8),
              qx=g((M, K // 2), torch.uint8), sx=g((M, K // 32), torch.uint8))
    d.update(over)
    return d


@pytest.mark.parametrize("key,bad,msg", [
    ("qx", g((M, K // 4), torch.uint8), "qx must have shape"),
    ("sx", g((M, K // 64), torch.uint8), "sx_e8m0 must have shape"),
    ("sx", g((M, K // 32), torch.float32), "sx_e8m0 must have dtype"),
    ("ws", g((N, K // 64), torch.uint8), "w_e8m0 must hold"),
    ("sx", g((M, K // 32), torch.uint8, "cuda:1"), "different devices"),
])
def test_fused_mx_debug_entry_rejects_mismatched_tensors(key, bad, msg):
    d = mx_layer()
    d[key] = bad
    with pytest.raises(ValueError, match=msg):
        S.svdq_debug_fused_forward_mxfp4(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"],
                                         S.SVDQ_ACT_NONE, d["Y"], d["qx"], d["sx"])

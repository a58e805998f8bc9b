"""Run-to-run determinism of the forward, through the C ABI.

Every kernel of the forward is deterministic by construction: no atomics, and
every reduction (the K loop, the K-split shares in the fixup, the waves'
partial T, the slices of T) sums in a fixed order.  So the same inputs must give
the same output bit for bit on every launch, whatever ran before and however
the launch interleaves with other work.  A difference would mean a race: a read
of memory that another wave or launch writes without ordering.  The shapes
cover every tile class of both GEMMs (the DiT projection's 256 x 192 tiles, the
two-per-CU 128 x 192 tiles of the 4608-token layers, the K-split with its
fixup, the small tiles) and both fused kernels; inputs are seeded random codes
and scales (only determinism is checked here), workspaces are left
uninitialized, and launches of other layers run between the repeats.
"""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("bit_diffusion_model_svdq_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
REPEATS = 8

# (label, M, K, N, r): tile classes of both GEMMs and the fused kernels
SHAPES = [
    ("dit_proj", 4096, 3072, 3072, 32),        # 256 x 192 tiles, one wave
    ("dit_out_r48", 4608, 3072, 3072, 48),     # 128 x 192 tiles two per CU; two rank chunks
    ("mlp_up", 4608, 3072, 12288, 32),         # 128 x 192 tiles two per CU
    ("mlp_down", 4608, 12288, 3072, 32),       # remainder split along K, fixup pass
    ("smallk_1280", 1024, 1280, 1280, 32),     # small tiles (two kernels)
    ("smallk_640", 4096, 640, 640, 32),        # small tiles (int4) / fused (MXFP4)
    ("fused_1024x640", 1024, 640, 640, 32),    # fused (both formats)
]


def layer(M, K, N, r, mx, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    bf = lambda *shape, scale=1.0: (torch.randn(*shape, generator=g, device=DEV) * scale).to(
        torch.bfloat16).view(torch.int16)
    d = dict(X=bf(M, K), s=torch.rand(K, generator=g, device=DEV) + 0.5,
             L1=bf(r, K, scale=0.05), L2=bf(N, r, scale=0.05),
             Wq=torch.randint(0, 256, (N, K // 2), generator=g, device=DEV, dtype=torch.uint8),
             b=bf(N, scale=0.3), Y=torch.empty((M, N), dtype=torch.int16, device=DEV))
    if mx:
        d["ws"] = torch.randint(118, 126, (S.svdq_mxfp4_tiled_scale_bytes(N, K),), generator=g, device=DEV,
                                dtype=torch.uint8)
        nbytes = S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r)
    else:
        d["ws"] = torch.rand((N, K // 64), generator=g, device=DEV) * 0.02 + 0.001
        nbytes = S.svdq_forward_workspace_bytes(M, K, N, r)
    d["work"] = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    return d


def forward(d, mx):
    f = S.svdq_linear_forward_mxfp4 if mx else S.svdq_linear_forward
    f(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], d["Y"], d["work"])


@pytest.mark.parametrize("mx", [False, True], ids=["int4", "mxfp4"])
@pytest.mark.parametrize("label,M,K,N,r", SHAPES, ids=[s[0] for s in SHAPES])
def test_forward_is_bit_identical_across_launches(label, M, K, N, r, mx):
    print(f"determinism {label} {'mxfp4' if mx else 'int4'}", flush=True)
    d = layer(M, K, N, r, mx, seed=M + K + N + r)
    other = layer(512, 1024, 1024, 16, not mx, seed=7)     # interleaved work of the other format
    forward(d, mx)
    torch.cuda.synchronize()
    Y0 = d["Y"].clone()
    for rep in range(REPEATS):
        d["Y"].fill_(0x7FC0)                                  # a NaN pattern: every element rewritten
        d["work"].fill_(rep * 37 % 251)                       # stale workspace contents change too
        for _ in range(rep % 3):
            forward(other, not mx)
        forward(d, mx)
        torch.cuda.synchronize()
        assert torch.equal(d["Y"], Y0), f"{label}: launch {rep + 1} differs from the first"

"""Seeded synthetic workloads for the SVDQuant W4A4 linear layer.

This module only draws inputs.  It holds none of the method's arithmetic
(no smoothing, no SVD, no quantization): both the CPU oracle and the HIP
path receive the same arrays from here, and nothing here depends on either.

Shapes and distributions follow the workloads the SVDQuant pages motivate:
diffusion-transformer activations with a few outlier channels (the
"SVDQuant Low-Rank Residual Quantization Algorithm Terminology Entry",
section 2, describes outlier channels in diffusion-model activations) and
weights with a low-rank spike over Gaussian noise (section 2.2 of the same
entry: outliers migrated into the weights show low-rank structure).

Every tensor is drawn with numpy's PCG64 from its own seed,
``20241107 + 100 * workload.seed_index + tensor_id``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BASE_SEED = 20241107

# tensor ids (added to the workload's seed base)
_TID_X = 1
_TID_XCAL = 2
_TID_WNOISE = 3
_TID_U = 4
_TID_V = 5
_TID_BIAS = 6
_TID_OUTLIER = 7
_TID_LORA_A = 8
_TID_LORA_B = 9


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed_index: int          # seed base = BASE_SEED + 100 * seed_index
    M: int                   # tokens
    K: int                   # in-features
    N: int                   # out-features
    rank: int                # low-rank branch rank r
    n_outliers: int          # outlier input channels
    outlier_lo: float        # outlier factor range; lo == hi means a fixed factor
    outlier_hi: float
    spike: tuple             # singular values of the weight's low-rank spike
    calib_rows: int          # rows of the separate calibration draw
    act: str = "gauss"       # "gauss": N(0,1); "gelu": GELU_tanh(N(0, 1.5^2))
    alpha: float = 0.5
    bias_std: float = 0.1


def _lin(a, b, n):
    return tuple(float(v) for v in np.linspace(a, b, n))


WORKLOADS = {
    # M=256, K=N=1024, r=16; 1% outlier channels x50; rank-8 spike 5..1.
    "tiny": Workload("tiny", 0, 256, 1024, 1024, 16, 10, 50.0, 50.0, _lin(5, 1, 8), 256),
    # DiT attention projection: M=4096, K=N=3072, r=32; 0.5% outliers x30..x100
    # log-uniform; rank-16 spike (5..1 by analogy with the tiny case).
    "dit_proj": Workload("dit_proj", 1, 4096, 3072, 3072, 32, 15, 30.0, 100.0, _lin(5, 1, 16), 1024),
    # DiT MLP pair (the two linears on their own).
    "mlp_up": Workload("mlp_up", 2, 4608, 3072, 12288, 32, 15, 30.0, 100.0, _lin(5, 1, 16), 1024),
    "mlp_down": Workload("mlp_down", 2, 4608, 12288, 3072, 32, 61, 30.0, 100.0, _lin(5, 1, 16), 1024,
                         act="gelu"),
    # DiT block at width 3072, 4608 tokens: fused QKV projection and the
    # attention output projection (the MLP pair above completes the block).
    "dit_qkv": Workload("dit_qkv", 4, 4608, 3072, 9216, 32, 15, 30.0, 100.0, _lin(5, 1, 16), 1024),
    "dit_out": Workload("dit_out", 4, 4608, 3072, 3072, 32, 15, 30.0, 100.0, _lin(5, 1, 16), 1024),
    # Small-K, memory-bound UNet widths.
    "smallk_640": Workload("smallk_640", 3, 4096, 640, 640, 32, 3, 30.0, 100.0, _lin(5, 1, 16), 1024),
    "smallk_1280": Workload("smallk_1280", 3, 1024, 1280, 1280, 32, 6, 30.0, 100.0, _lin(5, 1, 16), 1024),
}

# distinct seed offsets for workloads that share a seed_index
_SUB = {"mlp_down": 50, "smallk_1280": 50, "dit_out": 50}


def _rng(w: Workload, tid: int) -> np.random.Generator:
    seed = BASE_SEED + 100 * w.seed_index + _SUB.get(w.name, 0) + tid
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _gelu_tanh(z: np.ndarray) -> np.ndarray:
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * z * (1.0 + np.tanh(c * (z + 0.044715 * z ** 3)))


def outlier_channels(w: Workload):
    """Outlier channel indices and their factors (shared by X and the calibration draw)."""
    g = _rng(w, _TID_OUTLIER)
    ch = np.sort(g.choice(w.K, size=w.n_outliers, replace=False))
    if w.outlier_lo == w.outlier_hi:
        f = np.full(w.n_outliers, w.outlier_lo, dtype=np.float64)
    else:
        f = np.exp(g.uniform(math.log(w.outlier_lo), math.log(w.outlier_hi), size=w.n_outliers))
    return ch, f


def _activations(w: Workload, rows: int, tid: int, row0: int = 0, nrows: int | None = None) -> np.ndarray:
    g = _rng(w, tid)
    if w.act == "gauss":
        x = g.standard_normal((rows, w.K), dtype=np.float32)
    else:
        x = _gelu_tanh(1.5 * g.standard_normal((rows, w.K), dtype=np.float32)).astype(np.float32)
    ch, f = outlier_channels(w)
    x[:, ch] *= f.astype(np.float32)[None, :]
    if nrows is not None:
        x = x[row0:row0 + nrows]
    return f32_to_bf16_bits(x)


def activations(w: Workload, M: int | None = None) -> np.ndarray:
    """X as bf16 bit patterns, uint16 [M, K] (M defaults to the workload's)."""
    return _activations(w, w.M if M is None else M, _TID_X)


def calibration_activations(w: Workload) -> np.ndarray:
    """Separate calibration draw, bf16 bits [calib_rows, K], same outlier channels and factors."""
    return _activations(w, w.calib_rows, _TID_XCAL)


def weight(w: Workload) -> np.ndarray:
    """W float32 [N, K] = N(0, 0.02) + U diag(spike) V^T with U, V orthonormal."""
    noise = _rng(w, _TID_WNOISE).standard_normal((w.N, w.K)) * 0.02
    k = len(w.spike)
    U, _ = np.linalg.qr(_rng(w, _TID_U).standard_normal((w.N, k)))
    V, _ = np.linalg.qr(_rng(w, _TID_V).standard_normal((w.K, k)))
    spike = (U * np.asarray(w.spike)[None, :]) @ V.T
    return (noise + spike).astype(np.float32)


def bias(w: Workload) -> np.ndarray:
    """bias as bf16 bits [N], N(0, bias_std)."""
    return f32_to_bf16_bits((_rng(w, _TID_BIAS).standard_normal(w.N) * w.bias_std).astype(np.float32))


def lora_factors(w: Workload, rank: int = 16, std: float = 0.01):
    """A seeded off-the-shelf LoRA for the layer: A [K, rank] (down) and
    B [rank, N] (up), float32 N(0, std^2); it adds X A B to the output."""
    A = (_rng(w, _TID_LORA_A).standard_normal((w.K, rank)) * std).astype(np.float32)
    B = (_rng(w, _TID_LORA_B).standard_normal((rank, w.N)) * std).astype(np.float32)
    return A, B


def rng_for(name: str, tid: int) -> np.random.Generator:
    """Extra seeded stream for test-only draws (tid >= 100 to stay clear of the tensors above)."""
    return _rng(WORKLOADS[name], 100 + tid)

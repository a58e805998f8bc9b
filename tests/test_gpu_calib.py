"""GPU calibration statistic (A_scale of E2, Terminology Entry section 2.3): the
device abs-max is bit-exact against the oracle on every workload's calibration
draw, on an edge set, across calls, and on ragged K (the per-channel load path)."""
import sys

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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def gpu_absmax(X, start=None):
    K = X.shape[1]
    amax = torch.zeros(K, dtype=torch.float32, device=DEV) if start is None else \
        torch.from_numpy(np.ascontiguousarray(start, np.float32)).to(DEV)
    S.svdq_act_absmax_update_device(dev16(X), amax)
    torch.cuda.synchronize()
    return amax.cpu().numpy()


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_absmax_bit_exact_on_calibration_draw(name):
    say(f"absmax {name}")
    w = synth.WORKLOADS[name]
    Xc = synth.calibration_activations(w)
    got = gpu_absmax(Xc)
    np.testing.assert_array_equal(got.view(np.uint32), O.act_absmax(Xc).view(np.uint32))


def _edge_rows(K, seed=5):
    g = np.random.default_rng(seed)
    vals = np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -133, -(2.0 ** -133), 2.0 ** -126, -3.0e38, 3.0e38,
                     np.inf, -np.inf, 1e-40, -7.5], np.float32)
    rows = g.choice(vals, size=(37, K))
    rows[:, 0] = -0.0                       # a channel that only ever sees negative zero
    rows[:, 1] = -(2.0 ** -133)             # only negative subnormals
    rows[3, 2] = -np.inf                    # one infinity among finite values
    return synth.f32_to_bf16_bits(rows)


@pytest.mark.parametrize("K", [1024, 200, 7, 513])
def test_absmax_edge_values_and_ragged_k(K):
    say(f"absmax edges K={K}")
    X = _edge_rows(K)
    got = gpu_absmax(X)
    want = O.act_absmax(X)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    assert got[0] == 0.0 and not np.signbit(got[0])
    assert got[1] == np.float32(2.0 ** -133)


def test_absmax_is_a_running_max_across_calls():
    w = synth.WORKLOADS["dit_proj"]
    Xc = synth.calibration_activations(w)
    a, b = Xc[:300], Xc[300:]
    first = gpu_absmax(a)
    both = gpu_absmax(b, start=first)
    np.testing.assert_array_equal(both.view(np.uint32), O.act_absmax(Xc).view(np.uint32))
    # and it agrees with the host function element for element
    host = np.zeros(Xc.shape[1], np.float32)
    S.svdq_act_absmax_update(Xc, host)
    np.testing.assert_array_equal(both.view(np.uint32), host.view(np.uint32))


def test_absmax_many_rows_single_channel_band():
    """Tall input: 70000 rows over 64 channels takes the wide row bands."""
    g = np.random.default_rng(11)
    X = synth.f32_to_bf16_bits((g.standard_normal((70000, 64)) * 3).astype(np.float32))
    got = gpu_absmax(X)
    np.testing.assert_array_equal(got.view(np.uint32), O.act_absmax(X).view(np.uint32))


def test_absmax_empty_batch_changes_nothing():
    start = np.arange(16, dtype=np.float32)
    amax = torch.from_numpy(start.copy()).to(DEV)
    S.svdq_act_absmax_update_device(torch.zeros((0, 16), dtype=torch.int16, device=DEV), amax)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(amax.cpu().numpy(), start)

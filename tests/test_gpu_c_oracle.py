"""GPU parity of the HIP path against the plain C oracle (oracle/svdq_ref.c), through the C ABI.

The other GPU tests compare against the numpy oracle; these compare the same
launches with the C one, the second independent implementation: codes and
scales and the int32 group partials bit-exact, Y within the output tolerance
(relative Frobenius error <= 5e-3, max |error| <= 1e-2 max |Y_ref|).  The layer's
s, L1 and L2 come from the library's packer, and Q(R) from the C oracle (checked
equal to the library's on the host first).
"""
import sys

import numpy as np
import pytest

import synth
from oracle import svdq_ref as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("bit_diffusion_model_svdq_amd")

F32, F64 = np.float32, np.float64
Y_REL_FRO = 5e-3
Y_MAX_ABS = 1e-2

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


def layer(name, mx=False):
    w = synth.WORKLOADS[name]
    X, W, b = synth.activations(w), synth.weight(w), synth.bias(w)
    A = np.zeros(w.K, F32)
    S.svdq_act_absmax_update(synth.calibration_activations(w), A)
    pk = S.svdq_pack_weights(W, A, w.alpha, w.rank)
    s, L1, L2 = pk["smooth"], pk["L1"], pk["L2"]
    if mx:
        Wq, we = C.quantize_residual_mx(W, s, L1, L2)
        Wl, wl = S.svdq_quantize_residual_mxfp4(W, s, L1, L2)
    else:
        Wq, we = C.quantize_residual(W, s, L1, L2)
        Wl, wl = pk["Wq"], pk["w_scales"]
    np.testing.assert_array_equal(Wq, Wl)
    np.testing.assert_array_equal(np.asarray(we).view(np.uint8), np.asarray(wl).view(np.uint8))
    return dict(X=X, b=b, s=s, L1=L1, L2=L2, Wq=Wq, we=we, M=w.M, K=w.K, N=w.N, r=w.rank)


def run_forward(p, mx=False):
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    Y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    if mx:
        ws = torch.empty(S.svdq_forward_workspace_bytes_mxfp4(M, K, N, r), dtype=torch.uint8, device=DEV)
        S.svdq_linear_forward_mxfp4(dev(p["X"]), dev(p["s"]), dev(p["L1"]), dev(p["L2"]), dev(p["Wq"]),
                                    dev(S.svdq_mxfp4_tile_scales(p["we"])), dev(p["b"]), Y, ws)
    else:
        ws = torch.empty(S.svdq_forward_workspace_bytes(M, K, N, r), dtype=torch.uint8, device=DEV)
        S.svdq_linear_forward(dev(p["X"]), dev(p["s"]), dev(p["L1"]), dev(p["L2"]), dev(p["Wq"]),
                              dev(p["we"]), dev(p["b"]), Y, ws)
    torch.cuda.synchronize()
    return C.bf16_to_f64(Y.cpu().numpy().view(np.uint16))


def check_y(Yg, Yref, label):
    rf, ma = C.rel_fro(Yg, Yref), C.max_abs_ratio(Yg, Yref)
    say(f"{label}: rel_fro {rf:.3e} max_abs/max {ma:.3e}")
    assert rf <= Y_REL_FRO and ma <= Y_MAX_ABS


def test_tiny_codes_partials_and_output_against_the_c_oracle():
    """256 x 1024 -> 1024, r = 16: k1's codes and scales, the full P of k2's main
    loop, and every output of the forward."""
    say("c oracle: tiny int4")
    p = layer("tiny")
    M, K, N, r = p["M"], p["K"], p["N"], p["r"]
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    sx = torch.empty((M, K // 64), dtype=torch.float32, device=DEV)
    T = torch.empty((M, r), dtype=torch.float32, device=DEV)
    S.svdq_quantize_activations(dev(p["X"]), dev(p["s"]), dev(p["L1"]), qx, sx, T)
    P = torch.empty((M, N, K // 64), dtype=torch.int32, device=DEV)
    S.svdq_debug_group_partials(qx, dev(p["Wq"]), 0, M, 0, N, P)
    torch.cuda.synchronize()
    qc, sc, Tc, _ = C.quantize_activations(p["X"], p["s"], p["L1"])
    np.testing.assert_array_equal(qx.cpu().numpy(), qc)
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), sc.view(np.uint32))
    assert C.rel_fro(T.cpu().numpy(), Tc) <= 1e-4
    np.testing.assert_array_equal(P.cpu().numpy(), C.group_partials(qc, p["Wq"]))
    check_y(run_forward(p), C.forward(p["X"], p["s"], p["L1"], p["L2"], p["Wq"], p["we"], p["b"]),
            "tiny int4")


@pytest.mark.parametrize("name,rows", [("dit_proj", 96), ("smallk_640", 256)])
def test_forward_rows_against_the_c_oracle(name, rows):
    """The forward over the whole layer, in the launch plan the bench times; Y checked
    on evenly spaced rows (the first and the last included) against the C oracle."""
    say(f"c oracle: {name} int4, {rows} rows")
    p = layer(name)
    Yg = run_forward(p)
    idx = np.unique(np.linspace(0, p["M"] - 1, rows).astype(int))
    Yref = np.concatenate([C.forward(p["X"], p["s"], p["L1"], p["L2"], p["Wq"], p["we"], p["b"],
                                     rows=(int(m), int(m) + 1)) for m in idx])
    check_y(Yg[idx], Yref, name)


@pytest.mark.parametrize("name,rows", [("tiny", 256), ("smallk_640", 128)])
def test_mxfp4_forward_against_the_c_oracle(name, rows):
    """The MXFP4 forward (the fused kernel at 4096 x 640, the two kernels at 256 x 1024)
    against the C oracle's MXFP4 forward."""
    say(f"c oracle: {name} mxfp4, {rows} rows")
    p = layer(name, mx=True)
    Yg = run_forward(p, mx=True)
    idx = np.unique(np.linspace(0, p["M"] - 1, rows).astype(int))
    Yref = np.concatenate([C.forward_mx(p["X"], p["s"], p["L1"], p["L2"], p["Wq"], p["we"], p["b"],
                                        rows=(int(m), int(m) + 1)) for m in idx])
    check_y(Yg[idx], Yref, f"{name} mxfp4")

"""The allocation-free forward against the workspace forward, through the C ABI.

svdq_linear_forward_noalloc runs the same kernels as svdq_linear_forward_act
with the library's static device workspace in place of a caller's, so its
output must be bit-identical; two calls in a row, the second on a smaller
input (the array keeps the first call's contents), and both within the
oracle's tolerance on sampled rows.
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


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def layer(name, M=None):
    w = synth.WORKLOADS[name]
    X = synth.activations(w)[:M or w.M]
    pk = O.pack_weights(synth.weight(w), O.act_absmax(synth.calibration_activations(w)), w.alpha, rank=w.rank)
    return dict(X=X, b=synth.bias(w), s=pk["s"], L1=pk["L1"], L2=pk["L2"], Wq=pk["Wq"], ws=pk["w_scales"])


def both(p, act):
    M, K = p["X"].shape
    N, r = p["Wq"].shape[0], p["L1"].shape[0]
    d = {k: dev(v) for k, v in p.items()}
    Y_ws = torch.full((M, N), 0x7FC0, dtype=torch.int16, device=DEV)
    ws = torch.empty(S.svdq_forward_workspace_bytes(M, K, N, r), dtype=torch.uint8, device=DEV)
    S.svdq_linear_forward_act(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], act, Y_ws, ws)
    Y_na = torch.full((M, N), 0x7FC0, dtype=torch.int16, device=DEV)
    S.svdq_linear_forward_noalloc(d["X"], d["s"], d["L1"], d["L2"], d["Wq"], d["ws"], d["b"], act, Y_na)
    torch.cuda.synchronize()
    return Y_ws.cpu().numpy().view(np.uint16), Y_na.cpu().numpy().view(np.uint16)


def test_noalloc_forward_matches_workspace_forward_on_two_calls():
    assert S.svdq_static_workspace_bytes() == 64 << 20
    big = layer("dit_proj")                       # 4096 x 3072 -> 3072, r = 32: 8.1 MB of workspace
    # then the same layer on its first 1024 tokens with GELU: a smaller workspace in the
    # same array (still the two-kernel forward, which uses it; small layers fuse and do not)
    small = dict(big, X=big["X"][:1024])
    M2, K2 = small["X"].shape
    assert not S.svdq_forward_fused(M2, K2, small["Wq"].shape[0], small["L1"].shape[0])
    for p, act, tag in ((big, S.SVDQ_ACT_NONE, "dit_proj"), (small, S.SVDQ_ACT_GELU_TANH, "dit_proj 1024 rows")):
        print(f"noalloc {tag}", flush=True)
        Yws, Yna = both(p, act)
        np.testing.assert_array_equal(Yna, Yws, err_msg=tag)
        M = p["X"].shape[0]
        rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(M - 8, M)]))
        Yref = O.forward(p["X"][rows], p["s"], p["L1"], p["L2"], p["Wq"], p["ws"], p["b"],
                         activation="gelu_tanh" if act == S.SVDQ_ACT_GELU_TANH else None)
        Yg = O.bf16_to_f64(Yna[rows])
        assert O.rel_fro(Yg, Yref) <= 5e-3 and O.max_abs_ratio(Yg, Yref) <= 1e-2

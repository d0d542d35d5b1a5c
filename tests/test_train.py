"""GPU checks of the training path: moe_forward keeping the expert pre-activations
(moe_opts.activations) and moe_backward reading them instead of recomputing them.

Both routes of moe_backward must give the same gradients bit for bit (the kept a, b come from the
same tiled product the backward pass would run), and the forward that keeps them must give the
same layer output: bit for bit where the regular forward uses the tiled product as well (large
groups), and to the bf16 bar of the layer against the oracle everywhere (small groups use the
streaming product, whose sums run in another order).
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from helpers import dev, gaps, host, rel_err, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2
TIE = 1e-4  # the routing bar: tokens with a closer K-th/(K+1)-th logit pair are compared under the GPU's selection


@pytest.fixture(scope="module")
def M():
    import sparse_mixture_experts_33_amd as moe
    moe.lib()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return moe


CASES = {
    # large groups: the regular forward runs the tiled product too
    "tiled_e4": dict(w=mi.Workload("train_tiled_e4", T=700, d=256, F=512, E=4, K=2, dtype="bf16", seed=811),
                     tiled=True, packed=False),
    "tiled_packed": dict(w=mi.Workload("train_tiled_pk", T=1100, d=256, F=256, E=4, K=2, dtype="bf16", seed=812),
                         tiled=True, packed=True),
    # small groups: the regular forward streams the weights
    "stream_e8": dict(w=mi.Workload("train_stream_e8", T=200, d=256, F=512, dtype="bf16", seed=813),
                      tiled=False, packed=False),
    # more experts, four kept, and a router bias (the routing both calls recompute must agree)
    "e16_k4_bias": dict(w=mi.Workload("train_e16_k4", T=600, d=256, F=256, E=16, K=4, dtype="bf16", seed=814),
                        tiled=False, packed=False, bias=True),
}


def run(M, w, W, x, packed, keep, bias=None):
    """moe_forward (optionally keeping the activations), then moe_backward with or without them."""
    layout = M.MOE_LAYOUT_PACKED if packed else M.MOE_LAYOUT_ROWMAJOR
    dm = M.Dims(w.T, w.d, w.F, w.E, w.K, M.MOE_BF16, layout)
    dW = {k: dev(W[k]) for k in ("w_gate", "w1", "w3", "w2")}
    fw = dict(dW)
    if packed:
        for k, which in (("w1", M.MOE_W_UP), ("w3", M.MOE_W_UP), ("w2", M.MOE_W_DOWN)):
            out = torch.empty_like(dW[k])
            M.moe_pack_weights(dm, which, dW[k], out)
            fw[k] = out
    xd = dev(x)
    act = torch.full((2 * w.T * w.K * w.F,), float("nan"), dtype=torch.float32, device="cuda") if keep else None
    y = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(M.moe_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    b = None if bias is None else dev(bias)
    M.moe_forward(dm, xd, fw["w_gate"], fw["w1"], fw["w3"], fw["w2"], y, ws, gate_bias=b, activations=act)
    # the backward pass takes the same weights (packed ones give the gradients in packed order)
    bws = torch.empty(M.moe_backward_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    g = {"dx": torch.empty((w.T, w.d), **f32), "dw_gate": torch.empty((w.d, w.E), **f32),
         "dw1": torch.empty((w.E, w.F, w.d), **f32), "dw3": torch.empty((w.E, w.F, w.d), **f32),
         "dw2": torch.empty((w.E, w.d, w.F), **f32), "dlogits": torch.empty((w.T, w.E), **f32)}
    dy = dev(mi.upstream_grad(w))
    M.moe_backward(dm, xd, fw["w_gate"], fw["w1"], fw["w3"], fw["w2"], dy, g["dx"], g["dw_gate"], g["dw1"],
                   g["dw3"], g["dw2"], bws, dlogits=g["dlogits"], gate_bias=b, activations=act)
    torch.cuda.synchronize()
    out = {k: host(v) for k, v in g.items()}
    out["y"] = host(y)
    if keep:
        out["act"] = host(act)
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_kept_activations(M, name):
    c = CASES[name]
    w = c["w"]
    say(f"[train] {name} T={w.T} d={w.d} F={w.F} E={w.E} K={w.K} packed={c['packed']}")
    W = mi.layer_weights(w)
    x = mi.tokens(w)
    bias = (0.5 * np.random.default_rng(w.seed).standard_normal(w.E)).astype(np.float32) if c.get("bias") else None
    kept = run(M, w, W, x, c["packed"], keep=True, bias=bias)
    plain = run(M, w, W, x, c["packed"], keep=False, bias=bias)
    # every routed row's a and b were written (the buffer started as NaN)
    assert np.isfinite(kept["act"]).all()
    for k in ("dx", "dw_gate", "dw1", "dw3", "dw2", "dlogits"):
        assert np.array_equal(kept[k], plain[k]), k
    if c["tiled"]:
        assert np.array_equal(kept["y"], plain["y"])
    r = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], w.K, bias=bias)
    keep = gaps(r["logits"], w.K)[0] > TIE
    assert keep.mean() > 0.99
    err = rel_err(kept["y"][keep], r["y"][keep])
    say(f"  y max|d|/max|ref| = {err:.3e}; gradients bit-identical with and without the kept activations")
    assert err <= TOL
    # near-ties: the output under the GPU's own selection (moe_route makes moe_forward's selection)
    und = np.flatnonzero(~keep).astype(np.int64)
    if len(und):
        dm = M.Dims(w.T, w.d, w.F, w.E, w.K, M.MOE_BF16)
        gi = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
        gw = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")
        M.moe_route(dm, dev(x), dev(W["w_gate"]), gi, gw, gate_bias=None if bias is None else dev(bias))
        torch.cuda.synchronize()
        gi = host(gi)
        ru = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], w.K, bias=bias, tokens=und, select=gi[und])
        e2 = rel_err(kept["y"][und], ru["y"])
        say(f"  {len(und)} near-tie tokens under the GPU's selection: max|d|/max|ref| = {e2:.3e}")
        assert e2 <= TOL

"""GPU parity of moe_backward against the oracle's backward (fp64) on the same seeded inputs.

Bars (bf16 operands, fp32 sums): for every gradient, max|d| / max|ref| <= 2e-2, the bf16 output bar
of the forward. Expected errors are ~1e-3 (bf16 rounding of dy, h, da, db averages down over the
d or F terms of each sum). Inputs are chosen so that no token has a near-tie between its K-th and
(K+1)-th logits (the selection, which the gradient holds fixed, is then the same on both sides);
this is asserted. Weight gradients of an expert with no tokens must be exactly zero.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from helpers import dev, gaps, host, rel_err, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TIE = 1e-4
TOL = 2e-2


@pytest.fixture(scope="module")
def M():
    import sparse_mixture_experts_33_amd as moe
    moe.lib()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return moe


CASES = {
    # small groups (about 75 rows per expert): every product runs on the LDS-tiled kernels, whose
    # token blocks past a group's end cost no MFMAs, so mostly partly filled tiles
    "stream_e8": dict(w=mi.Workload("bwd_stream_e8", T=300, d=256, F=512, dtype="bf16", seed=801), bias=None),
    # large groups: several full tiles per expert
    "tiled_e4": dict(w=mi.Workload("bwd_tiled_e4", T=700, d=256, F=512, E=4, K=2, dtype="bf16", seed=802), bias=None),
    "e16_k4_bias": dict(w=mi.Workload("bwd_e16_k4", T=130, d=256, F=256, E=16, K=4, dtype="bf16", seed=803),
                        bias="rand"),
    # expert 5 gets no token: its three weight gradients must be exactly zero
    "empty_expert": dict(w=mi.Workload("bwd_empty", T=200, d=256, F=256, E=8, K=2, dtype="bf16", seed=804),
                         bias="kill5"),
    "dense_e1_k1": dict(w=mi.Workload("bwd_dense", T=64, d=256, F=256, E=1, K=1, dtype="bf16", seed=805), bias=None),
}


def make_bias(kind, E, seed):
    if kind is None:
        return None
    rng = np.random.default_rng(seed)
    b = (0.5 * rng.standard_normal(E)).astype(np.float32)
    if kind == "kill5":
        b[:] = 0.0
        b[5] = -100.0
    return b


def dy_for(w):
    return mi.upstream_grad(w)


def packed_order(a):
    """[E][N][K] -> flat, in the element order moe.h gives the packed bf16 weights (V = 8): element
    (e, n, k) at ((e (N/16) + n/16) (K/32) + k/32) 512 + (n%16 + 16 ((k/8)%4)) 8 + k%8."""
    E, N, K = a.shape
    return a.reshape(E, N // 16, 16, K // 32, 4, 8).transpose(0, 1, 3, 4, 2, 5).reshape(-1)


def gpu_backward(M, w, W, x, dy, bias, dlogits=True, packed=False):
    dm = M.Dims(w.T, w.d, w.F, w.E, w.K, M.MOE_BF16, M.MOE_LAYOUT_PACKED if packed else M.MOE_LAYOUT_ROWMAJOR)
    wd = {k: dev(W[k]) for k in ("w1", "w3", "w2")}
    if packed:
        for k, which in (("w1", M.MOE_W_UP), ("w3", M.MOE_W_UP), ("w2", M.MOE_W_DOWN)):
            out = torch.empty_like(wd[k])
            M.moe_pack_weights(dm, which, wd[k], out)
            wd[k] = out
    ws = torch.empty(M.moe_backward_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    out = {"dx": torch.empty((w.T, w.d), **f32), "dw_gate": torch.empty((w.d, w.E), **f32),
           "dw1": torch.empty((w.E, w.F, w.d), **f32), "dw3": torch.empty((w.E, w.F, w.d), **f32),
           "dw2": torch.empty((w.E, w.d, w.F), **f32),
           "dlogits": torch.empty((w.T, w.E), **f32) if dlogits else None}
    M.moe_backward(dm, dev(x), dev(W["w_gate"]), wd["w1"], wd["w3"], wd["w2"], dev(dy), out["dx"],
                   out["dw_gate"], out["dw1"], out["dw3"], out["dw2"], ws, dlogits=out["dlogits"],
                   gate_bias=None if bias is None else dev(bias))
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items() if v is not None}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_small(M, name):
    c = CASES[name]
    w = c["w"]
    say(f"[backward] {name} T={w.T} d={w.d} F={w.F} E={w.E} K={w.K}")
    W = mi.layer_weights(w)
    x = mi.tokens(w)
    bias = make_bias(c["bias"], w.E, w.seed)
    dy = dy_for(w)
    logits, idx, _ = oracle.route(x, W["w_gate"], w.K, bias=bias)
    if w.K < w.E:
        assert gaps(logits, w.K)[0].min() > TIE, "pick a seed without near-ties"
    got = gpu_backward(M, w, W, x, dy, bias)
    ref = oracle.backward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], w.K, dy.astype(np.float64), bias=bias)
    for k in ("dx", "dlogits", "dw_gate", "dw1", "dw3", "dw2"):
        err = rel_err(got[k], ref[k])
        say(f"  {k:8s} max|d|/max|ref| = {err:.3e}")
        assert err <= TOL, k
    # logits of experts not kept have exactly zero gradient
    mask = np.ones((w.T, w.E), bool)
    mask[np.arange(w.T)[:, None], idx] = False
    assert np.all(got["dlogits"][mask] == 0.0)
    if c["bias"] == "kill5":
        assert not np.any(idx == 5)
        for k in ("dw1", "dw3", "dw2"):
            assert np.all(got[k][5] == 0.0), k


@pytest.mark.parametrize("name", ["tiled_e4", "e16_k4_bias", "empty_expert"])
def test_backward_packed_weights(M, name):
    """Fragment-packed weights give the row-major pass's gradients bit for bit: dx, dlogits and dW_g
    as they are, dw1, dw3, dw2 in the packed element order of the weights (the products run the same
    sums in the same order; only the weight loads and the gradient stores are addressed differently)."""
    c = CASES[name]
    w = c["w"]
    say(f"[backward] packed weights, {name} T={w.T} d={w.d} F={w.F} E={w.E} K={w.K}")
    W = mi.layer_weights(w)
    x = mi.tokens(w)
    bias = make_bias(c["bias"], w.E, w.seed)
    dy = dy_for(w)
    rm = gpu_backward(M, w, W, x, dy, bias)
    pk = gpu_backward(M, w, W, x, dy, bias, packed=True)
    for k in ("dx", "dlogits", "dw_gate"):
        assert np.array_equal(rm[k], pk[k]), k
    for k in ("dw1", "dw3", "dw2"):
        assert pk[k].shape == rm[k].shape
        assert np.array_equal(packed_order(rm[k]), pk[k].reshape(-1)), k


def test_backward_is_deterministic(M):
    c = CASES["tiled_e4"]
    w = c["w"]
    W = mi.layer_weights(w)
    x = mi.tokens(w)
    dy = dy_for(w)
    a = gpu_backward(M, w, W, x, dy, None)
    b = gpu_backward(M, w, W, x, dy, None)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_backward_full_size_sampled(M):
    """Mixtral prefill shape (T=4096, d=4096, F=14336, E=8, K=2, bf16) on sampled outputs: dx and
    dlogits of a few tokens, single entries of every expert's three weight gradients (each a sum
    over all ~1024 rows of its group), and dW_g = x^T dlogits checked in fp64 on the GPU's dlogits."""
    w = mi.WORKLOADS["prefill_T4096"]
    say(f"[backward] full size {w.name}")
    W = mi.layer_weights(w)
    x = mi.tokens(w)
    dy = dy_for(w)
    got = gpu_backward(M, w, W, x, dy, None)
    logits, idx, _ = oracle.route(x, W["w_gate"], w.K)
    gk = gaps(logits, w.K)[0]
    rng = np.random.default_rng(7)
    toks = rng.choice(np.flatnonzero(gk > TIE), size=4, replace=False).astype(np.int64)
    dx, dl = oracle.backward_tokens(x, W["w_gate"], W["w1"], W["w3"], W["w2"], w.K, dy.astype(np.float64), toks)
    err_dx = rel_err(got["dx"][toks], dx)
    err_dl = np.abs(got["dlogits"][toks] - dl).max() / max(np.abs(dl).max(), 1e-30)
    say(f"  dx (4 tokens) {err_dx:.3e}, dlogits {err_dl:.3e}")
    assert err_dx <= TOL and err_dl <= TOL
    # weight-gradient entries: 2 per matrix per expert, (which, e, i, j)
    q = []
    for e in range(w.E):
        for which in (1, 3, 2):
            for _ in range(2):
                i = rng.integers(w.F if which != 2 else w.d)
                j = rng.integers(w.d if which != 2 else w.F)
                q.append((which, e, i, j))
    q = np.array(q)
    ref = oracle.backward_wsample(x, W["w_gate"], W["w1"], W["w3"], W["w2"], w.K, dy.astype(np.float64), q)
    name = {1: "dw1", 3: "dw3", 2: "dw2"}
    val = np.array([got[name[a]][e, i, j] for a, e, i, j in q])
    # entry-wise relative to the spread of that gradient (sampled from the GPU result)
    for a in (1, 3, 2):
        sel = q[:, 0] == a
        scale = np.abs(got[name[a]]).max()
        err = np.abs(val[sel] - ref[sel]).max() / scale
        say(f"  {name[a]} ({sel.sum()} entries) max|d|/max|dW| = {err:.3e}")
        assert err <= TOL
    # router weight gradient: x^T dlogits in fp64 from the GPU's own dlogits
    xr = mi.bf16_bits_to_f32(x).astype(np.float64)
    dwg_ref = xr.T @ got["dlogits"].astype(np.float64)
    err = rel_err(got["dw_gate"], dwg_ref)
    say(f"  dw_gate vs x^T dlogits: {err:.3e}")
    assert err <= 1e-4


def test_backward_packed_weights_full_size(M):
    """The packed-weight pass at the Mixtral prefill shape (T=4096, d=4096, F=14336, E=8, K=2) against
    the row-major pass on the same inputs, every element: dx, dlogits, dW_g equal, and dw1, dw3, dw2
    equal after the row-major gradients are put in the packed order (compared on the GPU). The
    row-major pass is pinned to the oracle by the sampled full-size test above."""
    w = mi.WORKLOADS["prefill_T4096"]
    say(f"[backward] packed weights, full size {w.name}")
    W = mi.layer_weights(w)
    x, dy = dev(mi.tokens(w)), dev(mi.upstream_grad(w))
    f32 = dict(dtype=torch.float32, device="cuda")

    def run(packed):
        dm = M.Dims(w.T, w.d, w.F, w.E, w.K, M.MOE_BF16, M.MOE_LAYOUT_PACKED if packed else M.MOE_LAYOUT_ROWMAJOR)
        wd = {k: dev(W[k]) for k in ("w1", "w3", "w2")}
        if packed:
            for k, which in (("w1", M.MOE_W_UP), ("w3", M.MOE_W_UP), ("w2", M.MOE_W_DOWN)):
                out = torch.empty_like(wd[k])
                M.moe_pack_weights(dm, which, wd[k], out)
                wd[k] = out
        ws = torch.empty(M.moe_backward_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
        g = {"dx": torch.empty((w.T, w.d), **f32), "dw_gate": torch.empty((w.d, w.E), **f32),
             "dw1": torch.empty((w.E, w.F, w.d), **f32), "dw3": torch.empty((w.E, w.F, w.d), **f32),
             "dw2": torch.empty((w.E, w.d, w.F), **f32), "dlogits": torch.empty((w.T, w.E), **f32)}
        M.moe_backward(dm, x, dev(W["w_gate"]), wd["w1"], wd["w3"], wd["w2"], dy, g["dx"], g["dw_gate"], g["dw1"],
                       g["dw3"], g["dw2"], ws, dlogits=g["dlogits"])
        torch.cuda.synchronize()
        return g

    rm = run(False)
    pk = run(True)
    for k in ("dx", "dlogits", "dw_gate"):
        assert torch.equal(rm[k], pk[k]), k
    for k in ("dw1", "dw3", "dw2"):
        E, N, K = rm[k].shape
        order = rm[k].reshape(E, N // 16, 16, K // 32, 4, 8).permute(0, 1, 3, 4, 2, 5).reshape(-1)
        assert torch.equal(order, pk[k].reshape(-1)), k
        say(f"  {k}: all {E * N * K} entries equal in the packed order")

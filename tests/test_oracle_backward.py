"""Pins of the oracle's backward pass (CPU only).

The pages define the forward layer; its gradient follows from that definition (chain rule, TopK
selection held fixed). The oracle's backward is pinned against things other than itself:
  - central finite differences of the oracle's exact-logit forward (a property of any gradient),
    in fp64 storage, along random directions for every input tensor;
  - an independent dense-mask formulation of the layer (all experts evaluated, gate matrix with
    zeros off the TopK, softmax over the kept logits) differentiated by torch autograd in fp64;
  - softmax-gradient invariants (the logit gradient sums to zero over the kept experts and is
    zero elsewhere; with K = 1 it vanishes);
  - the sampled entry points agree with the full one.
"""
import numpy as np
import pytest

import oracle

CASES = [
    dict(T=5, d=8, F=12, E=4, K=2, bias=False, seed=1),
    dict(T=6, d=16, F=8, E=8, K=2, bias=True, seed=2),
    dict(T=4, d=8, F=8, E=5, K=1, bias=False, seed=3),
    dict(T=4, d=8, F=16, E=6, K=3, bias=True, seed=4),
    dict(T=3, d=8, F=8, E=3, K=3, bias=False, seed=5),  # K = E: dense softmax gating
]


def layer(c, dtype=np.float64):
    rng = np.random.default_rng(c["seed"])
    T, d, F, E = c["T"], c["d"], c["F"], c["E"]
    L = dict(
        x=rng.standard_normal((T, d)),
        w_gate=rng.standard_normal((d, E)) / np.sqrt(d),
        w1=rng.standard_normal((E, F, d)) / np.sqrt(d),
        w3=rng.standard_normal((E, F, d)) / np.sqrt(d),
        w2=rng.standard_normal((E, d, F)) / np.sqrt(F),
    )
    L = {k: v.astype(dtype) for k, v in L.items()}
    L["bias"] = (0.3 * rng.standard_normal(E)).astype(np.float32) if c["bias"] else None
    L["dy"] = rng.standard_normal((T, d))
    return L


def loss(L, K, **override):
    a = dict(L)
    a.update(override)
    y, idx = oracle.forward_exact(a["x"], a["w_gate"], a["w1"], a["w3"], a["w2"], K, bias=a["bias"])
    return float((y * L["dy"]).sum()), idx


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"T{c['T']}d{c['d']}F{c['F']}E{c['E']}K{c['K']}")
def test_backward_matches_finite_differences(c):
    L = layer(c)
    K = c["K"]
    g = oracle.backward(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], K, L["dy"], bias=L["bias"])
    rng = np.random.default_rng(100 + c["seed"])
    eps = 1e-6
    for name, gname in (("x", "dx"), ("w_gate", "dw_gate"), ("w1", "dw1"), ("w3", "dw3"), ("w2", "dw2")):
        for _ in range(2):
            delta = rng.standard_normal(L[name].shape)
            lp, ip = loss(L, K, **{name: L[name] + eps * delta})
            lm, im = loss(L, K, **{name: L[name] - eps * delta})
            assert np.array_equal(ip, im), "selection changed under the perturbation"
            fd = (lp - lm) / (2 * eps)
            an = float((g[gname] * delta).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def torch_dense_grads(L, K, idx):
    """The layer written as a dense mixture (every expert evaluated, gates zero off the TopK),
    differentiated by torch autograd in fp64, with the selection idx held fixed."""
    torch = pytest.importorskip("torch")
    t = {k: torch.tensor(L[k], dtype=torch.float64, requires_grad=True)
         for k in ("x", "w_gate", "w1", "w3", "w2")}
    logits = t["x"] @ t["w_gate"]
    if L["bias"] is not None:
        logits = logits + torch.tensor(L["bias"], dtype=torch.float64)
    T, E = logits.shape
    mask = torch.zeros((T, E), dtype=torch.float64)
    mask[torch.arange(T).unsqueeze(1), torch.tensor(idx, dtype=torch.long)] = 1.0
    m = logits.detach().max(dim=1, keepdim=True).values
    ex = torch.exp(logits - m) * mask
    gates = ex / ex.sum(dim=1, keepdim=True)                      # [T][E], zero off the TopK
    a = torch.einsum("efd,td->tef", t["w1"], t["x"])
    b = torch.einsum("efd,td->tef", t["w3"], t["x"])
    h = a * torch.sigmoid(a) * b                                  # silu(a) * b
    o = torch.einsum("edf,tef->ted", t["w2"], h)                  # every expert's output
    y = (gates.unsqueeze(2) * o).sum(dim=1)
    (y * torch.tensor(L["dy"], dtype=torch.float64)).sum().backward()
    return {"dx": t["x"].grad.numpy(), "dw_gate": t["w_gate"].grad.numpy(), "dw1": t["w1"].grad.numpy(),
            "dw3": t["w3"].grad.numpy(), "dw2": t["w2"].grad.numpy()}


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"T{c['T']}d{c['d']}F{c['F']}E{c['E']}K{c['K']}")
def test_backward_matches_dense_autograd(c):
    L = layer(c)
    K = c["K"]
    g = oracle.backward(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], K, L["dy"], bias=L["bias"])
    _, idx = oracle.forward_exact(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], K, bias=L["bias"])
    ref = torch_dense_grads(L, K, idx)
    for k, v in ref.items():
        assert np.allclose(g[k], v, rtol=1e-10, atol=1e-12), k


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"T{c['T']}d{c['d']}F{c['F']}E{c['E']}K{c['K']}")
def test_logit_gradient_invariants(c):
    L = layer(c)
    K = c["K"]
    g = oracle.backward(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], K, L["dy"], bias=L["bias"])
    _, idx = oracle.forward_exact(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], K, bias=L["bias"])
    dl = g["dlogits"]
    assert np.allclose(dl.sum(axis=1), 0.0, atol=1e-12)
    for t in range(c["T"]):
        off = np.setdiff1d(np.arange(c["E"]), idx[t])
        assert np.all(dl[t, off] == 0.0)
    if K == 1:
        assert np.all(dl == 0.0)
    # dW_g = x^T dlogits (the router is linear in W_g)
    assert np.allclose(g["dw_gate"], L["x"].T @ dl, rtol=1e-12, atol=1e-14)


def test_sampled_entry_points_agree_with_full():
    c = CASES[1]
    L = layer(c)
    K = c["K"]
    g = oracle.backward(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], K, L["dy"], bias=L["bias"])
    toks = np.array([0, 3, 5], dtype=np.int64)
    dx, dl = oracle.backward_tokens(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], K, L["dy"], toks, bias=L["bias"])
    assert np.allclose(dx, g["dx"][toks], rtol=1e-12, atol=1e-14)
    assert np.allclose(dl, g["dlogits"][toks], rtol=1e-12, atol=1e-14)
    q = np.array([[1, 0, 3, 5], [3, 2, 7, 1], [2, 5, 9, 4], [1, 7, 0, 15], [2, 1, 15, 7], [3, 4, 2, 2]])
    v = oracle.backward_wsample(L["x"], L["w_gate"], L["w1"], L["w3"], L["w2"], K, L["dy"], q, bias=L["bias"])
    name = {1: "dw1", 3: "dw3", 2: "dw2"}
    ref = np.array([g[name[w]][e, i, j] for w, e, i, j in q])
    assert np.allclose(v, ref, rtol=1e-12, atol=1e-14)


def test_bf16_storage_backward_matches_finite_differences_of_widened_inputs():
    """bf16 bit patterns are widened exactly: the gradient equals the fp64 one of the widened values."""
    import moe_inputs as mi
    c = CASES[0]
    L = layer(c)
    Lb = {k: (mi.f32_to_bf16_bits(v.astype(np.float32)) if k in ("x", "w_gate", "w1", "w3", "w2") else v)
          for k, v in L.items()}
    Lw = {k: (mi.bf16_bits_to_f32(v).astype(np.float64) if k in ("x", "w_gate", "w1", "w3", "w2") else v)
          for k, v in Lb.items()}
    gb = oracle.backward(Lb["x"], Lb["w_gate"], Lb["w1"], Lb["w3"], Lb["w2"], c["K"], L["dy"])
    gw = oracle.backward(Lw["x"], Lw["w_gate"], Lw["w1"], Lw["w3"], Lw["w2"], c["K"], L["dy"])
    for k in gb:
        assert np.array_equal(gb[k], gw[k]), k

"""Pins for the CPU oracle: each check ties it to something other than itself.

- the pages' worked two-expert example (blog.csdn.net section 2.3) as a golden fixture;
- closed forms (K=2 gate = logistic of the logit gap; silu identities; RMSNorm RMS);
- the alternative order "softmax over all n, TopK, renormalise" (csdn section 3.2), which
  gives the same weights;
- brute force on tiny inputs: every expert computed for every token, then a dense gating
  vector with exact zeros (csdn sections 1 and 2.4);
- reduction to textbook cases: E=1/K=1 is a dense SwiGLU FFN, K=E is dense softmax gating;
- the permutation against a stable sort; the shapes against the pages' parameter counts.
"""
import json
import math
import os

import numpy as np
import pytest

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    mi.build()
    oracle.build()


def f64(a):
    return mi.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def silu_np(z):
    return z / (1.0 + np.exp(-z))


def small_layer(seed, T, d, F, E, dtype="f32"):
    w = mi.Workload("t", T=T, d=d, F=F, E=E, dtype=dtype, seed=seed)
    x = mi.tokens(w)
    W = mi.layer_weights(w)
    return x, W


# ---------------------------------------------------------------- routing

def test_worked_example_experts_3_and_5():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_experts_3_5.json")))
    l = np.array(g["logits"], np.float32)
    n, K = g["n_experts"], g["K"]
    x = l[None, :].copy()                      # with W_g = I the logits are x itself
    wg = np.eye(n, dtype=np.float32)
    logits, idx, w = oracle.route(x, wg, K)
    assert idx[0].tolist() == g["selected_in_slot_order"]
    l3, l5 = float(l[3]), float(l[5])
    g3 = math.exp(l3) / (math.exp(l3) + math.exp(l5))
    g5 = math.exp(l5) / (math.exp(l3) + math.exp(l5))
    assert abs(w[0, 0] - g3) < 1e-15 and abs(w[0, 1] - g5) < 1e-15
    assert abs(w[0].sum() - 1.0) < 1e-15


def test_gate_closed_form_and_invariants():
    x, W = small_layer(11, 300, 64, 64, 8)
    logits, idx, w = oracle.route(x, W["w_gate"], 2)
    # K=2: g0 = 1/(1+exp(l1-l0)) (logistic of the gap), g1 = 1-g0, 1/2 <= g0 <= 1
    l0 = np.take_along_axis(logits, idx[:, :1], 1)[:, 0]
    l1 = np.take_along_axis(logits, idx[:, 1:2], 1)[:, 0]
    assert np.allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=0, atol=1e-15)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    assert (w[:, 0] >= 0.5).all() and (w[:, 0] <= 1.0).all()
    assert (idx[:, 0] != idx[:, 1]).all()


def test_logits_match_matmul_and_topk_matches_sort():
    x, W = small_layer(12, 257, 96, 64, 8)
    bias = mi.skew_bias(8)
    logits, idx, w = oracle.route(x, W["w_gate"], 2, bias=bias)
    ref = (f64(x) @ f64(W["w_gate"]) + bias.astype(np.float64)).astype(np.float32).astype(np.float64)
    # same double value up to summation order, then rounded to fp32: equal or one fp32 ulp apart
    assert np.all(np.abs(ref - logits) <= np.abs(ref) * 2.0 ** -23 + 1e-30)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :2]
    assert np.array_equal(order, idx)


def test_topk_ties_go_to_lower_index():
    d, E = 4, 8
    wg = np.zeros((d, E), np.float32)
    wg[0, :] = [1.0, 3.0, 3.0, 0.5, 3.0, -1.0, 2.0, 2.0]   # three-way tie at 3.0, tie at 2.0
    x = np.array([[1.0, 0, 0, 0], [-1.0, 0, 0, 0]], np.float32)
    _, idx, w = oracle.route(x, wg, 2)
    assert idx[0].tolist() == [1, 2]                      # ties: lower index first
    assert idx[1].tolist() == [5, 3]                      # -l: 1.0 (e5) > -0.5 (e3) > -1 (e0)
    assert w[0, 0] == w[0, 1] == 0.5


def test_softmax_then_topk_renormalised_is_the_same():
    x, W = small_layer(13, 200, 64, 64, 8)
    logits, idx, w = oracle.route(x, W["w_gate"], 2)
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)                          # softmax over all n first
    top = np.argsort(-p, axis=1, kind="stable")[:, :2]
    assert np.array_equal(top, idx)                        # softmax is monotone
    pk = np.take_along_axis(p, top, 1)
    pk /= pk.sum(1, keepdims=True)                         # renormalise the kept ones
    assert np.allclose(pk, w, rtol=0, atol=1e-14)


def test_general_k():
    x, W = small_layer(14, 50, 64, 64, 16)
    for K in (1, 3, 4, 16):
        logits, idx, w = oracle.route(x, W["w_gate"], K)
        assert np.array_equal(idx, np.argsort(-logits, 1, kind="stable")[:, :K])
        assert np.allclose(w.sum(1), 1.0, atol=1e-14)
        if K == 1:
            assert np.all(w == 1.0)


# ---------------------------------------------------------------- permutation

def test_permute_against_stable_sort():
    T, E, K = 1000, 8, 2
    idx = mi.synthetic_routing(5, T, E, K, skew=2.0)
    counts, offsets, row_token, token_row = oracle.permute(idx, E)
    assert counts.sum() == T * K
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and np.array_equal(offsets[1:], np.cumsum(counts))
    slots = np.argsort(idx.ravel(), kind="stable")          # slot s = t*K + k, stable by expert
    assert np.array_equal(row_token, slots // K)
    assert np.array_equal(token_row.ravel()[slots], np.arange(T * K))
    for e in range(E):
        grp = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(grp) > 0)                      # ascending tokens, each once
        assert np.all((idx[grp] == e).any(1))


def test_permute_empty_experts_and_gather():
    T, E, K = 37, 8, 2
    idx = np.stack([np.full(T, 6), np.full(T, 2)], 1).astype(np.int32)   # only experts 2 and 6
    counts, offsets, row_token, token_row = oracle.permute(idx, E)
    assert counts.tolist() == [0, 0, T, 0, 0, 0, T, 0]
    assert offsets.tolist() == [0, 0, 0, T, T, T, T, 2 * T, 2 * T]
    x = mi.normal(mi.key(9, 0, 0), (T, 64), 1.0, "bf16")
    xp = oracle.gather(x, row_token)
    assert np.array_equal(xp, x[row_token])


# ---------------------------------------------------------------- expert FFN

@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_silu_identities_through_the_ffn(sign):
    # E=1, K=1, d=F=1: y = silu(a*x) * (b*x) * c with w1=[[a]], w3=[[b]], w2=[[c]].
    def y_of(a, b, c, xv):
        z = lambda v: np.array([[[v]]], np.float32)
        return oracle.forward(np.array([[xv]], np.float32), np.ones((1, 1), np.float32), z(a), z(b), z(c), 1)["y"][0, 0]

    a = np.float32(sign * 1.75)
    # silu(a) - silu(-a) = a: fails for a flipped exponent sign or for gating on w3 instead of w1
    assert abs((y_of(a, 1.0, 1.0, 1.0) - y_of(-a, 1.0, 1.0, 1.0)) - float(a)) < 1e-15
    assert abs(y_of(a, 2.5, 1.0, 1.0) - y_of(-a, 2.5, 1.0, 1.0) - 2.5 * float(a)) < 1e-14
    assert y_of(0.0, 3.0, 1.0, 1.0) == 0.0                              # silu(0) = 0
    l3 = np.float32(math.log(3.0))
    assert abs(y_of(l3, 1.0, 1.0, 1.0) / float(l3) - 0.75) < 1e-7        # sigma(ln 3) = 3/4
    assert abs(y_of(a, 1.0, -2.0, 1.0) + 2.0 * y_of(a, 1.0, 1.0, 1.0)) < 1e-15   # linear in w2


def test_expert_ffn_rows_use_their_group():
    x, W = small_layer(15, 120, 64, 128, 4)
    idx = mi.synthetic_routing(6, 120, 4, 2, skew=1.0)
    counts, offsets, row_token, token_row = oracle.permute(idx, 4)
    xp = oracle.gather(x, row_token)
    y, h = oracle.expert_ffn(xp, offsets, W["w1"], W["w3"], W["w2"], want_hidden=True)
    for r in [0, 5, int(offsets[1]), int(offsets[2]) + 3, 239]:
        e = int(np.searchsorted(offsets, r, side="right") - 1)
        xv = f64(xp[r])
        hid = silu_np(f64(W["w1"][e]) @ xv) * (f64(W["w3"][e]) @ xv)
        assert np.allclose(h[r], hid, rtol=1e-12, atol=1e-14)
        assert np.allclose(y[r], f64(W["w2"][e]) @ hid, rtol=1e-12, atol=1e-13)


def test_reduces_to_dense_swiglu_when_e1_k1():
    x, W = small_layer(16, 40, 64, 96, 1)
    r = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], 1)
    assert np.all(r["idx"] == 0) and np.all(r["w"] == 1.0)
    X = f64(x)
    dense = (silu_np(X @ f64(W["w1"][0]).T) * (X @ f64(W["w3"][0]).T)) @ f64(W["w2"][0]).T
    assert np.allclose(r["y"], dense, rtol=1e-12, atol=1e-13)


def _dense_bruteforce(x, W, K, bias=None):
    """All experts for all tokens, then a dense gating vector with exact zeros."""
    X = f64(x)
    E = W["w1"].shape[0]
    l = X @ f64(W["w_gate"])
    if bias is not None:
        l = l + bias.astype(np.float64)
    l = l.astype(np.float32).astype(np.float64)               # decision precision: fp32
    keep = np.argsort(-l, axis=1, kind="stable")[:, :K]
    masked = np.full_like(l, -np.inf)
    np.put_along_axis(masked, keep, np.take_along_axis(l, keep, 1), 1)
    G = np.exp(masked - masked.max(1, keepdims=True))        # exp(-inf) = 0
    G /= G.sum(1, keepdims=True)
    y = np.zeros_like(X)
    for e in range(E):
        out = (silu_np(X @ f64(W["w1"][e]).T) * (X @ f64(W["w3"][e]).T)) @ f64(W["w2"][e]).T
        y += G[:, e:e + 1] * out
    return y, G


@pytest.mark.parametrize("dtype,bias", [("f32", False), ("bf16", False), ("bf16", True)])
def test_sparse_equals_dense_bruteforce(dtype, bias):
    w = mi.WORKLOADS["tiny_f32"].with_(dtype=dtype, skew_bias=bias)
    x = mi.tokens(w)
    W = mi.layer_weights(w)
    r = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], 2, bias=W["bias"])
    y, G = _dense_bruteforce(x, W, 2, W["bias"])
    assert np.abs(r["y"] - y).max() <= 1e-12 * np.abs(y).max()
    assert ((G > 0).sum(1) == 2).all()                          # exactly K non-zeros per token
    assert np.allclose(np.take_along_axis(G, r["idx"].astype(np.int64), 1), r["w"], atol=1e-15)


def test_k_equals_e_is_dense_softmax_gating():
    x, W = small_layer(17, 30, 64, 64, 4)
    r = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], 4)
    l = (f64(x) @ f64(W["w_gate"])).astype(np.float32).astype(np.float64)
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    y = sum(p[:, e:e + 1] * ((silu_np(f64(x) @ f64(W["w1"][e]).T) * (f64(x) @ f64(W["w3"][e]).T)) @ f64(W["w2"][e]).T)
            for e in range(4))
    assert np.abs(r["y"] - y).max() <= 1e-12 * np.abs(y).max()


def test_stage_pipeline_equals_forward():
    """route -> permute -> gather -> expert_ffn -> combine equals the per-token forward."""
    w = mi.WORKLOADS["tiny_f32"]
    x = mi.tokens(w)
    W = mi.layer_weights(w)
    logits, idx, gw = oracle.route(x, W["w_gate"], 2)
    counts, offsets, row_token, token_row = oracle.permute(idx, 8)
    yp = oracle.expert_ffn(oracle.gather(x, row_token), offsets, W["w1"], W["w3"], W["w2"])
    y = oracle.combine(yp.astype(np.float32), token_row, gw.astype(np.float32))
    ref = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], 2)["y"]
    assert np.abs(y - ref).max() <= 1e-6 * np.abs(ref).max()     # fp32 staging of y_perm and w


def test_combine_closed_form():
    T, K, d = 5, 2, 8
    token_row = np.array([[3, 0], [1, 9], [2, 4], [8, 5], [7, 6]], np.int32)
    y_perm = np.repeat(np.arange(10, dtype=np.float32)[:, None], d, 1)      # row r holds the value r
    gw = np.array([[0.75, 0.25], [0.5, 0.5], [1.0, 0.0], [0.625, 0.375], [0.875, 0.125]], np.float32)
    y = oracle.combine(y_perm, token_row, gw)
    expect = (gw * token_row).sum(1)
    assert np.array_equal(y, np.repeat(expect[:, None], d, 1))


def test_expert_equivariance_under_relabelling():
    x, W = small_layer(18, 64, 64, 64, 8)
    r = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], 2)
    perm = np.array([5, 2, 7, 0, 1, 6, 3, 4])
    r2 = oracle.forward(x, W["w_gate"][:, perm], W["w1"][perm], W["w3"][perm], W["w2"][perm], 2)
    assert np.array_equal(perm[r2["idx"]], r["idx"])
    assert np.allclose(r2["y"], r["y"], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- RMSNorm / deep layer

def test_rmsnorm_closed_forms():
    h = mi.normal(mi.key(3, 0, 0), (16, 256), 2.0, "f32").astype(np.float64)
    eps = 1e-5
    xb, ex = oracle.rmsnorm_bf16(h, eps, want_exact=True)
    ms = (h ** 2).mean(1)
    rms_out = np.sqrt((ex ** 2).mean(1))
    assert np.allclose(rms_out, 1.0 / np.sqrt(1.0 + eps / ms), rtol=1e-13)
    c = np.full((1, 64), 3.0)
    _, exc = oracle.rmsnorm_bf16(c, eps, want_exact=True)
    assert np.allclose(exc, 3.0 / math.sqrt(9.0 + eps), rtol=1e-15)
    # bf16 result is the round-to-nearest of the exact value: within half a bf16 ulp
    xf = f64(xb)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(ex))) - 7)
    assert np.all(np.abs(xf - ex) <= 0.5 * ulp * (1 + 1e-9))


def test_deep_layer_residual():
    w = mi.Workload("deep_tiny", T=12, d=64, F=128, layers=2, seed=21)
    W = mi.layer_weights(w)
    h = mi.residual0(w).astype(np.float64)
    h0 = h.copy()
    Wz = dict(W, w2=np.zeros_like(W["w2"]))
    oracle.deep_layer(h, Wz["w_gate"], Wz["w1"], Wz["w3"], Wz["w2"], 2, w.eps)
    assert np.array_equal(h, h0)                      # expert output 0 -> residual unchanged
    idx, _ = oracle.deep_layer(h, W["w_gate"], W["w1"], W["w3"], W["w2"], 2, w.eps)
    x = oracle.rmsnorm_bf16(h0, w.eps)
    ref = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], 2)
    assert np.array_equal(idx, ref["idx"])
    assert np.allclose(h, h0 + ref["y"], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- shapes

def test_parameter_arithmetic_pins_the_expert_shape():
    g = json.load(open(os.path.join(GOLDEN, "parameter_counts.json")))
    L, d, F, E, K = g["layers"], g["d"], g["F"], g["E"], g["K"]
    per_expert = 3 * d * F                 # w1, w3: F x d; w2: d x F
    inactive = L * (E - K) * per_expert    # parameters a token does not touch
    assert abs(inactive / 1e9 - (g["total_params_B"] - g["active_params_B"])) < 0.05
    assert L * E * per_expert / 1e9 < g["total_params_B"]    # rest: attention + embeddings
    assert abs(L * E * per_expert / 1e9 - 45.10) < 0.01


def test_generator_is_counter_based():
    k = mi.key(7, 3, 2)
    a = mi.normal(k, (1000,), 1.0, "bf16")
    b = mi.normal(k, (400,), 1.0, "bf16", start=600)
    assert np.array_equal(a[600:], b)
    assert not np.array_equal(a, mi.normal(mi.key(7, 4, 2), (1000,), 1.0, "bf16"))
    f = mi.normal(mi.key(7, 3, 3), (200000,), 1.0, "f32")
    assert abs(f.mean()) < 0.01 and abs(f.std() - 1.0) < 0.01


# ---------------------------------------------------------------- selection override (ties in TopK)
# TopK keeps "the K largest values" (csdn section 2.2); where kept and dropped logits are equal within
# the decision precision more than one selection satisfies it, and the layer's output under each is
# a correct result. The oracle then evaluates the layer under a given selection.

def _masked_bruteforce(x, W, sel, bias=None):
    """Every expert for every token, then a dense gating vector that is the softmax over the logits of
    the given experts and exactly 0 elsewhere (csdn sections 1, 2.3 and 2.4)."""
    X = f64(x)
    E = W["w1"].shape[0]
    l = X @ f64(W["w_gate"])
    if bias is not None:
        l = l + bias.astype(np.float64)
    l = l.astype(np.float32).astype(np.float64)
    masked = np.full_like(l, -np.inf)
    np.put_along_axis(masked, sel.astype(np.int64), np.take_along_axis(l, sel.astype(np.int64), 1), 1)
    G = np.exp(masked - masked.max(1, keepdims=True))
    G /= G.sum(1, keepdims=True)
    y = np.zeros_like(X)
    for e in range(E):
        out = (silu_np(X @ f64(W["w1"][e]).T) * (X @ f64(W["w3"][e]).T)) @ f64(W["w2"][e]).T
        y += G[:, e:e + 1] * out
    return y, G


@pytest.mark.parametrize("dtype,bias,E,K", [("f32", False, 8, 2), ("bf16", True, 8, 2), ("bf16", False, 16, 3),
                                            ("f32", True, 8, 1)])
def test_own_selection_reproduces_forward_bit_for_bit(dtype, bias, E, K):
    w = mi.Workload("sel_own", T=70, d=64, F=96, E=E, K=K, dtype=dtype, skew_bias=bias, seed=1301)
    x, W = mi.tokens(w), mi.layer_weights(w)
    tok = np.array([0, 3, 17, 69], np.int64)
    r = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], K, bias=W["bias"], tokens=tok)
    s = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], K, bias=W["bias"], tokens=tok, select=r["idx"])
    for k in ("y", "logits", "idx", "w"):
        assert np.array_equal(r[k], s[k]), k


@pytest.mark.parametrize("dtype,bias,E,K", [("f32", False, 8, 2), ("bf16", True, 8, 2), ("bf16", False, 16, 3)])
def test_forced_selection_equals_masked_bruteforce(dtype, bias, E, K):
    """A selection other than the TopK (the experts ranked 2..K+1, slots in reverse order) equals the
    dense compute-all-experts brute force gated by the softmax over that selection."""
    w = mi.Workload("sel_forced", T=50, d=64, F=128, E=E, K=K, dtype=dtype, skew_bias=bias, seed=1302)
    x, W = mi.tokens(w), mi.layer_weights(w)
    own = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], K, bias=W["bias"])
    order = np.argsort(-own["logits"], axis=1, kind="stable")
    sel = order[:, 1:K + 1][:, ::-1].astype(np.int32)          # not the TopK set, not in logit order
    r = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], K, bias=W["bias"], select=sel)
    assert np.array_equal(r["idx"], sel)
    y, G = _masked_bruteforce(x, W, sel, W["bias"])
    assert np.abs(r["y"] - y).max() <= 1e-12 * np.abs(y).max()
    assert np.allclose(np.take_along_axis(G, sel.astype(np.int64), 1), r["w"], rtol=0, atol=1e-15)
    assert np.allclose(r["w"].sum(1), 1.0, rtol=0, atol=1e-15)
    assert not np.allclose(r["y"], own["y"])                    # the override changes the result


def test_exact_tie_either_selection():
    """Two experts with identical router columns tie exactly: the oracle keeps the lower index (the
    tie reading), and the output under the other selection is that of the same layer with the two
    experts' weights swapped."""
    w = mi.Workload("sel_tie", T=30, d=64, F=64, E=4, K=1, dtype="f32", seed=1303)
    x, W = mi.tokens(w), mi.layer_weights(w)
    W["w_gate"][:, 1] += 10.0 / 64                              # experts 1 and 2 lead for most tokens
    W["w_gate"][:, 2] = W["w_gate"][:, 1]
    r = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], 1)
    tied = np.flatnonzero(r["logits"][:, 1] == r["logits"].max(1))
    assert len(tied) > 0 and np.all(r["idx"][tied, 0] == 1)
    alt = r["idx"].copy()
    alt[tied, 0] = 2
    a = oracle.forward(x, W["w_gate"], W["w1"], W["w3"], W["w2"], 1, select=alt)
    sw = [0, 2, 1, 3]
    b = oracle.forward(x, W["w_gate"], W["w1"][sw], W["w3"][sw], W["w2"][sw], 1)
    assert np.array_equal(a["y"][tied], b["y"][tied])

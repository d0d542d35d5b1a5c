"""Pins of the oracle's decoder-block functions (CPU only).

The pages fix the block only by its numbers (32 heads, 8 key-value heads, width 4096, a
pre-norm transformer whose feed-forward sub-block is the MoE layer); the rest is the reading
written out in oracle.cpp. What pins each part here, other than the oracle itself:
  - rotary embedding: the same rotation written as complex multiplication (numpy), identity at
    position 0, norm preservation, and dot products that depend only on the position difference;
  - attention: torch's scaled_dot_product_attention (fp64, causal) with the key-value heads
    repeated, the one-position case (output = value), the zero-query case (output = running
    mean of the values), and outputs inside the range of the values they mix;
  - block: with a zero output projection it is exactly the deep-stack layer (pinned elsewhere),
    and its attention half matches an independent torch fp64 composition.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle

torch = pytest.importorskip("torch")


def rope_complex(x, n_heads, D, base, p0=0):
    T = x.shape[0]
    x = x.reshape(T, n_heads, D).astype(np.float64)
    half = D // 2
    z = x[..., :half] + 1j * x[..., half:]
    pos = (p0 + np.arange(T))[:, None, None]
    ang = pos * base ** (-2.0 * np.arange(half) / D)[None, None, :]
    z = z * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1).reshape(T, n_heads * D)


@pytest.mark.parametrize("base", [10000.0, 1e6])
def test_rope_matches_complex_rotation(base):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 3 * 16))
    got = oracle.rope(x, 3, 16, base, p0=5)
    assert np.allclose(got, rope_complex(x, 3, 16, base, p0=5), rtol=1e-12, atol=1e-12)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(2)
    D, base = 32, 1e6
    x = rng.standard_normal((1, D))
    assert np.array_equal(oracle.rope(x, 1, D, base, p0=0), x)
    xs = rng.standard_normal((6, D))
    r = oracle.rope(xs, 1, D, base, p0=100)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(xs, axis=1), rtol=1e-13)
    q, k = rng.standard_normal((1, D)), rng.standard_normal((1, D))
    for p, s in ((7, 3), (1000, 250), (20000, 19999)):
        a = float((oracle.rope(q, 1, D, base, p0=p) @ oracle.rope(k, 1, D, base, p0=s).T)[0, 0])
        b = float((oracle.rope(q, 1, D, base, p0=p + 11) @ oracle.rope(k, 1, D, base, p0=s + 11).T)[0, 0])
        assert abs(a - b) <= 1e-9 * max(1.0, abs(a)), (p, s, a, b)


def sdpa_reference(q, k, v, Hq, Hkv):
    T = q.shape[0]
    D = q.shape[1] // Hq
    G = Hq // Hkv
    tq = torch.tensor(q.reshape(T, Hq, D).transpose(1, 0, 2), dtype=torch.float64)
    tk = torch.tensor(k.reshape(T, Hkv, D).transpose(1, 0, 2), dtype=torch.float64).repeat_interleave(G, dim=0)
    tv = torch.tensor(v.reshape(T, Hkv, D).transpose(1, 0, 2), dtype=torch.float64).repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    return o.numpy().transpose(1, 0, 2).reshape(T, Hq * D)


@pytest.mark.parametrize("T,Hq,Hkv,D", [(13, 4, 1, 16), (9, 8, 2, 8), (5, 2, 2, 4)])
def test_attention_matches_torch_sdpa(T, Hq, Hkv, D):
    rng = np.random.default_rng(T * 100 + Hq)
    q = rng.standard_normal((T, Hq * D))
    k = rng.standard_normal((T, Hkv * D))
    v = rng.standard_normal((T, Hkv * D))
    got = oracle.attention(q, k, v, Hq, Hkv)
    assert np.allclose(got, sdpa_reference(q, k, v, Hq, Hkv), rtol=1e-12, atol=1e-12)
    # selected positions give the same rows
    sel = np.array([T - 1, 0, T // 2])
    assert np.allclose(oracle.attention(q, k, v, Hq, Hkv, tokens=sel), got[sel], rtol=0, atol=0)


def test_attention_closed_forms():
    rng = np.random.default_rng(3)
    Hq, Hkv, D, T = 4, 2, 8, 6
    k = rng.standard_normal((T, Hkv * D))
    v = rng.standard_normal((T, Hkv * D))
    # one position: the output is the value of the head's key-value head
    out1 = oracle.attention(rng.standard_normal((1, Hq * D)), k[:1], v[:1], Hq, Hkv)
    for hq in range(Hq):
        hk = hq // (Hq // Hkv)
        assert np.allclose(out1[0, hq * D:(hq + 1) * D], v[0, hk * D:(hk + 1) * D], rtol=0, atol=1e-15)
    # zero queries: uniform weights over the causal prefix -> running mean of the values
    out0 = oracle.attention(np.zeros((T, Hq * D)), k, v, Hq, Hkv)
    run = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    for hq in range(Hq):
        hk = hq // (Hq // Hkv)
        assert np.allclose(out0[:, hq * D:(hq + 1) * D], run[:, hk * D:(hk + 1) * D], rtol=1e-13, atol=1e-14)
    # a convex combination stays inside the range of the values it mixes
    q = 3.0 * rng.standard_normal((T, Hq * D))
    out = oracle.attention(q, k, v, Hq, Hkv)
    for t in range(T):
        for hq in range(Hq):
            hk = hq // (Hq // Hkv)
            pv = v[:t + 1, hk * D:(hk + 1) * D]
            o = out[t, hq * D:(hq + 1) * D]
            assert np.all(o <= pv.max(axis=0) + 1e-12) and np.all(o >= pv.min(axis=0) - 1e-12)


def block_weights(seed, d, Hq, Hkv, D, F, E):
    rng = np.random.default_rng(seed)
    bf = lambda a: mi.f32_to_bf16_bits(a.astype(np.float32))
    return dict(
        w_qkv=bf(rng.standard_normal(((Hq + 2 * Hkv) * D, d)) / np.sqrt(d)),
        w_o=bf(rng.standard_normal((d, Hq * D)) / np.sqrt(Hq * D)),
        w_gate=bf(rng.standard_normal((d, E)) / np.sqrt(d)),
        w1=bf(rng.standard_normal((E, F, d)) / np.sqrt(d)),
        w3=bf(rng.standard_normal((E, F, d)) / np.sqrt(d)),
        w2=bf(rng.standard_normal((E, d, F)) / np.sqrt(F)),
    )


def test_block_with_zero_output_projection_is_the_deep_stack_layer():
    T, d, Hq, Hkv, D, F, E, K = 7, 32, 4, 2, 8, 16, 4, 2
    W = block_weights(4, d, Hq, Hkv, D, F, E)
    W["w_o"] = np.zeros_like(W["w_o"])
    h = np.random.default_rng(5).standard_normal((T, d))
    got = oracle.block(h, W["w_qkv"], W["w_o"], W["w_gate"], W["w1"], W["w3"], W["w2"], K, Hq, Hkv, 1e6, 1e-5)
    ref = h.copy()
    idx, _ = oracle.deep_layer(ref, W["w_gate"], W["w1"], W["w3"], W["w2"], K, 1e-5)
    assert np.array_equal(got["h1"], h)
    assert np.array_equal(got["idx"], idx)
    assert np.allclose(got["h2"], ref, rtol=1e-14, atol=1e-14)


def test_block_attention_half_matches_torch_composition():
    T, d, Hq, Hkv, D, F, E, K = 11, 32, 4, 1, 8, 16, 4, 2
    base, eps = 1e6, 1e-5
    W = block_weights(6, d, Hq, Hkv, D, F, E)
    h = 2.0 * np.random.default_rng(7).standard_normal((T, d))
    got = oracle.block(h, W["w_qkv"], W["w_o"], W["w_gate"], W["w1"], W["w3"], W["w2"], K, Hq, Hkv, base, eps)
    # independent composition: torch rms norm, bf16 cast (round to nearest even), matmuls,
    # rotary as complex rotation, torch sdpa
    th = torch.tensor(h, dtype=torch.float64)
    u = (th / torch.sqrt((th * th).mean(dim=1, keepdim=True) + eps)).to(torch.float32).to(torch.bfloat16)
    u = u.to(torch.float64).numpy()
    wqkv = mi.bf16_bits_to_f32(W["w_qkv"]).astype(np.float64)
    wo = mi.bf16_bits_to_f32(W["w_o"]).astype(np.float64)
    qkv = u @ wqkv.T
    q = rope_complex(qkv[:, :Hq * D], Hq, D, base)
    k = rope_complex(qkv[:, Hq * D:(Hq + Hkv) * D], Hkv, D, base)
    v = qkv[:, (Hq + Hkv) * D:]
    o = sdpa_reference(q, k, v, Hq, Hkv)
    assert np.allclose(got["h1"], h + o @ wo.T, rtol=1e-11, atol=1e-12)
    # x2 is the bf16 rms norm of h1, h2 = h1 + MoE(x2) on the selected rows too
    sel = np.array([10, 3])
    part = oracle.block(h, W["w_qkv"], W["w_o"], W["w_gate"], W["w1"], W["w3"], W["w2"], K, Hq, Hkv, base, eps,
                        tokens=sel)
    for key in ("h1", "x2", "h2", "idx"):
        assert np.array_equal(part[key], got[key][sel]), key


def test_block_selection_override():
    """The MoE sub-block under a selection override: the block's own selection reproduces it bit for
    bit; another selection changes h2 by exactly the layer's difference under the two selections
    (evaluated by the layer oracle on the block's own x2)."""
    T, d, Hq, Hkv, D, F, E, K = 9, 32, 4, 2, 8, 16, 4, 2
    base, eps = 1e6, 1e-5
    W = block_weights(8, d, Hq, Hkv, D, F, E)
    h = np.random.default_rng(9).standard_normal((T, d))
    args = (W["w_qkv"], W["w_o"], W["w_gate"], W["w1"], W["w3"], W["w2"], K, Hq, Hkv, base, eps)
    got = oracle.block(h, *args)
    same = oracle.block(h, *args, select=got["idx"])
    for key in ("h1", "x2", "h2", "idx", "logits"):
        assert np.array_equal(same[key], got[key]), key
    alt = np.argsort(-got["logits"], axis=1, kind="stable")[:, 1:K + 1].astype(np.int32)
    other = oracle.block(h, *args, select=alt)
    assert np.array_equal(other["x2"], got["x2"]) and np.array_equal(other["idx"], alt)
    y_own = oracle.forward(got["x2"], W["w_gate"], W["w1"], W["w3"], W["w2"], K)["y"]
    y_alt = oracle.forward(got["x2"], W["w_gate"], W["w1"], W["w3"], W["w2"], K, select=alt)["y"]
    assert np.allclose(other["h2"] - got["h2"], y_alt - y_own, rtol=0, atol=1e-12)

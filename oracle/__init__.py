"""CPU oracle for the Mixtral sparse mixture-of-experts layer (ctypes wrapper of oracle.cpp).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the product path never does. It shares no code with the HIP
library and does not import it. Inputs are numpy arrays: ``float32`` for fp32
storage and ``uint16`` for bf16 bit patterns. Results are float64.

Every function follows the definitions of "Mixtral of Experts" (arXiv
2401.04088) as restated on the blog.csdn.net page (sections 1 and 2.1-2.4:
logits x.W_g, TopK with -inf, softmax over the kept logits, gate-weighted sum)
and the xyznot.com summary ("Método": n=8 SwiGLU experts, K=2). See oracle.cpp
for the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-pthread", "-fPIC", "-shared", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()  # compiles only when the library is missing or older than oracle.cpp
        L = ctypes.CDLL(_LIB)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L.oracle_route.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32]
        L.oracle_permute.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_gather.argtypes = [i64, i64, vp, vp, vp]
        L.oracle_expert_ffn.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, i64, vp, vp, vp, i32]
        L.oracle_combine.argtypes = [i64, vp, i32, i32, vp, vp, vp, vp]
        L.oracle_forward.argtypes = [i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp,
                                     vp, vp, i32]
        L.oracle_rmsnorm_bf16.argtypes = [i64, i32, dbl, vp, vp, vp]
        L.oracle_deep_layer.argtypes = [i64, i32, i32, i32, i32, dbl, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        L.oracle_forward_exact.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp]
        L.oracle_backward.argtypes = [i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp]
        L.oracle_backward_tokens.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp,
                                             i32]
        L.oracle_backward_wsample.argtypes = [i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp,
                                              vp, i32]
        L.oracle_rope.argtypes = [i64, i32, i32, dbl, i64, i32, vp, vp]
        L.oracle_attention.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, i64, vp, vp, i32]
        L.oracle_block.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32, dbl, dbl, i32, vp, vp, vp, vp, vp, vp,
                                   vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, i32]
        L.oracle_abi_version.restype = i32
        assert L.oracle_abi_version() == 2, "liboracle.so is out of date: rebuild it (oracle.build(force=True))"
        _lib = L
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float64:
        return 2
    raise TypeError(f"storage dtype must be float32, uint16 (bf16 bits) or float64, got {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def route(x, w_gate, K, bias=None, threads=0):
    """Returns (logits [T][E] (fp32-rounded, as float64), topk_idx [T][K] int32, topk_w [T][K] float64)."""
    x, w_gate = _c(x), _c(w_gate)
    bias = _c(bias, np.float32)
    T, d = x.shape
    E = w_gate.shape[1]
    dt = _dtype_code(x)
    assert _dtype_code(w_gate) == dt and w_gate.shape[0] == d
    logits = np.empty((T, E), np.float64)
    idx = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    lib().oracle_route(T, d, E, K, dt, _p(x), _p(w_gate), _p(bias), _p(logits), _p(idx), _p(w), threads)
    return logits, idx, w


def permute(topk_idx, E):
    """Returns (counts [E], offsets [E+1], row_token [T*K], token_row [T][K]), all int32."""
    topk_idx = _c(topk_idx, np.int32)
    T, K = topk_idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_token = np.empty(T * K, np.int32)
    token_row = np.empty((T, K), np.int32)
    lib().oracle_permute(T, E, K, _p(topk_idx), _p(counts), _p(offsets), _p(row_token), _p(token_row))
    return counts, offsets, row_token, token_row


def gather(x, row_token):
    x = _c(x)
    row_token = _c(row_token, np.int32)
    out = np.empty((row_token.shape[0], x.shape[1]), x.dtype)
    lib().oracle_gather(row_token.shape[0], x.shape[1] * x.itemsize, _p(x), _p(row_token), _p(out))
    return out


def expert_ffn(x_perm, offsets, w1, w3, w2, rows=None, want_hidden=False, threads=0):
    """y rows [n_sel][d] (float64) of the expert FFN over expert-contiguous rows."""
    x_perm, w1, w3, w2 = _c(x_perm), _c(w1), _c(w3), _c(w2)
    offsets = _c(offsets, np.int32)
    dt = _dtype_code(x_perm)
    E, F, d = w1.shape
    assert w3.shape == (E, F, d) and w2.shape == (E, d, F) and x_perm.shape[1] == d
    rows = np.arange(x_perm.shape[0], dtype=np.int64) if rows is None else _c(rows, np.int64)
    y = np.empty((rows.shape[0], d), np.float64)
    h = np.empty((rows.shape[0], F), np.float64) if want_hidden else None
    lib().oracle_expert_ffn(d, F, E, dt, _p(x_perm), _p(offsets), _p(w1), _p(w3), _p(w2), rows.shape[0],
                            _p(rows), _p(h), _p(y), threads)
    return (y, h) if want_hidden else y


def combine(y_perm, token_row, topk_w, tokens=None):
    y_perm = _c(y_perm, np.float32)
    token_row = _c(token_row, np.int32)
    topk_w = _c(topk_w, np.float32)
    T, K = token_row.shape
    d = y_perm.shape[1]
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    y = np.empty((tokens.shape[0], d), np.float64)
    lib().oracle_combine(tokens.shape[0], _p(tokens), d, K, _p(y_perm), _p(token_row), _p(topk_w), _p(y))
    return y


def _selection(select, n, K, E):
    """A selection override: [n][K] distinct expert ids per row, in slot order (None: TopK's own)."""
    if select is None:
        return None
    s = _c(np.asarray(select).reshape(n, K), np.int32)
    assert ((s >= 0) & (s < E)).all(), "expert ids out of range"
    assert all(len(set(r)) == K for r in s.tolist()), "the K experts of a token must be distinct"
    return s


def forward(x, w_gate, w1, w3, w2, K, bias=None, tokens=None, threads=0, select=None):
    """Full layer on selected tokens. Returns dict(y, logits, idx, w) for those tokens.

    select [n][K] (optional): the experts each selected token keeps, in slot order, instead of the
    TopK by argmax; for tokens whose TopK is not unique (kept and dropped logits equal within the
    decision precision), so that the layer can be evaluated under another valid selection. The gates
    are then the softmax over the logits of the given experts."""
    x, w_gate, w1, w3, w2 = _c(x), _c(w_gate), _c(w1), _c(w3), _c(w2)
    bias = _c(bias, np.float32)
    T, d = x.shape
    E, F, _ = w1.shape
    dt = _dtype_code(x)
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    n = tokens.shape[0]
    sel = _selection(select, n, K, E)
    y = np.empty((n, d), np.float64)
    logits = np.empty((n, E), np.float64)
    idx = np.empty((n, K), np.int32)
    w = np.empty((n, K), np.float64)
    lib().oracle_forward(T, d, F, E, K, dt, _p(x), _p(w_gate), _p(bias), _p(w1), _p(w3), _p(w2), n, _p(tokens),
                         _p(sel), _p(y), _p(logits), _p(idx), _p(w), threads)
    return {"y": y, "logits": logits, "idx": idx, "w": w}


def rmsnorm_bf16(h, eps, want_exact=False):
    h = _c(h, np.float64)
    T, d = h.shape
    out = np.empty((T, d), np.uint16)
    ex = np.empty((T, d), np.float64) if want_exact else None
    lib().oracle_rmsnorm_bf16(T, d, float(eps), _p(h), _p(out), _p(ex))
    return (out, ex) if want_exact else out


def deep_layer(h, w_gate, w1, w3, w2, K, eps, bias=None, threads=0):
    """In place on h [n][d] float64: h <- h + MoE(bf16(rmsnorm(h))). Returns (idx, logits)."""
    assert h.dtype == np.float64 and h.flags.c_contiguous
    w_gate, w1, w3, w2 = _c(w_gate), _c(w1), _c(w3), _c(w2)
    bias = _c(bias, np.float32)
    n, d = h.shape
    E, F, _ = w1.shape
    idx = np.empty((n, K), np.int32)
    logits = np.empty((n, E), np.float64)
    lib().oracle_deep_layer(n, d, F, E, K, float(eps), _p(h), _p(w_gate), _p(bias), _p(w1), _p(w3), _p(w2),
                            _p(idx), _p(logits), threads)
    return idx, logits


# ----------------------------------------------------------------------------- backward pass
# The pages define the forward layer only; the gradient follows from it by the chain rule with
# the TopK selection held fixed (formulas in oracle.cpp). Gates come from the unrounded logits.

def _layer_args(x, w_gate, w1, w3, w2, bias):
    x, w_gate, w1, w3, w2 = _c(x), _c(w_gate), _c(w1), _c(w3), _c(w2)
    dt = _dtype_code(x)
    for a in (w_gate, w1, w3, w2):
        assert _dtype_code(a) == dt
    T, d = x.shape
    E, F, _ = w1.shape
    assert w_gate.shape == (d, E) and w3.shape == (E, F, d) and w2.shape == (E, d, F)
    return x, w_gate, w1, w3, w2, _c(bias, np.float32), T, d, F, E, dt


def forward_exact(x, w_gate, w1, w3, w2, K, bias=None, tokens=None):
    """Forward with unrounded double logits (the function the backward differentiates).
    Returns (y [n][d], idx [n][K])."""
    x, w_gate, w1, w3, w2, bias, T, d, F, E, dt = _layer_args(x, w_gate, w1, w3, w2, bias)
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    n = tokens.shape[0]
    y = np.empty((n, d), np.float64)
    idx = np.empty((n, K), np.int32)
    lib().oracle_forward_exact(d, F, E, K, dt, _p(x), _p(w_gate), _p(bias), _p(w1), _p(w3), _p(w2), n,
                               _p(tokens), _p(y), _p(idx))
    return y, idx


def backward(x, w_gate, w1, w3, w2, K, dy, bias=None):
    """Full backward (small shapes). Returns dict(dx, dlogits, dw_gate, dw1, dw3, dw2), float64."""
    x, w_gate, w1, w3, w2, bias, T, d, F, E, dt = _layer_args(x, w_gate, w1, w3, w2, bias)
    dy = _c(dy, np.float64)
    assert dy.shape == (T, d)
    out = {"dx": np.empty((T, d)), "dlogits": np.empty((T, E)), "dw_gate": np.empty((d, E)),
           "dw1": np.empty((E, F, d)), "dw3": np.empty((E, F, d)), "dw2": np.empty((E, d, F))}
    lib().oracle_backward(T, d, F, E, K, dt, _p(x), _p(w_gate), _p(bias), _p(w1), _p(w3), _p(w2), _p(dy),
                          _p(out["dx"]), _p(out["dlogits"]), _p(out["dw_gate"]), _p(out["dw1"]), _p(out["dw3"]),
                          _p(out["dw2"]))
    return out


def backward_tokens(x, w_gate, w1, w3, w2, K, dy, tokens, bias=None, threads=0):
    """dx and dlogits of selected tokens: (dx [n][d], dlogits [n][E]), float64."""
    x, w_gate, w1, w3, w2, bias, T, d, F, E, dt = _layer_args(x, w_gate, w1, w3, w2, bias)
    dy = _c(dy, np.float64)
    tokens = _c(tokens, np.int64)
    n = tokens.shape[0]
    dx = np.empty((n, d))
    dl = np.empty((n, E))
    lib().oracle_backward_tokens(d, F, E, K, dt, _p(x), _p(w_gate), _p(bias), _p(w1), _p(w3), _p(w2), _p(dy), n,
                                 _p(tokens), _p(dx), _p(dl), threads)
    return dx, dl


def backward_wsample(x, w_gate, w1, w3, w2, K, dy, queries, bias=None, threads=0):
    """Single weight-gradient entries. queries: int array [n][4] of (which, e, i, j) with which 1 (dw1[e][i][j]),
    3 (dw3[e][i][j]) or 2 (dw2[e][i][j]). Returns float64 [n]."""
    x, w_gate, w1, w3, w2, bias, T, d, F, E, dt = _layer_args(x, w_gate, w1, w3, w2, bias)
    dy = _c(dy, np.float64)
    q = _c(np.asarray(queries).reshape(-1, 4), np.int32)
    val = np.empty(q.shape[0])
    lib().oracle_backward_wsample(T, d, F, E, K, dt, _p(x), _p(w_gate), _p(bias), _p(w1), _p(w3), _p(w2), _p(dy),
                                  q.shape[0], _p(q), _p(val), threads)
    return val


# ----------------------------------------------------------------------------- decoder block
# The block around the MoE layer (formulas and readings in oracle.cpp): pre-norm residual,
# grouped-query causal attention with rotary positions, then the MoE sub-block.

def rope(x, n_heads, D, base, p0=0):
    """Rotary embedding of rows x [T][n_heads*D] at positions p0..p0+T-1. Returns float64."""
    x = _c(x)
    T = x.shape[0]
    assert x.shape[1] == n_heads * D and D % 2 == 0
    out = np.empty((T, n_heads * D), np.float64)
    lib().oracle_rope(T, n_heads, D, float(base), int(p0), _dtype_code(x), _p(x), _p(out))
    return out


def attention(q, k, v, Hq, Hkv, tokens=None, threads=0):
    """Causal grouped-query attention. q [T][Hq*D], k, v [T][Hkv*D] (same storage dtype),
    positions 0..T-1. Returns out [n][Hq*D] float64 for the selected positions."""
    q, k, v = _c(q), _c(k), _c(v)
    T = q.shape[0]
    D = q.shape[1] // Hq
    dt = _dtype_code(q)
    assert q.shape == (T, Hq * D) and k.shape == (T, Hkv * D) and v.shape == (T, Hkv * D) and Hq % Hkv == 0
    assert _dtype_code(k) == dt and _dtype_code(v) == dt
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    out = np.empty((tokens.shape[0], Hq * D), np.float64)
    lib().oracle_attention(T, Hq, Hkv, D, dt, _p(q), _p(k), _p(v), tokens.shape[0], _p(tokens), _p(out), threads)
    return out


def block(h, w_qkv, w_o, w_gate, w1, w3, w2, K, Hq, Hkv, base, eps, tokens=None, bias=None, threads=0,
          select=None):
    """One decoder block of a single sequence. h [T][d] float64 (residual stream in), weights as
    bf16 bit patterns: w_qkv [(Hq+2Hkv)*D][d], w_o [d][Hq*D], MoE weights as in forward().
    select: a selection override for the MoE sub-block of the selected tokens, as in forward().
    Returns dict(h1, x2, h2, idx, logits) for the selected tokens."""
    h = _c(h, np.float64)
    w_qkv, w_o, w_gate, w1, w3, w2 = _c(w_qkv), _c(w_o), _c(w_gate), _c(w1), _c(w3), _c(w2)
    bias = _c(bias, np.float32)
    T, d = h.shape
    E, F, _ = w1.shape
    D = w_o.shape[1] // Hq
    for a in (w_qkv, w_o, w_gate, w1, w3, w2):
        assert a.dtype == np.uint16, "block weights are bf16 bit patterns"
    assert w_qkv.shape == ((Hq + 2 * Hkv) * D, d) and w_o.shape == (d, Hq * D) and Hq % Hkv == 0
    tokens = np.arange(T, dtype=np.int64) if tokens is None else _c(tokens, np.int64)
    n = tokens.shape[0]
    sel = _selection(select, n, K, E)
    out = {"h1": np.empty((n, d)), "x2": np.empty((n, d), np.uint16), "h2": np.empty((n, d)),
           "idx": np.empty((n, K), np.int32), "logits": np.empty((n, E))}
    lib().oracle_block(T, d, Hq, Hkv, D, F, E, K, float(base), float(eps), 1, _p(h), _p(w_qkv), _p(w_o),
                       _p(w_gate), _p(bias), _p(w1), _p(w3), _p(w2), n, _p(tokens), _p(sel), _p(out["h1"]),
                       _p(out["x2"]),
                       _p(out["h2"]), _p(out["idx"]), _p(out["logits"]), threads)
    return out

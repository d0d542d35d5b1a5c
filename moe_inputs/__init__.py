"""Seeded synthetic inputs shared by the HIP library's tests/bench and the CPU oracle.

This package holds no mixture-of-experts arithmetic. It turns a
(seed, layer, tensor id, element index) counter into Gaussian samples
(SplitMix64 + Box-Muller, implemented in ``gen.c``) and stores them as fp32 or
as bf16 bit patterns (``numpy.uint16``). Both sides of a parity test read the
very same bits.

The workloads follow the Mixtral 8x7B mixture-of-experts layer ("Mixtral of
Experts", arXiv 2401.04088): d=4096, expert hidden size 14336, n=8 experts,
top-2 routing (xyznot.com summary page, section "Método"). Distributions:
x ~ N(0,1); W_g, w1, w3 ~ N(0, 1/d); w2 ~ N(0, 1/F).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libmoe_inputs.so")

# tensor ids inside one layer
X, W_GATE, W1, W3, W2, H0, DY = 0, 1, 2, 3, 4, 5, 6
Q_IN, K_IN, V_IN, W_QKV, W_O = 7, 8, 9, 10, 11  # decoder block: attention inputs and weights


def build(force: bool = False) -> str:
    """Compile gen.c into libmoe_inputs.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, dbl, vp = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        L.gen_key.restype = u64
        L.gen_key.argtypes = [u64, u64, u64]
        L.gen_mix64.restype = u64
        L.gen_mix64.argtypes = [u64]
        L.gen_normal_f32.argtypes = [u64, u64, u64, dbl, vp]
        L.gen_normal_bf16.argtypes = [u64, u64, u64, dbl, vp]
        L.gen_uniform_int.argtypes = [u64, u64, u64, u64, vp]
        _lib = L
    return _lib


def key(seed: int, layer: int, tensor: int) -> int:
    return int(lib().gen_key(seed, layer, tensor))


def normal(k: int, shape, sigma: float, dtype: str, start: int = 0) -> np.ndarray:
    """Gaussian N(0, sigma^2) tensor; dtype 'f32' -> float32, 'bf16' -> uint16 bit patterns."""
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        lib().gen_normal_f32(k, start, n, float(sigma), out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        lib().gen_normal_bf16(k, start, n, float(sigma), out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def uniform_int(k: int, n: int, m: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int64)
    lib().gen_uniform_int(k, start, n, m, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


@dataclass(frozen=True)
class Workload:
    """One synthetic workload. Shapes follow the Mixtral expert layer."""
    name: str
    T: int
    d: int
    F: int
    E: int = 8
    K: int = 2
    dtype: str = "bf16"
    layers: int = 1
    skew_bias: bool = False
    eps: float = 1e-5
    seed: int = 1
    # decoder block around the layer (xyznot.com "Método": 32 heads, 8 key-value heads)
    n_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    rope_base: float = 1e6

    @property
    def sigma_in(self) -> float:       # W_g, w1, w3 ~ N(0, 1/d)
        return 1.0 / math.sqrt(self.d)

    @property
    def sigma_out(self) -> float:      # w2 ~ N(0, 1/F)
        return 1.0 / math.sqrt(self.F)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=64, d=128, F=256, dtype="f32", seed=101),
    "decode_T32": Workload("decode_T32", T=32, d=4096, F=14336, seed=202),
    "prefill_T4096": Workload("prefill_T4096", T=4096, d=4096, F=14336, seed=303),
    "skewed_T16384": Workload("skewed_T16384", T=16384, d=4096, F=14336, skew_bias=True, seed=404),
    "deep32_T2048": Workload("deep32_T2048", T=2048, d=4096, F=14336, layers=32, seed=505),
    # one decoder block (attention + the layer) over a single sequence
    "block_T4096": Workload("block_T4096", T=4096, d=4096, F=14336, seed=606),
    "block_T32768": Workload("block_T32768", T=32768, d=4096, F=14336, seed=707),
}


def skew_bias(E: int) -> np.ndarray:
    """Fixed router bias b_e = 1.5 * ln(1/(e+1)) (natural log), fp32."""
    return np.array([1.5 * math.log(1.0 / (e + 1)) for e in range(E)], dtype=np.float32)


def layer_weights(w: Workload, layer: int = 0, experts=None) -> dict:
    """w_gate [d][E], w1/w3 [E][F][d], w2 [E][d][F] for one layer (dtype bits)."""
    s = w.seed
    out = {
        "w_gate": normal(key(s, layer, W_GATE), (w.d, w.E), w.sigma_in, w.dtype),
        "w1": normal(key(s, layer, W1), (w.E, w.F, w.d), w.sigma_in, w.dtype),
        "w3": normal(key(s, layer, W3), (w.E, w.F, w.d), w.sigma_in, w.dtype),
        "w2": normal(key(s, layer, W2), (w.E, w.d, w.F), w.sigma_out, w.dtype),
    }
    out["bias"] = skew_bias(w.E) if w.skew_bias else None
    return out


def block_weights(w: Workload, layer: int = 0) -> dict:
    """Attention weights of a decoder block (bf16 bits): w_qkv [(Hq + 2 Hkv) * D][d] ~ N(0, 1/d)
    (rows: the query heads, then the key heads, then the value heads), w_o [d][Hq * D] ~ N(0, 1/(Hq D))."""
    s, D = w.seed, w.head_dim
    hd = w.n_heads * D
    return {
        "w_qkv": normal(key(s, layer, W_QKV), ((w.n_heads + 2 * w.n_kv_heads) * D, w.d), 1.0 / math.sqrt(w.d), "bf16"),
        "w_o": normal(key(s, layer, W_O), (w.d, hd), 1.0 / math.sqrt(hd), "bf16"),
    }


def attention_inputs(w: Workload) -> dict:
    """Token-major attention inputs ~ N(0,1), bf16 bits: q [T][Hq * D], k, v [T][Hkv * D]."""
    s, D = w.seed, w.head_dim
    return {
        "q": normal(key(s, 0, Q_IN), (w.T, w.n_heads * D), 1.0, "bf16"),
        "k": normal(key(s, 0, K_IN), (w.T, w.n_kv_heads * D), 1.0, "bf16"),
        "v": normal(key(s, 0, V_IN), (w.T, w.n_kv_heads * D), 1.0, "bf16"),
    }


def tokens(w: Workload) -> np.ndarray:
    """x [T][d] ~ N(0,1) in the workload's dtype (layer-0 input of a single layer)."""
    return normal(key(w.seed, 0, X), (w.T, w.d), 1.0, w.dtype)


def residual0(w: Workload) -> np.ndarray:
    """Initial residual stream h_0 [T][d] ~ N(0,1), fp32 (deep stack)."""
    return normal(key(w.seed, 0, H0), (w.T, w.d), 1.0, "f32")


def upstream_grad(w: Workload) -> np.ndarray:
    """dy [T][d] ~ N(0,1), fp32: the gradient of a loss with respect to the layer output (backward pass)."""
    return normal(key(w.seed, 0, DY), (w.T, w.d), 1.0, "f32")


def synthetic_routing(seed: int, T: int, E: int, K: int, skew: float = 0.0) -> np.ndarray:
    """topk_idx [T][K] int32: K distinct experts per token drawn from the counter stream.

    skew > 0 biases draws toward low expert ids (u**(1+skew)), giving unequal groups.
    """
    u = uniform_int(key(seed, 0, 90), T * E, 1 << 30).reshape(T, E).astype(np.float64) / float(1 << 30)
    if skew > 0:
        score = -(u ** (1.0 + skew)) - np.arange(E)[None, :] * skew * 0.05
    else:
        score = u
    idx = np.argsort(-score, axis=1, kind="stable")[:, :K]
    return np.ascontiguousarray(idx.astype(np.int32))

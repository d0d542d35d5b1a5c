/*
 * CPU oracle for the sparse mixture-of-experts layer of Mixtral 8x7B.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or load
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header or table with the HIP library.
 *
 * It is the plain definition written out, in double precision, one token at a
 * time, with loops a reader can check against the pages by eye:
 *
 *   logits      l = x . W_g, W_g in R^{d x n}                ("Mixtral of Experts"
 *               blog on blog.csdn.net, section 2.1; xyznot.com summary, "Método")
 *   TopK        keep the K largest logits, the others become -inf
 *               (csdn blog section 2.2; xyznot.com "Método"; K = 2)
 *   Softmax     over the kept logits, so the K weights sum to 1 and the
 *               others are exactly 0 (csdn blog sections 2.3 and 2.4, with the
 *               worked form for two selected experts)
 *   Output      y = sum_i G(x)_i * E_i(x) (csdn blog section 1; xyznot.com
 *               "Método"); only the K selected experts are evaluated, because
 *               an expert with gate 0 adds nothing (ja.news.hada.io summary)
 *   Expert      SwiGLU feed-forward block with hidden size 14336
 *               (xyznot.com "Método" and "Términos clave": Swish times an
 *               elementwise product), read as w2 . (silu(w1 . x) * (w3 . x)),
 *               silu(z) = z / (1 + exp(-z)), no biases.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - ties in TopK go to the lower expert index; slot 0 holds the larger logit;
 *   - the TopK decision is taken on logits rounded to fp32, the precision the
 *     GPU kernel decides in; the sums themselves are exact-order double;
 *   - rows of one expert group are ordered by ascending token index;
 *   - the deep-stack layer is h <- h + MoE(bf16(h / sqrt(mean(h^2) + eps)))
 *     with a unit norm weight (the pages do not describe a norm);
 *   - TopK keeps "the K largest values" (csdn blog section 2.2), which names no
 *     single answer when kept and dropped logits are equal within the precision
 *     the decision is taken in. Any K experts whose logits are all at least as
 *     large as every dropped one then satisfy the definition. For those tokens
 *     the forward and block entry points accept a selection override: the given
 *     K experts, in the given slot order, replace the argmax choice, and the
 *     gates are the softmax over their logits, exactly as for a chosen set. The
 *     rest of the computation is unchanged, so passing the oracle's own
 *     selection reproduces its result bit for bit.
 *
 * Storage types of inputs: dtype 0 = fp32, dtype 1 = bf16 bit patterns, dtype 2 =
 * fp64 (used by the finite-difference checks of the backward pass). A bf16 value
 * is widened exactly (its 16 bits become the top half of an fp32).
 *
 * Backward pass. The pages define only the forward layer; its gradient follows
 * from that definition by the chain rule, with the TopK selection held fixed
 * (it is piecewise constant in the inputs). For a token t with kept experts
 * e_k, gates g_k and an upstream gradient dy_t:
 *   o_k = w2[e_k] . h_k, h_k = silu(a_k) * b_k, a_k = w1[e_k] . x, b_k = w3[e_k] . x
 *   dg_k = dy_t . o_k;  d logit_{e_k} = g_k (dg_k - sum_j g_j dg_j)   (softmax over the kept logits)
 *   do_k = g_k dy_t;  dh_k = w2[e_k]^T do_k
 *   da_k = dh_k * b_k * silu'(a_k),  db_k = dh_k * silu(a_k),  silu'(z) = s(z) (1 + z (1 - s(z)))
 *   dx_t = sum_k (w1[e_k]^T da_k + w3[e_k]^T db_k) + W_g . d logit_t
 *   dw2[e_k] += do_k h_k^T,  dw1[e_k] += da_k x^T,  dw3[e_k] += db_k x^T,  dW_g += x d logit_t^T
 * The gates of the backward come from the unrounded double logits (the forward
 * above uses fp32-rounded ones, a difference of ~1e-7 relative); the TopK
 * decision is taken on fp32-rounded logits in both.
 *
 * Decoder block. The pages give the surrounding transformer only as numbers
 * (xyznot.com summary, "Método": 32 layers, model width 4096, 32 attention
 * heads, 8 key-value heads; Mixtral keeps the Mistral 7B architecture and swaps
 * each feed-forward sub-block for the MoE layer; a full 32k-token context). The
 * block is read as the pre-norm residual form of that family:
 *   u  = bf16(h / sqrt(mean(h^2) + eps))                      (unit norm weight, as above)
 *   q, k, v = u . Wq^T, u . Wk^T, u . Wv^T                     (no biases; W_qkv stacks the three)
 *   rotary position embedding on q and k: in each head of width D, the pair (i, i + D/2)
 *   of position p is turned by the angle p * base^(-2i/D)
 *   per query head hq, with key-value head hq / (Hq/Hkv): causal softmax attention
 *   o_t = sum_{j<=t} softmax_j(q_t . k_j / sqrt(D)) v_j
 *   h1 = h + o . Wo^T;   h2 = h1 + MoE(bf16(h1 / sqrt(mean(h1^2) + eps)))
 * Head width D = 4096/32 = 128 follows from the numbers; the rotary base and the
 * pair convention are readings (the pages name no position encoding).
 */
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

double load(const void* p, int dtype, int64_t i) {
  if (dtype == 0) return (double)static_cast<const float*>(p)[i];
  if (dtype == 2) return static_cast<const double*>(p)[i];
  uint32_t bits = (uint32_t)static_cast<const uint16_t*>(p)[i] << 16;
  float f;
  std::memcpy(&f, &bits, 4);
  return (double)f;
}

uint16_t round_to_bf16(double v) {
  // double -> fp32 (round to nearest even) -> bf16 (round to nearest even)
  float f = (float)v;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if (std::isnan(f)) return 0x7FC0;
  uint32_t rounding = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + rounding) >> 16);
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

int pick_threads(int threads) {
  if (threads > 0) return threads;
  unsigned h = std::thread::hardware_concurrency();
  return h ? (int)h : 1;
}

// Runs body(i) for i in [0, n) on `threads` workers, each taking a contiguous block.
template <class F>
void parallel_for(int64_t n, int threads, F body) {
  int nt = (int)std::min<int64_t>(pick_threads(threads), std::max<int64_t>(n, 1));
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) body(i);
    return;
  }
  std::vector<std::thread> pool;
  for (int w = 0; w < nt; ++w) {
    int64_t lo = n * w / nt, hi = n * (w + 1) / nt;
    pool.emplace_back([=, &body]() { for (int64_t i = lo; i < hi; ++i) body(i); });
  }
  for (auto& t : pool) t.join();
}

// Router for one token: logits, TopK by repeated argmax on the fp32-rounded logits, softmax of
// the kept ones. round_logits: the returned logits (and so the gates) are the fp32-rounded values
// (forward) or the unrounded double sums (backward and its finite-difference checks). forced
// (nullable, K distinct expert ids): the selection to keep instead of the argmax choice, in slot
// order (the override for tokens whose TopK is not unique; see the header).
void route_token(int d, int E, int K, int dtype, const void* x, int64_t t, const void* w_gate,
                 const float* bias, double* logits, int32_t* idx, double* w, bool round_logits = true,
                 const int32_t* forced = nullptr) {
  std::vector<double> decide(E);
  for (int e = 0; e < E; ++e) {
    double s = 0.0;
    for (int k = 0; k < d; ++k) s += load(x, dtype, t * d + k) * load(w_gate, dtype, (int64_t)k * E + e);
    if (bias) s += (double)bias[e];
    decide[e] = (double)(float)s;
    logits[e] = round_logits ? decide[e] : s;
  }
  std::vector<char> taken(E, 0);
  for (int j = 0; j < K; ++j) {
    int best = -1;
    if (forced) {
      best = forced[j];
    } else {
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || decide[e] > decide[best])) best = e;
    }
    taken[best] = 1;
    idx[j] = best;
  }
  // Softmax over TopK(l): entries set to -inf contribute exp(-inf) = 0, so only the kept ones remain.
  double m = logits[idx[0]];
  double z = 0.0;
  for (int j = 0; j < K; ++j) z += std::exp(logits[idx[j]] - m);
  for (int j = 0; j < K; ++j) w[j] = std::exp(logits[idx[j]] - m) / z;
}

// One expert applied to one d-vector: out = w2[e] . (silu(w1[e] . v) * (w3[e] . v)).
void expert_apply(int d, int F, int e, int dtype, const void* v, int64_t v_off, int v_dtype,
                  const void* w1, const void* w3, const void* w2, double* hid, double* out) {
  const int64_t base13 = (int64_t)e * F * d;
  for (int f = 0; f < F; ++f) {
    double a = 0.0, b = 0.0;
    for (int k = 0; k < d; ++k) {
      double xv = load(v, v_dtype, v_off + k);
      a += load(w1, dtype, base13 + (int64_t)f * d + k) * xv;
      b += load(w3, dtype, base13 + (int64_t)f * d + k) * xv;
    }
    hid[f] = silu(a) * b;
  }
  const int64_t base2 = (int64_t)e * d * F;
  for (int n = 0; n < d; ++n) {
    double s = 0.0;
    for (int f = 0; f < F; ++f) s += load(w2, dtype, base2 + (int64_t)n * F + f) * hid[f];
    out[n] = s;
  }
}

double dsilu(double z) {
  const double s = 1.0 / (1.0 + std::exp(-z));
  return s * (1.0 + z * (1.0 - s));
}

// Pieces of one kept (token, expert) pair that the backward needs, in double:
// a = w1[e].x, b = w3[e].x (F-vectors) and, given the slot's output gradient do_k, dh = w2[e]^T do_k.
void pair_hidden(int d, int F, int e, int dtype, const void* x, int64_t t, const void* w1, const void* w3,
                 double* a, double* b) {
  const int64_t base13 = (int64_t)e * F * d;
  for (int f = 0; f < F; ++f) {
    double sa = 0.0, sb = 0.0;
    for (int k = 0; k < d; ++k) {
      double xv = load(x, dtype, t * d + k);
      sa += load(w1, dtype, base13 + (int64_t)f * d + k) * xv;
      sb += load(w3, dtype, base13 + (int64_t)f * d + k) * xv;
    }
    a[f] = sa;
    b[f] = sb;
  }
}

// Backward of one token (formulas in the header). Adds its contributions to dx_t [d] and
// dlog_t [E] (both zeroed here) and, when the pointers are non-null, to the weight gradients
// dwg [d][E], dw1/dw3 [E][F][d], dw2 [E][d][F].
void token_backward(int d, int F, int E, int K, int dtype, const void* x, int64_t t, const void* w_gate,
                    const float* bias, const void* w1, const void* w3, const void* w2, const double* dy_t,
                    double* dx_t, double* dlog_t, double* dwg, double* dw1, double* dw3, double* dw2) {
  std::vector<double> logits(E), g(K), dg(K), a(F), b(F), h(F), dh(F), da(F), db(F), o(d);
  std::vector<int32_t> idx(K);
  route_token(d, E, K, dtype, x, t, w_gate, bias, logits.data(), idx.data(), g.data(), false);
  for (int j = 0; j < d; ++j) dx_t[j] = 0.0;
  for (int e = 0; e < E; ++e) dlog_t[e] = 0.0;
  for (int k = 0; k < K; ++k) {
    const int e = idx[k];
    const int64_t base13 = (int64_t)e * F * d, base2 = (int64_t)e * d * F;
    pair_hidden(d, F, e, dtype, x, t, w1, w3, a.data(), b.data());
    for (int f = 0; f < F; ++f) h[f] = silu(a[f]) * b[f];
    // o = w2[e] . h and dg_k = dy . o
    double s_dg = 0.0;
    for (int n = 0; n < d; ++n) {
      double s = 0.0;
      for (int f = 0; f < F; ++f) s += load(w2, dtype, base2 + (int64_t)n * F + f) * h[f];
      o[n] = s;
      s_dg += dy_t[n] * s;
    }
    dg[k] = s_dg;
    // dh = w2[e]^T (g_k dy)
    for (int f = 0; f < F; ++f) {
      double s = 0.0;
      for (int n = 0; n < d; ++n) s += load(w2, dtype, base2 + (int64_t)n * F + f) * g[k] * dy_t[n];
      dh[f] = s;
      da[f] = dh[f] * b[f] * dsilu(a[f]);
      db[f] = dh[f] * silu(a[f]);
    }
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int f = 0; f < F; ++f)
        s += load(w1, dtype, base13 + (int64_t)f * d + j) * da[f] + load(w3, dtype, base13 + (int64_t)f * d + j) * db[f];
      dx_t[j] += s;
    }
    if (dw2)
      for (int n = 0; n < d; ++n)
        for (int f = 0; f < F; ++f) dw2[base2 + (int64_t)n * F + f] += g[k] * dy_t[n] * h[f];
    if (dw1)
      for (int f = 0; f < F; ++f)
        for (int j = 0; j < d; ++j) {
          const double xv = load(x, dtype, t * d + j);
          dw1[base13 + (int64_t)f * d + j] += da[f] * xv;
          dw3[base13 + (int64_t)f * d + j] += db[f] * xv;
        }
  }
  // softmax over the kept logits: d logit_{e_k} = g_k (dg_k - sum_j g_j dg_j)
  double gdg = 0.0;
  for (int k = 0; k < K; ++k) gdg += g[k] * dg[k];
  for (int k = 0; k < K; ++k) dlog_t[idx[k]] = g[k] * (dg[k] - gdg);
  for (int j = 0; j < d; ++j) {
    double s = 0.0;
    for (int e = 0; e < E; ++e) s += load(w_gate, dtype, (int64_t)j * E + e) * dlog_t[e];
    dx_t[j] += s;
    if (dwg)
      for (int e = 0; e < E; ++e) dwg[(int64_t)j * E + e] += load(x, dtype, t * d + j) * dlog_t[e];
  }
}

}  // namespace

extern "C" {

int oracle_abi_version() { return 2; }

// logits [T][E] (double holding fp32-rounded values), topk_idx [T][K], topk_w [T][K].
void oracle_route(int64_t T, int d, int E, int K, int dtype, const void* x, const void* w_gate,
                  const float* bias, double* logits, int32_t* topk_idx, double* topk_w, int threads) {
  parallel_for(T, threads, [&](int64_t t) {
    route_token(d, E, K, dtype, x, t, w_gate, bias, logits + t * E, topk_idx + t * K, topk_w + t * K);
  });
}

// Per-expert counts, exclusive-scan offsets [E+1], and the stable expert-contiguous order:
// row_token[row] = token, token_row[t*K + k] = row. Rows of one expert follow ascending token index.
void oracle_permute(int64_t T, int E, int K, const int32_t* topk_idx, int32_t* counts,
                    int32_t* offsets, int32_t* row_token, int32_t* token_row) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t s = 0; s < T * K; ++s) counts[topk_idx[s]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> next(offsets, offsets + E);
  for (int64_t t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      int e = topk_idx[t * K + k];
      int32_t row = next[e]++;
      row_token[row] = (int32_t)t;
      token_row[t * K + k] = row;
    }
}

// x_perm[row] = x[row_token[row]] (byte copy of whole rows).
void oracle_gather(int64_t rows, int64_t row_bytes, const void* x, const int32_t* row_token, void* x_perm) {
  for (int64_t r = 0; r < rows; ++r)
    std::memcpy((char*)x_perm + r * row_bytes, (const char*)x + (int64_t)row_token[r] * row_bytes, row_bytes);
}

// Expert FFN over expert-contiguous rows: for the selected rows, y_sel[i] = Expert_e(x_perm[rows_sel[i]])
// with e the group that holds that row. h_sel (nullable) receives the hidden vector [n_sel][F].
void oracle_expert_ffn(int d, int F, int E, int dtype, const void* x_perm, const int32_t* offsets,
                       const void* w1, const void* w3, const void* w2, int64_t n_sel,
                       const int64_t* rows_sel, double* h_sel, double* y_sel, int threads) {
  parallel_for(n_sel, threads, [&](int64_t i) {
    int64_t r = rows_sel[i];
    int e = 0;
    while (e < E - 1 && r >= offsets[e + 1]) ++e;
    std::vector<double> hid(F);
    expert_apply(d, F, e, dtype, x_perm, r * d, dtype, w1, w3, w2, hid.data(), y_sel + i * d);
    if (h_sel) std::copy(hid.begin(), hid.end(), h_sel + i * F);
  });
}

// y[t] = sum_k topk_w[t][k] * y_perm[token_row[t][k]] for the selected tokens, slot order.
void oracle_combine(int64_t n_sel, const int64_t* tok_sel, int d, int K, const float* y_perm,
                    const int32_t* token_row, const float* topk_w, double* y) {
  for (int64_t i = 0; i < n_sel; ++i) {
    int64_t t = tok_sel[i];
    for (int n = 0; n < d; ++n) {
      double s = 0.0;
      for (int k = 0; k < K; ++k)
        s += (double)topk_w[t * K + k] * (double)y_perm[(int64_t)token_row[t * K + k] * d + n];
      y[i * d + n] = s;
    }
  }
}

// Whole layer for selected tokens (tokens are independent): y_sel [n_sel][d];
// also returns each selected token's logits [n_sel][E], topk_idx [n_sel][K], topk_w [n_sel][K].
// sel_in [n_sel][K] (nullable): a selection override per selected token (see the header).
void oracle_forward(int64_t T, int d, int F, int E, int K, int dtype, const void* x, const void* w_gate,
                    const float* bias, const void* w1, const void* w3, const void* w2, int64_t n_sel,
                    const int64_t* tok_sel, const int32_t* sel_in, double* y_sel, double* logits_sel,
                    int32_t* idx_sel, double* w_sel, int threads) {
  (void)T;
  for (int64_t i = 0; i < n_sel; ++i)
    route_token(d, E, K, dtype, x, tok_sel[i], w_gate, bias, logits_sel + i * E, idx_sel + i * K, w_sel + i * K,
                true, sel_in ? sel_in + i * K : nullptr);
  std::vector<double> outs((size_t)n_sel * K * d);
  parallel_for(n_sel * K, threads, [&](int64_t u) {
    int64_t i = u / K;
    int k = (int)(u % K);
    std::vector<double> hid(F);
    expert_apply(d, F, idx_sel[i * K + k], dtype, x, tok_sel[i] * d, dtype, w1, w3, w2, hid.data(),
                 outs.data() + (size_t)u * d);
  });
  for (int64_t i = 0; i < n_sel; ++i)
    for (int n = 0; n < d; ++n) {
      double s = 0.0;
      for (int k = 0; k < K; ++k) s += w_sel[i * K + k] * outs[((size_t)i * K + k) * d + n];
      y_sel[i * d + n] = s;
    }
}

// x = bf16(h / sqrt(mean(h^2) + eps)) per row (unit norm weight). x_exact (nullable) gets the unrounded value.
void oracle_rmsnorm_bf16(int64_t T, int d, double eps, const double* h, uint16_t* x_bf16, double* x_exact) {
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int k = 0; k < d; ++k) ss += h[t * d + k] * h[t * d + k];
    double inv = 1.0 / std::sqrt(ss / d + eps);
    for (int k = 0; k < d; ++k) {
      double v = h[t * d + k] * inv;
      if (x_exact) x_exact[t * d + k] = v;
      x_bf16[t * d + k] = round_to_bf16(v);
    }
  }
}

// One deep-stack layer on n rows of the residual stream (double, in place):
// x = bf16(rmsnorm(h)); h <- h + MoE(x). idx_out [n][K] and logits_out [n][E] report the routing.
void oracle_deep_layer(int64_t n, int d, int F, int E, int K, double eps, double* h, const void* w_gate,
                       const float* bias, const void* w1, const void* w3, const void* w2,
                       int32_t* idx_out, double* logits_out, int threads) {
  std::vector<uint16_t> x((size_t)n * d);
  oracle_rmsnorm_bf16(n, d, eps, h, x.data(), nullptr);
  std::vector<int64_t> sel(n);
  for (int64_t i = 0; i < n; ++i) sel[i] = i;
  std::vector<double> y((size_t)n * d), w((size_t)n * K);
  oracle_forward(n, d, F, E, K, 1, x.data(), w_gate, bias, w1, w3, w2, n, sel.data(), nullptr, y.data(),
                 logits_out, idx_out, w.data(), threads);
  for (size_t i = 0; i < (size_t)n * d; ++i) h[i] += y[i];
}

// The forward above with unrounded double logits (gates from the exact logits, TopK decided on
// fp32-rounded ones): the function whose gradient the backward computes. y_sel [n_sel][d].
void oracle_forward_exact(int d, int F, int E, int K, int dtype, const void* x, const void* w_gate,
                          const float* bias, const void* w1, const void* w3, const void* w2, int64_t n_sel,
                          const int64_t* tok_sel, double* y_sel, int32_t* idx_sel) {
  std::vector<double> logits(E), g(K), hid(F), o(d);
  for (int64_t i = 0; i < n_sel; ++i) {
    route_token(d, E, K, dtype, x, tok_sel[i], w_gate, bias, logits.data(), idx_sel + i * K, g.data(), false);
    for (int n = 0; n < d; ++n) y_sel[i * d + n] = 0.0;
    for (int k = 0; k < K; ++k) {
      expert_apply(d, F, idx_sel[i * K + k], dtype, x, tok_sel[i] * d, dtype, w1, w3, w2, hid.data(), o.data());
      for (int n = 0; n < d; ++n) y_sel[i * d + n] += g[k] * o[n];
    }
  }
}

// Full backward over all T tokens (small shapes): dy [T][d] -> dx [T][d], dlogits [T][E],
// dwg [d][E], dw1, dw3 [E][F][d], dw2 [E][d][F]; all double, tokens accumulated in ascending order.
void oracle_backward(int64_t T, int d, int F, int E, int K, int dtype, const void* x, const void* w_gate,
                     const float* bias, const void* w1, const void* w3, const void* w2, const double* dy,
                     double* dx, double* dlogits, double* dwg, double* dw1, double* dw3, double* dw2) {
  std::fill(dwg, dwg + (int64_t)d * E, 0.0);
  std::fill(dw1, dw1 + (int64_t)E * F * d, 0.0);
  std::fill(dw3, dw3 + (int64_t)E * F * d, 0.0);
  std::fill(dw2, dw2 + (int64_t)E * d * F, 0.0);
  for (int64_t t = 0; t < T; ++t)
    token_backward(d, F, E, K, dtype, x, t, w_gate, bias, w1, w3, w2, dy + t * d, dx + t * d, dlogits + t * E,
                   dwg, dw1, dw3, dw2);
}

// Per-token part of the backward for selected tokens: dx_sel [n_sel][d], dlogits_sel [n_sel][E].
void oracle_backward_tokens(int d, int F, int E, int K, int dtype, const void* x, const void* w_gate,
                            const float* bias, const void* w1, const void* w3, const void* w2, const double* dy,
                            int64_t n_sel, const int64_t* tok_sel, double* dx_sel, double* dlogits_sel, int threads) {
  parallel_for(n_sel, threads, [&](int64_t i) {
    const int64_t t = tok_sel[i];
    token_backward(d, F, E, K, dtype, x, t, w_gate, bias, w1, w3, w2, dy + t * d, dx_sel + i * d,
                   dlogits_sel + i * E, nullptr, nullptr, nullptr, nullptr);
  });
}

// Single entries of the expert weight gradients, each summed over every (token, slot) routed to
// its expert: query q = (which, e, i, j) with which 1: dw1[e][i][j], 3: dw3[e][i][j] (i < F, j < d),
// 2: dw2[e][i][j] (i < d, j < F). val [n_q].
void oracle_backward_wsample(int64_t T, int d, int F, int E, int K, int dtype, const void* x, const void* w_gate,
                             const float* bias, const void* w1, const void* w3, const void* w2, const double* dy,
                             int64_t n_q, const int32_t* q, double* val, int threads) {
  std::vector<int32_t> idx((size_t)T * K);
  std::vector<double> g((size_t)T * K), logits((size_t)T * E);
  parallel_for(T, threads, [&](int64_t t) {
    route_token(d, E, K, dtype, x, t, w_gate, bias, logits.data() + t * E, idx.data() + t * K, g.data() + t * K,
                false);
  });
  parallel_for(n_q, threads, [&](int64_t u) {
    const int which = q[4 * u], e = q[4 * u + 1], i = q[4 * u + 2], j = q[4 * u + 3];
    const int64_t base13 = (int64_t)e * F * d, base2 = (int64_t)e * d * F;
    double acc = 0.0;
    for (int64_t t = 0; t < T; ++t)
      for (int k = 0; k < K; ++k) {
        if (idx[t * K + k] != e) continue;
        const double gk = g[t * K + k];
        const int f = which == 2 ? j : i;  // hidden unit of the entry
        double a = 0.0, b = 0.0;
        for (int m = 0; m < d; ++m) {
          const double xv = load(x, dtype, t * d + m);
          a += load(w1, dtype, base13 + (int64_t)f * d + m) * xv;
          b += load(w3, dtype, base13 + (int64_t)f * d + m) * xv;
        }
        if (which == 2) {
          acc += gk * dy[t * d + i] * silu(a) * b;  // do[i] * h[f]
          continue;
        }
        double dh = 0.0;
        for (int n = 0; n < d; ++n) dh += load(w2, dtype, base2 + (int64_t)n * F + f) * gk * dy[t * d + n];
        const double xj = load(x, dtype, t * d + j);
        acc += (which == 1 ? dh * b * dsilu(a) : dh * silu(a)) * xj;
      }
    val[u] = acc;
  });
}

// ----------------------------------------------------------------------------- decoder block

// Rotary position embedding, in place on one head vector x [D] at position p.
static void rope_head(double* x, int D, int64_t p, double base) {
  const int half = D / 2;
  for (int i = 0; i < half; ++i) {
    const double ang = (double)p * std::pow(base, -2.0 * i / D);
    const double c = std::cos(ang), sn = std::sin(ang);
    const double a = x[i], b = x[i + half];
    x[i] = a * c - b * sn;
    x[i + half] = a * sn + b * c;
  }
}

// RoPE of T rows of n_heads heads (row t = position p0 + t): in [T][n_heads*D] (storage dtype),
// out [T][n_heads*D] double.
void oracle_rope(int64_t T, int n_heads, int D, double base, int64_t p0, int dtype, const void* in, double* out) {
  const int64_t W = (int64_t)n_heads * D;
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < n_heads; ++h) {
      double* x = out + t * W + (int64_t)h * D;
      for (int i = 0; i < D; ++i) x[i] = load(in, dtype, t * W + (int64_t)h * D + i);
      rope_head(x, D, p0 + t, base);
    }
}

// Causal grouped-query attention for selected positions: q [T][Hq*D], k, v [T][Hkv*D] (storage
// dtype), query head hq reads key-value head hq / (Hq/Hkv); out [n_sel][Hq*D] double.
void oracle_attention(int64_t T, int Hq, int Hkv, int D, int dtype, const void* q, const void* k, const void* v,
                      int64_t n_sel, const int64_t* tok_sel, double* out, int threads) {
  (void)T;
  const int G = Hq / Hkv;
  const double scale = 1.0 / std::sqrt((double)D);
  parallel_for(n_sel * Hq, threads, [&](int64_t u) {
    const int64_t i = u / Hq, t = tok_sel[i];
    const int hq = (int)(u % Hq), hk = hq / G;
    std::vector<double> s(t + 1);
    double m = -INFINITY;
    for (int64_t j = 0; j <= t; ++j) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c)
        acc += load(q, dtype, t * Hq * D + (int64_t)hq * D + c) * load(k, dtype, j * Hkv * D + (int64_t)hk * D + c);
      s[j] = acc * scale;
      m = std::max(m, s[j]);
    }
    double z = 0.0;
    for (int64_t j = 0; j <= t; ++j) {
      s[j] = std::exp(s[j] - m);
      z += s[j];
    }
    double* o = out + i * Hq * D + (int64_t)hq * D;
    for (int c = 0; c < D; ++c) o[c] = 0.0;
    for (int64_t j = 0; j <= t; ++j) {
      const double p = s[j] / z;
      for (int c = 0; c < D; ++c) o[c] += p * load(v, dtype, j * Hkv * D + (int64_t)hk * D + c);
    }
  });
}

// One decoder block for selected tokens of a single sequence of T tokens (positions 0..T-1):
// h [T][d] double (the residual stream entering the block), w_qkv [(Hq+2Hkv)*D][d] and
// w_o [d][Hq*D] in storage dtype (bf16 or fp32, as the MoE weights). Returns for the selected
// tokens h1 [n_sel][d] (after attention), x2 [n_sel][d] (bf16 bits of the MoE input) and
// h2 [n_sel][d] (after the MoE), plus the routing of x2 (idx [n_sel][K], logits [n_sel][E]).
// Rows 0..max(tok_sel) are projected to keys and values, as causal attention needs them.
// sel_in [n_sel][K] (nullable): a selection override for the MoE sub-block (see the header).
void oracle_block(int64_t T, int d, int Hq, int Hkv, int D, int F, int E, int K, double base, double eps,
                  int dtype, const double* h, const void* w_qkv, const void* w_o, const void* w_gate,
                  const float* bias, const void* w1, const void* w3, const void* w2, int64_t n_sel,
                  const int64_t* tok_sel, const int32_t* sel_in, double* h1_sel, uint16_t* x2_sel, double* h2_sel,
                  int32_t* idx_sel,
                  double* logits_sel, int threads) {
  (void)T;
  int64_t n = 0;  // rows needed: 0..max selected position
  for (int64_t i = 0; i < n_sel; ++i) n = std::max<int64_t>(n, tok_sel[i] + 1);
  const int64_t Wq = (int64_t)Hq * D, Wk = (int64_t)Hkv * D;
  std::vector<uint16_t> u((size_t)n * d);
  oracle_rmsnorm_bf16(n, d, eps, h, u.data(), nullptr);
  // keys and values of every needed row, queries of the selected rows (double, after RoPE)
  std::vector<double> kk((size_t)n * Wk), vv((size_t)n * Wk), qq((size_t)n_sel * Wq);
  auto proj = [&](int64_t t, int64_t row0, int64_t nrows, double* dst) {
    for (int64_t r = 0; r < nrows; ++r) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += load(w_qkv, dtype, (row0 + r) * d + c) * load(u.data(), 1, t * d + c);
      dst[r] = acc;
    }
  };
  parallel_for(n, threads, [&](int64_t t) {
    proj(t, Wq, Wk, kk.data() + t * Wk);
    proj(t, Wq + Wk, Wk, vv.data() + t * Wk);
    for (int hk = 0; hk < Hkv; ++hk) rope_head(kk.data() + t * Wk + (int64_t)hk * D, D, t, base);
  });
  parallel_for(n_sel, threads, [&](int64_t i) {
    const int64_t t = tok_sel[i];
    proj(t, 0, Wq, qq.data() + i * Wq);
    for (int hq = 0; hq < Hq; ++hq) rope_head(qq.data() + i * Wq + (int64_t)hq * D, D, t, base);
  });
  // attention of the selected rows (queries stored compactly: pass positions through a remap)
  std::vector<double> o((size_t)n_sel * Wq);
  const int G = Hq / Hkv;
  const double scale = 1.0 / std::sqrt((double)D);
  parallel_for(n_sel * Hq, threads, [&](int64_t uu) {
    const int64_t i = uu / Hq, t = tok_sel[i];
    const int hq = (int)(uu % Hq), hk = hq / G;
    std::vector<double> s(t + 1);
    double m = -INFINITY;
    for (int64_t j = 0; j <= t; ++j) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += qq[i * Wq + (int64_t)hq * D + c] * kk[j * Wk + (int64_t)hk * D + c];
      s[j] = acc * scale;
      m = std::max(m, s[j]);
    }
    double z = 0.0;
    for (int64_t j = 0; j <= t; ++j) {
      s[j] = std::exp(s[j] - m);
      z += s[j];
    }
    double* oo = o.data() + i * Wq + (int64_t)hq * D;
    for (int c = 0; c < D; ++c) oo[c] = 0.0;
    for (int64_t j = 0; j <= t; ++j)
      for (int c = 0; c < D; ++c) oo[c] += s[j] / z * vv[j * Wk + (int64_t)hk * D + c];
  });
  // output projection and residual, then the MoE sub-block on the selected rows
  for (int64_t i = 0; i < n_sel; ++i)
    for (int r = 0; r < d; ++r) {
      double acc = 0.0;
      for (int64_t c = 0; c < Wq; ++c) acc += load(w_o, dtype, (int64_t)r * Wq + c) * o[i * Wq + c];
      h1_sel[i * d + r] = h[tok_sel[i] * d + r] + acc;
    }
  oracle_rmsnorm_bf16(n_sel, d, eps, h1_sel, x2_sel, nullptr);
  std::vector<int64_t> all(n_sel);
  for (int64_t i = 0; i < n_sel; ++i) all[i] = i;
  std::vector<double> y((size_t)n_sel * d), w((size_t)n_sel * K);
  oracle_forward(n_sel, d, F, E, K, 1, x2_sel, w_gate, bias, w1, w3, w2, n_sel, all.data(), sel_in, y.data(),
                 logits_sel, idx_sel, w.data(), threads);
  for (int64_t i = 0; i < n_sel * d; ++i) h2_sel[i] = h1_sel[i] + y[i];
}

}  // extern "C"

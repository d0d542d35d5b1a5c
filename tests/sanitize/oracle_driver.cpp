// Host driver for the sanitizer build of the CPU oracle and the seeded input generator: every
// oracle entry point on small shapes (fp32, bf16 and fp64 storage; K = 1, 2, 3; a router bias; a
// selection override), so that AddressSanitizer and UndefinedBehaviorSanitizer see every loop and
// index of both files. Prints "oracle driver ok" and exits 0 when every result is finite and the
// few cross-checks below hold; any sanitizer report aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

extern "C" {
uint64_t gen_key(uint64_t seed, uint64_t layer, uint64_t tensor);
void gen_normal_f32(uint64_t key, uint64_t start, uint64_t n, double sigma, float* out);
void gen_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double sigma, uint16_t* out);
void gen_uniform_int(uint64_t key, uint64_t start, uint64_t n, uint64_t m, int64_t* out);

int oracle_abi_version();
void oracle_route(int64_t T, int d, int E, int K, int dtype, const void* x, const void* w_gate, const float* bias,
                  double* logits, int32_t* topk_idx, double* topk_w, int threads);
void oracle_permute(int64_t T, int E, int K, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                    int32_t* row_token, int32_t* token_row);
void oracle_gather(int64_t rows, int64_t row_bytes, const void* x, const int32_t* row_token, void* x_perm);
void oracle_expert_ffn(int d, int F, int E, int dtype, const void* x_perm, const int32_t* offsets, const void* w1,
                       const void* w3, const void* w2, int64_t n_sel, const int64_t* rows_sel, double* h_sel,
                       double* y_sel, int threads);
void oracle_combine(int64_t n_sel, const int64_t* tok_sel, int d, int K, const float* y_perm,
                    const int32_t* token_row, const float* topk_w, double* y);
void oracle_forward(int64_t T, int d, int F, int E, int K, int dtype, const void* x, const void* w_gate,
                    const float* bias, const void* w1, const void* w3, const void* w2, int64_t n_sel,
                    const int64_t* tok_sel, const int32_t* sel_in, double* y_sel, double* logits_sel,
                    int32_t* idx_sel, double* w_sel, int threads);
void oracle_rmsnorm_bf16(int64_t T, int d, double eps, const double* h, uint16_t* x_bf16, double* x_exact);
void oracle_deep_layer(int64_t n, int d, int F, int E, int K, double eps, double* h, const void* w_gate,
                       const float* bias, const void* w1, const void* w3, const void* w2, int32_t* idx_out,
                       double* logits_out, int threads);
void oracle_forward_exact(int d, int F, int E, int K, int dtype, const void* x, const void* w_gate, const float* bias,
                          const void* w1, const void* w3, const void* w2, int64_t n_sel, const int64_t* tok_sel,
                          double* y_sel, int32_t* idx_sel);
void oracle_backward(int64_t T, int d, int F, int E, int K, int dtype, const void* x, const void* w_gate,
                     const float* bias, const void* w1, const void* w3, const void* w2, const double* dy, double* dx,
                     double* dlogits, double* dwg, double* dw1, double* dw3, double* dw2);
void oracle_backward_tokens(int d, int F, int E, int K, int dtype, const void* x, const void* w_gate,
                            const float* bias, const void* w1, const void* w3, const void* w2, const double* dy,
                            int64_t n_sel, const int64_t* tok_sel, double* dx_sel, double* dlogits_sel, int threads);
void oracle_backward_wsample(int64_t T, int d, int F, int E, int K, int dtype, const void* x, const void* w_gate,
                             const float* bias, const void* w1, const void* w3, const void* w2, const double* dy,
                             int64_t n_q, const int32_t* q, double* val, int threads);
void oracle_rope(int64_t T, int n_heads, int D, double base, int64_t p0, int dtype, const void* in, double* out);
void oracle_attention(int64_t T, int Hq, int Hkv, int D, int dtype, const void* q, const void* k, const void* v,
                      int64_t n_sel, const int64_t* tok_sel, double* out, int threads);
void oracle_block(int64_t T, int d, int Hq, int Hkv, int D, int F, int E, int K, double base, double eps, int dtype,
                  const double* h, const void* w_qkv, const void* w_o, const void* w_gate, const float* bias,
                  const void* w1, const void* w3, const void* w2, int64_t n_sel, const int64_t* tok_sel,
                  const int32_t* sel_in, double* h1_sel, uint16_t* x2_sel, double* h2_sel, int32_t* idx_sel,
                  double* logits_sel, int threads);
}

namespace {

int failures = 0;

void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

bool finite(const std::vector<double>& v) {
  for (double a : v)
    if (!std::isfinite(a)) return false;
  return true;
}

// Tensor storage in one of the oracle's dtypes: 0 fp32, 1 bf16 bits, 2 fp64.
struct Tensor {
  int dtype;
  std::vector<float> f;
  std::vector<uint16_t> b;
  std::vector<double> d;
  Tensor(int dt, uint64_t key, size_t n, double sigma) : dtype(dt) {
    if (dt == 1) {
      b.resize(n);
      gen_normal_bf16(key, 0, n, sigma, b.data());
    } else {
      f.resize(n);
      gen_normal_f32(key, 0, n, sigma, f.data());
      if (dt == 2) d.assign(f.begin(), f.end());
    }
  }
  const void* p() const { return dtype == 1 ? (const void*)b.data() : dtype == 2 ? (const void*)d.data() : f.data(); }
};

void layer_case(int dtype, int T, int d, int F, int E, int K, bool bias_on, uint64_t seed) {
  Tensor x(dtype, gen_key(seed, 0, 0), (size_t)T * d, 1.0);
  Tensor wg(dtype, gen_key(seed, 0, 1), (size_t)d * E, 1.0 / std::sqrt((double)d));
  Tensor w1(dtype, gen_key(seed, 0, 2), (size_t)E * F * d, 1.0 / std::sqrt((double)d));
  Tensor w3(dtype, gen_key(seed, 0, 3), (size_t)E * F * d, 1.0 / std::sqrt((double)d));
  Tensor w2(dtype, gen_key(seed, 0, 4), (size_t)E * d * F, 1.0 / std::sqrt((double)F));
  std::vector<float> bias(E);
  for (int e = 0; e < E; ++e) bias[e] = (float)(1.5 * std::log(1.0 / (e + 1)));
  const float* bp = bias_on ? bias.data() : nullptr;

  std::vector<double> logits((size_t)T * E), w((size_t)T * K);
  std::vector<int32_t> idx((size_t)T * K);
  oracle_route(T, d, E, K, dtype, x.p(), wg.p(), bp, logits.data(), idx.data(), w.data(), 3);
  require(finite(logits) && finite(w), "route finite");

  std::vector<int32_t> counts(E), offsets(E + 1), row_token((size_t)T * K), token_row((size_t)T * K);
  oracle_permute(T, E, K, idx.data(), counts.data(), offsets.data(), row_token.data(), token_row.data());
  require(offsets[E] == T * K, "offsets[E] = T K");

  if (dtype != 2) {
    const size_t es = dtype == 1 ? 2 : 4;
    std::vector<uint8_t> xp((size_t)T * K * d * es);
    oracle_gather((int64_t)T * K, (int64_t)d * es, x.p(), row_token.data(), xp.data());
    std::vector<int64_t> rows((size_t)T * K);
    for (size_t r = 0; r < rows.size(); ++r) rows[r] = (int64_t)r;
    std::vector<double> h((size_t)T * K * F), yp((size_t)T * K * d);
    oracle_expert_ffn(d, F, E, dtype, xp.data(), offsets.data(), w1.p(), w3.p(), w2.p(), (int64_t)rows.size(),
                      rows.data(), h.data(), yp.data(), 3);
    require(finite(h) && finite(yp), "expert ffn finite");
    std::vector<float> ypf(yp.begin(), yp.end()), wf(w.begin(), w.end());
    std::vector<int64_t> toks(T);
    for (int t = 0; t < T; ++t) toks[t] = t;
    std::vector<double> y((size_t)T * d), y2((size_t)T * d), lg((size_t)T * E), ws((size_t)T * K);
    oracle_combine(T, toks.data(), d, K, ypf.data(), token_row.data(), wf.data(), y.data());
    std::vector<int32_t> idx2((size_t)T * K);
    oracle_forward(T, d, F, E, K, dtype, x.p(), wg.p(), bp, w1.p(), w3.p(), w2.p(), T, toks.data(), nullptr,
                   y2.data(), lg.data(), idx2.data(), ws.data(), 3);
    double err = 0, mx = 0;
    for (size_t i = 0; i < y.size(); ++i) {
      err = std::max(err, std::fabs(y[i] - y2[i]));
      mx = std::max(mx, std::fabs(y2[i]));
    }
    require(err <= 1e-5 * mx, "stage pipeline equals forward");
    // a selection override: the experts ranked 2..K+1 (or the top one when K = E)
    std::vector<int32_t> sel((size_t)T * K);
    for (int t = 0; t < T; ++t)
      for (int k = 0; k < K; ++k) sel[(size_t)t * K + k] = idx2[(size_t)t * K + (k + 1) % K];
    oracle_forward(T, d, F, E, K, dtype, x.p(), wg.p(), bp, w1.p(), w3.p(), w2.p(), T, toks.data(), sel.data(),
                   y2.data(), lg.data(), idx2.data(), ws.data(), 3);
    require(finite(y2) && finite(ws), "forward under a selection override finite");
  }

  // backward pieces (fp64 storage is what the finite-difference checks use)
  std::vector<double> dy((size_t)T * d);
  {
    std::vector<float> tmp(dy.size());
    gen_normal_f32(gen_key(seed, 0, 6), 0, tmp.size(), 1.0, tmp.data());
    dy.assign(tmp.begin(), tmp.end());
  }
  std::vector<int64_t> toks(T);
  for (int t = 0; t < T; ++t) toks[t] = t;
  std::vector<double> ye((size_t)T * d);
  std::vector<int32_t> ie((size_t)T * K);
  oracle_forward_exact(d, F, E, K, dtype, x.p(), wg.p(), bp, w1.p(), w3.p(), w2.p(), T, toks.data(), ye.data(),
                       ie.data());
  std::vector<double> dx((size_t)T * d), dl((size_t)T * E), dwg((size_t)d * E), dw1((size_t)E * F * d),
      dw3((size_t)E * F * d), dw2((size_t)E * d * F);
  oracle_backward(T, d, F, E, K, dtype, x.p(), wg.p(), bp, w1.p(), w3.p(), w2.p(), dy.data(), dx.data(), dl.data(),
                  dwg.data(), dw1.data(), dw3.data(), dw2.data());
  require(finite(dx) && finite(dl) && finite(dw1) && finite(dw2), "backward finite");
  std::vector<double> dxs((size_t)2 * d), dls((size_t)2 * E);
  const int64_t two[2] = {0, T - 1};
  oracle_backward_tokens(d, F, E, K, dtype, x.p(), wg.p(), bp, w1.p(), w3.p(), w2.p(), dy.data(), 2, two, dxs.data(),
                         dls.data(), 2);
  for (int j = 0; j < d; ++j) require(std::fabs(dxs[d + j] - dx[(size_t)(T - 1) * d + j]) <= 1e-9, "dx of a token");
  const int32_t q[12] = {1, 0, 0, 0, 3, E - 1, F - 1, d - 1, 2, E / 2, d - 1, F - 1};
  double val[3];
  oracle_backward_wsample(T, d, F, E, K, dtype, x.p(), wg.p(), bp, w1.p(), w3.p(), w2.p(), dy.data(), 3, q, val, 2);
  const double dw2_last = dw2[(size_t)(E / 2) * d * F + (size_t)(d - 1) * F + F - 1];
  require(std::fabs(val[0] - dw1[0]) <= 1e-9 && std::fabs(val[2] - dw2_last) <= 1e-9, "weight-gradient samples");
}

void block_case(uint64_t seed) {
  const int T = 19, d = 64, Hq = 4, Hkv = 2, D = 16, F = 32, E = 4, K = 2;
  Tensor wqkv(1, gen_key(seed, 0, 10), (size_t)(Hq + 2 * Hkv) * D * d, 1.0 / 8);
  Tensor wo(1, gen_key(seed, 0, 11), (size_t)d * Hq * D, 1.0 / 8);
  Tensor wg(1, gen_key(seed, 0, 1), (size_t)d * E, 1.0 / 8);
  Tensor w1(1, gen_key(seed, 0, 2), (size_t)E * F * d, 1.0 / 8);
  Tensor w3(1, gen_key(seed, 0, 3), (size_t)E * F * d, 1.0 / 8);
  Tensor w2(1, gen_key(seed, 0, 4), (size_t)E * d * F, 1.0 / std::sqrt((double)F));
  std::vector<float> hf((size_t)T * d);
  gen_normal_f32(gen_key(seed, 0, 5), 0, hf.size(), 1.0, hf.data());
  std::vector<double> h(hf.begin(), hf.end());
  const int64_t sel[3] = {0, 7, T - 1};
  std::vector<double> h1(3 * d), h2(3 * d), lg(3 * E);
  std::vector<uint16_t> x2(3 * d);
  std::vector<int32_t> idx(3 * K);
  oracle_block(T, d, Hq, Hkv, D, F, E, K, 1e6, 1e-5, 1, h.data(), wqkv.p(), wo.p(), wg.p(), nullptr, w1.p(), w3.p(),
               w2.p(), 3, sel, nullptr, h1.data(), x2.data(), h2.data(), idx.data(), lg.data(), 2);
  require(finite(h1) && finite(h2), "block finite");
  std::vector<int32_t> other(3 * K);
  for (int i = 0; i < 3; ++i) {  // another valid selection: the two experts after the first kept one
    other[i * K] = (idx[i * K] + 1) % E;
    other[i * K + 1] = (idx[i * K] + 2) % E;
  }
  oracle_block(T, d, Hq, Hkv, D, F, E, K, 1e6, 1e-5, 1, h.data(), wqkv.p(), wo.p(), wg.p(), nullptr, w1.p(), w3.p(),
               w2.p(), 3, sel, other.data(), h1.data(), x2.data(), h2.data(), idx.data(), lg.data(), 2);
  require(finite(h2), "block under a selection override finite");

  std::vector<double> r((size_t)T * Hq * D);
  oracle_rope(T, Hq, D, 1e6, 3, 1, wqkv.p(), r.data());
  require(finite(r), "rope finite");
  Tensor q(1, gen_key(seed, 0, 7), (size_t)T * Hq * D, 1.0), k(1, gen_key(seed, 0, 8), (size_t)T * Hkv * D, 1.0),
      v(1, gen_key(seed, 0, 9), (size_t)T * Hkv * D, 1.0);
  std::vector<double> o(3 * Hq * D);
  oracle_attention(T, Hq, Hkv, D, 1, q.p(), k.p(), v.p(), 3, sel, o.data(), 2);
  require(finite(o), "attention finite");

  std::vector<double> hh(h.begin(), h.begin() + 5 * d), ex(5 * d), lgd(5 * E);
  std::vector<uint16_t> xb(5 * d);
  oracle_rmsnorm_bf16(5, d, 1e-5, hh.data(), xb.data(), ex.data());
  require(finite(ex), "rmsnorm finite");
  std::vector<int32_t> id(5 * K);
  oracle_deep_layer(5, d, F, E, K, 1e-5, hh.data(), wg.p(), nullptr, w1.p(), w3.p(), w2.p(), id.data(), lgd.data(), 2);
  require(finite(hh), "deep layer finite");
}

}  // namespace

int main() {
  require(oracle_abi_version() == 2, "oracle ABI version");
  std::vector<int64_t> u(100);
  gen_uniform_int(gen_key(1, 2, 3), 0, u.size(), 7, u.data());
  for (int64_t v : u) require(v >= 0 && v < 7, "uniform ints in range");
  layer_case(0, 37, 64, 96, 8, 2, false, 11);
  layer_case(1, 29, 64, 64, 8, 2, true, 12);
  layer_case(1, 21, 32, 32, 5, 3, false, 13);
  layer_case(2, 13, 32, 32, 4, 1, true, 14);
  layer_case(0, 9, 32, 32, 4, 4, false, 15);
  block_case(16);
  if (failures) return 1;
  std::printf("oracle driver ok\n");
  return 0;
}

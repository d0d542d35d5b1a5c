// C ABI of the mixture-of-experts library (declarations and contracts in include/moe.h).
// Validation runs before any launch; every call only enqueues kernels on the caller's stream.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "moe.h"

namespace moe {
DispatchEvents& pending_dispatch_events() {
  thread_local DispatchEvents ev;
  return ev;
}
}  // namespace moe

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

enum : unsigned { USE_D = 1, USE_F = 2, USE_EK = 4, USE_DTYPE = 8, USE_LAYOUT = 16 };

moe_status check_dims(const moe_dims* dims, unsigned use) {
  if (!dims) return fail(MOE_ERR_INVALID_ARG, "dims is NULL");
  const moe_dims& m = *dims;
  if (m.T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld is negative", (long long)m.T);
  if ((use & USE_D) && m.d <= 0) return fail(MOE_ERR_INVALID_ARG, "d = %d must be positive", m.d);
  if ((use & USE_F) && m.F <= 0) return fail(MOE_ERR_INVALID_ARG, "F = %d must be positive", m.F);
  if (use & USE_EK) {
    if (m.E <= 0 || m.K <= 0) return fail(MOE_ERR_INVALID_ARG, "E = %d and K = %d must be positive", m.E, m.K);
    if (m.K > m.E) return fail(MOE_ERR_INVALID_ARG, "K = %d exceeds E = %d", m.K, m.E);
    if (m.E > moe::kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "E = %d > %d", m.E, moe::kMaxExperts);
    if (m.K > moe::kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "K = %d > %d", m.K, moe::kMaxTopK);
    if (m.T * (int64_t)m.K >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "T*K must be < 2^31");
  }
  if ((use & USE_DTYPE) && m.dtype != MOE_F32 && m.dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "dtype = %d is not MOE_F32 or MOE_BF16", m.dtype);
  if ((use & USE_D) && (m.d % 64 != 0 || m.d > 65536))
    return fail(MOE_ERR_UNSUPPORTED, "d = %d must be a multiple of 64 and <= 65536", m.d);
  if ((use & USE_F) && (m.F % 64 != 0 || m.F > (1 << 24)))
    return fail(MOE_ERR_UNSUPPORTED, "F = %d must be a multiple of 64 and <= 2^24", m.F);
  if ((use & USE_LAYOUT) && m.weight_layout != MOE_LAYOUT_ROWMAJOR && m.weight_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "weight_layout = %d is not a moe_layout", m.weight_layout);
  return MOE_OK;
}

moe_status check_ptr(const void* p, const char* name, bool required = true) {
  if (!p) return required ? fail(MOE_ERR_INVALID_ARG, "%s is NULL", name) : MOE_OK;
  if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

#define MOE_TRY(expr)                \
  do {                               \
    moe_status s_ = (expr);          \
    if (s_ != MOE_OK) return s_;     \
  } while (0)

moe_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

size_t elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct Workspace {
  size_t topk_idx, topk_w, counts, offsets, row_token, token_row, h, y_perm, y_part, total;
  int ksplit;  // k-ranges of the down projection (partials 1.. live at y_part)
};

Workspace layout(const moe_dims& m) {
  const size_t S = (size_t)m.T * m.K;
  Workspace w{};
  size_t o = 0;
  w.topk_idx = o;  o = align256(o + S * 4);
  w.topk_w = o;    o = align256(o + S * 4);
  w.counts = o;    o = align256(o + (size_t)m.E * 4);
  w.offsets = o;   o = align256(o + (size_t)(m.E + 1) * 4);
  w.row_token = o; o = align256(o + S * 4);
  w.token_row = o; o = align256(o + S * 4);
  // h: row-major, or fragment-packed with each group padded to 16 rows (tiled path)
  w.h = o;         o = align256(o + (S + 15 * (size_t)m.E) * (size_t)m.F * elem_bytes(m.dtype));
  w.y_perm = o;    o = align256(o + S * (size_t)m.d * 4);
  w.ksplit = moe::tile_down_ksplit(m.dtype, (int64_t)S, m.E, m.d, m.F);
  w.y_part = o;    o = align256(o + (size_t)(w.ksplit - 1) * S * (size_t)m.d * 4);
  w.total = o;
  return w;
}

// Backward workspace.
struct BwdWorkspace {
  size_t topk_idx, topk_w, counts, offsets, row_token, token_row, x_perm, dy_perm, do_perm, dhp, h, dab, dgp,
      row_g, sink, dg, dlog, dxp, dxp_part, dwg_part, total;
  int dx_ksplit;  // k-ranges of the product [da|db] . [w1|w3] (partials 1.. at dxp_part)
};

BwdWorkspace bwd_layout(const moe_dims& m) {
  const size_t S = (size_t)m.T * m.K, d = (size_t)m.d, F = (size_t)m.F, E = (size_t)m.E;
  BwdWorkspace w{};
  size_t o = 0;
  auto take = [&](size_t& field, size_t bytes) {
    field = o;
    o = align256(o + bytes);
  };
  take(w.topk_idx, S * 4);
  take(w.topk_w, S * 4);
  take(w.counts, E * 4);
  take(w.offsets, (E + 1) * 4);
  take(w.row_token, S * 4);
  take(w.token_row, S * 4);
  take(w.x_perm, S * d * 2);
  take(w.dy_perm, S * d * 2);
  take(w.do_perm, S * d * 2);
  take(w.dhp, S * F * 4);
  take(w.h, S * F * 2);
  take(w.dab, S * 2 * F * 2);
  take(w.dgp, F / 64 * S * 4);
  take(w.row_g, S * 4);
  take(w.sink, 16);
  take(w.dg, S * 4);
  take(w.dlog, (size_t)m.T * E * 4);
  take(w.dxp, S * d * 4);
  w.dx_ksplit = moe::tile_down_ksplit(m.dtype, (int64_t)S, m.E, m.d, 2 * m.F);
  take(w.dxp_part, (size_t)(w.dx_ksplit - 1) * S * d * 4);
  take(w.dwg_part, (size_t)moe::dwgate_chunks(m.T) * d * E * 4);
  w.total = o;
  return w;
}

moe_status check_backward_sizes(const moe_dims& m) {
  if (m.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the backward pass supports bf16 only (dtype = %d)", m.dtype);
  if (m.d % 256 != 0 || m.F % 256 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "the backward pass needs d and F multiples of 256 (d = %d, F = %d)", m.d, m.F);
  return MOE_OK;
}

const moe_opts kDefaultOpts = {nullptr, -1, 0, nullptr, nullptr};

// Saved expert pre-activations (moe_opts.activations): the tiled product that writes them needs
// bf16 and d, F multiples of 256.
moe_status check_activations(const moe_dims& m, const moe_opts* o) {
  if (!o || !o->activations) return MOE_OK;
  if (!aligned16(o->activations)) return fail(MOE_ERR_INVALID_ARG, "activations is not 16-byte aligned");
  if (m.dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "saved activations need bf16 (dtype = %d)", m.dtype);
  if (m.d % 256 != 0 || m.F % 256 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "saved activations need d and F multiples of 256 (d = %d, F = %d)", m.d, m.F);
  return MOE_OK;
}

moe_status check_attn(const moe_attn_dims* a) {
  if (!a) return fail(MOE_ERR_INVALID_ARG, "attn is NULL");
  if (a->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld is negative", (long long)a->T);
  if (a->d <= 0 || a->n_heads <= 0 || a->n_kv_heads <= 0 || a->head_dim <= 0)
    return fail(MOE_ERR_INVALID_ARG, "d, n_heads, n_kv_heads and head_dim must be positive");
  if (a->n_heads % a->n_kv_heads != 0)
    return fail(MOE_ERR_INVALID_ARG, "n_heads = %d is not a multiple of n_kv_heads = %d", a->n_heads, a->n_kv_heads);
  if (!(a->rope_base > 1.0f)) return fail(MOE_ERR_INVALID_ARG, "rope_base must be > 1");
  if (!(a->eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
  if (a->head_dim != 128) return fail(MOE_ERR_UNSUPPORTED, "head_dim = %d (128 is supported)", a->head_dim);
  if ((a->n_heads / a->n_kv_heads) % 4 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "n_heads / n_kv_heads = %d must be a multiple of 4",
                a->n_heads / a->n_kv_heads);
  if (a->T >= (int64_t(1) << 31) / 4) return fail(MOE_ERR_UNSUPPORTED, "T must be < 2^29");
  return MOE_OK;
}

// Block workspace: the layer's own workspace first, then the block's buffers.
struct BlockWorkspace {
  size_t moe, offsets, u, qkv, q, k, v, o, a, x2, total;
};

BlockWorkspace block_layout(const moe_dims& m, const moe_attn_dims& at) {
  const size_t T = (size_t)at.T, d = (size_t)at.d, D = (size_t)at.head_dim;
  const size_t Hq = (size_t)at.n_heads, Hkv = (size_t)at.n_kv_heads;
  BlockWorkspace w{};
  size_t o = 0;
  auto take = [&](size_t& field, size_t bytes) {
    field = o;
    o = align256(o + bytes);
  };
  take(w.moe, layout(m).total);
  take(w.offsets, 2 * 4);
  take(w.u, T * d * 2);
  take(w.qkv, T * (Hq + 2 * Hkv) * D * 4);
  take(w.q, Hq * T * D * 2);
  take(w.k, Hkv * T * D * 2);
  take(w.v, Hkv * T * D * 2);
  take(w.o, T * Hq * D * 2);
  take(w.a, T * d * 4);
  take(w.x2, T * d * 2);
  w.total = o;
  return w;
}

moe_status check_block(const moe_dims* dims, const moe_attn_dims* attn) {
  MOE_TRY(check_dims(dims, USE_D | USE_F | USE_EK | USE_DTYPE | USE_LAYOUT));
  MOE_TRY(check_attn(attn));
  if (dims->T != attn->T || dims->d != attn->d)
    return fail(MOE_ERR_INVALID_ARG, "moe (T = %lld, d = %d) and attn (T = %lld, d = %d) disagree",
                (long long)dims->T, dims->d, (long long)attn->T, attn->d);
  if (dims->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the decoder block supports bf16 only");
  if (attn->d % 256 != 0) return fail(MOE_ERR_UNSUPPORTED, "d = %d must be a multiple of 256", attn->d);
  return MOE_OK;
}

moe_status check_opts(const moe_dims& m, const moe_opts* o, int* y_dtype) {
  const moe_opts& op = o ? *o : kDefaultOpts;
  if (op.accumulate != 0 && op.accumulate != 1)
    return fail(MOE_ERR_INVALID_ARG, "accumulate = %d must be 0 or 1", op.accumulate);
  int yd = op.y_dtype;
  if (!o) yd = m.dtype;
  if (op.accumulate) yd = MOE_F32;
  if (yd != MOE_F32 && yd != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "y_dtype = %d is not valid", yd);
  *y_dtype = yd;
  return MOE_OK;
}

// Scratch of moe_forward_noalloc: the workspace moe_forward would take from its caller, in a
// static device array (one copy per device, held until the process ends). Host code never uses
// the array's name as an address: each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
__device__ __align__(256) static uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev, kScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 5; }

const char* moe_status_string(moe_status s) {
  // A C caller may pass any int; reading it as the enum type would be undefined in C++ for values
  // outside the enumerators' range, so the bits are taken as an int.
  int v = 0;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_STATUS_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

moe_status moe_route(const moe_dims* dims, const moe_opts* opts, const void* x, const void* w_gate,
                     int32_t* topk_idx, float* topk_w, float* logits, void* stream) {
  MOE_TRY(check_dims(dims, USE_D | USE_EK | USE_DTYPE));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(w_gate, "w_gate"));
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(logits, "logits", false));
  const moe_dims& m = *dims;
  if (m.T == 0) return MOE_OK;
  moe::launch_route(m.dtype, x, w_gate, opts ? opts->gate_bias : nullptr, m.T, m.d, m.E, m.K, topk_idx, topk_w,
                    logits, static_cast<hipStream_t>(stream));
  return check_launch("moe_route");
}

moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* row_token, int32_t* token_row, void* x_perm, void* stream) {
  MOE_TRY(check_dims(dims, USE_EK | (x_perm ? (USE_D | USE_DTYPE) : 0u)));
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(counts, "counts"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(row_token, "row_token"));
  MOE_TRY(check_ptr(token_row, "token_row"));
  MOE_TRY(check_ptr(x_perm, "x_perm", false));
  if (x_perm) MOE_TRY(check_ptr(x, "x"));
  const moe_dims& m = *dims;
  if (m.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::launch_permute_index(topk_idx, m.T, m.E, m.K, counts, offsets, row_token, token_row, s);
  MOE_TRY(check_launch("moe_permute (index)"));
  if (x_perm) {
    moe::launch_gather_rows(x, row_token, m.T * m.K, (int64_t)m.d * elem_bytes(m.dtype), x_perm, s);
    MOE_TRY(check_launch("moe_permute (gather)"));
  }
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_dims* dims, const void* x_perm, const int32_t* offsets, const void* w1,
                          const void* w3, const void* w2, void* h_ws, float* y_perm, void* stream) {
  MOE_TRY(check_dims(dims, USE_D | USE_F | USE_EK | USE_DTYPE | USE_LAYOUT));
  MOE_TRY(check_ptr(x_perm, "x_perm"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(w1, "w1"));
  MOE_TRY(check_ptr(w3, "w3"));
  MOE_TRY(check_ptr(w2, "w2"));
  MOE_TRY(check_ptr(h_ws, "h_ws"));
  MOE_TRY(check_ptr(y_perm, "y_perm"));
  const moe_dims& m = *dims;
  if (m.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::launch_expert_up(m.dtype, m.weight_layout, x_perm, nullptr, offsets, m.T * m.K, m.d, m.F, m.E, w1, w3, h_ws,
                        s);
  MOE_TRY(check_launch("moe_expert_ffn (up)"));
  moe::launch_expert_down(m.dtype, m.weight_layout, h_ws, offsets, m.T * m.K, m.d, m.F, m.E, w2, y_perm, 1, nullptr,
                          s);
  return check_launch("moe_expert_ffn (down)");
}

moe_status moe_combine(const moe_dims* dims, const moe_opts* opts, const float* y_perm, const int32_t* token_row,
                       const float* topk_w, void* y, void* stream) {
  MOE_TRY(check_dims(dims, USE_D | USE_EK | USE_DTYPE));
  MOE_TRY(check_ptr(y_perm, "y_perm"));
  MOE_TRY(check_ptr(token_row, "token_row"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(y, "y"));
  const moe_dims& m = *dims;
  int yd = 0;
  MOE_TRY(check_opts(m, opts, &yd));
  if (m.T == 0) return MOE_OK;
  moe::launch_combine(y_perm, nullptr, 0, token_row, topk_w, m.T, m.d, m.K, yd, opts ? opts->accumulate : 0, y,
                      static_cast<hipStream_t>(stream));
  return check_launch("moe_combine");
}

moe_status moe_pack_weights(const moe_dims* dims, int32_t which, const void* w, void* w_packed, void* stream) {
  if (!dims) return fail(MOE_ERR_INVALID_ARG, "dims is NULL");
  const moe_dims& m = *dims;
  if (m.E <= 0) return fail(MOE_ERR_INVALID_ARG, "E = %d must be positive", m.E);
  if (m.E > moe::kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "E = %d > %d", m.E, moe::kMaxExperts);
  MOE_TRY(check_dims(dims, USE_D | USE_F | USE_DTYPE));
  if (which != MOE_W_UP && which != MOE_W_DOWN) return fail(MOE_ERR_INVALID_ARG, "which = %d is not valid", which);
  MOE_TRY(check_ptr(w, "w"));
  MOE_TRY(check_ptr(w_packed, "w_packed"));
  const size_t bytes = (size_t)m.E * m.F * m.d * elem_bytes(m.dtype);
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(w_packed);
  if (a < b + bytes && b < a + bytes) return fail(MOE_ERR_INVALID_ARG, "w and w_packed overlap");
  const int N = which == MOE_W_UP ? m.F : m.d;
  const int K = which == MOE_W_UP ? m.d : m.F;
  moe::launch_pack_weights(m.dtype, w, m.E, N, K, w_packed, static_cast<hipStream_t>(stream));
  return check_launch("moe_pack_weights");
}

size_t moe_workspace_bytes(const moe_dims* dims) {
  if (check_dims(dims, USE_D | USE_F | USE_EK | USE_DTYPE) != MOE_OK) return 0;
  return layout(*dims).total;
}

moe_status moe_forward(const moe_dims* dims, const moe_opts* opts, const void* x, const void* w_gate, const void* w1,
                       const void* w3, const void* w2, void* y, void* workspace, size_t workspace_bytes,
                       void* stream) {
  MOE_TRY(check_dims(dims, USE_D | USE_F | USE_EK | USE_DTYPE | USE_LAYOUT));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(w_gate, "w_gate"));
  MOE_TRY(check_ptr(w1, "w1"));
  MOE_TRY(check_ptr(w3, "w3"));
  MOE_TRY(check_ptr(w2, "w2"));
  MOE_TRY(check_ptr(y, "y"));
  const moe_dims& m = *dims;
  int yd = 0;
  MOE_TRY(check_opts(m, opts, &yd));
  MOE_TRY(check_activations(m, opts));
  if (m.T == 0) return MOE_OK;
  const Workspace L = layout(m);
  MOE_TRY(check_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(MOE_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);

  char* ws = static_cast<char*>(workspace);
  int32_t* topk_idx = reinterpret_cast<int32_t*>(ws + L.topk_idx);
  float* topk_w = reinterpret_cast<float*>(ws + L.topk_w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* row_token = reinterpret_cast<int32_t*>(ws + L.row_token);
  int32_t* token_row = reinterpret_cast<int32_t*>(ws + L.token_row);
  void* h = ws + L.h;
  float* y_perm = reinterpret_cast<float*>(ws + L.y_perm);
  float* y_part = reinterpret_cast<float*>(ws + L.y_part);
  hipStream_t s = static_cast<hipStream_t>(stream);

  // Stage events: each stage is one kernel, which records its pair as its own dispatch
  // timestamps (see launch_kernel); a pair the stage left unconsumed is recorded directly.
  void* const* ev = opts ? opts->stage_events : nullptr;
  auto arm = [&](int st) {
    if (ev) moe::pending_dispatch_events() = {static_cast<hipEvent_t>(ev[2 * st]), static_cast<hipEvent_t>(ev[2 * st + 1])};
  };
  auto disarm = [&]() -> moe_status {
    moe::DispatchEvents& p = moe::pending_dispatch_events();
    const moe::DispatchEvents left = p;
    p = moe::DispatchEvents{};
    for (hipEvent_t e : {left.start, left.stop}) {
      if (!e) continue;
      hipError_t r = hipEventRecord(e, s);
      if (r != hipSuccess) return fail(MOE_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(r));
    }
    return MOE_OK;
  };

  arm(MOE_STAGE_ROUTE);
  moe::launch_route(m.dtype, x, w_gate, opts ? opts->gate_bias : nullptr, m.T, m.d, m.E, m.K, topk_idx, topk_w,
                    nullptr, s);
  MOE_TRY(disarm());
  MOE_TRY(check_launch("moe_forward (route)"));
  arm(MOE_STAGE_PERMUTE);
  moe::launch_permute_index(topk_idx, m.T, m.E, m.K, counts, offsets, row_token, token_row, s);
  MOE_TRY(disarm());
  MOE_TRY(check_launch("moe_forward (permute)"));
  float* act = opts ? opts->activations : nullptr;
  // on the tiled path h stays fragment-packed between the two products (both take the same path)
  const bool hpk = moe::tile_gemm_applies(m.dtype, m.T * m.K, m.E, m.d, m.F);
  if (act) {
    // training: the pre-activations a, b in fp32 (kept for the backward pass) and h, in one product
    float* a = act;
    float* b = act + (size_t)m.T * m.K * m.F;
    arm(MOE_STAGE_EXPERT_UP);
    moe::launch_tile_up_pair(m.weight_layout, x, row_token, offsets, m.T * m.K, m.d, m.F, m.E, w1, w3, a, b, s, h,
                             hpk);
  } else {
    arm(MOE_STAGE_EXPERT_UP);
    moe::launch_expert_up(m.dtype, m.weight_layout, x, row_token, offsets, m.T * m.K, m.d, m.F, m.E, w1, w3, h, s,
                          hpk);
  }
  MOE_TRY(disarm());
  MOE_TRY(check_launch("moe_forward (expert up)"));
  arm(MOE_STAGE_EXPERT_DOWN);
  moe::launch_expert_down(m.dtype, m.weight_layout, h, offsets, m.T * m.K, m.d, m.F, m.E, w2, y_perm, L.ksplit, y_part,
                          s, hpk);
  MOE_TRY(disarm());
  MOE_TRY(check_launch("moe_forward (expert down)"));
  arm(MOE_STAGE_COMBINE);
  moe::launch_combine(y_perm, y_part, L.ksplit - 1, token_row, topk_w, m.T, m.d, m.K, yd, opts ? opts->accumulate : 0,
                      y, s);
  MOE_TRY(disarm());
  return check_launch("moe_forward (combine)");
}

moe_status moe_forward_noalloc(const moe_dims* dims, const moe_opts* opts, const void* x, const void* w_gate,
                               const void* w1, const void* w3, const void* w2, void* y, void* stream) {
  // moe_forward validates everything else; the size limit is checked first, before any HIP call
  MOE_TRY(check_dims(dims, USE_D | USE_F | USE_EK | USE_DTYPE | USE_LAYOUT));
  const size_t need = layout(*dims).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: these sizes need %zu bytes of workspace; the static scratch holds %zu "
                "(call moe_forward with a workspace instead)", need, kScratchBytes);
  if (dims->T == 0) return moe_forward(dims, opts, x, w_gate, w1, w3, w2, y, nullptr, 0, stream);
  void* ws = nullptr;
  MOE_TRY(scratch_of_current_device(&ws));
  return moe_forward(dims, opts, x, w_gate, w1, w3, w2, y, ws, kScratchBytes, stream);
}

size_t moe_backward_workspace_bytes(const moe_dims* dims) {
  if (check_dims(dims, USE_D | USE_F | USE_EK | USE_DTYPE | USE_LAYOUT) != MOE_OK) return 0;
  if (check_backward_sizes(*dims) != MOE_OK) return 0;
  return bwd_layout(*dims).total;
}

moe_status moe_backward(const moe_dims* dims, const moe_opts* opts, const void* x, const void* w_gate, const void* w1,
                        const void* w3, const void* w2, const float* dy, float* dx, float* dw_gate, float* dw1,
                        float* dw3, float* dw2, float* dlogits, void* workspace, size_t workspace_bytes,
                        void* stream) {
  MOE_TRY(check_dims(dims, USE_D | USE_F | USE_EK | USE_DTYPE | USE_LAYOUT));
  const moe_dims& m = *dims;
  MOE_TRY(check_backward_sizes(m));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(w_gate, "w_gate"));
  MOE_TRY(check_ptr(w1, "w1"));
  MOE_TRY(check_ptr(w3, "w3"));
  MOE_TRY(check_ptr(w2, "w2"));
  MOE_TRY(check_ptr(dy, "dy"));
  MOE_TRY(check_ptr(dx, "dx"));
  MOE_TRY(check_ptr(dw_gate, "dw_gate"));
  MOE_TRY(check_ptr(dw1, "dw1"));
  MOE_TRY(check_ptr(dw3, "dw3"));
  MOE_TRY(check_ptr(dw2, "dw2"));
  if (dlogits && !aligned16(dlogits)) return fail(MOE_ERR_INVALID_ARG, "dlogits is not 16-byte aligned");
  int yd = 0;
  MOE_TRY(check_opts(m, opts, &yd));
  MOE_TRY(check_activations(m, opts));
  if (m.T == 0) return MOE_OK;
  const BwdWorkspace L = bwd_layout(m);
  MOE_TRY(check_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(MOE_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);

  char* ws = static_cast<char*>(workspace);
  auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
  int32_t* topk_idx = static_cast<int32_t*>(at(L.topk_idx));
  float* topk_w = static_cast<float*>(at(L.topk_w));
  int32_t* counts = static_cast<int32_t*>(at(L.counts));
  int32_t* offsets = static_cast<int32_t*>(at(L.offsets));
  int32_t* row_token = static_cast<int32_t*>(at(L.row_token));
  int32_t* token_row = static_cast<int32_t*>(at(L.token_row));
  const float* saved = opts ? opts->activations : nullptr;
  float* dgp = static_cast<float*>(at(L.dgp));
  float* dhp = static_cast<float*>(at(L.dhp));
  float* dg = static_cast<float*>(at(L.dg));
  float* dlog = dlogits ? dlogits : static_cast<float*>(at(L.dlog));
  float* dxp = static_cast<float*>(at(L.dxp));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t S = m.T * m.K;
  const int lay = m.weight_layout;
  const bool pk = lay == MOE_LAYOUT_PACKED;  // packed weights: gradients in the same packed order

  // Every product below runs on the LDS-tiled kernels (any group size is handled; token blocks past
  // a group's end cost no MFMAs); the ones on transposed weights read w2 and w1, w3 as they lie
  // (row-major or fragment-packed).
  // forward pieces: routing, permutation, gathered rows
  moe::launch_route(m.dtype, x, w_gate, opts ? opts->gate_bias : nullptr, m.T, m.d, m.E, m.K, topk_idx, topk_w,
                    nullptr, s);
  moe::launch_permute_index(topk_idx, m.T, m.E, m.K, counts, offsets, row_token, token_row, s);
  moe::launch_gather_rows(x, row_token, S, (int64_t)m.d * 2, at(L.x_perm), s);
  // dh' = w2^T dy per row (w2 [E][d][F] is the transposed weight of this product)
  float* row_g = static_cast<float*>(at(L.row_g));
  moe::launch_gather_dy(dy, row_token, token_row, topk_w, m.K, S, m.d, at(L.dy_perm), at(L.do_perm), row_g, s);
  moe::launch_tile_wt(lay, at(L.dy_perm), offsets, S, m.F, m.d, m.E, w2, nullptr, dhp, 1, nullptr, s);
  // the SwiGLU derivative: from the kept pre-activations, or in the epilogue of their recomputation
  // (a = x.w1^T, b = x.w3^T never leave the registers); then the softmax derivative
  if (saved)
    moe::launch_swiglu_bwd(saved, saved + (size_t)S * m.F, dhp, row_token, token_row, topk_w, m.K, S, m.F, at(L.h),
                           at(L.dab), dgp, s);
  else
    moe::launch_tile_up_pair_bwd(lay, x, row_token, offsets, S, m.d, m.F, m.E, w1, w3, dhp, row_g, at(L.h), at(L.dab),
                                 dgp, at(L.sink), s);
  moe::launch_dg_sum(dgp, m.F, S, dg, s);
  moe::launch_router_bwd(dg, token_row, topk_idx, topk_w, m.T, m.E, m.K, dlog, s);
  MOE_TRY(check_launch("moe_backward (dgrad)"));
  // dx = sum_k (w1^T da + w3^T db) + W_g dlogit; dW_g = x^T dlogit
  float* dxp_part = static_cast<float*>(at(L.dxp_part));
  moe::launch_tile_wt(lay, at(L.dab), offsets, S, m.d, 2 * m.F, m.E, w1, w3, dxp, L.dx_ksplit, dxp_part, s);
  moe::launch_dx(dxp, dxp_part, L.dx_ksplit - 1, token_row, dlog, w_gate, m.T, m.d, m.E, m.K, dx, s);
  moe::launch_dwgate(x, dlog, m.T, m.d, m.E, static_cast<float*>(at(L.dwg_part)), dw_gate, s);
  MOE_TRY(check_launch("moe_backward (dx)"));
  // expert weight gradients: products over each group's rows, read as they lie
  const uint16_t* dab = static_cast<const uint16_t*>(at(L.dab));  // bf16 [T*K][2F]
  moe::launch_tile_wgrad(dab, m.F, 2 * m.F, at(L.x_perm), m.d, m.d, offsets, m.E, dw1, s, pk);
  moe::launch_tile_wgrad(dab + m.F, m.F, 2 * m.F, at(L.x_perm), m.d, m.d, offsets, m.E, dw3, s, pk);
  moe::launch_tile_wgrad(at(L.do_perm), m.d, m.d, at(L.h), m.F, m.F, offsets, m.E, dw2, s, pk);
  return check_launch("moe_backward (weight gradients)");
}

moe_status moe_attention(const moe_attn_dims* attn, const void* q, const void* k, const void* v, void* o,
                         void* stream) {
  MOE_TRY(check_attn(attn));
  MOE_TRY(check_ptr(q, "q"));
  MOE_TRY(check_ptr(k, "k"));
  MOE_TRY(check_ptr(v, "v"));
  MOE_TRY(check_ptr(o, "o"));
  if (attn->T == 0) return MOE_OK;
  moe::launch_attention(q, k, v, o, attn->T, attn->n_heads, attn->n_kv_heads, static_cast<hipStream_t>(stream));
  return check_launch("moe_attention");
}

size_t moe_block_workspace_bytes(const moe_dims* dims, const moe_attn_dims* attn) {
  if (check_block(dims, attn) != MOE_OK) return 0;
  return block_layout(*dims, *attn).total;
}

moe_status moe_block_forward(const moe_dims* dims, const moe_attn_dims* attn, const moe_opts* opts, float* h,
                             const void* w_qkv, const void* w_o, const void* w_gate, const void* w1, const void* w3,
                             const void* w2, void* workspace, size_t workspace_bytes, void* stream) {
  MOE_TRY(check_block(dims, attn));
  MOE_TRY(check_ptr(h, "h"));
  MOE_TRY(check_ptr(w_qkv, "w_qkv"));
  MOE_TRY(check_ptr(w_o, "w_o"));
  MOE_TRY(check_ptr(w_gate, "w_gate"));
  MOE_TRY(check_ptr(w1, "w1"));
  MOE_TRY(check_ptr(w3, "w3"));
  MOE_TRY(check_ptr(w2, "w2"));
  const moe_attn_dims& at = *attn;
  if (at.T == 0) return MOE_OK;
  const BlockWorkspace L = block_layout(*dims, at);
  MOE_TRY(check_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(MOE_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  auto at_ = [&](size_t off) { return static_cast<void*>(ws + off); };
  int32_t* off = static_cast<int32_t*>(at_(L.offsets));
  float* qkv = static_cast<float*>(at_(L.qkv));
  float* a = static_cast<float*>(at_(L.a));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = at.head_dim, Hq = at.n_heads, Hkv = at.n_kv_heads;
  const int rm = MOE_LAYOUT_ROWMAJOR;

  // attention sub-block: the two dense products run on the grouped kernels with one group of T rows
  moe::launch_set_offsets(off, at.T, s);
  moe::launch_rmsnorm(h, at.T, at.d, at.eps, at_(L.u), s);
  moe::launch_expert_down(MOE_BF16, rm, at_(L.u), off, at.T, (Hq + 2 * Hkv) * D, at.d, 1, w_qkv, qkv, 1, nullptr, s);
  moe::launch_rope_qkv(qkv, at.T, Hq, Hkv, (double)at.rope_base, at_(L.q), at_(L.k), at_(L.v), s);
  void* const* ev = opts ? opts->stage_events : nullptr;
  if (ev)  // the attention kernel records its own dispatch (see launch_kernel)
    moe::pending_dispatch_events() = {static_cast<hipEvent_t>(ev[2 * MOE_STAGE_ATTENTION]),
                                      static_cast<hipEvent_t>(ev[2 * MOE_STAGE_ATTENTION + 1])};
  moe::launch_attention(at_(L.q), at_(L.k), at_(L.v), at_(L.o), at.T, Hq, Hkv, s);
  moe::pending_dispatch_events() = moe::DispatchEvents{};
  moe::launch_expert_down(MOE_BF16, rm, at_(L.o), off, at.T, at.d, Hq * D, 1, w_o, a, 1, nullptr, s);
  moe::launch_residual_norm(h, a, at.T, at.d, at.eps, at_(L.x2), s);
  MOE_TRY(check_launch("moe_block_forward (attention)"));
  // mixture-of-experts sub-block, added to the residual stream
  moe_opts o2 = opts ? *opts : kDefaultOpts;
  o2.accumulate = 1;
  o2.y_dtype = MOE_F32;
  o2.activations = nullptr;  // the block keeps no activations (documented as ignored)
  return moe_forward(dims, &o2, at_(L.x2), w_gate, w1, w3, w2, h, at_(L.moe), layout(*dims).total, stream);
}

moe_status moe_rmsnorm(int64_t T, int32_t d, float eps, const float* h, void* x_bf16, void* stream) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld is negative", (long long)T);
  if (d <= 0) return fail(MOE_ERR_INVALID_ARG, "d = %d must be positive", d);
  if (!(eps >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "eps must be >= 0");
  if (d % 64 != 0 || d > 65536) return fail(MOE_ERR_UNSUPPORTED, "d = %d must be a multiple of 64", d);
  MOE_TRY(check_ptr(h, "h"));
  MOE_TRY(check_ptr(x_bf16, "x_bf16"));
  if (T == 0) return MOE_OK;
  moe::launch_rmsnorm(h, T, d, eps, x_bf16, static_cast<hipStream_t>(stream));
  return check_launch("moe_rmsnorm");
}

}  // extern "C"

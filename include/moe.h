/*
 * moe.h — C ABI of the MI355X (gfx950) sparse mixture-of-experts layer library.
 *
 * The layer is the one of "Mixtral of Experts" (arXiv 2401.04088):
 *
 *     G(x) = Softmax(TopK(x . W_g)),     y = sum_i G(x)_i * SwiGLU_i(x)
 *
 * with n = E experts, K of them kept per token (Mixtral: E = 8, K = 2), and each
 * expert SwiGLU_i(x) = w2_i . (silu(w1_i . x) * (w3_i . x)). The gating formula
 * and the output sum are those of the xyznot.com summary ("Método") and of the
 * blog.csdn.net explainer (sections 1 and 2.1-2.4); SwiGLU with hidden size
 * 14336 on d = 4096 comes from the same summary. Experts whose gate is 0 are
 * not evaluated (ja.news.hada.io summary), and the number of tokens per expert
 * varies from call to call (zh.newsflash.city article, section on the
 * mixture-of-experts layer), which is why the calls below group tokens by
 * expert before the expert matmuls and return them to token order afterwards.
 *
 * The five calls mirror the stages of the layer one to one:
 *     moe_route       logits, TopK, softmax over the kept logits
 *     moe_permute     per-expert counts, exclusive scan, stable scatter/gather
 *     moe_expert_ffn  grouped SwiGLU expert FFN over expert-contiguous rows
 *     moe_combine     gate-weighted sum back in token order
 *     moe_forward     all of the above in one call
 * and moe_backward computes the gradients of the layer; moe_attention and moe_block_forward run
 * the decoder block the layer sits in (below).
 *
 * Conventions shared by every call
 *  - Tensors are DEVICE pointers (hipMalloc'ed or torch CUDA/HIP tensors),
 *    row-major and contiguous, each aligned to 16 bytes.
 *  - Element type of x and of every weight: dims->dtype (MOE_F32 or MOE_BF16).
 *    Accumulation is fp32 in every case.
 *  - Ownership: the caller allocates and frees every buffer, the workspace
 *    included. The library allocates nothing and keeps no pointer after a call
 *    returns. (moe_forward_noalloc, for callers that cannot allocate, uses a
 *    static per-device scratch array instead of a workspace; see there.)
 *  - Asynchrony: a call only enqueues kernels on `stream` (a hipStream_t passed
 *    as void*, NULL = the default stream) and returns. Outputs are valid once
 *    the stream reaches that point; inputs must stay alive until then. No call
 *    synchronises or reads device memory on the host.
 *  - Errors: arguments are validated before anything is launched. On a non-OK
 *    status nothing has been enqueued and outputs are untouched (except
 *    MOE_ERR_HIP, raised by a failed launch). moe_last_error() returns a
 *    thread-local description of the last failure. T = 0 is valid: MOE_OK,
 *    nothing is launched and no output is written. No C++ exception crosses this interface.
 *  - Routing decisions are taken on fp32 logits; ties between equal logits go
 *    to the lower expert index, and slot k = 0 holds the largest logit.
 *  - Determinism: no call uses floating-point atomics; the same inputs give
 *    bit-identical outputs on every run.
 *  - Calls on different streams share no state and may run concurrently
 *    (except moe_forward_noalloc calls on one device, which share its scratch).
 *
 * Supported sizes: 1 <= E <= 64, 1 <= K <= min(E, 8), d and F multiples of 64,
 * d <= 65536, T*K < 2^31. Other valid sizes return MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, negative or zero size, K > E, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2, /* valid arguments outside the supported sizes listed above */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 4          /* a HIP launch failed; see moe_last_error() */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_LAYOUT_ROWMAJOR = 0, /* w1, w3 [E][F][d] and w2 [E][d][F], row-major */
  MOE_LAYOUT_PACKED = 1    /* the fragment-packed layout written by moe_pack_weights (below) */
} moe_layout;

/* Problem sizes. T tokens, model dim d, expert hidden dim F, E experts, K kept per token. */
typedef struct {
  int64_t T;
  int32_t d, F, E, K;
  int32_t dtype;         /* moe_dtype of x and of all weights */
  int32_t weight_layout; /* moe_layout of w1, w3, w2 (w_gate is always [d][E] row-major) */
} moe_dims;

typedef struct {
  const float* gate_bias; /* [E] fp32 added to the logits before TopK, or NULL (no bias) */
  int32_t y_dtype;        /* moe_dtype of y; ignored when accumulate = 1 */
  int32_t accumulate;     /* 0: y = result (rounded to y_dtype, nearest-even);
                             1: y is fp32 and receives y += result (residual stream) */
  void* const* stage_events; /* optional instrumentation for moe_forward, or NULL: an array of
                                2 * MOE_NUM_STAGES hipEvent_t (passed as void*, created by the
                                caller); entries 2s and 2s+1 receive the start and the end of
                                stage s's kernel, taken from the dispatch itself (no extra queue
                                packets, so timing does not slow the step). NULL entries are
                                skipped; with T = 0 nothing is launched or recorded. */
  float* activations;        /* optional, for training, or NULL: [2][T*K][F] fp32 = the expert
                                pre-activations a = x . w1[e]^T (first half) and b = x . w3[e]^T
                                (second half) of every routed row, rows in the permuted order of
                                moe_permute. moe_forward writes them (its expert product
                                stores a, b in fp32 besides h = silu(a) b, the same h as without
                                them on the tiled path); moe_backward given the same x,
                                w_gate, gate_bias and weights reads them instead of recomputing
                                them. Needs dims->dtype = MOE_BF16 and d, F multiples of 256. */
} moe_opts;

/* Stages of moe_forward, in launch order (one kernel each). */
enum {
  MOE_STAGE_ROUTE = 0,       /* logits, TopK, softmax */
  MOE_STAGE_PERMUTE = 1,     /* counts, offsets, stable row maps */
  MOE_STAGE_EXPERT_UP = 2,   /* gathered rows x w1, w3 and the SwiGLU product (grouped GEMM 1) */
  MOE_STAGE_EXPERT_DOWN = 3, /* hidden x w2 (grouped GEMM 2) */
  MOE_STAGE_COMBINE = 4,     /* gate-weighted sum back to token order */
  MOE_NUM_STAGES = 5,
  MOE_STAGE_ATTENTION = 5,   /* moe_block_forward only: the attention kernel */
  MOE_BLOCK_NUM_STAGES = 6   /* moe_block_forward's stage_events array holds 2 * MOE_BLOCK_NUM_STAGES entries */
};

/* Router (csdn explainer sections 2.1-2.3; xyznot.com "Método").
 *   x        [T][d] dtype        token representations
 *   w_gate   [d][E] dtype        router weight W_g (logits = x . W_g)
 *   topk_idx [T][K] int32  out   kept experts, slot 0 = largest logit, ties -> lower index
 *   topk_w   [T][K] fp32   out   softmax over the K kept logits (sums to 1 per token)
 *   logits   [T][E] fp32   out   optional (NULL = not written): x . W_g + bias in fp32
 * opts may be NULL (no bias). */
moe_status moe_route(const moe_dims* dims, const moe_opts* opts, const void* x, const void* w_gate,
                     int32_t* topk_idx, float* topk_w, float* logits, void* stream);

/* Token permutation into expert-contiguous order (variable tokens per expert:
 * zh.newsflash.city article, mixture-of-experts layer section).
 *   topk_idx  [T][K] int32 in    values in [0, E); the K experts of a token are distinct
 *   x         [T][d] dtype in
 *   counts    [E]    int32 out   tokens routed to each expert
 *   offsets   [E+1]  int32 out   exclusive scan of counts; offsets[E] = T*K
 *   row_token [T*K]  int32 out   token of each permuted row; rows of one expert follow
 *                                ascending token index
 *   token_row [T][K] int32 out   permuted row of (token, slot)
 *   x_perm    [T*K][d] dtype out x_perm[r] = x[row_token[r]]; may be NULL (maps only)
 * Out-of-range expert ids give undefined maps (not checked on the device). */
moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* row_token, int32_t* token_row, void* x_perm, void* stream);

/* Grouped SwiGLU expert FFN (xyznot.com "Método" and "Términos clave").
 * Rows [offsets[e], offsets[e+1]) of x_perm belong to expert e:
 *   h_ws[r]   = silu(x_perm[r] . w1[e]^T) * (x_perm[r] . w3[e]^T)   (stored in dtype)
 *   y_perm[r] = h_ws[r] . w2[e]^T                                    (fp32)
 *   x_perm  [T*K][d] dtype     offsets [E+1] int32 (device)
 *   w1, w3  [E][F][d] dtype    w2 [E][d][F] dtype   (or packed: dims->weight_layout)
 *   h_ws    [T*K][F] dtype     caller-provided scratch, overwritten
 *   y_perm  [T*K][d] fp32 out
 * Experts with no rows cost nothing. */
moe_status moe_expert_ffn(const moe_dims* dims, const void* x_perm, const int32_t* offsets, const void* w1,
                          const void* w3, const void* w2, void* h_ws, float* y_perm, void* stream);

/* Gate-weighted combine back to token order (csdn explainer section 1: y = sum_i G(x)_i E_i(x)).
 *   y[t] = sum_{k=0..K-1} topk_w[t][k] * y_perm[token_row[t][k]], summed in fp32 in slot order
 *   y_perm [T*K][d] fp32, token_row [T][K] int32, topk_w [T][K] fp32
 *   y      [T][d]  opts->y_dtype, or fp32 with y += result when opts->accumulate = 1
 * opts may be NULL (y_dtype = dims->dtype, no accumulation). */
moe_status moe_combine(const moe_dims* dims, const moe_opts* opts, const float* y_perm, const int32_t* token_row,
                       const float* topk_w, void* y, void* stream);

/* Expert weights in the fragment-packed layout (MOE_LAYOUT_PACKED).
 *
 * A matrix W[E][N][K] (row-major; N, K multiples of 16 and 4V) is stored as 1 KB fragments of
 * 16 rows x 4V columns, V = 16 / element size (8 for bf16, 4 for fp32). Element W[e][n][k] goes to
 *     ((e*(N/16) + n/16) * (K/(4V)) + k/(4V)) * 64V  +  lane*V  +  k%V,
 *     lane = n%16 + 16 * ((k/V) % 4).
 * Each fragment is one wavefront's matrix-core operand in lane order, and the fragments of one
 * 16-row block follow each other along k, so a wavefront streaming that block reads one
 * contiguous region with 1 KB per load instruction (the row-major rows of a block are K*elem
 * bytes apart, which keeps many more DRAM pages open at once). Packing is a one-time
 * rearrangement of the weights (same size); the packed and row-major paths give bit-identical
 * results.
 *   which = MOE_W_UP:   w (w1 or w3) [E][F][d]  (N = F, K = d)
 *   which = MOE_W_DOWN: w (w2)       [E][d][F]  (N = d, K = F)
 * w and w_packed are device buffers of E*F*d elements of dims->dtype and must not overlap. */
enum { MOE_W_UP = 0, MOE_W_DOWN = 1 };
moe_status moe_pack_weights(const moe_dims* dims, int32_t which, const void* w, void* w_packed, void* stream);

/* Bytes of device workspace moe_forward needs for these sizes (0 for invalid dims). */
size_t moe_workspace_bytes(const moe_dims* dims);

/* The whole layer: route -> permute -> expert FFN -> combine, all on `stream`.
 *   x [T][d] dtype, w_gate [d][E], w1/w3 [E][F][d], w2 [E][d][F] (dtype; w1/w3/w2 packed when
 *   dims->weight_layout = MOE_LAYOUT_PACKED)
 *   y [T][d] as in moe_combine (y may not alias x unless accumulate = 1 and y is a separate fp32 stream)
 *   workspace: >= moe_workspace_bytes(dims) bytes of device memory, 256-byte aligned
 * The token rows are gathered by the first expert matmul itself, so no x_perm copy is made. */
moe_status moe_forward(const moe_dims* dims, const moe_opts* opts, const void* x, const void* w_gate, const void* w1,
                       const void* w3, const void* w2, void* y, void* workspace, size_t workspace_bytes,
                       void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation). The workspace
 * moe_forward would take lives in a static device array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB), one
 * copy per device, which the library keeps until the process ends; the call runs on the current
 * device and allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   Arguments as in moe_forward, minus workspace and workspace_bytes.
 *   Sizes whose moe_workspace_bytes() exceeds the scratch return MOE_ERR_WORKSPACE before anything
 *   is launched (at d = 4096, F = 14336, E = 8, K = 2 the limit is 517 tokens, the decode batches:
 *   from 512 tokens the k-split partial sums of the tiled path join the workspace; larger batches
 *   call moe_forward with a workspace).
 *   Every call on a device shares that device's scratch and leaves its contents behind; nothing in
 *   it needs to start at zero (every value that enters a result is written before it is read; the
 *   padding rows of the packed hidden activations are read but feed only discarded output rows). Calls that overlap in time
 *   on one device (on different streams, or from different host threads without ordering between
 *   their streams) race on the scratch and give undefined results; calls ordered on one stream are
 *   safe. Results are bit-identical to moe_forward's. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_dims* dims, const moe_opts* opts, const void* x, const void* w_gate,
                               const void* w1, const void* w3, const void* w2, void* y, void* stream);

/* Backward pass of the layer (moe_forward with accumulate = 0). The pages define the forward
 * only; its gradient follows by the chain rule with the TopK selection held fixed. For token t,
 * kept experts e_k with gates g_k, a_k = w1[e_k] x, b_k = w3[e_k] x, h_k = silu(a_k) b_k,
 * o_k = w2[e_k] h_k and upstream gradient dy:
 *   dg_k = dy . o_k,  dlogit_{e_k} = g_k (dg_k - sum_j g_j dg_j)   (softmax over the kept logits)
 *   dh_k = w2[e_k]^T (g_k dy),  da_k = dh_k * b_k * silu'(a_k),  db_k = dh_k * silu(a_k)
 *   dx   = sum_k (w1[e_k]^T da_k + w3[e_k]^T db_k) + W_g dlogit
 *   dw2[e] = sum (g_k dy) h_k^T,  dw1[e] = sum da_k x^T,  dw3[e] = sum db_k x^T,  dW_g = x^T dlogit
 * The routing is recomputed from x; a_k, b_k are too, unless opts->activations holds them from a
 * moe_forward call on the same inputs.
 *   x, w_gate, w1, w3, w2  as in moe_forward (dims->dtype = MOE_BF16; weights row-major, or
 *                          fragment-packed with weight_layout = MOE_LAYOUT_PACKED)
 *   dy       [T][d]    fp32 in   gradient of the loss with respect to y
 *   dx       [T][d]    fp32 out
 *   dw_gate  [d][E]    fp32 out
 *   dw1, dw3 [E][F][d] fp32 out  (overwritten; an expert without tokens gets zeros)
 *   dw2      [E][d][F] fp32 out
 *                          With MOE_LAYOUT_PACKED, dw1, dw3 and dw2 come out in the element order of
 *                          the packed bf16 weights: gradient W[e][n][k] at the index that
 *                          moe_pack_weights gives bf16 W[e][n][k] (V = 8), so gradient element i
 *                          belongs to packed weight element i (an elementwise optimizer step can
 *                          run on the packed weights directly).
 *   dlogits  [T][E]    fp32 out  optional (NULL = not written): gradient of the logits,
 *                                zero for the experts not kept
 *   workspace: >= moe_backward_workspace_bytes(dims) bytes of device memory, 256-byte aligned
 * Operands of the matrix products are bf16 (dy, g_k dy, h_k, da_k and db_k rounded to nearest
 * even); all sums are fp32 in a fixed order, so results are reproducible bit for bit.
 * opts: gate_bias and activations as in the forward; y_dtype, accumulate and stage_events are
 * ignored.
 * Supported: dims->dtype = MOE_BF16, either weight layout, d and F multiples of 256 (with the
 * general limits above); other valid arguments return MOE_ERR_UNSUPPORTED. Packed and row-major
 * weights give the same gradients bit for bit (up to the order of dw1, dw3, dw2). */
size_t moe_backward_workspace_bytes(const moe_dims* dims);
moe_status moe_backward(const moe_dims* dims, const moe_opts* opts, const void* x, const void* w_gate, const void* w1,
                        const void* w3, const void* w2, const float* dy, float* dx, float* dw_gate, float* dw1,
                        float* dw3, float* dw2, float* dlogits, void* workspace, size_t workspace_bytes, void* stream);

/* RMSNorm of a residual stream for a stack of mixture-of-experts layers (the pages
 * do not describe the norm; unit weight): x_bf16[t] = bf16(h[t] / sqrt(mean_j h[t][j]^2 + eps)),
 * rounded to nearest even. h [T][d] fp32 in, x_bf16 [T][d] bf16 out. */
moe_status moe_rmsnorm(int64_t T, int32_t d, float eps, const float* h, void* x_bf16, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Decoder block around the layer. The pages give the rest of the transformer by its numbers only
 * (xyznot.com summary, "Método": 32 layers of width 4096, 32 attention heads, 8 key-value heads;
 * Mixtral keeps the Mistral 7B architecture and replaces each feed-forward sub-block by the
 * mixture-of-experts layer; a full 32k-token context). This library reads the block as the
 * pre-norm residual form of that architecture, for one sequence of T positions 0..T-1:
 *     u  = bf16(rmsnorm(h))                      (unit weight, eps as given)
 *     [q | k | v] = u . W_qkv^T                   (no biases)
 *     q, k: rotary embedding, in each head of width D the pair (i, i + D/2) of position p turns by
 *           the angle p * rope_base^(-2i/D)
 *     o_t = sum_{j<=t} softmax_j(q_t . k_j / sqrt(D)) v_j per query head; query head h reads
 *           key-value head h / (n_heads / n_kv_heads)
 *     h  += o . W_o^T;     h += MoE(bf16(rmsnorm(h)))
 * The rotary form and its base are readings (the pages name no position encoding).
 * Precision: bf16 operands of every product, fp32 sums; q, k, v, the attention weights and o are
 * rounded to bf16 (nearest even); h stays fp32. */
typedef struct {
  int64_t T;          /* positions of the sequence */
  int32_t d;          /* model width (the residual stream) */
  int32_t n_heads;    /* query heads */
  int32_t n_kv_heads; /* key-value heads; n_heads / n_kv_heads must be a multiple of 4 */
  int32_t head_dim;   /* D; 128 is supported */
  float rope_base;    /* base of the rotary angles (> 1) */
  float eps;          /* RMS norm epsilon (>= 0) */
} moe_attn_dims;

/* Causal grouped-query attention (the o_t line above):
 *   q [n_heads][T][D], k, v [n_kv_heads][T][D] bf16 in (q and k already rotated),
 *   o [T][n_heads * D] bf16 out (token-major, the input of the output projection).
 * Supported: head_dim = 128, n_heads a multiple of 4 * n_kv_heads. */
moe_status moe_attention(const moe_attn_dims* attn, const void* q, const void* k, const void* v, void* o,
                         void* stream);

/* One decoder block, in place on the fp32 residual stream h [T][d]:
 *   w_qkv [(n_heads + 2 n_kv_heads) * D][d] bf16, row-major (rows: the q heads, then k, then v)
 *   w_o   [d][n_heads * D] bf16, row-major
 *   w_gate, w1, w3, w2: the layer's weights as for moe_forward (dims->dtype must be MOE_BF16)
 *   moe->T and moe->d must equal attn->T and attn->d. opts: gate_bias as for moe_forward;
 *   stage_events, if not NULL, an array of 2 * MOE_BLOCK_NUM_STAGES events: entries 0 .. 2 *
 *   MOE_NUM_STAGES - 1 time the layer's stages as in moe_forward, entries 2 * MOE_STAGE_ATTENTION
 *   and 2 * MOE_STAGE_ATTENTION + 1 the attention kernel; y_dtype, accumulate and activations are
 *   ignored (the layer's output is added to h).
 *   workspace: >= moe_block_workspace_bytes() bytes of device memory, 256-byte aligned.
 * Supported: bf16, head_dim 128, n_heads a multiple of 4 * n_kv_heads, d a multiple of 256
 * (with the layer's limits). */
size_t moe_block_workspace_bytes(const moe_dims* moe, const moe_attn_dims* attn);
moe_status moe_block_forward(const moe_dims* moe, const moe_attn_dims* attn, const moe_opts* opts, float* h,
                             const void* w_qkv, const void* w_o, const void* w_gate, const void* w1, const void* w3,
                             const void* w2, void* workspace, size_t workspace_bytes, void* stream);

/* Static name of a status code. */
const char* moe_status_string(moe_status s);

/* Thread-local detail of the last non-OK status returned on this thread ("" if none). */
const char* moe_last_error(void);

/* ABI version of this header (bumped on any signature change). */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */

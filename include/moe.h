/*
 * moe.h -- C ABI of libmoeffn: the forward pass of one Mixture-of-Experts FFN
 * layer on an AMD Instinct MI355X (gfx950), plus an expert slot pool that keeps
 * only the experts the router selects in HBM and streams the rest from pinned
 * host memory.
 *
 * Sources (the pages this library follows):
 *  [NOVA]  "NovaLLM: Running Massive MoE Models Fully In-Memory", sections 2-3:
 *          a router picks a handful of experts per token and only those run;
 *          each expert is stored on its own and loaded just before it runs;
 *          all weights stay resident in pinned host memory; loads overlap compute.
 *  [BTB]   "The Billion-Token Bottleneck", sections "The Geometry of the Problem"
 *          (experts are feed-forward networks chosen by a router), "Tiered
 *          Memory" (HBM hot tier, host DDR warm tier over PCIe) and "Predictive
 *          Prefetching" (asynchronous host-to-HBM copies guarded by a residency
 *          check, then compute on resident weights).
 *  [VVLLM] "Running 35B MoE Models on 8GB GPUs: How vvllm-ms Caches Experts in
 *          System RAM", section "Technical Insight": a paged expert cache that
 *          intercepts the router's expert list, keeps whole expert bundles
 *          (weights and quantisation scales as one unit) in VRAM under LRU
 *          eviction, and when a batch needs more experts than fit, blocks,
 *          transfers, then executes in deterministic waves.
 * The router arithmetic, the SwiGLU expert and the number formats are not fixed
 * by the pages; each call below states the reading it implements.
 *
 * Conventions (all calls):
 *  - Every call returns a moe_status; 0 is success. On failure the call has
 *    enqueued nothing, and moe_last_error() returns a thread-local message.
 *    Nothing aborts, throws or prints.
 *  - Pointers are device pointers (HBM) unless the name ends in _host.
 *    Tensors are row-major, contiguous and caller-owned; the library never
 *    frees or retains a caller pointer beyond the call, except the slot pool
 *    and host bundles registered with expert_slot_cache_create.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls are
 *    asynchronous on it, except expert_slot_cache_acquire, which waits for the
 *    expert histogram (the one host synchronisation per decode step).
 *  - Device errors of earlier asynchronous work surface as MOE_EHIP at a later
 *    call.
 *  - Scratch memory is caller-provided; sizes come from the *_workspace_size
 *    queries. The library allocates device memory in no compute call.
 */
#ifndef MOEFFN_MOE_H
#define MOEFFN_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad argument: null pointer, bad size, misalignment */
  MOE_EUNSUPPORTED = -2,  /* valid but not implemented (dtype/shape combination) */
  MOE_EHIP = -3,          /* a HIP runtime call failed */
  MOE_ECAPACITY = -4,     /* workspace or pool too small */
  MOE_ENOMEM = -5,        /* host allocation failed */
  MOE_ESTATE = -6         /* call out of order (e.g. wave before acquire) */
};

/* Element types. MOE_FP8_E4M3 is the OCP 8-bit E4M3 ("fn": bias 7, max 448,
 * no infinities), always paired with fp32 scales as described per call.
 * MOE_MXFP4 (expert weights only) is OCP MXFP4: FP4 E2M1 codes (bias 1, values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives) with one E8M0 scale 2^(e-127)
 * per 32 consecutive inputs of an output column ([LVLLM] "Highlights" names
 * MXFP4 among the expert formats to carry).
 * MOE_MXFP8 (activations only) is OCP MXFP8: E4M3 codes with one E8M0 scale
 * 2^(e-127) per 32 consecutive values of a row, stored as uint8 bytes; it is the
 * A operand of MXFP4 experts on the block-scaled matrix instructions. */
enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP4 = 3, MOE_MXFP8 = 4 };
enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 };

/* Human-readable message for the last failing call on this thread ("" if none). */
const char* moe_last_error(void);
/* Library version string. */
const char* moe_version(void);

/* ------------------------------------------------------------------ route --
 * Router scores, top-k gating and the expert histogram ([BTB] "The Geometry
 * of the Problem": a router decides which experts handle each token; [NOVA]
 * section 3: only the selected experts are touched).
 *
 * Reading implemented (the pages leave the router math open):
 *  logits  l[t,e] = sum_i x[t,i] * w_router[e,i] (+ logit_bias[e]), fp32
 *          accumulation of the stored (fp32 or bf16) values;
 *  keys    softmax: key = l;  sigmoid: s = 1/(1+exp(-l)), key = s (+ select_bias[e]);
 *  groups  if n_groups > 1: group g = experts [g*E/G, (g+1)*E/G); group score =
 *          fp32 sum, largest first, of the group's group_topn largest keys; the
 *          topk_groups best groups are kept (ties -> lower group index);
 *  top-k   the k best kept experts by (key desc, expert index asc), best first;
 *  gates   softmax: exp(l_j - l_max_sel) / sum over the selection (renormalize=1)
 *          or the full softmax probability (renormalize=0); sigmoid: s_j / sum of
 *          selected s (renormalize=1) or s_j; both then times route_scale;
 *  shared  if w_shared_gate != NULL: shared_gate[t] = sigmoid(x[t] . w_shared_gate).
 *
 * Arguments:
 *  x            [T, d] act_dtype (MOE_F32 or MOE_BF16)
 *  w_router     [E, d] act_dtype: row e holds expert e's router weights
 *  logit_bias   [E] fp32 or NULL: added to every token's logits (a prior)
 *  select_bias  [E] fp32 or NULL: sigmoid only; steers selection, not gates
 *  w_shared_gate[d] act_dtype or NULL;  shared_gate [T] fp32 out (with it)
 *  scores       [T, E] fp32 out: the exact keys top-k selected on
 *  topk_idx     [T, k] int32 out;  topk_gate [T, k] fp32 out
 *  counts       [E] int32 out or NULL: counts[e] = #(t, j) with topk_idx = e
 * Errors: MOE_EINVAL for T < 0, d < 1, E < 1, k outside [1, E], d % 8 != 0,
 *  n_groups not dividing E, topk_groups > n_groups, group_topn outside
 *  [1, min(E/n_groups, 8)], k > topk_groups*E/n_groups, E > 1024, null required pointers,
 *  select_bias with softmax. T = 0 is a no-op (the configuration is still checked;
 *  tensor pointers may then be NULL).
 */
typedef struct {
  int32_t T, d_model, n_experts, top_k;
  int32_t score_fn;      /* MOE_SOFTMAX | MOE_SIGMOID */
  int32_t renormalize;   /* 1: gates renormalised over the selected experts */
  float route_scale;     /* multiplies every gate (1.0 unless stated) */
  int32_t n_groups;      /* 1 = no group limit */
  int32_t topk_groups;
  int32_t group_topn;
  int32_t act_dtype;     /* MOE_F32 | MOE_BF16 */
} moe_route_cfg;

moe_status moe_route(const moe_route_cfg* cfg, const void* x, const void* w_router,
                     const float* logit_bias, const float* select_bias,
                     const void* w_shared_gate, float* shared_gate, float* scores,
                     int32_t* topk_idx, float* topk_gate, int32_t* counts, void* stream);

/* ---------------------------------------------------------------- permute --
 * Grouping of the (token, slot) pairs by expert, the step that lets each
 * selected expert run once over all of its tokens ([NOVA] section 3: per-expert
 * execution of only the experts that were hit; [VVLLM] "Technical Insight": the
 * router's expert list is intercepted before expert compute).
 *
 * Reading implemented: a stable counting sort of p = t*k + j by expert id:
 *  offsets[e]  = number of pairs routed to experts < e (offsets[E] = T*k);
 *  perm_src[r] = p for the r-th row, rows expert-major, tokens ascending;
 *  perm_dst[p] = r (the inverse).
 * Optional row materialisation when x_out != NULL:
 *  gather = 1: x_out[r] = cvt(x[perm_src[r] / k]) for r < T*k;
 *  gather = 0: x_out[t] = cvt(x[t]) for t < T (token order, e.g. quantise once);
 *  cvt is a copy when out_dtype == x_dtype, or the per-row per-128-column e4m3
 *  quantisation when out_dtype == MOE_FP8_E4M3: a = max|v| over the 128-block,
 *  scale = a / 448 (1 if a == 0) in IEEE fp32, code = e4m3_rne(clamp(v/scale,
 *  +-448)); x_out_scale [rows, d/128] fp32 receives the scales;
 *  or the OCP MXFP8 conversion when out_dtype == MOE_MXFP8: per 32 consecutive
 *  values the shared exponent X = floor(log2 max|v|) - 8 clamped to
 *  [-127, 127] (-127 for a zero block), code = e4m3_rne(clamp(v * 2^-X, +-448)),
 *  and x_out_scale (read as uint8 [rows, d/32], so d % 32 == 0) receives the
 *  E8M0 bytes X + 127.
 * Workspace: moe_permute_workspace_size(T, k, E) bytes at `ws` (256-B aligned).
 * Errors: MOE_EINVAL on bad sizes/null pointers, MOE_ECAPACITY if ws_bytes is
 *  short, MOE_EUNSUPPORTED for an unsupported conversion. Indices outside
 *  [0, E) in topk_idx are not checked on the device (they come from moe_route).
 */
size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E);
moe_status moe_permute(int32_t T, int32_t k, int32_t E, const int32_t* topk_idx,
                       int32_t* offsets, int32_t* perm_src, int32_t* perm_dst,
                       int32_t d, const void* x, int32_t x_dtype, void* x_out,
                       int32_t out_dtype, float* x_out_scale, int32_t gather,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ route + permute --
 * moe_route followed by moe_permute without row materialisation (x_out NULL), as
 * one call: the router's expert list goes straight to the grouping that decides
 * which experts run ([VVLLM] "Technical Insight": the expert list is intercepted
 * between the router and the expert kernels). The outputs, their meaning, the
 * routing contract and the errors are those of the two calls; counts may be NULL.
 * Batches of 1..64 bf16 tokens with d % 32 == 0 and E <= 256 (a decode step) split
 * the logits over K across many workgroups (so the router weights stream through
 * many CUs); for up to 16 tokens one workgroup then adds the K slices in order,
 * selects and groups, for 17..64 a wavefront per token adds and selects and the
 * grouping follows. Their logits are therefore summed in another order than
 * moe_route's and can differ from them in the last bits. Other batches make the
 * two calls.
 * Workspace: moe_route_permute_workspace_size(T, k, E, d_model) bytes at `ws`
 * (256-B aligned); MOE_ECAPACITY if short.
 */
size_t moe_route_permute_workspace_size(int32_t T, int32_t k, int32_t E, int32_t d_model);
moe_status moe_route_permute(const moe_route_cfg* cfg, const void* x, const void* w_router,
                             const float* logit_bias, const float* select_bias,
                             const void* w_shared_gate, float* shared_gate, float* scores,
                             int32_t* topk_idx, float* topk_gate, int32_t* counts,
                             int32_t* offsets, int32_t* perm_src, int32_t* perm_dst,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ expert table --
 * Where each expert's bundle lives. A bundle is one contiguous block holding an
 * expert's three matrices and, for fp8, their scales: the atomic unit of
 * residency ([VVLLM] "Technical Insight": weights and quantisation scales move
 * together). slot_of_expert maps expert e to bundle slot s at
 * pool + s * slot_stride, or -1 to skip the expert in this call.
 *
 * Bundle layout (moe_pack_expert writes it; offsets are multiples of 256 B):
 *  MOE_BF16: W_gu then W_dn, each in 1 KiB MFMA tiles: for an [N, K] matrix the
 *   tile (nb, kb) covers rows 16nb..16nb+15 and columns 32kb..32kb+31, stored at
 *   ((nb * K/32) + kb) * 1024 bytes; inside, lane l (0..63) holds 8 consecutive
 *   elements: row 16nb + l%16, columns 32kb + 8*(l/16) + 0..7.
 *   W_gu is [2F, d] (N = 2F, K = d): rows 32j..32j+15 are W_gate columns
 *   16j..16j+15 and rows 32j+16..32j+31 are W_up columns 16j..16j+15 (the
 *   gate and up halves of every 16 hidden units are adjacent).
 *   W_dn is [d, F] (N = d, K = F): row n is W_down column n.
 *  MOE_FP8_E4M3: same row orders, 2 KiB tiles of 16 rows x 128 columns at
 *   ((nb * K/128) + kb) * 2048 bytes; byte h*1024 + 16*l + b (h = 0, 1; lane
 *   l = 0..63; b = 0..15) holds row 16nb + l%16, column 128kb + 32*(l/16) +
 *   16h + b (each half is one contiguous 1 KiB wave load of 16 bytes per lane);
 *   then three fp32 scale grids: gate [F/128][d/128], up [F/128][d/128],
 *   down [d/128][F/128] (one scale per 128x128 block of the original matrix).
 *  MOE_MXFP4: same row orders; each matrix [N, K] as codes then scales. Codes:
 *   chunks of 16 rows x 128 columns at ((nb * K/128) + kc) * 1024 bytes; byte
 *   16*l + 4*c + j (lane l = 0..63, k-step c = 0..3, j = 0..3) holds row
 *   16nb + l%16, columns 128kc + 32c + 8*(l/16) + 2j (low nibble) and + 1 (high
 *   nibble). Scales (256 B after the codes): 64 bytes per chunk at
 *   ((nb * K/128) + kc) * 64, byte 4r + c the E8M0 exponent of row 16nb + r,
 *   columns 128kc + 32c .. + 31. Order: W_gu codes, W_gu scales, W_dn codes,
 *   W_dn scales.
 *  MOE_F32: W_gate^T [F, d], W_up^T [F, d], W_down^T [d, F], plain row-major.
 * Requirements: d % 32 == 0 and F % 32 == 0 (bf16); d % 128 == 0 and
 *  F % 128 == 0 (fp8, mxfp4); d % 4 == 0 (f32).
 */
typedef struct {
  const void* pool;               /* device base address of slot 0 */
  int64_t slot_stride;            /* bytes between slots, >= bundle bytes, % 256 == 0 */
  const int32_t* slot_of_expert;  /* device [n_experts]: slot or -1 (skip) */
  int32_t n_experts, d_model, d_ff;
  int32_t w_dtype;                /* MOE_F32 | MOE_BF16 | MOE_FP8_E4M3 | MOE_MXFP4 */
} moe_expert_table;

/* Bytes of one expert bundle for this layout (0 on invalid sizes). */
size_t moe_bundle_bytes(int32_t d_model, int32_t d_ff, int32_t w_dtype);

/* Host-side packer: writes one bundle from the expert's matrices in their
 * natural layouts, W_gate and W_up [d, F], W_down [F, d] (element type w_dtype;
 * fp8 codes as uint8), plus for fp8 the block scales gate/up [d/128][F/128] and
 * down [F/128][d/128] (fp32). For MXFP4 the matrices hold one FP4 code (0..15)
 * per uint8 and the scales are gate/up [d/32][F] and down [F/32][d], fp32 powers
 * of two 2^(e-127), e in 0..254 (MOE_EINVAL for any other value or a code above
 * 15). bundle_host must hold moe_bundle_bytes(...) bytes.
 * Pure host code; no device is touched. */
moe_status moe_pack_expert(int32_t d_model, int32_t d_ff, int32_t w_dtype,
                           const void* w_gate_host, const void* w_up_host,
                           const void* w_down_host, const float* s_gate_host,
                           const float* s_up_host, const float* s_down_host,
                           void* bundle_host);

/* ------------------------------------------------------------- grouped FFN --
 * The selected experts' SwiGLU feed-forward networks, each run once over the
 * rows grouped to it ([BTB] "The Geometry of the Problem": experts are
 * feed-forward networks; [NOVA] section 3: only the experts that were hit run).
 *
 * Reading implemented: for every expert e with slot_of_expert[e] >= 0 and rows
 * r in [offsets[e], offsets[e+1]):
 *   A_r = a[a_row_src ? a_row_src[r] / a_row_div : r]          (row of `a`)
 *   H_r = silu(A_r W_gate_e) * (A_r W_up_e)    (fp32 accumulation; rounded to
 *         bf16 for bf16 weights, re-quantised per row per 128 to e4m3 for fp8)
 *   y_r = H_r W_down_e                          (fp32 accumulation, y_dtype)
 * Rows of skipped experts are left untouched in y.
 *  a        [*, d] act_dtype: MOE_F32 (f32 weights), MOE_BF16 (bf16 or MXFP4
 *           weights), MOE_FP8_E4M3 codes (fp8 weights) with a_scale [*, d/128]
 *           fp32, or MOE_MXFP8 codes (MXFP4 weights) with a_scale pointing at
 *           the uint8 E8M0 bytes [*, d/32].
 *           MXFP4 weights with bf16 activations are decoded exactly to bf16
 *           (E2M1 times a power of two) for bf16 MFMAs and run at most 64 rows
 *           per expert (decode batches; more is MOE_EUNSUPPORTED). With MXFP8
 *           activations they run on the block-scaled MFMA (E4M3 x E2M1, both
 *           E8M0 scales applied by the instruction), any number of rows; H is
 *           then re-quantised to MXFP8 (per row per 32) before the down GEMM.
 *  offsets  device [n_experts + 1] int32 (from moe_permute, or [0, rows] for a
 *           single dense expert such as a shared expert)
 *  y        [rows, d] y_dtype (MOE_F32 or MOE_BF16)
 * Workspace: moe_grouped_ffn_workspace_size(table, rows, act_dtype) bytes.
 * Errors: MOE_EINVAL on bad sizes/pointers/alignment (16 B for a, y, pool),
 *  MOE_EUNSUPPORTED for dtype combinations not listed, MOE_ECAPACITY for a
 *  short workspace. Slot values are not range-checked on the device; the slot
 *  pool owner (e.g. expert_slot_cache) is responsible for them.
 */
size_t moe_grouped_ffn_workspace_size(const moe_expert_table* table, int32_t rows,
                                      int32_t act_dtype);
moe_status moe_grouped_ffn(const moe_expert_table* table, int32_t rows, const int32_t* offsets,
                           const void* a, const float* a_scale, int32_t act_dtype,
                           const int32_t* a_row_src, int32_t a_row_div,
                           void* y, int32_t y_dtype, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- grouped FFN batch --
 * One or two independent grouped FFN problems, each with exactly the meaning,
 * argument rules and errors of a moe_grouped_ffn call with the same fields (the
 * problem's index is named in error messages). Meant for the routed experts and
 * the always-resident shared expert of one layer ([VVLLM] "Gotcha": shared
 * experts sit outside the routed set): when both problems are bf16 with at most
 * 64 rows per expert (a decode step), they share one gate/up launch and one down
 * launch, with the first problem's work dispatched first, instead of running
 * on two streams that a graph must fork and join. Two fp8 problems (or two
 * MXFP4 problems with MXFP8 activations) of the same d_model likewise share one
 * launch per GEMM: the second is one more group of the first's tile list.
 * Otherwise the problems run one after the other on `stream`. n must be 1 or 2.
 * Workspace: moe_grouped_ffn_batch_workspace_size(problems, n) bytes at `ws`
 * (256-B aligned): each problem's moe_grouped_ffn workspace, in order, each
 * rounded up to a multiple of 256 B.
 */
typedef struct {
  const moe_expert_table* table;
  int32_t rows;
  const int32_t* offsets;
  const void* a;
  const float* a_scale;
  int32_t act_dtype;
  const int32_t* a_row_src;
  int32_t a_row_div;
  void* y;
  int32_t y_dtype;
} moe_ffn_problem;

size_t moe_grouped_ffn_batch_workspace_size(const moe_ffn_problem* problems, int32_t n);
moe_status moe_grouped_ffn_batch(const moe_ffn_problem* problems, int32_t n, void* ws, size_t ws_bytes,
                                 void* stream);

/* ---------------------------------------------------------------- combine --
 * Gate-weighted sum of each token's expert outputs back in token order, plus
 * the always-resident shared expert ([VVLLM] "Gotcha": shared experts sit
 * outside the routed set; here they never enter the slot pool).
 *  out[t] = sum_{j<k} topk_gate[t,j] * y[perm_dst[t*k+j]]
 *           + (shared_y ? (shared_gate ? shared_gate[t] : 1) * shared_y[t] : 0)
 * accumulated in fp32 in that order (j ascending, shared last), rounded once to
 * out_dtype. y and shared_y are [*, d] in y_dtype (MOE_F32 or MOE_BF16).
 * Errors: MOE_EINVAL on bad sizes/pointers. T = 0 is a no-op.
 */
moe_status moe_combine(int32_t T, int32_t k, int32_t d, const void* y, int32_t y_dtype,
                       const int32_t* perm_dst, const float* topk_gate,
                       const void* shared_y, const float* shared_gate,
                       void* out, int32_t out_dtype, void* stream);

/* ------------------------------------------- decode FFN with the combine --
 * A decode step's grouped FFN and combine in one call (two launches): the
 * routed experts and, optionally, the always-resident shared expert ([VVLLM]
 * "Gotcha": shared experts sit outside the routed set), then the gate-weighted
 * sum back to token order, which the last workgroup to finish each 32-column
 * group of the down projection computes for that group ([NOVA] section 3,
 * Optimization #3: fewer launches per decode step).
 * The result equals, bit for bit, moe_grouped_ffn_batch over {shared, routed}
 * (or {routed}) followed by moe_combine(T, k, d, routed.y, routed.y_dtype,
 * perm_dst, topk_gate, shared.y, shared_gate, out, out_dtype): each expert
 * output is rounded to its problem's y_dtype and the sum runs in fp32, j
 * ascending, shared term last, rounded once to out_dtype.
 *  routed  the routed problem: rows = T*k, a_row_src = perm_src, a_row_div = k
 *  shared  NULL or the shared expert: one group, offsets [0, T], rows = T
 *  The problems' y pointers are not used (may be NULL): the expert outputs
 *  stay in the workspace. Only out [T, d] (16-B aligned) is written.
 * Both problems must be decode problems (bf16 weights and activations, T <= 64
 * tokens); otherwise MOE_EUNSUPPORTED (use the batch call and moe_combine).
 * Workspace: moe_grouped_ffn_combine_workspace_size(routed, shared) bytes,
 * 256-B aligned. Calls that share a workspace must not overlap.
 * Errors: as moe_grouped_ffn for each problem; MOE_EINVAL for rows that do
 * not match T and k, MOE_ECAPACITY for a short workspace. T = 0 is a no-op.
 */
typedef struct {
  int32_t T, k;
  const int32_t* perm_dst;   /* [T*k] device: row of the routed outputs */
  const float* topk_gate;    /* [T*k] device */
  const float* shared_gate;  /* [T] device, or NULL = 1 (used only with a shared problem) */
  void* out;                 /* [T, d] device, out_dtype */
  int32_t out_dtype;         /* MOE_F32 or MOE_BF16 */
} moe_combine_args;

size_t moe_grouped_ffn_combine_workspace_size(const moe_ffn_problem* routed, const moe_ffn_problem* shared);
moe_status moe_grouped_ffn_combine(const moe_ffn_problem* routed, const moe_ffn_problem* shared,
                                   const moe_combine_args* comb, void* ws, size_t ws_bytes, void* stream);

/* moe_grouped_ffn_combine without allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments and results as moe_grouped_ffn_combine
 * (bit for bit), minus the workspace: it lives in a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES, one per GPU the library runs on, held until the
 * process ends. The caller still passes every input and output. No device
 * memory is allocated or freed by the call.
 * Limit: a step whose moe_grouped_ffn_combine_workspace_size exceeds
 * MOE_NOALLOC_SCRATCH_BYTES is rejected with MOE_ECAPACITY before any launch.
 * Every call on a GPU uses that GPU's one array: calls that overlap on the same
 * GPU (other streams or threads) race and must be serialised by the caller.
 * Errors: as moe_grouped_ffn_combine; MOE_ECAPACITY as above; MOE_EHIP if the
 * array's device address cannot be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_grouped_ffn_combine_noalloc(const moe_ffn_problem* routed, const moe_ffn_problem* shared,
                                           const moe_combine_args* comb, void* stream);

/* ------------------------------------------------------------- decode step --
 * A whole decode step of a resident layer in one call: moe_route_permute, the
 * routed experts' and the shared expert's FFN, and the combine ([NOVA]
 * section 3, Optimization #3: a decode step is many small launches, whose
 * overhead and idle gaps the step should not pay). Three launches (four past
 * 4 tokens, where the combine is its own launch):
 *  1. the router logits split over K beside the shared expert's gate/up
 *     projection, which needs no routing ([VVLLM] "Gotcha": the shared expert
 *     sits outside the routed set), so its weights stream while the routing
 *     runs; the last routing workgroups to finish select and group;
 *  2. the shared expert's down projection beside the routed experts' gate/up;
 *  3. the routed experts' down projection, with the combine folded in for
 *     T <= 4 (as moe_grouped_ffn_combine), else followed by moe_combine.
 * Results are bit-identical to moe_route_permute(cfg, ...) followed by, for
 * T <= 4, moe_grouped_ffn_combine and otherwise moe_grouped_ffn_batch plus
 * moe_combine, with both problems' y_dtype MOE_BF16 (each expert output is
 * rounded to bf16; the sum runs in fp32, j ascending, shared term last).
 *  cfg       routing as for moe_route_permute; act_dtype MOE_BF16, 1 <= T <= 64,
 *            d_model % 32 == 0, n_experts <= 256
 *  x [T, d] bf16, w_router [E, d] bf16, logit_bias / select_bias / w_shared_gate
 *            as for moe_route_permute (w_shared_gate given iff o->shared_gate)
 *  routed    the table of the E routed experts (bf16 or MXFP4 bundles)
 *  shared    NULL, or a one-expert table of the same d_model and format (its
 *            rows are the T tokens; no offsets are needed)
 *  o         the routing outputs of moe_route_permute (counts may be NULL) and
 *            out [T, d] (16-B aligned) in out_dtype (MOE_F32 or MOE_BF16)
 * Workspace: moe_decode_step_workspace_size(cfg, routed, shared) bytes, 256-B
 * aligned. Its first 256 bytes are arrival counters that must be zero when
 * the first call on that workspace starts (e.g. a zero-filled allocation);
 * every call leaves them zero. Calls that share a workspace must not overlap.
 * Errors: as moe_route_permute and moe_grouped_ffn for each problem;
 * MOE_EUNSUPPORTED outside the sizes above (use the separate calls).
 */
typedef struct {
  float* shared_gate;   /* [T] or NULL (given iff w_shared_gate) */
  float* scores;        /* [T, E] */
  int32_t* topk_idx;    /* [T, k] */
  float* topk_gate;     /* [T, k] */
  int32_t* counts;      /* [E] or NULL */
  int32_t* offsets;     /* [E + 1] */
  int32_t* perm_src;    /* [T * k] */
  int32_t* perm_dst;    /* [T * k] */
  void* out;            /* [T, d] out_dtype */
  int32_t out_dtype;    /* MOE_F32 or MOE_BF16 */
} moe_decode_out;

size_t moe_decode_step_workspace_size(const moe_route_cfg* cfg, const moe_expert_table* routed,
                                      const moe_expert_table* shared);
moe_status moe_decode_step(const moe_route_cfg* cfg, const void* x, const void* w_router,
                           const float* logit_bias, const float* select_bias, const void* w_shared_gate,
                           const moe_expert_table* routed, const moe_expert_table* shared,
                           const moe_decode_out* o, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- expert slot cache --
 * Expert-granular residency: a fixed pool of n_slots bundle slots in HBM backed
 * by every expert's bundle in pinned host memory ([NOVA] section 3,
 * Optimization #2: weights resident in pinned memory; [BTB] "Tiered Memory" and
 * "Predictive Prefetching": HBM hot tier, host warm tier, asynchronous copies
 * guarded by a residency check; [VVLLM] "Technical Insight": LRU eviction of
 * whole bundles, blocking transfer waves when a batch needs more experts than
 * fit).
 *
 * Reading implemented, per decode step:
 *  1. acquire: copy counts[E] to the host and wait (the interception of the
 *     router's expert list); touched = experts with counts > 0; access order =
 *     resident touched experts (ascending id), then non-resident (ascending);
 *     cut into waves of <= n_slots; each access is an LRU access (hit refreshes
 *     recency; a miss takes the lowest free slot, else evicts the least recently
 *     used expert; eviction copies nothing back since weights are read-only).
 *  2. per wave w, part 0 (hits): writes the slot table holding the wave's hits
 *     only and starts the wave's miss copies (host bundle -> slot) on the cache's
 *     side stream, each after the last compute read of its victim slot;
 *     part 1 (misses): makes `stream` wait for those copies and writes the
 *     table holding the wave's misses only. The caller runs moe_grouped_ffn with
 *     each table, so hit experts compute while misses are in flight.
 *     In blocking mode (cfg.blocking = 1) the wave's copies start only after
 *     all work enqueued on `stream` so far, part 0 waits for them and holds
 *     every expert of the wave, and part 1 is empty: block, transfer, then
 *     execute, with no copy/compute overlap.
 *  3. release(w): records that the wave's slots were read by the work enqueued
 *     so far on `stream` (a later copy into those slots waits for it).
 * Device-side state is only the pool (caller memory) and the slot tables it
 * writes (caller memory). The host tables, one side stream, events and a small
 * pinned staging area are allocated in create and freed in destroy.
 * dry_run = 1 creates a host-only planner (no HIP calls; acquire/wave/release
 * fail with MOE_ESTATE) for expert_slot_cache_plan_host.
 * Errors: MOE_EINVAL (sizes, null pointers, a bundle not in pinned host memory),
 *  MOE_ECAPACITY (n_slots < 1, slot_stride < bundle_bytes), MOE_ESTATE (calls
 *  out of order), MOE_EHIP (a copy or event call failed). A failed bundle copy
 *  fails loudly instead of letting a wave run on an incomplete bundle ("Running
 *  35B MoE Models on 8GB GPUs", section "Technical Insight"): the call returns
 *  MOE_EHIP, the expert whose copy failed and every miss of the step whose copy
 *  was not issued yet leave the residency table (their slots become free, so a
 *  later step misses on them again), and the step ends: expert_slot_cache_wave
 *  returns MOE_ESTATE until the next acquire. For tests, the environment
 *  variable MOEFFN_FAIL_COPY_AT=n (read at create) makes the n-th bundle copy of
 *  the cache (misses and prefetches, counted from 1) fail this way without
 *  calling hipMemcpyAsync.
 */
typedef struct expert_slot_cache expert_slot_cache;

typedef struct {
  int32_t n_experts;
  int32_t n_slots;
  int64_t bundle_bytes;
  int64_t slot_stride;              /* >= bundle_bytes, multiple of 256 */
  const void* const* bundles_host;  /* [n_experts] pinned host bundles (NULL if dry_run) */
  void* pool;                       /* device, n_slots * slot_stride bytes (NULL if dry_run) */
  int32_t blocking;                 /* 1: wait for all copies, then execute */
  int32_t dry_run;                  /* 1: host-only planner */
} moe_cache_cfg;

typedef struct {
  int64_t steps, hits, misses, evictions, waves;
  int64_t h2d_bytes, d2h_bytes;   /* h2d includes prefetch copies */
  double copy_ms;   /* sum over steps of side-stream copy spans of the steps' misses (events) */
  int64_t prefetches;     /* bundles copied by expert_slot_cache_prefetch */
  int64_t prefetch_used;  /* of those, bundles a later step hit before they were evicted */
  double wait_ms;   /* sum over waves of the compute stream's wait for the wave's copies (events on
                       the compute stream before and after the wait); 0 for the device-planned cache */
} moe_cache_stats;

/* One entry of a wave's plan (host query for tests and tools). */
typedef struct {
  int32_t expert, slot, hit, evicted;  /* evicted = expert evicted for it, or -1 */
} moe_cache_entry;

moe_status expert_slot_cache_create(const moe_cache_cfg* cfg, expert_slot_cache** out);
moe_status expert_slot_cache_destroy(expert_slot_cache* c);
moe_status expert_slot_cache_reset(expert_slot_cache* c);
moe_status expert_slot_cache_acquire(expert_slot_cache* c, const int32_t* counts, void* stream,
                                     int32_t* n_waves_out);
moe_status expert_slot_cache_plan_host(expert_slot_cache* c, const int32_t* counts_host,
                                       int32_t* n_waves_out);
moe_status expert_slot_cache_wave(expert_slot_cache* c, int32_t wave, int32_t part, void* stream,
                                  int32_t* slot_of_expert, int32_t* n_experts_in_part);
moe_status expert_slot_cache_release(expert_slot_cache* c, int32_t wave, void* stream);
/* Victim order for a pool shared by the layers of a stack. With n_layers > 1
 * the cache's entries are n_layers layer-major groups of n_experts / n_layers
 * (entry l * (n_experts / n_layers) + e is expert e of layer l), the layers run
 * in the cyclic order 0, 1, ..., n_layers - 1, 0, ..., and every step touches
 * entries of one layer only (else acquire / plan_host fail with MOE_EINVAL).
 * A miss (or a prefetch) then evicts, among the entries it may evict, one of
 * the layer whose next step is furthest away, (layer - current - 1) mod
 * n_layers largest, and within that layer the least recently used one.
 * n_layers = 1 (the default) is plain LRU. This goes beyond the pages, whose
 * cache is plain LRU and which name that as its weakness ("Running 35B MoE
 * Models on 8GB GPUs", section "Gotcha"): a stack that cycles through more
 * experts than the pool holds makes LRU evict exactly the entries needed next.
 * Host planner only (not expert_slot_cache_dev).
 * Errors: MOE_EINVAL (n_layers < 1 or not a divisor of n_experts). */
moe_status expert_slot_cache_set_layers(expert_slot_cache* c, int32_t n_layers);

/* Frequency-aware victims (beyond the pages, like the layer order). With
 * decay in (0, 1] every planned step first updates, for every entry,
 * freq = decay * freq + counts (the step's routed rows per entry), and a victim
 * is then chosen (after the layer order, if set) by the smallest freq, ties to
 * the least recently used. decay = 0 (the default) turns it off: plain
 * recency. Setting it clears the frequencies. The pages' cache evicts by
 * recency alone ("Running 35B MoE Models on 8GB GPUs", section "Technical
 * Insight") and they call that blind to which experts will be needed (section
 * "Gotcha"); under a skewed, slowly drifting routing prior the experts routed
 * to most often are the ones needed next. Host planner only.
 * Errors: MOE_EINVAL (decay outside [0, 1]). */
moe_status expert_slot_cache_set_frequency(expert_slot_cache* c, double decay);

/* Prefetch of predicted experts ahead of the step that routes to them.
 * The pages: a background reader fetches the next layer while the current one
 * computes ("NovaLLM: Running Massive MoE Models Fully In-Memory", section 3,
 * Optimization #1); predicted experts that are not resident are copied
 * host -> HBM asynchronously before the model reaches their layer, the experts
 * most in demand first ("The Billion-Token Bottleneck", sections "Predictive
 * Prefetching: Looking into the Future" and "The Orchestration Layer").
 * The prediction itself is the caller's (a list of expert ids, highest
 * priority first). Readings implemented, in list order:
 *  - a resident expert has its recency refreshed, and is not copied;
 *  - a non-resident expert takes the lowest free slot, else the slot of the
 *    least recently used expert that neither the last planned step (acquire or
 *    plan_host) accessed nor a prefetch since then named: a prefetch never
 *    evicts an expert of that step, whose kernels may still read it, nor one
 *    it has just brought in. If every slot holds such an expert, the rest of
 *    the list is dropped;
 *  - a prefetched expert is resident for the planner: the next step that
 *    touches it counts a hit (stats.prefetch_used) and runs it with the wave's
 *    hits (part 0), after `stream`-side waits for its copy if that copy may
 *    still be in flight.
 * Copies go on the cache's side stream, after every copy issued before (so
 * call this after the current step's waves have been issued, or its miss
 * copies queue behind the prediction), each after the last compute read of
 * its victim slot. Under dry_run only the plan changes.
 * n_copies_out (optional) = bundles copied by this call.
 * Errors: MOE_EINVAL (an id outside [0, n_experts), n < 0, NULL list with
 *  n > 0), MOE_ESTATE (a blocking cache, which only transfers what a step
 *  needs), MOE_EHIP (a copy failed; that expert is left non-resident). */
moe_status expert_slot_cache_prefetch(expert_slot_cache* c, const int32_t* experts_host, int32_t n,
                                      int32_t* n_copies_out);
moe_status expert_slot_cache_wave_plan(const expert_slot_cache* c, int32_t wave,
                                       moe_cache_entry* entries_host, int32_t capacity,
                                       int32_t* n_entries);
moe_status expert_slot_cache_stats(const expert_slot_cache* c, moe_cache_stats* out);

/* ------------------------------------------------- device-planned cache --
 * The slot pool with the residency check and plan made on the device, so a
 * decode step never waits for the host (the per-step interception of the
 * router's expert list is a host synchronisation in "Running 35B MoE Models on
 * 8GB GPUs", section "Technical Insight"; "NovaLLM", section 3, removes launch
 * overhead with graph capture). Same readings as expert_slot_cache: per step
 * the touched experts (counts > 0) are accessed resident-first, then the
 * others, each in ascending id, in waves of at most n_slots accesses; LRU with
 * the lowest free slot first. Resident experts are all hits of wave 0.
 *
 * Per step, all on `stream` unless said otherwise:
 *  expert_slot_cache_dev_step: one plan kernel. Reads counts[E], updates the
 *    device-resident table and writes hit_table[E] (slot of each wave-0 hit,
 *    else -1) and miss_tables[w*E + e] for w < expert_slot_cache_dev_max_waves
 *    (slot of expert e if it is loaded in wave w, else -1).
 *  for each wave w < max_waves (waves the step does not need cost one empty
 *  copy launch and the caller's launches over an all -1 table):
 *    expert_slot_cache_dev_copy(w): the cache's side stream waits for the work
 *      enqueued on `stream` so far (so wave w-1's kernels are done before its
 *      slots are reused), then one copy kernel reads wave w's missed bundles
 *      from pinned host memory (their device mapping) into their slots;
 *    (w = 0) the caller runs moe_grouped_ffn over hit_table, concurrent with
 *      the copies;
 *    expert_slot_cache_dev_join(w): `stream` waits for wave w's copies;
 *    the caller runs moe_grouped_ffn over miss_tables + w*E.
 * All of it may be captured into one graph (the join of every copied wave
 * must be captured too: it rejoins the side stream). Steps on one cache are
 * issued on one stream, in order.
 * cfg: blocking = dry_run = 0; n_experts, n_slots <= 1024; bundle_bytes a
 * multiple of 16; bundles in pinned host memory, 16-byte aligned; the pool and
 * the tables are caller memory. The library allocates the device-side table,
 * one side stream and two events per wave in create. stats and reset
 * synchronise the device.
 * Errors: MOE_EINVAL (sizes, NULL, a bundle without a device mapping, a wave
 *  out of range), MOE_ECAPACITY (slots), MOE_ESTATE (copy or join before any
 *  step), MOE_EHIP. */
typedef struct expert_slot_cache_dev expert_slot_cache_dev;
moe_status expert_slot_cache_dev_create(const moe_cache_cfg* cfg, expert_slot_cache_dev** out);
moe_status expert_slot_cache_dev_destroy(expert_slot_cache_dev* c);
moe_status expert_slot_cache_dev_reset(expert_slot_cache_dev* c);
int32_t expert_slot_cache_dev_max_waves(const expert_slot_cache_dev* c);   /* ceil(n_experts / n_slots) */
/* Frequency-aware victims, as expert_slot_cache_set_frequency (same doubles:
 * the device rounds the multiply and the add separately). The victim is the
 * lowest free slot, else, outside the current wave, the smallest frequency,
 * then the least recently used. decay = 0 (default) is plain LRU. Setting it
 * synchronises the device and clears the frequencies; the decay lives in device
 * memory, so graphs captured before see the new value. Errors: MOE_EINVAL. */
moe_status expert_slot_cache_dev_set_frequency(expert_slot_cache_dev* c, double decay);
/* The layer order, as expert_slot_cache_set_layers, applied before the
 * frequency and recency stages; a step's layer is that of its lowest touched
 * entry. A step touching entries of several layers is not rejected when it is
 * planned (the plan kernel cannot return an error without a host sync): it is
 * planned with the layer of its lowest touched entry, counted on the device,
 * and the next expert_slot_cache_dev_stats call returns MOE_ESTATE for it (the
 * host-planned cache and its oracle reject such a step at once).
 * Synchronises the device; kept in device memory like the decay. */
moe_status expert_slot_cache_dev_set_layers(expert_slot_cache_dev* c, int32_t n_layers);
moe_status expert_slot_cache_dev_step(expert_slot_cache_dev* c, const int32_t* counts, void* stream,
                                      int32_t* hit_table, int32_t* miss_tables);
moe_status expert_slot_cache_dev_copy(expert_slot_cache_dev* c, int32_t wave, void* stream);
moe_status expert_slot_cache_dev_join(expert_slot_cache_dev* c, int32_t wave, void* stream);
/* hits, misses, evictions, steps, waves; h2d_bytes = misses x bundle_bytes;
 * copy_ms and the prefetch fields are 0. */
moe_status expert_slot_cache_dev_stats(expert_slot_cache_dev* c, moe_cache_stats* out);

/* ---------------------------------------------------------------- profile --
 * Optional per-kernel timing for measurement tools (not part of the layer's
 * arithmetic). While enabled, moe_grouped_ffn records a hipEvent pair on its
 * stream around each of its heavy kernels; moe_profile_read waits for the
 * recorded pairs and returns the summed milliseconds and launch counts per
 * kernel kind since the last moe_profile_enable call (which also resets).
 * Kinds: 0 gate/up GEMM with the SwiGLU epilogue, 1 down GEMM (many rows per
 * expert), 2 and 3 the same for the decode kernels (at most 64 rows per expert).
 * Launches made while the calling thread's label is 1 (moe_profile_label) are
 * recorded under kind + 4 instead, so a caller can keep, say, a shared expert
 * running concurrently on another stream apart from the routed experts.
 * Errors: MOE_EINVAL for a NULL out or a label other than 0 and 1, MOE_EHIP if an
 * event cannot be read.
 */
enum {
  MOE_PROF_GATEUP = 0,
  MOE_PROF_DOWN = 1,
  MOE_PROF_DEC_GATEUP = 2,
  MOE_PROF_DEC_DOWN = 3,
  MOE_PROF_LABELED = 4, /* offset of the kinds recorded under label 1 */
  MOE_PROF_KINDS = 8
};
typedef struct {
  double ms[MOE_PROF_KINDS];
  int64_t launches[MOE_PROF_KINDS];
} moe_profile;
moe_status moe_profile_enable(int32_t on);
moe_status moe_profile_label(int32_t label);
moe_status moe_profile_read(moe_profile* out);

#ifdef __cplusplus
}
#endif
#endif /* MOEFFN_MOE_H */

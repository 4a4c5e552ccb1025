/*
 * mxfp4_moe.h -- C ABI of the MI355X (gfx950) MXFP4 mixture-of-experts
 * expert-projection library (libmxfp4_moe.so).
 *
 * The method (gpt-oss-20b files page):
 *   - README section "MXFP4", checkpoint tensor table: expert weights are
 *     stored as u8 blocks [Experts, Rows, K/32, 16] holding two E2M1 codes per
 *     byte (low nibble = even element) and u8 E8M0 scales [Experts, Rows, K/32];
 *     a weight is its E2M1 value times 2 ** (scale - 127).
 *   - README section "Dense routing" and src/experts.linnet (fn ranks, route,
 *     experts_of, weights_of): each token keeps its TopK highest router logits,
 *     ties to the lower expert index, highest first; the router weights are the
 *     softmax over the kept logits.
 *   - README section "Loading" and src/experts.linnet (fn forward_topk,
 *     forward_routed): the experts multiply only the tokens routed to them; the
 *     gate/up projection reads the token's input, the down projection each
 *     slot's own input; every projection adds its per-row bias; the expert sum
 *     is taken in f32 with the router weights.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers to row-major, contiguous memory on
 *     the current HIP device.  bf16 values are passed as their uint16_t bit
 *     patterns.  The caller owns every buffer; the library never allocates or
 *     frees device memory and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous and stream-ordered; nothing synchronizes the host.
 *   - Every argument the host can check is checked before anything is
 *     enqueued.  On failure the call returns a nonzero mxfp4_status, enqueues
 *     nothing, and mxfp4_last_error() describes the failure (thread-local).
 *     Argument checks come before any HIP call, so they also run on a host
 *     without a GPU.
 *   - Only gfx950 devices are supported (MXFP4_ERR_UNSUPPORTED_DEVICE).
 *   - Values written to outputs are deterministic: the same inputs give
 *     bit-identical outputs (no floating-point atomics).
 */
#ifndef MXFP4_MOE_H
#define MXFP4_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFP4_OK = 0,
  MXFP4_ERR_INVALID_ARG = 1,        /* a null pointer, a bad size or a bad combination */
  MXFP4_ERR_WORKSPACE = 2,          /* workspace missing or smaller than required */
  MXFP4_ERR_UNSUPPORTED_DEVICE = 3, /* the current device is not gfx950 */
  MXFP4_ERR_HIP = 4                 /* a HIP runtime call failed (text in mxfp4_last_error) */
} mxfp4_status;

/* Bits of the optional device error word written by mxfp4_moe_route_group. */
#define MXFP4_ROUTE_ERR_ID_RANGE 1  /* a given expert id was outside [0, E), or a token's logits held a NaN */
/* A token with either error keeps a defined result: gate 0 in every slot it
 * could not route (all k slots for a NaN logit), so moe_combine gives that
 * token's y the sum over its valid slots only (0 for a NaN logit). */
#define MXFP4_ROUTE_ERR_ID_DUP 2    /* a token's given expert ids were not distinct */

/* Library limits. */
#define MXFP4_MAX_EXPERTS 512
#define MXFP4_MAX_TOPK 32
#define MXFP4_GEMM_MAX_K 8192        /* grouped-GEMM path: a weight panel's scale rows staged in LDS */
#define MXFP4_DECODE_MAX_EXPERTS 64  /* mxfp4_moe_decode: experts routed in one wave */
#define MXFP4_DECODE_MAX_K 3072      /* mxfp4_moe_decode: all of a row's loads in flight at once */
#define MXFP4_DECODE_MAX_T 64        /* mxfp4_moe_decode_batch: tokens ranked one per lane */

/* Projection paths for mxfp4_expert_proj. */
#define MXFP4_PATH_AUTO 0  /* GEMV while T * k <= 16 * min(E, T * k), grouped GEMM otherwise */
#define MXFP4_PATH_GEMV 1  /* decode GEMV: 128-bit weight streaming, exact bf16 products, fp32 sums */
#define MXFP4_PATH_GEMM 2  /* grouped GEMM on scaled-FP4 MFMA, activations as two to four MX-FP6 terms */

/* Static text for a status code. */
const char* mxfp4_status_string(int status);

/* Detail text of the last failure on the calling thread ("" if none). */
const char* mxfp4_last_error(void);

/*
 * Route tokens to experts and group the routed rows by expert.
 * (README "Dense routing"; src/experts.linnet fn ranks / route / experts_of /
 * weights_of; README "Loading": the tokens each expert was chosen for.)
 *
 *   logits      [T, E] bf16, or NULL.  Router logits.
 *   ids_in      [T, k] i32, or NULL.   Given expert ids.
 *               Exactly one of the two routes is taken:
 *               - ids_in == NULL: topk_ids[t, s] = the expert of rank s among
 *                 token t's logits, where an expert's rank counts the experts
 *                 with a larger logit or an equal logit and a lower index
 *                 (logits is then required).  A NaN logit has no rank:
 *                 such a token gets -1 and gate 0 in all k slots (its rows
 *                 are left out of the grouping) and MXFP4_ROUTE_ERR_ID_RANGE.
 *               - ids_in != NULL: topk_ids = ids_in (slot order kept).  Ids must
 *                 lie in [0, E) and be distinct per token; violations set bits in
 *                 *error_word, an out-of-range id is written as -1, its row is
 *                 left out of the grouping and its gate is 0.
 *   T >= 0, 1 <= E <= MXFP4_MAX_EXPERTS, 1 <= k <= min(E, MXFP4_MAX_TOPK).
 *   topk_ids    [T, k] i32 out.
 *   gates       [T, k] f32 out, or NULL.  Written only when logits != NULL:
 *               gates[t, s] = exp(l_s - max) / sum_j exp(l_j - max) over the
 *               logits at the valid ids of topk_ids[t, :] (all k when the
 *               routing succeeded), fp32; 0 for a slot whose id is -1.
 *   expert_offsets [E + 1] i32 out: exclusive prefix sum of the number of routed
 *               rows per expert; expert_offsets[E] = number of grouped rows
 *               (T * k when every id is valid).
 *   sorted_rows [T * k] i32 out: the routed rows r = t * k + s, grouped by
 *               expert (expert e's rows are sorted_rows[offsets[e] : offsets[e+1]])
 *               and ascending within an expert.  Entries past offsets[E] are
 *               not written.
 *   error_word  [1] i32 out, or NULL: overwritten with the MXFP4_ROUTE_ERR_* bits
 *               found (0 = none).  With more than 64 rows the routing launch
 *               zeroes it and the grouping launch ORs in what each workgroup
 *               finds in its own rows, so the word is final when the call's
 *               work on the stream is done.
 * T * k <= 64: one kernel launch (a single workgroup); more rows: a routing
 * launch (one token per wave) and a grouping launch (ceil(T * k / 1024)
 * workgroups).  T = 0 writes zero offsets.
 */
int mxfp4_moe_route_group(const uint16_t* logits, const int32_t* ids_in, int T, int E, int k,
                          int32_t* topk_ids, float* gates, int32_t* expert_offsets,
                          int32_t* sorted_rows, int32_t* error_word, void* stream);

/*
 * Router logits of the MoE block: logits = x . w^T + bias, the Linear from the
 * hidden width to the experts whose output the routing ranks.
 * (src/experts.linnet block MixtureOfExperts, sub router: a Linear from H to
 * the experts, weight [E, H] and bias [E] in bf16.)
 *
 *   x       [T, H] bf16, 16-byte aligned.  T >= 0, H a positive multiple of 32.
 *   w       [E, H] bf16 (row e = expert e's weights), 16-byte aligned.
 *           1 <= E <= MXFP4_MAX_EXPERTS.
 *   bias    [E] bf16, or NULL for none.
 *   logits  [T, E] bf16 out: the bf16 rounding (to nearest even) of
 *           bias[e] + sum_j x[t, j] * w[e, j], with exact bf16 products summed
 *           in fp32 in a fixed order (deterministic).
 * One kernel launch; T = 0 returns MXFP4_OK and enqueues nothing.
 */
int mxfp4_moe_router(const uint16_t* x, const uint16_t* w, const uint16_t* bias, int T, int H, int E,
                     uint16_t* logits, void* stream);

/*
 * Dense router weights: every expert's probability, exactly zero outside each
 * token's top k -- the weights of the dense-routing form, which evaluates every
 * expert on every token (a validation mode of the sparse path: with all E
 * experts as given ids, mxfp4_expert_proj and moe_combine with these weights
 * give the sparse result up to fp32 rounding).
 * (README "Dense routing"; src/experts.linnet fn route: the experts ranked k or
 * worse are floored to -1e30 and the softmax taken over all E, so the floored
 * entries are exactly zero and the kept ones the softmax over the kept logits.)
 *
 *   logits  [T, E] bf16, finite.  T >= 0, 1 <= E <= MXFP4_MAX_EXPERTS, 1 <= k <= E.
 *   probs   [T, E] f32 out: probs[t, e] = exp(l_e - max) / sum over the kept of
 *           exp(l_j - max) if e ranks below k (ranking as mxfp4_moe_route_group),
 *           else 0.  The kept values equal mxfp4_moe_route_group's gates bit for bit.
 * T = 0 returns MXFP4_OK and enqueues nothing.
 */
int mxfp4_moe_dense_route(const uint16_t* logits, int T, int E, int k, float* probs, void* stream);

/*
 * Workspace bytes mxfp4_expert_proj needs for these sizes and this path
 * (MXFP4_PATH_AUTO resolves exactly as mxfp4_expert_proj does).  0 means none.
 * Returns (size_t)-1 for invalid sizes.
 */
size_t mxfp4_expert_proj_workspace_size(int E, int N, int T, int k, int K, int x_per_slot, int path);

/*
 * The routed expert projection.
 * (README "MXFP4" for the weight format; src/experts.linnet fn forward_topk
 * and forward_routed for the products; fn activate / down_bias_of for the
 * per-expert bias rows.)
 *
 *   blocks  [E, N, K/32, 16] u8   MXFP4 codes, low nibble = even element;
 *           one expert's N * K / 2 bytes at most 4 GiB.
 *   scales  [E, N, K/32]     u8   E8M0 exponents (bias 127); bytes 0..254.
 *   bias    [E, N] bf16, or NULL (no bias).
 *   E, N, K: 1 <= E <= MXFP4_MAX_EXPERTS, N >= 1, K >= 32 and K % 32 == 0.
 *   x       x_per_slot == 0: [T, K] bf16, one input per token shared by its k slots
 *                            (gate/up);
 *           x_per_slot != 0: [T, k, K] bf16, one input per routed row (down).
 *           Values must be finite.
 *   T >= 0, 1 <= k <= min(E, MXFP4_MAX_TOPK).
 *   expert_offsets [E + 1], sorted_rows [T * k]: as produced by
 *           mxfp4_moe_route_group.  Offsets outside [0, T * k] and rows outside
 *           [0, T * k) are clamped or skipped on the device, never dereferenced.
 *   out     [T, k, N] f32 out:
 *           out[t, s, n] = bias[e, n] + sum_j W[e, n, j] * x_src[j],  e the expert
 *           that row r = t * k + s is grouped under, W[e, n, j] =
 *           e2m1(code) * 2 ** (scales[e, n, j / 32] - 127).  Rows absent from the
 *           grouping are not written.
 *   path    MXFP4_PATH_AUTO / _GEMV / _GEMM.  GEMV multiplies exact bf16
 *           weights (the E2M1 value times the E8M0 factor) by the bf16 inputs
 *           (bf16 dot products for one token with K <= 3072, the bf16 MFMA
 *           otherwise) and sums in fp32; it needs K <= 4096 when T > 4
 *           (its LDS staging).  GEMM (K <= MXFP4_GEMM_MAX_K) feeds the weights
 *           to the MFMA as stored and writes each bf16 activation block of 32
 *           as a sum of MX-FP6 (E2M3) terms, one MFMA each: two for every block,
 *           then a third and a fourth while some block's residual exceeds 1/64
 *           of its mean magnitude without its largest element (outlier
 *           channels, heavy tails), decided per 32 rows x 64 inputs.  Its
 *           error is an approximation's, not a rounding's: it has
 *           stayed within 2e-3 * sum_j |W x| + 1e-5 per output on every input
 *           tested -- normal, log-normal (sigma <= 3), outlier channels up to
 *           1e5 x the rest, the gated activation's outputs -- and the GEMV path
 *           is the one with exact products for any input.
 *   workspace, workspace_bytes: device scratch of at least
 *           mxfp4_expert_proj_workspace_size(E, N, T, k, K, x_per_slot, path) bytes,
 *           16-byte aligned; may be NULL when that size is 0.  Calls that share
 *           a workspace must be ordered on one stream.
 * T = 0 returns MXFP4_OK and enqueues nothing.
 */
int mxfp4_expert_proj(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias,
                      int E, int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                      const int32_t* expert_offsets, const int32_t* sorted_rows, float* out,
                      int path, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mxfp4_expert_proj for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same arguments, paths, limits and results (bit for bit) as
 * mxfp4_expert_proj, without the workspace: the grouped-GEMM path's scratch
 * (the quantized activation terms, their scales and the repacked weight
 * scales) is a static device array of MXFP4_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; its device
 * address is looked up once per device.  Nothing is allocated or freed, and
 * nothing needs to start at zero: every call writes all of the scratch it
 * reads.  Every call on one GPU shares that GPU's array, so calls that
 * overlap on one GPU (on different streams, or from several threads) race:
 * order them on one stream.  A problem whose grouped GEMM would need more
 * than MXFP4_NOALLOC_SCRATCH_BYTES (mxfp4_expert_proj_workspace_size) returns
 * MXFP4_ERR_WORKSPACE and enqueues nothing; the GEMV path needs no scratch.
 */
#define MXFP4_NOALLOC_SCRATCH_BYTES (128u << 20)
int mxfp4_expert_proj_noalloc(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias,
                              int E, int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                              const int32_t* expert_offsets, const int32_t* sorted_rows, float* out,
                              int path, void* stream);

/*
 * The routed gate/up projection followed by the gpt-oss gated activation,
 * written as bf16 -- the down projection's per-slot input.
 * (src/experts.linnet: the gate and up weights share one tensor, interleaved
 * along its output rows, even rows gate and odd rows multiply; constants
 * LIMIT = 7 and ALPHA = 1.702 and fn activate: the biased gate clamped from
 * above at LIMIT, the biased multiplier clamped to [-LIMIT, LIMIT], then
 * (up + 1) * gate * sigmoid(ALPHA * gate).)
 *
 *   Arguments as for mxfp4_expert_proj, with N even, and in place of out:
 *   act     [T, k, N / 2] bf16 out:
 *           act[t, s, i] = bf16(swiglu(p[t, s, 2 i], p[t, s, 2 i + 1])), where p
 *           is what mxfp4_expert_proj would write to out (projection + bias,
 *           fp32) and swiglu is evaluated in fp32 (expf) and rounded to nearest
 *           even.  Rows absent from the grouping are not written.
 *   The same paths, limits, workspace size and errors as mxfp4_expert_proj
 *   (MXFP4_ERR_INVALID_ARG also for an odd N).
 */
int mxfp4_expert_proj_swiglu(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias,
                             int E, int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                             const int32_t* expert_offsets, const int32_t* sorted_rows, uint16_t* act,
                             int path, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode token: routing, grouping and the expert projection in a single
 * launch -- mxfp4_moe_route_group (logits route) followed by mxfp4_expert_proj
 * for T = 1, with the same results bit for bit.  Every workgroup ranks the
 * token's E logits itself, so no launch waits on another's outputs.
 * (README "Dense routing" for the routing; README "MXFP4" and
 * src/experts.linnet fn forward_topk for the one-token product, which streams
 * each chosen expert's four-bit bytes once.)
 *
 *   logits  [1, E] bf16, finite.  1 <= E <= MXFP4_DECODE_MAX_EXPERTS,
 *           1 <= k <= min(E, MXFP4_MAX_TOPK).
 *   blocks, scales, bias, N: as for mxfp4_expert_proj;
 *           32 <= K <= MXFP4_DECODE_MAX_K, K % 32 == 0.
 *   x       x_per_slot == 0: [1, K] bf16; x_per_slot != 0: [1, k, K] bf16.
 *   topk_ids [1, k] i32, gates [1, k] f32 (or NULL), expert_offsets [E + 1] i32,
 *   sorted_rows [k] i32, error_word [1] i32 (or NULL): out, exactly as
 *           mxfp4_moe_route_group writes them for T = 1.
 *   out     [1, k, N] f32 out, as mxfp4_expert_proj writes it (GEMV path).
 * One kernel launch, no workspace.  A NaN logit: as mxfp4_moe_route_group
 * (ids -1, gates 0, zero offsets, sorted_rows untouched, error_word
 * MXFP4_ROUTE_ERR_ID_RANGE) and out is not written.
 */
int mxfp4_moe_decode(const uint16_t* logits, int E, int k, const uint8_t* blocks, const uint8_t* scales,
                     const uint16_t* bias, int N, int K, const uint16_t* x, int x_per_slot, int32_t* topk_ids,
                     float* gates, int32_t* expert_offsets, int32_t* sorted_rows, int32_t* error_word, float* out,
                     void* stream);

/*
 * One decode token through the gate/up projection and the gated activation in
 * a single launch: mxfp4_moe_route_group (logits route) followed by
 * mxfp4_expert_proj_swiglu for T = 1, with the same results bit for bit.
 * (README "Dense routing"; src/experts.linnet fn forward_topk and fn activate:
 * the gate/up product of the token's experts through the gpt-oss activation,
 * even rows the gate and odd rows the multiplier.)
 *
 *   logits, E, k, blocks, scales, bias, K, topk_ids, gates, expert_offsets,
 *   sorted_rows, error_word: as for mxfp4_moe_decode (one shared input row x
 *           [1, K] bf16).  N even.
 *   act     [1, k, N / 2] bf16 out, as mxfp4_expert_proj_swiglu writes it.
 * One kernel launch, no workspace; the NaN-logit behaviour of mxfp4_moe_decode.
 */
int mxfp4_moe_decode_swiglu(const uint16_t* logits, int E, int k, const uint8_t* blocks, const uint8_t* scales,
                            const uint16_t* bias, int N, int K, const uint16_t* x, int32_t* topk_ids, float* gates,
                            int32_t* expert_offsets, int32_t* sorted_rows, int32_t* error_word, uint16_t* act,
                            void* stream);

/*
 * A decode batch of up to MXFP4_DECODE_MAX_T tokens: routing, grouping and the
 * expert projection in a single launch -- mxfp4_moe_route_group (logits route)
 * followed by mxfp4_expert_proj on the GEMV path, with the same results bit for
 * bit.  The workgroups of each expert rank that expert among every token's
 * logits themselves, so no launch waits on another's outputs; one more
 * workgroup routes and groups the batch into the routing outputs with the code
 * of the routing launch.  T = 1 runs mxfp4_moe_decode.
 * (README "Dense routing" for the routing; README "Loading" and
 * src/experts.linnet fn forward_topk for the decode product, which streams each
 * chosen expert's four-bit bytes once for all of its tokens.)
 *
 *   logits  [T, E] bf16.  1 <= T <= MXFP4_DECODE_MAX_T,
 *           1 <= E <= MXFP4_DECODE_MAX_EXPERTS, 1 <= k <= min(E, MXFP4_MAX_TOPK).
 *   blocks, scales, bias, N: as for mxfp4_expert_proj;
 *           32 <= K <= MXFP4_DECODE_MAX_K, K % 32 == 0.
 *   x       x_per_slot == 0: [T, K] bf16; x_per_slot != 0: [T, k, K] bf16.
 *           16-byte aligned.
 *   topk_ids [T, k] i32, gates [T, k] f32 (or NULL), expert_offsets [E + 1]
 *   i32, sorted_rows [T * k] i32, error_word [1] i32 (or NULL): out, exactly
 *           as mxfp4_moe_route_group writes them.
 *   out     [T, k, N] f32 out, as mxfp4_expert_proj writes it (GEMV path).
 * One kernel launch, no workspace.  A token with a NaN logit: as
 * mxfp4_moe_route_group (ids -1 and gates 0 in its slots, its rows left out of
 * the grouping, error_word MXFP4_ROUTE_ERR_ID_RANGE), and its rows of out are
 * not written.
 */
int mxfp4_moe_decode_batch(const uint16_t* logits, int T, int E, int k, const uint8_t* blocks,
                           const uint8_t* scales, const uint16_t* bias, int N, int K, const uint16_t* x,
                           int x_per_slot, int32_t* topk_ids, float* gates, int32_t* expert_offsets,
                           int32_t* sorted_rows, int32_t* error_word, float* out, void* stream);

/*
 * The same through the gate/up projection and the gated activation:
 * mxfp4_moe_route_group (logits route) followed by mxfp4_expert_proj_swiglu on
 * the GEMV path, with the same results bit for bit.  (src/experts.linnet fn
 * activate: even rows the gate, odd rows the multiplier.)
 *
 *   logits, T, E, k, blocks, scales, bias, K, topk_ids, gates, expert_offsets,
 *   sorted_rows, error_word: as for mxfp4_moe_decode_batch (x [T, K] bf16, one
 *           row per token).  N even.
 *   act     [T, k, N / 2] bf16 out, as mxfp4_expert_proj_swiglu writes it.
 * One kernel launch, no workspace; the NaN-logit behaviour of
 * mxfp4_moe_decode_batch.
 */
int mxfp4_moe_decode_batch_swiglu(const uint16_t* logits, int T, int E, int k, const uint8_t* blocks,
                                  const uint8_t* scales, const uint16_t* bias, int N, int K, const uint16_t* x,
                                  int32_t* topk_ids, float* gates, int32_t* expert_offsets, int32_t* sorted_rows,
                                  int32_t* error_word, uint16_t* act, void* stream);

/*
 * One decode token's projection through all of its k experts and the
 * gate-weighted combine, in one launch: mxfp4_expert_proj (T = 1, GEMV path)
 * followed by moe_combine, with the same results bit for bit.
 * (src/experts.linnet fn forward_topk: each slot's down product and the f32
 * sum over k; fn down_bias_of: the down bias weighed by the router weights.)
 *
 *   blocks, scales, bias, E, N: as for mxfp4_expert_proj;
 *           32 <= K <= MXFP4_DECODE_MAX_K, K % 32 == 0.
 *   x       x_per_slot == 0: [1, K] bf16; x_per_slot != 0: [1, k, K] bf16 (the
 *           down projection's per-slot inputs, e.g. mxfp4_moe_decode_swiglu's
 *           activations).  16-byte aligned.
 *   k       1 <= k <= min(E, MXFP4_MAX_TOPK).
 *   topk_ids [1, k] i32, gates [1, k] f32: the token's routing, as
 *           mxfp4_moe_route_group or mxfp4_moe_decode writes it.  A slot whose
 *           id lies outside [0, E) is not projected and, like a slot with
 *           gate 0, contributes nothing to y.
 *   out     [1, k, N] f32 out (each slot's projection, bias included), or NULL.
 *   y       [1, N] f32 out: y[n] = sum over slots, in slot order, of
 *           gates[s] * out[s, n] (one fused multiply-add per slot).
 * One kernel launch, no workspace.
 */
int mxfp4_expert_proj_combine(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                              int K, const uint16_t* x, int x_per_slot, int k, const int32_t* topk_ids,
                              const float* gates, float* out, float* y, void* stream);

/*
 * The routed projection of many tokens and the gate-weighted combine:
 * mxfp4_expert_proj followed by moe_combine, with the same out and y bit for
 * bit whenever every unrouted slot has gate 0 (as mxfp4_moe_route_group
 * writes them).  On the grouped-GEMM path the combine runs inside the GEMM:
 * per (token, 192-column weight panel) an arrival counter in the workspace,
 * set by the GEMM's pre-pass, counts the token's routed rows as their tiles
 * finish, and the tile that brings the last of them sums the token's k rows
 * over its panel in slot order.  On the GEMV path, while T * k <= E and K <=
 * MXFP4_DECODE_MAX_K, one launch: a workgroup runs all k slots of one token
 * over its weight rows and sums them (as mxfp4_expert_proj_combine does for
 * one token); otherwise the combine is a second launch.
 * (src/experts.linnet fn forward_routed: the routed rows' down products
 * summed per token with the router weights; fn down_bias_of: the bias
 * weighed by them, already inside out here.)
 *
 *   blocks, scales, bias, E, N, K, x, x_per_slot, T, k, expert_offsets,
 *   sorted_rows, path, workspace, workspace_bytes: as for mxfp4_expert_proj
 *           (the same workspace size).
 *   topk_ids [T, k] i32, gates [T, k] f32: the routing that expert_offsets and
 *           sorted_rows group, from the same mxfp4_moe_route_group call.  A slot
 *           is routed when its id lies in [0, E); the grouping must hold
 *           exactly the routed slots (otherwise y is unspecified, though every
 *           access stays inside the arrays).
 *   out     [T, k, N] f32 out, as mxfp4_expert_proj writes it; at most 4 GiB
 *           (T * k * N * 4 bytes; larger returns MXFP4_ERR_INVALID_ARG).
 *   y       [T, N] f32 out: y[t, n] = sum over slots s, in slot order, of
 *           gates[t, s] * out[t, s, n], one fused multiply-add per slot; an
 *           unrouted slot or one with gate 0 adds a zero product.  A token with
 *           no routed slot gets y = 0.
 * Deterministic: the sum order does not depend on the order in which tiles
 * finish.  T = 0 returns MXFP4_OK and enqueues nothing.
 */
int mxfp4_expert_proj_combine_routed(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E,
                                     int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                                     const int32_t* topk_ids, const float* gates, const int32_t* expert_offsets,
                                     const int32_t* sorted_rows, float* out, float* y, int path, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * MXFP4 -> bf16 dequantization of a weight tensor, in its own layout.
 * (README "MXFP4": rows of 32-element blocks, 16 code bytes per block with the
 * even element in the low nibble, one E8M0 scale byte per block, a weight is
 * its E2M1 value times 2 ** (scale - 127), and the values are exact in bf16;
 * dequantize_mxfp4 returns the checkpoint's [Experts, Rows, N] layout.)
 *
 *   blocks  [rows, K/32, 16] u8, 16-byte aligned (any leading dimensions
 *           flattened into rows, e.g. rows = E * N).
 *   scales  [rows, K/32] u8.
 *   rows >= 0, K >= 32 and K % 32 == 0.
 *   out     [rows, K] bf16 out, 16-byte aligned:
 *           out[r, j] = e2m1(code of element j) * 2 ** (scales[r, j / 32] - 127),
 *           exact (for scale bytes 0..252 every code's value is a bf16).
 * rows = 0 returns MXFP4_OK and enqueues nothing.
 */
int mxfp4_dequantize(const uint8_t* blocks, const uint8_t* scales, long long rows, int K, uint16_t* out,
                     void* stream);

/*
 * Gate-weighted combine of the k projections of each token.
 * (src/experts.linnet fn forward_topk: the sum over k in f32; fn down_bias_of:
 * the down bias carries the router weights -- here the bias is already inside
 * proj, so weighing proj weighs it too.)
 *
 *   proj  [T, k, N] f32, gates [T, k] f32, y [T, N] f32 out (overwritten):
 *   y[t, n] = sum_{s = 0}^{k-1} gates[t, s] * proj[t, s, n], accumulated in f32
 *   in slot order with fused multiply-adds.  A slot with gate 0 adds nothing
 *   whatever its proj row holds (the routing gives gate 0 to the slots it
 *   could not route, whose rows the projection never writes).
 *   T >= 0, k >= 1, N >= 1.  T = 0 returns MXFP4_OK and enqueues nothing.
 */
int moe_combine(const float* proj, const float* gates, int T, int k, int N, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_MOE_H */

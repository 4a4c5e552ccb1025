// Internal launchers of the gfx950 kernels.  Each enqueues on `stream` and
// returns the hipError_t of the launch; the arguments have been checked by
// the C ABI layer (capi.cpp) before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxfp4 {

// route_group.hip
hipError_t launch_route_group(const uint16_t* logits, const int32_t* ids_in, int T, int E, int k,
                              int32_t* topk_ids, float* gates, int32_t* offsets, int32_t* sorted_rows,
                              int32_t* error_word, hipStream_t stream);

// dense router weights [T, E]: softmax over the logits with every expert
// ranked k or worse floored (exactly zero)
hipError_t launch_dense_route(const uint16_t* logits, int T, int E, int k, float* probs, hipStream_t stream);

// expert_gemv.hip
size_t gemv_lds_bytes(int T, int K);
// act != NULL: the gated activation of (even, odd) output row pairs, bf16
// [T * k, N / 2], instead of out
hipError_t launch_expert_gemv(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias,
                              int E, int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                              const int32_t* offsets, const int32_t* sorted_rows, float* out, uint16_t* act,
                              hipStream_t stream);
hipError_t launch_moe_decode_t1(const uint16_t* logits, int E, int k, const uint8_t* blocks, const uint8_t* scales,
                                const uint16_t* bias, int N, int K, const uint16_t* x, int x_per_slot,
                                int32_t* topk_ids, float* gates, int32_t* offsets, int32_t* sorted_rows,
                                int32_t* error_word, float* out, uint16_t* act, hipStream_t stream);
// T <= 64 tokens (E <= 64): routing, grouping and the projection in one launch
hipError_t launch_moe_decode_batch(const uint16_t* logits, int T, int E, int k, const uint8_t* blocks,
                                   const uint8_t* scales, const uint16_t* bias, int N, int K, const uint16_t* x,
                                   int x_per_slot, int32_t* topk_ids, float* gates, int32_t* offsets,
                                   int32_t* sorted_rows, int32_t* error_word, float* out, uint16_t* act,
                                   hipStream_t stream);

// one token, k slots (topk_ids [k], gates [k]): out [k, N] (or NULL) and the
// gate-weighted combine y [N] in one launch
hipError_t launch_proj_combine_t1(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                                  int K, const uint16_t* x, int x_per_slot, int k, const int32_t* topk_ids,
                                  const float* gates, float* out, float* y, hipStream_t stream, int T = 1);
// the routed projection (GEMV path) and the gate-weighted combine: one launch
// while T * k <= E (and K <= 3072), else the projection and the combine
hipError_t launch_expert_gemv_combine(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E,
                                      int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                                      const int32_t* offsets, const int32_t* sorted_rows, const int32_t* topk_ids,
                                      const float* gates, float* out, float* y, hipStream_t stream);

// expert_gemm.hip
size_t gemm_workspace_bytes(int E, int N, int T, int k, int K, int x_per_slot);
// the static scratch of the current device (its device address; resolved once
// per device) and its size, = MXFP4_NOALLOC_SCRATCH_BYTES
constexpr size_t kGemmStaticScratchBytes = (size_t)128 << 20;
hipError_t gemm_static_scratch(void** ptr);
// y != NULL: out [T, k, N] and then, fused, y [T, N] = the gate-weighted
// combine of each token's routed slots (ids [T, k], gates [T, k])
hipError_t launch_expert_gemm(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias,
                              int E, int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                              const int32_t* offsets, const int32_t* sorted_rows, float* out, uint16_t* act,
                              void* workspace, hipStream_t stream, const int32_t* ids = nullptr,
                              const float* gates = nullptr, float* y = nullptr);

// dequantize.hip: nblocks MXFP4 blocks (16 code bytes + 1 scale byte each) ->
// 32 bf16 weights each
hipError_t launch_dequantize(const uint8_t* blocks, const uint8_t* scales, size_t nblocks, uint16_t* out,
                             hipStream_t stream);

// router.hip: logits [T, E] bf16 = x [T, H] . w [E, H]^T + bias (fp32 sums, rounded once)
hipError_t launch_router(const uint16_t* x, const uint16_t* w, const uint16_t* bias, int T, int H, int E,
                         uint16_t* logits, hipStream_t stream);

// combine.hip; ids != NULL: a slot whose id lies outside [0, E) adds nothing
// either (as a slot with gate 0)
hipError_t launch_combine(const float* proj, const float* gates, int T, int k, int N, float* y,
                          hipStream_t stream, const int32_t* ids = nullptr, int E = 0);

}  // namespace mxfp4

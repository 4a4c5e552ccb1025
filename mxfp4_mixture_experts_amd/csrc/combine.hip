// Gate-weighted combine of a token's k expert outputs, for gfx950.
//
// gpt-oss-20b files page, src/experts.linnet fn forward_topk: the expert sum
// is taken in f32; fn down_bias_of: the down bias is weighed by the router
// weights (it is already part of each projection row here).
//
// y[t, n] = sum_s gates[t, s] * proj[t, s, n], one fused multiply-add per slot
// in slot order, so the result does not depend on the launch shape.  A slot
// whose gate is 0 adds nothing, whatever its row holds: the routing gives gate
// 0 to the slots it could not route, whose projection rows are never written.
// (For a finite value v, fma(0, v, acc) = acc, so this changes no other sum.)
// Called with the routing's ids, a slot whose id lies outside [0, E) (never
// projected) adds a zero product too, whatever its gate.
// The kernel is a pure HBM stream: each thread owns 4 consecutive columns of
// one token (128-bit loads and stores), the k gates of the token are read
// once per thread from the cache.

#include "kernels.h"
#include "common.h"

namespace mxfp4 {
namespace {

constexpr int kCombineThreads = 256;

// the weight of slot row r: its gate, or 0 where ids marks the slot unrouted
__device__ __forceinline__ float slot_gate(const float* __restrict__ gates, const int32_t* __restrict__ ids, int E,
                                           size_t r) {
  const float g = gates[r];
  return (ids && (unsigned)ids[r] >= (unsigned)E) ? 0.f : g;
}

__global__ __launch_bounds__(kCombineThreads) void combine_vec4_kernel(
    const float* __restrict__ proj, const float* __restrict__ gates, int T, int k, int N4,
    float* __restrict__ y, const int32_t* __restrict__ ids, int E) {
  const size_t total = (size_t)T * N4;
  const size_t stride = (size_t)gridDim.x * kCombineThreads;
  for (size_t i = (size_t)blockIdx.x * kCombineThreads + threadIdx.x; i < total; i += stride) {
    const size_t t = i / N4;
    const size_t c = i - t * N4;
    const float4* p = reinterpret_cast<const float4*>(proj) + (t * k) * N4 + c;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < k; s++) {
      const float g = gates[t * k + s];
      float4 v = load_nt(p + (size_t)s * N4);  // unconditional: no branch per load
      if (slot_gate(gates, ids, E, t * k + s) == 0.f) v = make_float4(0.f, 0.f, 0.f, 0.f);
      acc.x = fmaf(g, v.x, acc.x);
      acc.y = fmaf(g, v.y, acc.y);
      acc.z = fmaf(g, v.z, acc.z);
      acc.w = fmaf(g, v.w, acc.w);
    }
    reinterpret_cast<float4*>(y)[i] = acc;
  }
}

__global__ __launch_bounds__(kCombineThreads) void combine_scalar_kernel(
    const float* __restrict__ proj, const float* __restrict__ gates, int T, int k, int N,
    float* __restrict__ y, const int32_t* __restrict__ ids, int E) {
  const size_t total = (size_t)T * N;
  const size_t stride = (size_t)gridDim.x * kCombineThreads;
  for (size_t i = (size_t)blockIdx.x * kCombineThreads + threadIdx.x; i < total; i += stride) {
    const size_t t = i / N;
    const size_t n = i - t * N;
    float acc = 0.f;
    for (int s = 0; s < k; s++) {
      const float g = gates[t * k + s];
      const float v = proj[(t * k + s) * N + n];
      acc = fmaf(g, slot_gate(gates, ids, E, t * k + s) == 0.f ? 0.f : v, acc);
    }
    y[i] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const float* proj, const float* gates, int T, int k, int N, float* y,
                          hipStream_t stream, const int32_t* ids, int E) {
  const bool vec = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(proj) | reinterpret_cast<uintptr_t>(y)) % 16 == 0);
  const size_t items = (size_t)T * (vec ? N / 4 : N);
  size_t blocks = (items + kCombineThreads - 1) / kCombineThreads;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
  if (vec)
    hipLaunchKernelGGL(combine_vec4_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0, stream, proj,
                       gates, T, k, N / 4, y, ids, E);
  else
    hipLaunchKernelGGL(combine_scalar_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0, stream, proj,
                       gates, T, k, N, y, ids, E);
  return hipGetLastError();
}

}  // namespace mxfp4

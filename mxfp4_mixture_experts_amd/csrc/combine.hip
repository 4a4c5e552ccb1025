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

// one-wave workgroups: more of them spread over the CUs (T = 64 down decode
// 3.5 -> 3.2 us, Zipf down prefill 21.4 -> 20.3 us against 256 threads)
constexpr int kCombineThreads = 64;

// the weight of slot row r: its gate, or 0 where ids marks the slot unrouted
__device__ __forceinline__ float slot_gate(const float* __restrict__ gates, const int32_t* __restrict__ ids, int E,
                                           size_t r) {
  const float g = gates[r];
  return (ids && (unsigned)ids[r] >= (unsigned)E) ? 0.f : g;
}

// I: the index type, 32-bit whenever every float4 index of proj fits (no
// 64-bit divisions then)
template <typename I>
__global__ __launch_bounds__(kCombineThreads) void combine_vec4_kernel(
    const float* __restrict__ proj, const float* __restrict__ gates, int T, int k, int N4,
    float* __restrict__ y, const int32_t* __restrict__ ids, int E) {
  const I total = (I)T * (I)N4;
  const I stride = (I)gridDim.x * kCombineThreads;
  for (I i = (I)blockIdx.x * kCombineThreads + threadIdx.x; i < total; i += stride) {
    const I t = i / (I)N4;
    const I c = i - t * (I)N4;
    const float4* p = reinterpret_cast<const float4*>(proj) + (t * k) * N4 + c;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // four slots' loads in flight at a time (unconditional, from a clamped
    // slot), then their sums in slot order
    for (int s0 = 0; s0 < k; s0 += 4) {
      float4 v[4];
      float g[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int s = min(s0 + u, k - 1);
        v[u] = load_nt(p + (size_t)s * N4);
        g[u] = slot_gate(gates, ids, E, t * k + s);
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        if (s0 + u >= k) break;
        if (g[u] == 0.f) v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        acc.x = fmaf(g[u], v[u].x, acc.x);
        acc.y = fmaf(g[u], v[u].y, acc.y);
        acc.z = fmaf(g[u], v[u].z, acc.z);
        acc.w = fmaf(g[u], v[u].w, acc.w);
      }
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
  if (vec && (size_t)T * k * (N / 4) + (size_t)blocks * kCombineThreads < 0xFFFFFFFFull)
    hipLaunchKernelGGL(combine_vec4_kernel<uint32_t>, dim3((unsigned)blocks), dim3(kCombineThreads), 0, stream, proj,
                       gates, T, k, N / 4, y, ids, E);
  else if (vec)
    hipLaunchKernelGGL(combine_vec4_kernel<size_t>, dim3((unsigned)blocks), dim3(kCombineThreads), 0, stream, proj,
                       gates, T, k, N / 4, y, ids, E);
  else
    hipLaunchKernelGGL(combine_scalar_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0, stream, proj,
                       gates, T, k, N, y, ids, E);
  return hipGetLastError();
}

}  // namespace mxfp4

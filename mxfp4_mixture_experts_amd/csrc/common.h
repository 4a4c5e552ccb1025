// Small device helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace mxfp4 {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 128-bit loads marked non-temporal (streamed data that is read once)
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_nt(const float4* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, rounded to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The gpt-oss gated activation of one (gate, up) pair of projection outputs
// (gpt-oss-20b files page, src/experts.linnet: constants LIMIT = 7 and
// ALPHA = 1.702, fn activate): the gate clamped from above at LIMIT, the
// multiplier to [-LIMIT, LIMIT], then (up + 1) * gate * sigmoid(ALPHA * gate).
// fp32, with sigmoid(ALPHA g) = 1 / (1 + 2^(-ALPHA log2(e) g)) on the
// hardware exp2 and reciprocal (each within 1 ulp); a very negative gate gives
// 2^(+large) = inf and a zero product.
constexpr float kSwigluLimit = 7.0f;
constexpr float kSwigluAlphaLog2e = (float)(1.702 * 1.4426950408889634);
__device__ __forceinline__ float swiglu(float gate, float up) {
  const float g = fminf(gate, kSwigluLimit);
  const float u = fminf(fmaxf(up, -kSwigluLimit), kSwigluLimit);
  const float e = __builtin_amdgcn_exp2f(-kSwigluAlphaLog2e * g);
  return (u + 1.0f) * (g * __builtin_amdgcn_rcpf(1.0f + e));
}

// The value of lane l ^ 1 (a swap within lane pairs, one DPP move)
__device__ __forceinline__ float pair_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// popcount of the lanes below this one in a 64-bit lane mask
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

// Sum over the 64 lanes of a wave; every lane receives the total.  The order
// of the additions is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v += __shfl_xor(v, 32, 64);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 8, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 1, 64);
  return v;
}

// A kernel's dynamic-LDS limit raised once per device: the attribute belongs
// to the device the call is made on, and launches from several host threads
// may race to set it.
class DynLdsLimit {
 public:
  DynLdsLimit(const void* func, int bytes) : func_(func), bytes_(bytes) {}
  hipError_t ensure() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu_);
    if (done_[dev]) return hipSuccess;
    e = hipFuncSetAttribute(func_, hipFuncAttributeMaxDynamicSharedMemorySize, bytes_);
    if (e == hipSuccess) done_[dev] = true;
    return e;
  }

 private:
  static constexpr int kDevices = 64;
  const void* func_;
  int bytes_;
  std::mutex mu_;
  bool done_[kDevices] = {};
};

}  // namespace mxfp4

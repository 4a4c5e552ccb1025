// MXFP4 -> bf16 dequantization of a weight tensor in the checkpoint's own
// layout (gpt-oss-20b files page, README "MXFP4": rows of 32-element blocks,
// 16 code bytes with the even element in the low nibble, one E8M0 scale byte
// per block; a weight is its E2M1 value times 2 ** (scale - 127); the values
// are exact in bf16, and dequantize_mxfp4 keeps the [Experts, Rows, N] layout).
//
// HBM streaming: four consecutive lanes share a block, lane taking word
// i % 4 of it (8 codes) and the block's scale byte, so that the word loads and
// the 16-byte stores of consecutive lanes are contiguous (eight such loads per
// lane in flight); each code byte
// becomes two bf16 weights through the gfx950 convert
// v_cvt_scalef32_pk_bf16_fp4 (E2M1 value times the block's E8M0 factor).  A
// grid-stride loop covers any number of blocks.

#include "kernels.h"
#include "common.h"

namespace mxfp4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kDqThreads = 256;

__device__ __forceinline__ float e8m0_factor(uint32_t s) {
  // 2^(s - 127) as an fp32 bit pattern; s = 0 is the subnormal 2^-127
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

constexpr int kDqUnroll = 8;  // words per thread in flight: each wave has 8 x 256 contiguous bytes requested

__global__ __launch_bounds__(kDqThreads) void dequantize_kernel(const uint32_t* __restrict__ words,
                                                                const uint8_t* __restrict__ scales,
                                                                size_t nwords, uint4* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const size_t wave = ((size_t)blockIdx.x * kDqThreads + threadIdx.x) >> 6;
  const size_t waves = (size_t)gridDim.x * (kDqThreads / 64);
  // wave-sized spans of 64 * kDqUnroll words; load u of a lane is word span + 64 u + lane
  for (size_t base = wave * 64 * kDqUnroll; base < nwords; base += waves * 64 * kDqUnroll) {
    uint32_t w[kDqUnroll];
    uint32_t sb[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; u++) {
      const size_t i = min(base + 64 * u + lane, nwords - 1);  // unconditional loads; stores masked
      w[u] = __builtin_nontemporal_load(words + i);
      sb[u] = scales[i >> 2];
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; u++) {
      const size_t i = base + 64 * u + lane;
      const float sf = e8m0_factor(sb[u]);
      // byte j of the word: elements 2 j (low nibble) and 2 j + 1 of the word's 8
      const uint32_t o0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], sf, 0));
      const uint32_t o1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], sf, 1));
      const uint32_t o2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], sf, 2));
      const uint32_t o3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], sf, 3));
      if (i < nwords) __builtin_nontemporal_store(u32x4_t{o0, o1, o2, o3}, reinterpret_cast<u32x4_t*>(out + i));
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* blocks, const uint8_t* scales, size_t nblocks, uint16_t* out,
                             hipStream_t stream) {
  const size_t nwords = nblocks * 4;
  const size_t per_wg = (size_t)kDqThreads * kDqUnroll;
  const size_t want = (nwords + per_wg - 1) / per_wg;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);  // 32 workgroups per CU, then grid-stride
  hipLaunchKernelGGL(dequantize_kernel, dim3(grid), dim3(kDqThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(blocks), scales, nwords, reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace mxfp4

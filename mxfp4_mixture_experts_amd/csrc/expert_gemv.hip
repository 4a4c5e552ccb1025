// Decode expert projection: an HBM-streaming MXFP4 GEMV for gfx950.
//
// Computes, for every routed row r grouped under expert e,
//   out[r, n] = bias[e, n] + sum_j W[e, n, j] * x_src(r)[j]
// with W[e, n, j] = e2m1(code) * 2 ** (scale[e, n, j / 32] - 127)
// (gpt-oss-20b files page, README "MXFP4" for the format; src/experts.linnet
// fn forward_topk for the decode product, which reads each chosen expert's
// four-bit bytes in place).
//
// Work decomposition.  A workgroup (4 waves) serves one expert that has at
// least one routed row (blockIdx.y = the g-th such expert) and 16 consecutive
// weight rows (4 per wave).  The expert's x rows (at most MAXM per pass) are
// staged in LDS as bf16.  A wave treats its 4 weight rows, which are
// contiguous in memory (4 * K/32 blocks of 16 bytes), as one flat stream:
// lane l loads block f = 64 * u + l with a 128-bit load, so every load
// instruction of the wave reads 1 KiB of consecutive HBM; UNROLL loads per lane
// are issued before any is used.  A block's 32 codes are decoded in registers
// by the gfx950 FP4->bf16 convert (v_cvt_scalef32_pk_bf16_fp4, scale 1: the
// hardware 16-entry code table), multiplied with bf16 x in pairs by
// v_dot2_f32_bf16 (bf16 x bf16 products are exact in fp32), and the block's
// partial sum is scaled by its E8M0 exponent with v_ldexp_f32 (exact).  Each
// lane keeps one fp32 accumulator per (x row, weight row); a fixed-order
// butterfly over the 64 lanes finishes each output.  No atomics: the result is
// deterministic.

#include "kernels.h"
#include "common.h"

namespace mxfp4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kRowsPerWave = 4;
constexpr int kUnroll = 6;

__device__ __forceinline__ float dot2_bf16(bf16x2_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(w, __builtin_bit_cast(bf16x2_t, x), acc, false);
}

// The g-th expert (in index order) that has at least one grouped row.
__device__ __forceinline__ bool find_group(const int32_t* offsets, int E, int R, int g, int& e_out,
                                           int& m0, int& m1) {
  int c = 0;
  int prev = min(max(offsets[0], 0), R);
  for (int e = 0; e < E; e++) {
    const int nxt = min(max(offsets[e + 1], prev), R);
    if (nxt > prev) {
      if (c == g) {
        e_out = e;
        m0 = prev;
        m1 = nxt;
        return true;
      }
      c++;
    }
    prev = nxt;
  }
  return false;
}

template <int MAXM>
__global__ __launch_bounds__(kGemvThreads) void expert_gemv_kernel(
    const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ bias, int E, int N, int K, const uint16_t* __restrict__ x,
    int x_per_slot, int T, int k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_rows, float* __restrict__ out) {
  extern __shared__ uint4 xs[];  // [MAXM][K / 8] bf16 x rows of this expert
  const int KB = K >> 5;
  const int K8 = K >> 3;
  const int R = T * k;
  int e, m0, m1;
  if (!find_group(offsets, E, R, blockIdx.y, e, m0, m1)) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_first = (blockIdx.x * kGemvWaves + wave) * kRowsPerWave;
  const int nrows = min(kRowsPerWave, N - n_first);
  const int total = nrows * KB;  // 16-byte blocks in this wave's stream
  const uint4* wp = reinterpret_cast<const uint4*>(blocks + ((size_t)e * N + max(n_first, 0)) * KB * 16);
  const uint8_t* sp = scales + ((size_t)e * N + max(n_first, 0)) * KB;

  for (int mb = m0; mb < m1; mb += MAXM) {
    const int mc = min(MAXM, m1 - mb);
    for (int i = threadIdx.x; i < MAXM * K8; i += kGemvThreads) {
      const int m = i / K8;
      const int c = i - m * K8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < mc) {
        const int r = sorted_rows[mb + m];
        if (r >= 0 && r < R) {
          const size_t src = x_per_slot ? (size_t)r : (size_t)(r / k);
          v = reinterpret_cast<const uint4*>(x + src * K)[c];
        }
      }
      xs[i] = v;
    }
    __syncthreads();

    if (nrows > 0) {
      float acc[MAXM][kRowsPerWave];
#pragma unroll
      for (int m = 0; m < MAXM; m++)
#pragma unroll
        for (int j = 0; j < kRowsPerWave; j++) acc[m][j] = 0.f;

      for (int f0 = 0; f0 < total; f0 += 64 * kUnroll) {
        uint4 w[kUnroll];
        int s[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
          const int f = f0 + 64 * u + lane;
          if (f < total) {
            w[u] = load_nt(wp + f);
            s[u] = sp[f];
          } else {
            w[u] = make_uint4(0u, 0u, 0u, 0u);
            s[u] = 127;
          }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
          const int f = f0 + 64 * u + lane;
          if (f < total) {
            const int rr = (f >= KB) + (f >= 2 * KB) + (f >= 3 * KB);
            const int kb = f - rr * KB;
            bf16x2_t wv[16];
            const uint32_t wd[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
            for (int d = 0; d < 4; d++) {
              wv[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 0);
              wv[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 1);
              wv[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 2);
              wv[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], 1.0f, 3);
            }
#pragma unroll
            for (int m = 0; m < MAXM; m++) {
              if (m < mc) {
                const uint4* xp = xs + m * K8 + kb * 4;
                float p = 0.f;
#pragma unroll
                for (int d = 0; d < 4; d++) {
                  const uint4 xv = xp[d];
                  p = dot2_bf16(wv[4 * d + 0], xv.x, p);
                  p = dot2_bf16(wv[4 * d + 1], xv.y, p);
                  p = dot2_bf16(wv[4 * d + 2], xv.z, p);
                  p = dot2_bf16(wv[4 * d + 3], xv.w, p);
                }
                const float v = ldexpf(p, s[u] - 127);
#pragma unroll
                for (int j = 0; j < kRowsPerWave; j++) acc[m][j] += (rr == j) ? v : 0.f;
              }
            }
          }
        }
      }

#pragma unroll
      for (int m = 0; m < MAXM; m++) {
        if (m < mc) {
          const int r = sorted_rows[mb + m];
#pragma unroll
          for (int j = 0; j < kRowsPerWave; j++) {
            const float tot = wave_sum(acc[m][j]);
            if (lane == 0 && j < nrows && r >= 0 && r < R) {
              const int n = n_first + j;
              const float b = bias ? bf16_bits_to_f32(bias[(size_t)e * N + n]) : 0.f;
              out[(size_t)r * N + n] = tot + b;
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_expert_gemv(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias,
                              int E, int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                              const int32_t* offsets, const int32_t* sorted_rows, float* out,
                              hipStream_t stream) {
  const int R = T * k;
  const int groups = R < E ? R : E;
  const int rows_per_block = kGemvWaves * kRowsPerWave;
  const dim3 grid((N + rows_per_block - 1) / rows_per_block, groups);
  if (T == 1) {
    hipLaunchKernelGGL(expert_gemv_kernel<1>, grid, dim3(kGemvThreads), (size_t)1 * K * 2, stream, blocks,
                       scales, bias, E, N, K, x, x_per_slot, T, k, offsets, sorted_rows, out);
  } else if (T == 2) {
    hipLaunchKernelGGL(expert_gemv_kernel<2>, grid, dim3(kGemvThreads), (size_t)2 * K * 2, stream, blocks,
                       scales, bias, E, N, K, x, x_per_slot, T, k, offsets, sorted_rows, out);
  } else {
    hipLaunchKernelGGL(expert_gemv_kernel<4>, grid, dim3(kGemvThreads), (size_t)4 * K * 2, stream, blocks,
                       scales, bias, E, N, K, x, x_per_slot, T, k, offsets, sorted_rows, out);
  }
  return hipGetLastError();
}

}  // namespace mxfp4

// Decode expert projection: an HBM-streaming MXFP4 GEMV for gfx950 whose
// products are exact.
//
// Computes, for every routed row r grouped under expert e,
//   out[r, n] = bias[e, n] + sum_j W[e, n, j] * x_src(r)[j]
// with W[e, n, j] = e2m1(code) * 2 ** (scale[e, n, j / 32] - 127)
// (gpt-oss-20b files page, README "MXFP4" for the format; src/experts.linnet
// fn forward_topk for the decode product, which reads each chosen expert's
// four-bit bytes in place).
//
// Work decomposition.  A workgroup serves one expert that has routed rows
// (blockIdx.y = the g-th such expert, found with one ballot over the expert
// offsets) and WAVES * 16 consecutive weight rows, 16 per wave.  Lane l of a
// wave streams weight row (16-row base + l % 16), MX block 4 * i + l / 16 for
// i = 0, 1, ...: one 128-bit load per lane per i, and every load of the wave
// covers 16 rows x 64 contiguous bytes.  The loads run a two-stage pipeline
// over chunks of NCH 128-element K groups (the next chunk is in flight while
// the current one is multiplied), and the first chunk is issued before the
// expert's token rows (up to MT per pass) are staged in LDS as bf16; the four
// MFMAs of a load accumulate into four independent accumulators.
//
// Arithmetic.  Each 32-bit word of a block (8 codes) becomes 8 bf16 weights
// through the gfx950 convert v_cvt_scalef32_pk_bf16_fp4 with the block's E8M0
// factor as its scale operand: fp4 value x 2^(s-127) is exact in bf16.  The
// weights and the bf16 activations feed v_mfma_f32_16x16x32_bf16 (16 weight
// rows x up to 16 token rows per instruction, fp32 accumulation; bf16 x bf16
// products are exact in fp32), so no lane-to-lane reduction is needed: lane l
// ends up holding out[token 4 * (l / 16) + i][row l % 16].  Deterministic.

#include "kernels.h"
#include "common.h"

namespace mxfp4 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));


// The g-th expert (in index order) with at least one routed row, found by each
// wave on its own: one ballot per 64 experts.  Offsets are clamped to [0, R].
__device__ __forceinline__ bool find_group(const int32_t* offsets, int E, int R, int g, int lane, int& e_out,
                                           int& m0, int& m1) {
  int seen = 0;
  for (int c0 = 0; c0 < E; c0 += 64) {
    const int e = c0 + lane;
    int a = 0, b = 0;
    if (e < E) {
      a = min(max(offsets[e], 0), R);
      b = min(max(offsets[e + 1], 0), R);
    }
    const bool nonempty = e < E && b > a;
    const uint64_t mask = __ballot(nonempty);
    const int cnt = __popcll(mask);
    if (g < seen + cnt) {
      const bool mine = nonempty && lanes_below(mask) == g - seen;
      const uint64_t who = __ballot(mine);
      const int src = __ffsll((long long)who) - 1;
      e_out = __shfl(e, src, 64);
      m0 = __shfl(a, src, 64);
      m1 = __shfl(b, src, 64);
      return true;
    }
    seen += cnt;
  }
  return false;
}

__device__ __forceinline__ float e8m0_to_float(uint32_t s) {
  // 2^(s - 127) as an fp32 bit pattern; s = 0 is the subnormal 2^-127
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

template <int MT, int WAVES, int NCH>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2))) void expert_gemv_kernel(
    const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ scales, const uint16_t* __restrict__ bias,
    int E, int N, int K, const uint16_t* __restrict__ x, int x_per_slot, int T, int k,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows, float* __restrict__ out) {
  // [MT + 1][XS] bf16 token rows, 16 bytes per entry: rows >= the pass's count and
  // the extra last row are zero, as is every entry past K, so every read below
  // is unconditional.  XS = 16 entries per K group (groups rounded up to whole
  // chunks of NCH) + 1 (the +1 puts 16 rows on distinct banks).
  extern __shared__ uint4 xs[];
  __shared__ int rows_lds[MT];
  const int KB = K >> 5;
  const int K8 = K >> 3;
  const int NIT = (KB + 3) >> 2;
  const int NITC = (NIT + NCH - 1) / NCH * NCH;
  const int XS = NITC * 16 + 1;
  const int R = T * k;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  int e, m0, m1;
  if (!find_group(offsets, E, R, blockIdx.y, lane, e, m0, m1)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  m1 = __builtin_amdgcn_readfirstlane(m1);

  const int n_base = (blockIdx.x * WAVES + wave) * 16;
  const int row = n_base + (lane & 15);
  const int kq = lane >> 4;
  const bool row_ok = row < N;
  // rows past N and blocks past K read real (clamped) weights and meet zero activations
  const uint4* wrow = reinterpret_cast<const uint4*>(blocks) + ((size_t)e * N + min(row, N - 1)) * KB;
  const uint8_t* srow = scales + ((size_t)e * N + min(row, N - 1)) * KB;
  const float bias_v = (bias && row_ok) ? bf16_bits_to_f32(bias[(size_t)e * N + row]) : 0.f;

  auto load_chunk = [&](int c0, uint4 (&w)[NCH], uint32_t (&s)[NCH]) {
    // groups past K re-read the row's last block; they meet zero activations
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int kb = min((c0 + i) * 4 + kq, KB - 1);
      w[i] = load_nt(wrow + kb);
      s[i] = srow[kb];
    }
  };

  for (int mb = m0; mb < m1; mb += MT) {
    const int mc = min(MT, m1 - mb);
    // ---- the first two chunks of weights are in flight while the token rows are staged
    uint4 wa[NCH], wb[NCH];
    uint32_t sa[NCH], sb[NCH];
    load_chunk(0, wa, sa);
    if (NCH < NIT) load_chunk(NCH, wb, sb);
    __syncthreads();  // the previous pass is done with the staged rows
    // token row m's source: uniform per m, so these are scalar loads
    int src[MT + 1];
#pragma unroll
    for (int m = 0; m <= MT; m++) {
      int r = -1;
      if (m < mc) {
        r = sorted_rows[mb + m];
        if (r < 0 || r >= R) r = -1;
      }
      if (threadIdx.x == 0 && m < MT) rows_lds[m] = r;
      src[m] = r < 0 ? -1 : (x_per_slot ? r : r / k);
    }
    // all of a thread's activation loads first, then the LDS stores
    constexpr int kPerRow = MT == 1 ? 4 : (MT <= 4 ? 2 : 1);  // entries per thread per row and round
    for (int c0 = 0; c0 < XS; c0 += kPerRow * WAVES * 64) {
      uint4 v[MT + 1][kPerRow];
#pragma unroll
      for (int m = 0; m <= MT; m++)
#pragma unroll
        for (int j = 0; j < kPerRow; j++) {
          const int c = c0 + j * WAVES * 64 + threadIdx.x;
          v[m][j] = (src[m] >= 0 && c < K8) ? reinterpret_cast<const uint4*>(x + (size_t)src[m] * K)[c]
                                            : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
      for (int m = 0; m <= MT; m++)
#pragma unroll
        for (int j = 0; j < kPerRow; j++) {
          const int c = c0 + j * WAVES * 64 + threadIdx.x;
          if (c < XS) xs[m * XS + c] = v[m][j];
        }
    }
    __syncthreads();

    f32x4_v acc[4];
#pragma unroll
    for (int d = 0; d < 4; d++) acc[d] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    const uint4* xrow = xs + ((lane & 15) < mc ? (lane & 15) : MT) * XS + kq * 4;

    // ---- two-stage pipeline over chunks of NCH K groups: chunk c + 1 loads
    // while chunk c converts and multiplies (4 MFMAs per 128-bit load into four
    // independent accumulators; A = token rows, lane l: row l % 16; B = weights)
    auto compute_chunk = [&](int c0, const uint4 (&w)[NCH], const uint32_t (&s)[NCH]) {
      uint4 xv[4], xn[4];
#pragma unroll
      for (int d = 0; d < 4; d++) xv[d] = xrow[c0 * 16 + d];
#pragma unroll
      for (int i = 0; i < NCH; i++) {
        if (i + 1 < NCH) {
#pragma unroll
          for (int d = 0; d < 4; d++) xn[d] = xrow[(c0 + i + 1) * 16 + d];
        }
        const float sf = e8m0_to_float(s[i]);
        const uint32_t wd[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int d = 0; d < 4; d++) {
          const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 0);
          const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 1);
          const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 2);
          const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 3);
          const bf16x8_t bw = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv[d]), bw, acc[d], 0, 0, 0);
        }
        if (i + 1 < NCH) {
#pragma unroll
          for (int d = 0; d < 4; d++) xv[d] = xn[d];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int c0 = 0; c0 < NIT; c0 += 2 * NCH) {
      compute_chunk(c0, wa, sa);
      if (c0 + 2 * NCH < NIT) load_chunk(c0 + 2 * NCH, wa, sa);
      if (c0 + NCH >= NIT) break;
      compute_chunk(c0 + NCH, wb, sb);
      if (c0 + 3 * NCH < NIT) load_chunk(c0 + 3 * NCH, wb, sb);
    }
    const f32x4_v tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);

    // ---- lane l holds tokens 4 * (l / 16) + i of weight row l % 16
    if (row_ok) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int m = 4 * kq + i;
        if (m < mc && m < MT) {
          const int r = rows_lds[m];
          if (r >= 0) out[(size_t)r * N + row] = tot[i] + bias_v;
        }
      }
    }
  }
}

template <int MT, int WAVES, int NCH>
hipError_t launch_gemv_shape(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N, int K,
                             const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                             const int32_t* sorted_rows, float* out, hipStream_t stream) {
  const int nit = (K / 32 + 3) / 4;
  const size_t lds = (size_t)(MT + 1) * ((nit + NCH - 1) / NCH * NCH * 16 + 1) * 16;
  static bool attr_set = false;  // raise the dynamic LDS limit once per instantiation
  if (!attr_set && lds > 65536) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&expert_gemv_kernel<MT, WAVES, NCH>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const int R = T * k;
  const int groups = R < E ? R : E;
  const int rows_per_block = WAVES * 16;
  const dim3 grid((N + rows_per_block - 1) / rows_per_block, groups);
  hipLaunchKernelGGL((expert_gemv_kernel<MT, WAVES, NCH>), grid, dim3(WAVES * 64), lds, stream, blocks, scales, bias, E,
                     N, K, x, x_per_slot, T, k, offsets, sorted_rows, out);
  return hipGetLastError();
}

}  // namespace

namespace {
// K groups (128 elements) per fully unrolled chunk
int gemv_chunk(int K) { return (K / 32 + 3) / 4 <= 4 ? 4 : 8; }
}  // namespace

size_t gemv_lds_bytes(int T, int K) {
  const int mt = T <= 1 ? 1 : (T <= 4 ? 4 : 16);
  const int nch = gemv_chunk(K);
  const int nit = (K / 32 + 3) / 4;
  return (size_t)(mt + 1) * ((nit + nch - 1) / nch * nch * 16 + 1) * 16;
}

hipError_t launch_expert_gemv(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N, int K,
                              const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                              const int32_t* sorted_rows, float* out, hipStream_t stream) {
#define MXFP4_GEMV_LAUNCH(MT, W, NCH)                                                                      \
  return launch_gemv_shape<MT, W, NCH>(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, offsets, sorted_rows, \
                                       out, stream)
  const bool small_k = gemv_chunk(K) == 4;
  if (T <= 1) {
    if (small_k) MXFP4_GEMV_LAUNCH(1, 4, 4);
    MXFP4_GEMV_LAUNCH(1, 4, 8);
  }
  if (T <= 4) {
    if (small_k) MXFP4_GEMV_LAUNCH(4, 4, 4);
    MXFP4_GEMV_LAUNCH(4, 4, 8);
  }
  if (small_k) MXFP4_GEMV_LAUNCH(16, 8, 4);
  MXFP4_GEMV_LAUNCH(16, 8, 8);
#undef MXFP4_GEMV_LAUNCH
}

}  // namespace mxfp4

// Router logits of the MoE block, for gfx950.
//
//   logits[t, e] = bf16(sum_j x[t, j] * w[e, j] + bias[e])
//
// (gpt-oss-20b files page, src/experts.linnet block MixtureOfExperts: the
// router is a Linear from the hidden width H to the experts, weight [E, H] and
// bias [E] in bf16, whose output feeds the top-k ranking and the softmax.)
//
// MI355X design.  bf16 x bf16 products are exact in fp32, so the contraction
// runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation: A = 16 token rows,
// B = 16 (or 32, two MFMAs) expert rows, both read as stored (row-major
// [rows, H]): lane l supplies row l % 16 and elements 8 (l / 16) .. + 7 of
// each 32-wide K step, one 16-byte load per operand.  A workgroup owns a tile
// of 16 tokens x EXP experts and splits K over its 16 waves; each wave issues
// every load of a chunk of kChunk K steps before its first MFMA, so a single
// token (the decode) costs about one memory round trip.  The 16 partial tiles
// are added in LDS in wave order (deterministic), the bias is added in fp32
// and the sum rounded to bf16 (round to nearest even).  Up to 16 tokens take a
// row-per-workgroup form instead (router_rows_kernel below).

#include "kernels.h"
#include "common.h"

namespace mxfp4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

constexpr int kRouterWaves = 16;
constexpr int kRouterTok = 16;
constexpr int kChunk = 6;  // K steps of 32 whose loads are in flight together

template <int EXP>
__global__ __launch_bounds__(kRouterWaves * 64) void router_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ w,
                                                                   const uint16_t* __restrict__ bias, int T, int H,
                                                                   int E, uint16_t* __restrict__ logits) {
  constexpr int NB = EXP / 16;  // MFMAs per K step
  __shared__ float red[kRouterWaves][kRouterTok * EXP];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRouterTok;
  const int e0 = blockIdx.y * EXP;
  const int r = lane & 15;  // operand row within 16
  const int kq = lane >> 4;  // which 8 elements of a K step
  // rows past T or E re-read the last row; their results are not stored
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + r, T - 1) * H);
  const uint4* wr[NB];
#pragma unroll
  for (int b = 0; b < NB; b++) wr[b] = reinterpret_cast<const uint4*>(w + (size_t)min(e0 + 16 * b + r, E - 1) * H);
  const int steps = H >> 5;
  f32x4_v acc[NB];
#pragma unroll
  for (int b = 0; b < NB; b++) acc[b] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  // wave w takes the chunks of kChunk consecutive steps starting at
  // kChunk * (w + 16 i)
  for (int s0 = wave * kChunk; s0 < steps; s0 += kRouterWaves * kChunk) {
    uint4 xa[kChunk], wb[kChunk][NB];
#pragma unroll
    for (int c = 0; c < kChunk; c++) {
      const int piece = min(s0 + c, steps - 1) * 4 + kq;  // steps past H re-read the last one, unused
      xa[c] = xr[piece];
#pragma unroll
      for (int b = 0; b < NB; b++) wb[c][b] = wr[b][piece];
    }
#pragma unroll
    for (int c = 0; c < kChunk; c++) {
      if (s0 + c < steps) {
#pragma unroll
        for (int b = 0; b < NB; b++)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[c]),
                                                           __builtin_bit_cast(bf16x8_t, wb[c][b]), acc[b], 0, 0, 0);
      }
    }
  }
  // lane l holds tokens 4 kq + i of experts 16 b + r
#pragma unroll
  for (int b = 0; b < NB; b++)
#pragma unroll
    for (int i = 0; i < 4; i++) red[wave][(4 * kq + i) * EXP + 16 * b + r] = acc[b][i];
  __syncthreads();
  for (int v = threadIdx.x; v < kRouterTok * EXP; v += kRouterWaves * 64) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kRouterWaves; q++) s += red[q][v];
    const int t = t0 + v / EXP, e = e0 + v % EXP;
    if (t < T && e < E) {
      const float bv = bias ? bf16_bits_to_f32(bias[e]) : 0.f;
      logits[(size_t)t * E + e] = (uint16_t)f32_to_bf16_bits(s + bv);
    }
  }
}

// A few tokens (T <= kRowsMaxT): one workgroup per expert row, so that the
// router weights are read by E CUs at once rather than by two (for one token
// the MFMA tiles above would leave 15 of their 16 token rows empty).  At the
// gpt-oss widths (H = 2880, E = 32): 2.0 us for one token against 4.9 us with
// the MFMA tiles, 3.4 against 5.8 for 8 tokens, 4.7 against 6.8 for 16.  Thread i
// takes the 16-byte pieces i, i + 256, ... of the expert's row and of each
// token row, multiplies them with v_dot2_f32_bf16 (bf16 x bf16 products, fp32
// sums), and the sums meet in a fixed order: the lanes of a wave by shuffles,
// then the four waves in LDS; the bias is added in fp32 and the sum rounded to
// bf16.
constexpr int kRowsMaxT = 16;
constexpr int kRowsThreads = 256;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int TT>
__global__ __launch_bounds__(kRowsThreads) void router_rows_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ w,
                                                                   const uint16_t* __restrict__ bias, int H, int E,
                                                                   uint16_t* __restrict__ logits) {
  __shared__ float red[kRowsThreads / 64][TT];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H8 = H >> 3;
  const uint4* wr = reinterpret_cast<const uint4*>(w + (size_t)e * H);
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; t++) acc[t] = 0.f;
  for (int i = threadIdx.x; i < H8; i += kRowsThreads) {
    const uint4 wv = wr[i];
    uint4 xv[TT];
#pragma unroll
    for (int t = 0; t < TT; t++) xv[t] = reinterpret_cast<const uint4*>(x + (size_t)t * H)[i];
    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int t = 0; t < TT; t++) {
      const uint32_t xd[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
      for (int d = 0; d < 4; d++)
        acc[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wd[d]),
                                                 __builtin_bit_cast(bf16x2_t, xd[d]), acc[t], false);
    }
  }
#pragma unroll
  for (int t = 0; t < TT; t++) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc[t] += __shfl_xor(acc[t], o, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < TT; t++) red[wave][t] = acc[t];
  }
  __syncthreads();
  if (threadIdx.x < TT) {
    const int t = threadIdx.x;
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kRowsThreads / 64; q++) s += red[q][t];
    const float bv = bias ? bf16_bits_to_f32(bias[e]) : 0.f;
    logits[(size_t)t * E + e] = (uint16_t)f32_to_bf16_bits(s + bv);
  }
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* w, const uint16_t* bias, int T, int H, int E,
                         uint16_t* logits, hipStream_t stream) {
  // Up to 16 tokens: a workgroup per expert row; up to 64: 16-expert tiles, so
  // that more CUs share the router weights; more: 32-expert tiles, so that each
  // token tile is read half as often.
  const unsigned tx = (unsigned)((T + kRouterTok - 1) / kRouterTok);
  if (T <= kRowsMaxT) {
#define MXFP4_ROUTER_ROWS(TT)                                                                                 \
  case TT:                                                                                                    \
    hipLaunchKernelGGL(router_rows_kernel<TT>, dim3(E), dim3(kRowsThreads), 0, stream, x, w, bias, H, E, logits); \
    break;
    switch (T) {
      MXFP4_ROUTER_ROWS(1)
      MXFP4_ROUTER_ROWS(2)
      MXFP4_ROUTER_ROWS(3)
      MXFP4_ROUTER_ROWS(4)
      MXFP4_ROUTER_ROWS(5)
      MXFP4_ROUTER_ROWS(6)
      MXFP4_ROUTER_ROWS(7)
      MXFP4_ROUTER_ROWS(8)
      MXFP4_ROUTER_ROWS(9)
      MXFP4_ROUTER_ROWS(10)
      MXFP4_ROUTER_ROWS(11)
      MXFP4_ROUTER_ROWS(12)
      MXFP4_ROUTER_ROWS(13)
      MXFP4_ROUTER_ROWS(14)
      MXFP4_ROUTER_ROWS(15)
      default:
        hipLaunchKernelGGL(router_rows_kernel<kRowsMaxT>, dim3(E), dim3(kRowsThreads), 0, stream, x, w, bias, H, E,
                           logits);
        break;
    }
#undef MXFP4_ROUTER_ROWS
  } else if (T <= 64) {
    hipLaunchKernelGGL(router_kernel<16>, dim3(tx, (unsigned)((E + 15) / 16)), dim3(kRouterWaves * 64), 0, stream, x,
                       w, bias, T, H, E, logits);
  } else {
    hipLaunchKernelGGL(router_kernel<32>, dim3(tx, (unsigned)((E + 31) / 32)), dim3(kRouterWaves * 64), 0, stream, x,
                       w, bias, T, H, E, logits);
  }
  return hipGetLastError();
}

}  // namespace mxfp4

// Prefill expert projection: a grouped GEMM on gfx950 scaled-FP4 MFMA.
//
// For every expert e with M_e routed rows (grouped by mxfp4_moe_route_group):
//   C_e[M_e, N] = X_e[M_e, K] * W_e^T + bias_e,  scattered to out[r, :]
// (gpt-oss-20b files page, README "Loading": one grouped product over the
// tokens sorted by expert, each expert multiplying only the tokens that chose
// it; README "MXFP4" for the weight format).
//
// MI355X design:
//  * The weights are fed to v_mfma_scale_f32_32x32x64_f8f6f4 exactly as the
//    checkpoint stores them: a lane of the B operand holds one 16-byte MXFP4
//    block (32 E2M1 codes, low nibble first) of one weight row, and its E8M0
//    byte is that lane's B scale.  No dequantization anywhere.
//  * bf16 activations have no MX form, so a pre-pass (quantize_act_kernel)
//    splits every 32-element block of every input row once into two MX-FP6
//    (E2M3) terms, hi + lo, each with its own E8M0 scale; the GEMM issues one
//    MFMA per term.  hi is the block rounded to E2M3 under the smallest power
//    of two scale that keeps its largest magnitude <= 7.5; lo is the exact
//    fp32 residual rounded the same way.  E2M3 x E2M1 runs at the FP4 MFMA
//    rate on gfx950.
//  * Workgroup = 4 waves, output tile BM x BN, K staged 128 at a time (four MX
//    blocks) through double-buffered LDS; each wave owns (BM/WM) x (BN/WN) of
//    the tile as 32x32 MFMA sub-tiles with fp32 accumulators.
//  * The tile schedule is derived on the device from expert_offsets: blockIdx.y
//    enumerates (expert, row-tile) pairs in expert order; workgroups past the
//    last pair exit at once.  No host synchronisation, any skew of rows per
//    expert.
//  * Routed rows are gathered through sorted_rows when the A tile is loaded and
//    the results are scattered through it in the epilogue (bias added there).

#include "kernels.h"
#include "common.h"

namespace mxfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBlocksPerKTile = 4;       // MX blocks per K stage (K = 128)
constexpr int kQBytesPerBlock = 48;      // hi (24 B) + lo (24 B) packed E2M3 codes
constexpr int kFmtFp6E2M3 = 2;           // MFMA operand format codes
constexpr int kFmtFp4E2M1 = 4;

__host__ __device__ inline int round_up4(int v) { return (v + 3) & ~3; }

// ---------------------------------------------------------------------------
// activation quantization: bf16 block of 32 -> two MX-FP6 (E2M3) terms
// ---------------------------------------------------------------------------

// smallest e with amax * 2^-e <= 7.5 (the E2M3 maximum); amax a normal float
__device__ __forceinline__ int mx_exponent(float amax) {
  const int ex = (int)((__float_as_uint(amax) >> 23) & 255u) - 127;  // floor(log2(amax))
  int e = ex - 2;
  if (ldexpf(amax, -e) > 7.5f) e += 1;
  return e;
}

// magnitude code of u in [0, 7.5], round to nearest even: the E2M3 grid has
// step 1/8 on [0, 2), 1/4 on [2, 4), 1/2 on [4, 7.5] and codes that increase
// with the value.
__device__ __forceinline__ int e2m3_magnitude_code(float u) {
  int c;
  if (u < 2.f)
    c = (int)rintf(u * 8.f);
  else if (u < 4.f)
    c = 8 + (int)rintf(u * 4.f);
  else
    c = 16 + (int)rintf(u * 2.f);
  return c > 31 ? 31 : c;
}

__device__ __forceinline__ float e2m3_magnitude(int c) {
  const int ef = c >> 3, m = c & 7;
  return ef == 0 ? (float)m * 0.125f : ldexpf(1.f + (float)m * 0.125f, ef - 1);
}

// quantize 32 values v (in place: v becomes the residual) into packed codes and
// the E8M0 byte; blocks whose largest magnitude is below 2^-125 become zero.
__device__ __forceinline__ void quantize_term(float (&v)[32], uint32_t (&packed)[6], uint32_t& scale_byte) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(v[j]));
  int codes[32];
  if (amax < 0x1p-125f) {
#pragma unroll
    for (int j = 0; j < 32; j++) codes[j] = 0;
    scale_byte = 127u;
  } else {
    const int e = mx_exponent(amax);
    scale_byte = (uint32_t)(e + 127);
#pragma unroll
    for (int j = 0; j < 32; j++) {
      const float u = ldexpf(fabsf(v[j]), -e);
      const int c = e2m3_magnitude_code(u);
      const float q = ldexpf(e2m3_magnitude(c), e);
      const bool neg = v[j] < 0.f;
      codes[j] = c | (neg ? 32 : 0);
      v[j] = v[j] - (neg ? -q : q);  // exact residual
    }
  }
  uint32_t g[8];
#pragma unroll
  for (int i = 0; i < 8; i++)
    g[i] = (uint32_t)codes[4 * i] | ((uint32_t)codes[4 * i + 1] << 6) | ((uint32_t)codes[4 * i + 2] << 12) |
           ((uint32_t)codes[4 * i + 3] << 18);
  packed[0] = g[0] | (g[1] << 24);
  packed[1] = (g[1] >> 8) | (g[2] << 16);
  packed[2] = (g[2] >> 16) | (g[3] << 8);
  packed[3] = g[4] | (g[5] << 24);
  packed[4] = (g[5] >> 8) | (g[6] << 16);
  packed[5] = (g[6] >> 16) | (g[7] << 8);
}

// One thread per (row, block).  q: [Rq][KBp][48], s: [Rq][KBp][2].
__global__ __launch_bounds__(kThreads) void quantize_act_kernel(const uint16_t* __restrict__ x, int Rq, int K,
                                                                int KBp, uint8_t* __restrict__ q,
                                                                uint8_t* __restrict__ s) {
  const int KB = K >> 5;
  const size_t total = (size_t)Rq * KBp;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const size_t row = idx / KBp;
  const int kb = (int)(idx - row * KBp);
  uint32_t hi[6] = {0, 0, 0, 0, 0, 0}, lo[6] = {0, 0, 0, 0, 0, 0};
  uint32_t sh = 127u, sl = 127u;
  if (kb < KB) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * K + (size_t)kb * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint4 p = src[i];
      const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        v[8 * i + 2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
        v[8 * i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      }
    }
    quantize_term(v, hi, sh);
    quantize_term(v, lo, sl);
  }
  uint4* dst = reinterpret_cast<uint4*>(q + idx * kQBytesPerBlock);
  dst[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  dst[1] = make_uint4(hi[4], hi[5], lo[0], lo[1]);
  dst[2] = make_uint4(lo[2], lo[3], lo[4], lo[5]);
  reinterpret_cast<uint16_t*>(s)[idx] = (uint16_t)(sh | (sl << 8));
}

// ---------------------------------------------------------------------------
// grouped GEMM
// ---------------------------------------------------------------------------

template <int BM, int BN, int WM, int WN>
struct GemmShape {
  static constexpr int MS = BM / WM / 32;  // 32-row sub-tiles per wave
  static constexpr int NS = BN / WN / 32;  // 32-col sub-tiles per wave
  static constexpr int A_BYTES = BM * kBlocksPerKTile * kQBytesPerBlock;
  static constexpr int AS_BYTES = BM * kBlocksPerKTile * 2;
  static constexpr int B_BYTES = BN * kBlocksPerKTile * 16;
  static constexpr int BS_BYTES = BN * kBlocksPerKTile;
  static constexpr int STAGE = A_BYTES + AS_BYTES + B_BYTES + BS_BYTES;
  static constexpr int A_CHUNKS = A_BYTES / 16;
  static constexpr int A_PER_T = (A_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int B_CHUNKS = B_BYTES / 16;
  static constexpr int B_PER_T = (B_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int BS_PER_T = (BS_BYTES + kThreads - 1) / kThreads;
  static_assert(WM * WN == kThreads / 64, "4 waves");
  static_assert(MS >= 1 && NS >= 1, "tile too small");
  static_assert(BM <= kThreads, "one thread per tile row for the scale loads");
};

// Find the (expert, row tile) for tile index mt.
__device__ __forceinline__ bool find_tile(const int32_t* offsets, int E, int R, int BM, int mt, int& e_out,
                                          int& m_begin, int& m_count) {
  int prev = min(max(offsets[0], 0), R);
  for (int e = 0; e < E; e++) {
    const int nxt = min(max(offsets[e + 1], prev), R);
    const int tiles = (nxt - prev + BM - 1) / BM;
    if (mt < tiles) {
      e_out = e;
      m_begin = prev + mt * BM;
      m_count = min(BM, nxt - m_begin);
      return true;
    }
    mt -= tiles;
    prev = nxt;
  }
  return false;
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void expert_gemm_kernel(
    const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ wscales, const uint16_t* __restrict__ bias,
    int E, int N, int K, const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, int KBp,
    int x_per_slot, int T, int k, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows,
    float* __restrict__ out) {
  using S = GemmShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::STAGE];
  __shared__ int rows_lds[BM];  // routed row of each tile row, -1 if none
  __shared__ int src_lds[BM];   // quantized-input row of each tile row, -1 if none

  const int R = T * k;
  int e, m_begin, m_count;
  if (!find_tile(offsets, E, R, BM, blockIdx.y, e, m_begin, m_count)) return;
  const int KB = K >> 5;
  const int n0 = blockIdx.x * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  for (int i = tid; i < BM; i += kThreads) {
    int r = -1;
    if (i < m_count) {
      r = sorted_rows[m_begin + i];
      if (r < 0 || r >= R) r = -1;
    }
    rows_lds[i] = r;
    src_lds[i] = r < 0 ? -1 : (x_per_slot ? r : r / k);
  }
  __syncthreads();

  // ---- global -> register -> LDS staging of one K tile
  uint4 ra[S::A_PER_T];
  uint2 ras = make_uint2(0u, 0u);
  uint4 rb[S::B_PER_T];
  uint32_t rbs[S::BS_PER_T];

  auto load_tile = [&](int kt) {
    const int kb0 = kt * kBlocksPerKTile;
#pragma unroll
    for (int i = 0; i < S::A_PER_T; i++) {
      const int c = tid + i * kThreads;
      ra[i] = make_uint4(0u, 0u, 0u, 0u);
      if (c < S::A_CHUNKS) {
        const int row = c / (kBlocksPerKTile * 3);
        const int part = c - row * (kBlocksPerKTile * 3);
        const int src = src_lds[row];
        if (src >= 0)
          ra[i] = *reinterpret_cast<const uint4*>(aq + ((size_t)src * KBp + kb0) * kQBytesPerBlock + part * 16);
      }
    }
    if (tid < BM) {
      const int src = src_lds[tid];
      ras = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
      if (src >= 0) ras = *reinterpret_cast<const uint2*>(as + ((size_t)src * KBp + kb0) * 2);
    }
#pragma unroll
    for (int i = 0; i < S::B_PER_T; i++) {
      const int c = tid + i * kThreads;
      rb[i] = make_uint4(0u, 0u, 0u, 0u);
      if (c < S::B_CHUNKS) {
        const int n = c >> 2;
        const int kb = kb0 + (c & 3);
        if (n0 + n < N && kb < KB)
          rb[i] = load_nt(reinterpret_cast<const uint4*>(blocks + (((size_t)e * N + n0 + n) * KB + kb) * 16));
      }
    }
#pragma unroll
    for (int i = 0; i < S::BS_PER_T; i++) {
      const int c = tid + i * kThreads;
      rbs[i] = 127u;
      if (c < S::BS_BYTES) {
        const int n = c >> 2;
        const int kb = kb0 + (c & 3);
        if (n0 + n < N && kb < KB) rbs[i] = wscales[((size_t)e * N + n0 + n) * KB + kb];
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint8_t* st = smem + buf * S::STAGE;
#pragma unroll
    for (int i = 0; i < S::A_PER_T; i++) {
      const int c = tid + i * kThreads;
      if (c < S::A_CHUNKS) reinterpret_cast<uint4*>(st)[c] = ra[i];
    }
    if (tid < BM) reinterpret_cast<uint2*>(st + S::A_BYTES)[tid] = ras;
#pragma unroll
    for (int i = 0; i < S::B_PER_T; i++) {
      const int c = tid + i * kThreads;
      if (c < S::B_CHUNKS) reinterpret_cast<uint4*>(st + S::A_BYTES + S::AS_BYTES)[c] = rb[i];
    }
#pragma unroll
    for (int i = 0; i < S::BS_PER_T; i++) {
      const int c = tid + i * kThreads;
      if (c < S::BS_BYTES) st[S::A_BYTES + S::AS_BYTES + S::B_BYTES + c] = (uint8_t)rbs[i];
    }
  };

  v16f acc[S::MS][S::NS];
#pragma unroll
  for (int i = 0; i < S::MS; i++)
#pragma unroll
    for (int j = 0; j < S::NS; j++)
#pragma unroll
      for (int q = 0; q < 16; q++) acc[i][j][q] = 0.f;

  const int KT = KBp / kBlocksPerKTile;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int l32 = lane & 31;
  const int lhalf = lane >> 5;
  for (int kt = 0; kt < KT; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);
    const uint8_t* st = smem + cur * S::STAGE;
    const uint8_t* sA = st;
    const uint16_t* sAS = reinterpret_cast<const uint16_t*>(st + S::A_BYTES);
    const uint8_t* sB = st + S::A_BYTES + S::AS_BYTES;
    const uint8_t* sBS = sB + S::B_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const int blk = ks * 2 + lhalf;
      v8i bfrag[S::NS];
      int bscale[S::NS];
#pragma unroll
      for (int ns = 0; ns < S::NS; ns++) {
        const int n = wn * (BN / WN) + ns * 32 + l32;
        const uint4 v = *reinterpret_cast<const uint4*>(sB + (n * kBlocksPerKTile + blk) * 16);
        bfrag[ns] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        bscale[ns] = sBS[n * kBlocksPerKTile + blk];
      }
#pragma unroll
      for (int ms = 0; ms < S::MS; ms++) {
        const int row = wm * (BM / WM) + ms * 32 + l32;
        const uint8_t* p = sA + (row * kBlocksPerKTile + blk) * kQBytesPerBlock;
        const uint4 q0 = *reinterpret_cast<const uint4*>(p);
        const uint2 q1 = *reinterpret_cast<const uint2*>(p + 16);
        const uint2 q2 = *reinterpret_cast<const uint2*>(p + 24);
        const uint4 q3 = *reinterpret_cast<const uint4*>(p + 32);
        const v8i ahi = v8i{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, 0, 0};
        const v8i alo = v8i{(int)q2.x, (int)q2.y, (int)q3.x, (int)q3.y, (int)q3.z, (int)q3.w, 0, 0};
        const uint32_t sc = sAS[row * kBlocksPerKTile + blk];
        const int sh = (int)(sc & 0xffu);
        const int sl = (int)(sc >> 8);
#pragma unroll
        for (int ns = 0; ns < S::NS; ns++) {
          acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ahi, bfrag[ns], acc[ms][ns], kFmtFp6E2M3,
                                                                        kFmtFp4E2M1, 0, sh, 0, bscale[ns]);
          acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(alo, bfrag[ns], acc[ms][ns], kFmtFp6E2M3,
                                                                        kFmtFp4E2M1, 0, sl, 0, bscale[ns]);
        }
      }
    }
    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: bias and scatter to the routed rows
#pragma unroll
  for (int ns = 0; ns < S::NS; ns++) {
    const int n = n0 + wn * (BN / WN) + ns * 32 + l32;
    if (n >= N) continue;
    const float b = bias ? bf16_bits_to_f32(bias[(size_t)e * N + n]) : 0.f;
#pragma unroll
    for (int ms = 0; ms < S::MS; ms++) {
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int row = wm * (BM / WM) + ms * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
        const int r = rows_lds[row];
        if (r >= 0) out[(size_t)r * N + n] = acc[ms][ns][i] + b;
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_gemm_shape(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                             int K, const uint8_t* aq, const uint8_t* as, int KBp, int x_per_slot, int T, int k,
                             const int32_t* offsets, const int32_t* sorted_rows, float* out,
                             hipStream_t stream) {
  const int R = T * k;
  const int groups = R < E ? R : E;
  const dim3 grid((N + BN - 1) / BN, (R + BM - 1) / BM + groups);
  hipLaunchKernelGGL((expert_gemm_kernel<BM, BN, WM, WN>), grid, dim3(kThreads), 0, stream, blocks, scales, bias,
                     E, N, K, aq, as, KBp, x_per_slot, T, k, offsets, sorted_rows, out);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int T, int k, int K, int x_per_slot) {
  const size_t rq = x_per_slot ? (size_t)T * k : (size_t)T;
  const size_t kbp = (size_t)round_up4(K / 32);
  const size_t qbytes = (rq * kbp * kQBytesPerBlock + 255) & ~(size_t)255;
  return qbytes + rq * kbp * 2;
}

hipError_t launch_expert_gemm(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                              int K, const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                              const int32_t* sorted_rows, float* out, void* workspace, hipStream_t stream) {
  const int Rq = x_per_slot ? T * k : T;
  const int KBp = round_up4(K / 32);
  uint8_t* aq = static_cast<uint8_t*>(workspace);
  const size_t qbytes = ((size_t)Rq * KBp * kQBytesPerBlock + 255) & ~(size_t)255;
  uint8_t* as = aq + qbytes;
  const size_t nblk = (size_t)Rq * KBp;
  hipLaunchKernelGGL(quantize_act_kernel, dim3((unsigned)((nblk + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, x, Rq, K, KBp, aq, as);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int R = T * k;
  const int E_used = R < E ? R : E;
  // rows per used expert decide the tile height
  if (R <= 48 * E_used)
    return launch_gemm_shape<32, 128, 1, 4>(blocks, scales, bias, E, N, K, aq, as, KBp, x_per_slot, T, k, offsets,
                                            sorted_rows, out, stream);
  return launch_gemm_shape<128, 128, 2, 2>(blocks, scales, bias, E, N, K, aq, as, KBp, x_per_slot, T, k, offsets,
                                           sorted_rows, out, stream);
}

}  // namespace mxfp4

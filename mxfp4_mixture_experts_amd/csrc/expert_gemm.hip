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
//    (E2M3) terms, hi + lo, each with its own E8M0 scale, using the gfx950
//    converts v_cvt_scalef32_pk32_fp6_bf16 (round to nearest even of x/2^e)
//    and v_cvt_scalef32_pk32_f32_fp6: hi is the block under the smallest power
//    of two that keeps its largest magnitude <= 7.5, lo the residual x - hi
//    (exact, and exactly a bf16) quantized the same way.  The GEMM issues one
//    MFMA per term; E2M3 x E2M1 runs at the FP4 MFMA rate on gfx950.
//  * Workgroup = 4 waves side by side along N; the output tile is
//    (32 * MS) rows x (4 * 32 * NS) weight rows.  K advances by a group of
//    eight MX blocks (four MFMA k-steps; in k-step s the lanes of half h of
//    the wave use block 4h + s, so each lane reads four adjacent blocks = 64
//    contiguous bytes of a weight row, and a lane pair a whole cache line).
//  * Activation tiles go through double-buffered LDS (row pitch padded by 16
//    bytes so the 32 rows one MFMA operand reads hit distinct banks).  Weight
//    fragments go straight from global memory to registers -- each belongs to
//    exactly one wave -- double-buffered, so a group's weights are requested
//    one whole group ahead.  The MFMAs of a k-step run over 2 * MS * NS
//    independent accumulators.
//  * The tile schedule is derived on the device from expert_offsets: each
//    workgroup counts the tiles, and tile t runs on XCD t / ceil(tiles / 8)
//    (workgroups are dispatched round-robin over the 8 XCDs), ordered so that
//    the row tiles sharing a weight panel run back to back on one XCD and
//    read the panel from its L2.  Surplus workgroups exit at once.  No host
//    synchronisation; any skew of rows per expert.
//  * Routed rows are gathered through sorted_rows when the activation tile is
//    staged and the results are scattered through it in the epilogue (bias
//    added there).

#include "kernels.h"
#include "common.h"

namespace mxfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kGroupBlocks = 8;          // MX blocks per K group (K = 256)
constexpr int kKPadBlocks = 16;          // the quantized activations are padded to pairs of groups
constexpr int kQBytes = 48;              // hi (24 B) + lo (24 B) packed E2M3 codes per block
constexpr int kFmtFp6E2M3 = 2;           // MFMA operand format codes
constexpr int kFmtFp4E2M1 = 4;
constexpr int kXcds = 8;

__host__ __device__ inline int round_up(int v, int m) { return (v + m - 1) / m * m; }

// ---------------------------------------------------------------------------
// activation quantization: bf16 block of 32 -> two MX-FP6 (E2M3) terms
// ---------------------------------------------------------------------------

// E8M0 exponent e for a block whose largest magnitude has bf16 bits `amax`:
// the smallest e with amax * 2^-e <= 7.5.  Blocks below 2^-120 count as zero
// (returns false).
__device__ __forceinline__ bool block_exponent(uint32_t amax, int& e) {
  const int ex = (int)(amax >> 7) - 127;          // amax is a positive bf16: exponent field
  if (ex < -120) return false;
  e = ex - 2 + (((amax & 0x7f) > 112) ? 1 : 0);   // 4 * (1 + m/128) > 7.5  <=>  m > 112
  return true;
}

__device__ __forceinline__ uint32_t max_abs_bf16(const uint32_t (&w)[16]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) m = max(m, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  return m;
}

// One thread per (row, block).  q: [Rq][KBp][48], s: [Rq][KBp][2] (hi scale, lo scale).
__global__ __launch_bounds__(kThreads) void quantize_act_kernel(const uint16_t* __restrict__ x, int Rq, int K,
                                                                int KBp, uint8_t* __restrict__ q,
                                                                uint8_t* __restrict__ s) {
  const int KB = K >> 5;
  const size_t total = (size_t)Rq * KBp;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const size_t row = idx / KBp;
  const int kb = (int)(idx - row * KBp);
  v6i hi = {0, 0, 0, 0, 0, 0}, lo = {0, 0, 0, 0, 0, 0};
  uint32_t sh = 127u, sl = 127u;
  if (kb < KB) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * K + (size_t)kb * 32);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint4 p = src[i];
      w[4 * i] = p.x; w[4 * i + 1] = p.y; w[4 * i + 2] = p.z; w[4 * i + 3] = p.w;
    }
    int e;
    if (block_exponent(max_abs_bf16(w), e)) {
      sh = (uint32_t)(e + 127);
      const float scale = __uint_as_float(sh << 23);
      hi = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(__builtin_bit_cast(bf16x32_t, w), scale);
      const v32f hv = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(hi, scale);
      uint32_t r[16];
#pragma unroll
      for (int i = 0; i < 16; i++) {
        // residuals are exact in fp32 and fit bf16 exactly: keep the top halves
        const float a = bf16_bits_to_f32(w[i] & 0xffffu) - hv[2 * i];
        const float b = bf16_bits_to_f32(w[i] >> 16) - hv[2 * i + 1];
        r[i] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
      }
      int e2;
      if (block_exponent(max_abs_bf16(r), e2)) {
        sl = (uint32_t)(e2 + 127);
        lo = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(__builtin_bit_cast(bf16x32_t, r),
                                                         __uint_as_float(sl << 23));
      }
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(q + idx * kQBytes);
  dst[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  dst[1] = make_uint4(hi[4], hi[5], lo[0], lo[1]);
  dst[2] = make_uint4(lo[2], lo[3], lo[4], lo[5]);
  reinterpret_cast<uint16_t*>(s)[idx] = (uint16_t)(sh | (sl << 8));
}

// ---------------------------------------------------------------------------
// grouped GEMM
// ---------------------------------------------------------------------------

constexpr int kMS = 2;                        // 32-row sub-tiles per wave
constexpr int kNS = 2;                        // 32-column sub-tiles per wave
constexpr int kBM = 32 * kMS;                 // routed rows per tile (= lanes of a wave)
constexpr int kBN = kWaves * 32 * kNS;        // weight rows per tile
constexpr int kParts = kQBytes / 16;          // 16-byte parts of a block's codes
// LDS stage: codes as [block][part][row] x 16 bytes (a wave's 64 lanes store one
// (block, part) column for the 64 rows; MFMA operand reads by 32 consecutive
// rows are conflict-free), then scales as [row] x 16 bytes (8 blocks x (hi, lo)).
constexpr int kCodeBytes = kGroupBlocks * kParts * kBM * 16;
constexpr int kStage = kCodeBytes + kBM * 16;
static_assert(kBM == 64, "one lane per tile row in the activation staging");

struct TileCoord {
  int e, m_begin, m_count, n0;
};

// Tile t of the grouped problem: experts in order; within an expert the weight
// panel (n-tile) varies slowest so that its row tiles are consecutive.
__device__ __forceinline__ bool locate_tile(const int32_t* offsets, int E, int R, int NT, TileCoord& c) {
  int total = 0;
  int prev = min(max(offsets[0], 0), R);
  for (int e = 0; e < E; e++) {
    const int nxt = min(max(offsets[e + 1], prev), R);
    total += (nxt - prev + kBM - 1) / kBM * NT;
    prev = nxt;
  }
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int L = blockIdx.x;
  const int j = L / kXcds;
  if (j >= per_xcd) return false;
  int t = (L % kXcds) * per_xcd + j;
  if (t >= total) return false;
  prev = min(max(offsets[0], 0), R);
  for (int e = 0; e < E; e++) {
    const int nxt = min(max(offsets[e + 1], prev), R);
    const int mt = (nxt - prev + kBM - 1) / kBM;
    if (t < mt * NT) {
      const int nt = t / mt;
      const int mi = t - nt * mt;
      c.e = e;
      c.m_begin = prev + mi * kBM;
      c.m_count = min(kBM, nxt - c.m_begin);
      c.n0 = nt * kBN;
      return true;
    }
    t -= mt * NT;
    prev = nxt;
  }
  return false;
}

constexpr int kAChunks = kGroupBlocks * kParts * kBM / kThreads;  // staged chunks per thread per group


// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load (its fence covers global memory), which would drain
// the weight prefetch at every K group.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// SCALE_PAIRS: the weight scale rows are 2-byte aligned (K/32 even), so each
// lane reads its four scale bytes as two 16-bit loads.
template <bool SCALE_PAIRS>
__global__ __launch_bounds__(kThreads) void expert_gemm_kernel(
    const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ wscales, const uint16_t* __restrict__ bias,
    int E, int N, int K, const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as, int KBp,
    int x_per_slot, int T, int k, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows,
    float* __restrict__ out) {
  // the two LDS stages of the activation double buffer
  __shared__ __attribute__((aligned(16))) uint8_t stage0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[kStage];
  __shared__ int rows_lds[kBM];  // routed row of each tile row, -1 if none

  const int R = T * k;
  const int NT = (N + kBN - 1) / kBN;
  TileCoord tc;
  if (!locate_tile(offsets, E, R, NT, tc)) return;
  const int e = tc.e;
  const int KB = K >> 5;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // lane l of every wave stages tile row l: its quantized-input row (clamped to
  // a real row when the tile row is empty; such rows are never stored)
  int r_lane = -1;
  if (lane < tc.m_count) {
    r_lane = sorted_rows[tc.m_begin + lane];
    if (r_lane < 0 || r_lane >= R) r_lane = -1;
  }
  if (wave == 0) rows_lds[lane] = r_lane;  // read only in the epilogue, after several barriers
  const int src_lane = r_lane < 0 ? 0 : (x_per_slot ? r_lane : r_lane / k);
  const uint8_t* a_row = aq + (size_t)src_lane * KBp * kQBytes;
  const uint8_t* as_row = as + (size_t)src_lane * KBp * 2;

  // ---- activations: global -> registers -> LDS.  Thread t stages 16-byte
  // chunks c = t + 256 i: tile row c % 64 (its own lane's row), (block, part)
  // column c / 64 = wave + 4 i, stored at chunk c of the [block][part][row]
  // layout; plus its row's 16 bytes of scales (all four waves store the same
  // bytes: no branch).  Staged values are plain vector variables (A_* macros)
  // so that nothing of the pipeline lands in scratch memory.
  static_assert(kAChunks == 6, "the A_* macros stage six chunks per thread");
  auto a_src = [&](int g, int i) {
    const int c = wave + kWaves * i;
    const int blk = c / kParts;
    const int part = c - blk * kParts;
    return reinterpret_cast<const u32x4_t*>(a_row + (size_t)(g * kGroupBlocks + blk) * kQBytes + part * 16);
  };
  auto a_dst = [&](uint8_t* st, int i) {
    return reinterpret_cast<u32x4_t*>(st + ((wave + kWaves * i) * kBM + lane) * 16);
  };
#define A_DECL(p) u32x4_t p##0, p##1, p##2, p##3, p##4, p##5, p##s
#define A_LOAD(p, g)                                                                          \
  do {                                                                                        \
    const int g_ = (g);                                                                       \
    p##0 = *a_src(g_, 0); p##1 = *a_src(g_, 1); p##2 = *a_src(g_, 2);                          \
    p##3 = *a_src(g_, 3); p##4 = *a_src(g_, 4); p##5 = *a_src(g_, 5);                          \
    p##s = *reinterpret_cast<const u32x4_t*>(as_row + (size_t)g_ * kGroupBlocks * 2);         \
  } while (0)
#define A_STORE(p, st)                                                                        \
  do {                                                                                        \
    *a_dst(st, 0) = p##0; *a_dst(st, 1) = p##1; *a_dst(st, 2) = p##2;                          \
    *a_dst(st, 3) = p##3; *a_dst(st, 4) = p##4; *a_dst(st, 5) = p##5;                          \
    *reinterpret_cast<u32x4_t*>(st + kCodeBytes + lane * 16) = p##s;                          \
  } while (0)

  // ---- weights: lane (half h, row l32 of sub-tile ns) reads the four adjacent
  // blocks kb0 + 4h .. kb0 + 4h + 3 of its row (64 contiguous bytes; k-step s
  // uses block kb0 + 4h + s).  Rows past N and blocks past K re-read real
  // (clamped) blocks; they meet zero activations or are not stored.
  static_assert(kNS == 2, "the B_* macros hold two sub-tiles");
  const int n_wave = tc.n0 + wave * 32 * kNS;
  const int n0c = min(n_wave + l32, N - 1);
  const int n1c = min(n_wave + 32 + l32, N - 1);
  const u32x4_t* wrow0 = reinterpret_cast<const u32x4_t*>(blocks) + ((size_t)e * N + n0c) * KB;
  const u32x4_t* wrow1 = reinterpret_cast<const u32x4_t*>(blocks) + ((size_t)e * N + n1c) * KB;
  const uint8_t* srow0 = wscales + ((size_t)e * N + n0c) * KB;
  const uint8_t* srow1 = wscales + ((size_t)e * N + n1c) * KB;
  // scale bytes of blocks kb, kb + 1 as one 16-bit load (rows are 2-byte aligned
  // when K/32 is even) or as two byte loads
  auto scale_pair = [&](const uint8_t* srow, int kb) -> uint32_t {
    if (SCALE_PAIRS) return *reinterpret_cast<const uint16_t*>(srow + min(kb, KB - 2));
    return (uint32_t)srow[min(kb, KB - 1)] | ((uint32_t)srow[min(kb + 1, KB - 1)] << 8);
  };
#define B_DECL(p) u32x4_t p##q00, p##q01, p##q02, p##q03, p##q10, p##q11, p##q12, p##q13; uint32_t p##s00, p##s01, p##s10, p##s11
#define B_LOAD(p, g)                                                                          \
  do {                                                                                        \
    const int kb_ = (g) * kGroupBlocks + 4 * half;                                            \
    p##q00 = wrow0[min(kb_, KB - 1)]; p##q01 = wrow0[min(kb_ + 1, KB - 1)];                   \
    p##q02 = wrow0[min(kb_ + 2, KB - 1)]; p##q03 = wrow0[min(kb_ + 3, KB - 1)];               \
    p##q10 = wrow1[min(kb_, KB - 1)]; p##q11 = wrow1[min(kb_ + 1, KB - 1)];                   \
    p##q12 = wrow1[min(kb_ + 2, KB - 1)]; p##q13 = wrow1[min(kb_ + 3, KB - 1)];               \
    p##s00 = scale_pair(srow0, kb_); p##s01 = scale_pair(srow0, kb_ + 2);                     \
    p##s10 = scale_pair(srow1, kb_); p##s11 = scale_pair(srow1, kb_ + 2);                     \
  } while (0)

  v16f acc[kMS][kNS];
#pragma unroll
  for (int i = 0; i < kMS; i++)
#pragma unroll
    for (int j = 0; j < kNS; j++)
#pragma unroll
      for (int q = 0; q < 16; q++) acc[i][j][q] = 0.f;

  // one k-step: the activation fragments of (ms, s) from LDS, then 2 x MS x NS MFMAs
  auto kstep = [&](const uint8_t* st, int s, u32x4_t q0, u32x4_t q1, uint32_t sp0, uint32_t sp1) {
    v8i ahi[kMS], alo[kMS];
    int ash[kMS], asl[kMS];
#pragma unroll
    for (int ms = 0; ms < kMS; ms++) {
      const int row = ms * 32 + l32;
      const int blk = 4 * half + s;
      const u32x4_t p0 = *reinterpret_cast<const u32x4_t*>(st + ((blk * kParts + 0) * kBM + row) * 16);
      const u32x4_t p1 = *reinterpret_cast<const u32x4_t*>(st + ((blk * kParts + 1) * kBM + row) * 16);
      const u32x4_t p2 = *reinterpret_cast<const u32x4_t*>(st + ((blk * kParts + 2) * kBM + row) * 16);
      ahi[ms] = v8i{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, 0, 0};
      alo[ms] = v8i{(int)p1.z, (int)p1.w, (int)p2.x, (int)p2.y, (int)p2.z, (int)p2.w, 0, 0};
      const uint32_t sc = *reinterpret_cast<const uint16_t*>(st + kCodeBytes + row * 16 + blk * 2);
      ash[ms] = (int)(sc & 0xffu);
      asl[ms] = (int)(sc >> 8);
    }
    const v8i bf0 = v8i{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, 0, 0, 0, 0};
    const v8i bf1 = v8i{(int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w, 0, 0, 0, 0};
    const int bs0 = (int)((sp0 >> (8 * (s & 1))) & 0xffu);
    const int bs1 = (int)((sp1 >> (8 * (s & 1))) & 0xffu);
#pragma unroll
    for (int term = 0; term < 2; term++)
#pragma unroll
      for (int ms = 0; ms < kMS; ms++) {
        const v8i a = term ? alo[ms] : ahi[ms];
        const int as_ = term ? asl[ms] : ash[ms];
        acc[ms][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bf0, acc[ms][0], kFmtFp6E2M3, kFmtFp4E2M1,
                                                                     0, as_, 0, bs0);
        acc[ms][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bf1, acc[ms][1], kFmtFp6E2M3, kFmtFp4E2M1,
                                                                     0, as_, 0, bs1);
      }
  };
  // one K group (4 k-steps; blocks past K hold zero activation codes)
#define B_COMPUTE(p, st)                                     \
  do {                                                       \
    kstep(st, 0, p##q00, p##q10, p##s00, p##s10);            \
    kstep(st, 1, p##q01, p##q11, p##s00, p##s10);            \
    kstep(st, 2, p##q02, p##q12, p##s01, p##s11);            \
    kstep(st, 3, p##q03, p##q13, p##s01, p##s11);            \
  } while (0)

  const int NG = KBp / kGroupBlocks;  // even: K is padded to whole pairs of groups
  // Software pipeline over pairs of K groups (g, g + 1), with fixed register
  // sets: weights b0 (even groups) / b1 (odd groups), staged activations ra1
  // (odd groups) / ra0 (even groups).  Every prefetch is consumed in the NEXT
  // iteration, so the compiler cannot sink a prefetch load down to its use (a
  // loop-carried value cannot cross the back edge): weights are requested one
  // group ahead, activations one and a half groups ahead.  Past the last group
  // the prefetch repeats it (no branch; the same loads are outstanding on every
  // path).  Stage 0 holds even groups, stage 1 odd ones; the stage a store
  // writes was last read before the preceding barrier.
  A_DECL(ra0);
  A_DECL(ra1);
  B_DECL(b0);
  B_DECL(b1);
  A_LOAD(ra0, 0);
  A_STORE(ra0, stage0);
  lds_barrier();
  A_LOAD(ra1, min(1, NG - 1));
  A_LOAD(ra0, min(2, NG - 1));
  B_LOAD(b0, 0);
  B_LOAD(b1, min(1, NG - 1));
  for (int g = 0; g < NG; g += 2) {
    B_COMPUTE(b0, stage0);               // group g
    B_LOAD(b0, min(g + 2, NG - 1));
    A_STORE(ra1, stage1);                // group g + 1
    lds_barrier();
    A_LOAD(ra1, min(g + 3, NG - 1));
    B_COMPUTE(b1, stage1);               // group g + 1
    B_LOAD(b1, min(g + 3, NG - 1));
    A_STORE(ra0, stage0);                // group g + 2
    lds_barrier();
    A_LOAD(ra0, min(g + 4, NG - 1));
  }
#undef A_DECL
#undef A_LOAD
#undef A_STORE
#undef B_DECL
#undef B_LOAD
#undef B_COMPUTE

  // ---- epilogue: bias and scatter to the routed rows
#pragma unroll
  for (int ns = 0; ns < kNS; ns++) {
    const int n = n_wave + ns * 32 + l32;
    if (n >= N) continue;
    const float bv = bias ? bf16_bits_to_f32(bias[(size_t)e * N + n]) : 0.f;
#pragma unroll
    for (int ms = 0; ms < kMS; ms++) {
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int row = ms * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        const int r = rows_lds[row];
        if (r >= 0) out[(size_t)r * N + n] = acc[ms][ns][i] + bv;
      }
    }
  }
}

}  // namespace

size_t gemm_workspace_bytes(int T, int k, int K, int x_per_slot) {
  const size_t rq = x_per_slot ? (size_t)T * k : (size_t)T;
  const size_t kbp = (size_t)round_up(K / 32, kKPadBlocks);
  const size_t qbytes = (rq * kbp * kQBytes + 255) & ~(size_t)255;
  return qbytes + rq * kbp * 2;
}

hipError_t launch_expert_gemm(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                              int K, const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                              const int32_t* sorted_rows, float* out, void* workspace, hipStream_t stream) {
  const int Rq = x_per_slot ? T * k : T;
  const int KBp = round_up(K / 32, kKPadBlocks);
  uint8_t* aq = static_cast<uint8_t*>(workspace);
  const size_t qbytes = ((size_t)Rq * KBp * kQBytes + 255) & ~(size_t)255;
  uint8_t* as = aq + qbytes;
  const size_t nblk = (size_t)Rq * KBp;
  hipLaunchKernelGGL(quantize_act_kernel, dim3((unsigned)((nblk + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, x, Rq, K, KBp, aq, as);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int R = T * k;
  const int used = R < E ? R : E;
  const long long NT = (N + kBN - 1) / kBN;
  const long long tiles_max = ((long long)(R + kBM - 1) / kBM + used) * NT;
  const long long grid = (tiles_max + kXcds - 1) / kXcds * kXcds;
  const int KB = K / 32;
  if (KB % 2 == 0)
    hipLaunchKernelGGL(expert_gemm_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, blocks, scales,
                       bias, E, N, K, aq, as, KBp, x_per_slot, T, k, offsets, sorted_rows, out);
  else
    hipLaunchKernelGGL(expert_gemm_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, blocks, scales,
                       bias, E, N, K, aq, as, KBp, x_per_slot, T, k, offsets, sorted_rows, out);
  return hipGetLastError();
}

}  // namespace mxfp4

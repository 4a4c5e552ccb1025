// Prefill expert projection: a grouped GEMM on gfx950 scaled-FP4 MFMA.
//
// For every expert e with M_e routed rows (grouped by mxfp4_moe_route_group):
//   C_e[M_e, N] = X_e[M_e, K] * W_e^T + bias_e,  scattered to out[r, :]
// (gpt-oss-20b files page, README "Loading": one grouped product over the
// tokens sorted by expert, each expert multiplying only the tokens that chose
// it; README "MXFP4" for the weight format).
//
// MI355X design:
//  * The weight codes are fed to v_mfma_scale_f32_32x32x64_f8f6f4 exactly as
//    the checkpoint stores them: a lane of the B operand holds one 16-byte
//    MXFP4 block (32 E2M1 codes, low nibble first) of one weight row, and its
//    E8M0 byte is that lane's B scale.  No dequantization anywhere.
//  * bf16 activations have no MX form, so a pre-pass (quantize_act_kernel)
//    splits every 32-element block of every input row once into two MX-FP6
//    (E2M3) terms, hi + lo, each with its own E8M0 scale, using the gfx950
//    converts v_cvt_scalef32_pk32_fp6_bf16 (round to nearest even of x/2^e)
//    and v_cvt_scalef32_pk32_f32_fp6: hi is the block under the smallest power
//    of two that keeps its largest magnitude <= 7.5, lo the residual x - hi
//    (exact, and exactly a bf16) quantized the same way.  The GEMM issues one
//    MFMA per term; E2M3 x E2M1 runs at the FP4 MFMA rate on gfx950.
//  * Every operand byte reaches LDS by LDS DMA (global_load_lds_dwordx4 /
//    _dword), through a ring of three stages; nothing is staged in registers
//    and the main loop issues no other vector-memory instruction.  A stage is
//    one MFMA k-step: two MX blocks, block 2g + h for the lanes of half h.
//    The address unit, not HBM, bounds this kernel (each DMA instruction
//    gathers 32 rows), so the layouts are chosen for few instructions per
//    stage: the activation records keep the two halves' 16-byte pieces
//    adjacent, and the weight scales are repacked per call (an LDS transpose
//    in repack_wscales_kernel) so that a tile's scales for one stage are 512
//    contiguous bytes.
//  * Tile = 128 routed rows x 256 weight rows; 4 waves as 2 x 2, each owning
//    2 x 4 sub-tiles of 32 x 32 (8 accumulators); 66 KB of LDS, so two
//    workgroups share a CU and cover each other's barriers and prologues.
//  * The tile schedule is derived on the device from expert_offsets (wave
//    scans), ordered so that the row tiles sharing a weight panel run back to
//    back on one XCD and read the panel from its L2.  Surplus workgroups exit
//    at once.  No host synchronisation; any skew of rows per expert.
//  * Routed rows are gathered through sorted_rows by the activation DMA and
//    the results are scattered through it in the epilogue (bias added there).

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
constexpr int kStageBlocks = 2;          // MX blocks per pipeline stage (one MFMA k-step)
constexpr int kStagePad = 3;             // stage counts are padded to a multiple of 3 (the ring)
constexpr int kRecBytes = 96;            // activation record of one (row, stage): [part 3][half 2][16 B]
constexpr int kFmtFp6E2M3 = 2;           // MFMA operand format codes
constexpr int kFmtFp4E2M1 = 4;
constexpr int kXcds = 8;
constexpr int kBM = 128;                 // routed rows per tile: 4 sub-tiles of 32
constexpr int kBN = 256;                 // weight rows per tile: 8 sub-tiles of 32
constexpr int kScaleChunk = 16;          // stages per weight-scale repack workgroup

__host__ __device__ inline int round_up(int v, int m) { return (v + m - 1) / m * m; }

// pipeline stages for K: one per two blocks, padded to a multiple of 3
__host__ __device__ inline int stage_count(int K) {
  return round_up(((K >> 5) + kStageBlocks - 1) / kStageBlocks, kStagePad);
}

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

// One thread per (row, block kb), kb < 2 * NG (blocks past K are zero).
// q: per row and stage g = kb / 2 a 96-byte record [part p][half h][16 B],
//    h = kb % 2; the 48 bytes of a block are hi codes 0..23 | lo codes 0..23,
//    split into parts of 16 (so an MFMA operand is part 0 + half of part 1,
//    or the other half of part 1 + part 2).
// s: [Rq][2 * NG] u32 = hi scale | lo scale << 8.
__global__ __launch_bounds__(kThreads) void quantize_act_kernel(const uint16_t* __restrict__ x, int Rq, int K,
                                                                int NG, uint8_t* __restrict__ q,
                                                                uint32_t* __restrict__ s) {
  const int KB = K >> 5;
  const int KBp = 2 * NG;
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
  uint8_t* rec = q + (row * NG + (kb >> 1)) * kRecBytes + (kb & 1) * 16;
  *reinterpret_cast<uint4*>(rec) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  *reinterpret_cast<uint4*>(rec + 32) = make_uint4(hi[4], hi[5], lo[0], lo[1]);
  *reinterpret_cast<uint4*>(rec + 64) = make_uint4(lo[2], lo[3], lo[4], lo[5]);
  s[idx] = sh | (sl << 8);
}

// ---------------------------------------------------------------------------
// weight-scale repack: [E][N][KB] bytes -> [E][NT][NG][256 rows][2 halves]
// ---------------------------------------------------------------------------

// Workgroup = one (expert, 256-row panel, 16 stages).  Each thread gathers the
// 32 scale bytes of one row, blocks kb0 .. kb0 + 31, from the three aligned
// 16-byte blocks covering them (an aligned block that holds a needed byte
// never leaves that byte's page; past the last needed byte's block the
// blocks repeat it), funnel-shifts them into 8 dwords, and the workgroup
// transposes them through LDS into 16 x 512 contiguous bytes.  Rows past N
// repeat row N - 1 and blocks past K repeat block K - 1: they meet zero
// activations or are never stored.
__global__ __launch_bounds__(kThreads) void repack_wscales_kernel(const uint8_t* __restrict__ scales, int E, int N,
                                                                  int KB, int NT, int NG, uint8_t* __restrict__ out) {
  __shared__ uint32_t tile[kThreads][9];
  const int chunks = (NG + kScaleChunk - 1) / kScaleChunk;
  const int c = blockIdx.x % chunks;
  const int nt = (blockIdx.x / chunks) % NT;
  const int e = blockIdx.x / (chunks * NT);
  const int t = threadIdx.x;
  const int n = min(nt * kBN + t, N - 1);
  const int kb0 = min(c * kScaleChunk * 2, KB - 1);
  const int kb1 = min(c * kScaleChunk * 2 + kScaleChunk * 2 - 1, KB - 1);
  const uintptr_t base = reinterpret_cast<uintptr_t>(scales);
  const uintptr_t first = base + ((size_t)e * N + n) * KB + kb0;
  const uintptr_t blk0 = first & ~(uintptr_t)15;
  const uintptr_t blk1 = (base + ((size_t)e * N + n) * KB + kb1) & ~(uintptr_t)15;
  // the blocks through the (global) scales pointer, so the loads stay global
  const uint4* blocks16 = reinterpret_cast<const uint4*>(scales - (base - blk0));
  const int last16 = (int)((blk1 - blk0) >> 4);
  uint32_t wv[12];
#pragma unroll
  for (int i = 0; i < 3; i++) {
    const uint4 v = blocks16[min(i, last16)];
    wv[4 * i] = v.x; wv[4 * i + 1] = v.y; wv[4 * i + 2] = v.z; wv[4 * i + 3] = v.w;
  }
  const int sh = (int)(first - blk0);  // < 16
  const int sd = sh >> 2, sb = sh & 3;
  auto pick = [&](int i) { return sd == 0 ? wv[i] : sd == 1 ? wv[i + 1] : sd == 2 ? wv[i + 2] : wv[i + 3]; };
#pragma unroll
  for (int m = 0; m < 8; m++) tile[t][m] = __builtin_amdgcn_alignbyte(pick(m + 1), pick(m), sb);
  __syncthreads();
  // stage gs = c * 16 + st: 512 bytes = 128 dwords (row pair 2j, 2j + 1; halves 0, 1)
  auto byte_at = [&](int r, int col) { return (tile[r][col >> 2] >> (8 * (col & 3))) & 0xffu; };
  uint32_t* dst = reinterpret_cast<uint32_t*>(out + (((size_t)e * NT + nt) * NG + (size_t)c * kScaleChunk) * 512);
  for (int i = t; i < kScaleChunk * 128; i += kThreads) {
    const int st = i >> 7, j = i & 127;
    const int gs = c * kScaleChunk + st;
    if (gs >= NG) break;
    const int c0 = min(2 * gs, KB - 1) - kb0, c1 = min(2 * gs + 1, KB - 1) - kb0;
    dst[i] = byte_at(2 * j, c0) | (byte_at(2 * j, c1) << 8) | (byte_at(2 * j + 1, c0) << 16) |
             (byte_at(2 * j + 1, c1) << 24);
  }
}

// ---------------------------------------------------------------------------
// grouped GEMM
// ---------------------------------------------------------------------------

// LDS of one ring slot
constexpr int kACodeBytes = 4 * 3 * 64 * 16;   // [row sub-tile][part][lane] x 16 B
constexpr int kAScaleBytes = 4 * 64 * 4;       // [row sub-tile][lane] x u32
constexpr int kBCodeBytes = 8 * 64 * 16;       // [column sub-tile][lane] x 16 B
constexpr int kBScaleBytes = 512;              // [256 rows][2 halves] bytes
constexpr int kASlot = kACodeBytes + kAScaleBytes;
constexpr int kBSlot = kBCodeBytes + kBScaleBytes;
// LDS DMAs one wave issues per stage: 3 activation-code parts, 1 activation
// scale word, 2 weight-code sub-tiles, 1 weight-scale half
constexpr int kDmaPerStage = 7;

struct TileCoord {
  int e, m_begin, m_count, nt;
};

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Routed rows [b, f) of expert e, both ends clamped into [0, R], so no offset
// can send a read outside sorted_rows.
__device__ __forceinline__ void expert_rows(const int32_t* offsets, int e, int R, int& b, int& f) {
  b = min(max(offsets[e], 0), R);
  f = min(max(offsets[e + 1], b), R);
}

// Tile t of the grouped problem: experts in order; within an expert the weight
// panel (n-tile) varies slowest so that the row tiles sharing a panel are
// consecutive.  Workgroup L takes tile (L % 8) * ceil(tiles / 8) + L / 8:
// workgroups are dispatched round-robin over the 8 XCDs, so consecutive tiles
// run on one XCD and share its L2.  Each wave decodes its tile itself (wave
// scans over 64 experts at a time), so no barrier is needed.
__device__ __forceinline__ bool locate_tile(const int32_t* offsets, int E, int R, int NT, int lane, TileCoord& c) {
  int total = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    int cnt = 0;
    if (e < E) {
      int b, f;
      expert_rows(offsets, e, R, b, f);
      cnt = (f - b + kBM - 1) / kBM * NT;
    }
    total += wave_sum_i(cnt);
  }
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int L = blockIdx.x;
  const int j = L / kXcds;
  if (j >= per_xcd) return false;
  const int t = (L % kXcds) * per_xcd + j;
  if (t >= total) return false;
  int before = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    int cnt = 0, b = 0, f = 0;
    if (e < E) {
      expert_rows(offsets, e, R, b, f);
      cnt = (f - b + kBM - 1) / kBM * NT;
    }
    const int incl = wave_incl_scan(cnt, lane);
    const int tl = t - before;
    const uint64_t hit = wave_ballot(cnt > 0 && incl - cnt <= tl && tl < incl);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int eb = __shfl(b, src, 64), ef = __shfl(f, src, 64);
      const int local = tl - (__shfl(incl, src, 64) - __shfl(cnt, src, 64));
      const int mt = (ef - eb + kBM - 1) / kBM;
      const int nt = local / mt;
      const int mi = local - nt * mt;
      // wave-uniform by construction; say so, so that branches on them are scalar
      c.e = __builtin_amdgcn_readfirstlane(base + src);
      c.m_begin = __builtin_amdgcn_readfirstlane(eb + mi * kBM);
      c.m_count = __builtin_amdgcn_readfirstlane(min(kBM, ef - (eb + mi * kBM)));
      c.nt = __builtin_amdgcn_readfirstlane(nt);
      return true;
    }
    before += __shfl(incl, 63, 64);
  }
  return false;
}

#define MXFP4_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// 16 (or 4) bytes per lane from global memory straight into LDS at dst + 16 *
// lane (4 * lane).
__device__ __forceinline__ void dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, MXFP4_LDS(dst), 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, MXFP4_LDS(dst), 4, 0, 0);
}

// Wait until at most VM of this wave's vector-memory instructions are
// outstanding and all its LDS instructions are done, then meet the other waves.
// The LDS DMAs of a stage count in the vector-memory counter, so after the
// barrier every wave sees every wave's finished stages.  Only compiler-level
// fences: a workgroup fence would also wait for the DMAs still in flight.
template <int VM>
__device__ __forceinline__ void stage_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));  // vmcnt(VM) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup = 4 waves as 2 x 2 over the 128 x 256 tile: wave (wm, wn) owns the
// row sub-tiles wm and wm + 2 and the column sub-tiles wn + 2q, q < 4 (the
// interleave spreads the work of a ragged last tile over the waves).  K
// advances one MFMA k-step (two MX blocks) per stage through a ring of three
// LDS slots: stage g + 2 is requested while stage g is multiplied.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void expert_gemm_kernel(
    const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ bsc, const uint16_t* __restrict__ bias,
    int E, int N, int K, const uint8_t* __restrict__ aq, const uint32_t* __restrict__ as, int x_per_slot, int T,
    int k, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows, float* __restrict__ out) {
  // one LDS array per ring slot and operand: the compiler tracks DMA writes per array
  __shared__ __attribute__((aligned(16))) uint8_t sA0[kASlot];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[kASlot];
  __shared__ __attribute__((aligned(16))) uint8_t sA2[kASlot];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[kBSlot];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[kBSlot];
  __shared__ __attribute__((aligned(16))) uint8_t sB2[kBSlot];
  __shared__ int rows_lds[kBM];  // routed row of each tile row, -1 if none

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  // Never taken (K >= 32).  Arrays written only by LDS DMA look unwritten to
  // the optimizer, which would then fold their loads away.
  if (K < 0) sA0[tid] = sA1[tid] = sA2[tid] = sB0[tid] = sB1[tid] = sB2[tid] = 0;

  const int R = T * k;
  const int NT = (N + kBN - 1) / kBN;
  TileCoord tc;
  if (!locate_tile(offsets, E, R, NT, lane, tc)) return;
  const int e = tc.e;
  const int KB = K >> 5;
  const int NG = stage_count(K);
  const int wm = wave & 1, wn = wave >> 1;

  auto routed = [&](int i) -> int {
    if (i >= tc.m_count) return -1;
    const int r = sorted_rows[tc.m_begin + i];
    return (r < 0 || r >= R) ? -1 : r;
  };
  // quantized-input row of a routed row (row 0 stands in for empty tile rows,
  // whose results are never stored)
  auto src_of = [&](int r) { return r < 0 ? 0 : (x_per_slot ? r : r / k); };
  if (tid < kBM) rows_lds[tid] = routed(tid);

  // activation DMA: wave w stages row sub-tile w.  Lane (l32, h) reads the
  // three 16-byte parts of block 2g + h of its row; the scale DMA its word.
  const int src = src_of(routed(wave * 32 + l32));
  const uint8_t* a_dma = aq + (size_t)src * NG * kRecBytes + half * 16;
  const uint32_t* as_dma = as + (size_t)src * 2 * NG + half;
  // weight-code DMA: wave w stages column sub-tiles 2w and 2w + 1 (rows past
  // N re-read row N - 1; they are never stored)
  const int n_base = tc.nt * kBN;
  const uint8_t* b_dma0 = blocks + ((size_t)e * N + min(n_base + 64 * wave + l32, N - 1)) * KB * 16;
  const uint8_t* b_dma1 = blocks + ((size_t)e * N + min(n_base + 64 * wave + 32 + l32, N - 1)) * KB * 16;
  // weight-scale DMA: the 512 bytes of a stage as two 256-byte halves; waves
  // 0 / 2 and 1 / 3 stage the same half (the same bytes to the same place)
  const uint8_t* bs_dma = bsc + ((size_t)e * NT + tc.nt) * NG * 512 + (wave & 1) * 256 + lane * 4;
  // bias of the wave's own column sub-tiles
  int ncol[4];
  float bias_v[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    ncol[q] = n_base + 32 * (wn + 2 * q) + l32;
    bias_v[q] = bias ? bf16_bits_to_f32(bias[(size_t)e * N + min(ncol[q], N - 1)]) : 0.f;
  }
  const bool valid0 = wm * 32 < tc.m_count;
  const bool valid1 = (wm + 2) * 32 < tc.m_count;

  // ---- one stage's requests: 7 LDS DMAs
  auto issue = [&](int g, uint8_t* sa, uint8_t* sb) {
    const int kbc = min(2 * g + half, KB - 1);
    const uint8_t* a = a_dma + (size_t)g * kRecBytes;
    dma16(a, sa + (wave * 3 + 0) * 1024);
    dma16(a + 32, sa + (wave * 3 + 1) * 1024);
    dma16(a + 64, sa + (wave * 3 + 2) * 1024);
    dma4(as_dma + 2 * g, sa + kACodeBytes + wave * 256);
    dma16(b_dma0 + (size_t)kbc * 16, sb + (2 * wave) * 1024);
    dma16(b_dma1 + (size_t)kbc * 16, sb + (2 * wave + 1) * 1024);
    dma4(bs_dma + (size_t)g * 512, sb + kBCodeBytes + (wave & 1) * 256);
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int q = 0; q < 16; q++) acc[i][j][q] = 0.f;

  // ---- one stage's MFMAs.  A wave whose row sub-tiles are empty (a ragged
  // last tile) skips their MFMAs; it still requests its share of every stage.
  auto compute = [&](const uint8_t* sa, const uint8_t* sb) {
    if (!valid0) return;
    v8i bf[4];
    int bs[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int c = wn + 2 * q;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sb + (c * 64 + lane) * 16);
      bf[q] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      bs[q] = sb[kBCodeBytes + (c * 32 + l32) * 2 + half];
    }
    auto subtile = [&](int i) {
      const int ms = wm + 2 * i;
      const uint8_t* base = sa + (ms * 3 * 64 + lane) * 16;
      const u32x4_t p0 = *reinterpret_cast<const u32x4_t*>(base);
      const u32x4_t p1 = *reinterpret_cast<const u32x4_t*>(base + 64 * 16);
      const u32x4_t p2 = *reinterpret_cast<const u32x4_t*>(base + 2 * 64 * 16);
      const int sc = *reinterpret_cast<const int*>(sa + kACodeBytes + (ms * 64 + lane) * 4);
      const v8i ahi = v8i{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, 0, 0};
      const v8i alo = v8i{(int)p1.z, (int)p1.w, (int)p2.x, (int)p2.y, (int)p2.z, (int)p2.w, 0, 0};
#pragma unroll
      for (int q = 0; q < 4; q++)
        acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ahi, bf[q], acc[i][q], kFmtFp6E2M3, kFmtFp4E2M1,
                                                                    0, sc, 0, bs[q]);
#pragma unroll
      for (int q = 0; q < 4; q++)
        acc[i][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(alo, bf[q], acc[i][q], kFmtFp6E2M3, kFmtFp4E2M1,
                                                                    1, sc, 0, bs[q]);
    };
    subtile(0);
    if (valid1) subtile(1);
  };

  // ---- the pipeline: slot g % 3 holds stage g.  At stage g: wait for this
  // wave's requests of stage g (only those of stage g + 1 may still be in
  // flight), barrier (every wave's stage g has landed and every wave is done
  // reading stage g - 1), request stage g + 2 into the slot of stage g - 1,
  // multiply stage g.  The stage count is a multiple of 3 (the padding blocks
  // hold zero activation codes), so the loop body is three straight-line
  // steps; the last three are peeled off because they request less.
  issue(0, sA0, sB0);
  issue(1, sA1, sB1);
  int g = 0;
  for (; g + 3 < NG; g += 3) {
    stage_barrier<kDmaPerStage>();
    issue(g + 2, sA2, sB2);
    compute(sA0, sB0);
    stage_barrier<kDmaPerStage>();
    issue(g + 3, sA0, sB0);
    compute(sA1, sB1);
    stage_barrier<kDmaPerStage>();
    issue(g + 4, sA1, sB1);
    compute(sA2, sB2);
  }
  stage_barrier<kDmaPerStage>();
  issue(g + 2, sA2, sB2);
  compute(sA0, sB0);
  stage_barrier<kDmaPerStage>();
  compute(sA1, sB1);
  stage_barrier<0>();
  compute(sA2, sB2);

  // ---- epilogue: bias and scatter to the routed rows (rows_lds was written
  // before the first stage barrier)
#pragma unroll
  for (int i = 0; i < 2; i++) {
    if (!(i == 0 ? valid0 : valid1)) continue;
    const int ms = wm + 2 * i;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int n = ncol[q];
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int row = ms * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
        const int r = rows_lds[row];
        if (r >= 0) out[(size_t)r * N + n] = acc[i][q][j] + bias_v[q];
      }
    }
  }
}

struct GemmLayout {
  size_t codes, scales, wscales, total;
};

GemmLayout gemm_layout(int E, int N, int T, int k, int K, int x_per_slot) {
  const size_t rq = x_per_slot ? (size_t)T * k : (size_t)T;
  const size_t ng = (size_t)stage_count(K);
  const size_t nt = (size_t)((N + kBN - 1) / kBN);
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  GemmLayout l;
  l.codes = 0;
  l.scales = al(rq * ng * kRecBytes);
  l.wscales = l.scales + al(rq * 2 * ng * 4);
  l.total = l.wscales + al((size_t)E * nt * ng * 512);
  return l;
}

}  // namespace

size_t gemm_workspace_bytes(int E, int N, int T, int k, int K, int x_per_slot) {
  return gemm_layout(E, N, T, k, K, x_per_slot).total;
}

hipError_t launch_expert_gemm(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                              int K, const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                              const int32_t* sorted_rows, float* out, void* workspace, hipStream_t stream) {
  const int Rq = x_per_slot ? T * k : T;
  const int NG = stage_count(K);
  const int NT = (N + kBN - 1) / kBN;
  const GemmLayout l = gemm_layout(E, N, T, k, K, x_per_slot);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* aq = ws + l.codes;
  uint32_t* as = reinterpret_cast<uint32_t*>(ws + l.scales);
  uint8_t* bsc = ws + l.wscales;
  const size_t nblk = (size_t)Rq * 2 * NG;
  hipLaunchKernelGGL(quantize_act_kernel, dim3((unsigned)((nblk + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, x, Rq, K, NG, aq, as);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long rep = (long long)E * NT * ((NG + kScaleChunk - 1) / kScaleChunk);
  hipLaunchKernelGGL(repack_wscales_kernel, dim3((unsigned)rep), dim3(kThreads), 0, stream, scales, E, N, K / 32, NT,
                     NG, bsc);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int R = T * k;
  const int used = R < E ? R : E;
  const long long tiles_max = ((long long)(R + kBM - 1) / kBM + used) * NT;
  const long long grid = (tiles_max + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(expert_gemm_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, blocks, bsc, bias, E, N,
                     K, aq, as, x_per_slot, T, k, offsets, sorted_rows, out);
  return hipGetLastError();
}

}  // namespace mxfp4

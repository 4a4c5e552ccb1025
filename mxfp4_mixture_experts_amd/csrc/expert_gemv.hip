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
// offsets) and row blocks of WAVES * 16 consecutive weight rows, 16 per wave:
// blocks blockIdx.x, blockIdx.x + gridDim.x, ... streamed back to back with
// the token rows staged once.  A wave streams
// its 16 weight rows in squares of 16 rows x 8 MX blocks: each 128-bit load
// of the wave covers 8 rows x 128 contiguous bytes (whole lines), and the
// square then passes through the wave's LDS so that lane l holds row l % 16,
// block 4 g + l / 16 of K group g, as the MFMA wants it.  The loads run a
// ring of two to four chunks of NCH 128-element K groups (the next chunks are
// in flight while the current one is multiplied), and the first chunks are
// issued before the expert's token rows (up to MT per pass) are staged in LDS
// as bf16, with zeros past K so that the padded K groups need no mask; the
// four MFMAs of a group accumulate into four independent accumulators.
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
#include "mxfp4_moe.h"
#include "route_common.h"

namespace mxfp4 {
namespace {

constexpr int kFusedMaxE = MXFP4_DECODE_MAX_EXPERTS;  // fused decode: experts ranked per lane
constexpr int kFusedMaxT = MXFP4_DECODE_MAX_T;        // fused decode: tokens, one per lane
static_assert(kFusedMaxE <= 64 && kFusedMaxT <= 64, "one wave");

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

#define MXFP4_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// 16 bytes per lane from global memory straight into LDS at dst + 16 * lane.
__device__ __forceinline__ void dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, MXFP4_LDS(dst), 16, 0, 0);
}

// Wait until at most VM vector-memory instructions of this wave are
// outstanding and its LDS instructions are done, then meet the other waves.
// Only compiler-level fences: a workgroup fence would also wait for the LDS
// DMAs and weight loads still in flight.
template <int VM>
__device__ __forceinline__ void bare_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));  // vmcnt(VM) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier that orders LDS only: __syncthreads() would also wait for
// every weight load in flight (its fence covers global memory).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// the bias of a projection without one
__device__ const uint16_t kZeroBf16 = 0;

// word 3 of a raw buffer resource (stride 0, byte offsets, 32-bit data format)
constexpr int kWBufferFlags = 0x00020000;
// cache policy of a buffer load: non-temporal (streamed data read once)
constexpr int kNtPolicy = 2;

__device__ __forceinline__ float e8m0_to_float(uint32_t s) {
  // 2^(s - 127) as an fp32 bit pattern; s = 0 is the subnormal 2^-127
  return __uint_as_float(max(s << 23, 0x00400000u));  // s >= 1: at least 2^-126 = 0x00800000
}

// The routing a fused decode launch computes itself (the outputs of
// mxfp4_moe_route_group for its logits).
struct FusedRoute {
  const uint16_t* logits;
  int32_t* topk_ids;
  float* gates;
  int32_t* offsets;
  int32_t* sorted_rows;
  int32_t* error_word;
};

// The routing outputs of a fused decode launch that concern expert e, by the
// expert's workgroup chosen for it, from the batch's logits staged in lg (T
// rows of LP floats).  Wave w takes tokens w, w + WAVES, ..., one at a time,
// lane j holding expert j's logit: the token's kept experts are found as
// route_ranked keeps them (k rounds of the largest remaining logit, the lowest
// lane first among equal ones), its gates as route_ranked computes them (the
// exponentials relative to the largest logit over the same wave sum), so that
// every output equals the routing launch's bit for bit.  Writes the id and gate
// of every slot that holds e, offsets[e] (offsets[E] for the last expert), e's
// segment of sorted_rows (rows, m of them), and for e = 0 the slots of the
// tokens with a NaN logit and the error word.  cnt: WAVES x 64 ints; nan_seen:
// zero on entry.  Every thread of the workgroup calls it.
template <int WAVES>
__device__ __forceinline__ void fused_write_routing(const FusedRoute fr, int T, int E, int k, int e, int lane,
                                                    int wave, const float* lg, int LP, const int* rows, int m,
                                                    int* cnt, int* nan_seen) {
  int kept_count = 0;  // lane j: this wave's tokens that keep expert j
  for (int t = wave; t < T; t += WAVES) {
    const float l = lane < E ? lg[t * LP + lane] : -INFINITY;
    if (__ballot(lane < E && l != l)) {
      if (lane == 0) *nan_seen = 1;
      if (e == 0 && lane < k) {
        fr.topk_ids[(size_t)t * k + lane] = -1;
        if (fr.gates) fr.gates[(size_t)t * k + lane] = 0.f;
      }
      continue;
    }
    bool taken = false;
    int slot = 0;
    float mx = 0.f;
    for (int s = 0; s < k; s++) {
      const float top = wave_max(taken || lane >= E ? -INFINITY : l);
      const uint64_t cand = __ballot(!taken && lane < E && l == top);
      if (lane == __ffsll((long long)cand) - 1) {
        taken = true;
        slot = s;
      }
      if (s == 0) mx = top;
    }
    const float num = taken ? expf(l - mx) : 0.f;
    const float sum = wave_sum(num);
    if (lane == e && taken) {
      fr.topk_ids[(size_t)t * k + slot] = e;
      if (fr.gates) fr.gates[(size_t)t * k + slot] = num / sum;
    }
    kept_count += taken ? 1 : 0;
  }
  cnt[wave * 64 + lane] = kept_count;
  __syncthreads();
  if (wave == 0) {
    int tot = 0;
    for (int w = 0; w < WAVES; w++) tot += cnt[w * 64 + lane];
    int inc = tot;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d, 64);
      if (lane >= d) inc += o;
    }
    const int off = __builtin_amdgcn_readlane(inc - tot, e);
    const int total = __builtin_amdgcn_readlane(inc, 63);
    if (lane < m) fr.sorted_rows[off + lane] = rows[lane];
    if (lane == 0) {
      fr.offsets[e] = off;
      if (e == E - 1) fr.offsets[E] = total;
      if (e == 0 && fr.error_word) *fr.error_word = *nan_seen ? MXFP4_ROUTE_ERR_ID_RANGE : 0;
    }
  }
}

// A fused decode launch of T <= 64 tokens (E <= 64): the workgroup of expert e
// finds its routed rows itself.  The batch's logits are staged in LDS (lg,
// T x (E + 1) floats: rows padded so that one lane per token reads without
// bank conflicts) with coalesced loads, all in flight at once; then lane t of
// wave 0 ranks expert e among token t's logits (the rank definition of
// route_ranked, evaluated for one expert).  The rows t * k + rank of the
// tokens that keep e, in ascending t, are the rows mxfp4_moe_route_group
// groups under e, in its order; a token with a NaN logit keeps no expert.
// Wave 0 writes them to rows_out; the workgroup chosen to (route) then writes
// the routing outputs for e, with WAVES x 64 + 1 ints of LDS after lg.
// Returns the row count (every wave).
template <int WAVES>
__device__ __forceinline__ int fused_expert_rows(const FusedRoute fr, int T, int E, int k, int e, int lane, int wave,
                                                 bool route, float* lg, int* rows_out, int* count) {
  const int LP = E + 1;
  int* scratch = reinterpret_cast<int*>(lg + T * LP);
  constexpr int kPer = (kFusedMaxT + WAVES - 1) / WAVES;  // token rows per wave
  uint32_t v[kPer];
#pragma unroll
  for (int q = 0; q < kPer; q++) {
    const int t = wave + q * WAVES;
    v[q] = fr.logits[(size_t)min(t, T - 1) * E + min(lane, E - 1)];  // unconditional loads
  }
#pragma unroll
  for (int q = 0; q < kPer; q++) {
    const int t = wave + q * WAVES;
    if (t < T && lane < E) lg[t * LP + lane] = bf16_bits_to_f32(v[q]);
  }
  if (threadIdx.x == 0) scratch[WAVES * 64] = 0;
  __syncthreads();
  if (wave == 0) {
    const float* row = lg + min(lane, T - 1) * LP;
    const float le = row[e];
    int rank = 0;
    bool nan = false;
    for (int j = 0; j < E; j++) {
      const float lj = row[j];
      rank += (lj > le || (lj == le && j < e)) ? 1 : 0;
      nan |= lj != lj;
    }
    const bool keep = lane < T && !nan && rank < k;
    const uint64_t mask = __ballot(keep);
    if (keep) rows_out[lanes_below(mask)] = lane * k + rank;
    if (lane == 0) *count = __popcll(mask);
  }
  __syncthreads();
  const int m = *count;
  if (route) fused_write_routing<WAVES>(fr, T, E, k, e, lane, wave, lg, LP, rows_out, m, scratch, scratch + WAVES * 64);
  __syncthreads();
  return m;
}

template <int MT, int WAVES, int NCH, int NST, int KS, int OCC, bool SWIGLU, bool FR = false, bool TR2 = false>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(OCC))) void expert_gemv_kernel(
    const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ scales, const uint16_t* __restrict__ bias,
    int E, int N, int K, const uint16_t* __restrict__ x, int x_per_slot, int T, int k,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows, float* __restrict__ out,
    uint16_t* __restrict__ act, int sc_blk, FusedRoute fr) {
  // [MT][XS] bf16 token rows, 16 bytes per entry (16 per K group), staged by
  // LDS DMA; entries past K and rows past the pass's count are zeroed in
  // registers when read.  Then, per row block of the workgroup, sc_blk
  // entries of weight scales.
  extern __shared__ uint4 xs[];
  __shared__ int rows_lds[MT];
  __shared__ int fused_rows[FR ? kFusedMaxT : 1];  // FR: the expert's routed rows and their count
  __shared__ int fused_count;
  // KS > 1: the KS waves of a row group split K and add their partial sums here
  constexpr int RW = WAVES / KS;  // row groups (16 weight rows each) per workgroup
  static_assert(WAVES % KS == 0, "whole row groups");
  __shared__ f32x4_v red[KS > 1 ? RW * (KS - 1) * 64 : 1];
  const int KB = K >> 5;
  const int K8 = K >> 3;
  const int NIT = (KB + 3) >> 2;
  // K groups padded to whole rounds of NST chunks per K part (padding groups
  // re-read the row's last block and meet zero activations)
  const int NITC = (NIT + KS * NST * NCH - 1) / (KS * NST * NCH) * (KS * NST * NCH);
  const int XS = (NITC * 16 + 63) / 64 * 64 + 1;  // whole 64-entry DMAs, +1 spreads rows over banks
  static_assert(NST >= 2 && NST <= 4, "two to four chunks in flight");
  static_assert(NCH % 2 == 0, "whole squares of 16 rows x 8 blocks");
  const int R = T * k;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  int e, m0, m1;
  if constexpr (FR) {
    // one row of workgroups per expert by index; the last workgroup of each
    // (one with the fewest weight-row blocks, done early) writes the expert's
    // routing outputs
    e = blockIdx.y;
    m0 = 0;
    m1 = __builtin_amdgcn_readfirstlane(fused_expert_rows<WAVES>(fr, T, E, k, e, lane, wave,
                                                                 blockIdx.x == gridDim.x - 1,
                                                                 reinterpret_cast<float*>(xs), fused_rows,
                                                                 &fused_count));
    if (m1 == 0) return;
  } else {
    if (!find_group(offsets, E, R, blockIdx.y, lane, e, m0, m1)) return;
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    m1 = __builtin_amdgcn_readfirstlane(m1);
  }

  // Row blocks of RW * 16 weight rows: this workgroup takes blocks
  // blockIdx.x + j * gridDim.x, j < nb, and streams them back to back (the
  // first chunks of block j + 1 are requested while block j finishes), so
  // the token rows are staged once for all of them.
  const int nblk = (N + RW * 16 - 1) / (RW * 16);
  const int nb = (nblk - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int rw = wave / KS, kpart = wave % KS;
  const int kq = lane >> 4;
  auto block_row0 = [&](int j) { return ((int)blockIdx.x + j * (int)gridDim.x) * RW * 16; };
  // this lane's weight row in block j (rows past N re-read row N - 1 and meet zero activations)
  auto lane_row = [&](int j) { return block_row0(j) + rw * 16 + (lane & 15); };
  // the wave's first weight row in block j
  auto wrow_of = [&](int j) { return block_row0(j) + rw * 16; };
  // A chunk is NCH / 2 squares of 16 rows x 8 blocks (2 K groups).  Load i
  // covers half i % 2 of square i / 2, 8 rows x 128 contiguous bytes (whole
  // lines; the MFMA's own layout, 16 rows x 64 bytes, streams markedly
  // slower): lane l takes row 8 (i % 2) + l / 8, block l % 8 of the square.
  // step 1: the chunk's groups; step 0: the first square again (a placeholder
  // request, almost free).  Rows past N re-read row N - 1 and blocks past K
  // the row's last block; they meet zero activations.
  // The expert's codes as one buffer resource (at most 4 GiB, checked on the
  // host): a 32-bit lane offset per row half and the K position in the scalar
  // offset.  A lane's blocks past K fall in the next row, or past the expert's
  // last byte, where the resource returns zeros: finite codes that meet zero
  // activations.
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(blocks + (size_t)e * N * KB * 16), (short)0, (int)((uint32_t)N * (uint32_t)(KB * 16)),
      kWBufferFlags);
  auto load_chunk = [&](int wr, int c0, uint4 (&w)[NCH], int step = 1) {
    const uint32_t voff[2] = {(uint32_t)min(wr + (lane >> 3), N - 1) * (uint32_t)(KB * 16) + (lane & 7) * 16,
                              (uint32_t)min(wr + 8 + (lane >> 3), N - 1) * (uint32_t)(KB * 16) + (lane & 7) * 16};
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const u32x4_t v =
          __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)voff[i & 1], (c0 + (i & ~1) * step) * 64, kNtPolicy);
      w[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  // The MFMA wants lane l on row l % 16 and block 4 g + l / 16 of K group g.
  // TR2: each square passes through the wave's own 2 KB of LDS, [16 rows][8
  // pieces of 16 bytes] with piece b of row r at b ^ (r / 2 % 8), written by
  // every lane before the square's first group.  Otherwise (less LDS, for the
  // widest K) each K group passes through 1 KB, [16 rows][4 pieces] with piece
  // b of row r at b ^ (r / 4 % 4), written by the lanes that hold it.  Either
  // way the writes (2 rows per 16 lanes) and the reads (16 rows, one piece)
  // hit distinct banks.  A wave's LDS accesses complete in order.
  constexpr int kTrBytes = TR2 ? 2048 : 1024;
  uint8_t* trw = reinterpret_cast<uint8_t*>(xs + MT * XS) + wave * kTrBytes;
  auto tr_at = [&](int r, int b) {
    return TR2 ? trw + r * 128 + ((b ^ ((r >> 1) & 7)) << 4) : trw + r * 64 + ((b ^ ((r >> 2) & 3)) << 4);
  };

  // ---- weight scales of block j: rows row0 .. row0 + RW * 16 - 1 (clamped to
  // N - 1), contiguous in memory: the aligned 16-byte blocks from the one
  // holding the first byte to the one holding the last (an aligned block that
  // holds a valid byte never leaves that byte's page).  Lane byte (row, kb)
  // then sits at sc_base + (row - row0) * KB + kb of the block's LDS region.
  const uintptr_t sbase = reinterpret_cast<uintptr_t>(scales);
  auto sc_span = [&](int j, int& n_sblk, int& sc_base, const uint4*& s_blocks) {
    const int row0 = block_row0(j);
    const int rows_b = min(RW * 16, N - row0);
    const uintptr_t s_first = sbase + ((size_t)e * N + row0) * KB;
    const uintptr_t s_blk0 = s_first & ~(uintptr_t)15;
    const uintptr_t s_blk1 = (s_first + (size_t)rows_b * KB - 1) & ~(uintptr_t)15;
    n_sblk = (int)((s_blk1 - s_blk0) >> 4) + 1;
    sc_base = (int)(s_first - s_blk0);
    // the same blocks through the (global) scales pointer, so loads stay global
    s_blocks = reinterpret_cast<const uint4*>(scales - (sbase - s_blk0));
  };
  uint4* sc_lds = xs + MT * XS + WAVES * (kTrBytes / 16);

  for (int mb = m0; mb < m1; mb += MT) {
    const int mc = min(MT, m1 - mb);
    // ---- prologue.  The token rows and every block's weight-scale blocks go
    // to LDS by LDS DMA (no registers), issued before all of this wave's first
    // NST chunks of weights; the wave then waits for its DMAs only (the weight
    // loads are younger, and the counter is in order) and meets the others.
    // Every wave issues the same number of DMAs (a wave with fewer real ones
    // repeats one: the same bytes to the same place).  Lanes past the data
    // read a clamped source into padding that is never read.
    bare_barrier<63>();  // the previous pass is done with the staged rows (its reads have returned)
    uint4 wq[NST][NCH];  // the ring of chunks in flight
    const int g_first = kpart * (NITC / KS);  // this wave's first K group
    // Without fused routing the first weight chunks go out first: their
    // addresses need only the expert, and the routed rows below are read with
    // scalar loads, whose counter is not behind them.
    if constexpr (!FR) {
      const int wr0 = wrow_of(0);
#pragma unroll
      for (int st = 0; st < NST; st++) load_chunk(wr0, g_first + st * NCH, wq[st]);
    }
    // the pass's routed rows (lane m: row m, clamped indices read
    // unconditionally), then token row m's source as a uniform value
    int src[MT];
    {
      int r;
      if constexpr (FR) {
        r = fused_rows[mb + min(lane, mc - 1)];
      } else {
        const int32_t* srp = sorted_rows + mb;
        r = -1;
#pragma unroll
        for (int m = 0; m < MT; m++) {
          const int rm = srp[min(m, mc - 1)];
          r = lane == m ? rm : r;
        }
      }
      if (lane >= mc || r < 0 || r >= R) r = -1;
      const int s = r < 0 ? 0 : (x_per_slot ? r : r / k);  // row 0 stands in: masked when read
#pragma unroll
      for (int m = 0; m < MT; m++) src[m] = __builtin_amdgcn_readlane(s, m);
      if (threadIdx.x < MT) rows_lds[threadIdx.x] = r;
    }
    {
      // scale blocks: 64 per DMA, instructions spread over the waves
      for (int j = 0; j < nb; j++) {
        int n_sblk, sc_base;
        const uint4* s_blocks;
        sc_span(j, n_sblk, sc_base, s_blocks);
        const int n_si = (n_sblk + 63) >> 6;
        const int per_wave = (n_si + WAVES - 1) / WAVES;
        for (int q = 0; q < per_wave; q++) {
          const int ins = (q * WAVES + wave) % n_si;
          const int b = min(ins * 64 + lane, n_sblk - 1);
          dma16(s_blocks + b, reinterpret_cast<uint8_t*>(sc_lds + j * sc_blk + ins * 64));
        }
      }
      // token rows: 64 entries per DMA, the lanes below K only
      const int x_per_row = (NITC * 16 + 63) >> 6;
      const int n_xi = mc * x_per_row;
      const int xper_wave = (n_xi + WAVES - 1) / WAVES;
      for (int q = 0; q < xper_wave; q++) {
        const int ins = (q * WAVES + wave) % n_xi;
        const int m = ins / x_per_row, jx = ins - m * x_per_row;
        const int c = jx * 64 + lane;
        if (c < K8)
          dma16(reinterpret_cast<const uint4*>(x + (size_t)src[m] * K) + c,
                reinterpret_cast<uint8_t*>(xs + m * XS + jx * 64));
      }
      // the entries past K that the padded K groups read are zeros (they meet
      // the finite codes past each row's end); rows past the pass's count are
      // not written: they feed only output rows that are never stored
      const int npad = NITC * 16 - K8;
      for (int i = threadIdx.x; i < MT * npad; i += WAVES * 64) {
        const int m = i / npad;
        xs[m * XS + K8 + (i - m * npad)] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    asm volatile("" ::: "memory");  // the weight loads stay behind the DMAs
    if constexpr (FR) {
      const int wr0 = wrow_of(0);
#pragma unroll
      for (int st = 0; st < NST; st++) load_chunk(wr0, g_first + st * NCH, wq[st]);
      bare_barrier<NST * NCH>();  // every wave's DMAs have landed
    } else {
      bare_barrier<0>();  // every wave's DMAs (and the older first chunks) have landed
    }

    const uint4* xrow = xs + min(lane & 15, mc - 1) * XS + kq * 4;
    auto xread = [&](int idx) { return xrow[idx]; };

    for (int j = 0; j < nb; j++) {
      const int row0 = block_row0(j);
      const int row = lane_row(j);
      const bool row_ok = row < N;
      const int wrow = wrow_of(j);
      const bool more = j + 1 < nb;  // uniform
      const int wnext = wrow_of(min(j + 1, nb - 1));
      const int nstep = more ? 1 : 0;   // after the last block: placeholder requests
      const int nfirst = more ? g_first : 0;
      // the row's bias, loaded unconditionally (from a zero without bias: a
      // load under a branch ends in a wait for every load in flight) through
      // an opaque address (so it is not sunk to its use), consumed at the end
      uint32_t bias_bits;
      {
        const uint16_t* bp = bias ? bias + (size_t)e * N + min(row, N - 1) : &kZeroBf16;
        asm volatile("" : "+v"(bp));
        bias_bits = *(const __attribute__((address_space(1))) uint16_t*)(bp);
      }
      int sc_base;
      {
        int n_sblk;
        const uint4* s_blocks;
        sc_span(j, n_sblk, sc_base, s_blocks);
      }
      const int rows_b = min(RW * 16, N - row0);
      const uint8_t* srow = reinterpret_cast<const uint8_t*>(sc_lds + j * sc_blk) + sc_base +
                            (size_t)min(row - row0, rows_b - 1) * KB;

      f32x4_v acc[4];
#pragma unroll
      for (int d = 0; d < 4; d++) acc[d] = f32x4_v{0.f, 0.f, 0.f, 0.f};

      // ---- NST chunks of NCH K groups in flight: a chunk is converted and
      // multiplied while the later ones load (4 MFMAs per 128-bit load into four
      // independent accumulators; A = token rows, lane l: row l % 16; B = weights)
      // At 3 waves per SIMD the next group's token rows are not prefetched from
      // LDS (the registers are needed for the weights in flight; the other waves
      // cover the LDS latency).
      constexpr bool kXPrefetch = OCC < 3;
      auto compute_chunk = [&](int c0, const uint4 (&wl)[NCH]) {
        uint32_t sv[NCH];
#pragma unroll
        for (int i = 0; i < NCH; i++) sv[i] = srow[min((c0 + i) * 4 + kq, KB - 1)];
        uint4 xv[4], xn[4];
#pragma unroll
        for (int d = 0; d < 4; d++) xv[d] = xread(c0 * 16 + d);
#pragma unroll
        for (int i = 0; i < NCH; i++) {
          if (kXPrefetch && i + 1 < NCH) {
#pragma unroll
            for (int d = 0; d < 4; d++) xn[d] = xread((c0 + i + 1) * 16 + d);
          }
          if (!kXPrefetch && i > 0) {
#pragma unroll
            for (int d = 0; d < 4; d++) xv[d] = xread((c0 + i) * 16 + d);
          }
          // group i is blocks 4 (i % 2) .. 4 (i % 2) + 3 of square i / 2
          if constexpr (TR2) {
            if ((i & 1) == 0) {  // the whole square, before its first group
              *reinterpret_cast<uint4*>(tr_at(lane >> 3, lane & 7)) = wl[i];
              *reinterpret_cast<uint4*>(tr_at(8 + (lane >> 3), lane & 7)) = wl[i + 1];
            }
          } else if (((lane >> 2) & 1) == (i & 1)) {  // the lanes that loaded the group
            *reinterpret_cast<uint4*>(tr_at(lane >> 3, lane & 3)) = wl[i & ~1];
            *reinterpret_cast<uint4*>(tr_at(8 + (lane >> 3), lane & 3)) = wl[i | 1];
          }
          asm volatile("" ::: "memory");
          const uint4 w = *reinterpret_cast<const uint4*>(tr_at(lane & 15, TR2 ? 4 * (i & 1) + kq : kq));
          const float sf = e8m0_to_float(sv[i]);
          const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int d = 0; d < 4; d++) {
            const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 0);
            const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 1);
            const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 2);
            const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 3);
            const bf16x8_t bw = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv[d]), bw, acc[d], 0, 0, 0);
          }
          if (kXPrefetch && i + 1 < NCH) {
#pragma unroll
            for (int d = 0; d < 4; d++) xv[d] = xn[d];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // rounds of NST chunks: every round but the last requests the next round,
      // the last one the first round of the next block (the requests are
      // unconditional, so the compiler's wait counts stay exact: after the last
      // block they re-read its first chunks, which its own loads just brought in)
      const int rounds = NITC / (KS * NST * NCH);
      for (int rd = 0; rd + 1 < rounds; rd++) {
        const int c0 = g_first + rd * NST * NCH;
#pragma unroll
        for (int st = 0; st < NST; st++) {
          compute_chunk(c0 + st * NCH, wq[st]);
          load_chunk(wrow, c0 + (NST + st) * NCH, wq[st]);
        }
      }
      {
        const int c0 = g_first + (rounds - 1) * NST * NCH;
#pragma unroll
        for (int st = 0; st < NST; st++) {
          compute_chunk(c0 + st * NCH, wq[st]);
          load_chunk(wnext, nfirst + st * NCH * nstep, wq[st], nstep);
        }
      }
      asm volatile("" : "+v"(bias_bits));
      const float bias_v = row_ok ? bf16_bits_to_f32(bias_bits) : 0.f;
      f32x4_v tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      if (KS > 1) {  // K parts 1.. hand their sums to part 0 (fixed order: deterministic)
        if (kpart > 0) red[(rw * (KS - 1) + kpart - 1) * 64 + lane] = tot;
        lds_barrier();
        if (kpart == 0) {
#pragma unroll
          for (int q = 0; q < KS - 1; q++) tot += red[(rw * (KS - 1) + q) * 64 + lane];
        }
        lds_barrier();  // the partial sums are read before the next block writes them
      }

      // ---- lane l holds tokens 4 * (l / 16) + i of weight row l % 16
      if constexpr (SWIGLU) {
        // rows 2 i (gate) and 2 i + 1 (up) sit in lanes l and l ^ 1 (row0 is a
        // multiple of 16): swap within lane pairs (every lane takes part),
        // then the even lane writes activation column row / 2
        float v[4], pv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          v[i] = tot[i] + bias_v;
          pv[i] = pair_swap(v[i]);
        }
        if (row_ok && kpart == 0 && (row & 1) == 0) {
          const int NA = N >> 1;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int m = 4 * kq + i;
            if (m < mc) {
              const int r = rows_lds[m];
              if (r >= 0) act[(size_t)r * NA + (row >> 1)] = (uint16_t)f32_to_bf16_bits(swiglu(v[i], pv[i]));
            }
          }
        }
      } else if (row_ok && kpart == 0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int m = 4 * kq + i;
          if (m < mc) {
            const int r = rows_lds[m];
            if (r >= 0) out[(size_t)r * N + row] = tot[i] + bias_v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// single token: row-contiguous streaming with lane dot products
// ---------------------------------------------------------------------------
//
// With one token the MFMA above does one row of useful work, and its operand
// layout (16 rows x 64 bytes per load) streams HBM markedly slower than loads
// that cover longer runs of a row.  Here 16 lanes share a weight row: lane
// (row q, j) of a wave holds block 16 i + j of the row, so a load covers 4 rows
// x 256 contiguous bytes.  Each lane turns its block into 32 exact bf16
// weights (v_cvt_scalef32_pk_bf16_fp4 with the block's E8M0 factor) and takes
// v_dot2_f32_bf16 products with the token row (bf16 x bf16 is exact in fp32;
// fp32 sums); the 16 lanes of a row then add their sums with shuffles in a
// fixed order.  All of K's loads (K <= 3072) are in flight at once.

constexpr int kT1MaxKB = 96;                    // K <= 3072
constexpr int kT1Ins = kT1MaxKB / 16;           // loads per quad and lane

// QUADS groups of 4 weight rows per wave, WAVES waves per workgroup
template <int QUADS, int WAVES>
struct T1Shape {
  static constexpr int kRows = WAVES * 4 * QUADS;
  // the workgroup's scale bytes (kRows x K/32) plus alignment slack, in whole 64-block DMAs
  static constexpr int kScBlocks = ((kRows * kT1MaxKB + 31) / 16 + 63) / 64 * 64;
};

// Routing parameters of the fused single-token decode: the token's router
// logits in, the routing outputs (written by workgroup (0, 0)) out.
// One MXFP4 block's 32 products with 32 staged bf16 inputs, added to a: the
// block's four code words w (8 codes each) become exact bf16 weights through
// v_cvt_scalef32_pk_bf16_fp4 with the E8M0 factor sf, and v_dot2_f32_bf16
// multiplies them by the inputs x0 .. x3 (8 each) and sums in fp32, in element
// order.  keep = 0 zeroes the block (a block past K).
__device__ __forceinline__ float block_dot(const uint4 w, uint32_t keep, float sf, const uint4 x0, const uint4 x1,
                                           const uint4 x2, const uint4 x3, float a) {
  const uint32_t wd[4] = {w.x & keep, w.y & keep, w.z & keep, w.w & keep};
  const uint4 xv[4] = {x0, x1, x2, x3};
#pragma unroll
  for (int d = 0; d < 4; d++) {
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 0),
                                        __builtin_bit_cast(bf16x2_t, xv[d].x), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 1),
                                        __builtin_bit_cast(bf16x2_t, xv[d].y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 2),
                                        __builtin_bit_cast(bf16x2_t, xv[d].z), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[d], sf, 3),
                                        __builtin_bit_cast(bf16x2_t, xv[d].w), a, false);
  }
  return a;
}

// FUSED: the workgroup routes the token itself (E <= 64) instead of reading
// expert offsets: every lane e counts the experts whose logit beats its own
// (a larger logit, or an equal one at a lower index), the k with count < k
// are chosen, and workgroup row blockIdx.y takes the blockIdx.y-th chosen
// expert in index order; its slot is its count, its routed row the slot.
// The same arithmetic as the routing kernel, so the outputs are identical.
// The routing outputs of a fused one-row-per-workgroup decode of T tokens
// (T * k <= E <= 64), by the first workgroup: the tokens' logits staged in LDS
// by all its waves, then wave 0 routes them one at a time with the routing
// launch's arithmetic (lane e: expert e's rank; the gates over the same wave
// sum), writes ids and gates, counts the rows per expert, and places each row
// after the rows of its expert with a lower token (the grouping's order).
template <int WAVES>
__device__ __forceinline__ void multi_route_outputs(const FusedRoute& fr, int T, int E, int k, int lane, int wave) {
  __shared__ uint16_t lg[kFusedMaxT * kFusedMaxE];  // T rows of E logits (T * k <= E)
  __shared__ int8_t slot[kFusedMaxT * 64];        // token t, expert e: its slot, or -1
  for (int i = threadIdx.x; i < T * E; i += WAVES * 64) lg[i] = fr.logits[i];
  __syncthreads();
  if (wave != 0) return;
  int cnt = 0;  // lane e: rows of expert e
  bool nan_seen = false;
  for (int t = 0; t < T; t++) {
    const float l = lane < E ? bf16_bits_to_f32(lg[t * E + lane]) : -INFINITY;
    int rank = 0;
    for (int j = 0; j < E; j++) {
      const float lj = readlane_f(l, j);
      rank += (lj > l || (lj == l && j < lane)) ? 1 : 0;
    }
    const bool ok = __ballot(lane < E && l != l) == 0;
    const bool chosen = ok && lane < E && rank < k;
    if (ok) {
      const float mx = readlane_f(l, __ffsll((long long)__ballot(chosen && rank == 0)) - 1);
      const float num = chosen ? expf(l - mx) : 0.f;
      const float sum = wave_sum(num);
      if (chosen) {
        fr.topk_ids[(size_t)t * k + rank] = lane;
        if (fr.gates) fr.gates[(size_t)t * k + rank] = num / sum;
      }
    } else {
      nan_seen = true;
      if (lane < k) {
        fr.topk_ids[(size_t)t * k + lane] = -1;
        if (fr.gates) fr.gates[(size_t)t * k + lane] = 0.f;
      }
    }
    slot[t * 64 + lane] = (int8_t)(chosen ? rank : -1);
    cnt += chosen ? 1 : 0;
  }
  int inc = cnt;
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  const int total = __shfl(inc, 63, 64);
  if (lane < E) fr.offsets[lane] = inc - cnt;
  if (lane == 0) {
    fr.offsets[E] = total;
    if (fr.error_word) *fr.error_word = nan_seen ? MXFP4_ROUTE_ERR_ID_RANGE : 0;
  }
  int run = inc - cnt;
  for (int t = 0; t < T; t++) {
    const int s = slot[t * 64 + lane];
    if (s >= 0) fr.sorted_rows[run++] = t * k + s;
  }
}

template <int QUADS, int WAVES, bool FUSED, bool SWIGLU, bool MULTI = false>
__global__ __launch_bounds__(WAVES * 64) void expert_gemv_t1_kernel(
    const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ scales, const uint16_t* __restrict__ bias,
    int E, int N, int K, const uint16_t* __restrict__ x, int x_per_slot, int k,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows, float* __restrict__ out,
    uint16_t* __restrict__ act, FusedRoute fr, int T) {
  using Sh = T1Shape<QUADS, WAVES>;
  __shared__ uint4 xs1[kT1MaxKB * 4];        // the token row: 4 entries of 8 bf16 per block
  __shared__ uint4 sc1[Sh::kScBlocks];       // the workgroup's scale rows, from their aligned blocks
  const int KB = K >> 5;
  const int K8 = K >> 3;
  const int R = T * k;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int e, m0, m1;
  int fused_row = -1;
  if constexpr (FUSED) {
    // MULTI: workgroup row blockIdx.y serves token blockIdx.y / k and the
    // (blockIdx.y % k)-th of its experts in index order; else one token
    const int tok = MULTI ? (int)blockIdx.y / k : 0;
    const int jsel = (int)blockIdx.y - tok * k;
    const uint16_t* lrow = fr.logits + (size_t)tok * E;
    float l = -INFINITY;
    int rank = 0;
    if (E == 32) {
      // gpt-oss-20b's 32 experts: the logits as 16 words through the scalar
      // cache (one wave-uniform load; about 0.5 us sooner than a vector load
      // of the same 64 bytes by every wave); lane i < 16 takes word i and
      // each lane its expert's word from lane e / 2.  Every wave
      // of the launch (about 22 per CU) ranks the token at the same moment,
      // so the ranking is held to a few instructions: lane e's logit becomes
      // a unique integer key (the bf16 bits in an order-preserving form, -0
      // as +0, above 255 - e, so equal logits favour the lower index: the
      // order of the rank below), and k rounds of a wave maximum over the
      // keys (DPP within rows of 16, then the 4 row maxima) each take the
      // next expert.  The comparisons of 32 uniform logits with each lane's
      // took about 220 vector and 300 scalar instructions per wave.  Other
      // counts take the vector load below (a second specialised path made
      // the kernel larger and its start slower).
      const __attribute__((address_space(4))) uint32_t* lw =
          (const __attribute__((address_space(4))) uint32_t*)(uintptr_t)(lrow);
      uint32_t wv[16];
#pragma unroll
      for (int i = 0; i < 16; i++) wv[i] = lw[i];
      int words = 0;
#pragma unroll
      for (int i = 0; i < 16; i++) words = lane == i ? (int)wv[i] : words;
      const uint32_t wsel = (uint32_t)__builtin_amdgcn_ds_bpermute((lane >> 1) << 2, words);
      const uint32_t b = (lane & 1) ? (wsel >> 16) : (wsel & 0xffffu);
      l = lane < 32 ? __uint_as_float(b << 16) : -INFINITY;
      const uint32_t bz = b == 0x8000u ? 0u : b;
      const uint32_t ord = (bz & 0x8000u) ? (~bz & 0xffffu) : (bz | 0x8000u);
      uint32_t key = lane < 32 ? (ord << 8) | (uint32_t)(255 - lane) : 0u;
      rank = 64;  // not chosen
      for (int r = 0; r < k; r++) {
        uint32_t v = key;
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
        v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
        const uint32_t m = max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
                               max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
        if (lane == 255 - (int)(m & 0xffu)) {
          rank = r;
          key = 0u;
        }
      }
    } else {
      l = lane < E ? bf16_bits_to_f32(lrow[lane]) : -INFINITY;
      for (int jj = 0; jj < E; jj++) {
        const float lj = readlane_f(l, jj);
        rank += (lj > l || (lj == l && jj < lane)) ? 1 : 0;
      }
    }
    // Logits without NaN rank the lanes 0 .. E - 1, each rank once.  A NaN
    // compares false both ways and breaks that: then, as in the routing
    // kernel, every slot gets id -1 and gate 0, and no row is grouped or
    // projected.
    const bool ok = __ballot(lane < E && l != l) == 0;
    const bool chosen = ok && lane < E && rank < k;
    const uint64_t mask = __ballot(chosen);
    if (MULTI && blockIdx.x == 0 && blockIdx.y == 0) {
      multi_route_outputs<WAVES>(fr, T, E, k, lane, (int)(threadIdx.x >> 6));
    } else if (!MULTI && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) {
      // the routing outputs: ids and gates by slot, offsets, grouped rows
      if (ok) {
        const float mx = readlane_f(l, __ffsll((long long)__ballot(chosen && rank == 0)) - 1);
        const float num = chosen ? expf(l - mx) : 0.f;
        const float sum = wave_sum(num);
        if (chosen) {
          fr.topk_ids[rank] = lane;
          if (fr.gates) fr.gates[rank] = num / sum;
          fr.sorted_rows[lanes_below(mask)] = rank;
        }
      } else if (lane < k) {
        fr.topk_ids[lane] = -1;
        if (fr.gates) fr.gates[lane] = 0.f;
      }
      if (lane < E) fr.offsets[lane] = __popcll(mask & ((1ull << lane) - 1));
      if (lane == 0) {
        fr.offsets[E] = __popcll(mask);
        if (fr.error_word) *fr.error_word = ok ? 0 : MXFP4_ROUTE_ERR_ID_RANGE;
      }
    }
    const uint64_t mine = __ballot(chosen && lanes_below(mask) == jsel);
    if (mine == 0) return;
    e = __builtin_amdgcn_readfirstlane(__ffsll((long long)mine) - 1);
    fused_row = tok * k + __builtin_amdgcn_readlane(rank, e);
    m0 = 0;
    m1 = 1;
  } else {
    if (!find_group(offsets, E, R, blockIdx.y, lane, e, m0, m1)) return;
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    m1 = __builtin_amdgcn_readfirstlane(m1);
  }
  // Never taken (K >= 32): arrays written only by LDS DMA look unwritten to the
  // optimizer, which would then fold their loads away.
  if (K < 0) { xs1[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u); sc1[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u); }

  const int wg_row0 = blockIdx.x * Sh::kRows;
  const int rows_wg = min(Sh::kRows, N - wg_row0);
  const int j = lane & 15;            // block lane within a row
  const int q4 = lane >> 4;           // row within a quad
  int rowq[QUADS];
  const uint4* wrow[QUADS];
#pragma unroll
  for (int q = 0; q < QUADS; q++) {
    rowq[q] = wg_row0 + (wave * QUADS + q) * 4 + q4;
    wrow[q] = reinterpret_cast<const uint4*>(blocks) + ((size_t)e * N + min(rowq[q], N - 1)) * KB;
  }
  // scale rows wg_row0 .. wg_row0 + rows_wg - 1, contiguous: the aligned 16-byte
  // blocks from the one holding the first byte to the one holding the last (an
  // aligned block that holds a valid byte never leaves that byte's page)
  const uintptr_t sbase = reinterpret_cast<uintptr_t>(scales);
  const uintptr_t s_first = sbase + ((size_t)e * N + wg_row0) * KB;
  const uintptr_t s_blk0 = s_first & ~(uintptr_t)15;
  const uintptr_t s_blk1 = (s_first + (size_t)rows_wg * KB - 1) & ~(uintptr_t)15;
  const int n_sblk = (int)((s_blk1 - s_blk0) >> 4) + 1;
  const int sc_base = (int)(s_first - s_blk0);
  const uint4* s_blocks = reinterpret_cast<const uint4*>(scales - (sbase - s_blk0));

  // the bias values, loaded ahead of the weights (they land with the staged
  // rows, which every wave waits for anyway), so that the end of the row waits
  // on no memory round trip.  Unconditional loads (from a zero when there is
  // no bias: a load under a branch ends in a wait for every load in flight)
  // through an opaque address (a load through the restrict pointer counts as
  // invariant and would be sunk to its use, behind the arithmetic).
  uint32_t bias_bits[QUADS];
#pragma unroll
  for (int q = 0; q < QUADS; q++) {
    const uint16_t* bp = bias ? bias + (size_t)e * N + min(rowq[q], N - 1) : &kZeroBf16;
    asm volatile("" : "+v"(bp));
    bias_bits[q] = *(const __attribute__((address_space(1))) uint16_t*)(bp);
  }

  for (int mb = m0; mb < m1; mb++) {  // one routed row per expert unless given ids repeat
    // With one shared token row the output row is not needed until the store:
    // its load then waits behind the weight loads instead of in front of them.
    int src = 0;
    if (FUSED) {
      src = x_per_slot ? fused_row : fused_row / k;
    } else if (x_per_slot || T > 1) {
      const int r_raw = sorted_rows[mb];
      src = (r_raw < 0 || r_raw >= R) ? 0 : (x_per_slot ? r_raw : r_raw / k);
    }
    if (mb > m0) bare_barrier<63>();  // the previous row is done with the staged token row
    // ---- LDS DMAs (scale blocks, then the token row), spread over the waves;
    // they are older than every weight load, which is all the wait below needs
    {
      const int n_si = (n_sblk + 63) >> 6;
      for (int ins = wave; ins < n_si; ins += WAVES)
        dma16(s_blocks + min(ins * 64 + lane, n_sblk - 1), reinterpret_cast<uint8_t*>(sc1 + ins * 64));
      const int n_xi = (K8 + 63) >> 6;
      const uint4* xrow = reinterpret_cast<const uint4*>(x + (size_t)src * K);
      for (int ins = wave; ins < n_xi; ins += WAVES)
        dma16(xrow + min(ins * 64 + lane, K8 - 1), reinterpret_cast<uint8_t*>(xs1 + ins * 64));
    }
    asm volatile("" ::: "memory");  // the weight loads stay behind the DMAs
    // ---- all of the wave's weights: QUADS x kT1Ins loads, blocks past K
    // re-read the row's last block (zeroed below)
    uint4 w[QUADS][kT1Ins];
#pragma unroll
    for (int q = 0; q < QUADS; q++)
#pragma unroll
      for (int i = 0; i < kT1Ins; i++) w[q][i] = load_nt(wrow[q] + min(16 * i + j, KB - 1));
    asm volatile("" ::: "memory");
    const int r_raw = FUSED ? fused_row : sorted_rows[mb];
    const int r = (r_raw < 0 || r_raw >= R) ? -1 : r_raw;
    bare_barrier<QUADS * kT1Ins>();  // every wave's DMAs have landed
    const uint8_t* scb = reinterpret_cast<const uint8_t*>(sc1) + sc_base;
    float acc[QUADS];
#pragma unroll
    for (int q = 0; q < QUADS; q++) acc[q] = 0.f;
#pragma unroll
    for (int i = 0; i < kT1Ins; i++) {
      const int b = 16 * i + j;
      const int bc = min(b, KB - 1);
      const uint32_t keep = b < KB ? 0xffffffffu : 0u;
      const uint4 x0 = xs1[bc * 4 + 0], x1 = xs1[bc * 4 + 1], x2 = xs1[bc * 4 + 2], x3 = xs1[bc * 4 + 3];
#pragma unroll
      for (int q = 0; q < QUADS; q++) {
        const int rl = (wave * QUADS + q) * 4 + q4;
        const float sf = e8m0_to_float(scb[min(rl, rows_wg - 1) * KB + bc]);
        acc[q] = block_dot(w[q][i], keep, sf, x0, x1, x2, x3, acc[q]);
      }
    }
    // ---- the 16 lanes of a row add their sums (fixed order: deterministic)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
#pragma unroll
      for (int q = 0; q < QUADS; q++) acc[q] += __shfl_xor(acc[q], o, 64);
    if constexpr (SWIGLU) {
      // rows 4 m + (0, 1) and 4 m + (2, 3) are (gate, up) pairs: row q4 ^ 1
      // sits 16 lanes away; lanes of even rows write activation column row / 2
#pragma unroll
      for (int q = 0; q < QUADS; q++) {
        uint32_t bb = bias_bits[q];
        asm volatile("" : "+v"(bb));
        const float v = acc[q] + bf16_bits_to_f32(bb);
        const float pv = __shfl_xor(v, 16, 64);
        if (j == 0 && (q4 & 1) == 0 && r >= 0 && rowq[q] < N)
          act[(size_t)r * (N >> 1) + (rowq[q] >> 1)] = (uint16_t)f32_to_bf16_bits(swiglu(v, pv));
      }
    } else if (j == 0 && r >= 0) {
#pragma unroll
      for (int q = 0; q < QUADS; q++)
        if (rowq[q] < N) {
          // consumed here, not hoisted (with its wait) in front of the loop
          uint32_t bb = bias_bits[q];
          asm volatile("" : "+v"(bb));
          out[(size_t)r * N + rowq[q]] = acc[q] + bf16_bits_to_f32(bb);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// a token's projection of every slot and the gate-weighted combine
// ---------------------------------------------------------------------------
//
// y[t, n] = sum over token t's slots s of gates[t, s] * (bias[e_s, n] + sum_j
// W[e_s, n, j] * x_s[j]) (src/experts.linnet fn forward_topk: each slot's down
// product and the f32 sum over k; fn down_bias_of: the down bias weighed by the
// router).  A workgroup owns 4 * WPS weight rows of token blockIdx.y and runs
// kT1Group slots of the token over them at a time, WPS waves per slot, so the
// combine needs no other workgroup's results (an expert two tokens chose is
// streamed once per token: for batches with no more routed rows than
// experts).  Each slot's value is the row-streaming kernel's (the same lane
// split, products, fixed lane sum and bias added last); the values
// meet in LDS and the first slot's waves sum them in slot order with one fused
// multiply-add each, as moe_combine does: y equals mxfp4_expert_proj followed
// by moe_combine bit for bit.
constexpr int kT1Group = 4;  // slots per round, WPS waves each

template <int WPS>
__global__ __launch_bounds__(WPS * kT1Group * 64) void expert_gemv_combine_t1_kernel(
    const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ scales, const uint16_t* __restrict__ bias,
    int E, int N, int K, const uint16_t* __restrict__ x, int x_per_slot, int k,
    const int32_t* __restrict__ topk_ids, const float* __restrict__ gates, float* __restrict__ out,
    float* __restrict__ y) {
  // this workgroup's token: its slots, input rows, out rows and y row
  const int tok = blockIdx.y;
  topk_ids += (size_t)tok * k;
  gates += (size_t)tok * k;
  x += (size_t)tok * (x_per_slot ? k : 1) * K;
  if (out) out += (size_t)tok * k * N;
  y += (size_t)tok * N;
  using Sh = T1Shape<1, WPS>;
  constexpr int kRows = Sh::kRows;
  __shared__ uint4 xs1[kT1Group][kT1MaxKB * 4];   // the slots' input rows: 4 entries of 8 bf16 per block
  __shared__ uint4 sc1[kT1Group][Sh::kScBlocks];   // each slot's expert's scale rows, from their aligned blocks
  __shared__ float vals[kT1Group][kRows];          // each slot's projection of the workgroup's rows
  const int KB = K >> 5;
  const int K8 = K >> 3;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = wave / WPS;     // this wave's slot in the round
  const int wq = wave % WPS;    // and its 4 rows among the slot's
  const int j = lane & 15;      // block lane within a row
  const int q4 = lane >> 4;     // row within the wave's 4
  const int wg_row0 = blockIdx.x * kRows;
  const int rows_wg = min(kRows, N - wg_row0);
  const int rl = wq * 4 + q4;   // row within the workgroup
  const int row = wg_row0 + rl;
  // Never taken (K >= 32): arrays written only by LDS DMA look unwritten to the
  // optimizer, which would then fold their loads away.
  if (K < 0) {
    xs1[0][threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    sc1[0][threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  }
  const uintptr_t sbase = reinterpret_cast<uintptr_t>(scales);
  float yacc = 0.f;  // the first slot's waves: the combine of their rows
  for (int s0 = 0; s0 < k; s0 += kT1Group) {
    const int ng = min(kT1Group, k - s0);
    const bool active = g < ng;  // uniform
    const int s = min(s0 + g, k - 1);
    const int e_raw = topk_ids[s];
    const bool ok = active && e_raw >= 0 && e_raw < E;  // a slot without a valid expert contributes nothing
    const int e = ok ? e_raw : 0;
    // the bias value first (see the row-streaming kernel: unconditional, through an opaque address)
    uint32_t bias_bits;
    {
      const uint16_t* bp = bias ? bias + (size_t)e * N + min(row, N - 1) : &kZeroBf16;
      asm volatile("" : "+v"(bp));
      bias_bits = *(const __attribute__((address_space(1))) uint16_t*)(bp);
    }
    if (s0 > 0) bare_barrier<63>();  // the previous round is done with the staged rows and values
    // ---- LDS DMAs of this wave's slot: the expert's scale blocks and the
    // slot's input row (one shared row without x_per_slot, staged by slot 0's
    // waves), spread over the slot's waves; older than every weight load
    const uintptr_t s_first = sbase + ((size_t)e * N + wg_row0) * KB;
    const uintptr_t s_blk0 = s_first & ~(uintptr_t)15;
    const uintptr_t s_blk1 = (s_first + (size_t)rows_wg * KB - 1) & ~(uintptr_t)15;
    const int n_sblk = (int)((s_blk1 - s_blk0) >> 4) + 1;
    const int sc_base = (int)(s_first - s_blk0);
    if (active) {
      const uint4* s_blocks = reinterpret_cast<const uint4*>(scales - (sbase - s_blk0));
      const int n_si = (n_sblk + 63) >> 6;
      for (int ins = wq; ins < n_si; ins += WPS)
        dma16(s_blocks + min(ins * 64 + lane, n_sblk - 1), reinterpret_cast<uint8_t*>(&sc1[g][ins * 64]));
      if (x_per_slot || g == 0) {
        const uint4* xrow = reinterpret_cast<const uint4*>(x + (size_t)(x_per_slot ? s : 0) * K);
        const int n_xi = (K8 + 63) >> 6;
        for (int ins = wq; ins < n_xi; ins += WPS)
          dma16(xrow + min(ins * 64 + lane, K8 - 1), reinterpret_cast<uint8_t*>(&xs1[g][ins * 64]));
      }
    }
    asm volatile("" ::: "memory");  // the weight loads stay behind the DMAs
    // ---- all of this lane's weights of the slot: kT1Ins loads (blocks past K
    // re-read the row's last block, zeroed below)
    uint4 w[kT1Ins];
    const uint4* wrow = reinterpret_cast<const uint4*>(blocks) + ((size_t)e * N + min(row, N - 1)) * KB;
#pragma unroll
    for (int i = 0; i < kT1Ins; i++) w[i] = load_nt(wrow + min(16 * i + j, KB - 1));
    asm volatile("" ::: "memory");
    bare_barrier<kT1Ins>();  // every wave's DMAs have landed
    {
      // every wave multiplies, so that its loads are used where they were
      // issued (a load used only under a branch is sunk into it, behind the
      // barrier); a wave without a slot discards its result
      const uint4* xg = xs1[x_per_slot ? g : 0];
      const uint8_t* scb = reinterpret_cast<const uint8_t*>(sc1[g]) + sc_base;
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < kT1Ins; i++) {
        const int b = 16 * i + j;
        const int bc = min(b, KB - 1);
        const uint32_t keep = b < KB ? 0xffffffffu : 0u;
        const uint4 x0 = xg[bc * 4 + 0], x1 = xg[bc * 4 + 1], x2 = xg[bc * 4 + 2], x3 = xg[bc * 4 + 3];
        const float sf = e8m0_to_float(scb[min(rl, rows_wg - 1) * KB + bc]);
        a = block_dot(w[i], keep, sf, x0, x1, x2, x3, a);
      }
      // the 16 lanes of a row add their sums (fixed order), then the bias
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) a += __shfl_xor(a, o, 64);
      uint32_t bb = bias_bits;
      asm volatile("" : "+v"(bb));
      const float v = a + bf16_bits_to_f32(bb);
      if (j == 0 && active) {
        vals[g][rl] = v;
        if (ok && out && row < N) out[(size_t)s * N + row] = v;
      }
    }
    lds_barrier();  // every slot's values are in LDS
    if (g == 0) {
      for (int h = 0; h < ng; h++) {  // slot order
        const int sh = s0 + h;
        const int eh = topk_ids[sh];
        if (eh >= 0 && eh < E && gates[sh] != 0.f) yacc = fmaf(gates[sh], vals[h][rl], yacc);
      }
    }
  }
  if (g == 0 && j == 0 && row < N) y[row] = yacc;
}

#ifndef MXFP4_T1_QUADS
#define MXFP4_T1_QUADS 1
#endif
#ifndef MXFP4_T1_WAVES
#define MXFP4_T1_WAVES 4
#endif
constexpr int kT1Quads = MXFP4_T1_QUADS;
constexpr int kT1Waves = MXFP4_T1_WAVES;
constexpr int kT1Rows = T1Shape<kT1Quads, kT1Waves>::kRows;

// The one-token kernel's streaming (a workgroup row per expert, or per routed
// row when it routes) while the routed rows number no more than the experts:
// few experts then hold two rows, and the multi-token kernel's 16-row MFMA
// tiles would run mostly empty (at the gpt-oss decode shapes, 2 to 4 tokens:
// 21-33 against 30-42 us).  K <= 3072: all of a row's loads in flight at once.
inline bool gemv_one_row(int T, int k, int E, int K) { return (long long)T * k <= E && K / 32 <= kT1MaxKB; }

// largest dynamic LDS a launch may use (the rest of the 160 KB holds rows_lds)
constexpr int kGemvMaxDynLds = 160 * 1024 - 1024;

// LDS of one workgroup, in 16-byte entries: the MT staged token rows, and the
// weight-scale rows of one row block of 16 * WAVES / KS weight rows (+2
// blocks of alignment slack, in whole 64-entry DMAs).
size_t gemv_xs_entries(int MT, int NCH, int NST, int KS, int K) {
  const int nit = (K / 32 + 3) / 4;
  const int r = KS * NST * NCH;
  return (size_t)MT * (((nit + r - 1) / r * r * 16 + 63) / 64 * 64 + 1);
}
size_t gemv_sc_entries(int WAVES, int KS, int K) {
  const size_t blocks = ((size_t)(WAVES / KS) * 16 * (K / 32) + 15) / 16 + 2;
  return (blocks + 63) / 64 * 64;
}
// LDS of one workgroup, in 16-byte entries: the staged token rows, each
// wave's transpose region (2 KB with tr2, else 1 KB), then the weight-scale
// rows of each of its nbpw row blocks.
size_t gemv_lds_for(int MT, int WAVES, int NCH, int NST, int KS, int K, int nbpw, bool tr2 = false) {
  return (gemv_xs_entries(MT, NCH, NST, KS, K) + (size_t)WAVES * (tr2 ? 128 : 64) +
          (size_t)nbpw * gemv_sc_entries(WAVES, KS, K)) * 16;
}

template <int MT, int WAVES, int NCH, int NST, int KS, int OCC, bool SWIGLU, bool FR, bool TR2>
hipError_t launch_gemv_tr(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N, int K,
                          const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                          const int32_t* sorted_rows, float* out, uint16_t* act, hipStream_t stream,
                          const FusedRoute& fr) {
  // Row blocks per workgroup: enough workgroups for one wave of them over the
  // 256 CUs (as many per CU as the waves allow), each streaming its share of
  // an expert's row blocks with the token rows staged once, within the LDS.
  const int R = T * k;
  const int groups = R < E ? R : E;
  constexpr int RW = WAVES / KS;
  const int nblk = (N + RW * 16 - 1) / (RW * 16);
  const size_t xs = gemv_xs_entries(MT, NCH, NST, KS, K) + (size_t)WAVES * (TR2 ? 128 : 64),
               sc = gemv_sc_entries(WAVES, KS, K);
  const int nbpw_max = (int)((kGemvMaxDynLds / 16 - xs) / sc);  // >= 1: checked by the caller
  constexpr int kPerCu = (OCC * 4) / WAVES > 0 ? (OCC * 4) / WAVES : 1;
  int G = (256 * kPerCu + groups - 1) / groups;
  G = G < (nblk + nbpw_max - 1) / nbpw_max ? (nblk + nbpw_max - 1) / nbpw_max : G;
  G = G > nblk ? nblk : G;
  const int nbpw = (nblk + G - 1) / G;
  size_t lds = gemv_lds_for(MT, WAVES, NCH, NST, KS, K, nbpw, TR2);
  // fused routing: the staged logits, T x (E + 1) floats, and the routing
  // writer's WAVES x 64 + 1 counters
  if (FR && lds < ((size_t)T * (E + 1) + WAVES * 64 + 1) * 4) lds = ((size_t)T * (E + 1) + WAVES * 64 + 1) * 4;
  // above 64 KB the dynamic LDS limit is raised (to what any K may need)
  static DynLdsLimit gemv_lds(
      reinterpret_cast<const void*>(&expert_gemv_kernel<MT, WAVES, NCH, NST, KS, OCC, SWIGLU, FR, TR2>),
      kGemvMaxDynLds);
  if (lds > 65536) {
    const hipError_t err = gemv_lds.ensure();
    if (err != hipSuccess) return err;
  }
  // fused routing: one row of workgroups per expert by index (those of
  // unused experts write its offset and exit)
  const dim3 grid(G, FR ? E : groups);
  hipLaunchKernelGGL((expert_gemv_kernel<MT, WAVES, NCH, NST, KS, OCC, SWIGLU, FR, TR2>), grid, dim3(WAVES * 64), lds,
                     stream, blocks, scales, bias, E, N, K, x, x_per_slot, T, k, offsets, sorted_rows, out, act, (int)sc,
                     fr);
  return hipGetLastError();
}

// The 2 KB transpose regions where one row block's LDS fits with them (every
// K the gpt-oss widths use), else the 1 KB ones.
template <int MT, int WAVES, int NCH, int NST, int KS, int OCC, bool SWIGLU, bool FR = false>
hipError_t launch_gemv_shape(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N, int K,
                             const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                             const int32_t* sorted_rows, float* out, uint16_t* act, hipStream_t stream,
                             const FusedRoute& fr = FusedRoute{}) {
  if (gemv_lds_for(MT, WAVES, NCH, NST, KS, K, 1, true) <= kGemvMaxDynLds)
    return launch_gemv_tr<MT, WAVES, NCH, NST, KS, OCC, SWIGLU, FR, true>(blocks, scales, bias, E, N, K, x, x_per_slot,
                                                                         T, k, offsets, sorted_rows, out, act, stream,
                                                                         fr);
  return launch_gemv_tr<MT, WAVES, NCH, NST, KS, OCC, SWIGLU, FR, false>(blocks, scales, bias, E, N, K, x, x_per_slot, T,
                                                                        k, offsets, sorted_rows, out, act, stream, fr);
}

// Chunk length NCH (K groups of 128 elements) for a ring of NST chunks per K
// part: the candidate that pads K's groups to whole rounds least (ties: the
// longer chunk).
int gemv_pick_chunk(int ks, int nst, int K, const int* cand, int ncand) {
  const int nit = (K / 32 + 3) / 4;
  int best = cand[0], best_pad = 1 << 30;
  for (int i = 0; i < ncand; i++) {
    const int r = ks * nst * cand[i];
    const int pad = (nit + r - 1) / r * r - nit;
    if (pad < best_pad || (pad == best_pad && cand[i] > best)) best = cand[i], best_pad = pad;
  }
  return best;
}

// Launch shape by batch size.  One token: workgroups of 2 waves that share 16
// weight rows and split K (so that all of a row group's weights are requested
// at once without exceeding the registers of 3 waves per SIMD); the many small
// workgroups spread evenly over the CUs.  Larger batches: wider workgroups
// share the staged token rows.  Chunk lengths are those that fit the registers
// without spilling.
struct GemvShape {
  int mt, waves, nch, nst, ks;
};
GemvShape gemv_shape(int T, int K) {
  static const int c1[] = {4}, c4[] = {4}, c16[] = {4, 6, 8};
  if (T <= 1) return {1, 2, gemv_pick_chunk(2, 3, K, c1, 1), 3, 2};
  if (T <= 4) return {4, 4, gemv_pick_chunk(1, 3, K, c4, 1), 3, 1};
  return {16, 8, gemv_pick_chunk(1, 2, K, c16, 3), 2, 1};
}

template <bool SWIGLU>
hipError_t launch_gemv_any(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N, int K,
                           const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                           const int32_t* sorted_rows, float* out, uint16_t* act, hipStream_t stream) {
  if (gemv_one_row(T, k, E, K)) {
    const dim3 grid((N + kT1Rows - 1) / kT1Rows, T * k < E ? T * k : E);
    hipLaunchKernelGGL((expert_gemv_t1_kernel<kT1Quads, kT1Waves, false, SWIGLU>), grid, dim3(kT1Waves * 64), 0,
                       stream, blocks, scales, bias, E, N, K, x, x_per_slot, k, offsets, sorted_rows, out, act,
                       FusedRoute{}, T);
    return hipGetLastError();
  }
#define MXFP4_GEMV_LAUNCH(MT, W, NCH, NST, KS, OCC)                                                               \
  return launch_gemv_shape<MT, W, NCH, NST, KS, OCC, SWIGLU>(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, \
                                                             offsets, sorted_rows, out, act, stream)
  const GemvShape g = gemv_shape(T, K);
  if (g.mt == 1) MXFP4_GEMV_LAUNCH(1, 2, 4, 3, 2, 2);
  if (g.mt == 4) MXFP4_GEMV_LAUNCH(4, 4, 4, 3, 1, 2);
  if (g.nch == 4) MXFP4_GEMV_LAUNCH(16, 8, 4, 2, 1, 2);
  if (g.nch == 6) MXFP4_GEMV_LAUNCH(16, 8, 6, 2, 1, 2);
  MXFP4_GEMV_LAUNCH(16, 8, 8, 2, 1, 2);
#undef MXFP4_GEMV_LAUNCH
}

// T = 2 .. 64 tokens routed by the projection launch itself (FusedRoute): the
// shapes of launch_gemv_any.
template <bool SWIGLU>
hipError_t launch_gemv_fused(const FusedRoute& fr, const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias,
                             int E, int N, int K, const uint16_t* x, int x_per_slot, int T, int k, float* out,
                             uint16_t* act, hipStream_t stream) {
#define MXFP4_GEMV_FUSED(MT, W, NCH, NST, KS, OCC)                                                                  \
  return launch_gemv_shape<MT, W, NCH, NST, KS, OCC, SWIGLU, true>(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, \
                                                                   nullptr, nullptr, out, act, stream, fr)
  const GemvShape g = gemv_shape(T, K);
  if (g.mt == 4) MXFP4_GEMV_FUSED(4, 4, 4, 3, 1, 2);
  if (g.nch == 4) MXFP4_GEMV_FUSED(16, 8, 4, 2, 1, 2);
  if (g.nch == 6) MXFP4_GEMV_FUSED(16, 8, 6, 2, 1, 2);
  MXFP4_GEMV_FUSED(16, 8, 8, 2, 1, 2);
#undef MXFP4_GEMV_FUSED
}

}  // namespace

size_t gemv_lds_bytes(int T, int K) {
  if (T == 1 && K / 32 <= kT1MaxKB) return 0;  // static LDS only (more tokens: the larger of the two shapes)
  const GemvShape g = gemv_shape(T, K);
  return gemv_lds_for(g.mt, g.waves, g.nch, g.nst, g.ks, K, 1);
}

hipError_t launch_expert_gemv(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N, int K,
                              const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                              const int32_t* sorted_rows, float* out, uint16_t* act, hipStream_t stream) {
  if (act)
    return launch_gemv_any<true>(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, offsets, sorted_rows, nullptr,
                                 act, stream);
  return launch_gemv_any<false>(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, offsets, sorted_rows, out,
                                nullptr, stream);
}

// T tokens: every slot's projection and the gate-weighted combine in one launch.
hipError_t launch_proj_combine_t1(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                                  int K, const uint16_t* x, int x_per_slot, int k, const int32_t* topk_ids,
                                  const float* gates, float* out, float* y, hipStream_t stream, int T) {
  // 4 rows per workgroup, one wave per slot: 720 workgroups per token at N =
  // 2880 (at the gpt-oss down decode of one token 7.1 us, against 7.8 us with
  // two waves per slot and 9.0 us with four; the token rows are staged more
  // often, but more, smaller workgroups start sooner)
  constexpr int kWps = 1;
  constexpr int kRows = T1Shape<1, kWps>::kRows;
  hipLaunchKernelGGL(expert_gemv_combine_t1_kernel<kWps>, dim3((N + kRows - 1) / kRows, T),
                     dim3(kWps * kT1Group * 64), 0, stream, blocks, scales, bias, E, N, K, x, x_per_slot, k, topk_ids,
                     gates, out, y);
  return hipGetLastError();
}

// The projection of the routed rows and the gate-weighted combine on the GEMV
// path: one launch while the routed rows number no more than the experts (a
// workgroup per token and 4 weight rows; measured at the gpt-oss down decode
// against the projection and then the combine: 1 token 7.1 against 9.3 us, 2
// tokens 11.0 against 12.6, 4 tokens 17.6 against 20.5, 6 tokens 24.7 against
// 26.3, 8 tokens 31.3 against 31.2), else the projection and then the combine.
hipError_t launch_expert_gemv_combine(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E,
                                      int N, int K, const uint16_t* x, int x_per_slot, int T, int k,
                                      const int32_t* offsets, const int32_t* sorted_rows, const int32_t* topk_ids,
                                      const float* gates, float* out, float* y, hipStream_t stream) {
  if (gemv_one_row(T, k, E, K))
    return launch_proj_combine_t1(blocks, scales, bias, E, N, K, x, x_per_slot, k, topk_ids, gates, out, y, stream, T);
  hipError_t e = launch_expert_gemv(blocks, scales, bias, E, N, K, x, x_per_slot, T, k, offsets, sorted_rows, out,
                                    nullptr, stream);
  if (e != hipSuccess) return e;
  return launch_combine(out, gates, T, k, N, y, stream, topk_ids, E);
}

// One token: routing, grouping and the projection in one launch (act != NULL:
// through the gated activation, bf16 [k, N / 2], instead of out).
hipError_t launch_moe_decode_t1(const uint16_t* logits, int E, int k, const uint8_t* blocks, const uint8_t* scales,
                                const uint16_t* bias, int N, int K, const uint16_t* x, int x_per_slot,
                                int32_t* topk_ids, float* gates, int32_t* offsets, int32_t* sorted_rows,
                                int32_t* error_word, float* out, uint16_t* act, hipStream_t stream) {
  const dim3 grid((N + kT1Rows - 1) / kT1Rows, k);
  const FusedRoute fr{logits, topk_ids, gates, offsets, sorted_rows, error_word};
  if (act) {
    hipLaunchKernelGGL((expert_gemv_t1_kernel<kT1Quads, kT1Waves, true, true>), grid, dim3(kT1Waves * 64), 0, stream,
                       blocks, scales, bias, E, N, K, x, x_per_slot, k, nullptr, nullptr, nullptr, act, fr, 1);
  } else {
    hipLaunchKernelGGL((expert_gemv_t1_kernel<kT1Quads, kT1Waves, true, false>), grid, dim3(kT1Waves * 64), 0, stream,
                       blocks, scales, bias, E, N, K, x, x_per_slot, k, nullptr, nullptr, out, nullptr, fr, 1);
  }
  return hipGetLastError();
}

}  // namespace mxfp4

namespace mxfp4 {

// T <= 64 decode tokens: routing, grouping and the projection in one launch
// (act != NULL: through the gated activation instead of out).
hipError_t launch_moe_decode_batch(const uint16_t* logits, int T, int E, int k, const uint8_t* blocks,
                                   const uint8_t* scales, const uint16_t* bias, int N, int K, const uint16_t* x,
                                   int x_per_slot, int32_t* topk_ids, float* gates, int32_t* offsets,
                                   int32_t* sorted_rows, int32_t* error_word, float* out, uint16_t* act,
                                   hipStream_t stream) {
  if (T == 1)
    return launch_moe_decode_t1(logits, E, k, blocks, scales, bias, N, K, x, x_per_slot, topk_ids, gates, offsets,
                                sorted_rows, error_word, out, act, stream);
  const FusedRoute fr{logits, topk_ids, gates, offsets, sorted_rows, error_word};
  if (gemv_one_row(T, k, E, K)) {
    // as expert_proj's GEMV for so few rows: one routed row per workgroup row
    const dim3 grid((N + kT1Rows - 1) / kT1Rows, T * k);
    if (act)
      hipLaunchKernelGGL((expert_gemv_t1_kernel<kT1Quads, kT1Waves, true, true, true>), grid, dim3(kT1Waves * 64), 0,
                         stream, blocks, scales, bias, E, N, K, x, 0, k, nullptr, nullptr, nullptr, act, fr, T);
    else
      hipLaunchKernelGGL((expert_gemv_t1_kernel<kT1Quads, kT1Waves, true, false, true>), grid, dim3(kT1Waves * 64), 0,
                         stream, blocks, scales, bias, E, N, K, x, x_per_slot, k, nullptr, nullptr, out, nullptr, fr, T);
    return hipGetLastError();
  }
  if (act) return launch_gemv_fused<true>(fr, blocks, scales, bias, E, N, K, x, x_per_slot, T, k, nullptr, act, stream);
  return launch_gemv_fused<false>(fr, blocks, scales, bias, E, N, K, x, x_per_slot, T, k, out, nullptr, stream);
}

}  // namespace mxfp4

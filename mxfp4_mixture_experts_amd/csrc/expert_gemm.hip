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
//    the checkpoint stores them: a lane of the A operand holds one 16-byte
//    MXFP4 block (32 E2M1 codes, low nibble first) of one weight row, and its
//    E8M0 byte is that lane's A scale.  No dequantization anywhere.  The
//    activations are the B operand, so the accumulators hold the transposed
//    product: a lane ends with runs of 4 consecutive output columns of one
//    routed row.
//  * bf16 activations have no MX form, so a pre-pass (quantize_tile in prepare_kernel)
//    splits every 32-element block of every routed row once into two MX-FP6
//    (E2M3) terms, hi + lo, each with its own E8M0 scale, using the gfx950
//    converts v_cvt_scalef32_pk32_fp6_bf16 (round to nearest even of x/2^e)
//    and v_cvt_scalef32_pk32_f32_fp6: hi is the block under the smallest power
//    of two that keeps its largest magnitude <= 7.5, lo the residual x - hi
//    (exact, and exactly a bf16) quantized the same way.  The GEMM issues one
//    MFMA per term; E2M3 x E2M1 runs at the FP4 MFMA rate on gfx950.
//  * The pre-pass also gathers the routed rows into row tiles (per expert, in
//    routed order), written in the register image of the MFMA B operand, so
//    that a wave fetches one k-step of its 32 rows with four contiguous loads
//    straight into registers, two k-steps ahead.
//  * Tile = 128 routed rows x 192 weight rows, 4 waves; wave w owns routed
//    rows 32w .. 32w + 31 and all 192 weight rows (6 accumulators of 32 x 32).
//    192 divides both gpt-oss widths (2880, 5760), so no weight panel is
//    padded, and the registers the accumulators leave free hold a second
//    stage of weights in flight: weight loads have two stages to arrive.
//    The weight tile is the only operand shared by the waves, and it is the
//    light one (16 bytes per row and block against 48 for the two activation
//    terms), so it alone goes through LDS.  Two workgroups share a CU.
//  * Weight codes are staged 8 blocks (one 128-byte line of each weight row)
//    at a time: each wave loads 1 KB pieces of 8 rows x 128 bytes into
//    registers and writes them to LDS, the rows' blocks in an XOR-swizzled
//    order so that the MFMA lanes' 16-byte reads (32 rows, one block) hit
//    distinct LDS banks.  Double-buffered, written in two halves while the
//    current stage is multiplied, one barrier per stage.
//  * Weight scales are repacked per call (repack_panel in prepare_kernel) into the
//    per-lane words of a stage: 4 bytes, one per k-step, picked by the MFMA's
//    scale byte select.
//  * The tile schedule is derived on the device from expert_offsets (wave
//    scans), ordered so that the row tiles sharing a weight panel run back to
//    back on one XCD and read the panel from its L2.  Surplus workgroups exit
//    at once.  No host synchronisation; any skew of rows per expert.
//  * The accumulators start at the bias.  The epilogue passes each wave's
//    results through LDS so that every store instruction writes whole
//    128-byte lines (4 rows x 256 bytes), scattered through sorted_rows.

#include <type_traits>

#include "kernels.h"
#include "common.h"

namespace mxfp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v12i __attribute__((ext_vector_type(12)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;    // GEMM workgroup
constexpr int kQThreads = 256;           // pre-pass workgroups (one wave per row sub-tile)
constexpr int kBM = 128;                 // routed rows per tile: one 32-row sub-tile per wave
constexpr int kBN = 192;                 // weight rows per tile: 6 sub-tiles of 32 (192 divides 2880 and 5760)
constexpr int kSubN = kBN / 32;
constexpr int kSubW = 8;                 // repacked weight-scale words per lane and stage (kSubN used)
static_assert(kThreads >= kBN && kThreads >= kBM, "the prologue has one thread per tile column and row");
static_assert(kSubN <= kSubW, "scale words");
constexpr int kStepsPerStage = 4;        // MFMA k-steps (two MX blocks each) per weight stage
constexpr int kStageBlocks = 2 * kStepsPerStage;
constexpr int kStagePad = 2;             // stage counts are padded to a multiple of 2 (the ring)
constexpr int kAUnit = 3 * 1024;         // activation codes of one (row sub-tile, k-step)
constexpr int kFmtFp6E2M3 = 2;           // MFMA operand format codes
constexpr int kFmtFp4E2M1 = 4;
constexpr int kXcds = 8;
// word 3 of a raw buffer resource (stride 0, byte offsets, 32-bit data format)
constexpr int kBufferFlags = 0x00020000;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__host__ __device__ inline int round_up(int v, int m) { return (v + m - 1) / m * m; }

// weight stages for K (8 blocks each), padded to a multiple of 2; the padding
// blocks are zero activation codes
__host__ __device__ inline int stage_count(int K) {
  return round_up(((K >> 5) + kStageBlocks - 1) / kStageBlocks, kStagePad);
}

// ---------------------------------------------------------------------------
// activation quantization: bf16 block of 32 -> two to four MX-FP6 (E2M3) terms
// ---------------------------------------------------------------------------

// The E8M0 exponent of a term for a block whose largest magnitude has bf16
// bits `amax` (nonzero): the smallest e with amax * 2^-e <= 7.5, raised to the
// format's least exponent -127 for tinier blocks (their codes are then the
// E2M3 subnormals of 2^-127, or zero).
__device__ __forceinline__ int block_exponent(uint32_t amax) {
  const int ex = (int)(amax >> 7) - 127;          // exponent field (a bf16 subnormal reads as -127)
  const int e = ex - 2 + (((amax & 0x7f) > 112) ? 1 : 0);  // 4 * (1 + m/128) > 7.5  <=>  m > 112
  return e < -127 ? -127 : e;
}

// A block of 32 held as fp32: ev[i] = element 2 i, od[i] = element 2 i + 1,
// the order in which v_cvt_scalef32_2xpk16_fp6_f32 takes them (the same codes
// as v_cvt_scalef32_pk32_fp6_bf16 on the bf16 words, element 2 i in the low
// half of word i).  Every value is a bf16 value: the inputs, and each residual
// (rounding a value of at most 8 significant bits to the E2M3 grid leaves a
// remainder of at most 8), so fp32 holds them exactly.
struct Block32 {
  v16f ev, od;
};

__device__ __forceinline__ void unpack_block(const uint32_t (&w)[16], Block32& b) {
#pragma unroll
  for (int i = 0; i < 16; i++) {
    b.ev[i] = __uint_as_float(w[i] << 16);
    b.od[i] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// the block's largest magnitude
__device__ __forceinline__ float max_abs(const Block32& b) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 16; i++) m = fmaxf(m, fmaxf(fabsf(b.ev[i]), fabsf(b.od[i])));
  return m;
}

// One MX-FP6 term of block b: its codes and E8M0 byte (127 for a zero block),
// and b replaced by the residual b - term (exact).  amax = max_abs(b), which
// the caller has at hand.  The convert rounds x / 2^e to the nearest E2M3
// value (ties to even).  Exponents below -100 run the convert on the block
// times 2^64 with the scale times 2^64 (the same codes; the scale argument
// stays a normal fp32), in place.
__device__ __forceinline__ void scale_block(Block32& b, float f) {
#pragma unroll
  for (int i = 0; i < 16; i++) {
    b.ev[i] *= f;
    b.od[i] *= f;
  }
}

__device__ __forceinline__ void fp6_term(Block32& b, float amax, v6i& codes, uint32_t& byte) {
  codes = v6i{0, 0, 0, 0, 0, 0};
  byte = 127u;
  if (amax == 0.f) return;
  const int e = block_exponent(__float_as_uint(amax) >> 16);
  byte = (uint32_t)(e + 127);
  // The block is multiplied by 1 or 2^64 per lane, under a branch taken by the
  // whole wave when any lane shifts (a per-lane select of the whole block
  // would double the registers it holds); none does for ordinary inputs.
  const bool shift = e < -100;
  const bool any_shift = wave_ballot(shift) != 0;
  if (any_shift) scale_block(b, shift ? 0x1p64f : 1.0f);
  const float scale = __uint_as_float((uint32_t)(e + (shift ? 64 : 0) + 127) << 23);
  codes = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(b.ev, b.od, scale);
  const v32f dv = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(codes, scale);
#pragma unroll
  for (int i = 0; i < 16; i++) {
    b.ev[i] -= dv[2 * i];
    b.od[i] -= dv[2 * i + 1];
  }
  if (any_shift) scale_block(b, shift ? 0x1p-64f : 1.0f);
}

// Whether a block whose residual after the terms so far has bf16 bits
// `rmax` (largest magnitude) takes another term: when that residual exceeds
// 1/64 of the block's mean magnitude without its largest element,
// (sum |x| - max |x|) / 31.  Blocks of like magnitudes pass with two terms;
// a block with an outlier channel, or heavy tails, takes three or four, so
// that its small elements keep their own precision.
constexpr float kExtraTermRatio = 31.0f * 64.0f;
__device__ __forceinline__ bool needs_term(float rmax, float sum_rest) {
  return rmax * kExtraTermRatio > sum_rest;
}

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

// Row tiles of the grouped problem: expert e's routed rows [b_e, f_e) are cut
// into ceil((f_e - b_e) / kBM) tiles, numbered over the experts in order.
// Finds the expert of row tile t (its rows [b, f) and its first tile tb) with
// one wave scan per 64 experts; false if t is past the last tile.
__device__ __forceinline__ bool locate_row_tile(const int32_t* offsets, int E, int R, int t, int lane, int& e_out,
                                                int& b_out, int& f_out, int& tb_out) {
  int before = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    int cnt = 0, b = 0, f = 0;
    if (e < E) {
      expert_rows(offsets, e, R, b, f);
      cnt = (f - b + kBM - 1) / kBM;
    }
    const int incl = wave_incl_scan(cnt, lane);
    const int tl = t - before;
    const uint64_t hit = wave_ballot(cnt > 0 && incl - cnt <= tl && tl < incl);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      e_out = __builtin_amdgcn_readfirstlane(base + src);
      b_out = __builtin_amdgcn_readfirstlane(__shfl(b, src, 64));
      f_out = __builtin_amdgcn_readfirstlane(__shfl(f, src, 64));
      tb_out = __builtin_amdgcn_readfirstlane(before + __shfl(incl - cnt, src, 64));
      return true;
    }
    before += __shfl(incl, 63, 64);
  }
  return false;
}

// Wave = row sub-tile sub of row tile t; lane (l32, h) = row 32 sub + l32, block 2 g + h of each k-step g.
// A wave's 32 rows x 2 blocks are one unit (t, sub, g) of the GEMM: one MFMA
// B operand per term.  Every block gets two terms (hi, lo); when any block of
// the unit needs a third (needs_term), all of them get one, and likewise a
// fourth.  Writes the register image of the MFMA B operand: per unit 3 KB, the
// 48 bytes of a lane's hi and lo operands (6 words each, in that order) as
// three chunks of [lane][16 B], so that a wave fetches a k-step with three
// full-width loads into twelve consecutive registers; the third and fourth
// terms in the same form in the unit's 3 KB extra record (written only when
// used); per (row tile, sub-tile, stage of 4 k-steps) [lane][4] u32 scale
// words, word j for k-step 4 stage + j (hi | lo << 8 | third << 16 | fourth <<
// 24), one load per stage; and the unit's count of extra terms (0, 1 or 2) in
// one byte.  The k-steps of a sub-tile are consecutive.  Rows past the
// expert's last routed row, and blocks past K, are zero codes with scale 127.
// A pair of terms (a: the first, b: the second) as the record's three chunks,
// each store a whole 16 bytes per lane (1 KB per wave instruction); has_b =
// false (a third term without a fourth): the first two chunks only, the
// fourth term's half of the second zero (never read).
__device__ __forceinline__ void put_terms(uint8_t* rec, int lane, const v6i& a, const v6i& b, bool has_b) {
  *reinterpret_cast<uint4*>(rec + lane * 16) = make_uint4(a[0], a[1], a[2], a[3]);
  *reinterpret_cast<uint4*>(rec + 1024 + lane * 16) = make_uint4(a[4], a[5], has_b ? b[0] : 0, has_b ? b[1] : 0);
  if (has_b) *reinterpret_cast<uint4*>(rec + 2048 + lane * 16) = make_uint4(b[2], b[3], b[4], b[5]);
}

// Workgroup blk = (row tile t, group of kQSteps k-steps): each wave locates
// its rows once and walks the group's k-steps with the blocks of the next
// kQAhead k-steps in flight while the current one is split (loads are
// unconditional, from a clamped address, and masked afterwards).
constexpr int kQSteps = 8;
constexpr int kQAhead = 4;

__device__ __forceinline__ void load_block(const uint4* p, uint32_t (&w)[16]) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint4 v = p[i];
    w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
}

__device__ __forceinline__ void quantize_tile(int blk, const uint16_t* __restrict__ x, int x_per_slot, int k, int R,
                                              int E, int K, int NKP, const int32_t* __restrict__ offsets,
                                              const int32_t* __restrict__ sorted_rows, uint8_t* __restrict__ q,
                                              uint8_t* __restrict__ qx, uint32_t* __restrict__ s,
                                              uint8_t* __restrict__ qf) {
  const int NQ = (NKP + kQSteps - 1) / kQSteps;
  const int t = blk / NQ;
  const int g0 = (blk - t * NQ) * kQSteps;
  const int g1 = min(g0 + kQSteps, NKP);
  const int lane = threadIdx.x & 63;
  const int sub = threadIdx.x >> 6;
  int e, b, f, tb;
  if (!locate_row_tile(offsets, E, R, t, lane, e, b, f, tb)) return;
  const int l32 = lane & 31, h = lane >> 5;
  const int p = b + (t - tb) * kBM + sub * 32 + l32;
  int r = -1;
  if (p < f) {
    r = sorted_rows[p];
    if (r < 0 || r >= R) r = -1;
  }
  const int KB = K >> 5;
  const uint4* row = reinterpret_cast<const uint4*>(x + (size_t)(r < 0 ? 0 : (x_per_slot ? r : r / k)) * K);
  auto src = [&](int g) { return row + (size_t)min(2 * g + h, KB - 1) * 4; };  // 4 x 16 bytes per block
  uint32_t ring[kQAhead][16];
#pragma unroll
  for (int d = 0; d < kQAhead; d++) load_block(src(min(g0 + d, g1 - 1)), ring[d]);
  uint32_t sw4[4] = {0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu};
  uint64_t flags = 0;
  static_assert(kQSteps % 4 == 0 && kQSteps <= 8, "whole stages of scale words; eight flag bytes");
#pragma unroll
  for (int j = 0; j < kQSteps; j++) {
    const int g = g0 + j;
    if (g >= g1) break;
    uint32_t w[16];
    const bool real = r >= 0 && 2 * g + h < KB;
#pragma unroll
    for (int i = 0; i < 16; i++) w[i] = real ? ring[j % kQAhead][i] : 0u;
    if (j + kQAhead < kQSteps) load_block(src(min(g + kQAhead, g1 - 1)), ring[j % kQAhead]);
    Block32 blk;
    unpack_block(w, blk);
    // the block's magnitude without its largest element, in element order
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      sum += fabsf(blk.ev[i]);
      sum += fabsf(blk.od[i]);
    }
    float amax = max_abs(blk);
    const float sum_rest = sum - amax;
    // Terms 0 and 1 always; terms 2 and 3 when the unit needs them (unit-wide
    // decisions by ballot: the extra MFMAs serve all 32 rows x 2 blocks).  Terms
    // are stored in pairs, whole chunks at a time; one loop body (not
    // unrolled), so that few registers are live.
    const size_t unit = ((size_t)t * kWaves + sub) * NKP + g;
    uint8_t* rec = q + unit * kAUnit;
    uint8_t* xrec = qx + unit * kAUnit;
    uint32_t bytes = 0x7f7f7f7fu;
    int nterm = 0;
    v6i first = v6i{0, 0, 0, 0, 0, 0};
#pragma unroll 1
    for (; nterm < 4; nterm++) {
      if (nterm >= 2 && __ballot(needs_term(amax, sum_rest)) == 0) break;
      v6i c;
      uint32_t byte;
      fp6_term(blk, amax, c, byte);
      amax = max_abs(blk);  // the residual's, for the next term
      if (nterm & 1)
        put_terms(nterm < 2 ? rec : xrec, lane, first, c, true);
      else
        first = c;
      bytes = (bytes & ~(0xffu << (8 * nterm))) | (byte << (8 * nterm));
    }
    if (nterm == 3) put_terms(xrec, lane, first, first, false);
    // the scale words of a stage's four k-steps (g0 is a multiple of 4) as one
    // 16-byte store per lane, the counts of extra terms of the group's k-steps
    // as one store of lane 0
    sw4[j & 3] = bytes;
    if ((j & 3) == 3 || g + 1 == g1)
      *reinterpret_cast<uint4*>(s + (unit - g) * 64 + (g >> 2) * 256 + lane * 4) =
          make_uint4(sw4[0], sw4[1], sw4[2], sw4[3]);
    flags |= (uint64_t)(nterm - 2) << (8 * j);
  }
  if (lane == 0) {
    uint8_t* fl = qf + ((size_t)t * kWaves + sub) * NKP + g0;
    if (g1 - g0 == kQSteps)
      *reinterpret_cast<uint2*>(fl) = make_uint2((uint32_t)flags, (uint32_t)(flags >> 32));
    else
      for (int j = 0; j < g1 - g0; j++) fl[j] = (uint8_t)(flags >> (8 * j));
  }
}

// ---------------------------------------------------------------------------
// weight-scale repack: [E][N][KB] bytes -> per (e, n-tile, stage) 64 lanes x
// 8 sub-tile words; byte j of word c of lane (l32, h) = scale of row
// 32 c + l32, block 8 s + 2 j + h.  Rows past N repeat row N - 1 and blocks
// past K repeat block K - 1: they meet zero activations or are never stored.
// ---------------------------------------------------------------------------

// Workgroup = one (expert, 256-row panel).  The panel's scale bytes are one
// contiguous range; the workgroup copies it into LDS with coalesced 4-byte
// loads (from the 4-byte boundary at or below its start; a last word that
// would reach past the end of the array is read byte by byte), then thread =
// one weight row writes, stage by stage, the two lane words of its row: lane
// (l32, h) with l32 = row % 32, word c = row / 32.
constexpr int kRepackMaxKB = 256;  // K <= 8192 (LDS: 256 rows x KB bytes + 4)

__device__ __forceinline__ void repack_panel(int blk, uint32_t* panel, const uint8_t* __restrict__ scales, int E,
                                             int N, int KB, int NT, int NS, uint32_t* __restrict__ out) {
  const int nt = blk % NT;
  const int e = blk / NT;
  const int t = threadIdx.x;  // row within the panel
  const int rows = min(kBN, N - nt * kBN);
  const size_t total = (size_t)E * N * KB;                   // bytes in the array
  const size_t first = ((size_t)e * N + (size_t)nt * kBN) * KB;
  const size_t a0 = first & ~(size_t)3;
  const int lead = (int)(first - a0);
  const int nwords = (int)((first + (size_t)rows * KB - a0 + 3) / 4);
  const uint32_t* src = reinterpret_cast<const uint32_t*>(scales) + a0 / 4;
  // words wholly inside the array; only the range's last word can fall short
  const int nsafe = (int)min((size_t)nwords, (total - a0) / 4);
  constexpr int kU = 24;  // independent loads in flight per thread (one pass for K <= 3072)
  for (int i0 = t; i0 < nsafe; i0 += kQThreads * kU) {
    uint32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; u++) v[u] = src[min(i0 + u * kQThreads, nsafe - 1)];
#pragma unroll
    for (int u = 0; u < kU; u++)
      if (i0 + u * kQThreads < nsafe) panel[i0 + u * kQThreads] = v[u];
  }
  if (t == 0 && nsafe < nwords) {
    const size_t byte = a0 + 4 * (size_t)nsafe;
    uint32_t v = 0;
    for (int q = 0; q < 4; q++)
      if (byte + q < total) v |= (uint32_t)scales[byte + q] << (8 * q);
    panel[nsafe] = v;
  }
  __syncthreads();
  const uint8_t* prow = reinterpret_cast<const uint8_t*>(panel) + lead + min(t, rows - 1) * KB;
  const int c = t >> 5, l32 = t & 31;
  if (t >= kBN) return;  // the threads past the panel's rows only helped stage it
  uint32_t* dst = out + ((size_t)e * NT + nt) * NS * (kSubW * 64) + l32 * kSubW + c;
  for (int s = 0; s < NS; s++) {
    uint32_t b[kStageBlocks];
#pragma unroll
    for (int i = 0; i < kStageBlocks; i++) b[i] = prow[min(kStageBlocks * s + i, KB - 1)];
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < kStepsPerStage; j++) {
      w0 |= b[2 * j] << (8 * j);
      w1 |= b[2 * j + 1] << (8 * j);
    }
    dst[(size_t)s * (kSubW * 64)] = w0;                // lane l32 (h = 0)
    dst[(size_t)s * (kSubW * 64) + 32 * kSubW] = w1;   // lane l32 + 32 (h = 1)
  }
}

// ---------------------------------------------------------------------------
// arrival counters of the fused combine: thread = one token t.  Its counter
// of every weight panel starts at k minus its routed slots (ids in [0, E)),
// so that the last routed row to arrive finds k - 1.  A token with no routed
// slot gets no arrival: its y row is written here, as the combine of k zero
// products, 0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void init_arrivals(int blk, const int32_t* __restrict__ ids, int T, int k, int E, int NT,
                                              int N, int32_t* __restrict__ cnt, float* __restrict__ y) {
  const int t = blk * kQThreads + threadIdx.x;
  if (t >= T) return;
  int routed = 0;
  for (int s = 0; s < k; s++) routed += (unsigned)ids[(size_t)t * k + s] < (unsigned)E ? 1 : 0;
  for (int nt = 0; nt < NT; nt++) cnt[(size_t)t * NT + nt] = k - routed;
  if (routed == 0)
    for (int n = 0; n < N; n++) y[(size_t)t * N + n] = 0.f;
}

// The passes before the GEMM in one launch (they are independent, so their
// workgroups run side by side): workgroups [0, nq) quantize one (row tile,
// k-step range) each, the next nrep repack the weight scales of one (expert,
// panel) each, and any after those set the fused combine's arrival counters.
// The long quantization workgroups go first (dispatched first, they no longer
// wait behind the repack).  Dynamic LDS: a panel's scale rows.
__global__ __launch_bounds__(kQThreads) void prepare_kernel(const uint8_t* __restrict__ scales, int E, int N, int KB,
                                                            int NT, int NS, uint32_t* __restrict__ wsc, int nrep,
                                                            const uint16_t* __restrict__ x, int x_per_slot, int k,
                                                            int R, int K, int NKP,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ sorted_rows,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ qx,
                                                            uint32_t* __restrict__ qs, uint8_t* __restrict__ qf, int nq,
                                                            const int32_t* __restrict__ ids, int32_t* __restrict__ cnt,
                                                            float* __restrict__ y) {
  extern __shared__ uint32_t panel[];  // (kBN * KB + 4) / 4 + 1 words
  if ((int)blockIdx.x < nq)
    quantize_tile(blockIdx.x, x, x_per_slot, k, R, E, K, NKP, offsets, sorted_rows, q, qx, qs, qf);
  else if ((int)blockIdx.x < nq + nrep)
    repack_panel(blockIdx.x - nq, panel, scales, E, N, KB, NT, NS, wsc);
  else
    init_arrivals(blockIdx.x - nq - nrep, ids, R / k, k, E, NT, N, cnt, y);
}

// ---------------------------------------------------------------------------
// grouped GEMM
// ---------------------------------------------------------------------------

struct TileCoord {
  int e, m_begin, m_count, nt, mtile;  // mtile: the row tile's number over all experts
};

// Tile t of the grouped problem (TM routed rows x one weight panel): experts
// in order; within an expert the weight panel (n-tile) varies slowest so that
// the row tiles sharing a panel are consecutive.  Workgroup L takes tile
// (L % 8) * ceil(tiles / 8) + L / 8: workgroups are dispatched round-robin
// over the 8 XCDs, so consecutive tiles run on one XCD and share its L2.  Each
// wave decodes its tile itself (wave scans over 64 experts at a time), so no
// barrier is needed.  c.mtile numbers the tile's first 128-row tile (the
// pre-pass's unit of activation records) over all experts.
template <int TM>
__device__ __forceinline__ bool locate_tile(const int32_t* offsets, int E, int R, int NT, int lane, TileCoord& c) {
  static_assert(TM % kBM == 0, "whole 128-row tiles");
  if (E <= 64) {
    // one lane per expert: one read of the offsets and one scan give both the
    // tile count and this workgroup's tile
    int b = 0, f = 0, cnt = 0, c128 = 0;
    if (lane < E) {
      expert_rows(offsets, lane, R, b, f);
      cnt = (f - b + TM - 1) / TM * NT;
      c128 = (f - b + kBM - 1) / kBM;
    }
    const int incl = wave_incl_scan(cnt, lane);
    const int incl128 = wave_incl_scan(c128, lane);
    const int total = __shfl(incl, 63, 64);
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int j = blockIdx.x / kXcds;
    if (j >= per_xcd) return false;
    const int t = (blockIdx.x % kXcds) * per_xcd + j;
    if (t >= total) return false;
    const uint64_t hit = wave_ballot(cnt > 0 && incl - cnt <= t && t < incl);
    const int src = __builtin_ctzll(hit);
    const int eb = __shfl(b, src, 64), ef = __shfl(f, src, 64);
    const int before = __shfl(incl, src, 64) - __shfl(cnt, src, 64);
    const int before128 = __shfl(incl128, src, 64) - __shfl(c128, src, 64);
    const int local = t - before;
    const int mt = (ef - eb + TM - 1) / TM;
    const int nt = local / mt;
    const int mi = local - nt * mt;
    c.e = __builtin_amdgcn_readfirstlane(src);
    c.m_begin = __builtin_amdgcn_readfirstlane(eb + mi * TM);
    c.m_count = __builtin_amdgcn_readfirstlane(min(TM, ef - (eb + mi * TM)));
    c.nt = __builtin_amdgcn_readfirstlane(nt);
    c.mtile = __builtin_amdgcn_readfirstlane(before128 + mi * (TM / kBM));
    return true;
  }
  int total = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    int cnt = 0;
    if (e < E) {
      int b, f;
      expert_rows(offsets, e, R, b, f);
      cnt = (f - b + TM - 1) / TM * NT;
    }
    total += wave_sum_i(cnt);
  }
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int L = blockIdx.x;
  const int j = L / kXcds;
  if (j >= per_xcd) return false;
  const int t = (L % kXcds) * per_xcd + j;
  if (t >= total) return false;
  int before = 0, before128 = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    int cnt = 0, c128 = 0, b = 0, f = 0;
    if (e < E) {
      expert_rows(offsets, e, R, b, f);
      cnt = (f - b + TM - 1) / TM * NT;
      c128 = (f - b + kBM - 1) / kBM;
    }
    const int incl = wave_incl_scan(cnt, lane);
    const int incl128 = wave_incl_scan(c128, lane);
    const int tl = t - before;
    const uint64_t hit = wave_ballot(cnt > 0 && incl - cnt <= tl && tl < incl);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int eb = __shfl(b, src, 64), ef = __shfl(f, src, 64);
      const int local = tl - (__shfl(incl, src, 64) - __shfl(cnt, src, 64));
      const int mt = (ef - eb + TM - 1) / TM;
      const int nt = local / mt;
      const int mi = local - nt * mt;
      // wave-uniform by construction; say so, so that branches on them are scalar
      c.e = __builtin_amdgcn_readfirstlane(base + src);
      c.m_begin = __builtin_amdgcn_readfirstlane(eb + mi * TM);
      c.m_count = __builtin_amdgcn_readfirstlane(min(TM, ef - (eb + mi * TM)));
      c.nt = __builtin_amdgcn_readfirstlane(nt);
      c.mtile = __builtin_amdgcn_readfirstlane(before128 + __shfl(incl128, src, 64) - __shfl(c128, src, 64) +
                                               mi * (TM / kBM));
      return true;
    }
    before += __shfl(incl, 63, 64);
    before128 += __shfl(incl128, 63, 64);
  }
  return false;
}

// Wait for this wave's LDS instructions and meet the other waves.  Only
// compiler-level fences: a workgroup fence would also wait for every load in
// flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XOR swizzle of a weight row's 8 blocks in its 128-byte LDS line: 8 (and 16)
// consecutive rows place any one block in distinct 16-byte bank groups.
__device__ __forceinline__ int row_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

constexpr int kAhead = 2;  // activation k-steps loaded ahead
// Keeps the main loop in the order it is written: no memory access crosses
// it (compiler fence) and no instruction at all (scheduling barrier).  Left
// free, the scheduler moves each MFMA up to the LDS read or activation load
// that feeds it, to shorten register lifetimes, and exposes their latency;
// with the operands addressed by buffer resources (one VGPR per stream) the
// written order fits in the registers of two waves per SIMD.
__device__ __forceinline__ void pipeline_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Every global read of the main loop is an ordinary load into registers (the
// weight stages are then written to LDS with ds_write): with LDS DMAs in
// flight beside register loads, the compiler's wait-count analysis treats the
// vector-memory counter as out of order and waits for every load before each
// use.  NS_T > 0: the stage count, known at compile time (straight-line
// pipeline); NS_T = 0: any K, with a loop.
// Cache policy of the fused combine's row stores and loads: sc1, the bit the
// compiler sets on device-scope (agent) relaxed atomic loads and stores.  An
// sc1 store is written through to the level all XCDs share, and is complete
// (vmcnt) once it is there; an sc1 load reads that level, never a stale line
// of its own XCD's L2.  With both, a tile's rows are visible to any other
// tile once its stores are complete, without writing back or invalidating
// whole L2s (a device-scope fence does both, and at one per tile it slowed
// the GEMM more than threefold).
constexpr int kCohPolicy = 16;
// byte offset of element i of out (out stays under 4 GiB: checked on the host)
__device__ __forceinline__ int coh_off(int i) { return (int)((uint32_t)i * 4u); }

// A wave's 32 routed rows x kBN columns (bias included) to out, with sc1
// stores through the buffer resource orsrc (out, byte offsets).  st: the
// wave's 8 KB of free LDS; wrows: the wave's 32 routed rows (-1: none).  Lane
// (l32, half) holds row l32 and, in elements 4 q + i of accumulator c, columns
// n0 + 32 c + 8 q + 4 half + i.
__device__ __forceinline__ void store_out_rows(const v16f (&acc)[kSubN], uint8_t* st, const int* wrows, int lane,
                                               int n0, int N, bool vec, __amdgpu_buffer_rsrc_t orsrc) {
  const int l32 = lane & 31;
  const int half = lane >> 5;
  if (vec) {
    // [32 rows][16 pieces of 16 bytes], XOR-swizzled; the rows a lane stores:
    // row 4 i + lane / 16, piece lane % 16.  kSubN / 2 rounds of 64 columns
    // (accumulators 2 rnd, 2 rnd + 1): element run (c, q) of a lane is piece
    // 8 (c - 2 rnd) + 2 q + half of its row; the columns are a multiple of 4,
    // so col < N covers a whole piece.  Each store instruction writes 4 rows x
    // 256 contiguous bytes: whole 128-byte lines.
    auto st_at = [&](int row, int piece) { return st + row * 256 + ((piece ^ (row & 15)) << 4); };
    const int piece = lane & 15;
    int rr[8];
#pragma unroll
    for (int i = 0; i < 8; i++) rr[i] = wrows[4 * i + (lane >> 4)];
#pragma unroll
    for (int rnd = 0; rnd < kSubN / 2; rnd++) {
#pragma unroll
      for (int cc = 0; cc < 2; cc++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int c = 2 * rnd + cc;
          *reinterpret_cast<f32x4_t*>(st_at(l32, 8 * cc + 2 * q + half)) =
              f32x4_t{acc[c][4 * q], acc[c][4 * q + 1], acc[c][4 * q + 2], acc[c][4 * q + 3]};
        }
      asm volatile("" ::: "memory");  // a wave's LDS accesses complete in order
      const int col = n0 + 64 * rnd + 4 * piece;
      u32x4_t v[8];  // all reads first: one wait, not one per store
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = *reinterpret_cast<const u32x4_t*>(st_at(4 * i + (lane >> 4), piece));
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 8; i++)
        if (rr[i] >= 0 && col < N)
          __builtin_amdgcn_raw_buffer_store_b128(v[i], orsrc, coh_off(rr[i] * N + col), 0, kCohPolicy);
    }
    return;
  }
  // any other width or alignment: 4-byte stores from the registers
  const int r = wrows[l32];
  if (r < 0) return;
  const int o = r * N + n0 + 4 * half;
#pragma unroll
  for (int c = 0; c < kSubN; c++)
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (n0 + 32 * c + 8 * q + 4 * half + i < N)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[c][4 * q + i]), orsrc,
                                                coh_off(o + 32 * c + 8 * q + i), 0, kCohPolicy);
}

// The gate-weighted combine fused into the projection (gpt-oss-20b files
// page, src/experts.linnet fn forward_routed: the routed rows' outputs summed
// per token with the router weights):
//   y[t, n] = sum over slots s in slot order of gates[t, s] * out[t, s, n],
// one fused multiply-add each; a slot that is not routed (id outside [0, E))
// or has gate 0 adds a zero product.  A token's k slot rows lie in up to k row
// tiles (one per chosen expert), run by different workgroups, possibly on
// different XCDs.  Per (token, weight panel) an arrival counter, set by the
// pre-pass to k minus the token's routed slots, takes one increment per routed
// row a tile has written (device-scope atomics); the increment that finds
// k - 1 belongs to the tile with the last of the token's rows, and that tile
// sums the token's rows over its panel's columns.  The rows were stored with
// sc1 and every wave waits for its stores to complete before the increments;
// the summing tile reads them with sc1 loads after its increment returned.
// The sum order is fixed whatever the arrival order, so y is deterministic and
// equal bit for bit to the separate combine's.
// The sums of the tokens last_t[0 .. nl) over the panel's columns n0 ..
// n0 + ncol (see combine_arrived).  Not inlined: its loads (kItems items x
// kSlots rows per thread in flight, enough bytes to cover the latency of the
// level all XCDs share) then do not weigh on the GEMM's register allocation.
constexpr int kSumItems = 4;  // items per thread in flight
constexpr int kSumSlots = 4;  // slot rows per item in flight
template <int NTH>
__device__ __noinline__ void sum_tokens(const int* last_t, int nl, int n0, int ncol, int N, int E, int k,
                                        const int32_t* __restrict__ ids, const float* __restrict__ gates, bool vec,
                                        __amdgpu_buffer_rsrc_t orsrc, float* __restrict__ y) {
  const int tid = threadIdx.x;
  // a slot's row counts when the slot is routed and its gate is not 0;
  // otherwise it adds a zero product (a zero weight times a zero), whatever
  // the row or the gate holds
  auto counts = [&](int id, float g) { return (unsigned)id < (unsigned)E && g != 0.f; };
  if (vec) {
    // item = (token, 4 columns)
    const int n4 = ncol >> 2;
    const int items = nl * n4;
    for (int it0 = tid; it0 < items; it0 += kSumItems * NTH) {
      int tt[kSumItems], cc[kSumItems];
      f32x4_t a[kSumItems];
#pragma unroll
      for (int u = 0; u < kSumItems; u++) {
        const int it = min(it0 + u * NTH, items - 1);  // past the end: a repeat, not stored
        const int i = it / n4;
        tt[u] = last_t[i];
        cc[u] = n0 + 4 * (it - i * n4);
        a[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      for (int s0 = 0; s0 < k; s0 += kSumSlots) {
        // every load of the pass first (slots past k re-read slot k - 1)
        u32x4_t v[kSumItems][kSumSlots];
        float g[kSumItems][kSumSlots];
        int id[kSumItems][kSumSlots];
#pragma unroll
        for (int u = 0; u < kSumItems; u++)
#pragma unroll
          for (int j = 0; j < kSumSlots; j++) {
            const int r = tt[u] * k + min(s0 + j, k - 1);
            v[u][j] = __builtin_amdgcn_raw_buffer_load_b128(orsrc, coh_off(r * N + cc[u]), 0, kCohPolicy);
            g[u][j] = gates[r];
            id[u][j] = ids[r];
          }
#pragma unroll
        for (int u = 0; u < kSumItems; u++)
#pragma unroll
          for (int j = 0; j < kSumSlots; j++) {
            if (s0 + j < k) {
              const bool c = counts(id[u][j], g[u][j]);
              const f32x4_t x = c ? __builtin_bit_cast(f32x4_t, v[u][j]) : f32x4_t{0.f, 0.f, 0.f, 0.f};
              const float gw = c ? g[u][j] : 0.f;
              a[u] = f32x4_t{fmaf(gw, x[0], a[u][0]), fmaf(gw, x[1], a[u][1]), fmaf(gw, x[2], a[u][2]),
                             fmaf(gw, x[3], a[u][3])};
            }
          }
      }
#pragma unroll
      for (int u = 0; u < kSumItems; u++)
        if (it0 + u * NTH < items) *reinterpret_cast<f32x4_t*>(y + (size_t)tt[u] * N + cc[u]) = a[u];
    }
    return;
  }
  for (int it = tid; it < nl * ncol; it += NTH) {
    const int i = it / ncol;
    const int col = n0 + (it - i * ncol);
    const int t = last_t[i];
    float a = 0.f;
    for (int s = 0; s < k; s++) {
      const int r = t * k + s;
      const float g = gates[r];
      const float v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(orsrc, coh_off(r * N + col), 0, kCohPolicy));
      const bool c = counts(ids[r], g);
      a = fmaf(c ? g : 0.f, c ? v : 0.f, a);
    }
    y[(size_t)t * N + col] = a;
  }
}

template <int TM, int NTH>
__device__ __forceinline__ void combine_arrived(const int* rows_lds, int nt, int NT, int n0, int N, int E, int k,
                                                const int32_t* __restrict__ ids, const float* __restrict__ gates,
                                                bool vec, __amdgpu_buffer_rsrc_t orsrc, int32_t* __restrict__ cnt,
                                                float* __restrict__ y) {
  __shared__ int last_n;
  __shared__ int last_t[TM];
  const int tid = threadIdx.x;
  if (tid == 0) last_n = 0;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's row stores are complete
  __syncthreads();
  if (tid < TM) {
    const int r = rows_lds[tid];
    if (r >= 0) {
      const int t = r / k;
      if (atomicAdd(&cnt[(size_t)t * NT + nt], 1) == k - 1) last_t[atomicAdd(&last_n, 1)] = t;
    }
  }
  __syncthreads();
  const int nl = last_n;
  if (nl == 0) return;
  sum_tokens<NTH>(last_t, nl, n0, min(kBN, N - n0), N, E, k, ids, gates, vec, orsrc, y);
}

// Epilogues: out (f32 rows), the gated activation (bf16 rows), or out followed
// by the gate-weighted combine of every token whose last slot this tile holds.
enum Epilogue { kEpiOut = 0, kEpiSwiglu = 1, kEpiCombine = 2 };

// W waves: a tile of 32 W routed rows (W / 4 of the pre-pass's 128-row tiles)
// x 192 weight rows; the weight stage is shared by all W waves, so eight waves
// move half the weight bytes per MFMA that four do.
template <int NS_T, int EPI, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2))) void expert_gemm_kernel(
    const uint8_t* __restrict__ blocks, const uint32_t* __restrict__ wsc, const uint16_t* __restrict__ bias, int E,
    int N, int K, const uint8_t* __restrict__ aq, const uint8_t* __restrict__ aqx, const uint32_t* __restrict__ as,
    const uint8_t* __restrict__ aqf, int T, int k, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_rows, float* __restrict__ out, uint16_t* __restrict__ act,
    const int32_t* __restrict__ ids, const float* __restrict__ gates, int32_t* __restrict__ cnt,
    float* __restrict__ y) {
  constexpr bool SWIGLU = EPI == kEpiSwiglu;
  constexpr bool COMBINE = EPI == kEpiCombine;
  constexpr int TM = 32 * W;              // routed rows per tile
  constexpr int kPieces = kBN / 8 / W;    // 1 KB weight pieces per wave and stage
  static_assert(W % kWaves == 0 && kPieces * 8 * W == kBN, "whole 128-row tiles, whole pieces");
  // weight stages, double-buffered: codes [192 rows][8 swizzled blocks] and
  // scale words [64 lanes][8 sub-tiles]; each slot large enough that the
  // epilogue's 8 KB per wave fits in the two
  constexpr int kSlot = kBN * 128 > W * 4096 ? kBN * 128 : W * 4096;
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kSlot];
  __shared__ __attribute__((aligned(16))) uint32_t sS0[kSubW * 64];
  __shared__ __attribute__((aligned(16))) uint32_t sS1[kSubW * 64];
  uint8_t* const sB0 = sB[0];
  uint8_t* const sB1 = sB[1];
  __shared__ __attribute__((aligned(16))) int rows_lds[TM];  // routed row of each tile row, -1 if none
  __shared__ __attribute__((aligned(16))) float bias_lds[kBN];  // bias of each tile column (0 without bias)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const int R = T * k;
  const int NT = (N + kBN - 1) / kBN;
  TileCoord tc;
  if (!locate_tile<TM>(offsets, E, R, NT, lane, tc)) return;
  const int e = tc.e;
  const int KB = K >> 5;
  const int NS = NS_T > 0 ? NS_T : stage_count(K);
  const int NKP = NS * kStepsPerStage;
  const int nks = (KB + 1) >> 1;  // k-steps holding real blocks

  if (tid < TM) {
    int r = -1;
    if (tid < tc.m_count) {
      r = sorted_rows[tc.m_begin + tid];
      if (r < 0 || r >= R) r = -1;
    }
    rows_lds[tid] = r;
  }
  // the tile's bias values, read here so that the epilogue waits on no global load
  if (tid < kBN)
    bias_lds[tid] = bias ? bf16_bits_to_f32(bias[(size_t)tc.e * N + min(tc.nt * kBN + tid, N - 1)]) : 0.f;
  const bool valid = wave * 32 < tc.m_count;

  // activations: this wave's row sub-tile (sub-tile wave % 4 of 128-row tile
  // mtile + wave / 4), k-steps consecutive.  Buffer loads: the wave's records
  // as one resource (SGPRs), a 32-bit lane offset in a VGPR and the k-step in
  // the scalar offset.
  const size_t unit0 = ((size_t)tc.mtile * kWaves + wave) * NKP;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(aq + unit0 * kAUnit), (short)0, NKP * kAUnit, kBufferFlags);
  const __amdgpu_buffer_rsrc_t as_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(as + unit0 * 64), (short)0, NKP * 256, kBufferFlags);

  // weight stage pieces: piece i = wave + W q (q < kPieces) covers tile rows
  // 8i .. 8i + 7 (1 KB); lane L takes row 8i + L / 8 and LDS slot L % 8, which
  // holds block (L % 8) ^ swizzle(row) of the stage (rows past N re-read row
  // N - 1, blocks past K re-read block K - 1)
  const int n0 = tc.nt * kBN;
  // the expert's codes as one resource (at most 4 GiB, checked on the host)
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(blocks + (size_t)e * N * KB * 16), (short)0, N * KB * 16, kBufferFlags);
  const int b_r0 = n0 + 8 * wave + (lane >> 3);  // row of piece q: b_r0 + 8 W q
  // swizzle(8 i + L / 8) = (L / 8) ^ (i & 1), and i = wave + W q has the parity of wave
  const int b_blk = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
  // weight-scale words: the 2 KB of a stage as two 1 KB halves; waves of equal
  // parity move the same half (the same bytes to the same place)
  const __amdgpu_buffer_rsrc_t bs_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(wsc + ((size_t)e * NT + tc.nt) * NS * kSubW * 64), (short)0, NS * kSubW * 256,
      kBufferFlags);
  const int bs_off = (wave & 1) * 1024 + lane * 16;

  // A stage's weights move global -> registers -> LDS, kPieces pieces and the
  // stage's scale words per wave.  Two register sets: set s % 2 is loaded with
  // stage s + 2 at the start of stage s (it held stage s, which is in LDS by
  // then) and written to LDS at the end of stage s + 1, so the loads have two
  // stages to arrive (HBM latency under load is about two k-steps' work).
  u32x4_t rbs[2][kPieces + 1];
  auto load_w = [&](int s, auto xc) {
    constexpr int X = decltype(xc)::value;
    const int blk = min(kStageBlocks * s + b_blk, KB - 1) * 16;
#pragma unroll
    for (int q = 0; q < kPieces; q++)
      rbs[X][q] = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, min(b_r0 + 8 * W * q, N - 1) * (KB * 16) + blk, 0, 0);
    rbs[X][kPieces] = __builtin_amdgcn_raw_buffer_load_b128(bs_rsrc, bs_off, s * (kSubW * 64 * 4), 0);
  };
  auto store_w = [&](uint8_t* sb, uint32_t* ss, auto xc) {
    constexpr int X = decltype(xc)::value;
#pragma unroll
    for (int q = 0; q < kPieces; q++) *reinterpret_cast<u32x4_t*>(sb + (wave + W * q) * 1024 + lane * 16) = rbs[X][q];
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<uint8_t*>(ss) + (wave & 1) * 1024 + lane * 16) = rbs[X][kPieces];
  };

  // this lane's offsets into a stage for the k-step j: row l32 of each 32-row
  // sub-tile (sub-tile c adds c * 4096), block 2 j + half
  const int swz = row_swizzle(l32);
  int b_off[kStepsPerStage];
#pragma unroll
  for (int j = 0; j < kStepsPerStage; j++) b_off[j] = l32 * 128 + (((2 * j + half) ^ swz) << 4);

  // Accumulator c is the 32 x 32 product block (weight rows 32 c .. 32 c + 31)
  // x (the wave's routed rows): the weights are the MFMA's A operand, the
  // activations its B operand.  Lane (l32, half) holds routed row l32 and, in
  // elements 4 q + i, weight rows 32 c + 8 q + 4 half + i: four consecutive
  // output columns of one row, as the stores want them.
  v16f acc[kSubN];

  // activation ring: k-step g lives in slot g % 2 from its load (two k-steps
  // ahead) until it is multiplied: three full-width loads of the unit's hi and
  // lo operands.  The scale words of a stage's four k-steps are one load,
  // made during the stage before.
  constexpr int kA = W == 8 ? 4 : kAhead;  // activation k-steps in flight
  v12i ra[kA];
  u32x4_t asw[2];
  auto load_a = [&](int g, auto jc) {
    constexpr int J = decltype(jc)::value % kA;
    const int so = g * kAUnit;
    const u32x4_t c0 = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, lane * 16, so, 0);
    const u32x4_t c1 = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, lane * 16 + 1024, so, 0);
    const u32x4_t c2 = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, lane * 16 + 2048, so, 0);
    ra[J] = v12i{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y,
                 (int)c1.z, (int)c1.w, (int)c2.x, (int)c2.y, (int)c2.z, (int)c2.w};
  };
  auto load_as = [&](int s, auto xc) {
    asw[decltype(xc)::value] = __builtin_amdgcn_raw_buffer_load_b128(as_rsrc, lane * 16, s * 1024, 0);
  };

  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;

  // The weight operands of one k-step: 8 sub-tiles, 16 bytes per lane each.
  v8i bq[kSubN];
  auto read_b = [&](const uint8_t* sb, int c, int j) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sb + c * 4096 + b_off[j]);
    bq[c] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  };

  // One k-step J of a stage: for each weight sub-tile c the hi and lo MFMAs,
  // then (NEXT) the read of sub-tile c for k-step J + 1 into the registers
  // they just freed, so the LDS latency hides under the remaining MFMAs.
  auto kstep = [&](const uint8_t* sb, const uint32_t (&bsc)[kSubN], uint32_t sw, auto jc, bool next) {
    constexpr int J = decltype(jc)::value;
    constexpr int A = J % kA;
    const v8i ahi = __builtin_shufflevector(ra[A], ra[A], 0, 1, 2, 3, 4, 5, -1, -1);
    const v8i alo = __builtin_shufflevector(ra[A], ra[A], 6, 7, 8, 9, 10, 11, -1, -1);
#pragma unroll
    for (int c = 0; c < kSubN; c++) {
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bq[c], ahi, acc[c], kFmtFp4E2M1, kFmtFp6E2M3, J,
                                                               bsc[c], 0, sw);
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bq[c], alo, acc[c], kFmtFp4E2M1, kFmtFp6E2M3, J,
                                                               bsc[c], 1, sw);
      if (next) read_b(sb, c, (J + 1) & 3);
      // the read stays here, 7 sub-tiles ahead of its MFMAs
      pipeline_fence();
    }
  };

  // The pipeline, for a wave with routed rows (V) or without (its MFMAs and
  // activation loads skipped; it still moves its share of the weights and
  // meets the barriers).  Slot s % 2 holds stage s (NS is even).
  auto pipeline = [&](auto vc) {
    constexpr bool V = decltype(vc)::value;
    // One stage s from slot (sb, ss), register set X = s % 2: load stage s + 2
    // into set X; multiply the four k-steps, each followed by the activation
    // loads of the k-step two later (none past the last); then write set
    // 1 - X (stage s + 1, loaded during stage s - 1) into the other slot (nb,
    // ns) and meet the other waves.  The other slot was last read in stage
    // s - 1, which every wave finished before the barrier that ended it.  The
    // compiler fences keep each load where it is written: otherwise it sinks
    // next to its use and exposes its latency.
    // Mode M: 0 a stage with two after it, 1 the next-to-last, 2 the last.
    auto stage = [&](int s, const uint8_t* sb, const uint32_t* ss, uint8_t* nb, uint32_t* ns, auto xc, auto mc) {
      constexpr int X = decltype(xc)::value;
      constexpr int M = decltype(mc)::value;
      constexpr bool last = M == 2;
      if (M == 0) load_w(s + 2, xc);
      pipeline_fence();
      if (V) {
        uint32_t bsc[kSubN];
        const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(ss + lane * kSubW);
        const u32x2_t v1 = *reinterpret_cast<const u32x2_t*>(ss + lane * kSubW + 4);
        static_assert(kSubN == 6, "the scale words of 6 sub-tiles");
        bsc[0] = v0.x; bsc[1] = v0.y; bsc[2] = v0.z; bsc[3] = v0.w;
        bsc[4] = v1.x; bsc[5] = v1.y;
#pragma unroll
        for (int c = 0; c < kSubN; c++) read_b(sb, c, 0);
        const int g = s * kStepsPerStage;
        pipeline_fence();  // the reads are issued before the first MFMA
        const u32x4_t sw = asw[X];
        if (kA == 4) {
          // each k-step is followed by the activation loads of the k-step
          // four later (the next stage's), into the ring slot it just freed
          // (in the last stage, k-steps past the last real block are skipped)
          kstep(sb, bsc, sw.x, J0{}, true);
          if (!last) load_a(g + 4, J0{});
          pipeline_fence();
          if (!last || g + 1 < nks) kstep(sb, bsc, sw.y, J1{}, true);
          if (!last) load_a(g + 5, J1{});
          pipeline_fence();
          if (!last || g + 2 < nks) kstep(sb, bsc, sw.z, J2{}, true);
          if (!last) {
            load_as(s + 1, std::integral_constant<int, 1 - X>{});
            load_a(g + 6, J2{});
          }
          pipeline_fence();
          if (!last || g + 3 < nks) kstep(sb, bsc, sw.w, J3{}, false);
          if (!last) load_a(g + 7, J3{});
          pipeline_fence();
        } else if (!last) {
          // each k-step is followed by the activation loads of the k-step
          // two later, into the ring slot it just freed; the next stage's
          // scale words go with the first of its k-steps
          kstep(sb, bsc, sw.x, J0{}, true);
          load_a(g + 2, J2{});
          pipeline_fence();
          kstep(sb, bsc, sw.y, J1{}, true);
          load_a(g + 3, J3{});
          pipeline_fence();
          kstep(sb, bsc, sw.z, J2{}, true);
          load_as(s + 1, std::integral_constant<int, 1 - X>{});
          load_a(g + 4, J0{});
          pipeline_fence();
          kstep(sb, bsc, sw.w, J3{}, false);
          load_a(g + 5, J1{});
          pipeline_fence();
        } else {
          // the last stage: k-steps past the last real block are skipped
          kstep(sb, bsc, sw.x, J0{}, true);
          load_a(g + 2, J2{});
          pipeline_fence();
          if (g + 1 < nks) kstep(sb, bsc, sw.y, J1{}, true);
          load_a(g + 3, J3{});
          pipeline_fence();
          if (g + 2 < nks) kstep(sb, bsc, sw.z, J2{}, true);
          if (g + 3 < nks) kstep(sb, bsc, sw.w, J3{}, false);
        }
      }
      if (!last) {
        store_w(nb, ns, std::integral_constant<int, 1 - X>{});
        lds_barrier();
      }
    };

    load_w(0, J0{});
    load_w(1, J1{});
    if (V) {
      load_as(0, J0{});
      load_a(0, J0{});
      load_a(1, J1{});
      if (kA == 4) {
        load_a(2, J2{});
        load_a(3, J3{});
      }
    }
    store_w(sB0, sS0, J0{});
    lds_barrier();
    if (V) {
      // the sums start at the bias of their columns (bias_lds is complete)
#pragma unroll
      for (int c = 0; c < kSubN; c++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const f32x4_t b = *reinterpret_cast<const f32x4_t*>(bias_lds + 32 * c + 8 * q + 4 * half);
#pragma unroll
          for (int i = 0; i < 4; i++) acc[c][4 * q + i] = b[i];
        }
    }
    using M0 = std::integral_constant<int, 0>;
    using M1 = std::integral_constant<int, 1>;
    using M2 = std::integral_constant<int, 2>;
    int s = 0;
#pragma unroll
    for (; s + 2 < NS; s += 2) {
      stage(s, sB0, sS0, sB1, sS1, J0{}, M0{});
      stage(s + 1, sB1, sS1, sB0, sS0, J1{}, M0{});
    }
    stage(s, sB0, sS0, sB1, sS1, J0{}, M1{});  // s = NS - 2
    stage(s + 1, sB1, sS1, nullptr, nullptr, J1{}, M2{});
  };
  if (valid)
    pipeline(std::true_type{});
  else
    pipeline(std::false_type{});

  // ---- the third and fourth activation terms of the units that have them
  // (quantize_tile decides per unit; blocks of like magnitudes have none).  A
  // flagged k-step g re-reads its weight operands from memory (the stages in
  // LDS are gone): the 16-byte block 2 g + half of each sub-tile row, and the
  // repacked scale words of stage g / 4, whose byte g % 4 is the block's.
  if (valid) {
    const uint8_t* fl = aqf + unit0;
    const int f0 = fl[min(lane, NKP - 1)];
    const int f1 = fl[min(lane + 64, NKP - 1)];
    uint64_t m0 = wave_ballot(lane < NKP && f0 != 0);
    uint64_t m1 = wave_ballot(lane + 64 < NKP && f1 != 0);
    while (m0 | m1) {
      int g, n;
      if (m0) {
        const int i = __builtin_ctzll(m0);
        m0 &= m0 - 1;
        g = i;
        n = __builtin_amdgcn_readlane(f0, i);
      } else {
        const int i = __builtin_ctzll(m1);
        m1 &= m1 - 1;
        g = 64 + i;
        n = __builtin_amdgcn_readlane(f1, i);
      }
      g = __builtin_amdgcn_readfirstlane(g);
      n = __builtin_amdgcn_readfirstlane(n);
      const int blk = min(2 * g + half, KB - 1) * 16;
      u32x4_t wq[kSubN];
#pragma unroll
      for (int c = 0; c < kSubN; c++)
        wq[c] = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, min(n0 + 32 * c + l32, N - 1) * (KB * 16) + blk, 0, 0);
      const u32x4_t s0 = __builtin_amdgcn_raw_buffer_load_b128(bs_rsrc, lane * 32, (g >> 2) * (kSubW * 64 * 4), 0);
      const u32x2_t s1 = __builtin_amdgcn_raw_buffer_load_b64(bs_rsrc, lane * 32 + 16, (g >> 2) * (kSubW * 64 * 4), 0);
      const uint32_t sw = __builtin_amdgcn_raw_buffer_load_b32(as_rsrc, lane * 16 + (g & 3) * 4, (g >> 2) * 1024, 0);
      const uint8_t* xr = aqx + (unit0 + g) * kAUnit;
      const int sh = 8 * (g & 3);
      const uint32_t wsc8[kSubN] = {s0.x >> sh, s0.y >> sh, s0.z >> sh, s0.w >> sh, s1.x >> sh, s1.y >> sh};
      // the extra record in the layout of the main one: the third term's six
      // words, then the fourth's
      const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(xr + lane * 16);
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(xr + 1024 + lane * 16);
      const v8i t2 = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, 0, 0};
#pragma unroll
      for (int c = 0; c < kSubN; c++) {
        const v8i wa = v8i{(int)wq[c].x, (int)wq[c].y, (int)wq[c].z, (int)wq[c].w, 0, 0, 0, 0};
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, t2, acc[c], kFmtFp4E2M1, kFmtFp6E2M3, 0,
                                                                 wsc8[c], 2, sw);
      }
      if (n > 1) {
        const u32x4_t x2 = *reinterpret_cast<const u32x4_t*>(xr + 2048 + lane * 16);
        const v8i t3 = v8i{(int)x1.z, (int)x1.w, (int)x2.x, (int)x2.y, (int)x2.z, (int)x2.w, 0, 0};
#pragma unroll
        for (int c = 0; c < kSubN; c++) {
          const v8i wa = v8i{(int)wq[c].x, (int)wq[c].y, (int)wq[c].z, (int)wq[c].w, 0, 0, 0, 0};
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, t3, acc[c], kFmtFp4E2M1, kFmtFp6E2M3, 0,
                                                                   wsc8[c], 3, sw);
        }
      }
    }
  }

  // ---- epilogue: scatter to the routed rows (bias included).  Each lane
  // holds one routed row and, per accumulator, 4 runs of 4 consecutive
  // columns.  The wide paths pass the wave's results through its own 8 KB of
  // the weight slots (free once every wave has passed the barrier below), so
  // that each store instruction writes 4 rows x 256 contiguous bytes: whole
  // 128-byte lines, as HBM wants them (stores of 32 bytes per row slow down
  // every workgroup still streaming its operands).
  // every wave is past the main loop: both weight slots are free for staging
  lds_barrier();
  if constexpr (COMBINE) {
    // every wave takes part in the arrival (its barriers), with rows or not
    // (two call sites: one guarded store keeps a few values of the main loop
    // live across the epilogue, past the registers)
    // out [T, k, N] as one buffer resource (under 4 GiB, checked on the host)
    const __amdgpu_buffer_rsrc_t orsrc =
        __builtin_amdgcn_make_buffer_rsrc(out, (short)0, coh_off(T * k * N), kBufferFlags);
    const bool vec = (N & 3) == 0 && ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(y)) & 15) == 0;
    if (!valid) {
      combine_arrived<TM, W * 64>(rows_lds, tc.nt, NT, n0, N, E, k, ids, gates, vec, orsrc, cnt, y);
      return;
    }
    store_out_rows(acc, sB[0] + wave * 8192, rows_lds + wave * 32, lane, n0, N, vec, orsrc);
    combine_arrived<TM, W * 64>(rows_lds, tc.nt, NT, n0, N, E, k, ids, gates, vec, orsrc, cnt, y);
    return;
  }
  if (!valid) return;
  uint8_t* st = sB[0] + wave * 8192;  // [32 rows][16 pieces of 16 bytes], XOR-swizzled (slots 0 and 1)
  static_assert(W * 8192 <= 2 * kSlot, "the staging fits the weight slots");
  auto st_at = [&](int row, int piece) { return st + row * 256 + ((piece ^ (row & 15)) << 4); };
  // the rows a lane stores: row 4 i + lane / 16 of the wave's 32, piece lane % 16
  auto out_rows = [&](int (&rr)[8]) {
#pragma unroll
    for (int i = 0; i < 8; i++) rr[i] = rows_lds[wave * 32 + 4 * i + (lane >> 4)];  // -1 past the tile's rows
  };
  const int piece = lane & 15;
  if constexpr (SWIGLU) {
    // Weight rows 2 i (gate) and 2 i + 1 (up) give activation column i; n0 and
    // 8 q + 4 half are even, so elements (4 q, 4 q + 1) and (4 q + 2, 4 q + 3)
    // are two pairs: activation columns a0 + 16 c + 4 q + 2 half + (0, 1).
    const int NA = N >> 1;
    const int a0 = n0 >> 1;
    auto pair_word = [&](int c, int q) {
      const float g0 = acc[c][4 * q], u0 = acc[c][4 * q + 1];
      const float g1 = acc[c][4 * q + 2], u1 = acc[c][4 * q + 3];
      return f32_to_bf16_bits(swiglu(g0, u0)) | (f32_to_bf16_bits(swiglu(g1, u1)) << 16);
    };
    if ((NA & 7) == 0 && (reinterpret_cast<uintptr_t>(act) & 15) == 0) {
      // per accumulator, lane half 0 assembles activation columns 16 c + 0 .. 7
      // of its row and half 1 columns 16 c + 8 .. 15 (the partner lane, 32
      // away, holds the other half of each run of 4): piece 2 c + half
#pragma unroll
      for (int c = 0; c < kSubN; c++) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; q++) w[q] = pair_word(c, q);
        const uint32_t r0 = (uint32_t)__shfl_xor((int)(half ? w[0] : w[2]), 32, 64);
        const uint32_t r1 = (uint32_t)__shfl_xor((int)(half ? w[1] : w[3]), 32, 64);
        *reinterpret_cast<u32x4_t*>(st_at(l32, 2 * c + half)) =
            half ? u32x4_t{r0, w[2], r1, w[3]} : u32x4_t{w[0], r0, w[1], r1};
      }
      int rr[8];
      out_rows(rr);
      asm volatile("" ::: "memory");  // a wave's LDS accesses complete in order
      const int col = a0 + 8 * piece;  // NA % 8 == 0: a piece is wholly inside or outside
      // a row of the panel's activations is 2 kSubN pieces; the lanes of the
      // other pieces have nothing to store
      const bool piece_ok = piece < 2 * kSubN;
      u32x4_t v[8];  // all reads first: one wait, not one per store
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = *reinterpret_cast<const u32x4_t*>(st_at(4 * i + (lane >> 4), piece));
#pragma unroll
      for (int i = 0; i < 8; i++)
        if (piece_ok && rr[i] >= 0 && col < NA)
          __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4_t*>(act + (size_t)rr[i] * NA + col));
      return;
    }
    // any other width: 2-byte stores from the registers
    const int r = rows_lds[wave * 32 + l32];
    if (r < 0) return;
#pragma unroll
    for (int c = 0; c < kSubN; c++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint32_t w = pair_word(c, q);
        const int col = a0 + 16 * c + 4 * q + 2 * half;
        if (col < NA) act[(size_t)r * NA + col] = (uint16_t)(w & 0xffffu);
        if (col + 1 < NA) act[(size_t)r * NA + col + 1] = (uint16_t)(w >> 16);
      }
    return;
  }
  // streamed out: the outputs must not push the weights and activation tiles
  // other workgroups still read out of the caches
  if ((N & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    // kSubN / 2 rounds of 64 columns (accumulators 2 rnd, 2 rnd + 1): element run
    // (c, q) of a lane is piece 8 (c - 2 rnd) + 2 q + half of its row; the
    // columns are a multiple of 4, so col < N covers a whole piece
    int rr[8];
    out_rows(rr);
#pragma unroll
    for (int rnd = 0; rnd < kSubN / 2; rnd++) {
#pragma unroll
      for (int cc = 0; cc < 2; cc++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int c = 2 * rnd + cc;
          *reinterpret_cast<f32x4_t*>(st_at(l32, 8 * cc + 2 * q + half)) =
              f32x4_t{acc[c][4 * q], acc[c][4 * q + 1], acc[c][4 * q + 2], acc[c][4 * q + 3]};
        }
      asm volatile("" ::: "memory");  // a wave's LDS accesses complete in order
      const int col = n0 + 64 * rnd + 4 * piece;
      f32x4_t v[8];  // all reads first: one wait, not one per store
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = *reinterpret_cast<const f32x4_t*>(st_at(4 * i + (lane >> 4), piece));
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 8; i++)
        if (rr[i] >= 0 && col < N)
          __builtin_nontemporal_store(v[i], reinterpret_cast<f32x4_t*>(out + (size_t)rr[i] * N + col));
    }
    return;
  }
  // any other width or alignment: 4-byte stores from the registers
  const int r = rows_lds[wave * 32 + l32];
  if (r < 0) return;
  float* orow = out + (size_t)r * N + n0 + 4 * half;
#pragma unroll
  for (int c = 0; c < kSubN; c++)
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (n0 + 32 * c + 8 * q + 4 * half + i < N) __builtin_nontemporal_store(acc[c][4 * q + i], orow + 32 * c + 8 * q + i);
}

// waves per GEMM workgroup for the fp32 epilogue: eight while the routed rows
// average at least 256 per expert, else four
int gemm_waves(int E, int R) { return (long long)R >= 256LL * E ? 8 : 4; }

struct GemmLayout {
  size_t codes, extra, scales, flags, wscales, counters, total;
};

// most row tiles any routing can give: ceil(R / kBM) plus one partial tile per
// expert that has rows
size_t row_tiles_max(int E, int T, int k) {
  const size_t R = (size_t)T * k;
  return (R + kBM - 1) / kBM + (R < (size_t)E ? R : (size_t)E);
}

GemmLayout gemm_layout(int E, int N, int T, int k, int K) {
  const size_t tiles = row_tiles_max(E, T, k);
  const size_t ns = (size_t)stage_count(K);
  const size_t nkp = ns * kStepsPerStage;
  const size_t nt = (size_t)((N + kBN - 1) / kBN);
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t units = tiles * kWaves * nkp;
  GemmLayout l;
  l.codes = 0;
  l.extra = al(units * kAUnit);
  l.scales = l.extra + al(units * kAUnit);
  l.flags = l.scales + al(units * 256);
  l.wscales = l.flags + al(units);
  l.counters = l.wscales + al((size_t)E * nt * ns * kSubW * 256);
  l.total = l.counters + al((size_t)T * nt * 4);  // the fused combine's arrival counters
  return l;
}

}  // namespace

// ---------------------------------------------------------------------------
// the grouped GEMM's scratch for callers that cannot allocate
// (mxfp4_expert_proj_noalloc): a static device array, one per GPU for the
// life of the process.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kGemmStaticScratchBytes];

hipError_t gemm_static_scratch(void** ptr) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!dev_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

size_t gemm_workspace_bytes(int E, int N, int T, int k, int K, int x_per_slot) {
  (void)x_per_slot;
  return gemm_layout(E, N, T, k, K).total;
}

hipError_t launch_expert_gemm(const uint8_t* blocks, const uint8_t* scales, const uint16_t* bias, int E, int N,
                              int K, const uint16_t* x, int x_per_slot, int T, int k, const int32_t* offsets,
                              const int32_t* sorted_rows, float* out, uint16_t* act, void* workspace,
                              hipStream_t stream, const int32_t* ids, const float* gates, float* y) {
  // the GEMM addresses a weight row within its expert with 32-bit offsets;
  // the scale repack stages a panel's scale rows in LDS
  if ((size_t)N * (size_t)(K / 32) * 16 > 0xFFFFFFFFull || K / 32 > kRepackMaxKB) return hipErrorInvalidValue;
  const int NS = stage_count(K);
  const int NKP = NS * kStepsPerStage;
  const int NT = (N + kBN - 1) / kBN;
  const GemmLayout l = gemm_layout(E, N, T, k, K);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* aq = ws + l.codes;
  uint8_t* aqx = ws + l.extra;
  uint32_t* as = reinterpret_cast<uint32_t*>(ws + l.scales);
  uint8_t* aqf = ws + l.flags;
  uint32_t* bsc = reinterpret_cast<uint32_t*>(ws + l.wscales);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + l.counters);
  const bool combine = y != nullptr;  // out is written too
  const int R = T * k;
  const size_t tiles = row_tiles_max(E, T, k);
  // dynamic LDS: a panel's scale rows (23 KB at K = 2880, so several
  // workgroups share a CU)
  const size_t panel_bytes = ((size_t)(kBN * (K / 32) + 4) / 4 + 1) * 4;
  hipError_t err;
  static DynLdsLimit prepare_lds(reinterpret_cast<const void*>(&prepare_kernel),
                                 (int)(((kBN * kRepackMaxKB + 4) / 4 + 1) * 4));
  if (panel_bytes > 65536) {
    err = prepare_lds.ensure();
    if (err != hipSuccess) return err;
  }
  const long long nrep = (long long)E * NT;
  const long long nq = (long long)tiles * ((NKP + kQSteps - 1) / kQSteps);
  const long long ninit = combine ? (T + kQThreads - 1) / kQThreads : 0;
  hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)(nrep + nq + ninit)), dim3(kQThreads), panel_bytes, stream, scales,
                     E, N, K / 32, NT, NS, bsc, (int)nrep, x, x_per_slot, k, R, K, NKP, offsets, sorted_rows, aq, aqx,
                     as, aqf, (int)nq, ids, cnt, y);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // Eight waves (256-row tiles) halve the weight bytes per MFMA where the
  // experts hold enough rows to fill them, for the fp32 epilogue; four where
  // many experts hold fewer than 256 rows (an odd 128-row tile leaves half of
  // an eight-wave tile idle), and for the gated-activation and combine
  // epilogues, whose work the second workgroup on the CU overlaps.
  const int W = (act || combine) ? 4 : gemm_waves(E, R);
  const int TM = 32 * W;
  const long long tiles_max = ((long long)(R + TM - 1) / TM + (R < E ? R : E)) * NT;
  const long long grid = (tiles_max + kXcds - 1) / kXcds * kXcds;
  // the gpt-oss-20b widths (K = 2880) have 12 stages
  auto kern = act       ? (NS == 12 ? expert_gemm_kernel<12, kEpiSwiglu, 4> : expert_gemm_kernel<0, kEpiSwiglu, 4>)
              : combine ? (NS == 12 ? expert_gemm_kernel<12, kEpiCombine, 4> : expert_gemm_kernel<0, kEpiCombine, 4>)
              : W == 8  ? (NS == 12 ? expert_gemm_kernel<12, kEpiOut, 8> : expert_gemm_kernel<0, kEpiOut, 8>)
                        : (NS == 12 ? expert_gemm_kernel<12, kEpiOut, 4> : expert_gemm_kernel<0, kEpiOut, 4>);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(W * 64), 0, stream, blocks, bsc, bias, E, N, K, aq, aqx, as,
                     aqf, T, k, offsets, sorted_rows, out, act, ids, gates, cnt, y);
  return hipGetLastError();
}

}  // namespace mxfp4

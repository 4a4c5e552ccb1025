// Router top-k, softmax gates and stable grouping of the routed rows by
// expert, for gfx950.
//
// Routing follows the gpt-oss-20b files page, README "Dense routing" and
// src/experts.linnet fn ranks / route / experts_of / weights_of: an expert's
// rank counts the experts with a larger logit, or an equal logit and a lower
// index; the k best are kept highest first; the router weights are the
// softmax over the kept logits.  Grouping (README "Loading": the tokens each
// expert was chosen for, sorted by expert) is a stable counting sort of the
// rows r = t * k + s.
//
// Routing: one wave per token.  Lane e holds expert e's logit (lane e + 64 i
// for more than 64 experts); every lane counts the experts that beat its own
// by broadcasting each logit in turn with v_readlane, so the rank definition
// above is evaluated directly and in parallel.  The lane whose rank is s
// writes slot s; the gates come from a wave max and a wave sum.
//
// Grouping (more than 64 rows): workgroup c of 16 waves places the rows of
// its 1024-row chunk.  Every workgroup reads all ids; per 64-row tile a ballot
// per id bit gives each lane the mask of lanes sharing its expert, and the
// lowest such lane adds the count into its wave's LDS counters (all rows,
// rows before the chunk, the wave's own chunk tile).  An exclusive scan over
// experts gives the offsets; the counts before the chunk and of the chunk's
// lower waves give each wave's bases; row r goes to base + (peers below it).
// Tiles are ranked by index and lanes within a tile too, so each expert's
// rows come out in ascending order.
//
// Tiny batches (T * k <= 64) route and group in a single workgroup, the
// grouping in one wave without LDS counters.  Larger batches route with many
// workgroups (a token per wave) and then group with ceil(T * k / 1024)
// workgroups.  A row whose given id is out of range is written as -1 and left
// out of the grouping; a repeated given id is flagged to the grouping pass in
// bit 30 of the id (cleared again there).

#include "kernels.h"
#include "common.h"
#include "mxfp4_moe.h"
#include "route_common.h"
#include <math.h>

namespace mxfp4 {
namespace {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kTilesPerLoad = 16;       // 64-row tiles whose ids a wave loads at once
constexpr int kExpertChunks = 8;        // 64 experts per lane chunk: E <= 512
constexpr int kRouteThreads = 256;      // multi-workgroup routing: 4 waves, 4 tokens per wave
constexpr int kTokensPerRouteWave = 4;
constexpr int kMaxRouteE = MXFP4_MAX_EXPERTS;
constexpr int kMaxRouteK = MXFP4_MAX_TOPK;


// Grouping of the R = T * k routed rows by G workgroups of 16 waves.
// Workgroup c places the rows of its chunk [c * kChunk, (c + 1) * kChunk)
// (wave w: the chunk's 64-row tile w).  Every workgroup reads all R ids
// (wave w: tiles w, w + 16, ...): the per-expert totals give the offsets (the
// exclusive scan), the counts in tiles before the chunk and in the chunk's
// tiles of lower waves give each expert's base for this wave's rows; a lane's
// place is then that base plus the lanes below it with the same id (one
// ballot per id bit).  Rows are placed in ascending order within an expert,
// so the result is the stable counting sort.  Workgroup 0 writes the offsets.
// A chunk's owner alone inspects its rows for errors (a -1 or an id >= E, a
// repeat flag), before it clears their repeat flags, and ORs what it found
// into the error word, which the routing launch zeroed.
constexpr int kChunk = kGroupThreads;

__global__ __launch_bounds__(kGroupThreads) void group_kernel(int32_t* __restrict__ topk_ids, int R, int E,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_rows,
                                                              int32_t* __restrict__ error_word) {
  extern __shared__ int lds[];
  int* cnt_all = lds;                          // [waves][E]: rows per expert (all tiles of the wave)
  int* cnt_pre = cnt_all + kGroupWaves * E;    // [waves][E]: rows per expert in tiles before the chunk
  int* cnt_own = cnt_pre + kGroupWaves * E;    // [waves][E]: rows per expert in the wave's chunk tile
  int* base = cnt_own + kGroupWaves * E;       // [E]
  __shared__ int err_sh;  // error bits found in this workgroup's chunk
  __shared__ int total_sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < 3 * kGroupWaves * E; i += kGroupThreads) lds[i] = 0;
  if (tid == 0) err_sh = 0;
  __syncthreads();
  int ebits = 1;
  while ((1 << ebits) < E) ebits++;
  const int tiles = (R + 63) >> 6;
  const int own_tile = (int)blockIdx.x * kGroupWaves + wave;  // this wave's chunk tile
  int errbits = 0;

  // the lanes of a tile whose rows share this lane's expert e (-1: no expert)
  auto peers_of = [&](int e) {
    const bool valid = e >= 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < ebits; b++) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    return peers;
  };

  // ---- counts over every tile (waves take tiles w, w + 16, ...)
  for (int t0 = wave; t0 < tiles; t0 += kGroupWaves * kTilesPerLoad) {
    int ev[kTilesPerLoad];
#pragma unroll
    for (int i = 0; i < kTilesPerLoad; i++) {
      const int r = (t0 + i * kGroupWaves) * 64 + lane;
      ev[i] = topk_ids[min(r, R - 1)];  // unconditional load, masked below
      if (r >= R) ev[i] = -1;
    }
#pragma unroll
    for (int i = 0; i < kTilesPerLoad; i++) {
      const int t = t0 + i * kGroupWaves;
      if (t >= tiles) break;  // wave-uniform
      const int r = t * 64 + lane;
      int e = ev[i];
      const bool dup = e >= 0 && (e & kDupFlag);
      if (dup) e &= ~kDupFlag;
      if (e >= E) e = -1;  // never written by the routing: counted as out of range
      if (t == own_tile && r < R) {
        // the chunk's owner: its rows' errors, then the repeat flags cleared
        if (e < 0) errbits |= MXFP4_ROUTE_ERR_ID_RANGE;
        if (dup) {
          errbits |= MXFP4_ROUTE_ERR_ID_DUP;
          topk_ids[r] = e;
        }
      }
      // counts only (their order is irrelevant): one LDS atomic per row into
      // the wave's own counters; the scatter below finds each row's place
      if (e >= 0) {
        atomicAdd(&cnt_all[wave * E + e], 1);
        if (t < (int)blockIdx.x * kGroupWaves) atomicAdd(&cnt_pre[wave * E + e], 1);
        if (t == own_tile) atomicAdd(&cnt_own[wave * E + e], 1);
      }
    }
  }
  if (errbits) atomicOr(&err_sh, errbits);
  __syncthreads();

  // ---- offsets (exclusive scan of the totals) and this chunk's bases
  if (wave == 0) {
    int carry = 0;
    for (int c0 = 0; c0 < E; c0 += 64) {
      const int e = c0 + lane;
      int tot = 0, pre = 0;
      if (e < E)
        for (int w = 0; w < kGroupWaves; w++) {
          tot += cnt_all[w * E + e];
          pre += cnt_pre[w * E + e];
        }
      int inc = tot;
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
      }
      if (e < E) {
        const int start = carry + inc - tot;
        base[e] = start + pre;
        if (blockIdx.x == 0) offsets[e] = start;
      }
      carry += __shfl(inc, 63, 64);
    }
    if (lane == 0) total_sh = carry;
  }
  __syncthreads();
  if (tid == 0) {
    if (blockIdx.x == 0) offsets[E] = total_sh;
    if (error_word && err_sh) atomicOr(error_word, err_sh);
  }
  // per wave: the base of its chunk tile's rows of expert e (the chunk's lower waves first)
  for (int e = tid; e < E; e += kGroupThreads) {
    int b = base[e];
    for (int w = 0; w < kGroupWaves; w++) {
      const int c = cnt_own[w * E + e];
      cnt_own[w * E + e] = b;
      b += c;
    }
  }
  __syncthreads();

  // ---- stable scatter of this wave's chunk tile
  if (own_tile < tiles) {
    const int r = own_tile * 64 + lane;
    int e = r < R ? topk_ids[r] : -1;  // flag cleared above by this wave (program order)
    if (e >= 0) e &= ~kDupFlag;
    if (e >= E) e = -1;
    const uint64_t peers = peers_of(e);
    if (e >= 0) sorted_rows[cnt_own[wave * E + e] + lanes_below(peers)] = r;
  }
}

// T * k <= 64: up to 16 waves route a token each, then one wave groups the
// rows without LDS counters or further barriers: lane r holds row r's id;
// offsets[e] counts the valid rows with an id below e, and row r goes to the
// rows with a smaller id plus the rows before it with the same id (the
// grouping's definition, evaluated directly with v_readlane broadcasts).
template <int EC>
__global__ __launch_bounds__(kGroupThreads) void route_group_tiny_kernel(
    const uint16_t* __restrict__ logits, const int32_t* __restrict__ ids_in, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ gates, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_rows, int32_t* __restrict__ error_word) {
  __shared__ int ids_lds[64];
  __shared__ int err_lds[kGroupWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  int errbits = 0;
  for (int t0 = wave; t0 < T; t0 += kRouteBatch * nwaves)
    errbits |= route_tokens<EC, kRouteBatch>(logits, ids_in, t0, nwaves, T, E, k, lane, topk_ids, gates, ids_lds);
  if (lane == 0) err_lds[wave] = errbits;
  __syncthreads();
  if (wave != 0) return;
  const int R = T * k;
  int err = 0;
  for (int w = 0; w < nwaves; w++) err |= err_lds[w];
  int id = lane < R ? ids_lds[lane] : -1;
  if (lane < R && id >= 0 && (id & kDupFlag)) {
    id &= ~kDupFlag;
    topk_ids[lane] = id;
    err |= MXFP4_ROUTE_ERR_ID_DUP;
  }
  if (id >= E) id = -1;  // never written by the routing: counted as out of range
  if (lane < R && id < 0) err |= MXFP4_ROUTE_ERR_ID_RANGE;
  err = (__ballot(err & MXFP4_ROUTE_ERR_ID_RANGE) ? MXFP4_ROUTE_ERR_ID_RANGE : 0) |
        (__ballot(err & MXFP4_ROUTE_ERR_ID_DUP) ? MXFP4_ROUTE_ERR_ID_DUP : 0);
  for (int c0 = 0; c0 <= E; c0 += 64) {
    const int e = c0 + lane;
    int cnt = 0;
    for (int r = 0; r < R; r++) {
      const int ir = __builtin_amdgcn_readlane(id, r);
      cnt += (ir >= 0 && ir < e) ? 1 : 0;
    }
    if (e <= E) offsets[e] = cnt;
  }
  int before = 0;
  for (int r = 0; r < R; r++) {
    const int ir = __builtin_amdgcn_readlane(id, r);
    before += (ir >= 0 && (ir < id || (ir == id && r < lane))) ? 1 : 0;
  }
  if (lane < R && id >= 0) sorted_rows[before] = lane;
  if (lane == 0 && error_word) *error_word = err;
}

// R > 64, first launch: routing, NB tokens per wave, many workgroups; the
// first thread zeroes the error word the grouping launch ORs its findings into
// (the routing's own errors reach the grouping through the ids it writes).
template <int EC, int NB>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const uint16_t* __restrict__ logits,
                                                             const int32_t* __restrict__ ids_in, int T, int E,
                                                             int k, int32_t* __restrict__ topk_ids,
                                                             float* __restrict__ gates, int32_t* __restrict__ error_word) {
  const int lane = threadIdx.x & 63;
  const int w = (blockIdx.x * kRouteThreads + threadIdx.x) >> 6;
  if (error_word && blockIdx.x == 0 && threadIdx.x == 0) *error_word = 0;
  route_tokens<EC, NB>(logits, ids_in, w * NB, 1, T, E, k, lane, topk_ids, gates, nullptr);
}

template <int EC>
hipError_t launch_ec(const uint16_t* logits, const int32_t* ids_in, int T, int E, int k, int32_t* topk_ids,
                     float* gates, int32_t* offsets, int32_t* sorted_rows, int32_t* error_word, hipStream_t stream) {
  if ((long long)T * k <= 64) {
    const int waves = T < 1 ? 1 : (T < kGroupWaves ? T : kGroupWaves);  // T = 0 still writes the zero offsets
    hipLaunchKernelGGL(route_group_tiny_kernel<EC>, dim3(1), dim3(64 * waves), 0, stream, logits, ids_in, T, E, k,
                       topk_ids, gates, offsets, sorted_rows, error_word);
    return hipGetLastError();
  }
  // one token per wave while that fills the chip, four beyond
  const bool one = T <= 16384;
  const int per_block = (kRouteThreads / 64) * (one ? 1 : kTokensPerRouteWave);
  const dim3 rgrid((T + per_block - 1) / per_block);
  if (one)
    hipLaunchKernelGGL((route_kernel<EC, 1>), rgrid, dim3(kRouteThreads), 0, stream, logits, ids_in, T, E, k, topk_ids,
                       gates, error_word);
  else
    hipLaunchKernelGGL((route_kernel<EC, kTokensPerRouteWave>), rgrid, dim3(kRouteThreads), 0, stream, logits,
                       ids_in, T, E, k, topk_ids, gates, error_word);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t glds = ((size_t)3 * kGroupWaves * E + E) * sizeof(int);
  // up to 3 * 16 * 512 + 512 ints: above 64 KB the dynamic LDS limit is raised
  static DynLdsLimit group_lds(reinterpret_cast<const void*>(&group_kernel),
                               (int)((3 * kGroupWaves + 1) * kMaxRouteE * sizeof(int)));
  if (glds > 65536) {
    err = group_lds.ensure();
    if (err != hipSuccess) return err;
  }
  const long long R = (long long)T * k;
  hipLaunchKernelGGL(group_kernel, dim3((unsigned)((R + kChunk - 1) / kChunk)), dim3(kGroupThreads), glds, stream,
                     topk_ids, (int)R, E, offsets, sorted_rows, error_word);
  return hipGetLastError();
}

// Dense router weights (src/experts.linnet fn route, README "Dense routing"):
// one wave per token ranks its logits as above, floors every expert ranked k
// or worse to -1e30 and takes the softmax over all E, whose floored entries
// are exactly zero, so the kept ones equal the gates of the sparse routing.
template <int EC>
__global__ __launch_bounds__(kRouteThreads) void dense_route_kernel(const uint16_t* __restrict__ logits, int T, int E,
                                                                   int k, float* __restrict__ probs) {
  const int lane = threadIdx.x & 63;
  const int t = (blockIdx.x * kRouteThreads + threadIdx.x) >> 6;
  if (t >= T) return;  // whole waves
  const uint16_t* lrow = logits + (size_t)t * E;
  float l[EC];
  int rank[EC];
#pragma unroll
  for (int i = 0; i < EC; i++) {
    const int e = lane + 64 * i;
    l[i] = bf16_bits_to_f32(lrow[min(e, E - 1)]);
    if (e >= E) l[i] = -INFINITY;
    rank[i] = 0;
  }
#pragma unroll
  for (int jc = 0; jc < EC; jc++) {
    const int jn = min(64, E - 64 * jc);
    for (int jj = 0; jj < jn; jj++) {
      const float lj = readlane_f(l[jc], jj);
      const int j = 64 * jc + jj;
#pragma unroll
      for (int i = 0; i < EC; i++) {
        const int e = lane + 64 * i;
        rank[i] += (lj > l[i] || (lj == l[i] && j < e)) ? 1 : 0;
      }
    }
  }
  // the largest kept logit (rank 0) is the softmax's maximum
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < EC; i++) {
    const uint64_t m = __ballot(lane + 64 * i < E && rank[i] == 0);
    if (m) mx = readlane_f(l[i], __ffsll((long long)m) - 1);
  }
  float num[EC];
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < EC; i++) {
    const int e = lane + 64 * i;
    // floored logits: exp(-1e30 - mx) is exactly 0 in fp32
    num[i] = (e < E && rank[i] < k) ? expf(l[i] - mx) : 0.f;
    part += num[i];
  }
  const float sum = wave_sum(part);
#pragma unroll
  for (int i = 0; i < EC; i++) {
    const int e = lane + 64 * i;
    if (e < E) probs[(size_t)t * E + e] = num[i] / sum;
  }
}

}  // namespace

hipError_t launch_dense_route(const uint16_t* logits, int T, int E, int k, float* probs, hipStream_t stream) {
  const dim3 grid((T + kRouteThreads / 64 - 1) / (kRouteThreads / 64));
  if (E <= 64)
    hipLaunchKernelGGL(dense_route_kernel<1>, grid, dim3(kRouteThreads), 0, stream, logits, T, E, k, probs);
  else if (E <= 128)
    hipLaunchKernelGGL(dense_route_kernel<2>, grid, dim3(kRouteThreads), 0, stream, logits, T, E, k, probs);
  else
    hipLaunchKernelGGL(dense_route_kernel<kExpertChunks>, grid, dim3(kRouteThreads), 0, stream, logits, T, E, k,
                       probs);
  return hipGetLastError();
}

hipError_t launch_route_group(const uint16_t* logits, const int32_t* ids_in, int T, int E, int k,
                              int32_t* topk_ids, float* gates, int32_t* offsets, int32_t* sorted_rows,
                              int32_t* error_word, hipStream_t stream) {
  if (E <= 64)
    return launch_ec<1>(logits, ids_in, T, E, k, topk_ids, gates, offsets, sorted_rows, error_word, stream);
  if (E <= 128)
    return launch_ec<2>(logits, ids_in, T, E, k, topk_ids, gates, offsets, sorted_rows, error_word, stream);
  return launch_ec<kExpertChunks>(logits, ids_in, T, E, k, topk_ids, gates, offsets, sorted_rows, error_word,
                                  stream);
}

}  // namespace mxfp4

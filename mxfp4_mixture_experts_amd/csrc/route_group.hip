// Router top-k, softmax gates and stable grouping of the routed rows by
// expert, in one single-workgroup kernel for gfx950.
//
// Routing follows the gpt-oss-20b files page, README "Dense routing" and
// src/experts.linnet fn ranks / route / experts_of / weights_of: an expert's
// rank counts the experts with a larger logit, or an equal logit and a lower
// index; the k best are kept highest first; the router weights are the
// softmax over the kept logits.  Grouping (README "Loading": the tokens each
// expert was chosen for, sorted by expert) is a stable counting sort of the
// rows r = t * k + s.
//
// Layout of the work inside the one workgroup of 1024 threads (16 waves):
//   phase 1  one thread per token: k selection passes over its E logits,
//            each pass taking the best expert that comes after the previous
//            pick in (logit desc, index asc) order -- O(k * E), no sort state;
//   phase 2  each wave owns a contiguous range of rows and counts, per
//            64-row tile, the lanes sharing an expert (a ballot per id bit
//            gives each lane the mask of its peers); the tile's leader lane
//            adds the count into the wave's LDS counter of that expert;
//   phase 3  per expert, the wave counters become running bases: expert start
//            (exclusive scan over experts) plus the counts of earlier waves;
//   phase 4  each wave walks its tiles again in order and scatters row r to
//            base + (peers below it); the leader then advances the base.
// Because waves own contiguous row ranges in order and lanes are ranked by
// lane index, the rows of each expert come out in ascending order.

#include "kernels.h"
#include "common.h"
#include <math.h>

namespace mxfp4 {
namespace {

constexpr int kRgThreads = 1024;
constexpr int kRgWaves = kRgThreads / 64;

__device__ __forceinline__ float logit_at(const uint16_t* row, int e) {
  return bf16_bits_to_f32(row[e]);
}

// gates over the k logits at ids[0..k) of one token (all ids valid)
__device__ void write_gates(const uint16_t* lrow, const int32_t* ids, int k, float* g) {
  float mx = -INFINITY;
  for (int s = 0; s < k; s++) mx = fmaxf(mx, logit_at(lrow, ids[s]));
  float sum = 0.f;
  for (int s = 0; s < k; s++) sum += expf(logit_at(lrow, ids[s]) - mx);
  for (int s = 0; s < k; s++) g[s] = expf(logit_at(lrow, ids[s]) - mx) / sum;
}

__global__ __launch_bounds__(kRgThreads) void route_group_kernel(
    const uint16_t* __restrict__ logits, const int32_t* __restrict__ ids_in, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ gates, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_rows, int32_t* __restrict__ error_word) {
  extern __shared__ int lds[];
  int* cnt = lds;                       // [kRgWaves][E] counters, later running bases
  int* start = lds + kRgWaves * E;      // [E] expert start offsets
  __shared__ int err_sh;
  __shared__ int total_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int i = tid; i < kRgWaves * E; i += kRgThreads) cnt[i] = 0;
  if (tid == 0) err_sh = 0;
  __syncthreads();

  // ---------------- phase 1: routing, one thread per token
  int errbits = 0;
  for (int t = tid; t < T; t += kRgThreads) {
    int32_t* ids = topk_ids + (size_t)t * k;
    const uint16_t* lrow = logits ? logits + (size_t)t * E : nullptr;
    bool all_valid = true;
    if (ids_in) {
      const int32_t* given = ids_in + (size_t)t * k;
      for (int s = 0; s < k; s++) {
        int e = given[s];
        if ((unsigned)e >= (unsigned)E) {
          errbits |= 1;
          all_valid = false;
          e = -1;
        } else {
          for (int s2 = 0; s2 < s; s2++)
            if (given[s2] == e) errbits |= 2;
        }
        ids[s] = e;
      }
    } else {
      float prev_l = INFINITY;
      int prev_e = -1;
      for (int s = 0; s < k; s++) {
        float best_l = -INFINITY;
        int best_e = -1;
        for (int e = 0; e < E; e++) {
          const float l = logit_at(lrow, e);
          const bool after_prev = (l < prev_l) || (l == prev_l && e > prev_e);
          const bool better = (best_e < 0) || (l > best_l);  // equal: keep the lower index
          if (after_prev && better) {
            best_l = l;
            best_e = e;
          }
        }
        if (best_e < 0) {
          errbits |= 1;
          all_valid = false;
        }
        ids[s] = best_e;
        prev_l = best_l;
        prev_e = best_e;
      }
    }
    if (gates && lrow && all_valid) write_gates(lrow, ids, k, gates + (size_t)t * k);
  }
  if (errbits) atomicOr(&err_sh, errbits);
  __syncthreads();  // topk_ids of every token visible to the whole workgroup

  // ---------------- phase 2: per-wave, per-expert counts
  const int R = T * k;
  int ebits = 1;
  while ((1 << ebits) < E) ebits++;
  const int per_wave = ((R + kRgWaves * 64 - 1) / (kRgWaves * 64)) * 64;
  const int w_begin = min(R, wave * per_wave);
  const int w_end = min(R, w_begin + per_wave);

  for (int base = w_begin; base < w_end; base += 64) {
    const int r = base + lane;
    const int e = (r < w_end) ? topk_ids[r] : -1;
    const bool valid = e >= 0;
    uint64_t peers = wave_ballot(valid);
    for (int b = 0; b < ebits; b++) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = wave_ballot(bit);
      peers &= bit ? m : ~m;
    }
    if (valid && lanes_below(peers) == 0) cnt[wave * E + e] += __popcll(peers);
  }
  __syncthreads();

  // ---------------- phase 3: expert starts and per-wave running bases
  if (wave == 0) {
    int carry = 0;
    for (int c0 = 0; c0 < E; c0 += 64) {
      const int e = c0 + lane;
      int tot = 0;
      if (e < E)
        for (int w = 0; w < kRgWaves; w++) tot += cnt[w * E + e];
      // inclusive scan over the 64 lanes
      int inc = tot;
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
      }
      if (e < E) start[e] = carry + inc - tot;
      carry += __shfl(inc, 63, 64);
    }
    if (lane == 0) total_sh = carry;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRgThreads) {
    int b = start[e];
    offsets[e] = b;
    for (int w = 0; w < kRgWaves; w++) {
      const int c = cnt[w * E + e];
      cnt[w * E + e] = b;
      b += c;
    }
  }
  if (tid == 0) {
    offsets[E] = total_sh;
    if (error_word) *error_word = err_sh;
  }
  __syncthreads();

  // ---------------- phase 4: stable scatter
  for (int base = w_begin; base < w_end; base += 64) {
    const int r = base + lane;
    const int e = (r < w_end) ? topk_ids[r] : -1;
    const bool valid = e >= 0;
    uint64_t peers = wave_ballot(valid);
    for (int b = 0; b < ebits; b++) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = wave_ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int below = lanes_below(peers);
    int pos = 0;
    if (valid) pos = cnt[wave * E + e] + below;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      sorted_rows[pos] = r;
      if (below == 0) cnt[wave * E + e] = pos + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_route_group(const uint16_t* logits, const int32_t* ids_in, int T, int E, int k,
                              int32_t* topk_ids, float* gates, int32_t* offsets, int32_t* sorted_rows,
                              int32_t* error_word, hipStream_t stream) {
  const size_t lds_bytes = (size_t)(kRgWaves + 1) * E * sizeof(int);
  hipLaunchKernelGGL(route_group_kernel, dim3(1), dim3(kRgThreads), lds_bytes, stream, logits, ids_in,
                     T, E, k, topk_ids, gates, offsets, sorted_rows, error_word);
  return hipGetLastError();
}

}  // namespace mxfp4

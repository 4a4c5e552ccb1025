// Routing of one token per wave, shared by the routing launches and the
// decode kernels that route their tokens themselves (gpt-oss-20b files page,
// README "Dense routing"; src/experts.linnet fn ranks / route / experts_of /
// weights_of): an expert's rank counts the experts with a larger logit, or an
// equal logit and a lower index; the k best are kept highest first; the router
// weights are the softmax over the kept logits.
#pragma once

#include <math.h>

#include "common.h"
#include "mxfp4_moe.h"

namespace mxfp4 {
namespace {

// a repeated given id, flagged in bit 30 of the id for the grouping pass
constexpr int32_t kDupFlag = 1 << 30;
// tokens a wave routes per batch
constexpr int kRouteBatch = 4;

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Token t with given expert ids: lane s < k holds the id e of slot s and, for
// the gates, the logit at e (lg).  Checks range and repeats, writes the ids
// (a repeat flagged in bit 30 for the grouping; an id out of range as -1) and
// the softmax over the logits of the slots in range (gate 0 for the others).
// Returns MXFP4_ROUTE_ERR_* bits (same on all lanes).
__device__ __forceinline__ int route_given(int e, float lg, int t, int E, int k, int lane, int32_t* __restrict__ topk_ids,
                           float* __restrict__ gates, bool with_gates, int32_t* ids_copy) {
  int32_t* ids = topk_ids + (size_t)t * k;
  int32_t* idc = ids_copy ? ids_copy + t * k : nullptr;  // the grouping's copy (LDS), if any
  const bool in_range = lane < k && (unsigned)e < (unsigned)E;
  bool dup = false;
  for (int j = 0; j < k; j++) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    dup |= (lane < k && j != lane && ej == e && in_range);
  }
  const uint64_t bad = __ballot(lane < k && !in_range);
  const uint64_t dups = __ballot(dup);
  const int idv = in_range ? (e | (dup ? kDupFlag : 0)) : -1;
  if (lane < k) {
    ids[lane] = idv;
    if (idc) idc[lane] = idv;
  }
  if (with_gates) {
    // softmax over the logits of the slots with an id in range; 0 for the others
    const float l = in_range ? lg : -INFINITY;
    const float mx = wave_max(l);
    const float num = in_range ? expf(l - mx) : 0.f;
    const float sum = wave_sum(num);
    if (lane < k) gates[(size_t)t * k + lane] = in_range ? num / sum : 0.f;
  }
  return (bad ? MXFP4_ROUTE_ERR_ID_RANGE : 0) | (dups ? MXFP4_ROUTE_ERR_ID_DUP : 0);
}

// Token t routed from its logits l (lane e + 64 i holds expert e + 64 i's
// logit, -inf past E); returns MXFP4_ROUTE_ERR_* bits (same on all lanes).
template <int EC>
__device__ __forceinline__ int route_ranked(const float (&l)[EC], int t, int E, int k, int lane, int32_t* __restrict__ topk_ids,
                            float* __restrict__ gates, int32_t* ids_copy) {
  int32_t* ids = topk_ids + (size_t)t * k;
  int32_t* idc = ids_copy ? ids_copy + t * k : nullptr;
  int rank[EC];
#pragma unroll
  for (int i = 0; i < EC; i++) rank[i] = 0;
  // rank[e] = #{j : l_j > l_e or (l_j == l_e and j < e)}
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
  // Logits without NaN rank the experts 0 .. E - 1, each rank once.  A NaN
  // compares false both ways, so it would rank 0 beside the largest logit and
  // break that: a token with a NaN logit gets id -1 and gate 0 in every slot
  // (its rows are left out of the grouping).
  bool has_nan = false;
#pragma unroll
  for (int i = 0; i < EC; i++) has_nan |= __ballot(lane + 64 * i < E && l[i] != l[i]) != 0;
  if (has_nan) {
    if (lane < k) {
      ids[lane] = -1;
      if (idc) idc[lane] = -1;
      if (gates) gates[(size_t)t * k + lane] = 0.f;
    }
    return MXFP4_ROUTE_ERR_ID_RANGE;
  }
  // slot s <- the expert of rank s; the largest kept logit has rank 0
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < EC; i++) {
    const int e = lane + 64 * i;
    const bool top = e < E && rank[i] == 0;
    const uint64_t m = __ballot(top);
    if (m) mx = readlane_f(l[i], __ffsll((long long)m) - 1);
  }
  float num[EC];
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < EC; i++) {
    const int e = lane + 64 * i;
    const bool kept = e < E && rank[i] < k;
    num[i] = kept ? expf(l[i] - mx) : 0.f;
    part += num[i];
    if (kept) {
      ids[rank[i]] = e;
      if (idc) idc[rank[i]] = e;
    }
  }
  if (gates) {
    const float sum = wave_sum(part);
#pragma unroll
    for (int i = 0; i < EC; i++) {
      const int e = lane + 64 * i;
      if (e < E && rank[i] < k) gates[(size_t)t * k + rank[i]] = num[i] / sum;
    }
  }
  return 0;
}

// Route the NB tokens t0 + stride * b (b < NB; those past T are skipped) with
// the calling wave.  Every load of the batch is issued before any token is
// ranked (tokens past T re-read token T - 1), so the batch pays one memory
// round trip (two with given ids and gates: the ids, then their logits).
template <int EC, int NB>
__device__ __forceinline__ int route_tokens(const uint16_t* __restrict__ logits, const int32_t* __restrict__ ids_in, int t0,
                            int stride, int T, int E, int k, int lane, int32_t* __restrict__ topk_ids,
                            float* __restrict__ gates, int32_t* ids_copy) {
  int err = 0;
  if (ids_in) {
    int e[NB];
    float lg[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const int tc = min(t0 + stride * b, T - 1);
      e[b] = ids_in[(size_t)tc * k + min(lane, k - 1)];
      if (lane >= k) e[b] = -1;
    }
    const bool with_gates = gates && logits;
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const int tc = min(t0 + stride * b, T - 1);
      lg[b] = with_gates ? bf16_bits_to_f32(logits[(size_t)tc * E + ((unsigned)e[b] < (unsigned)E ? e[b] : 0)]) : 0.f;
    }
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const int t = t0 + stride * b;
      if (t < T) err |= route_given(e[b], lg[b], t, E, k, lane, topk_ids, gates, with_gates, ids_copy);
    }
    return err;
  }
  float l[NB][EC];
#pragma unroll
  for (int b = 0; b < NB; b++) {
    const uint16_t* lrow = logits + (size_t)min(t0 + stride * b, T - 1) * E;
#pragma unroll
    for (int i = 0; i < EC; i++) {
      const int e = lane + 64 * i;
      l[b][i] = bf16_bits_to_f32(lrow[min(e, E - 1)]);  // unconditional load: no branch per load
      if (e >= E) l[b][i] = -INFINITY;
    }
  }
#pragma unroll
  for (int b = 0; b < NB; b++) {
    const int t = t0 + stride * b;
    if (t < T) err |= route_ranked<EC>(l[b], t, E, k, lane, topk_ids, gates, ids_copy);
  }
  return err;
}

}  // namespace
}  // namespace mxfp4

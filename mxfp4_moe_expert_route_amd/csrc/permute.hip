// Token-to-expert permutation: counts, offsets, sorted pair lists.
//
// Not on the pages; it is the bookkeeping a grouped expert computation needs.
// Definition: pair p = t*k + j; counts[e] pairs per expert; offsets is the
// exclusive prefix sum; sorted_pairs holds each expert's pairs in ascending p;
// pair_to_row is the inverse.
//
// Ids outside [0, E) are dropped (pair_to_row = -1, not counted) so that bad
// input cannot send a store out of bounds.
//
// One workgroup of 16 waves.  Wave w owns a contiguous range of pairs.
//  1. per-wave histograms in LDS (integer atomics: order-free, deterministic)
//  2. per-expert exclusive bases across waves, block scan over experts
//  3. each wave walks its range 64 pairs at a time; a pair's rank among the
//     earlier pairs of its expert in the same 64 comes from a ballot-based
//     match (one ballot per bit of the expert id), so the scatter is stable
//     without sorting.  The ids of 8 such groups are loaded at once, so the
//     walk pays one memory latency per 512 pairs.
#include "common.hpp"

namespace mxm {
namespace {

constexpr int kPermWaves = 16;
constexpr int kBatch = 8;                     // 64-pair groups whose ids load together
constexpr int kPermThreads = kPermWaves * kWave;

__global__ __launch_bounds__(kPermThreads) void k_permute(const int32_t* __restrict__ ids, int R,
                                                          int E, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_to_row) {
  extern __shared__ int32_t smem[];
  int32_t* hist = smem;                       // [kPermWaves][E]
  int32_t* tot = smem + kPermWaves * E;       // [E]
  __shared__ int32_t wave_sum[kPermWaves];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();

  for (int i = tid; i < kPermWaves * E; i += kPermThreads) hist[i] = 0;
  __syncthreads();

  const int per = (R + kPermWaves - 1) / kPermWaves;
  const int beg = min(R, wave * per);
  const int end = min(R, beg + per);
  int32_t* my_hist = hist + wave * E;
  for (int p = beg + lane; p < end; p += kWave) {
    const int key = ids[p];
    if (unsigned(key) < unsigned(E)) atomicAdd(&my_hist[key], 1);
  }
  __syncthreads();

  // 2a. exclusive base of each wave within each expert; totals
  for (int e = tid; e < E; e += kPermThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    tot[e] = run;
    counts[e] = run;
  }
  __syncthreads();

  // 2b. exclusive scan of the totals over experts (each thread: 2 experts)
  const int e0 = 2 * tid;
  const int v0 = (e0 < E) ? tot[e0] : 0;
  const int v1 = (e0 + 1 < E) ? tot[e0 + 1] : 0;
  const int s = v0 + v1;
  const int incl = wave_incl_scan(s);
  if (lane == kWave - 1) wave_sum[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += wave_sum[w];
  const int ex0 = wbase + incl - s;
  if (e0 < E) {
    offsets[e0] = ex0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) hist[w * E + e0] += ex0;
  }
  if (e0 + 1 < E) {
    offsets[e0 + 1] = ex0 + v0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) hist[w * E + e0 + 1] += ex0 + v0;
  }
  if (tid == 0) {
    int total = 0;
    for (int w = 0; w < kPermWaves; ++w) total += wave_sum[w];
    offsets[E] = total;                       // == R when every id is in range
  }
  __syncthreads();

  // 3. stable scatter; my_hist[e] is the next free row of expert e for this wave
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int c0 = beg; c0 < end; c0 += kBatch * kWave) {
    int raw[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = c0 + i * kWave + lane;
      raw[i] = (p < end) ? ids[p] : 0;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = c0 + i * kWave + lane;
      const bool valid = (p < end) && unsigned(raw[i]) < unsigned(E);
      const int key = valid ? raw[i] : 0;
      if (p < end && !valid) pair_to_row[p] = -1;   // out-of-range id: pair dropped
      unsigned long long m = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const unsigned long long bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
      }
      if (valid) {
        const int rank = __popcll(m & lt);
        const int pos = my_hist[key] + rank;
        sorted_pairs[pos] = p;
        pair_to_row[p] = pos;
        if ((m >> lane) == 1ull) my_hist[key] += __popcll(m);   // last lane of its expert
      }
    }
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_to_row,
                          hipStream_t s) {
  const int R = T * k;
  const size_t lds = size_t(kPermWaves + 1) * E * sizeof(int32_t);
  static bool attr_set = false;
  if (!attr_set) {                // E up to 1024: more than the default 64 KB
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_permute),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             int((kPermWaves + 1) * 1024 * sizeof(int32_t)));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  k_permute<<<1, kPermThreads, lds, s>>>(ids, R, E, counts, offsets, sorted_pairs, pair_to_row);
  return hipGetLastError();
}

}  // namespace mxm

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
// One workgroup of NW waves (4 for up to 1024 pairs, else 16); the first
// nw = min(NW, ceil(R / 256)) own contiguous ranges of pairs.
//  1. per-wave histograms in LDS (integer atomics: order-free, deterministic)
//  2. per-expert exclusive bases across waves, block scan over experts
//  3. each wave walks its range 64 pairs at a time; a pair's rank among the
//     earlier pairs of its expert in the same 64 comes from a ballot-based
//     match (one ballot per bit of the expert id), so the scatter is stable
//     without sorting.
// Ids are loaded 8 groups of 64 at a time; a range of at most 512 pairs (all
// of them up to 4096 pairs) stays in registers from the histogram to the
// scatter, so a small call pays one memory latency for its ids.
#include "common.hpp"

namespace mxm {
namespace {

constexpr int kBatch = 8;                     // 64-pair groups whose ids load together

template <int NW>
__global__ __launch_bounds__(NW * kWave) void k_permute(const int32_t* __restrict__ ids, int R,
                                                        int E, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_pairs,
                                                        int32_t* __restrict__ pair_to_row) {
  constexpr int NT = NW * kWave;
  extern __shared__ int32_t smem[];
  int32_t* hist = smem;                       // [nw][E]
  int32_t* tot = smem + NW * E;               // [E]
  __shared__ int32_t wave_sum[NW];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();

  const int nw = min(NW, max(1, (R + 255) / 256));   // waves that walk pairs
  for (int i = tid; i < nw * E; i += NT) hist[i] = 0;
  __syncthreads();

  const int per = (R + nw - 1) / nw;
  const int beg = wave < nw ? min(R, wave * per) : R;
  const int end = wave < nw ? min(R, beg + per) : R;
  const bool kept = end - beg <= kBatch * kWave;     // the range fits one batch
  int32_t* my_hist = hist + wave * E;
  int raw[kBatch];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = c0 + i * kWave + lane;
      raw[i] = (p < end) ? ids[p] : -1;
    }
  };
  for (int c0 = beg; c0 < end; c0 += kBatch * kWave) {
    load_batch(c0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (unsigned(raw[i]) < unsigned(E)) atomicAdd(&my_hist[raw[i]], 1);
  }
  __syncthreads();

  // 2a. exclusive base of each wave within each expert; totals
  for (int e = tid; e < E; e += NT) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    tot[e] = run;
    counts[e] = run;
  }
  __syncthreads();

  // 2b. exclusive scan of the totals over experts (each thread: ept experts)
  const int ept = (E + NT - 1) / NT;
  const int e0 = tid * ept;
  int local = 0;
  for (int i = 0; i < ept; ++i)
    if (e0 + i < E) local += tot[e0 + i];
  const int incl = wave_incl_scan(local);
  if (lane == kWave - 1) wave_sum[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wave_sum[w];
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    offsets[e] = run;
    for (int w = 0; w < nw; ++w) hist[w * E + e] += run;
    run += tot[e];
  }
  if (tid == 0) {
    int total = 0;
    for (int w = 0; w < NW; ++w) total += wave_sum[w];
    offsets[E] = total;                       // == R when every id is in range
  }
  __syncthreads();

  // 3. stable scatter; my_hist[e] is the next free row of expert e for this wave
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int c0 = beg; c0 < end; c0 += kBatch * kWave) {
    if (!kept) load_batch(c0);
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
  if (R <= 1024) {                // 5 E ints: within the default 64 KB for E <= 1024
    k_permute<4><<<1, 4 * kWave, size_t(5) * E * sizeof(int32_t), s>>>(
        ids, R, E, counts, offsets, sorted_pairs, pair_to_row);
    return hipGetLastError();
  }
  static bool attr_set = false;
  if (!attr_set) {                // 17 E ints, E up to 1024: more than the default 64 KB
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_permute<16>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             int(17 * 1024 * sizeof(int32_t)));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  k_permute<16><<<1, 16 * kWave, size_t(17) * E * sizeof(int32_t), s>>>(
      ids, R, E, counts, offsets, sorted_pairs, pair_to_row);
  return hipGetLastError();
}

}  // namespace mxm

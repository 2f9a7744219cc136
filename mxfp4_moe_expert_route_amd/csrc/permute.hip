// Token-to-expert permutation: counts, offsets, sorted pair lists.  The
// algorithm is permute_block in routing.hpp; this file launches it as one
// workgroup of 4 waves (up to 1024 pairs) or 16 (up to 8192), and above that
// as one workgroup per range of pairs (three kernels, below).
#include "routing.hpp"

namespace mxm {
namespace {

template <int NW>
__global__ __launch_bounds__(NW * kWave) void k_permute(const int32_t* __restrict__ ids, int R,
                                                        int E, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_pairs,
                                                        int32_t* __restrict__ pair_to_row) {
  extern __shared__ int32_t smem[];
  __shared__ int32_t wave_sum[NW];
  permute_block<NW>(ids, 0, R, E, nullptr, counts, offsets, sorted_pairs, pair_to_row, smem,
                    wave_sum);
}

// Large batches: the pairs are cut into ranges of kRangePairs (more for very
// large R, so at most kMaxRanges ranges) handled by one workgroup each.
//  k_perm_hist     per-range expert histograms -> ws[range][E]
//  k_perm_scan     one workgroup: counts, offsets, and ws[range][e] replaced
//                  by the first row of expert e for that range (offsets[e]
//                  plus the counts of the earlier ranges)
//  k_perm_scatter  per range: permute_block from those bases
// Ranges, waves and lanes keep pair order, so the lists are the single
// workgroup's lists bit for bit.
constexpr int kRangePairs = 1024;
constexpr int kMaxRanges = 1024;
constexpr int kSingleMaxPairs = 8192;

__device__ __forceinline__ void range_of(int R, int nr, int b, int& r0, int& r1) {
  const int cb = (R + nr - 1) / nr;
  r0 = min(R, b * cb);
  r1 = min(R, r0 + cb);
}

__global__ __launch_bounds__(256) void k_perm_hist(const int32_t* __restrict__ ids, int R, int E,
                                                   int nr, int32_t* __restrict__ ws) {
  extern __shared__ int32_t hist[];
  int r0, r1;
  range_of(R, nr, blockIdx.x, r0, r1);
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  for (int p = r0 + threadIdx.x; p < r1; p += 256) {
    const int id = ids[p];
    if (unsigned(id) < unsigned(E)) atomicAdd(&hist[id], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) ws[size_t(blockIdx.x) * E + e] = hist[e];
}

// one thread per expert (E <= 1024); a thread's counts over the ranges are
// read 16 at a time, all loads of a batch in flight together
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(1024) void k_perm_scan(int E, int nr, int32_t* __restrict__ ws,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int32_t wave_tot[1024 / kWave];
  const int e = threadIdx.x, lane = lane_id(), wave = e / kWave;
  int total = 0;
  if (e < E)
    for (int b0 = 0; b0 < nr; b0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = b0 + i < nr ? ws[size_t(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) total += v[i];
    }
  const int incl = wave_incl_scan(total);
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - total, all = 0;
  for (int w = 0; w < 1024 / kWave; ++w) {
    run += w < wave ? wave_tot[w] : 0;
    all += wave_tot[w];
  }
  if (e < E) {
    counts[e] = total;
    offsets[e] = run;
    for (int b0 = 0; b0 < nr; b0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = b0 + i < nr ? ws[size_t(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (b0 + i < nr) ws[size_t(b0 + i) * E + e] = run;
        run += v[i];
      }
    }
  }
  if (e == 0) offsets[E] = all;
}

__global__ __launch_bounds__(4 * kWave) void k_perm_scatter(const int32_t* __restrict__ ids,
                                                            int R, int E, int nr,
                                                            const int32_t* __restrict__ ws,
                                                            int32_t* __restrict__ sorted_pairs,
                                                            int32_t* __restrict__ pair_to_row) {
  extern __shared__ int32_t smem[];
  __shared__ int32_t wave_sum[4];
  int r0, r1;
  range_of(R, nr, blockIdx.x, r0, r1);
  permute_block<4>(ids, r0, r1, E, ws + size_t(blockIdx.x) * E, nullptr, nullptr, sorted_pairs,
                   pair_to_row, smem, wave_sum);
}

int ranges_for(int64_t R) {
  if (R <= kSingleMaxPairs) return 0;
  const int64_t n = (R + kRangePairs - 1) / kRangePairs;
  return int(n < kMaxRanges ? n : kMaxRanges);
}

}  // namespace

size_t permute_workspace_bytes(int T, int E, int k) {
  return size_t(ranges_for(int64_t(T) * k)) * E * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_to_row,
                          void* workspace, hipStream_t s) {
  const int R = T * k;
  const int nr = ranges_for(R);
  if (nr > 0) {
    int32_t* ws = static_cast<int32_t*>(workspace);
    k_perm_hist<<<nr, 256, size_t(E) * sizeof(int32_t), s>>>(ids, R, E, nr, ws);
    k_perm_scan<<<1, 1024, 0, s>>>(E, nr, ws, counts, offsets);
    k_perm_scatter<<<nr, 4 * kWave, size_t(5) * E * sizeof(int32_t), s>>>(ids, R, E, nr, ws,
                                                                          sorted_pairs, pair_to_row);
    return hipGetLastError();
  }
  if (R <= 1024) {                // 5 E ints: within the default 64 KB for E <= 1024
    k_permute<4><<<1, 4 * kWave, size_t(5) * E * sizeof(int32_t), s>>>(
        ids, R, E, counts, offsets, sorted_pairs, pair_to_row);
    return hipGetLastError();
  }
  static std::atomic<bool> lds_set[kMaxDevices];   // 17 E ints, E up to 1024: above 64 KB
  const hipError_t e = lds_limit_once(reinterpret_cast<const void*>(&k_permute<16>),
                                      int(17 * 1024 * sizeof(int32_t)), lds_set);
  if (e != hipSuccess) return e;
  k_permute<16><<<1, 16 * kWave, size_t(17) * E * sizeof(int32_t), s>>>(
      ids, R, E, counts, offsets, sorted_pairs, pair_to_row);
  return hipGetLastError();
}

}  // namespace mxm

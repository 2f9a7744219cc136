// Token-to-expert permutation: counts, offsets, sorted pair lists.  The
// algorithm is permute_block in routing.hpp; this file launches it as one
// workgroup of 4 waves (up to 1024 pairs) or 16.
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
  permute_block<NW>(ids, R, E, counts, offsets, sorted_pairs, pair_to_row, smem, wave_sum);
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

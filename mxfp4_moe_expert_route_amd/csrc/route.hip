// Top-k routing: one wave64 per token.
//
// The pages give 384 experts with 8 active per token (nxbn.cn article,
// "架构设计与配置详解") and no scoring rule.  Rule used (a reading): experts by
// descending logit, lower index first on equal logits, -0.0 == +0.0, NaN as
// -inf; weights = softmax over all experts renormalised over the chosen k,
// which equals exp(l_j - l_1) / sum_j' exp(l_j' - l_1) over the chosen.
//
// Each logit becomes a 64-bit key: an order-preserving 32-bit image of the
// float in the high word and (0xffffffff - index) in the low word, so the
// unsigned maximum is the largest logit with the lowest index.  k rounds of a
// wave-wide max (per-lane max, then a butterfly over ds_swizzle/DPP lanes)
// pick the experts; the picked key is cleared to 0, below every valid key.
#include "common.hpp"

namespace mxm {
namespace {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;   // NaN ranks as -inf
  if (u == 0x80000000u) u = 0u;                            // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int NPER>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int t = int((int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6);
  if (t >= T) return;                                      // whole wave leaves together
  const int lane = lane_id();
  const float* row = logits + int64_t(t) * E;
  uint64_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + kWave * i;
    key[i] = (e < E) ? (uint64_t(order_key(row[e])) << 32) | uint64_t(0xffffffffu - uint32_t(e))
                     : 0ull;
  }
  int my_id = 0;
  float my_l = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NPER; ++i) best = max_u64(best, key[i]);
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) {
      const uint32_t lo = __shfl_xor(uint32_t(best), d);
      const uint32_t hi = __shfl_xor(uint32_t(best >> 32), d);
      best = max_u64(best, (uint64_t(hi) << 32) | lo);
    }
#pragma unroll
    for (int i = 0; i < NPER; ++i) key[i] = (key[i] == best) ? 0ull : key[i];
    if (lane == j) {
      my_id = int(0xffffffffu - uint32_t(best));
      my_l = key_value(uint32_t(best >> 32));
    }
  }
  const float l1 = __shfl(my_l, 0);
  float ex = (lane < k) ? expf(my_l - l1) : 0.f;
  float sum = ex;
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);
  if (lane < k) {
    ids[int64_t(t) * k + lane] = my_id;
    w[int64_t(t) * k + lane] = ex / sum;
  }
}

template <int NPER>
hipError_t launch_n(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                    hipStream_t s) {
  const int64_t threads = int64_t(T) * kWave;
  const int grid = int((threads + 255) / 256);
  k_route_topk<NPER><<<grid, 256, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s) {
  const int nper = (E + kWave - 1) / kWave;               // E <= 1024 -> nper <= 16
  if (nper <= 1) return launch_n<1>(logits, T, E, k, ids, w, s);
  if (nper <= 2) return launch_n<2>(logits, T, E, k, ids, w, s);
  if (nper <= 4) return launch_n<4>(logits, T, E, k, ids, w, s);
  if (nper <= 8) return launch_n<8>(logits, T, E, k, ids, w, s);
  return launch_n<16>(logits, T, E, k, ids, w, s);
}

}  // namespace mxm

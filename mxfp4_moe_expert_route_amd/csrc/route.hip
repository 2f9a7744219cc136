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
// wave-wide max (per-lane max, then DPP row shifts and row broadcasts) pick
// the experts; the picked key is cleared to 0, below every valid key.
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

// v moved across lanes by the DPP control CTRL (rows and banks masked by
// RM); lanes whose source is outside the row read 0, below every key
template <int CTRL, int RM>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(v)), CTRL, RM, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(v >> 32)), CTRL, RM, 0xf, true);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

// Largest key of the wave, in every lane.  Row shifts build each 16-lane
// row's maximum in its lane 15, two row broadcasts carry them to lane 63;
// DPP keeps the whole reduction in the VALU (no LDS round trips).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0x111, 0xf>(v));   // row_shr:1
  v = max_u64(v, dpp_u64<0x112, 0xf>(v));   // row_shr:2
  v = max_u64(v, dpp_u64<0x114, 0xf>(v));   // row_shr:4
  v = max_u64(v, dpp_u64<0x118, 0xf>(v));   // row_shr:8
  v = max_u64(v, dpp_u64<0x142, 0xa>(v));   // row_bcast:15 into rows 1 and 3
  v = max_u64(v, dpp_u64<0x143, 0xc>(v));   // row_bcast:31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(v)), kWave - 1);
  const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(v >> 32)), kWave - 1);
  return (uint64_t(hi) << 32) | lo;
}

// Sum over the wave in a fixed order (the same reduction tree as above), in
// every lane.
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto add = [&](float x, int y) { return x + __int_as_float(y); };
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, true));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

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
  float my_l = 0.f, l1 = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NPER; ++i) best = max_u64(best, key[i]);
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < NPER; ++i) key[i] = (key[i] == best) ? 0ull : key[i];
    if (j == 0) l1 = key_value(uint32_t(best >> 32));
    if (lane == j) {
      my_id = int(0xffffffffu - uint32_t(best));
      my_l = key_value(uint32_t(best >> 32));
    }
  }
  const float ex = (lane < k) ? expf(my_l - l1) : 0.f;
  const float sum = wave_sum_f32(ex);
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

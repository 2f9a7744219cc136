// Top-k routing (one wave64 per token) and the router projection in front of
// it.
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

// Router projection: logits[t][e] = sum_h x[t][h] * w[e][h] (+ bias[e]), fp32
// accumulation in a fixed order (deterministic run to run).
//
// Decode sizes (T <= 64): one workgroup per EPW experts and block of 8
// tokens.  Its 256 lanes split the experts' weight rows (float4 each, 1 KB
// strides), so every load of a row is in flight at once and each row is read
// once per token block; each lane keeps one fma chain per (expert, token),
// then a DPP tree per wave and the four waves' sums in order.
template <int TB, int EPW>
__global__ __launch_bounds__(256) void k_router_rows(const uint16_t* __restrict__ x,
                                                     const float* __restrict__ wr,
                                                     const float* __restrict__ bias, int T, int H,
                                                     int E, float* __restrict__ logits) {
  __shared__ float part[4][EPW][TB];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int e0 = blockIdx.x * EPW;
  const int ne = min(EPW, E - e0);
  const int t0 = blockIdx.y * TB;
  const int nt = min(TB, T - t0);
  float acc[EPW][TB];
#pragma unroll
  for (int q = 0; q < EPW; ++q)
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[q][j] = 0.f;
#pragma unroll 6
  for (int h = 4 * tid; h < H; h += 1024) {
    float4 w[EPW];
#pragma unroll
    for (int q = 0; q < EPW; ++q)
      w[q] = *reinterpret_cast<const float4*>(wr + size_t(e0 + min(q, ne - 1)) * H + h);
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if (j < nt) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + size_t(t0 + j) * H + h);
        const float x0 = __uint_as_float(xv.x << 16), x1 = __uint_as_float(xv.x & 0xffff0000u);
        const float x2 = __uint_as_float(xv.y << 16), x3 = __uint_as_float(xv.y & 0xffff0000u);
#pragma unroll
        for (int q = 0; q < EPW; ++q) {
          acc[q][j] = fmaf(x0, w[q].x, acc[q][j]);
          acc[q][j] = fmaf(x1, w[q].y, acc[q][j]);
          acc[q][j] = fmaf(x2, w[q].z, acc[q][j]);
          acc[q][j] = fmaf(x3, w[q].w, acc[q][j]);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < EPW; ++q)
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if (j < nt) {
        const float sum = wave_sum_f32(acc[q][j]);
        if (lane == 0) part[wave][q][j] = sum;
      }
    }
  __syncthreads();
  if (tid < EPW * TB) {
    const int q = tid / TB, j = tid % TB;
    if (q < ne && j < nt) {
      const int e = e0 + q;
      const float b = bias ? bias[e] : 0.f;
      logits[size_t(t0 + j) * E + e] =
          ((part[0][q][j] + part[1][q][j]) + (part[2][q][j] + part[3][q][j])) + b;
    }
  }
}

// Larger T: tiles of RT tokens x RE experts (64 x 64, or 32 x 32 when that
// leaves too few workgroups), K in steps of 32 staged through LDS as fp32,
// K-major.  Each lane computes RT/16 tokens x RE/16 experts: per K element a
// vector of x and one of w from LDS feed all of its fmas.  The next step's
// global loads are issued before the current step's fmas.  Each step's 32
// products go into a fresh partial that is then added to the running total,
// so an output sees 32-term chains and one add per step (H % 32 == 0).
constexpr int kRK = 32;

template <int RT, int RE>
__global__ __launch_bounds__(256) void k_router_tiles(const uint16_t* __restrict__ x,
                                                      const float* __restrict__ wr,
                                                      const float* __restrict__ bias, int T,
                                                      int H, int E, float* __restrict__ logits) {
  constexpr int PT = RT / 16, PE = RE / 16;      // outputs per lane
  constexpr int XL = RT * kRK / 256;             // x elements each lane stages (8 or 4)
  constexpr int WL = RE * kRK / 256;             // w elements each lane stages
  static_assert(XL == 8 || XL == 4, "x staged as 16 or 8 bytes per lane");
  static_assert(WL == 8 || WL == 4, "w staged as 32 or 16 bytes per lane");
  __shared__ __attribute__((aligned(16))) float xs[kRK][RT];
  __shared__ __attribute__((aligned(16))) float ws[kRK][RE];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;        // experts PE tx.., tokens PT ty..
  const int t0 = blockIdx.y * RT, e0 = blockIdx.x * RE;
  // staging roles: x row tid / (32 / XL), K elements XL (tid % (32 / XL)) ..
  const int xr = tid / (kRK / XL), xk = XL * (tid % (kRK / XL));
  const int wrr = tid / (kRK / WL), wk = WL * (tid % (kRK / WL));
  const uint16_t* xsrc = x + size_t(min(t0 + xr, T - 1)) * H + xk;
  const float* wsrc = wr + size_t(min(e0 + wrr, E - 1)) * H + wk;
  uint32_t xv[XL / 2];
  float wv[WL];
  auto fetch = [&](int k0) {
    if constexpr (XL == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(xsrc + k0);
      xv[0] = v.x; xv[1] = v.y; xv[2] = v.z; xv[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(xsrc + k0);
      xv[0] = v.x; xv[1] = v.y;
    }
#pragma unroll
    for (int i = 0; i < WL; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(wsrc + k0 + i);
      wv[i] = v.x; wv[i + 1] = v.y; wv[i + 2] = v.z; wv[i + 3] = v.w;
    }
  };
  float tot[PT][PE];
#pragma unroll
  for (int i = 0; i < PT; ++i)
#pragma unroll
    for (int j = 0; j < PE; ++j) tot[i][j] = 0.f;
  fetch(0);
  for (int k0 = 0; k0 < H; k0 += kRK) {
    __syncthreads();                             // the previous step's reads are done
#pragma unroll
    for (int i = 0; i < XL / 2; ++i) {
      xs[xk + 2 * i][xr] = __uint_as_float(xv[i] << 16);
      xs[xk + 2 * i + 1][xr] = __uint_as_float(xv[i] & 0xffff0000u);
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) ws[wk + i][wrr] = wv[i];
    __syncthreads();
    if (k0 + kRK < H) fetch(k0 + kRK);
    float stp[PT][PE];
#pragma unroll
    for (int i = 0; i < PT; ++i)
#pragma unroll
      for (int j = 0; j < PE; ++j) stp[i][j] = 0.f;
#pragma unroll 8
    for (int kk = 0; kk < kRK; ++kk) {
      float av[PT], bv[PE];
#pragma unroll
      for (int i = 0; i < PT; ++i) av[i] = xs[kk][PT * ty + i];
#pragma unroll
      for (int j = 0; j < PE; ++j) bv[j] = ws[kk][PE * tx + j];
#pragma unroll
      for (int i = 0; i < PT; ++i)
#pragma unroll
        for (int j = 0; j < PE; ++j) stp[i][j] = fmaf(av[i], bv[j], stp[i][j]);
    }
#pragma unroll
    for (int i = 0; i < PT; ++i)
#pragma unroll
      for (int j = 0; j < PE; ++j) tot[i][j] += stp[i][j];
  }
#pragma unroll
  for (int j = 0; j < PE; ++j) {
    const int e = e0 + PE * tx + j;
    if (e >= E) continue;
    const float b = bias ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int t = t0 + PT * ty + i;
      if (t < T) logits[size_t(t) * E + e] = tot[i][j] + b;
    }
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const float* w_router, const float* bias, int T,
                                int H, int E, float* logits, hipStream_t s) {
  // the tiles load up to 16 bytes of x per lane: rows and base 16-byte aligned
  if (T <= 64 || H % kRK || reinterpret_cast<uintptr_t>(x) % 16) {
    // blocks of 8 tokens (32-token blocks: 44 us against 31 us at 64 tokens);
    // one expert per workgroup for a single block (15 us at 8 tokens, two:
    // 15.5, four: 18.4), four when several blocks re-read the weights (21 us
    // at 64 tokens against 31)
    if (T <= 8) {
      k_router_rows<8, 1><<<dim3(unsigned(E), 1), 256, 0, s>>>(x, w_router, bias, T, H, E, logits);
    } else {
      const dim3 grid(unsigned((E + 3) / 4), unsigned((T + 7) / 8));
      k_router_rows<8, 4><<<grid, 256, 0, s>>>(x, w_router, bias, T, H, E, logits);
    }
  } else if (int64_t((E + 63) / 64) * ((T + 63) / 64) >= 512) {
    const dim3 grid(unsigned((E + 63) / 64), unsigned((T + 63) / 64));
    k_router_tiles<64, 64><<<grid, 256, 0, s>>>(x, w_router, bias, T, H, E, logits);
  } else {
    const dim3 grid(unsigned((E + 31) / 32), unsigned((T + 31) / 32));
    k_router_tiles<32, 32><<<grid, 256, 0, s>>>(x, w_router, bias, T, H, E, logits);
  }
  return hipGetLastError();
}

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

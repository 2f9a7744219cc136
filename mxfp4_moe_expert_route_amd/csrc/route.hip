// Top-k routing (one wave64 per token), the same fused with the grouping of
// pairs by expert for small batches, and the router projection in front of
// them.  The top-k rule, its key encoding and the grouping are in
// routing.hpp.
#include "routing.hpp"

namespace mxm {
namespace {

constexpr int kFusedWaves = 16;

template <int NPER>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int t = int((int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6);
  if (t >= T) return;                                      // whole wave leaves together
  const int lane = lane_id();
  int my_id;
  float my_w;
  route_token<NPER>(logits + int64_t(t) * E, E, k, my_id, my_w);
  if (lane < k) {
    ids[int64_t(t) * k + lane] = my_id;
    w[int64_t(t) * k + lane] = my_w;
  }
}

// Small batches (T <= 16): routing and grouping in one workgroup of 16 waves.
// Wave t routes token t; the ids go to global memory and to LDS, and each
// chosen expert's token mask gets bit t.  After one barrier the workgroup
// groups the pairs from the masks (group_small).  Same routing function as
// k_route_topk and the same lists as k_permute, bit for bit; one launch and
// one round trip to memory fewer.
template <int NPER>
__global__ __launch_bounds__(kFusedWaves * kWave) void k_route_permute(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_to_row) {
  extern __shared__ int32_t smem[];            // mask [E], offsets [E + 1], ids [T k]
  __shared__ int32_t wave_sum[kFusedWaves];
  uint32_t* mask = reinterpret_cast<uint32_t*>(smem);
  int32_t* off_lds = smem + E;
  int32_t* lds_ids = smem + 2 * E + 1;
  for (int e = threadIdx.x; e < E; e += kFusedWaves * kWave) mask[e] = 0u;
  __syncthreads();
  const int t = threadIdx.x >> 6;
  const int lane = lane_id();
  if (t < T) {
    int my_id;
    float my_w;
    route_token<NPER>(logits + int64_t(t) * E, E, k, my_id, my_w);
    if (lane < k) {
      ids[int64_t(t) * k + lane] = my_id;
      w[int64_t(t) * k + lane] = my_w;
      lds_ids[t * k + lane] = my_id;
      atomicOr(&mask[my_id], 1u << t);
    }
  }
  __syncthreads();
  group_small<kFusedWaves>(lds_ids, mask, T * k, E, k, counts, offsets, off_lds, sorted_pairs,
                           pair_to_row, nullptr, nullptr, wave_sum);
}

template <int NPER>
hipError_t launch_fused_n(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                          int32_t* pair_to_row, hipStream_t s) {
  const size_t lds = (size_t(2) * E + 1 + size_t(T) * k) * sizeof(int32_t);
  k_route_permute<NPER><<<1, kFusedWaves * kWave, lds, s>>>(logits, T, E, k, ids, w, counts,
                                                            offsets, sorted_pairs, pair_to_row);
  return hipGetLastError();
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
// strides) and read the block's x at the same positions; every load of a
// lane is unconditional (rows past the block's last token re-read that
// token) and issued before the fmas, so they are all in flight at once (with
// a branch per token the loads of x went out one at a time, each waiting for
// the one before: 14.7 us at 8 tokens).  Each row is read once per token
// block; each lane keeps one fma chain per (expert, token), then a DPP tree
// per wave and the four waves' sums in order.  NT: the weight loads carry the
// non-temporal hint (one token block reads each row once).
template <int TB, int EPW, bool NT>
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
  const uint16_t* xr[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) xr[j] = x + size_t(t0 + min(j, nt - 1)) * H;
  const float* wrow[EPW];
#pragma unroll
  for (int q = 0; q < EPW; ++q) wrow[q] = wr + size_t(e0 + min(q, ne - 1)) * H;
  // kU steps of 1024 per pass: each lane loads its 4 elements of every step
  // (addresses clamped in range), then runs the fmas of the steps in range
  constexpr int kU = 6;
  for (int h0 = 4 * tid; h0 < H; h0 += kU * 1024) {
    float4 w[kU][EPW];
    uint2 xv[kU][TB];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int h = min(h0 + 1024 * u, H - 4);
#pragma unroll
      for (int q = 0; q < EPW; ++q) {
        if constexpr (NT) {
          const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(wrow[q] + h));
          w[u][q] = make_float4(t[0], t[1], t[2], t[3]);
        } else {
          w[u][q] = *reinterpret_cast<const float4*>(wrow[q] + h);
        }
      }
#pragma unroll
      for (int j = 0; j < TB; ++j) xv[u][j] = *reinterpret_cast<const uint2*>(xr[j] + h);
    }
    // keep every load of the pass ahead of the first fma (the scheduler
    // would otherwise sink each step's loads to its fmas, one round trip each)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool in = h0 + 1024 * u < H;
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        const uint2 v = xv[u][j];
        const float x0 = __uint_as_float(v.x << 16), x1 = __uint_as_float(v.x & 0xffff0000u);
        const float x2 = __uint_as_float(v.y << 16), x3 = __uint_as_float(v.y & 0xffff0000u);
#pragma unroll
        for (int q = 0; q < EPW; ++q) {
          float a = fmaf(x0, w[u][q].x, acc[q][j]);
          a = fmaf(x1, w[u][q].y, a);
          a = fmaf(x2, w[u][q].z, a);
          a = fmaf(x3, w[u][q].w, a);
          acc[q][j] = in ? a : acc[q][j];
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
      k_router_rows<8, 1, true><<<dim3(unsigned(E), 1), 256, 0, s>>>(x, w_router, bias, T, H, E,
                                                                    logits);
    } else {
      const dim3 grid(unsigned((E + 3) / 4), unsigned((T + 7) / 8));
      k_router_rows<8, 4, false><<<grid, 256, 0, s>>>(x, w_router, bias, T, H, E, logits);
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

bool route_permute_fusable(int T, int E, int k) {
  return T >= 1 && T <= kFusedWaves &&
         (size_t(2) * E + 1 + size_t(T) * k) * sizeof(int32_t) <= 64 * 1024;
}

hipError_t launch_route_permute(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                                int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                                int32_t* pair_to_row, hipStream_t s) {
  const int nper = (E + kWave - 1) / kWave;
  if (nper <= 1) return launch_fused_n<1>(logits, T, E, k, ids, w, counts, offsets, sorted_pairs, pair_to_row, s);
  if (nper <= 2) return launch_fused_n<2>(logits, T, E, k, ids, w, counts, offsets, sorted_pairs, pair_to_row, s);
  if (nper <= 4) return launch_fused_n<4>(logits, T, E, k, ids, w, counts, offsets, sorted_pairs, pair_to_row, s);
  if (nper <= 8) return launch_fused_n<8>(logits, T, E, k, ids, w, counts, offsets, sorted_pairs, pair_to_row, s);
  return launch_fused_n<16>(logits, T, E, k, ids, w, counts, offsets, sorted_pairs, pair_to_row, s);
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

// Weighted combine of each token's k expert outputs.
//
// out_t = sum_{j=0..k-1} w_tj * y[pair_to_row[t*k + j]], fp32, summed in slot
// order with fused multiply-adds, so the result is deterministic.  One thread
// produces 4 consecutive outputs (16-byte loads and stores); a dropped pair
// (pair_to_row < 0) contributes nothing.
#include "common.hpp"

namespace mxm {
namespace {

// One workgroup per (token, 1024 columns): the token's k rows and weights are
// read once into LDS, then every thread issues its k row loads together (no
// branch between them: a dropped pair reads row 0 and its term is not added)
// and accumulates them in slot order.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const float* __restrict__ w,
                                                 const int32_t* __restrict__ pair_to_row, int T,
                                                 int H, int k, float* __restrict__ out) {
  __shared__ int32_t srow[32];
  __shared__ float sw[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    srow[threadIdx.x] = pair_to_row[int64_t(t) * k + threadIdx.x];
    sw[threadIdx.x] = w[int64_t(t) * k + threadIdx.x];
  }
  __syncthreads();
  const int c = blockIdx.y * 1024 + threadIdx.x * 4;
  if (c >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (j0 + i < k) ? max(srow[j0 + i], 0) : 0;
      v[i] = *reinterpret_cast<const float4*>(y + int64_t(r) * H + c);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + i;
      if (j < k && srow[j] >= 0) {
        const float wj = sw[j];
        acc.x = fmaf(wj, v[i].x, acc.x);
        acc.y = fmaf(wj, v[i].y, acc.y);
        acc.z = fmaf(wj, v[i].z, acc.z);
        acc.w = fmaf(wj, v[i].w, acc.w);
      }
    }
  }
  *reinterpret_cast<float4*>(out + int64_t(t) * H + c) = acc;
}

}  // namespace

hipError_t launch_combine(const float* y, const float* w, const int32_t* pair_to_row, int T,
                          int H, int k, float* out, hipStream_t s) {
  k_combine<<<dim3(unsigned(T), unsigned((H + 1023) / 1024)), 256, 0, s>>>(y, w, pair_to_row, T,
                                                                          H, k, out);
  return hipGetLastError();
}

}  // namespace mxm

// Weighted combine of each token's k expert outputs.
//
// out_t = sum_{j=0..k-1} w_tj * y[pair_to_row[t*k + j]], fp32, summed in slot
// order with fused multiply-adds, so the result is deterministic.  One thread
// produces 4 consecutive outputs (16-byte loads and stores); a dropped pair
// (pair_to_row < 0) contributes nothing.
#include "common.hpp"

namespace mxm {
namespace {

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const float* __restrict__ w,
                                                 const int32_t* __restrict__ pair_to_row, int T,
                                                 int H, int k, float* __restrict__ out) {
  const int q = H >> 2;                                   // float4 columns per token
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(T) * q) return;
  const int64_t t = idx / q;
  const int c = int(idx - t * q) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int r = pair_to_row[t * k + j];
    if (r < 0) continue;
    const float wj = w[t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + int64_t(r) * H + c);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  *reinterpret_cast<float4*>(out + t * H + c) = acc;
}

}  // namespace

hipError_t launch_combine(const float* y, const float* w, const int32_t* pair_to_row, int T,
                          int H, int k, float* out, hipStream_t s) {
  const int64_t n = int64_t(T) * (H / 4);
  k_combine<<<dim3(unsigned((n + 255) / 256)), 256, 0, s>>>(y, w, pair_to_row, T, H, k, out);
  return hipGetLastError();
}

}  // namespace mxm

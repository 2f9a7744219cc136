// Weighted combine of each token's k expert outputs.
//
// out_t = sum_{j=0..k-1} w_tj * y[pair_to_row[t*k + j]], fp32, summed in slot
// order with fused multiply-adds, so the result is deterministic.  One thread
// produces 4 consecutive outputs (16-byte loads and stores); a dropped pair
// (pair_to_row < 0) contributes nothing.
#include "common.hpp"

namespace mxm {
namespace {

// One workgroup per (token, CW columns): the token's k rows and weights are
// read once into LDS, then every thread issues its row loads together (one
// 16-byte load per row, or two 1024 columns apart when CW = 2048; no branch
// between them: a dropped pair reads row 0 and its term is not added) and
// accumulates them in slot order.  Each row of y is read once, so the loads
// carry the non-temporal hint (at 8192 tokens x top-8: 380 -> 318 us).  A
// small batch takes CW = 1024, twice the workgroups (8 tokens: 48 instead of
// 24; the layer step 0.6 us shorter).
template <int CW>
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
  const int c0 = blockIdx.y * CW + threadIdx.x * 4;        // columns c0 (and c0 + 1024)
  const bool in1 = CW == 2048 && c0 + 1024 < H;
  if (c0 >= H) return;
  float4 acc0 = make_float4(0.f, 0.f, 0.f, 0.f), acc1 = acc0;
  for (int j0 = 0; j0 < k; j0 += 8) {
    f32x4 v0[8], v1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (j0 + i < k) ? max(srow[j0 + i], 0) : 0;
      const float* yr = y + int64_t(r) * H + c0;
      v0[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yr));
      v1[i] = in1 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yr + 1024))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = j0 + i;
      if (j < k && srow[j] >= 0) {
        const float wj = sw[j];
        acc0.x = fmaf(wj, v0[i][0], acc0.x); acc0.y = fmaf(wj, v0[i][1], acc0.y);
        acc0.z = fmaf(wj, v0[i][2], acc0.z); acc0.w = fmaf(wj, v0[i][3], acc0.w);
        acc1.x = fmaf(wj, v1[i][0], acc1.x); acc1.y = fmaf(wj, v1[i][1], acc1.y);
        acc1.z = fmaf(wj, v1[i][2], acc1.z); acc1.w = fmaf(wj, v1[i][3], acc1.w);
      }
    }
  }
  *reinterpret_cast<float4*>(out + int64_t(t) * H + c0) = acc0;
  if (in1) *reinterpret_cast<float4*>(out + int64_t(t) * H + c0 + 1024) = acc1;
}

}  // namespace

hipError_t launch_combine(const float* y, const float* w, const int32_t* pair_to_row, int T,
                          int H, int k, float* out, hipStream_t s) {
  if (int64_t(T) * ((H + 2047) / 2048) < 256)
    k_combine<1024><<<dim3(unsigned(T), unsigned((H + 1023) / 1024)), 256, 0, s>>>(
        y, w, pair_to_row, T, H, k, out);
  else
    k_combine<2048><<<dim3(unsigned(T), unsigned((H + 2047) / 2048)), 256, 0, s>>>(
        y, w, pair_to_row, T, H, k, out);
  return hipGetLastError();
}

}  // namespace mxm

// Streaming-read probe: the HBM read rate a plain kernel reaches on this
// device, the practical ceiling of the weight-streaming contractions.
//
// k_stream_xor XORs every 32-bit word of a buffer into one result word, so
// the loads cannot be dropped and the result can be checked.  Each workgroup
// reads 32 KB per iteration (eight 16-byte loads per lane, all in flight
// before any is used) and walks the buffer grid-stride; the grid is eight
// workgroups per CU.  NT selects the non-temporal load hint, the cache policy
// of the decode contraction's code stream.  Measured over 4 GiB of random
// words with non-temporal loads: four loads per lane 6.4 TB/s, eight loads
// 6.6-6.7 TB/s.  The same buffer filled with one repeated byte reads about 5%
// faster, so the ceiling is quoted on random words, as weight codes are.
#include "common.hpp"

namespace mxm {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kProbeChunk = kProbeThreads * kProbeUnroll;     // 16-byte words per iteration

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void k_stream_xor(const u32x4* __restrict__ src,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ result) {
  uint32_t acc = 0;
  const int64_t stride = int64_t(gridDim.x) * kProbeChunk;
  for (int64_t base = int64_t(blockIdx.x) * kProbeChunk; base < n16; base += stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t i = base + u * kProbeThreads + threadIdx.x;
      if (i < n16) {
        if constexpr (NT) v[u] = __builtin_nontemporal_load(src + i);
        else v[u] = src[i];
      } else {
        v[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // wave XOR, then one atomic per wave
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane_id() == 0) atomicXor(result, acc);
}

}  // namespace

hipError_t launch_stream_xor(const void* src, int64_t bytes, int nontemporal, uint32_t* result,
                             hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t chunks = (n16 + kProbeChunk - 1) / kProbeChunk;
  const int64_t cap = int64_t(8) * device_cus();
  const unsigned grid = unsigned(chunks < cap ? chunks : cap);
  const u32x4* p = static_cast<const u32x4*>(src);
  if (nontemporal)
    k_stream_xor<true><<<dim3(grid), kProbeThreads, 0, s>>>(p, n16, result);
  else
    k_stream_xor<false><<<dim3(grid), kProbeThreads, 0, s>>>(p, n16, result);
  return hipGetLastError();
}

}  // namespace mxm

// MXFP4 pack / unpack kernels.
//
// Format: MXFP4 with block size 32, as the pages fix for the expert weights
// ("MiMo-V2.5-Pro-FP4-DFlash" model card, §2 "FP4 Quantization"); element and
// scale encodings per OCP MX v1.0 (E2M1, E8M0).  Layout reading: blocks run
// along the row, byte j holds element 2j in its low nibble.
//
// Both directions build IEEE bit patterns with integer arithmetic, so results
// are exact (subnormal inputs and outputs included) and independent of the
// floating-point denormal mode.  One thread handles one 32-element block.
#include "common.hpp"

namespace mxm {
namespace {

// fp32 bit pattern of E2M1 code c (4 bits) times 2^(e-127), e in 0..255.
__device__ __forceinline__ uint32_t mx_value_bits(uint32_t c, uint32_t e) {
  if (e == 255u) return 0x7fc00000u;                 // NaN scale: NaN block
  const uint32_t sign = (c & 8u) << 28;
  const uint32_t m = c & 7u;
  if (m == 0u) return sign;                          // +-0
  // magnitude = (1 + q/2) * 2^p:  0.5 (p=-1), 1, 1.5 (p=0), 2, 3 (p=1), 4, 6 (p=2)
  const int p = int(m >> 1) - 1;
  const uint32_t q = (m >= 2u) ? (m & 1u) : 0u;
  const int be = p + int(e);                         // biased fp32 exponent
  if (be >= 255) return sign | 0x7f800000u;          // overflow to Inf
  if (be >= 1) return sign | (uint32_t(be) << 23) | (q << 22);
  // subnormal: (2 + q) * 2^(be - 128) = mantissa (2 + q) << (be + 21), be >= -1
  return sign | ((2u + q) << (be + 21));
}

__global__ __launch_bounds__(256) void k_unpack(const uint8_t* __restrict__ codes,
                                                const uint8_t* __restrict__ scales,
                                                int64_t nblocks, void* __restrict__ y,
                                                int y_bf16) {
  for (int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; b < nblocks;
       b += int64_t(gridDim.x) * blockDim.x) {
    const uint4 c = *reinterpret_cast<const uint4*>(codes + b * 16);
    const uint32_t e = scales[b];
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    if (y_bf16) {
      uint4* out = reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + b * 32);
#pragma unroll
      for (int d = 0; d < 4; ++d) {                  // dword d: elements 8d..8d+7
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = mx_value_bits((cw[d] >> (8 * i)) & 15u, e) >> 16;
          const uint32_t hi = mx_value_bits((cw[d] >> (8 * i + 4)) & 15u, e) >> 16;
          o[i] = lo | (hi << 16);
        }
        out[d] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    } else {
      uint4* out = reinterpret_cast<uint4*>(static_cast<float*>(y) + b * 32);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {                // 4 elements = 2 bytes per uint4
          const uint32_t b0 = (cw[d] >> (16 * h)) & 0xffu;
          const uint32_t b1 = (cw[d] >> (16 * h + 8)) & 0xffu;
          out[2 * d + h] = make_uint4(mx_value_bits(b0 & 15u, e), mx_value_bits(b0 >> 4, e),
                                      mx_value_bits(b1 & 15u, e), mx_value_bits(b1 >> 4, e));
        }
      }
    }
  }
}

// fp32 bits of (1 + mf/2^23) * 2^p * 2^(e-127) for the rounding midpoints;
// exact for every e the conversion can choose (see the caller).
__device__ __forceinline__ uint32_t midpoint_bits(int p, uint32_t mf, int e) {
  const int be = p + e;
  if (be >= 1) return (uint32_t(be) << 23) | mf;
  return (0x800000u | mf) >> (1 - be);               // be >= -2: exact shift
}

__global__ __launch_bounds__(256) void k_pack(const void* __restrict__ x, int x_bf16,
                                              int64_t nblocks, uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales) {
  for (int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; b < nblocks;
       b += int64_t(gridDim.x) * blockDim.x) {
    uint32_t v[32];
    if (x_bf16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + b * 32);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint4 w = src[d];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * d + 2 * i] = ww[i] << 16;
          v[8 * d + 2 * i + 1] = ww[i] & 0xffff0000u;
        }
      }
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + b * 32);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint4 w = src[d];
        v[4 * d] = w.x; v[4 * d + 1] = w.y; v[4 * d + 2] = w.z; v[4 * d + 3] = w.w;
      }
    }
    bool bad = false;
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t a = v[i] & 0x7fffffffu;
      bad |= (a >= 0x7f800000u);                     // Inf or NaN
      amax = max(amax, a);                           // |x| order == integer order
    }
    uint32_t out[4] = {0u, 0u, 0u, 0u};
    uint32_t e = 0;
    if (bad) {
      e = 255;
    } else {
      if (amax != 0u) {
        const int ef = int(amax >> 23);
        const int fl = ef > 0 ? ef - 127 : (31 - __clz(amax)) - 149;   // floor(log2 amax)
        e = uint32_t(min(max(fl - 2 + 127, 0), 254));
      }
      // E2M1 magnitude code = number of midpoints passed; at a midpoint the
      // even code wins: strict '>' below an even code, '>=' below an odd one.
      const int ei = int(e);
      const uint32_t t0 = midpoint_bits(-2, 0x000000u, ei);   // 0.25
      const uint32_t t1 = midpoint_bits(-1, 0x400000u, ei);   // 0.75
      const uint32_t t2 = midpoint_bits(0, 0x200000u, ei);    // 1.25
      const uint32_t t3 = midpoint_bits(0, 0x600000u, ei);    // 1.75
      const uint32_t t4 = midpoint_bits(1, 0x200000u, ei);    // 2.5
      const uint32_t t5 = midpoint_bits(1, 0x600000u, ei);    // 3.5
      const uint32_t t6 = midpoint_bits(2, 0x200000u, ei);    // 5
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t a = v[i] & 0x7fffffffu;
        uint32_t c = uint32_t(a > t0) + uint32_t(a >= t1) + uint32_t(a > t2) +
                     uint32_t(a >= t3) + uint32_t(a > t4) + uint32_t(a >= t5) +
                     uint32_t(a > t6);
        c |= (v[i] >> 28) & 8u;                      // sign bit of the input
        out[i >> 3] |= c << (4 * (i & 7));
      }
    }
    *reinterpret_cast<uint4*>(codes + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    scales[b] = uint8_t(e);
  }
}

int grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return int(g < (1 << 20) ? (g > 0 ? g : 1) : (1 << 20));
}

}  // namespace

hipError_t launch_unpack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                         void* y, int y_dtype, hipStream_t s) {
  const int64_t nb = rows * (K / 32);
  k_unpack<<<grid_for(nb), 256, 0, s>>>(codes, scales, nb, y, y_dtype == 1);
  return hipGetLastError();
}

hipError_t launch_pack(const void* x, int x_dtype, int64_t rows, int64_t K, uint8_t* codes,
                       uint8_t* scales, hipStream_t s) {
  const int64_t nb = rows * (K / 32);
  k_pack<<<grid_for(nb), 256, 0, s>>>(x, x_dtype == 1, nb, codes, scales);
  return hipGetLastError();
}

}  // namespace mxm

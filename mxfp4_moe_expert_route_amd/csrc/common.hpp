// Shared device helpers and the internal launcher interface of libmxfp4moe.
// gfx950 (CDNA4) only: wave64, MFMA, scaled FP4 conversions.
#pragma once
#include <atomic>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxm {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Workgroup barrier for kernels that manage their own s_waitcnt: no counter
// is waited on, and the "memory" clobber keeps the compiler from moving this
// wave's loads and stores across it (the s_barrier intrinsic alone does not,
// and LDS filled by asynchronous global->LDS loads must not be read early).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// E8M0 scale byte -> fp32 2^(e-127) for e in 1..254 (exact normal float).
// e == 0 gives +0.0f: 2^-127 is below the normal fp32 range; a block with
// scale byte 0 contributes at most 6 * 2^-127 per weight.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) { return __uint_as_float(e << 23); }

// Eight E2M1 codes of one dword (element 2b in the low nibble of byte b)
// times `scale`, converted to eight bf16 in element order.
__device__ __forceinline__ bf16x8 dequant8(uint32_t codes, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Inclusive prefix sum across the 64 lanes of a wave (all lanes active), in
// DPP steps: shifts by 1, 2, 4, 8 within each row of 16 lanes, then lane 15
// of rows 0 and 2 added into rows 1 and 3, then lane 31 into rows 2 and 3.
// Lanes whose source is out of range add 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, true);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, true);   // row_bcast:31
  return v;
}

// Tile of one expert's row segment: `rows` sorted rows starting at `row0`.
struct Tile {
  int e;
  int row0;
  int rows;
};

// Map tile index `tau` to (expert, row range) when every expert's segment of
// `offsets` is cut into tiles of `mt` rows, experts in order.  Only experts
// with lo <= rows < hi take part (the others own no tiles).  Executed by a
// whole wave (uniform control flow); returns false when tau is past the last
// tile.  Reads offsets[0..E].
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int mt,
                                          int tau, Tile& t, int lo = 1, int hi = 0x7fffffff) {
  const int lane = lane_id();
  int base = 0;
  for (int c0 = 0; c0 < E; c0 += kWave) {
    const int e = c0 + lane;
    int off = 0, cnt = 0;
    if (e < E) {
      off = offsets[e];
      cnt = offsets[e + 1] - off;
    }
    if (cnt < lo || cnt >= hi) cnt = 0;
    const int nt = (cnt + mt - 1) / mt;
    const int incl = wave_incl_scan(nt);
    const int total = __shfl(incl, kWave - 1);
    if (tau < base + total) {
      const int excl = base + incl - nt;
      const unsigned long long m = __ballot(tau >= excl && tau < excl + nt);
      const int src = __ffsll((long long)m) - 1;
      const int ti = tau - __shfl(excl, src);
      t.e = c0 + src;
      t.row0 = __shfl(off, src) + ti * mt;
      t.rows = min(mt, __shfl(cnt, src) - ti * mt);
      return true;
    }
    base += total;
  }
  return false;
}

// ---------------------------------------------------------------------------
// per-device launch state, kept for the life of the process (atomics: calls
// may come from several host threads)
constexpr int kMaxDevices = 64;
// CU count of the current device (256 when it cannot be read)
int device_cus();
// Raise fn's dynamic LDS limit to `bytes` on the current device, once per
// device: done[] holds one flag per device index.
hipError_t lds_limit_once(const void* fn, int bytes, std::atomic<bool>* done);

// ---------------------------------------------------------------------------
// internal launchers (defined in the kernel files, called by api.hip after
// host-side argument checks).  Each returns the hipError_t of its launch.

hipError_t launch_pack(const void* x, int x_dtype, int64_t rows, int64_t K, uint8_t* codes,
                       uint8_t* scales, hipStream_t s);
hipError_t launch_unpack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                         void* y, int y_dtype, hipStream_t s);
// routing and grouping in one workgroup, for T <= 16 (same results as the
// two launches below)
bool route_permute_fusable(int T, int E, int k);
hipError_t launch_route_permute(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                                int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                                int32_t* pair_to_row, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);
hipError_t launch_router_logits(const uint16_t* x, const float* w_router, const float* bias, int T,
                                int H, int E, float* logits, hipStream_t s);
size_t permute_workspace_bytes(int T, int E, int k);
hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_to_row,
                          void* workspace, hipStream_t s);
// Streaming kernels: experts with fewer than `hi` rows (all when hi is INT_MAX).
hipError_t launch_gate_up(const uint16_t* x, const int32_t* sorted_pairs, const int32_t* offsets,
                          int T, int H, int I, int E, int k, const uint8_t* codes,
                          const uint8_t* scales, uint16_t* h, int hi, hipStream_t s);
hipError_t launch_down(const uint16_t* h, const int32_t* offsets, int T, int H, int I, int E,
                       int k, const uint8_t* codes, const uint8_t* scales, float* y, int hi,
                       hipStream_t s);

// Persistent decode-size variant of the streaming kernels (16-row tiles, one
// workgroup per CU, LDS-staged weight stream).  Same arguments and results.
bool decode_supported(int T, int H, int I, int E, int k);
hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* sorted_pairs,
                                 const int32_t* offsets, int T, int H, int I, int E, int k,
                                 const uint8_t* codes, const uint8_t* scales, uint16_t* h, int hi,
                                 hipStream_t s);
hipError_t launch_down_decode(const uint16_t* h, const int32_t* offsets, int T, int H, int I,
                              int E, int k, const uint8_t* codes, const uint8_t* scales, float* y,
                              int hi, hipStream_t s);

// Grouped contractions for experts with many rows (LDS-tiled MFMA GEMM).
// Experts with fewer than `min_rows` rows are left to the streaming kernels.
bool dense_supported(int T, int H, int I, int E, int k);
int dense_min_rows();
hipError_t launch_gate_up_dense(const uint16_t* x, const int32_t* sorted_pairs,
                                const int32_t* offsets, int T, int H, int I, int E, int k,
                                const uint8_t* codes, const uint8_t* scales, uint16_t* h,
                                hipStream_t s);
hipError_t launch_down_dense(const uint16_t* h, const int32_t* offsets, int T, int H, int I,
                             int E, int k, const uint8_t* codes, const uint8_t* scales, float* y,
                             hipStream_t s);
// Persistent fused decode layer (routing, grouping, gate/up, down, combine in
// one cooperative launch) for T <= 16; its workspace is zero-filled by the
// caller before the first call and left zero-filled.
bool decode_layer_supported(int T, int H, int I, int E, int k);
size_t decode_layer_workspace_bytes();
hipError_t launch_decode_layer(const uint16_t* x, const float* logits, int T, int H, int I, int E,
                               int k, const uint8_t* w13c, const uint8_t* w13s,
                               const uint8_t* w2c, const uint8_t* w2s, int32_t* ids, float* w,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                               int32_t* pair_to_row, uint16_t* h, float* y, float* out,
                               void* workspace, hipStream_t s);
// Rejection-sampling verification of drafted blocks.
size_t verify_workspace_bytes(int B, int L);
hipError_t launch_verify(const float* target, const float* draft, const int32_t* tokens,
                         const float* uniforms, int B, int L, int V, int32_t* accept_len,
                         int32_t* next_token, void* workspace, hipStream_t s);
// XOR of every 32-bit word of src into *result (streaming-read probe).
hipError_t launch_stream_xor(const void* src, int64_t bytes, int nontemporal, uint32_t* result,
                             hipStream_t s);
hipError_t launch_combine(const float* y, const float* w, const int32_t* pair_to_row, int T,
                          int H, int k, float* out, hipStream_t s);

}  // namespace mxm

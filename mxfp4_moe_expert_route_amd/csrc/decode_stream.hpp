// Building blocks of the persistent decode-size expert contractions: the
// weight-stream geometry, the waits and LDS reads of the loader waves, the
// row mapping of a unit, and one stage of the MFMA waves.  Shared by the
// separate gate/up and down kernels (expert_decode.hip) and the fused decode
// layer (decode_layer.hip), so both compute every unit the same way, bit for
// bit.
//
// Geometry.  A unit is 256 weight rows x the whole K of one tile (<= 16 token
// rows of one expert).  A stage is 64 weight rows (a row group) x 512 K
// elements (a K chunk: 256 code bytes = 16 MX blocks per row); a unit runs K
// chunk by K chunk and, within a chunk, over its four row groups, so every
// load instruction reads 256 contiguous bytes of 4 rows.
//   codes   16 loads of 1 KB per stage into a ring slot; row r of the group
//           keeps MX block b at 16-byte slot b ^ (r % 16), so the MFMA lanes
//           (16 rows reading one block each) hit distinct banks
//   acts    per K chunk, one 1 KB load per token row: row j keeps its 16-byte
//           piece c at slot c ^ (j % 8)
//   scales  per unit, the 256 rows' scale bytes as they lie in memory (two
//           runs of 128 rows for gate/up, one for down)
// MFMA wave w owns, in row group g, the weight rows 64g + 16w .. + 15 of the
// unit: for gate/up the unit holds 128 gate columns then the same 128 up
// columns, so the gate rows of group 0 (1) meet their up rows in group 2 (3)
// inside the same wave.
#pragma once
#include "common.hpp"

namespace mxm {
namespace dec {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) int int4v;

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 layout:
// vmcnt low bits 3:0, high bits 15:14; expcnt 6:4 and lgkmcnt 11:8 at max).
#define MXM_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

constexpr int kMW = 4;                          // MFMA waves
constexpr int kCW = 2;                          // code loader waves
constexpr int kThreadsDec = (kMW + kCW + 2) * kWave;   // + activation and scale loaders
constexpr int kUnitRows = 256;                  // weight rows per unit
constexpr int kGroupRows = 64;                  // weight rows per stage
constexpr int kChunkK = 512;                    // K elements per stage
constexpr int kTokRows = 16;                    // token rows per tile
constexpr int kStageB = kGroupRows * kChunkK / 2;   // 16 KB of codes
constexpr int kPerLoader = kStageB / 1024 / kCW;    // loads per code loader per stage
constexpr int kRing = 4;                        // code stages in flight
// cache policy of the code loads: non-temporal.  Each code byte is read
// once, and the hinted stream runs faster (verify_t8: gate/up 141.6 -> 126.9
// us, down 79.0 -> 67.4 us; the measured HBM traffic also fell, to 1.002x
// and 1.008x of the bytes the kernels must read).
constexpr int kAuxNT = 2;
// cache policy bit sc1: coherent at device scope (loads do not hit lines
// another XCD's stores left stale in this XCD's L2; stores write through)
constexpr int kAuxSC1 = 16;
constexpr int kMaxK = 8192;
constexpr int kActBytes = kTokRows * 1024;      // one K chunk of 16 token rows
static_assert(kPerLoader * kCW * 1024 == kStageB, "whole loads per stage");
static_assert((kRing - 2) * kPerLoader <= 63, "vmcnt counts at most 63 loads");

__device__ __forceinline__ lds_void* lds_at(uint8_t* base, int off) {
  return (lds_void*)(base + off);
}

// at most PER * n loads of this wave outstanding, n in [0, NMAX]
template <int PER, int NMAX>
__device__ __forceinline__ void vmcnt_wait_stages(int n) {
  if constexpr (NMAX > 0) {
    if (n >= NMAX) {
      __builtin_amdgcn_s_waitcnt(MXM_VMCNT(PER * NMAX));
      return;
    }
    vmcnt_wait_stages<PER, NMAX - 1>(n);
  } else {
    __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
  }
}

// LDS reads of the loader waves go through inline asm with their wait inside:
// the compiler would otherwise guard every LDS read that follows an
// asynchronous global->LDS load with a full vmcnt drain.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_void*)p));
}
__device__ __forceinline__ int lds_read_i32(const uint8_t* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}
__device__ __forceinline__ int2 lds_read_i32x2(const uint8_t* p) {
  typedef __attribute__((ext_vector_type(2))) int int2v;
  int2v v;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return make_int2(v.x, v.y);
}
__device__ __forceinline__ int4v lds_read_i32x4(const uint8_t* p) {
  int4v v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

// Row (within the whole weight tensor) of unit row u (0..255) of column block
// nt of expert e.  Gate/up: unit rows 0..127 are gate columns 128 nt + u, rows
// 128..255 the same up columns.  Down: rows 256 nt + u.
template <bool GU>
__device__ __forceinline__ int64_t weight_row(int e, int nt, int u, int I, int H) {
  if constexpr (GU) {
    const int col = min(nt * 128 + (u & 127), I - 1);
    return int64_t(e) * 2 * I + (u >= 128 ? I : 0) + col;
  } else {
    return int64_t(e) * H + min(nt * kUnitRows + u, H - 1);
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// byte b of each of the four dwords, packed
__device__ __forceinline__ uint32_t pick_bytes(uint4 v, int b) {
  const int sh = 8 * b;
  return ((v.x >> sh) & 0xffu) | (((v.y >> sh) & 0xffu) << 8) | (((v.z >> sh) & 0xffu) << 16) |
         (((v.w >> sh) & 0xffu) << 24);
}

// Per-lane offsets of a code loader's loads within a row group's first chunk:
// load m of loader ld moves 4 rows x 256 bytes into 1 KB (ld + kCW m) of the
// stage.
__device__ __forceinline__ void code_load_offsets(int ld, int K, uint32_t (&loff)[kPerLoader]) {
  const int lane = lane_id();
#pragma unroll
  for (int m = 0; m < kPerLoader; ++m) {
    const int i = ld + kCW * m;
    const int rr = 4 * i + (lane >> 4);
    loff[m] = uint32_t(rr) * uint32_t(K / 2) + uint32_t(((lane & 15) ^ (rr & 15)) * 16);
  }
}

// Issue one stage of codes: row group base b (already at the stage's K chunk)
// into ring slot st.
__device__ __forceinline__ void code_load_stage(const uint8_t* b, uint8_t* st, int ld,
                                                const uint32_t (&loff)[kPerLoader]) {
#pragma unroll
  for (int m = 0; m < kPerLoader; ++m)
    __builtin_amdgcn_global_load_lds(b + loff[m], lds_at(st, (ld + kCW * m) * 1024), 16, 0,
                                     kAuxNT);
}

// The scale bytes an MFMA lane needs for two K chunks (kc and kc + 1) of its
// four row groups: blocks 16 kc + 4t + g, packed one byte per t.
__device__ __forceinline__ void read_scales(const uint8_t* scb, int nblk, int w, int kc,
                                            uint32_t (&sc4)[2][4]) {
  const int lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint8_t* sp = scb + (kGroupRows * a + 16 * w + r16) * nblk + 16 * kc;
    sc4[0][a] = pick_bytes(*reinterpret_cast<const uint4*>(sp), g);
    sc4[1][a] = pick_bytes(*reinterpret_cast<const uint4*>(sp + 16), g);
  }
}

// The activation operands of one K chunk: token row min(r16, rows - 1).
__device__ __forceinline__ void read_acts(const uint8_t* actb, int rows, uint4 (&xb)[4][4]) {
  const int lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int jr = min(r16, rows - 1);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int c = 16 * t + 4 * g + m;
      xb[t][m] = *reinterpret_cast<const uint4*>(actb + jr * 1024 + ((c ^ (jr & 7)) * 16));
    }
}

// One stage of an MFMA wave: its 16 weight rows of the stage (ring slot st)
// times the chunk's activations, with the stage's four scale bytes packed in
// sc (one per 128-element quarter of the chunk).
__device__ __forceinline__ void mfma_stage(const uint8_t* st, int w, uint32_t sc,
                                           const uint4 (&xb)[4][4], f32x4& acc) {
  const int lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const uint8_t* sr = st + (16 * w + r16) * (kChunkK / 2);
  uint4 cw[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) cw[t] = *reinterpret_cast<const uint4*>(sr + (((4 * t + g) ^ r16) * 16));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float scl = e8m0_to_f32((sc >> (8 * t)) & 0xffu);
    const uint32_t c4[4] = {cw[t].x, cw[t].y, cw[t].z, cw[t].w};
#pragma unroll
    for (int m = 0; m < 4; ++m)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(c4[m], scl), as_bf16x8(xb[t][m]),
                                                    acc, 0, 0, 0);
  }
}

}  // namespace dec
}  // namespace mxm

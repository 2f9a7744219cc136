// Grouped MXFP4 expert contractions for experts with many rows (prefill-like
// batches): an LDS-tiled bf16 MFMA GEMM with the FP4 weights dequantised from
// LDS, fused with SwiGLU (gate/up) or writing fp32 (down).
//
// The pages put the experts in MXFP4 (block 32) with bf16 activations
// ("MiMo-V2.5-Pro-FP4-DFlash" model card, §2 "FP4 Quantization"); when many
// tokens reach each expert the contraction is compute-bound and runs on the
// bf16 matrix cores with fp32 accumulation.
//
// Workgroup: one tile of up to 256 rows of one expert x 128 weight rows.
// Seven waves with separate jobs, so that each has its own in-order load
// counter:
//   waves 0-3  MFMA: a 2 x 2 grid, each wave 128 rows (8 interleaved 16-row
//              subtiles) x 64 weight rows (4 subtiles), 128 fp32 accumulators
//   waves 4-5  activations: global -> LDS ring of kRA stages (buffer loads
//              straight into LDS; rows past the tile's end are out of range
//              and cost no memory traffic)
//   wave  6    weights: codes and scale chunks -> LDS ring of kRW stages
//              (global loads straight into LDS, far ahead of use: they come
//              from HBM)
// A stage is 64 of K (two MX blocks); one barrier per stage hands the ring
// slots from the loaders to the MFMA waves and back.
//
// Register roles follow v_mfma_f32_16x16x32_bf16: weights are operand A (row
// = weight row), activations operand B (row = tile row).  In stage s, lane
// group g covers elements 16g..16g+15 of the stage, MFMA j the 8 from 16g+8j;
// weights and activations use the same assignment.
//
// Workgroup order is XCD-aware: consecutive workgroups go to different XCDs,
// so tile tau and its column tiles are given to one XCD, where they run back
// to back and share that XCD's L2 copy of the tile's activation rows.
#include "common.hpp"

namespace mxm {
namespace {

constexpr int kMT = 256;             // rows per tile (16 subtiles of 16)
constexpr int kNT = 128;             // weight rows per workgroup
constexpr int kKS = 64;              // K per stage (2 MX blocks)
constexpr int kRA = 3;               // activation ring depth, stages
constexpr int kRW = 8;               // weight ring depth, stages
constexpr int kScStages = 8;         // stages per scale chunk (16 blocks = 16 B per row)
constexpr int kMmaWaves = 4;
constexpr int kDThreads = 7 * kWave;
constexpr int kMinRows = 64;         // experts with fewer rows use the streaming kernels

constexpr int kAStage = kMT * kKS * 2;            // 32 KB
constexpr int kWStage = kNT * kKS / 2;            // 4 KB
constexpr int kSChunk = kNT * 16;                 // 2 KB
constexpr int kLdsW = kRA * kAStage;
constexpr int kLdsS = kLdsW + kRW * kWStage;
constexpr int kLdsBytes = kLdsS + 2 * kSChunk;    // 132 KB

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 layout:
// vmcnt low bits 3:0, high bits 15:14; expcnt 6:4 and lgkmcnt 11:8 at max).
#define MXM_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

__device__ __forceinline__ lds_void* lds_at(uint8_t* base, int off) {
  return (lds_void*)(base + off);   // generic -> LDS address space
}

template <bool GU>
__global__ __launch_bounds__(kDThreads) void k_dense(
    const uint16_t* __restrict__ act, uint32_t act_bytes, const int32_t* __restrict__ sorted_pairs,
    const int32_t* __restrict__ offsets, int K, int I, int H, int E, int k,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, void* __restrict__ out,
    int ntile_n, int min_rows) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int lane = lane_id();

  // XCD-aware tile order: blockIdx % 8 picks the XCD.
  const int xcd = blockIdx.x & 7;
  const int j = blockIdx.x >> 3;
  const int lt = j / ntile_n;
  const int nt = j - lt * ntile_n;
  Tile t;
  if (!find_tile(offsets, E, kMT, lt * 8 + xcd, t, min_rows)) return;   // whole workgroup
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
  t.rows = __builtin_amdgcn_readfirstlane(t.rows);

  const int nst = K / kKS;
  const int NW = GU ? 2 * I : H;                  // weight rows per expert
  // weight row (within the expert) of local row r of this workgroup's 128
  auto wrow = [&](int r) {
    if (GU) return r < 64 ? 64 * nt + r : I + 64 * nt + (r - 64);
    return kNT * nt + r;
  };

  if (wave == 6) {
    // ---------------- weight loader ----------------
    const uint8_t* cb = codes + size_t(t.e) * NW * (K / 2);
    const uint8_t* sb = scales + size_t(t.e) * NW * (K / 32);
    const uint8_t* crow[4];
    for (int i = 0; i < 4; ++i) {
      const int c = i * kWave + lane;                 // 16-byte chunk of the stage
      crow[i] = cb + size_t(wrow(c >> 1)) * (K / 2) + (c & 1) * 16;
    }
    const uint8_t* srow[2];
    for (int i = 0; i < 2; ++i) srow[i] = sb + size_t(wrow(i * kWave + lane)) * (K / 32);
    auto issue = [&](int st) {
      if (st % kScStages == 0) {                      // scale chunk before the codes
        const int q = st / kScStages;
        for (int i = 0; i < 2; ++i)
          __builtin_amdgcn_global_load_lds(srow[i] + q * 16,
                                           lds_at(lds, kLdsS + (q & 1) * kSChunk + i * 1024), 16,
                                           0, 0);
      }
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(crow[i] + st * 32,
                                         lds_at(lds, kLdsW + (st % kRW) * kWStage + i * 1024), 16,
                                         0, 0);
    };
    for (int st = 0; st < kRW - 1; ++st) issue(st);   // nst >= kRW (host check)
    __builtin_amdgcn_s_waitcnt(MXM_VMCNT((kRW - 2) * 4));
    __builtin_amdgcn_s_barrier();
    for (int s = 0; s < nst; ++s) {
      if (s + kRW - 1 < nst) {
        issue(s + kRW - 1);
        __builtin_amdgcn_s_waitcnt(MXM_VMCNT((kRW - 2) * 4));   // stage s+1 has landed
      } else {
        __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
      }
      __builtin_amdgcn_s_barrier();
    }
    return;
  }

  if (wave >= kMmaWaves) {
    // ---------------- activation loaders (waves 4, 5) ----------------
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(act), 0, int(act_bytes), 0x00020000);
    const int half = wave - kMmaWaves;                 // which 16 KB of the stage
    uint32_t voff[16];                                 // per chunk: row byte + swizzled chunk
    for (int i = 0; i < 16; ++i) {
      const int c = half * 1024 + i * kWave + lane;    // chunk of the stage, LDS slot c
      const int r = c >> 3;                            // tile row
      const int gc = (c & 7) ^ ((r >> 1) & 7);         // global 16-byte chunk kept in slot c
      const int row = t.row0 + min(r, t.rows - 1);    // unconditional, in-bounds read
      const uint32_t src = GU ? uint32_t(sorted_pairs[row] / k) : uint32_t(row);
      // rows past the tile's end get 2^31 added: out of the buffer's range
      // (act_bytes + K*2 < 2^31), so they cost no memory traffic
      voff[i] = src * uint32_t(K * 2) + uint32_t(gc * 16) + (uint32_t(r >= t.rows) << 31);
    }
    auto issue = [&](int st) {
      for (int i = 0; i < 16; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, lds_at(lds, (st % kRA) * kAStage + (half * 1024 + i * kWave) * 16), 16,
            voff[i] + uint32_t(st * kKS * 2), 0, 0, 0);
    };
    for (int st = 0; st < kRA - 1; ++st) issue(st);
    __builtin_amdgcn_s_waitcnt(MXM_VMCNT((kRA - 2) * 16));
    __builtin_amdgcn_s_barrier();
    for (int s = 0; s < nst; ++s) {
      if (s + kRA - 1 < nst) {
        issue(s + kRA - 1);
        __builtin_amdgcn_s_waitcnt(MXM_VMCNT((kRA - 2) * 16));
      } else {
        __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
      }
      __builtin_amdgcn_s_barrier();
    }
    return;
  }

  // ---------------- MFMA waves 0-3 ----------------
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int nsub = (t.rows + 15) >> 4;
  const int nvalid = max(0, min(8, (nsub - wm + 1) >> 1));   // subtiles wm, wm+2, ... in range
  int wl[4];                                                 // local weight row of subtile a
#pragma unroll
  for (int a = 0; a < 4; ++a)
    wl[a] = GU ? (a < 2 ? 32 * wn + 16 * a : 64 + 32 * wn + 16 * (a - 2)) : 64 * wn + 16 * a;

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[i][a] = f32x4{0.f, 0.f, 0.f, 0.f};

  __builtin_amdgcn_s_barrier();
  for (int s = 0; s < nst; ++s) {
    const uint8_t* wst = lds + kLdsW + (s % kRW) * kWStage;
    const uint8_t* sch = lds + kLdsS + ((s / kScStages) & 1) * kSChunk;
    const uint8_t* ast = lds + (s % kRA) * kAStage;
    const int sblk = (s % kScStages) * 2 + (g >> 1);
    bf16x8 wa[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int row = wl[a] + r16;
      const uint2 cw = *reinterpret_cast<const uint2*>(wst + row * 32 + 8 * g);
      const float sc = e8m0_to_f32(sch[row * 16 + sblk]);
      wa[a][0] = dequant8(cw.x, sc);
      wa[a][1] = dequant8(cw.y, sc);
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < nvalid) {
          const int m = (wm + 2 * i) * 16 + r16;
          const int slot = (2 * g + jj) ^ ((m >> 1) & 7);
          const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(ast + m * 128 + slot * 16));
#pragma unroll
          for (int a = 0; a < 4; ++a)
            acc[i][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[a][jj], b, acc[i][a], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_barrier();
  }

  // epilogue: lane holds D[4g+v][r16] = output column base + 4g + v of tile row m
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = (wm + 2 * i) * 16 + r16;
    if (m >= t.rows) continue;
    const size_t row = size_t(t.row0 + m);
    if (GU) {
      uint16_t* h = static_cast<uint16_t*>(out);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const f32x4 gv = acc[i][a];
        const f32x4 uv = acc[i][a + 2];
        uint32_t hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          hv[v] = f32_to_bf16_rne(gv[v] / (1.0f + __expf(-gv[v])) * uv[v]);
        const int col = 64 * nt + 32 * wn + 16 * a + 4 * g;
        *reinterpret_cast<uint2*>(h + row * I + col) =
            make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
      }
    } else {
      float* y = static_cast<float*>(out);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 v = acc[i][a];
        const int col = kNT * nt + 64 * wn + 16 * a + 4 * g;
        *reinterpret_cast<float4*>(y + row * H + col) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

template <bool GU>
hipError_t launch_dense(const uint16_t* act, uint32_t act_bytes, const int32_t* sorted_pairs,
                        const int32_t* offsets, int T, int H, int I, int E, int k,
                        const uint8_t* codes, const uint8_t* scales, void* out, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dense<GU>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int R = T * k;
  const int K = GU ? H : I;
  const int ntile_n = GU ? I / 64 : H / kNT;
  // tiles: experts with >= kMinRows rows, each cut into tiles of kMT rows
  const int big = min(E, R / kMinRows);
  int slots = big + R / kMT + 1;
  slots = (slots + 7) / 8 * 8;
  const int64_t grid = int64_t(slots) * ntile_n;
  k_dense<GU><<<dim3(unsigned(grid)), kDThreads, kLdsBytes, s>>>(
      act, act_bytes, sorted_pairs, offsets, K, I, H, E, k, codes, scales, out, ntile_n, kMinRows);
  return hipGetLastError();
}

}  // namespace

// The dense path needs K and the column tiles to be whole stages, scale
// chunks and rings, and byte offsets of activation rows that fit the 31-bit
// range of buffer addressing.
bool dense_supported(int T, int H, int I, int E, int k) {
  (void)E;
  const int64_t R = int64_t(T) * k;
  if (H % 512 || I % 512) return false;
  if (int64_t(T) * H * 2 + H * 2 >= (int64_t(1) << 31)) return false;
  if (R * I * 2 + I * 2 >= (int64_t(1) << 31)) return false;
  return R >= kMinRows;
}

int dense_min_rows() { return kMinRows; }

hipError_t launch_gate_up_dense(const uint16_t* x, const int32_t* sorted_pairs,
                                const int32_t* offsets, int T, int H, int I, int E, int k,
                                const uint8_t* codes, const uint8_t* scales, uint16_t* h,
                                hipStream_t s) {
  return launch_dense<true>(x, uint32_t(int64_t(T) * H * 2), sorted_pairs, offsets, T, H, I, E, k,
                            codes, scales, h, s);
}

hipError_t launch_down_dense(const uint16_t* h, const int32_t* offsets, int T, int H, int I,
                             int E, int k, const uint8_t* codes, const uint8_t* scales, float* y,
                             hipStream_t s) {
  return launch_dense<false>(h, uint32_t(int64_t(T) * k * I * 2), nullptr, offsets, T, H, I, E, k,
                             codes, scales, y, s);
}

}  // namespace mxm

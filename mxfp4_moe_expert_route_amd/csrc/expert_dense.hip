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
// Eleven waves with separate jobs, so that each has its own in-order load
// counter:
//   waves 0-7  MFMA: a 4 x 2 grid, each wave 64 rows (4 interleaved 16-row
//              subtiles) x 64 weight rows (4 subtiles), 64 fp32 accumulators;
//              two MFMA waves per SIMD hide each other's LDS and barrier waits
//   waves 8-9  activations: global -> LDS ring of kRA stages (buffer loads
//              straight into LDS; rows past the tile's end are out of range
//              and cost no memory traffic)
//   wave  10   weights: codes and scale chunks -> LDS ring of kRW stages
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
// LDS layouts are swizzled so that the MFMA waves' reads hit distinct banks
// (128-byte bank rows): activation row r keeps its 16-byte chunk c in slot
// c ^ (r & 7); weight row r keeps its two 16-byte blocks swapped when bit 2
// of r is set.
//
// Workgroup order is XCD-aware: consecutive workgroups go to different XCDs,
// so tile tau and its column tiles are given to one XCD, where they run back
// to back and share that XCD's L2 copy of the tile's activation rows.
#include "common.hpp"

namespace mxm {
namespace {

// Tunables (compile-time; defaults are the measured best on MI355X).
#ifndef MXM_DENSE_MT
#define MXM_DENSE_MT 256
#endif
#ifndef MXM_DENSE_RA
#define MXM_DENSE_RA 4
#endif
#ifndef MXM_DENSE_RW
#define MXM_DENSE_RW 6
#endif
constexpr int kMT = MXM_DENSE_MT;    // rows per tile (a multiple of 64: 4 row waves x 16)
constexpr int kNT = 128;             // weight rows per workgroup
constexpr int kKS = 64;              // K per stage (2 MX blocks)
constexpr int kRA = MXM_DENSE_RA;    // activation ring depth, stages
constexpr int kRW = MXM_DENSE_RW;    // weight ring depth, stages
constexpr int kMSub = kMT / 64;      // row subtiles per MFMA wave
constexpr int kAInstr = kMT / 16;    // 16-byte loads per lane per stage, per activation loader
constexpr int kScStages = 8;         // stages per scale chunk (16 blocks = 16 B per row)
constexpr int kMmaWaves = 8;
constexpr int kDThreads = 11 * kWave;
constexpr int kMinRows = 64;         // experts with fewer rows use the streaming kernels

constexpr int kAStage = kMT * kKS * 2;            // 32 KB at 256 rows
constexpr int kWStage = kNT * kKS / 2;            // 4 KB
constexpr int kSChunk = kNT * 16;                 // 2 KB
constexpr int kLdsW = kRA * kAStage;
constexpr int kLdsS = kLdsW + kRW * kWStage;
constexpr int kLdsBytes = kLdsS + 2 * kSChunk;    // 132 KB at the defaults
static_assert(kMT % 64 == 0 && kMSub <= 4, "tile rows");
static_assert(kLdsBytes <= 160 * 1024, "LDS");
static_assert((kRA - 2) * kAInstr <= 63 && (kRW - 2) * 4 <= 63, "vmcnt range");
// the two scale-chunk slots are reused 16 stages apart: chunk q+2 is issued
// kRW-1 stages before stage 8q+16, after chunk q's last use at stage 8q+7
static_assert(kRW <= 9, "scale chunk ring");

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 layout:
// vmcnt low bits 3:0, high bits 15:14; expcnt 6:4 and lgkmcnt 11:8 at max).
#define MXM_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

// s_waitcnt for "at most STAGES * n loads outstanding", n a runtime count in
// [0, NMAX] (the immediate must be a constant, hence the switch).
template <int STAGES, int NMAX>
__device__ __forceinline__ void vmcnt_wait_stages(int n) {
  if constexpr (NMAX > 0) {
    if (n == NMAX) {
      __builtin_amdgcn_s_waitcnt(MXM_VMCNT(STAGES * NMAX));
      return;
    }
    vmcnt_wait_stages<STAGES, NMAX - 1>(n);
  } else {
    __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
  }
}

__device__ __forceinline__ lds_void* lds_at(uint8_t* base, int off) {
  return (lds_void*)(base + off);   // generic -> LDS address space
}

// The MFMA waves' K loop for NV valid row subtiles (wm, wm+4, ...): one
// barrier per stage, then dequantise this wave's 4 weight subtiles from LDS
// and run NV x 4 x 2 MFMAs against the activation subtiles.
template <int NV>
__device__ __forceinline__ void mma_kloop(const uint8_t* lds, int nst, int wm, int g, int r16,
                                          const int (&wl)[4], f32x4 (&acc)[4][4]) {
  __builtin_amdgcn_s_barrier();
  for (int s = 0; s < nst; ++s) {
    const uint8_t* wst = lds + kLdsW + (s % kRW) * kWStage;
    const uint8_t* sch = lds + kLdsS + ((s / kScStages) & 1) * kSChunk;
    const uint8_t* ast = lds + (s % kRA) * kAStage;
    const int sblk = (s % kScStages) * 2 + (g >> 1);
    // issue every LDS read of the stage first: weight codes and scales of the
    // 4 weight subtiles, activation operands of both K halves
    uint2 cw[4];
    uint32_t sb[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int row = wl[a] + r16;
      const int slot = 2 * row + ((g >> 1) ^ ((row >> 2) & 1));
      cw[a] = *reinterpret_cast<const uint2*>(wst + slot * 16 + 8 * (g & 1));
      sb[a] = sch[row * 16 + sblk];
    }
    uint4 b[2][NV > 0 ? NV : 1];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int m = (wm + 4 * i) * 16 + r16;
        const int slot = (2 * g + jj) ^ (m & 7);
        b[jj][i] = *reinterpret_cast<const uint4*>(ast + m * 128 + slot * 16);
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      bf16x8 wa[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        wa[a] = dequant8(jj ? cw[a].y : cw[a].x, e8m0_to_f32(sb[a]));
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          acc[i][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[a], as_bf16x8(b[jj][i]),
                                                              acc[i][a], 0, 0, 0);
    }
    __builtin_amdgcn_s_barrier();
  }
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

  if (wave == kMmaWaves + 2) {
    // ---------------- weight loader ----------------
    const uint8_t* cb = codes + size_t(t.e) * NW * (K / 2);
    const uint8_t* sb = scales + size_t(t.e) * NW * (K / 32);
    const uint8_t* crow[4];
    for (int i = 0; i < 4; ++i) {
      const int c = i * kWave + lane;                 // LDS slot (16 bytes) of the stage
      const int r = c >> 1;                           // local weight row
      const int blk = (c & 1) ^ ((r >> 2) & 1);       // which of the row's 2 blocks sits here
      crow[i] = cb + size_t(wrow(r)) * (K / 2) + blk * 16;
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
    // ---------------- activation loaders (waves 8, 9) ----------------
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(act), 0, int(act_bytes), 0x00020000);
    const int half = wave - kMmaWaves;                 // which half of the stage's rows
    uint32_t voff[kAInstr];                            // per chunk: row byte + swizzled chunk
    for (int i = 0; i < kAInstr; ++i) {
      const int c = half * kAInstr * kWave + i * kWave + lane;   // chunk of the stage = LDS slot
      const int r = c >> 3;                            // tile row
      const int gc = (c & 7) ^ (r & 7);                // global 16-byte chunk kept in slot c
      const int row = t.row0 + min(r, t.rows - 1);    // unconditional, in-bounds read
      const uint32_t src = GU ? uint32_t(sorted_pairs[row] / k) : uint32_t(row);
      // rows past the tile's end get 2^31 added: out of the buffer's range
      // (act_bytes + K*2 < 2^31), so they cost no memory traffic
      voff[i] = src * uint32_t(K * 2) + uint32_t(gc * 16) + (uint32_t(r >= t.rows) << 31);
    }
    // one load instruction covers 8 tile rows: skip the ones wholly past the
    // tile's end (their LDS rows are never read)
    const int na = __builtin_amdgcn_readfirstlane(
        max(0, min(kAInstr, (t.rows - half * kAInstr * 8 + 7) >> 3)));
    auto issue = [&](int st) {
      for (int i = 0; i < kAInstr; ++i)
        if (i < na)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, lds_at(lds, (st % kRA) * kAStage + (half * kAInstr + i) * kWave * 16), 16,
              voff[i] + uint32_t(st * kKS * 2), 0, 0, 0);
    };
    // wait until at most (kRA-2) stages of this wave's loads are outstanding
    auto wait_lead = [&]() { vmcnt_wait_stages<kRA - 2, kAInstr>(na); };
    for (int st = 0; st < kRA - 1; ++st) issue(st);
    wait_lead();
    __builtin_amdgcn_s_barrier();
    for (int s = 0; s < nst; ++s) {
      if (s + kRA - 1 < nst) {
        issue(s + kRA - 1);
        wait_lead();
      } else {
        __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
      }
      __builtin_amdgcn_s_barrier();
    }
    return;
  }

  // ---------------- MFMA waves 0-7 ----------------
  const int wm = wave & 3;
  const int wn = wave >> 2;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int nsub = (t.rows + 15) >> 4;
  const int nvalid = max(0, min(kMSub, (nsub - wm + 3) >> 2));  // subtiles wm, wm+4, ... in range
  int wl[4];                                                 // local weight row of subtile a
#pragma unroll
  for (int a = 0; a < 4; ++a)
    wl[a] = GU ? (a < 2 ? 32 * wn + 16 * a : 64 + 32 * wn + 16 * (a - 2)) : 64 * wn + 16 * a;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[i][a] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The K loop is instantiated per count of valid row subtiles so that its
  // body has no branch and the compiler can keep LDS reads ahead of MFMAs.
  switch (nvalid) {
    case 4: mma_kloop<4>(lds, nst, wm, g, r16, wl, acc); break;
    case 3: mma_kloop<3>(lds, nst, wm, g, r16, wl, acc); break;
    case 2: mma_kloop<2>(lds, nst, wm, g, r16, wl, acc); break;
    case 1: mma_kloop<1>(lds, nst, wm, g, r16, wl, acc); break;
    default: mma_kloop<0>(lds, nst, wm, g, r16, wl, acc); break;
  }

  // epilogue: lane holds D[4g+v][r16] = output column base + 4g + v of tile row m
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = (wm + 4 * i) * 16 + r16;
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

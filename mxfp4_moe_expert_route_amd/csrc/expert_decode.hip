// Persistent grouped MXFP4 expert contractions for decode-sized batches
// (gate/up + SwiGLU, and down), one workgroup per CU.
//
// At a verify step (8 tokens per sequence, "MiMo-V2.5-Pro-FP4-DFlash" model
// card §3) nearly every chosen expert sees one or two token rows, so the cost
// is the stream of FP4 weight bytes (§2 "FP4 Quantization": E2M1 codes with
// an E8M0 scale per 32 weights).  To keep HBM saturated from the first byte
// to the last, this kernel
//   * keeps the weight stream in flight with asynchronous global->LDS loads
//     issued by three loader waves into a ring of stages, so the depth of the
//     stream does not depend on registers;
//   * splits the work into units of 256 weight rows x the whole K of one
//     tile (<= 16 token rows of one expert) and hands every workgroup an
//     equal contiguous run of units; the stream crosses unit boundaries
//     without a pause;
//   * runs the contraction on MFMA waves that read codes, scales and
//     activations from LDS (v_mfma_f32_16x16x32_bf16 after the scaled FP4 ->
//     bf16 conversion), with one workgroup barrier per stage.
//
// Stage = 4 MX blocks (128 K elements) of the unit, 21 asynchronous loads:
//   16 x codes  1 KB each: subtile i (16 rows) at i KB; lane L holds row L%16,
//               block 4s + L/16 (the MFMA operand layout: each lane reads back
//               its own 16 bytes)
//    1 x scales one sixteenth of the scale chunk that follows the current one
//    4 x acts   16 token rows x 256 bytes; the 16-byte chunk c of row j sits
//               at position c ^ j, so lanes reading different rows hit
//               different banks
// Scales travel in chunks of 64 MX blocks (16 stages) x 256 rows: one load
// covers 16 rows x 64 contiguous bytes, so it touches as few cache lines per
// byte as the code loads.  Three chunk buffers: a chunk is loaded during the
// previous chunk's stages, into the buffer freed two chunks before.
// Accumulation order per output is that of the streaming kernel (MX block
// 4s+g in lane group g, MFMA j over elements 8j..8j+7, steps in order), so the
// results are the same bit for bit.
#include "common.hpp"

namespace mxm {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) int int4v;

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 layout:
// vmcnt low bits 3:0, high bits 15:14; expcnt 6:4 and lgkmcnt 11:8 at max).
#define MXM_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

#ifndef MXM_DEC_MW
#define MXM_DEC_MW 4
#endif
#ifndef MXM_DEC_RING
#define MXM_DEC_RING 4
#endif
constexpr int kMW = MXM_DEC_MW;                 // MFMA waves (4 or 8)
constexpr int kNA = 16 / kMW;                   // 16-row weight subtiles per MFMA wave
constexpr int kLW = 3;                          // loader waves
constexpr int kThreadsDec = (kMW + kLW) * kWave;
constexpr int kUnitRows = 256;                  // weight rows per unit (16 subtiles)
constexpr int kTokRows = 16;                    // token rows per tile
constexpr int kCodesB = 16 * 1024;
constexpr int kStageB = kCodesB + kTokRows * 256;
constexpr int kRing = MXM_DEC_RING;             // stages in the LDS ring
constexpr int kChunkSteps = 16;                 // stages per scale chunk (64 MX blocks)
constexpr int kChunkB = kUnitRows * 64;
constexpr int kGroup = 21;                      // asynchronous loads per stage
constexpr int kPerLoader = kGroup / kLW;
constexpr int kMaxE = 1024;
constexpr int kMaxUnits = 64;                   // units per workgroup
constexpr int kMaxTokIds = (kMaxUnits + 2) * kTokRows;
constexpr int kLdsChunks = kRing * kStageB;
constexpr int kLdsUnits = kLdsChunks + 3 * kChunkB;           // {e, nt, row0, rows} per unit
constexpr int kLdsOffsets = kLdsUnits + kMaxUnits * 16;       // offsets[0..E]
constexpr int kLdsTok = kLdsOffsets + (kMaxE + 1) * 4 + 12;   // token ids, 16 slots per tile
constexpr int kLdsDec = kLdsTok + kMaxTokIds * 4;
static_assert(kMW == 4 || kMW == 8, "MFMA waves");
static_assert(kGroup % kLW == 0, "equal loads per loader wave");
static_assert((kRing - 1) * kPerLoader + 16 <= 63, "vmcnt counts at most 63 loads");
static_assert(kRing <= kChunkSteps, "chunk buffer reuse");
static_assert(kLdsDec <= 160 * 1024, "LDS per CU");

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
__device__ __forceinline__ int4v lds_read_i32x4(const uint8_t* p) {
  int4v v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

// Tiles of 16 rows over experts with 1 <= rows < hi (offsets in LDS; only
// the MFMA waves call these).  Whole wave, uniform results.
__device__ int count_tiles(const int* offs, int E, int hi) {
  const int lane = lane_id();
  int total = 0;
  for (int c0 = 0; c0 < E; c0 += kWave) {
    const int e = c0 + lane;
    int cnt = e < E ? offs[e + 1] - offs[e] : 0;
    if (cnt < 1 || cnt >= hi) cnt = 0;
    const int incl = wave_incl_scan((cnt + kTokRows - 1) / kTokRows);
    total += __shfl(incl, kWave - 1);
  }
  return __builtin_amdgcn_readfirstlane(total);
}

__device__ Tile tile_at(const int* offs, int E, int hi, int tau) {
  const int lane = lane_id();
  Tile t{0, 0, 1};
  int base = 0;
  for (int c0 = 0; c0 < E; c0 += kWave) {
    const int e = c0 + lane;
    int off = 0, cnt = 0;
    if (e < E) {
      off = offs[e];
      cnt = offs[e + 1] - off;
    }
    if (cnt < 1 || cnt >= hi) cnt = 0;
    const int nt = (cnt + kTokRows - 1) / kTokRows;
    const int incl = wave_incl_scan(nt);
    const int total = __shfl(incl, kWave - 1);
    if (tau < base + total) {
      const int excl = base + incl - nt;
      const unsigned long long m = __ballot(tau >= excl && tau < excl + nt);
      const int src = __ffsll((long long)m) - 1;
      const int ti = tau - __shfl(excl, src);
      t.e = __builtin_amdgcn_readfirstlane(c0 + src);
      t.row0 = __builtin_amdgcn_readfirstlane(__shfl(off, src) + ti * kTokRows);
      t.rows = __builtin_amdgcn_readfirstlane(min(kTokRows, __shfl(cnt, src) - ti * kTokRows));
      return t;
    }
    base += total;
  }
  return t;
}

// Weight row (within the whole tensor) of row r of unit subtile i (0..15) in
// column block nt of expert e.  Gate/up: MFMA wave w = i / kNA owns kNA/2
// column subtiles; its first kNA/2 subtiles are their gate rows, the others
// the matching up rows.  Rows past the end are clamped to a valid row whose
// results are never stored.
template <bool GU>
__device__ __forceinline__ int64_t weight_row(int e, int nt, int i, int r, int I, int H) {
  if constexpr (GU) {
    constexpr int kHalf = kNA / 2;
    const int w = i / kNA, a = i % kNA;
    const int col = min(nt * 128 + w * 16 * kHalf + 16 * (a % kHalf) + r, I - 1);
    return int64_t(e) * 2 * I + (a >= kHalf ? I : 0) + col;
  } else {
    return int64_t(e) * H + min(nt * kUnitRows + 16 * i + r, H - 1);
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// GU: act = x (bf16 [T, H]), K = H, out = h (bf16 [R, I]).
// !GU: act = h (bf16 [R, I]), K = I, out = y (fp32 [R, H]).
// Requires K % 2048 == 0 and a run of at most kMaxUnits units per workgroup.
// Experts with fewer than `hi` rows take part.
template <bool GU>
__global__ __launch_bounds__(kThreadsDec) void k_decode(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ sorted_pairs,
    const int32_t* __restrict__ offsets, int K, int I, int H, int E, int k,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, void* __restrict__ out,
    int ntile_n, int hi) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int nsteps = K / 128;
  const int nblk = K / 32;
  int* offs = reinterpret_cast<int*>(lds + kLdsOffsets);
  int* tok_ids = reinterpret_cast<int*>(lds + kLdsTok);
  int4v* units = reinterpret_cast<int4v*>(lds + kLdsUnits);

  // ---- set-up (MFMA waves; loaders issue no global loads besides their
  // asynchronous ones): expert offsets, then the run's unit table and the
  // token ids of its tiles
  if (wave < kMW)
    for (int i = threadIdx.x; i <= E; i += kMW * kWave) offs[i] = offsets[i];
  __syncthreads();
  const int G = gridDim.x;
  int u0 = 0, u1 = 0;
  if (wave < kMW) {
    const int U = count_tiles(offs, E, hi) * ntile_n;
    u0 = int((int64_t(U) * blockIdx.x) / G);
    u1 = int((int64_t(U) * (blockIdx.x + 1)) / G);
    if (u1 > u0) {
      const int tau0 = u0 / ntile_n;
      for (int tau = tau0 + wave; tau <= (u1 - 1) / ntile_n; tau += kMW) {
        const Tile t = tile_at(offs, E, hi, tau);
        if (GU && lane < t.rows)
          tok_ids[(tau - tau0) * kTokRows + lane] = sorted_pairs[t.row0 + lane] / k;
        const int ua = max(u0, tau * ntile_n), ub = min(u1, (tau + 1) * ntile_n);
        if (lane < ub - ua) units[ua - u0 + lane] = int4v{t.e, ua + lane - tau * ntile_n, t.row0, t.rows};
      }
    }
    if (wave == 0 && lane == 0) {
      offs[kMaxE + 1] = u0;         // the run, for the loader waves
      offs[kMaxE + 2] = u1;
    }
  }
  __syncthreads();
  if (wave >= kMW) {
    u0 = lds_read_i32(lds + kLdsOffsets + 4 * (kMaxE + 1));
    u1 = lds_read_i32(lds + kLdsOffsets + 4 * (kMaxE + 2));
  }
  u0 = __builtin_amdgcn_readfirstlane(u0);
  u1 = __builtin_amdgcn_readfirstlane(u1);
  const int nu = u1 - u0;
  const int Q = nu * nsteps;                              // stages of the run
  if (Q == 0) return;
  const int tau0 = u0 / ntile_n;
  const int nchunk = nu * (nsteps / kChunkSteps);         // scale chunks of the run

  if (wave >= kMW) {
    // ---------------- loader waves ----------------
    const int ld = wave - kMW;
    // unit info (e, nt, row0, rows) of the run's unit j
    auto unit = [&](int j) { return lds_read_i32x4(lds + kLdsUnits + 16 * j); };
    // activation row of token slot jj of unit info ui
    auto act_row = [&](const int4v& ui, int j, int jj) -> int64_t {
      const int jc = min(jj, ui.w - 1);
      if constexpr (GU) {
        const int tau = (u0 + j) / ntile_n;
        return lds_read_i32(lds + kLdsTok + 4 * ((tau - tau0) * kTokRows + jc));
      } else {
        return int64_t(ui.z) + jc;
      }
    };
    // scale chunk x (index in the run): load j (= subtile j: 16 rows x 64 B)
    auto issue_scale = [&](int x, int jld, int xbuf) {
      const int xu = min(x, nchunk - 1);                    // past the end: harmless reload
      const int cpu = nsteps / kChunkSteps;
      const int ju = xu / cpu, c = xu - ju * cpu;
      const int4v ui = unit(ju);
      const uint8_t* src = scales + weight_row<GU>(ui.x, ui.y, jld, lane >> 2, I, H) * nblk +
                           64 * c + 16 * (lane & 3);
      __builtin_amdgcn_global_load_lds(src, lds_at(lds, kLdsChunks + (xbuf % 3) * kChunkB + 1024 * jld),
                                       16, 0, 0);
    };
    // chunk 0: loads j = ld, ld + 3, ... before the first stage group
    for (int j = ld; j < 16; j += kLW) issue_scale(0, j, 0);
    // cached per unit: this lane's source of each owned load at step 0
    const uint8_t* src[kPerLoader];
    int cur = -1;
    auto issue = [&](int p) {                               // stage group p
      const int j = p / nsteps, s = p - j * nsteps;
      if (j != cur) {
        cur = j;
        const int4v ui = unit(j);
#pragma unroll
        for (int m = 0; m < kPerLoader; ++m) {
          const int idx = ld + kLW * m;
          if (idx < 16) {
            src[m] = codes + weight_row<GU>(ui.x, ui.y, idx, r16, I, H) * (K / 2) + g * 16;
          } else if (idx > 16) {
            const int mm = idx - 17, jj = 4 * mm + (lane >> 4), pos = lane & 15;
            const int c = pos ^ jj;                          // logical chunk stored at pos
            src[m] = reinterpret_cast<const uint8_t*>(act) +
                     (act_row(ui, j, jj) * K + (c >> 2) * 32 + (c & 3) * 8) * 2;
          }
        }
      }
      uint8_t* st = lds + (p % kRing) * kStageB;
#pragma unroll
      for (int m = 0; m < kPerLoader; ++m) {
        const int idx = ld + kLW * m;
        if (idx < 16) {
          __builtin_amdgcn_global_load_lds(src[m] + s * 64, lds_at(st, idx * 1024), 16, 0, 0);
        } else if (idx == 16) {
          const int x = j * (nsteps / kChunkSteps) + s / kChunkSteps;   // chunk of stage p
          issue_scale(x + 1, s % kChunkSteps, x + 1);
        } else {
          __builtin_amdgcn_global_load_lds(src[m] + s * 256, lds_at(st, kCodesB + 1024 * (idx - 17)),
                                           16, 0, 0);
        }
      }
    };
    const int pre = min(kRing - 1, Q);
    for (int p = 0; p < pre; ++p) issue(p);
    vmcnt_wait_stages<kPerLoader, kRing - 2>(pre - 1);     // chunk 0 and stage 0 landed
    for (int q = 0; q < Q; ++q) {
      __builtin_amdgcn_s_barrier();
      if (q + kRing - 1 < Q) issue(q + kRing - 1);
      if (q + 1 < Q) vmcnt_wait_stages<kPerLoader, kRing - 2>(min(q + kRing - 1, Q - 1) - (q + 1));
    }
    return;
  }

  // ---------------- MFMA waves ----------------
  const int w = wave;
  f32x4 acc[kNA];
  int4v ui{0, 0, 0, 1};
  int s = 0, j = 0, x = 0;
  for (int q = 0; q < Q; ++q) {
    if (s == 0) {
      ui = units[j];
#pragma unroll
      for (int a = 0; a < kNA; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_s_barrier();
    const uint8_t* st = lds + (q % kRing) * kStageB;
    const uint8_t* sc = lds + kLdsChunks + (x % 3) * kChunkB;
    uint4 cw[kNA];
    uint32_t sb[kNA];
    uint4 xb[4];
#pragma unroll
    for (int a = 0; a < kNA; ++a) {
      const int i = w * kNA + a;
      cw[a] = *reinterpret_cast<const uint4*>(st + i * 1024 + 16 * lane);
      sb[a] = sc[(16 * i + r16) * 64 + ((4 * s + g) & 63)];
    }
    const int jr = min(r16, ui.w - 1);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      xb[m] = *reinterpret_cast<const uint4*>(st + kCodesB + jr * 256 + 16 * ((4 * g + m) ^ jr));
#pragma unroll
    for (int a = 0; a < kNA; ++a) {
      const float scl = e8m0_to_f32(sb[a]);
      const uint32_t c4[4] = {cw[a].x, cw[a].y, cw[a].z, cw[a].w};
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dequant8(c4[m], scl), as_bf16x8(xb[m]),
                                                         acc[a], 0, 0, 0);
    }
    ++s;
    if (s % kChunkSteps == 0) ++x;
    if (s == nsteps) {
      // lane holds D[4g+v][r16]: weight row 4g+v of the subtile, token row r16
      const int nt = ui.y, row0 = ui.z, rows = ui.w;
      if (r16 < rows) {
        if constexpr (GU) {
          constexpr int kHalf = kNA / 2;
          uint16_t* h = reinterpret_cast<uint16_t*>(out);
#pragma unroll
          for (int a = 0; a < kHalf; ++a) {
            const int col = nt * 128 + w * 16 * kHalf + 16 * a + 4 * g;
            if (col < I) {
              const f32x4 gv = acc[a], uv = acc[a + kHalf];
              const uint32_t h0 = f32_to_bf16_rne(silu_mul(gv[0], uv[0]));
              const uint32_t h1 = f32_to_bf16_rne(silu_mul(gv[1], uv[1]));
              const uint32_t h2 = f32_to_bf16_rne(silu_mul(gv[2], uv[2]));
              const uint32_t h3 = f32_to_bf16_rne(silu_mul(gv[3], uv[3]));
              *reinterpret_cast<uint2*>(h + size_t(row0 + r16) * I + col) =
                  make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
            }
          }
        } else {
          float* y = reinterpret_cast<float*>(out);
#pragma unroll
          for (int a = 0; a < kNA; ++a) {
            const int n = nt * kUnitRows + 16 * (w * kNA + a) + 4 * g;
            if (n < H) {
              const f32x4 v = acc[a];
              *reinterpret_cast<float4*>(y + size_t(row0 + r16) * H + n) =
                  make_float4(v[0], v[1], v[2], v[3]);
            }
          }
        }
      }
      s = 0;
      ++j;
    }
  }
}

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
      v = 256;
    n = v;
  }
  return n;
}

// Upper bound of the units a workgroup can get (the host does not know the
// counts; tiles <= min(E, R) + R / 16).
int64_t max_units_per_wg(int R, int E, int ntile_n) {
  const int64_t tiles = int64_t(R < E ? R : E) + R / kTokRows;
  const int64_t U = tiles * ntile_n;
  const int G = cu_count();
  return (U + G - 1) / G + 1;
}

template <bool GU>
hipError_t launch_decode(const uint16_t* act, const int32_t* sp, const int32_t* off, int H, int I,
                         int E, int k, const uint8_t* c, const uint8_t* sc, void* out, int hi,
                         hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode<GU>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsDec);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int K = GU ? H : I;
  const int ntile_n = GU ? (I + 127) / 128 : (H + kUnitRows - 1) / kUnitRows;
  k_decode<GU><<<dim3(unsigned(cu_count())), kThreadsDec, kLdsDec, s>>>(
      act, sp, off, K, I, H, E, k, c, sc, out, ntile_n, hi);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int T, int H, int I, int E, int k) {
  if (H % 2048 || I % 2048 || E > kMaxE) return false;
  const int R = T * k;
  return max_units_per_wg(R, E, I / 128) <= kMaxUnits &&
         max_units_per_wg(R, E, (H + kUnitRows - 1) / kUnitRows) <= kMaxUnits;
}

hipError_t launch_gate_up_decode(const uint16_t* x, const int32_t* sorted_pairs,
                                 const int32_t* offsets, int T, int H, int I, int E, int k,
                                 const uint8_t* codes, const uint8_t* scales, uint16_t* h, int hi,
                                 hipStream_t s) {
  (void)T;
  return launch_decode<true>(x, sorted_pairs, offsets, H, I, E, k, codes, scales, h, hi, s);
}

hipError_t launch_down_decode(const uint16_t* h, const int32_t* offsets, int T, int H, int I,
                              int E, int k, const uint8_t* codes, const uint8_t* scales, float* y,
                              int hi, hipStream_t s) {
  (void)T;
  return launch_decode<false>(h, nullptr, offsets, H, I, E, k, codes, scales, y, hi, s);
}

}  // namespace mxm

// Persistent grouped MXFP4 expert contractions for decode-sized batches
// (gate/up + SwiGLU, and down), one workgroup per CU.
//
// At a verify step (8 tokens per sequence, "MiMo-V2.5-Pro-FP4-DFlash" model
// card §3) nearly every chosen expert sees one or two token rows, so the cost
// is the stream of FP4 weight bytes (§2 "FP4 Quantization": E2M1 codes with
// an E8M0 scale per 32 weights).  To keep HBM saturated from the first byte
// to the last, this kernel
//   * splits the work into units of 256 weight rows x the whole K of one
//     tile (<= 16 token rows of one expert) and hands every workgroup an
//     equal contiguous run of units; the stream crosses unit boundaries
//     without a pause;
//   * streams the codes with asynchronous global->LDS loads, issued by two
//     loader waves into a ring of stages; a third loader wave brings each K
//     chunk's activation rows and a fourth each unit's block scales (every
//     loader wave waits only on its own loads);
//   * runs the contraction on four MFMA waves (v_mfma_f32_16x16x32_bf16
//     after the scaled FP4 -> bf16 conversion), one workgroup barrier per
//     stage.
//
// The stage geometry, the LDS layouts of codes, activations and scales and
// the MFMA waves' row ownership are described in decode_stream.hpp.
#include "decode_stream.hpp"

namespace mxm {
namespace {

using namespace dec;

constexpr int kMaxE = 1024;
constexpr int kMaxUnits = 64;                   // units per workgroup
constexpr int kLdsActs = kRing * kStageB;                       // 16 rows x 1 KB
constexpr int kLdsScales = kLdsActs + kTokRows * 1024;          // 256 rows x K/32
constexpr int kLdsUnits = kLdsScales + kUnitRows * (kMaxK / 32);
constexpr int kLdsDec = kLdsUnits + kMaxUnits * 16;
// the set-up's per-wave sums live in the activation buffer until the first chunk lands
constexpr int kLdsWsum = kLdsActs;
static_assert(2 * kThreadsDec >= kMaxE, "two experts per thread in the set-up");
static_assert(kLdsDec <= 160 * 1024, "LDS per CU");

// GU: act = x (bf16 [T, H]), K = H, out = h (bf16 [R, I]).
// !GU: act = h (bf16 [R, I]), K = I, out = y (fp32 [R, H]).
// Requires K % 512 == 0, K <= kMaxK, I % 128 == 0, H % 256 == 0 and a run of
// at most kMaxUnits units per workgroup.  Experts with fewer than `hi` rows
// take part.
template <bool GU>
__global__ __launch_bounds__(kThreadsDec) void k_decode(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ sorted_pairs,
    const int32_t* __restrict__ offsets, int K, int I, int H, int E, int k,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, void* __restrict__ out,
    int ntile_n, int hi) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int nblk = K / 32;
  const int S = 4 * (K / kChunkK);                 // stages per unit
  int* wsum = reinterpret_cast<int*>(lds + kLdsWsum);
  int4v* units = reinterpret_cast<int4v*>(lds + kLdsUnits);

  // ---- set-up: thread t owns experts 2t and 2t + 1; their tiles, one
  // workgroup-wide scan over experts, then each thread writes the units of
  // its own tiles that fall in this workgroup's run
  const int ea = 2 * tid;
  int off[3] = {0, 0, 0};
  if (ea < E) {
    off[0] = offsets[ea];
    off[1] = offsets[ea + 1];
    if (ea + 1 < E) off[2] = offsets[ea + 2];
  }
  int cnt[2], nt[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    cnt[i] = ea + i < E ? off[i + 1] - off[i] : 0;
    if (cnt[i] < 1 || cnt[i] >= hi) cnt[i] = 0;
    nt[i] = (cnt[i] + kTokRows - 1) / kTokRows;
  }
  const int incl = wave_incl_scan(nt[0] + nt[1]);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0, tiles = 0;
#pragma unroll
  for (int v = 0; v < kThreadsDec / kWave; ++v) {
    const int ws = wsum[v];
    before += v < wave ? ws : 0;
    tiles += ws;
  }
  const int G = gridDim.x;
  const int U = tiles * ntile_n;
  const int u0 = __builtin_amdgcn_readfirstlane(int((int64_t(U) * blockIdx.x) / G));
  const int u1 = __builtin_amdgcn_readfirstlane(int((int64_t(U) * (blockIdx.x + 1)) / G));
  const int nu = u1 - u0;
  int tfirst = before + incl - nt[0] - nt[1];    // first tile of expert ea
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ulo = max(u0, tfirst * ntile_n), uhi = min(u1, (tfirst + nt[i]) * ntile_n);
    for (int u = ulo; u < uhi; ++u) {
      const int tau = u / ntile_n;
      const int ti = tau - tfirst;
      const int row0 = off[i] + ti * kTokRows;
      units[u - u0] = int4v{ea + i, u - tau * ntile_n, row0, min(kTokRows, cnt[i] - ti * kTokRows)};
    }
    tfirst += nt[i];
  }
  __syncthreads();
  const int Q = nu * S;                            // stages of the run
  if (Q == 0) return;
  const int pre = min(kRing - 1, Q);

  if (wave == kMW + kCW + 1) {
    // ---------------- scale loader ----------------
    const int half = 128 * nblk;                   // bytes of 128 rows (a multiple of 1 KB)
    const int nsl = kUnitRows * nblk / 1024;       // 1 KB loads per unit
    auto issue_scales = [&](int j, int m0, int m1) {
      const int4v ui = lds_read_i32x4(lds + kLdsUnits + 16 * j);
      for (int m = m0; m < m1; ++m) {
        const int o = 1024 * m + 16 * lane;
        const uint8_t* src;
        if constexpr (GU) {
          const int h2 = o >= half;
          src = scales + weight_row<true>(ui.x, ui.y, h2 ? 128 : 0, I, H) * nblk + (o - h2 * half);
        } else {
          src = scales + weight_row<false>(ui.x, ui.y, 0, I, H) * nblk + o;
        }
        __builtin_amdgcn_global_load_lds(src, lds_at(lds, kLdsScales + 1024 * m), 16, 0, 0);
      }
    };
    issue_scales(0, 0, nsl);
    __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
    for (int q = 0; q < Q; ++q) {
      wg_barrier();
      const int jq = q / S, sq = q - jq * S;
      // the unit's last scale read is at its stage S - 8; the next unit's
      // scales go out in three parts at stages S - 7 .. S - 5
      const int part = sq - (S - 7);
      if (jq + 1 < nu && part >= 0 && part < 3)
        issue_scales(jq + 1, nsl * part / 3, nsl * (part + 1) / 3);
      if (sq == S - 1) __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
    }
    return;
  }

  if (wave == kMW + kCW) {
    // ---------------- activation loader ----------------
    // gate/up: lane jj keeps the token of row jj of the current tile, fetched
    // when the unit's tile changes (three stages before its first chunk)
    int tok = 0, tok_row0 = -1;
    auto issue_acts = [&](int j, int kc) {
      const int4v ui = lds_read_i32x4(lds + kLdsUnits + 16 * j);
      if constexpr (GU) {
        if (ui.z != tok_row0) {
          tok_row0 = ui.z;
          tok = sorted_pairs[ui.z + min(lane, ui.w - 1)] / k;
        }
      }
      for (int jj = 0; jj < ui.w; ++jj) {
        int64_t row;
        if constexpr (GU) row = __builtin_amdgcn_readlane(tok, jj);
        else row = int64_t(ui.z) + jj;
        const int c = lane ^ (jj & 7);             // piece stored at slot `lane`
        const uint8_t* src = reinterpret_cast<const uint8_t*>(act) +
                             (row * K + int64_t(kc) * kChunkK) * 2 + c * 16;
        __builtin_amdgcn_global_load_lds(src, lds_at(lds, kLdsActs + 1024 * jj), 16, 0, 0);
      }
    };
    issue_acts(0, 0);
    __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
    for (int q = 0; q < Q; ++q) {
      wg_barrier();
      // a chunk's rows are read at its first stage; the next chunk goes out
      // three stages before its first stage, after that read
      const int p = q + 3;
      if (p < Q && (p & 3) == 0) {
        const int jn = p / S, sn = p - jn * S;
        issue_acts(jn, sn >> 2);
      }
      if (((q + 1) & 3) == 0) __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
    }
    return;
  }

  if (wave >= kMW) {
    // ---------------- code loaders ----------------
    const int ld = wave - kMW;
    // The loads of a stage go out right after its barrier and their issue
    // is on the critical path of the stream: each lane's offsets within a
    // row group are fixed, so only a scalar base changes per stage (the
    // weight rows of a row group are consecutive: I % 128 == 0 and
    // H % 256 == 0 keep weight_row from clamping).  Measured: 150.0 ->
    // 147.7 us for 4 gate/up units per workgroup.
    int cur = -1, j = 0, s = 0;
    // per lane, the byte offset of load m within a row group's first chunk
    uint32_t loff[kPerLoader];
    code_load_offsets(ld, K, loff);
    const uint8_t* ubase[4];                       // first byte of each row group of the unit
    auto issue = [&](int p) {                      // p = j S + s
      if (j != cur) {
        cur = j;
        const int4v ui = lds_read_i32x4(lds + kLdsUnits + 16 * j);
        const int ex = __builtin_amdgcn_readfirstlane(ui.x), nt = __builtin_amdgcn_readfirstlane(ui.y);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          ubase[rg] = codes + weight_row<GU>(ex, nt, kGroupRows * rg, I, H) * (K / 2);
      }
      const int kc = s >> 2, rg = s & 3;
      const uint8_t* b = (rg == 0 ? ubase[0] : rg == 1 ? ubase[1] : rg == 2 ? ubase[2] : ubase[3]) +
                         kc * (kChunkK / 2);
      code_load_stage(b, lds + (p % kRing) * kStageB, ld, loff);
      if (++s == S) {
        s = 0;
        ++j;
      }
    };
    for (int p = 0; p < pre; ++p) issue(p);
    vmcnt_wait_stages<kPerLoader, kRing - 2>(pre - 1);   // stage 0 landed
    for (int q = 0; q < Q; ++q) {
      wg_barrier();
      if (q + kRing - 1 < Q) issue(q + kRing - 1);
      if (q + 1 < Q) vmcnt_wait_stages<kPerLoader, kRing - 2>(min(q + kRing - 1, Q - 1) - (q + 1));
    }
    return;
  }

  // ---------------- MFMA waves ----------------
  const int w = wave;
  const uint8_t* scb = lds + kLdsScales;
  const uint8_t* actb = lds + kLdsActs;
  f32x4 acc[4];
  uint32_t sc4[2][4];
  uint4 xb[4][4];
  int4v ui{0, 0, 0, 1};
  int j = 0, s = 0;
  // S is a multiple of 8: two K chunks of four row groups per iteration
  for (int q0 = 0; q0 < Q; q0 += 8) {
#pragma unroll
    for (int st8 = 0; st8 < 8; ++st8) {
      const int q = q0 + st8;
      const int par = st8 >> 2, rg = st8 & 3;
      if (st8 == 0 && s == 0) {
        ui = units[j];
#pragma unroll
        for (int a = 0; a < 4; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      wg_barrier();
      if (st8 == 0) read_scales(scb, nblk, w, s >> 2, sc4);   // this chunk and the next
      if (rg == 0) read_acts(actb, ui.w, xb);
      mfma_stage(lds + (q % kRing) * kStageB, w, sc4[par][rg], xb, acc[rg]);
      ++s;
      if (st8 == 7 && s == S) {
        // lane holds D[4g+v][r16]: weight row 4g+v of the subtile, token row r16
        const int nt = ui.y, row0 = ui.z, rows = ui.w;
        if (r16 < rows) {
          if constexpr (GU) {
            uint16_t* h = reinterpret_cast<uint16_t*>(out);
#pragma unroll
            for (int a = 0; a < 2; ++a) {
              const int col = nt * 128 + kGroupRows * a + 16 * w + 4 * g;
              if (col < I) {
                const f32x4 gv = acc[a], uv = acc[a + 2];
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
            for (int a = 0; a < 4; ++a) {
              const int n = nt * kUnitRows + kGroupRows * a + 16 * w + 4 * g;
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
}

// Upper bound of the units a workgroup can get (the host does not know the
// counts; tiles <= min(E, R) + R / 16).
int64_t max_units_per_wg(int R, int E, int ntile_n) {
  const int64_t tiles = int64_t(R < E ? R : E) + R / kTokRows;
  const int64_t U = tiles * ntile_n;
  const int G = device_cus();
  return (U + G - 1) / G + 1;
}

template <bool GU>
hipError_t launch_decode(const uint16_t* act, const int32_t* sp, const int32_t* off, int H, int I,
                         int E, int k, const uint8_t* c, const uint8_t* sc, void* out, int hi,
                         hipStream_t s) {
  static std::atomic<bool> lds_set[kMaxDevices];
  const hipError_t e =
      lds_limit_once(reinterpret_cast<const void*>(&k_decode<GU>), kLdsDec, lds_set);
  if (e != hipSuccess) return e;
  const int K = GU ? H : I;
  const int ntile_n = GU ? I / 128 : H / kUnitRows;
  k_decode<GU><<<dim3(unsigned(device_cus())), kThreadsDec, kLdsDec, s>>>(
      act, sp, off, K, I, H, E, k, c, sc, out, ntile_n, hi);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int T, int H, int I, int E, int k) {
  if (H % 2048 || I % 2048 || H > kMaxK || I > kMaxK || E > kMaxE) return false;
  const int R = T * k;
  return max_units_per_wg(R, E, I / 128) <= kMaxUnits &&
         max_units_per_wg(R, E, H / kUnitRows) <= kMaxUnits;
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

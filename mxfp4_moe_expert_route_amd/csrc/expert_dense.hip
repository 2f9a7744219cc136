// Grouped MXFP4 expert contractions for experts with many rows (prefill-like
// batches): a persistent bf16 MFMA GEMM with the FP4 weights dequantised from
// LDS, fused with SwiGLU (gate/up) or writing fp32 (down).
//
// The pages put the experts in MXFP4 (block 32) with bf16 activations
// ("MiMo-V2.5-Pro-FP4-DFlash" model card, §2 "FP4 Quantization"); when many
// tokens reach each expert the contraction is compute-bound and runs on the
// bf16 matrix cores with fp32 accumulation.
//
// Work items: (expert, n-tile of 256 weight rows, m-tile of 192 token rows).
// Items are ordered expert by expert, n-tile by n-tile, m-tile fastest, and
// the list is cut into eight equal contiguous ranges, one per XCD (workgroup
// b runs on XCD b % 8).  The workgroups of an XCD (one per CU) take its items
// in rounds, one item each, in ascending order in even rounds and descending
// in odd ones (an expert's small last m-tile sits beside a full one, so a
// fixed order would hand the cheap items to the same workgroups round after
// round).  At any time they work on neighbouring items: the n-tiles of one
// m-tile read the same activation rows from that XCD's L2.  An m-tile
// covers every row of a typical expert, so each weight byte leaves HBM once.
//
// The loads are sized by cache lines, the currency of the CU's load path:
// weight codes arrive 128 bytes (a whole line, four stages' worth) per row in
// a super-stage, activations 64 bytes of each token row per load, and the
// scale bytes of a row 16 at a time (8 stages' worth) in a separate chunk
// buffer.  Weights are read once, so their loads carry the non-temporal hint
// and leave the L2 to the activations, which every n-tile re-reads.
//
// Workgroup: 8 waves in a 4 x 2 grid, two per SIMD; wave (wn, wm) computes
// 64 weight rows (4 subtiles of 16) x 96 token rows (the 16-row subtiles wm,
// wm+2, ..., wm+10 of the tile), 96 fp32 accumulators per lane.  Each weight
// row is dequantised by the two waves that share it, and each dequantised
// operand feeds six MFMAs: the FP4 conversion runs at half the VALU rate, so
// conversions per MFMA, not LDS bytes, set this split.  For gate/up the
// workgroup's 256 weight rows are 128 gate columns and the same 128 up
// columns; wave wn holds 32 of each, so SwiGLU pairs inside the wave.
//
// A stage is 64 of K (two MX blocks).  Activations go through a ring of
// three stages: every wave issues its three 1 KB blocks of stage s + 3 while
// it runs stage s's MFMAs, and reads stage s + 1's operands into registers
// in the same iteration, so LDS latency hides behind MFMAs.  Weight codes go
// through two super-stage slots of 32 KB: the four 1 KB loads per wave of
// super-stage S + 2 are issued right after the barriers of iterations
// 4S + 3 and 4S + 4, when every wave has read the last of super-stage S.
// Waves 0-3 load 1 KB of scale bytes every 8 stages.  One barrier per stage.
//
// Register roles follow v_mfma_f32_16x16x32_bf16: weights are operand A
// (row = weight row), activations operand B (row = token row).  In a stage,
// lane group g covers K elements 16g..16g+15 (half of MX block g/2), MFMA kk
// the 8 from 16g+8kk; weights and activations use the same assignment.
//
// LDS layouts are chosen for the MFMA waves' reads.  Activations are stored
// in 1 KB blocks, one per (16-row subtile, MFMA kk): lane l = 16g + r of the
// read finds its 16 bytes (row r, K chunk 2g + kk) at 16 l, so every operand
// read is one contiguous 1 KB; the load that fills a block fetches those 64
// pieces (half of each of 16 rows' 128 bytes).  Row-strided layouts, even
// xor-swizzled ones, read at about half that rate on gfx950.  A weight
// super-stage keeps each row's 128 bytes together, 16-byte block b in slot
// b ^ ((row >> 1) & 7), which makes the 8-byte code reads conflict-free.
//
// The epilogue goes through LDS too: a wave's 16-row output subtile is
// written to a free activation slot and read back row-major, so each store
// writes whole pieces of output rows rather than 16 rows x 64 bytes.
#include <type_traits>

#include "common.hpp"

namespace mxm {
namespace {

constexpr int kMT = 192;             // token rows per tile
constexpr int kNT = 256;             // weight rows per tile
constexpr int kKS = 64;              // K per stage (2 MX blocks)
constexpr int kRingA = 3;            // activation stages in the LDS ring
constexpr int kSS = 4;               // stages per weight super-stage (128 code bytes per row)
constexpr int kRingW = 2;            // weight super-stage slots
constexpr int kWaves = 8;            // two per SIMD
constexpr int kDThreads = kWaves * kWave;
// Experts with fewer rows use the streaming kernels.  Those take 16 token
// rows per pass over an expert's weights, the dense kernel all rows in one
// pass at about half the streaming rate, so the dense kernel wins from three
// passes (33 rows) on.  Measured on the 512-token Zipf batch: thresholds 17,
// 25, 33, 41, 49, 64 give 1.304, 1.248, 1.212, 1.230, 1.271, 1.338 ms.
constexpr int kMinRows = 33;
constexpr int kMaxE = 1024;
constexpr int kAB = kMT * kKS * 2;   // 24 KB of activations per stage
constexpr int kWSlot = kNT * kKS * kSS / 2;   // 32 KB of codes per super-stage
constexpr int kScStages = 8;         // stages per scale chunk (16 blocks = 16 B per row)
constexpr int kSChunk = kNT * 16;    // 4 KB
constexpr int kLdsA = 0;
constexpr int kLdsW = kLdsA + kRingA * kAB;
constexpr int kLdsS = kLdsW + kRingW * kWSlot;
constexpr int kLdsMpre = kLdsS + 2 * kSChunk;
constexpr int kLdsBytes = kLdsMpre + (kMaxE + 4) * 4;
constexpr int kActLoads = kAB / 1024 / kWaves;    // per wave per stage
constexpr int kWLoads = kWSlot / 1024 / kWaves;   // per wave per super-stage
constexpr int kWN = 4;                            // waves along weight rows
constexpr int kWM = kWaves / kWN;                 // waves along token rows
constexpr int kASub = kNT / kWN / 16;             // weight subtiles per wave (4)
constexpr int kMSub = kMT / 16 / kWM;             // token subtiles per wave
constexpr int kNT_AUX = 2;                        // buffer-load cache policy: non-temporal
static_assert(kLdsBytes <= 160 * 1024, "LDS per CU");
static_assert(kAB == kActLoads * kWaves * 1024 && kWSlot == kWLoads * kWaves * 1024 &&
              kSChunk == 4 * 1024 && kWLoads % 2 == 0 && kWaves >= 4,
              "every wave issues the same loads; waves 0-3 one scale load each");
static_assert(kActLoads + kWLoads / 2 + 1 <= 15, "loads per iteration within vmcnt_le");
static_assert(kScStages % kSS == 0 && kRingA == 3 && kRingW == 2, "the pipeline below");

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 layout:
// vmcnt low bits 3:0, high bits 15:14; expcnt 6:4 and lgkmcnt 11:8 at max).
#define MXM_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

__device__ __forceinline__ lds_void* lds_at(uint8_t* base, int off) {
  return (lds_void*)(base + off);   // generic -> LDS address space
}

// at most n (0..15) loads of this wave outstanding
__device__ __forceinline__ void vmcnt_le(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(9)); break;
    case 10: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(10)); break;
    case 11: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(11)); break;
    case 12: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(12)); break;
    case 13: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(13)); break;
    case 14: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(14)); break;
    default: __builtin_amdgcn_s_waitcnt(MXM_VMCNT(15)); break;
  }
}

// Expert of m-tile tau: the last e with mpre[e] <= tau.
__device__ __forceinline__ int expert_of(const int* mpre, int E, int tau) {
  int lo = 0, hi = E;               // mpre[lo] <= tau < mpre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mpre[mid] <= tau) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Local weight row (0..255 within the n-tile) of subtile a of wave wn: gate
// subtiles first, then the up subtiles of the same columns.
template <bool GU>
__device__ __forceinline__ int local_row(int wn, int a) {
  constexpr int h = kASub / 2;
  if constexpr (GU) return a < h ? 16 * h * wn + 16 * a : 128 + 16 * h * wn + 16 * (a - h);
  else return 16 * kASub * wn + 16 * a;
}

// Row in the whole weight tensor of local row r of n-tile n of expert e:
// gate/up n-tiles are 128 gate columns then the same 128 up columns.
template <bool GU>
__device__ __forceinline__ int64_t weight_row(int e, int n, int r, int I, int H) {
  if constexpr (GU) return int64_t(e) * 2 * I + (r < 128 ? 0 : I) + 128 * n + (r & 127);
  else return int64_t(e) * H + kNT * n + r;
}

// Scheduling pattern for one stage: N times (one VMEM read, then M MFMAs),
// the last group LAST MFMAs (0x020: VMEM reads, 0x008: MFMAs).
template <int N, int M, int LAST>
__device__ __forceinline__ void sched_loads_between_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  if constexpr (N == 1) {
    __builtin_amdgcn_sched_group_barrier(0x008, LAST, 0);
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    sched_loads_between_mfma<N - 1, M, LAST>();
  }
}

struct Item {
  int e, n, row0, rows;
};

// One work item: K loop over the ring, then the epilogue.  NV = this wave's
// valid token subtiles (wm, wm+2, ... below the tile's row count).
template <bool GU, int NV>
__device__ __forceinline__ void run_item(uint8_t* lds, const Item& it, int K, int I, int H, int k,
                                         const __amdgpu_buffer_rsrc_t& rs,
                                         const int32_t* __restrict__ sorted_pairs,
                                         const uint8_t* __restrict__ codes,
                                         const uint8_t* __restrict__ scales, void* __restrict__ out) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int wn = wave % kWN, wm = wave / kWN;
  const int nst = K / kKS;
  const int nss = nst / kSS;
  const int nblk = K / 32;
  const int rowb = K / 2;                 // code bytes per weight row

  // ---- this lane's load sources
  // activations: load j = wave + 8q fills the block of subtile j/2, MFMA
  // kk = j%2: lane 16g + r fetches tile row 16(j/2) + r, K chunk 2g + kk.
  // Rows past the tile's end get 2^31 added: out of the buffer's range, no
  // memory traffic.
  uint32_t voff[kActLoads];
#pragma unroll
  for (int q = 0; q < kActLoads; ++q) {
    const int j = wave + kWaves * q;
    const int tr = 16 * (j >> 1) + r16;
    const int row = it.row0 + min(tr, it.rows - 1);
    const uint32_t src = GU ? uint32_t(sorted_pairs[row] / k) : uint32_t(row);
    voff[q] = src * uint32_t(K * 2) + uint32_t((2 * g + (j & 1)) * 16) +
              (uint32_t(tr >= it.rows) << 31);
  }
  // codes: a buffer over this item's weight rows (gate/up: 128 gate rows,
  // then from row I on the 128 up rows).  Load q of a super-stage covers
  // local rows 8 (wave + W q) .. + 7 (W waves); lane -> row 8 W q + rl, slot
  // lane%8 holding 16-byte block (lane%8) ^ ((rl >> 1) & 7) of the row's 128
  // super-stage bytes.
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(codes + weight_row<GU>(it.e, it.n, 0, I, H) * rowb), 0,
      (GU ? I + 128 : kNT) * rowb, 0x00020000);
  const int rl = 8 * wave + (lane >> 3);
  const uint32_t wvoff = uint32_t(rl * rowb + 16 * ((lane & 7) ^ ((rl >> 1) & 7)));
  auto issue_w = [&](int W, int q) {      // load q of super-stage W
    const int lr0 = 8 * kWaves * q;        // first local row of the load (a multiple of 32)
    const int r0 = GU && lr0 >= 128 ? I + lr0 - 128 : lr0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rw, lds_at(lds, kLdsW + (W & 1) * kWSlot + 1024 * (wave + kWaves * q)), 16, wvoff,
        r0 * rowb + 128 * W, 0, kNT_AUX);
  };
  // scales (waves 0-3): local rows 64 wave + lane, 16 bytes (8 stages) each
  const bool scl_wave = wave < 4;
  const uint8_t* ssrc =
      scales + weight_row<GU>(it.e, it.n, 64 * (wave & 3) + lane, I, H) * nblk;
  auto issue_scales = [&](int c) {            // chunk c: stages 8c..8c+7
    if (scl_wave)
      __builtin_amdgcn_global_load_lds(ssrc + 16 * c,
                                       lds_at(lds, kLdsS + (c & 1) * kSChunk + 1024 * wave), 16,
                                       0, 0);
  };
  auto issue_a = [&](int s, int q) {      // activation load q of stage s
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, lds_at(lds, kLdsA + (s % kRingA) * kAB + 1024 * (wave + kWaves * q)), 16,
        voff[q] + uint32_t(s * kKS * 2), 0, 0, 0);
  };

  f32x4 acc[kASub][NV > 0 ? NV : 1];
#pragma unroll
  for (int a = 0; a < kASub; ++a)
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[a][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // every subtile row's place: a base plus a constant per subtile (subtile
  // rows are multiples of 16, so the swizzle bits come from r16)
  const int sw = (r16 >> 1) & 7;
  const int sbase = 16 * r16 + (g >> 1);
  int abase[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) abase[kk] = 1024 * (2 * wm + kk) + 16 * lane;

  // Activation operands of one stage, read from LDS one stage ahead of their
  // MFMAs; codes and scale bytes are read at the top of the iteration that
  // uses them, before its barrier.
  typedef uint4 Acts[2][NV > 0 ? NV : 1];
  auto read_acts = [&](int s, int kk, Acts& b) {
    if constexpr (NV > 0) {
      const uint8_t* st = lds + kLdsA + (s % kRingA) * kAB;
#pragma unroll
      for (int i = 0; i < NV; ++i)
        b[kk][i] = *reinterpret_cast<const uint4*>(st + abase[kk] + 2048 * kWM * i);
    }
  };
  // hook(j) runs before the j-th group of MFMAs (one dequantised operand
  // each), done(kk) after the MFMAs of half kk, whose activation registers
  // are then free for the next stage's.  A wave without token rows (NV = 0)
  // still runs the hooks: its share of the stage loads is issued there.
  auto compute = [&](const uint2 (&cw)[kASub], const uint32_t (&sb)[kASub], const Acts& b,
                     auto&& hook, auto&& done) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int a = 0; a < kASub; ++a) {
        hook(kk * kASub + a);
        if constexpr (NV > 0) {
          const bf16x8 wa = dequant8(kk ? cw[a].y : cw[a].x, e8m0_to_f32(sb[a]));
#pragma unroll
          for (int i = 0; i < NV; ++i)
            acc[a][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, as_bf16x8(b[kk][i]),
                                                                acc[a][i], 0, 0, 0);
        }
      }
      done(kk);
    }
  };

  // Pipeline.  Iteration s: read stage s's codes and scale bytes; wait until
  // stage s + 1 has landed; barrier; issue the scale chunk and weight loads
  // due in this iteration; run stage s's MFMAs, issuing stage s + 3's
  // activations into the slot of stage s (read in iteration s - 1) between
  // them (a burst of loads from all waves right after the barrier would fill
  // the address queue and stall the waves' MFMA issue), and reading each half
  // of stage s + 1's activations once the same half of stage s is consumed.
  // Weight super-stage W goes into slot W % 2 in iterations 4W - 5 (loads 0,
  // 1) and 4W - 4 (loads 2, 3): the slot's previous super-stage W - 2 was
  // last read at the top of iteration 4W - 5, before its barrier.  Scale
  // chunk c goes out in iteration 8c - 8 (its buffer held chunk c - 2, last
  // read at the top of iteration 8c - 9).  Everything a wave needs at
  // barrier s + 1 (stage s + 1 and its codes and scales) was issued by
  // iteration s - 1, so the wait at iteration s allows the loads of
  // iteration s - 1 to be in flight.  nst is a multiple of 8, nss of 2.
  auto chunk_at = [&](int i) { return scl_wave && i % kScStages == 0 && i + kScStages < nst; };
  auto w_at = [&](int i) {                // super-stage whose loads go out in iteration i
    const int t = i % kSS;
    const int W = t == kSS - 1 ? i / kSS + 2 : (t == 0 && i >= kSS) ? i / kSS + 1 : nss;
    return W < nss ? W : -1;
  };
  auto loads_in = [&](int i) {            // loads this wave issues in iteration i
    return (i + kRingA < nst ? kActLoads : 0) + (w_at(i) >= 0 ? kWLoads / 2 : 0) +
           (chunk_at(i) ? 1 : 0);
  };
  // prologue: chunk 0, super-stage 0, stage 0, super-stage 1, stages 1, 2
  issue_scales(0);
#pragma unroll
  for (int q = 0; q < kWLoads; ++q) issue_w(0, q);
#pragma unroll
  for (int q = 0; q < kActLoads; ++q) issue_a(0, q);
#pragma unroll
  for (int q = 0; q < kWLoads; ++q) issue_w(1, q);
#pragma unroll
  for (int p = 1; p < kRingA; ++p)
#pragma unroll
    for (int q = 0; q < kActLoads; ++q) issue_a(p, q);
  __builtin_amdgcn_s_waitcnt(MXM_VMCNT(kWLoads + 2 * kActLoads));   // chunk 0, W 0, stage 0
  wg_barrier();
  Acts ba, bb;
  read_acts(0, 0, ba);
  read_acts(0, 1, ba);
  // one iteration; PREFETCH (a stage s + 1 exists) is false only for the
  // last stage and ISSUE (a stage s + 3 exists) for the last three, so the
  // loop body is straight-line code and the compiler's counter waits stay
  // exact
  auto step = [&](auto prefetch, auto issue_next, int s, Acts& cur, Acts& nxt) {
    constexpr bool PREFETCH = decltype(prefetch)::value;
    constexpr bool ISSUE = decltype(issue_next)::value;
    uint2 cw[kASub];
    uint32_t sb[kASub];
    if constexpr (NV > 0) {
      const uint8_t* ws = lds + kLdsW + ((s / kSS) & 1) * kWSlot + 128 * r16 +
                          16 * ((2 * (s % kSS) + (g >> 1)) ^ sw) + 8 * (g & 1);
      const uint8_t* sc = lds + kLdsS + ((s / kScStages) & 1) * kSChunk + 2 * (s % kScStages);
#pragma unroll
      for (int a = 0; a < kASub; ++a) {
        const int lr = local_row<GU>(wn, a);
        cw[a] = *reinterpret_cast<const uint2*>(ws + 128 * lr);
        sb[a] = sc[sbase + 16 * lr];
      }
    }
    if constexpr (PREFETCH) {
      vmcnt_le(s == 0 ? kActLoads : loads_in(s - 1));
      wg_barrier();
      if (chunk_at(s)) issue_scales(s / kScStages + 1);
      const int W = w_at(s);
      if (W >= 0) {
        const int q0 = (s % kSS == kSS - 1) ? 0 : kWLoads / 2;
#pragma unroll
        for (int q = 0; q < kWLoads / 2; ++q) issue_w(W, q0 + q);
      }
    }
    constexpr int kEvery = 2 * kASub / kActLoads > 0 ? 2 * kASub / kActLoads : 1;
    static_assert(kEvery * (kActLoads - 1) < 2 * kASub, "loads inside the stage");
    compute(cw, sb, cur, [&](int j) {
      if constexpr (ISSUE) {
        if (j % kEvery == 0 && j / kEvery < kActLoads) issue_a(s + kRingA, j / kEvery);
      }
    }, [&](int kk) {
      if constexpr (PREFETCH) read_acts(s + 1, kk, nxt);
    });
    if constexpr (ISSUE && NV > 0) {
      // ask the scheduler for: load, kEvery NV MFMAs, load, ..., load, the
      // rest of the MFMAs
      sched_loads_between_mfma<kActLoads, kEvery * NV, (2 * kASub - kEvery * (kActLoads - 1)) * NV>();
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  // nst is a multiple of 8: stages 0 .. nst - 5 in pairs, then nst - 4 (the
  // last to issue), nst - 3, nst - 2 and nst - 1
  int s = 0;
  for (; s + 4 < nst; s += 2) {
    step(yes(), yes(), s, ba, bb);
    step(yes(), yes(), s + 1, bb, ba);
  }
  step(yes(), yes(), s, ba, bb);
  step(yes(), no(), s + 1, bb, ba);
  step(yes(), no(), s + 2, ba, bb);
  step(no(), no(), s + 3, bb, ba);

  // Epilogue.  Lane 16g + r holds D[4g+v][r]: weight row 4g+v of subtile a,
  // token row r of subtile wm + kWM i, so a direct store writes 16 rows x 64
  // (y) or 32 (h) bytes per instruction; the output rows go out faster as
  // whole pieces of a row (y: 256 bytes of four rows per instruction, h: 64
  // bytes of sixteen rows), so each subtile is transposed through LDS first.
  // The activation slots of stages nst - 2 and nst - 3 are free here: their
  // last reads came before barrier nst - 2, which every wave has passed, and
  // no load targets them any more.  Wave w uses its own part of them (y:
  // waves 0-4 in one slot, 5-7 in the other, 16 rows of 272 bytes each; h:
  // 16 rows of 80 bytes); a wave reads back only what it wrote, so no
  // barrier is needed, and the next item's prologue comes after the
  // workgroup barrier that ends this item.
  {
    const int sa = (nst - 2) % kRingA, sb2 = (nst - 3) % kRingA;
    constexpr int kRowY = 272, kRowH = 80;
    static_assert(5 * 16 * kRowY <= kAB && 3 * 16 * kRowY <= kAB && kWaves * 16 * kRowH <= kAB,
                  "epilogue transposes fit two activation slots");
    uint8_t* tb = GU ? lds + kLdsA + sa * kAB + wave * 16 * kRowH
                     : lds + kLdsA + (wave < 5 ? sa : sb2) * kAB + (wave < 5 ? wave : wave - 5) * 16 * kRowY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int mb = 16 * (wm + kWM * i);            // the subtile's first tile row
      if constexpr (GU) {
#pragma unroll
        for (int a = 0; a < kASub / 2; ++a) {
          const f32x4 gv = acc[a][i];
          const f32x4 uv = acc[a + kASub / 2][i];
          uint32_t hv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v)
            hv[v] = f32_to_bf16_rne(gv[v] / (1.0f + __expf(-gv[v])) * uv[v]);
          *reinterpret_cast<uint2*>(tb + r16 * kRowH + (16 * a + 4 * g) * 2) =
              make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
        }
        // lane L: row L/4, h columns 8 (L%4) .. + 7 of the wave's 32
        const uint4 hw = *reinterpret_cast<const uint4*>(tb + (lane >> 2) * kRowH + 16 * (lane & 3));
        const int m = mb + (lane >> 2);
        if (m < it.rows) {
          uint16_t* h = static_cast<uint16_t*>(out);
          const int col = 128 * it.n + 8 * kASub * wn + 8 * (lane & 3);
          *reinterpret_cast<uint4*>(h + size_t(it.row0 + m) * I + col) = hw;
        }
      } else {
#pragma unroll
        for (int a = 0; a < kASub; ++a) {
          const f32x4 v = acc[a][i];
          *reinterpret_cast<float4*>(tb + r16 * kRowY + (16 * a + 4 * g) * 4) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
        // store j, lane L: row 4j + L/16, columns 4 (L%16) .. + 3 of the wave's 64
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 yv =
              *reinterpret_cast<const float4*>(tb + (4 * j + (lane >> 4)) * kRowY + 16 * (lane & 15));
          const int m = mb + 4 * j + (lane >> 4);
          if (m < it.rows) {
            float* y = static_cast<float*>(out);
            const int col = kNT * it.n + 16 * kASub * wn + 4 * (lane & 15);
            *reinterpret_cast<float4*>(y + size_t(it.row0 + m) * H + col) = yv;
          }
        }
      }
    }
  }
}

// run_item with this wave's token subtile count as a constant
template <bool GU, int N>
__device__ __forceinline__ void run_nv(int nv, uint8_t* lds, const Item& it, int K, int I, int H,
                                       int k, const __amdgpu_buffer_rsrc_t& rs,
                                       const int32_t* __restrict__ sorted_pairs,
                                       const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ scales, void* __restrict__ out) {
  if constexpr (N == 0) {
    run_item<GU, 0>(lds, it, K, I, H, k, rs, sorted_pairs, codes, scales, out);
  } else {
    if (nv == N) run_item<GU, N>(lds, it, K, I, H, k, rs, sorted_pairs, codes, scales, out);
    else run_nv<GU, N - 1>(nv, lds, it, K, I, H, k, rs, sorted_pairs, codes, scales, out);
  }
}

template <bool GU>
__global__ __launch_bounds__(kDThreads, 1) void k_dense(
    const uint16_t* __restrict__ act, uint32_t act_bytes, const int32_t* __restrict__ sorted_pairs,
    const int32_t* __restrict__ offsets, int K, int I, int H, int E, int k,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, void* __restrict__ out,
    int min_rows) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int wm = wave / kWN;
  int* mpre = reinterpret_cast<int*>(lds + kLdsMpre);
  const int ntn = GU ? 2 * I / kNT : H / kNT;       // n-tiles per expert

  // m-tiles before each expert (experts with at least min_rows rows)
  if (wave == 0) {
    int base = 0;
    for (int c0 = 0; c0 < E; c0 += kWave) {
      const int e = c0 + lane;
      const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
      const int mt = cnt >= min_rows ? (cnt + kMT - 1) / kMT : 0;
      const int incl = wave_incl_scan(mt);
      if (e < E) mpre[e] = base + incl - mt;
      base += __shfl(incl, kWave - 1);
    }
    if (lane == 0) mpre[E] = base;
  }
  __syncthreads();
  const int nitems = mpre[E] * ntn;
  const int xcd = blockIdx.x & 7;
  const int gx = __builtin_amdgcn_readfirstlane(int(gridDim.x >> 3));   // workgroups per XCD
  const int v0 = int(int64_t(nitems) * xcd / 8);
  const int v1 = int(int64_t(nitems) * (xcd + 1) / 8);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(act), 0, int(act_bytes), 0x00020000);

  // round r of the XCD's items goes to its workgroups in ascending order when
  // r is even and descending when odd, so cheap and dear neighbours (the
  // small last m-tile of an expert beside a full one) even out over rounds
  const int wi = int(blockIdx.x >> 3);
  for (int r = 0;; ++r) {
    const int v = v0 + r * gx + ((r & 1) ? gx - 1 - wi : wi);
    if (v0 + r * gx >= v1) break;
    if (v >= v1) continue;
    const int tau = v / ntn;
    const int e = expert_of(mpre, E, tau);
    const int mt = mpre[e + 1] - mpre[e];
    const int local = v - mpre[e] * ntn;
    const int n = local / mt, m = local - n * mt;
    Item it;
    it.e = __builtin_amdgcn_readfirstlane(e);
    it.n = __builtin_amdgcn_readfirstlane(n);
    const int off0 = offsets[e];
    it.row0 = __builtin_amdgcn_readfirstlane(off0 + m * kMT);
    it.rows = __builtin_amdgcn_readfirstlane(min(kMT, offsets[e + 1] - off0 - m * kMT));
    const int nsub = (it.rows + 15) >> 4;
    const int nv =
        __builtin_amdgcn_readfirstlane(max(0, min(kMSub, (nsub - wm + kWM - 1) / kWM)));
    run_nv<GU, kMSub>(nv, lds, it, K, I, H, k, rs, sorted_pairs, codes, scales, out);
    __syncthreads();                 // the ring is free for the next item
  }
}

template <bool GU>
hipError_t launch_dense(const uint16_t* act, uint32_t act_bytes, const int32_t* sorted_pairs,
                        const int32_t* offsets, int H, int I, int E, int k, const uint8_t* codes,
                        const uint8_t* scales, void* out, hipStream_t s) {
  static std::atomic<bool> lds_set[kMaxDevices];
  const hipError_t e =
      lds_limit_once(reinterpret_cast<const void*>(&k_dense<GU>), kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  const int K = GU ? H : I;
  const int grid = (device_cus() + 7) / 8 * 8;      // one per CU, a multiple of 8
  k_dense<GU><<<dim3(unsigned(grid)), kDThreads, kLdsBytes, s>>>(
      act, act_bytes, sorted_pairs, offsets, K, I, H, E, k, codes, scales, out, kMinRows);
  return hipGetLastError();
}

}  // namespace

// The dense path needs K to be whole scale chunks, the n-tiles whole (128
// gate columns, 256 output rows), E within the LDS table and byte offsets of
// activation rows and of one item's weight rows that fit the 31-bit range
// of buffer addressing.
bool dense_supported(int T, int H, int I, int E, int k) {
  const int64_t R = int64_t(T) * k;
  if (H % 512 || I % 512 || E > kMaxE) return false;
  if (int64_t(T) * H * 2 + H * 2 >= (int64_t(1) << 31)) return false;
  if (R * I * 2 + I * 2 >= (int64_t(1) << 31)) return false;
  if (int64_t(I + 128) * H / 2 >= (int64_t(1) << 31)) return false;   // one item's code rows
  return R >= kMinRows;
}

int dense_min_rows() { return kMinRows; }

hipError_t launch_gate_up_dense(const uint16_t* x, const int32_t* sorted_pairs,
                                const int32_t* offsets, int T, int H, int I, int E, int k,
                                const uint8_t* codes, const uint8_t* scales, uint16_t* h,
                                hipStream_t s) {
  return launch_dense<true>(x, uint32_t(int64_t(T) * H * 2), sorted_pairs, offsets, H, I, E, k,
                            codes, scales, h, s);
}

hipError_t launch_down_dense(const uint16_t* h, const int32_t* offsets, int T, int H, int I,
                             int E, int k, const uint8_t* codes, const uint8_t* scales, float* y,
                             hipStream_t s) {
  return launch_dense<false>(h, uint32_t(int64_t(T) * k * I * 2), nullptr, offsets, H, I, E, k,
                             codes, scales, y, s);
}

}  // namespace mxm

// Persistent fused decode layer: routing, grouping, gate/up + SwiGLU, down and
// combine of a verify-sized batch (T <= 16 tokens) in one resident kernel.
//
// At a DFlash verify step ("MiMo-V2.5-Pro-FP4-DFlash" model card, §3: the
// backbone checks a drafted block of 8 tokens per sequence in one pass) the
// layer is a 1.2 GB stream of FP4 expert weights spread over a few short
// phases.  The pages credit the serving runtime's speed to one persistent
// engine kernel that removes the gaps at operator boundaries ("Xiaomi
// MiMo-V2.5-Pro-UltraSpeed" release notes, "TileRT 執行模型", item 1).  Here
// the whole layer is one launch of one workgroup per CU:
//
//   1. every workgroup routes all T tokens and groups the pairs by expert in
//      its own LDS, with the same device functions as moe_route_permute (so
//      ids and lists are bit-identical); workgroup 0 also writes them out.
//      No workgroup waits for another to learn the routing.
//   2. gate/up units (256 weight rows x the whole K of one expert's tile) are
//      taken from a shared queue in tile order (one atomic per unit, claimed
//      one unit ahead), so the tiles finish roughly in order; each finished
//      unit bumps its tile's counter.  Gate/up units never wait.
//   3. once the gate/up queue is empty, down units are taken from a second
//      queue, also in tile order.  A down unit needs its tile's whole h, so
//      the activation loader waits (bounded) until the tile's counter shows
//      all its gate/up units; the weight stream of the unit does not wait.
//      A workgroup drains its own gate/up units before it takes a down unit,
//      so it never waits on itself, and every unit it waits for was claimed by
//      a running workgroup that does not wait: no wait depends on workgroups
//      being resident together, so a plain launch is enough.
//   4. each finished down unit bumps its column block's counter; the
//      workgroup that brings a column block to the number of tiles combines
//      it (out = the slot-ordered weighted sum of the k expert rows), with no
//      wait.  The last workgroup to finish resets the counters for the next
//      call.
//
// Cross-workgroup data (h, y) is stored and loaded with the device-scope
// coherence bit (sc1: stores write through this XCD's L2, loads do not hit
// lines another XCD left stale), and the counters are device-scope atomics;
// no L2 write-back or invalidate is needed.  Every unit is computed with the
// same stage functions as the separate decode kernels, so h, y and out equal
// moe_mxfp4_layer's bit for bit.
#include "decode_stream.hpp"
#include "routing.hpp"

namespace mxm {
namespace {

using namespace dec;

constexpr int kDLWaves = kThreadsDec / kWave;     // 8
constexpr int kDLMaxT = 16;
constexpr int kDLMaxR = 512;                      // T * k
constexpr int kDLMaxE = 1024;
constexpr int kDLMaxTiles = kDLMaxR;              // T <= 16: one tile per touched expert
constexpr int kDLMaxNB = kMaxK / kUnitRows;       // down column blocks (H <= 8192)

// workspace words (device memory the caller zero-fills once; every call leaves
// them zero, except the sticky error word)
constexpr int kWsWgDone = 0;                      // workgroups finished
constexpr int kWsDnHead = 1;                      // next down unit of the queue
constexpr int kWsErr = 2;                         // nonzero: a bounded wait gave up
constexpr int kWsGuHead = 3;                      // next gate/up unit of the queue
constexpr int kWsGu = 4;                          // [tile] gate/up units finished
constexpr int kWsDn = kWsGu + kDLMaxTiles;        // [column block] down units finished
constexpr int kWsWords = kWsDn + kDLMaxNB;
constexpr size_t kWsBytes = 4096;
static_assert(kWsWords * 4 <= int(kWsBytes), "workspace words");

// s_waitcnt immediate that waits for lgkmcnt == 0 and nothing else (gfx9
// layout: vmcnt and expcnt at their maxima)
#define MXM_LGKMCNT0 ((15 | (3 << 14)) | (7 << 4))

// a wait for a tile's gate/up units polls at most this many times (each poll
// is a device-scope load, about a microsecond, then a short sleep): about a
// second, far beyond any real wait (at most one phase, ~0.1 ms)
constexpr int kMaxPolls = 1 << 20;

// LDS layout (bytes)
constexpr int kLActs = kRing * kStageB;                        // code ring first (64 KB)
constexpr int kLScales = kLActs + kActBytes;                   // 16 token rows x 1 KB
constexpr int kLTiles = kLScales + kUnitRows * (kMaxK / 32);   // 256 rows of scales
constexpr int kLPairs = kLTiles + kDLMaxTiles * 8;             // per tile {e | rows << 16, row0}
constexpr int kLP2R = kLPairs + kDLMaxR * 4;                   // sorted_pairs [R]
constexpr int kLW = kLP2R + kDLMaxR * 4;                       // pair_to_row [R]
constexpr int kLSlots = kLW + kDLMaxR * 4;                     // routing weights [R]
constexpr int kLMisc = kLSlots + 4 * 16;                       // 4 down-unit descriptors
constexpr int kLComb = kLMisc + 16;                            // ntiles, ncomb, last, -
constexpr int kLBytes = kLComb + kDLMaxNB * 4;                 // column blocks to combine
static_assert(kLBytes <= 160 * 1024, "LDS per CU");
// routing temporaries, in the code ring before the first weight load
constexpr int kLRIds = 0;                                      // ids [R]
constexpr int kLRMask = kLRIds + kDLMaxR * 4;                  // token mask per expert [E]
constexpr int kLRCounts = kLRMask + kDLMaxE * 4;               // counts [E]
constexpr int kLROffsets = kLRCounts + kDLMaxE * 4;            // offsets [E + 1], twice
static_assert(kLROffsets + 2 * (kDLMaxE + 1) * 4 <= kLActs, "routing tables fit the ring");

// A unit: expert e, column block nt (gate/up: 128 intermediate columns with
// their up rows; down: 256 output features), the tile's rows [row0, row0 +
// rows) of the sorted order, and the tile index.  e < 0 ends the sequence.
struct Unit {
  int e, nt, row0, rows, tile;
};

struct Layer {
  const uint16_t* x;
  const uint8_t *w13c, *w13s, *w2c, *w2s;
  uint16_t* h;
  float* y;
  uint32_t* ws;
  int H, I, k, ntiles, ntg, ntd;
};

__device__ __forceinline__ Unit tile_unit(const uint8_t* lds, int tile, int nt) {
  const int2 tv = lds_read_i32x2(lds + kLTiles + 8 * tile);
  return Unit{tv.x & 0xffff, nt, tv.y, tv.x >> 16, tile};
}

__device__ __forceinline__ Unit end_unit() { return Unit{-1, 0, 0, 1, 0}; }

__device__ __forceinline__ uint32_t load_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev64(void* p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_dev64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// The units of one phase: a queue in tile order (unit d: tile d / per,
// column block d % per), claimed one unit ahead.  This workgroup's unit i is
// in descriptor slot i % 4 in LDS (thread 0 writes unit 0's).  The scale
// loader takes unit i's number from the queue at the first stage of unit
// i - 1 and writes its slot at stage S - 9, so the atomic's round trip is
// off the path of the stage barriers (this file is built without the
// compiler's atomic aggregation, which would wait for the answer at once).
struct Units {
  const uint8_t* lds;
  uint32_t* head;              // the queue's next unit (workspace word)
  int total, per;              // units, units per tile (ntg or ntd)

  __device__ __forceinline__ Unit get(int i) const {
    const int4v v = lds_read_i32x4(lds + kLSlots + 16 * (i & 3));
    return Unit{v.x, v.y, v.z, v.w & 0xffff, v.w >> 16};
  }

  // one lane: the queue's next unit number
  __device__ __forceinline__ int take() const { return int(add_dev(head, 1u)); }

  // one lane: unit number d (past the end: the end marker) into slot i % 4
  __device__ __forceinline__ void put(int i, int d) const {
    int4v v{-1, 0, 0, 1};
    if (d < total) {
      const int tile = d / per;
      const Unit u = tile_unit(lds, tile, d - tile * per);
      v = int4v{u.e, u.nt, u.row0, u.rows | (u.tile << 16)};
    }
    *reinterpret_cast<int4v*>(const_cast<uint8_t*>(lds) + kLSlots + 16 * (i & 3)) = v;
  }

  // one lane: take the next unit into slot i % 4 now
  __device__ __forceinline__ void claim(int i) const { put(i, take()); }
};

// Unit completion, sent by thread 0 once every MFMA wave's stores of the unit
// are complete.  Down: returns true when this unit completes its column block.
template <bool GU>
__device__ __forceinline__ bool signal_unit(const Layer& L, const Unit& u) {
  if constexpr (GU) {
    add_dev(L.ws + kWsGu + u.tile, 1u);
    return false;
  } else {
    return add_dev(L.ws + kWsDn + u.nt, 1u) + 1u == uint32_t(L.ntiles);
  }
}

// One phase: the units of `src` streamed through the decode pipeline (code
// loaders, activation loader, scale loader, MFMA waves; one barrier per
// stage).  Returns, in the MFMA waves, the last unit, whose completion is not
// yet signalled.
template <bool GU>
__device__ Unit run_phase(uint8_t* lds, const Layer& L, const Units& src, uint8_t* comb) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = lane_id();
  const int H = L.H, I = L.I;
  const int K = GU ? H : I;
  const int nblk = K / 32;
  const int S = 4 * (K / kChunkK);                 // stages per unit, a multiple of 8
  const uint8_t* codes = GU ? L.w13c : L.w2c;
  const uint8_t* scales = GU ? L.w13s : L.w2s;
  Unit pending = end_unit();

  if (wave == kMW + kCW + 1) {
    // ---------------- scale loader (and the queue) ----------------
    const int half = 128 * nblk;
    const int nsl = kUnitRows * nblk / 1024;
    auto issue_scales = [&](const Unit& u, int m0, int m1) {
      for (int m = m0; m < m1; ++m) {
        const int o = 1024 * m + 16 * lane;
        const uint8_t* src_p;
        if constexpr (GU) {
          const int h2 = o >= half;
          src_p = scales + weight_row<true>(u.e, u.nt, h2 ? 128 : 0, I, H) * nblk + (o - h2 * half);
        } else {
          src_p = scales + weight_row<false>(u.e, u.nt, 0, I, H) * nblk + o;
        }
        __builtin_amdgcn_global_load_lds(src_p, lds_at(lds, kLScales + 1024 * m), 16, 0, 0);
      }
    };
    Unit un = src.get(0);
    if (un.e >= 0) issue_scales(un, 0, nsl);
    __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
    for (int j = 0;; ++j) {
      const Unit u = src.get(j);
      if (u.e < 0) break;
      int nd = 0;                                    // lane 0: unit j + 1's number
      for (int s = 0; s < S; ++s) {
        wg_barrier();
        // unit j + 1: its number at stage 0, its slot at stage S - 9 (the
        // activation loader reads it at S - 7, the code loaders at S - 4)
        if (s == 0 && lane == 0) nd = src.take();
        if (s == S - 9 && lane == 0) {
          src.put(j + 1, nd);
          __builtin_amdgcn_s_waitcnt(MXM_LGKMCNT0);
        }
        // the unit's last scale read is at its stage S - 8; the next unit's
        // scales go out in three parts at stages S - 7 .. S - 5
        if (s == S - 7) un = src.get(j + 1);
        const int part = s - (S - 7);
        if (un.e >= 0 && part >= 0 && part < 3) issue_scales(un, nsl * part / 3, nsl * (part + 1) / 3);
        if (s == S - 1) __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
      }
    }
    return pending;
  }

  if (wave == kMW + kCW) {
    // ---------------- activation loader ----------------
    const uint8_t* act = reinterpret_cast<const uint8_t*>(GU ? L.x : L.h);
    const int nch = K / kChunkK;
    int tok = 0, tok_row0 = -1;
    auto issue_acts = [&](const Unit& u, int kc, uint32_t seen) {
      if constexpr (GU) {
        if (u.row0 != tok_row0) {
          tok_row0 = u.row0;
          tok = lds_read_i32(lds + kLPairs + 4 * (u.row0 + min(lane, u.rows - 1))) / L.k;
        }
      } else {
        // the tile's h rows are written by other workgroups: wait (bounded)
        // until all its gate/up units are in (`seen`: the count read when the
        // unit became known, usually the whole tile already)
        if (kc == 0 && seen < uint32_t(L.ntg)) {
          const uint32_t* cnt = L.ws + kWsGu + u.tile;
          int polls = 0;
          while (load_dev(cnt) < uint32_t(L.ntg)) {
            // give up after kMaxPolls, or at once when another wait already
            // has (the outputs are then invalid, but every wave runs to its end)
            if (++polls > kMaxPolls || load_dev(L.ws + kWsErr) != 0u) {
              if (lane == 0) __hip_atomic_fetch_or(L.ws + kWsErr, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
      }
      for (int jj = 0; jj < u.rows; ++jj) {
        int64_t row;
        if constexpr (GU) row = __builtin_amdgcn_readlane(tok, jj);
        else row = int64_t(u.row0) + jj;
        const int c = lane ^ (jj & 7);             // piece stored at slot `lane`
        const uint8_t* srcp = act + (row * K + int64_t(kc) * kChunkK) * 2 + c * 16;
        __builtin_amdgcn_global_load_lds(srcp, lds_at(lds, kLActs + 1024 * jj), 16, 0,
                                         GU ? 0 : kAuxSC1);
      }
    };
    // next chunk to issue: chunk ca of unit ja.  Down: when unit ja + 1
    // becomes known (as the last chunk of unit ja goes out) its tile's count
    // is loaded, the last load of the wave; the wait at the end of that
    // chunk-group leaves it outstanding, and it is looked at when the unit's
    // first chunk goes out, four stages later.
    int ja = 0, ca = 0;
    Unit ua = src.get(0);
    uint32_t seen = 0;                             // down: ua's tile count, loaded early
    bool seen_pending = false;
    auto issue_next = [&]() {
      if (ua.e < 0) return;
      issue_acts(ua, ca, seen);
      if (++ca == nch) {
        ca = 0;
        ua = src.get(++ja);
        if constexpr (!GU) {
          seen = 0;
          if (ua.e >= 0) {
            seen = load_dev(L.ws + kWsGu + ua.tile);
            seen_pending = true;
          }
        }
      }
    };
    issue_next();
    __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
    int q = 0;
    for (int j = 0;; ++j) {
      const Unit u = src.get(j);
      if (u.e < 0) break;
      for (int s = 0; s < S; ++s, ++q) {
        wg_barrier();
        // a chunk's rows are read at its first stage; the next chunk goes
        // out three stages before its first stage, after that read
        if (((q + 3) & 3) == 0) issue_next();
        if (((q + 1) & 3) == 0) {
          if (seen_pending) {
            __builtin_amdgcn_s_waitcnt(MXM_VMCNT(1));   // all but the count load
            seen_pending = false;
          } else {
            __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
          }
        }
      }
    }
    return pending;
  }

  if (wave >= kMW) {
    // ---------------- code loaders ----------------
    const int ld = wave - kMW;
    uint32_t loff[kPerLoader];
    code_load_offsets(ld, K, loff);
    int ji = 0, si = 0, issued = 0;
    Unit ui = src.get(0);
    const uint8_t* ubase[4];
    auto bases = [&]() {
      const int ex = __builtin_amdgcn_readfirstlane(ui.e), nt = __builtin_amdgcn_readfirstlane(ui.nt);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        ubase[rg] = codes + weight_row<GU>(ex, nt, kGroupRows * rg, I, H) * (K / 2);
    };
    if (ui.e >= 0) bases();
    auto issue = [&]() {
      if (ui.e < 0) return;
      const int kc = si >> 2, rg = si & 3;
      const uint8_t* bp =
          (rg == 0 ? ubase[0] : rg == 1 ? ubase[1] : rg == 2 ? ubase[2] : ubase[3]) +
          kc * (kChunkK / 2);
      code_load_stage(bp, lds + (issued % kRing) * kStageB, ld, loff);
      ++issued;
      if (++si == S) {
        si = 0;
        ui = src.get(++ji);
        if (ui.e >= 0) bases();
      }
    };
    for (int p = 0; p < kRing - 1; ++p) issue();
    vmcnt_wait_stages<kPerLoader, kRing - 2>(max(0, issued - 1));   // stage 0 landed
    int q = 0;
    for (int j = 0;; ++j) {
      const Unit u = src.get(j);
      if (u.e < 0) break;
      for (int s = 0; s < S; ++s, ++q) {
        wg_barrier();
        issue();
        vmcnt_wait_stages<kPerLoader, kRing - 2>(max(0, issued - (q + 2)));
      }
    }
    return pending;
  }

  // ---------------- MFMA waves ----------------
  const int w = wave;
  const int r16 = lane & 15, g = lane >> 4;
  const uint8_t* scb = lds + kLScales;
  const uint8_t* actb = lds + kLActs;
  f32x4 acc[4];
  uint32_t sc4[2][4];
  uint4 xb[4][4];
  int q = 0;
  // down, thread 0: the previous unit's column-block count, sent at stage 4
  // and looked at at stage 7, so the atomic's round trip is off the path of
  // the stage barriers
  uint32_t blk_count = 0;
  int blk_nt = -1;
  for (int j = 0;; ++j) {
    const Unit u = src.get(j);
    if (u.e < 0) break;
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += 8) {
#pragma unroll
      for (int st8 = 0; st8 < 8; ++st8) {
        const int par = st8 >> 2, rg = st8 & 3;
        wg_barrier();
        if (pending.e >= 0 && s0 == 0) {
          // the previous unit's stores: complete by stage 3, signalled after
          // the barrier of stage 4 (every MFMA wave has waited by then).
          // Waiting at stage 1 instead cost 0.3-1 us per call: a store
          // written through to memory can take longer than a stage.
          if (st8 == 3) __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
          if (st8 == 4) {
            if (tid == 0) {
              if constexpr (GU) {
                signal_unit<GU>(L, pending);
              } else {
                blk_count = add_dev(L.ws + kWsDn + pending.nt, 1u);
                blk_nt = pending.nt;
              }
            }
            pending = end_unit();
          }
        }
        if (!GU && s0 == 0 && st8 == 7 && tid == 0 && blk_nt >= 0) {
          // the previous unit completed its column block: combine it at the end
          if (blk_count + 1u == uint32_t(L.ntiles)) {
            int* nc = reinterpret_cast<int*>(lds + kLMisc + 4);
            reinterpret_cast<int*>(comb)[*nc] = blk_nt;
            *nc += 1;
          }
          blk_nt = -1;
        }
        if (st8 == 0) read_scales(scb, nblk, w, (s0 + st8) >> 2, sc4);   // this chunk and the next
        if (rg == 0) read_acts(actb, u.rows, xb);
        mfma_stage(lds + (q % kRing) * kStageB, w, sc4[par][rg], xb, acc[rg]);
        ++q;
      }
    }
    // lane holds D[4g+v][r16]: weight row 4g+v of the subtile, token row r16
    if (r16 < u.rows) {
      if constexpr (GU) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int col = u.nt * 128 + kGroupRows * a + 16 * w + 4 * g;
          if (col < I) {
            const f32x4 gv = acc[a], uv = acc[a + 2];
            const uint32_t h0 = f32_to_bf16_rne(silu_mul(gv[0], uv[0]));
            const uint32_t h1 = f32_to_bf16_rne(silu_mul(gv[1], uv[1]));
            const uint32_t h2 = f32_to_bf16_rne(silu_mul(gv[2], uv[2]));
            const uint32_t h3 = f32_to_bf16_rne(silu_mul(gv[3], uv[3]));
            store_dev64(L.h + size_t(u.row0 + r16) * I + col,
                        uint64_t(h0 | (h1 << 16)) | (uint64_t(h2 | (h3 << 16)) << 32));
          }
        }
      } else {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int n = u.nt * kUnitRows + kGroupRows * a + 16 * w + 4 * g;
          if (n < H) {
            const f32x4 v = acc[a];
            float* yp = L.y + size_t(u.row0 + r16) * H + n;
            store_dev64(yp, uint64_t(__float_as_uint(v[0])) |
                                (uint64_t(__float_as_uint(v[1])) << 32));
            store_dev64(yp + 2, uint64_t(__float_as_uint(v[2])) |
                                    (uint64_t(__float_as_uint(v[3])) << 32));
          }
        }
      }
    }
    pending = u;
  }
  return pending;
}

// Wave w routes tokens w, w + 8 (route_token needs NPER * 64 >= E); the ids
// and weights go to LDS and, when ids_out is set, to the outputs, and each
// chosen expert's token mask gets the token's bit.
template <int NPER>
__device__ __forceinline__ void route_tokens(const float* __restrict__ logits, int T, int E, int k,
                                             int32_t* r_ids, uint32_t* r_mask, float* s_w,
                                             int32_t* ids_out, float* w_out) {
  const int lane = lane_id();
  for (int t = threadIdx.x >> 6; t < T; t += kDLWaves) {
    int my_id;
    float my_w;
    route_token<NPER>(logits + int64_t(t) * E, E, k, my_id, my_w);
    if (lane < k) {
      r_ids[t * k + lane] = my_id;
      s_w[t * k + lane] = my_w;
      atomicOr(&r_mask[my_id], 1u << t);
      if (ids_out) {
        ids_out[t * k + lane] = my_id;
        w_out[t * k + lane] = my_w;
      }
    }
  }
}

// After a phase: every MFMA wave's stores complete, then thread 0 signals the
// phase's last unit.
template <bool GU>
__device__ __forceinline__ void drain_phase(uint8_t* lds, const Layer& L, const Unit& pending,
                                            uint8_t* comb) {
  __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
  __syncthreads();
  if (threadIdx.x == 0 && pending.e >= 0 && signal_unit<GU>(L, pending)) {
    int* nc = reinterpret_cast<int*>(lds + kLMisc + 4);
    reinterpret_cast<int*>(comb)[*nc] = pending.nt;
    *nc += 1;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreadsDec) void k_decode_layer(
    const uint16_t* __restrict__ x, const float* __restrict__ logits, int T, int H, int I, int E,
    int k, const uint8_t* __restrict__ w13c, const uint8_t* __restrict__ w13s,
    const uint8_t* __restrict__ w2c, const uint8_t* __restrict__ w2s, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, int32_t* __restrict__ counts_out, int32_t* __restrict__ offsets_out,
    int32_t* __restrict__ sp_out, int32_t* __restrict__ p2r_out, uint16_t* __restrict__ h,
    float* __restrict__ y, float* __restrict__ out, uint32_t* __restrict__ ws) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int32_t wave_sum[kDLWaves];
  const int tid = threadIdx.x;
  const int R = T * k;
  const int b = blockIdx.x;

  // ---- 1. routing and grouping, in every workgroup ----
  int32_t* r_ids = reinterpret_cast<int32_t*>(lds + kLRIds);
  uint32_t* r_mask = reinterpret_cast<uint32_t*>(lds + kLRMask);
  int32_t* r_counts = reinterpret_cast<int32_t*>(lds + kLRCounts);
  int32_t* r_offsets = reinterpret_cast<int32_t*>(lds + kLROffsets);
  int32_t* s_pairs = reinterpret_cast<int32_t*>(lds + kLPairs);
  int32_t* s_p2r = reinterpret_cast<int32_t*>(lds + kLP2R);
  float* s_w = reinterpret_cast<float*>(lds + kLW);
  int* misc = reinterpret_cast<int*>(lds + kLMisc);
  uint8_t* comb = lds + kLComb;
  for (int e = tid; e < E; e += kThreadsDec) r_mask[e] = 0u;
  if (tid == 0) misc[1] = 0;                       // column blocks to combine
  __syncthreads();
  const int nper = (E + kWave - 1) / kWave;
  if (nper <= 2) route_tokens<2>(logits, T, E, k, r_ids, r_mask, s_w, b == 0 ? ids_out : nullptr, w_out);
  else if (nper <= 4) route_tokens<4>(logits, T, E, k, r_ids, r_mask, s_w, b == 0 ? ids_out : nullptr, w_out);
  else if (nper <= 6) route_tokens<6>(logits, T, E, k, r_ids, r_mask, s_w, b == 0 ? ids_out : nullptr, w_out);
  else if (nper <= 8) route_tokens<8>(logits, T, E, k, r_ids, r_mask, s_w, b == 0 ? ids_out : nullptr, w_out);
  else route_tokens<16>(logits, T, E, k, r_ids, r_mask, s_w, b == 0 ? ids_out : nullptr, w_out);
  __syncthreads();
  // counts, offsets, lists and the tiles (the touched experts in order)
  group_small<kDLWaves>(r_ids, r_mask, R, E, k, r_counts, r_offsets, r_offsets + kDLMaxE + 1,
                        s_pairs, s_p2r, reinterpret_cast<int2*>(lds + kLTiles), &misc[0],
                        wave_sum);
  __syncthreads();
  if (b == 0) {
    for (int e = tid; e < E; e += kThreadsDec) counts_out[e] = r_counts[e];
    for (int e = tid; e <= E; e += kThreadsDec) offsets_out[e] = r_offsets[e];
    for (int p = tid; p < R; p += kThreadsDec) {
      sp_out[p] = s_pairs[p];
      p2r_out[p] = s_p2r[p];
    }
  }
  __syncthreads();

  Layer L;
  L.x = x;
  L.w13c = w13c;
  L.w13s = w13s;
  L.w2c = w2c;
  L.w2s = w2s;
  L.h = h;
  L.y = y;
  L.ws = ws;
  L.H = H;
  L.I = I;
  L.k = k;
  L.ntiles = misc[0];
  L.ntg = I / 128;
  L.ntd = H / kUnitRows;

  // ---- 2. gate/up units from their queue ----
  {
    const Units src{lds, ws + kWsGuHead, L.ntiles * L.ntg, L.ntg};
    if (tid == 0) src.claim(0);
    __syncthreads();
    const Unit pend = run_phase<true>(lds, L, src, comb);
    drain_phase<true>(lds, L, pend, comb);
  }

  // ---- 3. down units from theirs ----
  {
    const Units src{lds, ws + kWsDnHead, L.ntiles * L.ntd, L.ntd};
    if (tid == 0) src.claim(0);
    __syncthreads();
    const Unit pend = run_phase<false>(lds, L, src, comb);
    drain_phase<false>(lds, L, pend, comb);
  }

  // ---- 4. combine the column blocks this workgroup completed ----
  const int ncomb = misc[1];
  for (int c = 0; c < ncomb; ++c) {
    const int nb = reinterpret_cast<const int*>(comb)[c];
    for (int i = tid; i < T * (kUnitRows / 4); i += kThreadsDec) {
      const int t = i / (kUnitRows / 4);
      const int n = nb * kUnitRows + (i - t * (kUnitRows / 4)) * 4;
      if (n >= H) continue;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j0 = 0; j0 < k; j0 += 8) {
        uint64_t v0[8], v1[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int r = (j0 + jj < k) ? max(s_p2r[t * k + j0 + jj], 0) : 0;
          const float* yr = y + int64_t(r) * H + n;
          v0[jj] = load_dev64(yr);
          v1[jj] = load_dev64(yr + 2);
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = j0 + jj;
          if (j < k && s_p2r[t * k + j] >= 0) {
            const float wj = s_w[t * k + j];
            acc.x = fmaf(wj, __uint_as_float(uint32_t(v0[jj])), acc.x);
            acc.y = fmaf(wj, __uint_as_float(uint32_t(v0[jj] >> 32)), acc.y);
            acc.z = fmaf(wj, __uint_as_float(uint32_t(v1[jj])), acc.z);
            acc.w = fmaf(wj, __uint_as_float(uint32_t(v1[jj] >> 32)), acc.w);
          }
        }
      }
      *reinterpret_cast<float4*>(out + int64_t(t) * H + n) = acc;
    }
  }

  // ---- 5. the last workgroup to finish resets the counters ----
  __syncthreads();
  if (tid == 0) misc[2] = add_dev(ws + kWsWgDone, 1u) + 1u == gridDim.x;
  __syncthreads();
  if (misc[2]) {
    for (int i = tid; i < L.ntiles; i += kThreadsDec)
      __hip_atomic_store(ws + kWsGu + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = tid; i < L.ntd; i += kThreadsDec)
      __hip_atomic_store(ws + kWsDn + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
      __hip_atomic_store(ws + kWsDnHead, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ws + kWsGuHead, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ws + kWsWgDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

bool decode_layer_supported(int T, int H, int I, int E, int k) {
  return T >= 1 && T <= kDLMaxT && k >= 1 && k <= 32 && E >= 1 && E <= kDLMaxE &&
         T * k <= kDLMaxR && H % 2048 == 0 && I % 2048 == 0 && H <= kMaxK && I <= kMaxK;
}

size_t decode_layer_workspace_bytes() { return kWsBytes; }

hipError_t launch_decode_layer(const uint16_t* x, const float* logits, int T, int H, int I, int E,
                               int k, const uint8_t* w13c, const uint8_t* w13s,
                               const uint8_t* w2c, const uint8_t* w2s, int32_t* ids, float* w,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                               int32_t* pair_to_row, uint16_t* h, float* y, float* out,
                               void* workspace, hipStream_t s) {
  static std::atomic<bool> lds_set[kMaxDevices];
  const hipError_t e =
      lds_limit_once(reinterpret_cast<const void*>(&k_decode_layer), kLBytes, lds_set);
  if (e != hipSuccess) return e;
  uint32_t* ws = static_cast<uint32_t*>(workspace);
  // one workgroup per CU; no wait in the kernel depends on workgroups being
  // resident together
  k_decode_layer<<<dim3(unsigned(device_cus())), kThreadsDec, kLBytes, s>>>(
      x, logits, T, H, I, E, k, w13c, w13s, w2c, w2s, ids, w, counts, offsets, sorted_pairs,
      pair_to_row, h, y, out, ws);
  return hipGetLastError();
}

}  // namespace mxm

// Device code shared by the routing kernels: the per-token top-k of one
// wave and the workgroup-wide grouping of token-expert pairs by expert.  The
// top-k kernel, the permutation kernel and the fused small-batch kernel all
// run these same functions, so their results are identical bit for bit.
//
// Top-k rule (a reading; the pages give 384 experts with 8 active per token,
// nxbn.cn article, "架构设计与配置详解", and no scoring rule): experts by
// descending logit, lower index first on equal logits, -0.0 == +0.0, NaN as
// -inf; weights = softmax over all experts renormalised over the chosen k,
// which equals exp(l_j - l_1) / sum_j' exp(l_j' - l_1) over the chosen.
//
// Each logit becomes a 64-bit key: an order-preserving 32-bit image of the
// float in the high word and (0xffffffff - index) in the low word, so the
// unsigned maximum is the largest logit with the lowest index.  k rounds of a
// wave-wide max (per-lane max, then DPP row shifts and row broadcasts) pick
// the experts; the picked key is cleared to 0, below every valid key.
//
// Grouping (not on the pages; the bookkeeping a grouped expert computation
// needs): pair p = t*k + j; counts[e] pairs per expert; offsets is the
// exclusive prefix sum; sorted_pairs holds each expert's pairs in ascending
// p; pair_to_row is the inverse.  Ids outside [0, E) are dropped
// (pair_to_row = -1, not counted) so that bad input cannot send a store out
// of bounds.  One workgroup of NW waves; the first nw = min(NW, ceil(R / 256))
// own contiguous ranges of pairs:
//  1. per-wave histograms in LDS (integer atomics: order-free, deterministic)
//  2. per-expert exclusive bases across waves, block scan over experts
//  3. each wave walks its range 64 pairs at a time; a pair's rank among the
//     earlier pairs of its expert in the same 64 comes from a ballot-based
//     match (one ballot per bit of the expert id), so the scatter is stable
//     without sorting.
// Ids are loaded 8 groups of 64 at a time; a range of at most 512 pairs (all
// of them up to 4096 pairs) stays in registers from the histogram to the
// scatter, so a small call pays one memory latency for its ids.
#pragma once
#include "common.hpp"

namespace mxm {
namespace {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;   // NaN ranks as -inf
  if (u == 0x80000000u) u = 0u;                            // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// v moved across lanes by the DPP control CTRL (rows and banks masked by
// RM); lanes whose source is outside the row read 0, below every key
template <int CTRL, int RM>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(v)), CTRL, RM, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(v >> 32)), CTRL, RM, 0xf, true);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

// Largest key of the wave, in every lane.  Row shifts build each 16-lane
// row's maximum in its lane 15, two row broadcasts carry them to lane 63;
// DPP keeps the whole reduction in the VALU (no LDS round trips).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0x111, 0xf>(v));   // row_shr:1
  v = max_u64(v, dpp_u64<0x112, 0xf>(v));   // row_shr:2
  v = max_u64(v, dpp_u64<0x114, 0xf>(v));   // row_shr:4
  v = max_u64(v, dpp_u64<0x118, 0xf>(v));   // row_shr:8
  v = max_u64(v, dpp_u64<0x142, 0xa>(v));   // row_bcast:15 into rows 1 and 3
  v = max_u64(v, dpp_u64<0x143, 0xc>(v));   // row_bcast:31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(v)), kWave - 1);
  const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(v >> 32)), kWave - 1);
  return (uint64_t(hi) << 32) | lo;
}

// Sum over the wave in a fixed order (the same reduction tree as above), in
// every lane.
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto add = [&](float x, int y) { return x + __int_as_float(y); };
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, true));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, true));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Top-k of token t's row of E logits by one whole wave (NPER * 64 >= E);
// lanes 0..k-1 end with the j-th chosen expert and its weight.
template <int NPER>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k,
                                            int& my_id, float& my_w) {
  const int lane = lane_id();
  // every load is unconditional (lanes past E re-read the last logit) and
  // issued before the first key is built, so they are in flight together; a
  // load per branch went out one at a time, each waiting for the one before
  float v[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) v[i] = row[min(lane + kWave * i, E - 1)];
  uint64_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + kWave * i;
    key[i] = (e < E) ? (uint64_t(order_key(v[i])) << 32) | uint64_t(0xffffffffu - uint32_t(e))
                     : 0ull;
  }
  my_id = 0;
  float my_l = 0.f, l1 = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < NPER; ++i) best = max_u64(best, key[i]);
    best = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < NPER; ++i) key[i] = (key[i] == best) ? 0ull : key[i];
    if (j == 0) l1 = key_value(uint32_t(best >> 32));
    if (lane == j) {
      my_id = int(0xffffffffu - uint32_t(best));
      my_l = key_value(uint32_t(best >> 32));
    }
  }
  const float ex = (lane < k) ? expf(my_l - l1) : 0.f;
  const float sum = wave_sum_f32(ex);
  my_w = ex / sum;
}

constexpr int kBatch = 8;                     // 64-pair groups whose ids load together

// Executed by a whole workgroup of exactly NW waves over the pairs [r0, r1);
// smem holds (NW + 1) * E ints and wave_sum NW.  ids may point to global
// memory or LDS.  With gbase == nullptr the workgroup holds every pair
// (r0 = 0, r1 = R) and writes counts and offsets; otherwise it is one of
// several workgroups over consecutive ranges and gbase[e] is the first row of
// expert e for its range (computed from all ranges' histograms beforehand).
template <int NW>
__device__ __forceinline__ void permute_block(const int32_t* ids, int r0, int r1, int E,
                                              const int32_t* gbase,
                                              int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ sorted_pairs,
                                              int32_t* __restrict__ pair_to_row, int32_t* smem,
                                              int32_t* wave_sum) {
  constexpr int NT = NW * kWave;
  int32_t* hist = smem;                       // [nw][E]
  int32_t* tot = smem + NW * E;               // [E]
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int len = r1 - r0;

  const int nw = min(NW, max(1, (len + 255) / 256));   // waves that walk pairs
  for (int i = tid; i < nw * E; i += NT) hist[i] = 0;
  __syncthreads();

  const int per = (len + nw - 1) / nw;
  const int beg = r0 + (wave < nw ? min(len, wave * per) : len);
  const int end = wave < nw ? min(r1, beg + per) : r1;
  const bool kept = end - beg <= kBatch * kWave;     // the range fits one batch
  int32_t* my_hist = hist + wave * E;
  int raw[kBatch];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = c0 + i * kWave + lane;
      raw[i] = (p < end) ? ids[p] : -1;
    }
  };
  for (int c0 = beg; c0 < end; c0 += kBatch * kWave) {
    load_batch(c0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (c0 + i * kWave >= end) break;          // past the range: the rest of the batch is empty
      if (unsigned(raw[i]) < unsigned(E)) atomicAdd(&my_hist[raw[i]], 1);
    }
  }
  __syncthreads();

  // 2a. exclusive base of each wave within each expert; totals
  for (int e = tid; e < E; e += NT) {
    int run = gbase ? gbase[e] : 0;
    for (int w = 0; w < nw; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    tot[e] = run;
    if (!gbase) counts[e] = run;
  }
  __syncthreads();
  if (!gbase) {

  // 2b. exclusive scan of the totals over experts (each thread: ept experts)
  const int ept = (E + NT - 1) / NT;
  const int e0 = tid * ept;
  int local = 0;
  for (int i = 0; i < ept; ++i)
    if (e0 + i < E) local += tot[e0 + i];
  const int incl = wave_incl_scan(local);
  if (lane == kWave - 1) wave_sum[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wave_sum[w];
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    offsets[e] = run;
    for (int w = 0; w < nw; ++w) hist[w * E + e] += run;
    run += tot[e];
  }
  if (tid == 0) {
    int total = 0;
    for (int w = 0; w < NW; ++w) total += wave_sum[w];
    offsets[E] = total;                       // == R when every id is in range
  }
  __syncthreads();
  }

  // 3. stable scatter; my_hist[e] is the next free row of expert e for this wave
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int c0 = beg; c0 < end; c0 += kBatch * kWave) {
    if (!kept) load_batch(c0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (c0 + i * kWave >= end) break;          // wave-uniform: no pair left in this batch
      const int p = c0 + i * kWave + lane;
      const bool valid = (p < end) && unsigned(raw[i]) < unsigned(E);
      const int key = valid ? raw[i] : 0;
      if (p < end && !valid) pair_to_row[p] = -1;   // out-of-range id: pair dropped
      unsigned long long m = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const unsigned long long bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
      }
      if (valid) {
        const int rank = __popcll(m & lt);
        const int pos = my_hist[key] + rank;
        sorted_pairs[pos] = p;
        pair_to_row[p] = pos;
        if ((m >> lane) == 1ull) my_hist[key] += __popcll(m);   // last lane of its expert
      }
    }
  }
}

// Grouping for small batches (T <= 32 tokens), by a whole workgroup of NW
// waves.  A token never picks an expert twice, so expert e's pairs are fixed
// by the set of tokens that chose it: mask[e] has bit t set when token t did
// (the caller clears it, sets the bits from its routing lanes, then
// barriers).  Then, for pair p = t k + j with expert e:
//   counts[e]  = popcount(mask[e])
//   offsets[e] = sum of the counts of experts below e (one block scan)
//   row        = offsets[e] + popcount(mask[e] & (2^t - 1)),
// which is the stable order by p within the expert, so the lists are those
// of permute_block bit for bit.  The same scan numbers the touched experts:
// when `tiles` is set, tile i (the i-th expert with pairs, in expert order)
// gets {e | count << 16, offsets[e]} and *ntiles the number of tiles.  ids
// [R] and mask [E] are in LDS; off_lds is an LDS copy of offsets [E + 1]; the
// other outputs may be global or LDS.
template <int NW>
__device__ __forceinline__ void group_small(const int32_t* ids, const uint32_t* mask, int R,
                                            int E, int k, int32_t* counts, int32_t* offsets,
                                            int32_t* off_lds, int32_t* sorted_pairs,
                                            int32_t* pair_to_row, int2* tiles, int* ntiles,
                                            int32_t* wave_sum) {
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int ept = (E + NT - 1) / NT;              // experts per thread, consecutive
  const int e0 = tid * ept;
  // count (bits 0..15) and touched flag (bits 16..31) of each expert, summed:
  // R <= 32 * 32 pairs and E <= 1024 experts fit their halves
  int local = 0;
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int c = __popc(mask[e]);
      local += c | ((c > 0) << 16);
    }
  }
  const int incl = wave_incl_scan(local);
  if (lane == kWave - 1) wave_sum[wave] = incl;
  __syncthreads();
  int run = incl - local, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int v = wave_sum[w];
    run += w < wave ? v : 0;
    total += v;
  }
  for (int i = 0; i < ept; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int c = __popc(mask[e]);
    const int off = run & 0xffff;
    counts[e] = c;
    offsets[e] = off;
    off_lds[e] = off;
    if (tiles && c > 0) tiles[run >> 16] = make_int2(e | (c << 16), off);
    run += c | ((c > 0) << 16);
  }
  if (tid == 0) {
    offsets[E] = total & 0xffff;
    off_lds[E] = total & 0xffff;
    if (ntiles) *ntiles = total >> 16;
  }
  __syncthreads();
  for (int p = tid; p < R; p += NT) {
    const int t = p / k, e = ids[p];
    const int row = off_lds[e] + __popc(mask[e] & ((1u << t) - 1u));
    sorted_pairs[row] = p;
    pair_to_row[p] = row;
  }
}

}  // namespace
}  // namespace mxm

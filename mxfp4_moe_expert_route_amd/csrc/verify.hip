// Rejection-sampling verification of drafted blocks.
//
// The pages' drafter proposes a whole block of tokens and the backbone
// verifies it in one step, with rejection sampling keeping the output
// lossless; blocks are capped at 8 ("MiMo-V2.5-Pro-FP4-DFlash" model card,
// §3 "Block-Diffusion Speculative Decoding (DFlash)").  Rule (a reading,
// the standard speculative-sampling one): position i is accepted when
// u_i * q_i(d_i) < p_i(d_i) with p_i = softmax(backbone logits), q_i the
// drafter's probabilities, d_i the drafted token; n = leading accepted
// positions; the next token is drawn from max(0, p_n - q_n) if n < L (p_n if
// that is all zero), else from p_L, by inverse CDF in vocabulary order with
// uniform u_L.
//
// Every row is split into P = 32 parts (the last one ragged) so that a
// batch of a few sequences still spreads over the chip:
//   k_verify_stats   one workgroup per (row, part): max and sum of exp over
//                    its part; values are held in registers a batch at a
//                    time, the batch's workgroup max is taken first, so each
//                    element costs one exp;
//   k_verify_parts   one workgroup per (sequence, part): every one combines
//                    the rows' part statistics in the same fixed order,
//                    decides n (lanes 0..L-1 of wave 0 test one position
//                    each), and sums the draw weights over its part of row n;
//   k_verify_draw    one workgroup per sequence: the part sums in order give
//                    the total and the part holding t = u_L * total; that
//                    part's weights are summed again per thread with the
//                    same arithmetic, so its within-part prefix ends exactly
//                    at the part sum, and the first thread whose prefix end
//                    passes t walks its elements to the token.
// A thread's elements in the two last kernels are contiguous, so thread
// order is vocabulary order.  All sums run in fixed orders: the result is
// deterministic, and the token always carries positive weight.
#include <math.h>

#include "common.hpp"

namespace mxm {
namespace {

constexpr int kVT = 256;
constexpr int kParts = 32;
constexpr int kBatch = 8;                      // float4 chunks a thread holds at once
constexpr int kMaxL = 32;

struct MS {
  float m, s;                                  // max and sum of exp(x - m)
};

// exp(y) for y <= 0, -inf giving 0: 2^(y log2 e) with the product split into
// its rounded value t and the remainder (exact through fma, plus the part of
// log2 e below float precision); v_exp_f32 on t and a first-order
// correction for the remainder, which is below 2^-16 in size.  Within a few
// ulp of exp over the whole range.
__device__ __forceinline__ float exp_neg(float y) {
  constexpr float kL2E = 1.44269502162933349609375f;   // log2(e) rounded to float
  constexpr float kL2ELo = 1.925963e-08f;              // log2(e) - kL2E
  constexpr float kLn2 = 0.693147180559945309f;
  y = fmaxf(y, -160.f);                                // exp(-160) underflows; keeps fma finite
  const float t = y * kL2E;
  const float lo = fmaf(y, kL2ELo, fmaf(y, kL2E, -t));
  const float r = __builtin_amdgcn_exp2f(t);
  return fmaf(r, lo * kLn2, r);
}

// butterfly reductions over the lanes of a wave (width w): every lane ends
// with the same value, since each step's operation is commutative
__device__ __forceinline__ float xor_max(float x, int w) {
  for (int off = w / 2; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float xor_sum(float x, int w) {
  for (int off = w / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// float4 chunks of a row's parts: part p covers chunks [p c, min(V / 4, (p + 1) c))
__device__ __forceinline__ int part_chunks(int V) { return (V / 4 + kParts - 1) / kParts; }
__device__ __forceinline__ int part_len(int V, int part) {
  const int nc = part_chunks(V);
  return max(0, min(V / 4 - part * nc, nc));
}

__global__ __launch_bounds__(kVT) void k_verify_stats(const float* __restrict__ target, int V,
                                                     float2* __restrict__ stats) {
  __shared__ float red[2][kVT / kWave];        // double-buffered per-wave values
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int row = blockIdx.x / kParts, part = blockIdx.x % kParts;
  const int nc = part_len(V, part);
  const float4* src =
      reinterpret_cast<const float4*>(target + size_t(row) * V) + size_t(part) * part_chunks(V);
  float M = -INFINITY, sum = 0.f;              // M is the same in every thread
  int ph = 0;
  for (int cb = 0; cb < nc; cb += kBatch * kVT) {
    float4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c = cb + j * kVT + tid;
      // the rows stream through once here (only row n of each block is read
      // again, in the next step): non-temporal loads, 90 -> 85 us at 64
      // blocks
      if (c < nc) {
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + c));
        v[j] = make_float4(t[0], t[1], t[2], t[3]);
      } else {
        v[j] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
    }
    float bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      bm = fmaxf(bm, fmaxf(fmaxf(v[j].x, v[j].y), fmaxf(v[j].z, v[j].w)));
    bm = xor_max(bm, kWave);
    if (lane == 0) red[ph][wave] = bm;
    __syncthreads();
    bm = fmaxf(fmaxf(red[ph][0], red[ph][1]), fmaxf(red[ph][2], red[ph][3]));
    ph ^= 1;
    if (bm > M) {
      sum *= exp_neg(M - bm);
      M = bm;
    }
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (cb + j * kVT + tid < nc) {
        s0 += exp_neg(v[j].x - M);
        s1 += exp_neg(v[j].y - M);
        s2 += exp_neg(v[j].z - M);
        s3 += exp_neg(v[j].w - M);
      }
    }
    sum += (s0 + s1) + (s2 + s3);
  }
  sum = xor_sum(sum, kWave);
  if (lane == 0) red[ph][wave] = sum;          // the other buffer's readers are past a barrier
  __syncthreads();
  if (tid == 0) {
    const float tot = (red[ph][0] + red[ph][1]) + (red[ph][2] + red[ph][3]);
    stats[blockIdx.x] = make_float2(M, M == -INFINITY ? 0.f : tot);
  }
}

// weight of element v of the draw row: p_n(v) - q_n(v) clipped at 0 for a
// residual, p_n(v) otherwise; inv_s = 1 / (sum of exp over row n)
__device__ __forceinline__ float draw_weight(float l, float q, float m, float inv_s,
                                             bool residual) {
  const float p = m == -INFINITY ? 0.f : exp_neg(l - m) * inv_s;
  return residual ? fmaxf(p - q, 0.f) : p;
}

// This thread's chunks [c0, c1) of a part of nc chunks: contiguous, so
// thread order is vocabulary order.
__device__ __forceinline__ void thread_chunks(int nc, int& c0, int& c1) {
  const int per = (nc + kVT - 1) / kVT;
  c0 = min(nc, int(threadIdx.x) * per);
  c1 = min(nc, c0 + per);
}

// Draw weights of this thread's chunks of one part.  Returns their sum in
// element order; the first batch's weights are left in w[] (zero past c1).
__device__ __forceinline__ float thread_weights(const float* lrow, const float* qrow, int V,
                                                int part, float m, float inv_s, bool residual,
                                                float (&w)[kBatch * 4], int& c0, int& c1) {
  const int nc = part_len(V, part);
  const float4* l4 = reinterpret_cast<const float4*>(lrow) + size_t(part) * part_chunks(V);
  const float4* q4 = reinterpret_cast<const float4*>(qrow) + size_t(part) * part_chunks(V);
  thread_chunks(nc, c0, c1);
  float sum = 0.f;
  for (int cb = c0; cb < c1; cb += kBatch) {
    float4 l[kBatch], q[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = cb + j < c1;
      l[j] = in ? l4[cb + j] : make_float4(0.f, 0.f, 0.f, 0.f);
      q[j] = in && residual ? q4[cb + j] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float t[kBatch * 4];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = cb + j < c1;
      t[4 * j + 0] = in ? draw_weight(l[j].x, q[j].x, m, inv_s, residual) : 0.f;
      t[4 * j + 1] = in ? draw_weight(l[j].y, q[j].y, m, inv_s, residual) : 0.f;
      t[4 * j + 2] = in ? draw_weight(l[j].z, q[j].z, m, inv_s, residual) : 0.f;
      t[4 * j + 3] = in ? draw_weight(l[j].w, q[j].w, m, inv_s, residual) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kBatch * 4; ++e) sum += t[e];
    if (cb == c0) {
#pragma unroll
      for (int e = 0; e < kBatch * 4; ++e) w[e] = t[e];
    }
  }
  if (c0 >= c1) {
#pragma unroll
    for (int e = 0; e < kBatch * 4; ++e) w[e] = 0.f;
  }
  return sum;
}

// Within-part prefix of the thread sums: an inclusive scan over each wave's
// lanes, wave totals added in wave order.  pre_in = prefix before this
// thread, pre_out = after it; the block's last pre_out is the part sum, and
// two calls on equal thread sums give bitwise equal results.
__device__ __forceinline__ void part_prefix(float ts, float* wtot, float& pre_in, float& pre_out,
                                            float& total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  float incl = ts;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  float excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.f;
  if (lane == kWave - 1) wtot[wave] = incl;
  __syncthreads();
  float base = 0.f, tot = 0.f;
#pragma unroll
  for (int v = 0; v < kVT / kWave; ++v) {
    if (v == wave) base = tot;
    tot += wtot[v];
  }
  pre_in = base + excl;
  pre_out = base + incl;
  total = tot;
  __syncthreads();                             // wtot may be reused
}

__global__ __launch_bounds__(kVT) void k_verify_parts(
    const float* __restrict__ target, const float* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, int L, int V,
    const float2* __restrict__ stats, float2* __restrict__ row_n_stats,
    float* __restrict__ part_sums, int* __restrict__ nacc) {
  __shared__ MS st[kMaxL + 1];
  __shared__ float wtot[kVT / kWave];
  __shared__ int sn;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / kParts, part = blockIdx.x % kParts;

  // the drafted tokens' logits and draft probabilities (lanes 0..L-1)
  float lg = 0.f, qd = 0.f, uu = 0.f;
  bool inr = false;
  if (tid < L) {
    const int d = tokens[size_t(b) * L + tid];
    uu = uniforms[size_t(b) * (L + 1) + tid];
    inr = d >= 0 && d < V;
    if (inr) {
      lg = target[(size_t(b) * (L + 1) + tid) * V + d];
      qd = draft[(size_t(b) * L + tid) * V + d];
    }
  }
  // row statistics: the 32 lanes of a row take the max of its part maxima,
  // then sum the part sums rescaled to it
  for (int base = 0; base < (L + 1) * kParts; base += kVT) {
    const int i = (base + tid) / kParts, p = (base + tid) % kParts;
    float2 v = make_float2(-INFINITY, 0.f);
    if (i <= L) v = stats[(size_t(b) * (L + 1) + i) * kParts + p];
    const float M = xor_max(v.x, kParts);
    const float S = xor_sum(v.y * exp_neg(v.x - M), kParts);
    if (p == 0 && i <= L) st[i] = MS{M, M == -INFINITY ? 0.f : S};
  }
  __syncthreads();
  if (tid < kWave) {
    bool fail = false;
    if (tid < L) {
      const MS s = st[tid];
      const float p = inr && s.m != -INFINITY ? exp_neg(lg - s.m) / s.s : 0.f;
      fail = !(uu * qd < p);                   // out of range: p = q = 0, rejected
    }
    const unsigned long long m = __ballot(fail);
    if (tid == 0) sn = m ? __ffsll((long long)m) - 1 : L;
  }
  __syncthreads();
  const int n = sn;
  const bool residual = n < L;
  const MS sn_st = st[n];
  const float* lrow = target + (size_t(b) * (L + 1) + n) * V;
  const float* qrow = draft + (size_t(b) * L + (residual ? n : 0)) * V;
  float w[kBatch * 4];
  int c0, c1;
  const float ts = thread_weights(lrow, qrow, V, part, sn_st.m, 1.f / sn_st.s, residual, w, c0, c1);
  float pre_in, pre_out, total;
  part_prefix(ts, wtot, pre_in, pre_out, total);
  if (tid == 0) {
    part_sums[blockIdx.x] = total;
    if (part == 0) {
      nacc[b] = n;
      row_n_stats[b] = make_float2(sn_st.m, sn_st.s);
    }
  }
}

__global__ __launch_bounds__(kVT) void k_verify_draw(
    const float* __restrict__ target, const float* __restrict__ draft,
    const float* __restrict__ uniforms, int L, int V, const float2* __restrict__ row_n_stats,
    const float* __restrict__ part_sums, const int* __restrict__ nacc,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ next_token) {
  __shared__ float ps[kParts];
  __shared__ float wtot[kVT / kWave];
  __shared__ unsigned long long first_m[kVT / kWave], pos_m[kVT / kWave];
  __shared__ int spart, sclaim, stok;
  __shared__ float sbase, starget;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int n = nacc[b];
  const float2 rs = row_n_stats[b];
  const float m = rs.x, inv_s = 1.f / rs.y;
  bool residual = n < L;
  const float* lrow = target + (size_t(b) * (L + 1) + n) * V;
  const float* qrow = draft + (size_t(b) * L + (residual ? n : 0)) * V;
  if (tid < kParts) ps[tid] = part_sums[size_t(b) * kParts + tid];
  __syncthreads();
  float total = 0.f;
  for (int p = 0; p < kParts; ++p) total += ps[p];
  float w[kBatch * 4];
  int c0, c1;
  if (residual && !(total > 0.f)) {
    // degenerate residual (p_n == q_n up to rounding): draw from p_n
    residual = false;
    for (int p = 0; p < kParts; ++p) {
      const float ts = thread_weights(lrow, qrow, V, p, m, inv_s, false, w, c0, c1);
      float a, bb, tot;
      part_prefix(ts, wtot, a, bb, tot);
      if (tid == 0) ps[p] = tot;
    }
    __syncthreads();
  }
  if (tid == 0) {
    float tot = 0.f;
    for (int p = 0; p < kParts; ++p) tot += ps[p];
    const float t = uniforms[size_t(b) * (L + 1) + L] * tot;
    float pre = 0.f, last_pre = 0.f;
    int k = -1, last = 0;
    for (int p = 0; p < kParts; ++p) {
      if (k < 0 && t < pre + ps[p]) {
        k = p;
        sbase = pre;
      }
      if (ps[p] > 0.f) {
        last = p;
        last_pre = pre;
      }
      pre += ps[p];
    }
    if (k < 0) {                               // t rounded onto the total: the last weight
      k = last;
      sbase = last_pre;
    }
    spart = k;
    starget = t;
  }
  __syncthreads();
  const int k = spart;
  const float t = starget, base = sbase;
  const float ts = thread_weights(lrow, qrow, V, k, m, inv_s, residual, w, c0, c1);
  float pre_in, pre_out, total_k;
  part_prefix(ts, wtot, pre_in, pre_out, total_k);
  // claim: the first thread with weight whose prefix end passes t; failing
  // that (rounding), the last thread with weight
  const bool pos = ts > 0.f;
  const unsigned long long fm = __ballot(pos && t < base + pre_out);
  const unsigned long long pm = __ballot(pos);
  if (lane_id() == 0) {
    first_m[tid / kWave] = fm;
    pos_m[tid / kWave] = pm;
  }
  __syncthreads();
  if (tid == 0) {
    int c = -1;
    for (int v = 0; v < kVT / kWave && c < 0; ++v)
      if (first_m[v]) c = v * kWave + __ffsll((long long)first_m[v]) - 1;
    for (int v = kVT / kWave - 1; v >= 0 && c < 0; --v)
      if (pos_m[v]) c = v * kWave + 63 - __clzll((long long)pos_m[v]);
    sclaim = c;
    stok = V - 1;                              // unreachable: part k has weight
  }
  __syncthreads();
  if (tid == sclaim) {
    // walk this thread's elements: the first with weight whose running sum
    // passes t, else its last element with weight
    const float4* l4 = reinterpret_cast<const float4*>(lrow) + size_t(k) * part_chunks(V);
    const float4* q4 = reinterpret_cast<const float4*>(qrow) + size_t(k) * part_chunks(V);
    const int v0 = 4 * (k * part_chunks(V) + c0);
    float acc = base + pre_in;
    int pick = -1, lastv = -1;
#pragma unroll
    for (int e = 0; e < kBatch * 4; ++e) {
      if (w[e] > 0.f) {
        lastv = v0 + e;
        acc += w[e];
        if (pick < 0 && acc > t) pick = v0 + e;
      }
    }
    for (int cb = c0 + kBatch; cb < c1 && pick < 0; ++cb) {   // threads with more than a batch
      const float4 l = l4[cb];
      const float4 q = residual ? q4[cb] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float x[4] = {draw_weight(l.x, q.x, m, inv_s, residual),
                          draw_weight(l.y, q.y, m, inv_s, residual),
                          draw_weight(l.z, q.z, m, inv_s, residual),
                          draw_weight(l.w, q.w, m, inv_s, residual)};
      for (int e = 0; e < 4; ++e) {
        if (x[e] > 0.f) {
          lastv = 4 * (k * part_chunks(V) + cb) + e;
          acc += x[e];
          if (pick < 0 && acc > t) pick = lastv;
        }
      }
    }
    stok = pick >= 0 ? pick : lastv;
  }
  __syncthreads();
  if (tid == 0) {
    accept_len[b] = n;
    next_token[b] = stok;
  }
}

}  // namespace

// workspace: part statistics [B][L+1][P] float2, row-n statistics [B] float2,
// part sums [B][P] float, n [B] int
size_t verify_workspace_bytes(int B, int L) {
  const size_t stats = size_t(B) * (L + 1) * kParts * sizeof(float2);
  const size_t rown = size_t(B) * sizeof(float2);
  const size_t parts = size_t(B) * kParts * sizeof(float);
  const size_t n = size_t(B) * sizeof(int);
  return stats + rown + parts + n;
}

hipError_t launch_verify(const float* target, const float* draft, const int32_t* tokens,
                         const float* uniforms, int B, int L, int V, int32_t* accept_len,
                         int32_t* next_token, void* workspace, hipStream_t s) {
  if (B == 0) return hipSuccess;
  float2* stats = static_cast<float2*>(workspace);
  float2* rown = stats + size_t(B) * (L + 1) * kParts;
  float* part_sums = reinterpret_cast<float*>(rown + B);
  int* nacc = reinterpret_cast<int*>(part_sums + size_t(B) * kParts);
  k_verify_stats<<<unsigned(B * (L + 1) * kParts), kVT, 0, s>>>(target, V, stats);
  k_verify_parts<<<unsigned(B * kParts), kVT, 0, s>>>(target, draft, tokens, uniforms, L, V, stats,
                                                      rown, part_sums, nacc);
  k_verify_draw<<<unsigned(B), kVT, 0, s>>>(target, draft, uniforms, L, V, rown, part_sums, nacc,
                                            accept_len, next_token);
  return hipGetLastError();
}

}  // namespace mxm

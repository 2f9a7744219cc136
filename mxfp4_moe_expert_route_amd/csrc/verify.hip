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
//   k_verify_stats   one workgroup per (row, part): online max / sum of
//                    exp over its part, combined in a fixed tree;
//   k_verify_parts   one workgroup per (sequence, part): every one combines
//                    the rows' part statistics in order, decides n (lanes
//                    0..L-1 of wave 0 test one position each), and sums the
//                    draw weights over its part of row n;
//   k_verify_draw    one workgroup per sequence: the part sums in order give
//                    the total and the part holding u_L * total; that part is
//                    summed again per thread in the same order (a thread's
//                    elements are contiguous, so thread order is vocabulary
//                    order), and the thread whose interval holds the target
//                    walks its elements to the token.
// All sums run in fixed orders, so the result is deterministic.
#include <math.h>

#include "common.hpp"

namespace mxm {
namespace {

constexpr int kVT = 256;
constexpr int kParts = 32;

struct MS {
  float m, s;
};

__device__ __forceinline__ MS ms_combine(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return MS{m, 0.f};
  return MS{m, a.s * expf(a.m - m) + b.s * expf(b.m - m)};
}

__device__ __forceinline__ void ms_add(MS& a, float x) {
  if (x > a.m) {
    a.s = (a.m == -INFINITY ? 0.f : a.s * expf(a.m - x)) + 1.f;
    a.m = x;
  } else if (x != -INFINITY) {
    a.s += expf(x - a.m);
  }
}

// float4 chunks of a row's parts: part p covers chunks [p c, min(V / 4, (p + 1) c))
__device__ __forceinline__ int part_chunks(int V) { return (V / 4 + kParts - 1) / kParts; }
__device__ __forceinline__ int part_len(int V, int part) {
  const int nc = part_chunks(V);
  return max(0, min(V / 4 - part * nc, nc));
}

__global__ __launch_bounds__(kVT) void k_verify_stats(const float* __restrict__ target, int V,
                                                     float2* __restrict__ stats) {
  __shared__ MS sm[kVT];
  const int tid = threadIdx.x;
  const int row = blockIdx.x / kParts, part = blockIdx.x % kParts;
  const int nc = part_len(V, part);
  const float4* src =
      reinterpret_cast<const float4*>(target + size_t(row) * V) + size_t(part) * part_chunks(V);
  MS a[4] = {{-INFINITY, 0.f}, {-INFINITY, 0.f}, {-INFINITY, 0.f}, {-INFINITY, 0.f}};
#pragma unroll 2
  for (int c = tid; c < nc; c += kVT) {      // four independent chains per thread
    const float4 v = src[c];
    ms_add(a[0], v.x);
    ms_add(a[1], v.y);
    ms_add(a[2], v.z);
    ms_add(a[3], v.w);
  }
  sm[tid] = ms_combine(ms_combine(a[0], a[1]), ms_combine(a[2], a[3]));
  __syncthreads();
  for (int st = kVT / 2; st > 0; st >>= 1) {
    if (tid < st) sm[tid] = ms_combine(sm[tid], sm[tid + st]);
    __syncthreads();
  }
  if (tid == 0) stats[blockIdx.x] = make_float2(sm[0].m, sm[0].s);
}

// weight of element v of the draw row: p_n(v) - q_n(v) clipped at 0 for a
// residual, p_n(v) otherwise
__device__ __forceinline__ float draw_weight(float l, float q, MS st, bool residual) {
  const float p = st.m == -INFINITY ? 0.f : expf(l - st.m) / st.s;
  return residual ? fmaxf(p - q, 0.f) : p;
}

// A thread's chunks of a part are contiguous, so thread order is vocabulary
// order: chunks [c0, c1) of the part.
__device__ __forceinline__ void thread_chunks(int nc, int& c0, int& c1) {
  const int per = (nc + kVT - 1) / kVT;
  c0 = min(nc, int(threadIdx.x) * per);
  c1 = min(nc, c0 + per);
}

// this thread's sum of the draw weights over its chunks of part `part`
__device__ __forceinline__ float thread_part_sum(const float* lrow, const float* qrow, int V,
                                                 int part, MS st, bool residual) {
  const int nc = part_len(V, part);
  const float4* l4 = reinterpret_cast<const float4*>(lrow) + size_t(part) * part_chunks(V);
  const float4* q4 = reinterpret_cast<const float4*>(qrow) + size_t(part) * part_chunks(V);
  float sum = 0.f;
  int c0, c1;
  thread_chunks(nc, c0, c1);
  for (int c = c0; c < c1; ++c) {
    const float4 l = l4[c];
    const float4 q = residual ? q4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    sum += draw_weight(l.x, q.x, st, residual);
    sum += draw_weight(l.y, q.y, st, residual);
    sum += draw_weight(l.z, q.z, st, residual);
    sum += draw_weight(l.w, q.w, st, residual);
  }
  return sum;
}

// row statistics of sequence b, parts combined in order, into sm_st[0..L]
__device__ __forceinline__ void row_stats(const float2* __restrict__ stats, int b, int L,
                                          MS* sm_st) {
  const int i = threadIdx.x;
  if (i <= L) {
    const float2* s = stats + (size_t(b) * (L + 1) + i) * kParts;
    MS a{s[0].x, s[0].y};
    for (int p = 1; p < kParts; ++p) a = ms_combine(a, MS{s[p].x, s[p].y});
    sm_st[i] = a;
  }
}

__global__ __launch_bounds__(kVT) void k_verify_parts(
    const float* __restrict__ target, const float* __restrict__ draft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uniforms, int L, int V,
    const float2* __restrict__ stats, float* __restrict__ part_sums, int* __restrict__ nacc) {
  __shared__ MS st[33];
  __shared__ float sm[kVT];
  __shared__ int sn;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / kParts, part = blockIdx.x % kParts;
  row_stats(stats, b, L, st);
  __syncthreads();
  if (tid < kWave) {
    bool fail = false;
    if (tid < L) {
      const int d = tokens[size_t(b) * L + tid];
      float p = 0.f, q = 0.f;
      if (d >= 0 && d < V) {
        const MS s = st[tid];
        p = s.m == -INFINITY ? 0.f : expf(target[(size_t(b) * (L + 1) + tid) * V + d] - s.m) / s.s;
        q = draft[(size_t(b) * L + tid) * V + d];
      }
      fail = !(uniforms[size_t(b) * (L + 1) + tid] * q < p);
    }
    const unsigned long long m = __ballot(fail);
    if (tid == 0) sn = m ? __ffsll((long long)m) - 1 : L;
  }
  __syncthreads();
  const int n = sn;
  const bool residual = n < L;
  const float* lrow = target + (size_t(b) * (L + 1) + n) * V;
  const float* qrow = draft + (size_t(b) * L + (residual ? n : 0)) * V;
  sm[tid] = thread_part_sum(lrow, qrow, V, part, st[n], residual);
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
    for (int j = 0; j < kVT; ++j) s += sm[j];
    part_sums[blockIdx.x] = s;
    if (part == 0) nacc[b] = n;
  }
}

__global__ __launch_bounds__(kVT) void k_verify_draw(
    const float* __restrict__ target, const float* __restrict__ draft,
    const float* __restrict__ uniforms, int L, int V, const float2* __restrict__ stats,
    const float* __restrict__ part_sums, const int* __restrict__ nacc,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ next_token) {
  __shared__ MS st[33];
  __shared__ float sm[kVT];
  __shared__ float pre_t[kVT + 1];
  __shared__ int spart, stok;
  __shared__ float sbase, starget;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  row_stats(stats, b, L, st);
  const int n = nacc[b];
  bool residual = n < L;
  float total = 0.f;
  for (int p = 0; p < kParts; ++p) total += part_sums[size_t(b) * kParts + p];
  const float* lrow = target + (size_t(b) * (L + 1) + n) * V;
  const float* qrow = draft + (size_t(b) * L + (residual ? n : 0)) * V;
  __syncthreads();
  float psum[kParts];
  if (residual && !(total > 0.f)) {
    // degenerate residual (p_n == q_n up to rounding): draw from p_n
    residual = false;
    for (int p = 0; p < kParts; ++p) {
      sm[tid] = thread_part_sum(lrow, qrow, V, p, st[n], false);
      __syncthreads();
      if (tid == 0) {
        float s = 0.f;
        for (int j = 0; j < kVT; ++j) s += sm[j];
        sbase = s;
      }
      __syncthreads();
      psum[p] = sbase;
      __syncthreads();
    }
  } else {
    for (int p = 0; p < kParts; ++p) psum[p] = part_sums[size_t(b) * kParts + p];
  }
  if (tid == 0) {
    float tot = 0.f;
    for (int p = 0; p < kParts; ++p) tot += psum[p];
    const float t = uniforms[size_t(b) * (L + 1) + L] * tot;
    float pre = 0.f;
    int k = -1;
    for (int p = 0; p < kParts; ++p) {
      if (t < pre + psum[p]) {
        k = p;
        break;
      }
      pre += psum[p];
    }
    spart = k;
    sbase = pre;
    starget = t;
    stok = V - 1;                              // t outside every interval
  }
  __syncthreads();
  const int k = spart;
  if (k >= 0) {
    sm[tid] = thread_part_sum(lrow, qrow, V, k, st[n], residual);
    __syncthreads();
    if (tid == 0) {                            // running sums in the part sum's order
      float s = 0.f;
      pre_t[0] = sbase;
      for (int j = 0; j < kVT; ++j) {
        s += sm[j];
        pre_t[j + 1] = sbase + s;
      }
    }
    __syncthreads();
    const float t = starget;
    if (pre_t[tid] <= t && t < pre_t[tid + 1]) {
      // walk this thread's elements: the first whose running sum passes t,
      // else (rounding at the segment's end) its last element with weight
      const int nc = part_len(V, k);
      const float4* l4 = reinterpret_cast<const float4*>(lrow) + size_t(k) * part_chunks(V);
      const float4* q4 = reinterpret_cast<const float4*>(qrow) + size_t(k) * part_chunks(V);
      float acc = pre_t[tid];
      int pick = -1, last = -1;
      int c0, c1;
      thread_chunks(nc, c0, c1);
      for (int c = c0; c < c1 && pick < 0; ++c) {
        const float4 l = l4[c];
        const float4 q = residual ? q4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float wv[4] = {draw_weight(l.x, q.x, st[n], residual),
                             draw_weight(l.y, q.y, st[n], residual),
                             draw_weight(l.z, q.z, st[n], residual),
                             draw_weight(l.w, q.w, st[n], residual)};
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * (k * part_chunks(V) + c) + e;
          if (wv[e] > 0.f) last = v;
          acc += wv[e];
          if (pick < 0 && acc > t && wv[e] > 0.f) pick = v;
        }
      }
      stok = pick >= 0 ? pick : (last >= 0 ? last : V - 1);
    }
  }
  __syncthreads();
  if (tid == 0) {
    accept_len[b] = n;
    next_token[b] = stok;
  }
}

}  // namespace

size_t verify_workspace_bytes(int B, int L) {
  const size_t stats = size_t(B) * (L + 1) * kParts * sizeof(float2);
  const size_t parts = size_t(B) * kParts * sizeof(float);
  const size_t n = size_t(B) * sizeof(int);
  return stats + parts + n;
}

hipError_t launch_verify(const float* target, const float* draft, const int32_t* tokens,
                         const float* uniforms, int B, int L, int V, int32_t* accept_len,
                         int32_t* next_token, void* workspace, hipStream_t s) {
  float2* stats = static_cast<float2*>(workspace);
  float* part_sums = reinterpret_cast<float*>(stats + size_t(B) * (L + 1) * kParts);
  int* nacc = reinterpret_cast<int*>(part_sums + size_t(B) * kParts);
  k_verify_stats<<<unsigned(B * (L + 1) * kParts), kVT, 0, s>>>(target, V, stats);
  k_verify_parts<<<unsigned(B * kParts), kVT, 0, s>>>(target, draft, tokens, uniforms, L, V, stats,
                                                      part_sums, nacc);
  k_verify_draw<<<unsigned(B), kVT, 0, s>>>(target, draft, uniforms, L, V, stats, part_sums, nacc,
                                            accept_len, next_token);
  return hipGetLastError();
}

}  // namespace mxm

// Grouped MXFP4 expert contractions: gate/up + SwiGLU, and down.
//
// The experts of the layer are stored in MXFP4 (block 32) and the activations
// stay bf16 ("MiMo-V2.5-Pro-FP4-DFlash" model card, §2 "FP4 Quantization",
// §5 "Deployment" --dtype bfloat16).  At a verify step of 8 tokens per
// sequence (model card §3, mask block capped at 8) most chosen experts see one
// or two rows, so the time is the stream of weight bytes from HBM; the
// contraction itself runs on MFMA so that the VALU only converts FP4 to bf16.
//
// Work decomposition
//   * Each expert's rows (a segment of the permutation) are cut into tiles of
//     up to MT = 16*MS rows.  The grid is sized on the host from T, k and E
//     only (an upper bound on the tile count); each workgroup finds its tile
//     from the device-side offsets and leaves if past the last one.  Nothing
//     waits on the host.
//   * A workgroup has 4 waves; each wave owns NSUB 16-row subtiles of output
//     features and streams the matching weight rows over the whole K.
//
// Register roles (v_mfma_f32_16x16x32_bf16, wave64).  Lane l supplies operand
// row (l % 16) for K-slots of lane group g = l / 16 and receives D rows
// 4g..4g+3 of column (l % 16).  A = weights (rows = output features, K along
// the weight row), B = activations (rows = token rows).
//   K assignment: at step s lane group g takes MX block 4s + g of its row
//   (16 code bytes + 1 scale byte, one 16-byte load); MFMA j = 0..3 of the
//   step uses elements 8j..8j+7 of that block.  A and B lanes follow the same
//   assignment, so each MFMA sums matching K indices whatever the hardware's
//   internal K order.
//   FP4 -> bf16: v_cvt_scalef32_pk_bf16_fp4 applies the block scale while
//   converting, 4 instructions per 8 weights.
#include "common.hpp"

namespace mxm {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

template <int NA, int MS>
struct Frag {
  uint4 c[NA];          // 32 E2M1 codes of this lane's block, per weight subtile
  uint32_t s[NA];       // the block's E8M0 scale byte
  uint4 x[MS][4];       // 32 bf16 activations of this lane's block, per row subtile
};

template <int NA, int MS>
__device__ __forceinline__ void load_frag(Frag<NA, MS>& f, const uint8_t* const (&wc)[NA],
                                          const uint8_t* const (&ws)[NA],
                                          const uint16_t* const (&xr)[MS], const bool (&xv)[MS],
                                          int blk, bool ok) {
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    if (ok) {
      f.c[a] = *reinterpret_cast<const uint4*>(wc[a] + size_t(blk) * 16);
      f.s[a] = ws[a][blk];
    } else {
      f.c[a] = make_uint4(0u, 0u, 0u, 0u);
      f.s[a] = 0u;
    }
  }
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const uint4* src = reinterpret_cast<const uint4*>(xr[m] + size_t(blk) * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      f.x[m][j] = (ok && xv[m]) ? src[j] : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int NA, int MS>
__device__ __forceinline__ void mma_frag(const Frag<NA, MS>& f, f32x4 (&acc)[NA][MS]) {
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const float sc = e8m0_to_f32(f.s[a]);
    const uint32_t cw[4] = {f.c[a].x, f.c[a].y, f.c[a].z, f.c[a].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 wa = dequant8(cw[j], sc);
#pragma unroll
      for (int m = 0; m < MS; ++m)
        acc[a][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, as_bf16x8(f.x[m][j]), acc[a][m],
                                                            0, 0, 0);
    }
  }
}

// acc[a][m] += W_a (16 rows x K) . X_m (16 rows x K)^T over all nblk MX blocks.
template <int NA, int MS>
__device__ __forceinline__ void stream_k(const uint8_t* const (&wc)[NA],
                                         const uint8_t* const (&ws)[NA],
                                         const uint16_t* const (&xr)[MS], const bool (&xv)[MS],
                                         int nblk, f32x4 (&acc)[NA][MS]) {
  const int g = lane_id() >> 4;
  const int nsteps = (nblk + 3) >> 2;
  Frag<NA, MS> cur;
  load_frag<NA, MS>(cur, wc, ws, xr, xv, g, g < nblk);
  for (int s = 0; s < nsteps; ++s) {
    Frag<NA, MS> nxt;
    const int blk = 4 * (s + 1) + g;
    if (s + 1 < nsteps) load_frag<NA, MS>(nxt, wc, ws, xr, xv, blk, blk < nblk);
    mma_frag<NA, MS>(cur, acc);
    cur = nxt;
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  A wave owns 16*NSUB intermediate columns: the matching
// gate rows and up rows of W13 (NA = 2*NSUB weight subtiles).

template <int MS, int NSUB>
__global__ __launch_bounds__(kThreads) void k_gate_up(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted_pairs,
    const int32_t* __restrict__ offsets, int H, int I, int E, int k,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    uint16_t* __restrict__ h, int ntile_n) {
  constexpr int NA = 2 * NSUB;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int slot = blockIdx.x / ntile_n;
  const int nt = blockIdx.x - slot * ntile_n;
  Tile t;
  if (!find_tile(offsets, E, 16 * MS, slot, t)) return;
  const int i0 = (nt * kWaves + wave) * 16 * NSUB;
  if (i0 >= I) return;

  const size_t erow = size_t(t.e) * 2 * I;
  const uint8_t* wc[NA];
  const uint8_t* ws[NA];
#pragma unroll
  for (int a = 0; a < NSUB; ++a) {
    const int col = min(i0 + 16 * a, I - 16) + r16;       // clamp keeps loads in bounds
    wc[a] = codes + (erow + col) * size_t(H / 2);
    ws[a] = scales + (erow + col) * size_t(H / 32);
    wc[NSUB + a] = codes + (erow + I + col) * size_t(H / 2);
    ws[NSUB + a] = scales + (erow + I + col) * size_t(H / 32);
  }
  const uint16_t* xr[MS];
  bool xv[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int mi = 16 * m + r16;
    xv[m] = mi < t.rows;
    const int row = t.row0 + min(mi, t.rows - 1);
    xr[m] = x + size_t(sorted_pairs[row] / k) * H;
  }
  f32x4 acc[NA][MS];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int m = 0; m < MS; ++m) acc[a][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  stream_k<NA, MS>(wc, ws, xr, xv, H / 32, acc);

  // lane holds D[4g+v][r16]: intermediate column i0+16a+4g+v of row r16
#pragma unroll
  for (int a = 0; a < NSUB; ++a) {
    if (i0 + 16 * a >= I) continue;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const int mi = 16 * m + r16;
      if (mi >= t.rows) continue;
      const f32x4 gv = acc[a][m];
      const f32x4 uv = acc[NSUB + a][m];
      const uint32_t h0 = f32_to_bf16_rne(silu_mul(gv[0], uv[0]));
      const uint32_t h1 = f32_to_bf16_rne(silu_mul(gv[1], uv[1]));
      const uint32_t h2 = f32_to_bf16_rne(silu_mul(gv[2], uv[2]));
      const uint32_t h3 = f32_to_bf16_rne(silu_mul(gv[3], uv[3]));
      uint2* dst = reinterpret_cast<uint2*>(h + size_t(t.row0 + mi) * I + i0 + 16 * a + 4 * g);
      *dst = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
    }
  }
}

// ---------------------------------------------------------------------------
// down.  A wave owns 16*NSUB output features (rows of W2).

template <int MS, int NSUB>
__global__ __launch_bounds__(kThreads) void k_down(
    const uint16_t* __restrict__ hin, const int32_t* __restrict__ offsets, int H, int I, int E,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, float* __restrict__ y,
    int ntile_n) {
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int slot = blockIdx.x / ntile_n;
  const int nt = blockIdx.x - slot * ntile_n;
  Tile t;
  if (!find_tile(offsets, E, 16 * MS, slot, t)) return;
  const int n0 = (nt * kWaves + wave) * 16 * NSUB;
  if (n0 >= H) return;

  const size_t erow = size_t(t.e) * H;
  const uint8_t* wc[NSUB];
  const uint8_t* ws[NSUB];
#pragma unroll
  for (int a = 0; a < NSUB; ++a) {
    const int n = min(n0 + 16 * a, H - 16) + r16;
    wc[a] = codes + (erow + n) * size_t(I / 2);
    ws[a] = scales + (erow + n) * size_t(I / 32);
  }
  const uint16_t* xr[MS];
  bool xv[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int mi = 16 * m + r16;
    xv[m] = mi < t.rows;
    xr[m] = hin + size_t(t.row0 + min(mi, t.rows - 1)) * I;
  }
  f32x4 acc[NSUB][MS];
#pragma unroll
  for (int a = 0; a < NSUB; ++a)
#pragma unroll
    for (int m = 0; m < MS; ++m) acc[a][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  stream_k<NSUB, MS>(wc, ws, xr, xv, I / 32, acc);

#pragma unroll
  for (int a = 0; a < NSUB; ++a) {
    if (n0 + 16 * a >= H) continue;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const int mi = 16 * m + r16;
      if (mi >= t.rows) continue;
      float4* dst = reinterpret_cast<float4*>(y + size_t(t.row0 + mi) * H + n0 + 16 * a + 4 * g);
      const f32x4 v = acc[a][m];
      *dst = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// Rows per tile: MS subtiles of 16.  Chosen from the mean rows per touched
// expert (an upper bound the host can compute without reading the counts).
int choose_ms(int R, int E) {
  const int touched = R < E ? R : E;
  const int avg = (R + touched - 1) / touched;
  if (avg <= 16) return 1;
  if (avg <= 32) return 2;
  return 4;
}

int tile_slots(int R, int E, int mt) { return (R < E ? R : E) + (R + mt - 1) / mt; }

template <int MS>
hipError_t gate_up_ms(const uint16_t* x, const int32_t* sp, const int32_t* off, int T, int H,
                      int I, int E, int k, const uint8_t* c, const uint8_t* sc, uint16_t* h,
                      hipStream_t s) {
  constexpr int NSUB = 1;
  const int R = T * k;
  const int ntile_n = (I + kWaves * 16 * NSUB - 1) / (kWaves * 16 * NSUB);
  const int64_t grid = int64_t(tile_slots(R, E, 16 * MS)) * ntile_n;
  k_gate_up<MS, NSUB><<<dim3(unsigned(grid)), kThreads, 0, s>>>(x, sp, off, H, I, E, k, c, sc, h,
                                                                  ntile_n);
  return hipGetLastError();
}

template <int MS>
hipError_t down_ms(const uint16_t* h, const int32_t* off, int T, int H, int I, int E, int k,
                   const uint8_t* c, const uint8_t* sc, float* y, hipStream_t s) {
  constexpr int NSUB = 4;
  const int R = T * k;
  const int ntile_n = (H + kWaves * 16 * NSUB - 1) / (kWaves * 16 * NSUB);
  const int64_t grid = int64_t(tile_slots(R, E, 16 * MS)) * ntile_n;
  k_down<MS, NSUB><<<dim3(unsigned(grid)), kThreads, 0, s>>>(h, off, H, I, E, c, sc, y, ntile_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const uint16_t* x, const int32_t* sorted_pairs, const int32_t* offsets,
                          int T, int H, int I, int E, int k, const uint8_t* codes,
                          const uint8_t* scales, uint16_t* h, hipStream_t s) {
  switch (choose_ms(T * k, E)) {
    case 1: return gate_up_ms<1>(x, sorted_pairs, offsets, T, H, I, E, k, codes, scales, h, s);
    case 2: return gate_up_ms<2>(x, sorted_pairs, offsets, T, H, I, E, k, codes, scales, h, s);
    default: return gate_up_ms<4>(x, sorted_pairs, offsets, T, H, I, E, k, codes, scales, h, s);
  }
}

hipError_t launch_down(const uint16_t* h, const int32_t* offsets, int T, int H, int I, int E,
                       int k, const uint8_t* codes, const uint8_t* scales, float* y,
                       hipStream_t s) {
  switch (choose_ms(T * k, E)) {
    case 1: return down_ms<1>(h, offsets, T, H, I, E, k, codes, scales, y, s);
    case 2: return down_ms<2>(h, offsets, T, H, I, E, k, codes, scales, y, s);
    default: return down_ms<4>(h, offsets, T, H, I, E, k, codes, scales, y, s);
  }
}

}  // namespace mxm

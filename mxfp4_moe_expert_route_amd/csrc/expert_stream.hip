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
//     up to MT = 16*MS rows.  The host bounds the tile count from T, k and E
//     only; each workgroup walks tile slots grid-stride, finds each tile from
//     the device-side offsets and stops at the first slot past the last tile
//     (the grid is capped, so a bound far above the real count, as when most
//     rows go to the dense kernel, costs few empty workgroups).  Nothing
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

// Tile shape (the measured best on MI355X).
constexpr int kWDepth = 2;          // fragments in flight per wave
constexpr int kGuNsub = 2;          // 16-column intermediate subtiles per wave (gate/up)
constexpr int kDnNsub = 4;          // 16-row output subtiles per wave (down)

// One step of a lane's streams: one MX block (16 code bytes) of each weight
// subtile and the 32 matching bf16 activations of each row subtile.
template <int NA, int MS>
struct Frag {
  uint4 c[NA];
  uint4 x[MS][4];
};

// Loads are unconditional (addresses clamped in bounds) so that no branch
// separates them: the compiler then keeps kWDepth steps in flight instead
// of draining the load queue before every step.  Rows past the tile's end
// read a valid row whose output column is never stored.
template <int NA, int MS>
__device__ __forceinline__ void load_frag(Frag<NA, MS>& f, const uint8_t* const (&wc)[NA],
                                          const uint16_t* const (&xr)[MS], int blk, int nblk) {
  const int b = blk < nblk ? blk : nblk - 1;
#pragma unroll
  for (int a = 0; a < NA; ++a) f.c[a] = *reinterpret_cast<const uint4*>(wc[a] + size_t(b) * 16);
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const uint4* src = reinterpret_cast<const uint4*>(xr[m] + size_t(b) * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.x[m][j] = src[j];
  }
}

// `sl[a]` points at this lane's row of subtile a's scales in LDS.  A block
// past the end of K gets scale 0, so it contributes nothing.
template <int NA, int MS>
__device__ __forceinline__ void mma_frag(const Frag<NA, MS>& f, const uint8_t* const (&sl)[NA],
                                         int blk, int nblk, f32x4 (&acc)[NA][MS]) {
  const bool ok = blk < nblk;
  const int b = ok ? blk : 0;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const float sc = ok ? e8m0_to_f32(sl[a][b]) : 0.f;
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

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 layout:
// vmcnt low bits 3:0, high bits 15:14; expcnt 6:4 and lgkmcnt 11:8 at max).
#define MXM_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

// One asynchronous 16-byte global->LDS load per lane: lane L writes its 16
// bytes at lds + 16L.
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// Start copying the scales of NA 16-row weight subtiles into this wave's LDS
// area.  Rows of a subtile are consecutive, so its scales are one contiguous
// run of 16*nblk bytes starting at a multiple of 16*nblk: whole 16-byte
// chunks, moved by asynchronous global->LDS loads (lane L of an instruction
// lands at its base + 16L), all issued back to back so the copy costs one
// memory latency.  The caller waits for vmcnt before reading the area.
template <int NA>
__device__ __forceinline__ void stage_scales(const uint8_t* const (&ws0)[NA], int nblk,
                                             uint8_t* lds) {
  const int lane = lane_id();
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    for (int i0 = 0; i0 < nblk; i0 += kWave) {
      if (i0 + lane < nblk)
        dma16(ws0[a] + size_t(i0 + lane) * 16, lds + a * 16 * nblk + i0 * 16);
    }
  }
}

// acc[a][m] += W_a (16 rows x K) . X_m (16 rows x K)^T over all nblk MX blocks,
// with kWDepth steps of code/activation loads in flight.  The step count is
// padded to a multiple of the depth with zero-scale steps so the ring of
// fragments has compile-time indices and the loop body has no branch.
template <int NA, int MS>
__device__ __forceinline__ void stream_k(const uint8_t* const (&wc)[NA],
                                         const uint8_t* const (&ws0)[NA], uint8_t* my_lds,
                                         const uint8_t* const (&sl)[NA],
                                         const uint16_t* const (&xr)[MS], int nblk,
                                         f32x4 (&acc)[NA][MS]) {
  constexpr int D = kWDepth;
  const int g = lane_id() >> 4;
  const int nsteps = (((nblk + 3) >> 2) + D - 1) / D * D;
  Frag<NA, MS> f[D];
#pragma unroll
  for (int d = 0; d < D; ++d) load_frag<NA, MS>(f[d], wc, xr, 4 * d + g, nblk);
  stage_scales<NA>(ws0, nblk, my_lds);
  // the first fragments and the scale copy land together
  __builtin_amdgcn_s_waitcnt(MXM_VMCNT(0));
  for (int s0 = 0; s0 < nsteps; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      mma_frag<NA, MS>(f[d], sl, 4 * (s0 + d) + g, nblk, acc);
      load_frag<NA, MS>(f[d], wc, xr, 4 * (s0 + d + D) + g, nblk);
    }
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
    uint16_t* __restrict__ h, int ntile_n, int hi) {
  constexpr int NA = 2 * NSUB;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int r16 = lane & 15;
  const int g = lane >> 4;
  for (int idx = blockIdx.x;; idx += gridDim.x) {
  const int slot = idx / ntile_n;
  const int nt = idx - slot * ntile_n;
  Tile t;
  if (!find_tile(offsets, E, 16 * MS, slot, t, 1, hi)) return;
  const int i0 = (nt * kWaves + wave) * 16 * NSUB;
  if (i0 >= I) continue;

  const int nblk = H / 32;
  const size_t erow = size_t(t.e) * 2 * I;
  const uint8_t* wc[NA];      // this lane's weight row, per subtile
  const uint8_t* ws0[NA];     // first scale byte of each subtile (16 rows)
  const uint8_t* sl[NA];      // this lane's scale row in LDS
  extern __shared__ uint8_t lds_scales[];
  uint8_t* my_lds = lds_scales + wave * NA * 16 * nblk;
#pragma unroll
  for (int a = 0; a < NSUB; ++a) {
    const int c0 = min(i0 + 16 * a, I - 16);             // clamp keeps loads in bounds
    wc[a] = codes + (erow + c0 + r16) * size_t(H / 2);
    wc[NSUB + a] = codes + (erow + I + c0 + r16) * size_t(H / 2);
    ws0[a] = scales + (erow + c0) * size_t(nblk);
    ws0[NSUB + a] = scales + (erow + I + c0) * size_t(nblk);
  }
#pragma unroll
  for (int a = 0; a < NA; ++a) sl[a] = my_lds + a * 16 * nblk + r16 * nblk;
  const uint16_t* xr[MS];          // rows past the tile's end re-read its last row
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int mi = 16 * m + r16;
    const int row = t.row0 + min(mi, t.rows - 1);
    xr[m] = x + size_t(sorted_pairs[row] / k) * H;
  }
  f32x4 acc[NA][MS];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int m = 0; m < MS; ++m) acc[a][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  stream_k<NA, MS>(wc, ws0, my_lds, sl, xr, nblk, acc);

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
}

// ---------------------------------------------------------------------------
// down.  A wave owns 16*NSUB output features (rows of W2).

template <int MS, int NSUB>
__global__ __launch_bounds__(kThreads) void k_down(
    const uint16_t* __restrict__ hin, const int32_t* __restrict__ offsets, int H, int I, int E,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, float* __restrict__ y,
    int ntile_n, int hi) {
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int r16 = lane & 15;
  const int g = lane >> 4;
  for (int idx = blockIdx.x;; idx += gridDim.x) {
  const int slot = idx / ntile_n;
  const int nt = idx - slot * ntile_n;
  Tile t;
  if (!find_tile(offsets, E, 16 * MS, slot, t, 1, hi)) return;
  const int n0 = (nt * kWaves + wave) * 16 * NSUB;
  if (n0 >= H) continue;

  const int nblk = I / 32;
  const size_t erow = size_t(t.e) * H;
  const uint8_t* wc[NSUB];
  const uint8_t* ws0[NSUB];
  const uint8_t* sl[NSUB];
  extern __shared__ uint8_t lds_scales[];
  uint8_t* my_lds = lds_scales + wave * NSUB * 16 * nblk;
#pragma unroll
  for (int a = 0; a < NSUB; ++a) {
    const int n0a = min(n0 + 16 * a, H - 16);
    wc[a] = codes + (erow + n0a + r16) * size_t(I / 2);
    ws0[a] = scales + (erow + n0a) * size_t(nblk);
    sl[a] = my_lds + a * 16 * nblk + r16 * nblk;
  }
  const uint16_t* xr[MS];          // rows past the tile's end re-read its last row
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int mi = 16 * m + r16;
    xr[m] = hin + size_t(t.row0 + min(mi, t.rows - 1)) * I;
  }
  f32x4 acc[NSUB][MS];
#pragma unroll
  for (int a = 0; a < NSUB; ++a)
#pragma unroll
    for (int m = 0; m < MS; ++m) acc[a][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  stream_k<NSUB, MS>(wc, ws0, my_lds, sl, xr, nblk, acc);

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

// workgroups launched: the tile-slot bound, capped at a few per CU.  After a
// dense pass (hi < INT_MAX) only experts below its row threshold are left,
// often none (a uniform prefill batch): one workgroup per CU then finds that
// out at a third of the cost of four, and walks the tiles there are
// grid-stride.
unsigned stream_grid(int64_t slots_times_n, int hi) {
  const int64_t cap = int64_t(hi == INT32_MAX ? 4 : 1) * device_cus();
  return unsigned(slots_times_n < cap ? slots_times_n : cap);
}

template <int MS>
hipError_t gate_up_ms(const uint16_t* x, const int32_t* sp, const int32_t* off, int T, int H,
                      int I, int E, int k, const uint8_t* c, const uint8_t* sc, uint16_t* h,
                      int hi, hipStream_t s) {
  constexpr int NSUB = kGuNsub;
  const int R = T * k;
  const int ntile_n = (I + kWaves * 16 * NSUB - 1) / (kWaves * 16 * NSUB);
  const unsigned grid = stream_grid(int64_t(tile_slots(R, E, 16 * MS)) * ntile_n, hi);
  // 8 H bytes of scales: above 64 KB (H > 8192) the kernel's LDS limit is
  // raised to the 128 KB that H = 16384 needs
  const size_t lds = size_t(kWaves) * 2 * NSUB * 16 * (H / 32);
  static std::atomic<bool> lds_set[kMaxDevices];
  if (lds > 65536) {
    const hipError_t e = lds_limit_once(reinterpret_cast<const void*>(&k_gate_up<MS, NSUB>),
                                        int(size_t(kWaves) * 2 * NSUB * 16 * (16384 / 32)),
                                        lds_set);
    if (e != hipSuccess) return e;
  }
  k_gate_up<MS, NSUB><<<dim3(grid), kThreads, lds, s>>>(x, sp, off, H, I, E, k, c, sc,
                                                                    h, ntile_n, hi);
  return hipGetLastError();
}

template <int MS>
hipError_t down_ms(const uint16_t* h, const int32_t* off, int T, int H, int I, int E, int k,
                   const uint8_t* c, const uint8_t* sc, float* y, int hi, hipStream_t s) {
  constexpr int NSUB = kDnNsub;
  const int R = T * k;
  const int ntile_n = (H + kWaves * 16 * NSUB - 1) / (kWaves * 16 * NSUB);
  const unsigned grid = stream_grid(int64_t(tile_slots(R, E, 16 * MS)) * ntile_n, hi);
  const size_t lds = size_t(kWaves) * NSUB * 16 * (I / 32);
  k_down<MS, NSUB><<<dim3(grid), kThreads, lds, s>>>(h, off, H, I, E, c, sc, y, ntile_n,
                                                               hi);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const uint16_t* x, const int32_t* sorted_pairs, const int32_t* offsets,
                          int T, int H, int I, int E, int k, const uint8_t* codes,
                          const uint8_t* scales, uint16_t* h, int hi, hipStream_t s) {
  switch (choose_ms(T * k, E)) {
    case 1:
      if (decode_supported(T, H, I, E, k))
        return launch_gate_up_decode(x, sorted_pairs, offsets, T, H, I, E, k, codes, scales, h, hi,
                                     s);
      return gate_up_ms<1>(x, sorted_pairs, offsets, T, H, I, E, k, codes, scales, h, hi, s);
    case 2: return gate_up_ms<2>(x, sorted_pairs, offsets, T, H, I, E, k, codes, scales, h, hi, s);
    default: return gate_up_ms<4>(x, sorted_pairs, offsets, T, H, I, E, k, codes, scales, h, hi, s);
  }
}

hipError_t launch_down(const uint16_t* h, const int32_t* offsets, int T, int H, int I, int E,
                       int k, const uint8_t* codes, const uint8_t* scales, float* y, int hi,
                       hipStream_t s) {
  switch (choose_ms(T * k, E)) {
    case 1:
      if (decode_supported(T, H, I, E, k))
        return launch_down_decode(h, offsets, T, H, I, E, k, codes, scales, y, hi, s);
      return down_ms<1>(h, offsets, T, H, I, E, k, codes, scales, y, hi, s);
    case 2: return down_ms<2>(h, offsets, T, H, I, E, k, codes, scales, y, hi, s);
    default: return down_ms<4>(h, offsets, T, H, I, E, k, codes, scales, y, hi, s);
  }
}

}  // namespace mxm

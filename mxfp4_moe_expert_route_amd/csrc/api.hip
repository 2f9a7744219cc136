// C ABI of libmxfp4moe: host-side argument checks, then kernel launches.
// Every check runs before anything is enqueued, and none of them touches the
// HIP runtime, so invalid calls return an error without a device.
#include "../../include/mxfp4moe.h"
#include "common.hpp"

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxH = 16384;
constexpr int kMaxI = 8192;
constexpr int kMaxRouterH = 1 << 20;     // size_t row offsets; int loop bounds
constexpr int kMaxVerifyL = 32;          // one lane of a wave per block position

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launched(hipError_t e) { return e == hipSuccess ? MXM_OK : MXM_ERR_LAUNCH; }

// Shared checks of the routing shape.
int check_route_shape(int T, int E, int k) {
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > kMaxK || k > E) return MXM_ERR_SHAPE;
  if (int64_t(T) * k > INT32_MAX) return MXM_ERR_SHAPE;
  return MXM_OK;
}

int check_ffn_shape(int T, int H, int I, int E, int k) {
  const int st = check_route_shape(T, E, k);
  if (st != MXM_OK) return st;
  if (H < 32 || I < 32 || H % 32 || I % 32) return MXM_ERR_SHAPE;
  // the streaming kernels stage every wave's scale rows in LDS: 8 H bytes
  // for gate/up (128 KB at H = 16384, the most a workgroup may hold) and 8 I
  // bytes for down
  if (H > kMaxH || I > kMaxI) return MXM_ERR_SHAPE;
  // weight element counts per expert must fit the kernels' size_t math and the
  // activation rows their int32 row indices
  if (int64_t(T) * k * int64_t(H > I ? H : I) > (int64_t(1) << 40)) return MXM_ERR_SHAPE;
  return MXM_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Null and alignment checks of the layer call's buffers.
int check_layer_pointers(const uint16_t* x_bf16, const float* logits, const uint8_t* w13_codes,
                         const uint8_t* w13_scales, const uint8_t* w2_codes,
                         const uint8_t* w2_scales, const int32_t* topk_ids, const float* topk_w,
                         const int32_t* counts, const int32_t* offsets,
                         const int32_t* sorted_pairs, const int32_t* pair_to_row,
                         const uint16_t* h_bf16, const float* y, const float* out) {
  if (!x_bf16 || !logits || !w13_codes || !w13_scales || !w2_codes || !w2_scales || !topk_ids ||
      !topk_w || !counts || !offsets || !sorted_pairs || !pair_to_row || !h_bf16 || !y || !out)
    return MXM_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w13_codes, 16) || !aligned(w2_codes, 16) ||
      !aligned(w13_scales, 16) || !aligned(w2_scales, 16) || !aligned(h_bf16, 16) ||
      !aligned(y, 16) || !aligned(out, 16) || !aligned(logits, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      !aligned(sorted_pairs, 4) || !aligned(pair_to_row, 4))
    return MXM_ERR_ALIGN;
  return MXM_OK;
}

// Scratch of moe_mxfp4_layer_noalloc: the grouping workspace (per-range
// expert histograms, then per-range bases) in a fixed device array, one copy
// per GPU, held until the process ends.  Host code uses the device address
// hipGetSymbolAddress returns for the current device, never the array's
// name (a host-side stand-in).
constexpr size_t kScratchBytes = size_t(1) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> scratch_ptr[mxm::kMaxDevices];

// This device's copy of `scratch` (looked up on the first call per device);
// nullptr when the address cannot be had.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= mxm::kMaxDevices) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

// Experts with many rows go to the LDS-tiled dense kernel, the rest to the
// streaming kernel.  Chosen from host-known sizes only: the dense pass is
// worth a launch when the mean rows per touched expert is at least 8 (so
// some experts may reach its row threshold).
bool use_dense(int T, int H, int I, int E, int k) {
  const int64_t R = int64_t(T) * k;
  const int64_t touched = R < E ? R : E;
  return mxm::dense_supported(T, H, I, E, k) && R >= 8 * touched;
}

}  // namespace

namespace mxm {

int device_cus() {
  static std::atomic<int> cus[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cache = dev >= 0 && dev < kMaxDevices;
  if (cache) {
    const int n = cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int v = 0;
  if (dev < 0 || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      v < 1)
    v = 256;
  if (cache) cus[dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t lds_limit_once(const void* fn, int bytes, std::atomic<bool>* done) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cache = dev >= 0 && dev < kMaxDevices;
  if (cache && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && cache) done[dev].store(true, std::memory_order_release);
  return e;
}

}  // namespace mxm

extern "C" {

int mxm_version(void) { return 100; }

const char* mxm_status_string(int status) {
  switch (status) {
    case MXM_OK: return "MXM_OK";
    case MXM_ERR_NULL: return "MXM_ERR_NULL: a required pointer is NULL";
    case MXM_ERR_SHAPE: return "MXM_ERR_SHAPE: a size is out of range";
    case MXM_ERR_DTYPE: return "MXM_ERR_DTYPE: unknown dtype code";
    case MXM_ERR_ALIGN: return "MXM_ERR_ALIGN: a pointer is misaligned";
    case MXM_ERR_LAUNCH: return "MXM_ERR_LAUNCH: a HIP kernel launch failed";
    case MXM_ERR_UNIMPLEMENTED: return "MXM_ERR_UNIMPLEMENTED";
    case MXM_ERR_WORKSPACE: return "MXM_ERR_WORKSPACE: workspace too small";
    case MXM_ERR_SCRATCH:
      return "MXM_ERR_SCRATCH: the call needs more scratch than the library's fixed 1 MiB "
             "device buffer holds";
    default: return "unknown mxfp4moe status";
  }
}

int mxfp4_pack(const void* x, int x_dtype, int64_t rows, int64_t K, uint8_t* codes,
               uint8_t* scales, void* stream) {
  if (x_dtype != MXM_F32 && x_dtype != MXM_BF16) return MXM_ERR_DTYPE;
  if (rows < 0 || K < 0 || K % 32) return MXM_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXM_OK;
  if (!x || !codes || !scales) return MXM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, 16)) return MXM_ERR_ALIGN;
  return launched(mxm::launch_pack(x, x_dtype, rows, K, codes, scales, as_stream(stream)));
}

int mxfp4_unpack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K, void* y,
                 int y_dtype, void* stream) {
  if (y_dtype != MXM_F32 && y_dtype != MXM_BF16) return MXM_ERR_DTYPE;
  if (rows < 0 || K < 0 || K % 32) return MXM_ERR_SHAPE;
  if (rows == 0 || K == 0) return MXM_OK;
  if (!codes || !scales || !y) return MXM_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(y, 16)) return MXM_ERR_ALIGN;
  return launched(mxm::launch_unpack(codes, scales, rows, K, y, y_dtype, as_stream(stream)));
}

int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                   void* stream) {
  const int st = check_route_shape(T, E, k);
  if (st != MXM_OK) return st;
  if (T == 0) return MXM_OK;
  if (!logits || !topk_ids || !topk_w) return MXM_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return MXM_ERR_ALIGN;
  return launched(mxm::launch_route_topk(logits, T, E, k, topk_ids, topk_w, as_stream(stream)));
}

int moe_router_topk(const uint16_t* x_bf16, const float* w_router, const float* bias, int T,
                    int H, int E, int k, float* logits, int32_t* topk_ids, float* topk_w,
                    void* stream) {
  const int st = check_route_shape(T, E, k);
  if (st != MXM_OK) return st;
  if (H < 4 || H % 4 || H > kMaxRouterH) return MXM_ERR_SHAPE;
  if (T == 0) return MXM_OK;
  if (!x_bf16 || !w_router || !logits || !topk_ids || !topk_w) return MXM_ERR_NULL;
  if (!aligned(x_bf16, 8) || !aligned(w_router, 16) || !aligned(logits, 4) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 4) || (bias && !aligned(bias, 4)))
    return MXM_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  if (mxm::launch_router_logits(x_bf16, w_router, bias, T, H, E, logits, s) != hipSuccess)
    return MXM_ERR_LAUNCH;
  return launched(mxm::launch_route_topk(logits, T, E, k, topk_ids, topk_w, s));
}

size_t dflash_verify_workspace_bytes(int B, int L, int V) {
  (void)V;
  if (B < 0 || L < 1 || L > kMaxVerifyL) return 0;
  return mxm::verify_workspace_bytes(B, L);
}

int dflash_verify_accept(const float* target_logits, const float* draft_probs,
                         const int32_t* draft_tokens, const float* uniforms, int B, int L, int V,
                         int32_t* accept_len, int32_t* next_token, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (B < 0 || L < 1 || L > kMaxVerifyL || V < 4 || V % 4) return MXM_ERR_SHAPE;
  if (int64_t(B) * (L + 1) * V > (int64_t(1) << 40) || int64_t(B) * (L + 1) * 8 > INT32_MAX)
    return MXM_ERR_SHAPE;
  if (B == 0) return MXM_OK;
  if (workspace_bytes < dflash_verify_workspace_bytes(B, L, V)) return MXM_ERR_WORKSPACE;
  if (!target_logits || !draft_probs || !draft_tokens || !uniforms || !accept_len ||
      !next_token || !workspace)
    return MXM_ERR_NULL;
  if (!aligned(target_logits, 16) || !aligned(draft_probs, 16) || !aligned(draft_tokens, 4) ||
      !aligned(uniforms, 4) || !aligned(accept_len, 4) || !aligned(next_token, 4) ||
      !aligned(workspace, 8))
    return MXM_ERR_ALIGN;
  return launched(mxm::launch_verify(target_logits, draft_probs, draft_tokens, uniforms, B, L, V,
                                     accept_len, next_token, workspace, as_stream(stream)));
}

size_t moe_permute_workspace_bytes(int T, int E, int k) {
  if (check_route_shape(T, E, k) != MXM_OK) return 0;
  return mxm::permute_workspace_bytes(T, E, k);
}

int moe_permute(const int32_t* topk_ids, int T, int E, int k, int32_t* counts, int32_t* offsets,
                int32_t* sorted_pairs, int32_t* pair_to_row, void* workspace,
                size_t workspace_bytes, void* stream) {
  const int st = check_route_shape(T, E, k);
  if (st != MXM_OK) return st;
  if (workspace_bytes < moe_permute_workspace_bytes(T, E, k)) return MXM_ERR_WORKSPACE;
  if (T == 0) return MXM_OK;
  if (!topk_ids || !counts || !offsets || !sorted_pairs || !pair_to_row) return MXM_ERR_NULL;
  if (moe_permute_workspace_bytes(T, E, k) > 0 && !workspace) return MXM_ERR_NULL;
  if (!aligned(topk_ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      !aligned(sorted_pairs, 4) || !aligned(pair_to_row, 4) || !aligned(workspace, 4))
    return MXM_ERR_ALIGN;
  return launched(mxm::launch_permute(topk_ids, T, E, k, counts, offsets, sorted_pairs,
                                      pair_to_row, workspace, as_stream(stream)));
}

int moe_route_permute(const float* logits, int T, int E, int k, int32_t* topk_ids,
                      float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                      int32_t* pair_to_row, void* workspace, size_t workspace_bytes,
                      void* stream) {
  const int st = check_route_shape(T, E, k);
  if (st != MXM_OK) return st;
  if (workspace_bytes < moe_permute_workspace_bytes(T, E, k)) return MXM_ERR_WORKSPACE;
  if (T == 0) return MXM_OK;
  if (!logits || !topk_ids || !topk_w || !counts || !offsets || !sorted_pairs || !pair_to_row)
    return MXM_ERR_NULL;
  if (moe_permute_workspace_bytes(T, E, k) > 0 && !workspace) return MXM_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) ||
      !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_pairs, 4) ||
      !aligned(pair_to_row, 4) || !aligned(workspace, 4))
    return MXM_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  if (mxm::route_permute_fusable(T, E, k))
    return launched(mxm::launch_route_permute(logits, T, E, k, topk_ids, topk_w, counts, offsets,
                                              sorted_pairs, pair_to_row, s));
  if (mxm::launch_route_topk(logits, T, E, k, topk_ids, topk_w, s) != hipSuccess)
    return MXM_ERR_LAUNCH;
  return launched(mxm::launch_permute(topk_ids, T, E, k, counts, offsets, sorted_pairs,
                                      pair_to_row, workspace, s));
}

int moe_mxfp4_gate_up_swiglu(const uint16_t* x_bf16, const int32_t* sorted_pairs,
                             const int32_t* offsets, int T, int H, int I, int E, int k,
                             const uint8_t* w13_codes, const uint8_t* w13_scales,
                             uint16_t* h_bf16, void* stream) {
  const int st = check_ffn_shape(T, H, I, E, k);
  if (st != MXM_OK) return st;
  if (T == 0) return MXM_OK;
  if (!x_bf16 || !sorted_pairs || !offsets || !w13_codes || !w13_scales || !h_bf16)
    return MXM_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w13_codes, 16) || !aligned(w13_scales, 16) ||
      !aligned(h_bf16, 8) || !aligned(sorted_pairs, 4) || !aligned(offsets, 4))
    return MXM_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  int hi = INT32_MAX;
  if (use_dense(T, H, I, E, k)) {
    if (mxm::launch_gate_up_dense(x_bf16, sorted_pairs, offsets, T, H, I, E, k, w13_codes,
                                  w13_scales, h_bf16, s) != hipSuccess)
      return MXM_ERR_LAUNCH;
    hi = mxm::dense_min_rows();
  }
  return launched(mxm::launch_gate_up(x_bf16, sorted_pairs, offsets, T, H, I, E, k, w13_codes,
                                      w13_scales, h_bf16, hi, s));
}

int moe_mxfp4_down(const uint16_t* h_bf16, const int32_t* offsets, int T, int H, int I, int E,
                   int k, const uint8_t* w2_codes, const uint8_t* w2_scales, float* y,
                   void* stream) {
  const int st = check_ffn_shape(T, H, I, E, k);
  if (st != MXM_OK) return st;
  if (T == 0) return MXM_OK;
  if (!h_bf16 || !offsets || !w2_codes || !w2_scales || !y) return MXM_ERR_NULL;
  if (!aligned(h_bf16, 16) || !aligned(w2_codes, 16) || !aligned(w2_scales, 16) ||
      !aligned(y, 16) || !aligned(offsets, 4))
    return MXM_ERR_ALIGN;
  hipStream_t s = as_stream(stream);
  int hi = INT32_MAX;
  if (use_dense(T, H, I, E, k)) {
    if (mxm::launch_down_dense(h_bf16, offsets, T, H, I, E, k, w2_codes, w2_scales, y, s) !=
        hipSuccess)
      return MXM_ERR_LAUNCH;
    hi = mxm::dense_min_rows();
  }
  return launched(mxm::launch_down(h_bf16, offsets, T, H, I, E, k, w2_codes, w2_scales, y, hi, s));
}

int moe_combine(const float* y, const float* topk_w, const int32_t* pair_to_row, int T, int H,
                int k, float* out, void* stream) {
  if (T < 0 || k < 1 || k > kMaxK || H < 32 || H % 32) return MXM_ERR_SHAPE;
  if (int64_t(T) * k > INT32_MAX) return MXM_ERR_SHAPE;
  if (T == 0) return MXM_OK;
  if (!y || !topk_w || !pair_to_row || !out) return MXM_ERR_NULL;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(topk_w, 4) || !aligned(pair_to_row, 4))
    return MXM_ERR_ALIGN;
  return launched(mxm::launch_combine(y, topk_w, pair_to_row, T, H, k, out, as_stream(stream)));
}

int moe_mxfp4_layer(const uint16_t* x_bf16, const float* logits, int T, int H, int I, int E,
                    int k, const uint8_t* w13_codes, const uint8_t* w13_scales,
                    const uint8_t* w2_codes, const uint8_t* w2_scales, int32_t* topk_ids,
                    float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                    int32_t* pair_to_row, uint16_t* h_bf16, float* y, float* out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  // check everything before enqueuing anything
  int st = check_ffn_shape(T, H, I, E, k);
  if (st != MXM_OK) return st;
  if (workspace_bytes < moe_permute_workspace_bytes(T, E, k)) return MXM_ERR_WORKSPACE;
  if (T == 0) return MXM_OK;
  if ((st = check_layer_pointers(x_bf16, logits, w13_codes, w13_scales, w2_codes, w2_scales,
                                 topk_ids, topk_w, counts, offsets, sorted_pairs, pair_to_row,
                                 h_bf16, y, out)) != MXM_OK)
    return st;
  if ((st = moe_route_permute(logits, T, E, k, topk_ids, topk_w, counts, offsets, sorted_pairs,
                              pair_to_row, workspace, workspace_bytes, stream)) != MXM_OK)
    return st;
  if ((st = moe_mxfp4_gate_up_swiglu(x_bf16, sorted_pairs, offsets, T, H, I, E, k, w13_codes,
                                     w13_scales, h_bf16, stream)) != MXM_OK)
    return st;
  if ((st = moe_mxfp4_down(h_bf16, offsets, T, H, I, E, k, w2_codes, w2_scales, y, stream)) !=
      MXM_OK)
    return st;
  return moe_combine(y, topk_w, pair_to_row, T, H, k, out, stream);
}

size_t moe_mxfp4_decode_layer_workspace_bytes(int T, int H, int I, int E, int k) {
  if (check_ffn_shape(T, H, I, E, k) != MXM_OK || !mxm::decode_layer_supported(T, H, I, E, k))
    return 0;
  return mxm::decode_layer_workspace_bytes();
}

int moe_mxfp4_decode_layer(const uint16_t* x_bf16, const float* logits, int T, int H, int I,
                           int E, int k, const uint8_t* w13_codes, const uint8_t* w13_scales,
                           const uint8_t* w2_codes, const uint8_t* w2_scales, int32_t* topk_ids,
                           float* topk_w, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_pairs, int32_t* pair_to_row, uint16_t* h_bf16,
                           float* y, float* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = check_ffn_shape(T, H, I, E, k);
  if (st != MXM_OK) return st;
  if (T == 0) return MXM_OK;
  if (!mxm::decode_layer_supported(T, H, I, E, k)) return MXM_ERR_UNIMPLEMENTED;
  if (workspace_bytes < mxm::decode_layer_workspace_bytes()) return MXM_ERR_WORKSPACE;
  if ((st = check_layer_pointers(x_bf16, logits, w13_codes, w13_scales, w2_codes, w2_scales,
                                 topk_ids, topk_w, counts, offsets, sorted_pairs, pair_to_row,
                                 h_bf16, y, out)) != MXM_OK)
    return st;
  if (!workspace) return MXM_ERR_NULL;
  if (!aligned(workspace, 16)) return MXM_ERR_ALIGN;
  return launched(mxm::launch_decode_layer(x_bf16, logits, T, H, I, E, k, w13_codes, w13_scales,
                                           w2_codes, w2_scales, topk_ids, topk_w, counts, offsets,
                                           sorted_pairs, pair_to_row, h_bf16, y, out, workspace,
                                           as_stream(stream)));
}

int moe_mxfp4_layer_noalloc(const uint16_t* x_bf16, const float* logits, int T, int H, int I,
                            int E, int k, const uint8_t* w13_codes, const uint8_t* w13_scales,
                            const uint8_t* w2_codes, const uint8_t* w2_scales, int32_t* topk_ids,
                            float* topk_w, int32_t* counts, int32_t* offsets,
                            int32_t* sorted_pairs, int32_t* pair_to_row, uint16_t* h_bf16,
                            float* y, float* out, void* stream) {
  int st = check_ffn_shape(T, H, I, E, k);
  if (st != MXM_OK) return st;
  const size_t need = moe_permute_workspace_bytes(T, E, k);
  if (need > kScratchBytes) return MXM_ERR_SCRATCH;
  if (T == 0) return MXM_OK;
  if ((st = check_layer_pointers(x_bf16, logits, w13_codes, w13_scales, w2_codes, w2_scales,
                                 topk_ids, topk_w, counts, offsets, sorted_pairs, pair_to_row,
                                 h_bf16, y, out)) != MXM_OK)
    return st;
  void* ws = nullptr;
  if (need > 0 && !(ws = scratch_on_current_device())) return MXM_ERR_LAUNCH;
  // the grouping kernels overwrite every workspace word they later read, so
  // the previous call's contents need no clearing
  return moe_mxfp4_layer(x_bf16, logits, T, H, I, E, k, w13_codes, w13_scales, w2_codes,
                         w2_scales, topk_ids, topk_w, counts, offsets, sorted_pairs, pair_to_row,
                         h_bf16, y, out, ws, need, stream);
}

int mxm_stream_xor(const void* src, int64_t bytes, int nontemporal, uint32_t* result,
                   void* stream) {
  if (bytes < 0 || bytes % 16) return MXM_ERR_SHAPE;
  if (bytes == 0) return MXM_OK;
  if (!src || !result) return MXM_ERR_NULL;
  if (!aligned(src, 16) || !aligned(result, 4)) return MXM_ERR_ALIGN;
  return launched(mxm::launch_stream_xor(src, bytes, nontemporal, result, as_stream(stream)));
}

}  // extern "C"

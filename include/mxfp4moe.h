/*
 * mxfp4moe.h — C ABI of the MXFP4 Mixture-of-Experts expert layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer: each token's router logits pick k of E experts; each chosen
 * expert is a SwiGLU FFN whose weights are stored in MXFP4 (4-bit E2M1
 * elements, one E8M0 power-of-two scale per 32 consecutive elements along the
 * reduction axis); activations are bf16, accumulation fp32; the k expert
 * outputs are mixed with the routing weights.  The pages this follows
 * ("MiMo-V2.5-Pro-FP4-DFlash" model card, §1 Introduction, §2 "FP4
 * Quantization", §3 DFlash, §4 "Model Summary"; nxbn.cn article
 * "MiMo-V2.5-Pro-FP4-DFlash万亿参数大模型推理效率的终极突破", sub-sections
 * "量化策略的智能选择" and "架构设计与配置详解") fix MXFP4 with block 32 for
 * the experts only, 384 experts with 8 active per token, hidden size 6144,
 * and verification of an 8-token draft block per sequence per step.  The
 * encodings are those of the OCP MX v1.0 specification.  The SwiGLU form,
 * the softmax-renormalised routing rule, the bit layout and the rounding of
 * the intermediate h to bf16 are readings of what the pages leave open; they
 * are stated at each call below.
 *
 * Conventions for every call
 *   - All array arguments are DEVICE pointers, allocated and owned by the
 *     caller.  The library never allocates or frees device memory and keeps
 *     no data between calls (it caches, per device, only the CU count and
 *     whether a kernel's LDS limit has been raised); calls are thread-safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Each call only enqueues kernels on it and returns; there is no host
 *     synchronisation.  Results are valid once the stream reaches them.
 *   - Errors are returned as a negative status (MXM_ERR_*).  Argument checks
 *     are done on the host before anything is enqueued; on an error nothing
 *     is launched and no output is touched.  MXM_ERR_LAUNCH reports a HIP
 *     launch failure after the checks passed.
 *   - An empty problem (T == 0, rows == 0) is a no-op that returns MXM_OK;
 *     its pointers may then be NULL.
 *   - Integer indices are int32 (T*k < 2^31).  H and I must be multiples of
 *     32 (no partial MX blocks); the expert contractions take H <= 16384 and
 *     I <= 8192.  1 <= k <= min(E, 32), E <= 1024.
 *   - Pointer alignment: codes, expert-weight scales, x (pack input), y
 *     (unpack output), x_bf16, h_bf16, y and out 16 bytes; everything else 4.
 *     Rows are densely packed (the leading stride is the row length).
 */
#ifndef MXFP4MOE_H
#define MXFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mxm_status {
  MXM_OK = 0,
  MXM_ERR_NULL = -1,          /* a required pointer is NULL */
  MXM_ERR_SHAPE = -2,         /* a size is out of range (K%32, k>E, E>1024, ...) */
  MXM_ERR_DTYPE = -3,         /* unknown dtype code */
  MXM_ERR_ALIGN = -4,         /* a pointer is not aligned as stated above */
  MXM_ERR_LAUNCH = -5,        /* a kernel launch failed (HIP error) */
  MXM_ERR_UNIMPLEMENTED = -6, /* reserved */
  MXM_ERR_WORKSPACE = -7,     /* workspace smaller than the call needs */
  MXM_ERR_SCRATCH = -8        /* moe_mxfp4_layer_noalloc: sizes need more than its fixed scratch */
};

enum mxm_dtype { MXM_F32 = 0, MXM_BF16 = 1 };

/* Library version as 10000*major + 100*minor + patch. */
int mxm_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* mxm_status_string(int status);

/*
 * mxfp4_pack — quantise a row-major matrix to MXFP4.
 *   x       [rows, K] f32 or bf16 (x_dtype = MXM_F32 / MXM_BF16), read only
 *   codes   [rows, K/2] uint8, written: byte j of a row holds element 2j in
 *           bits 3..0 and element 2j+1 in bits 7..4 (reading: the pages do
 *           not give the nibble order)
 *   scales  [rows, K/32] uint8 E8M0, written
 * Conversion per 32-element block (OCP MX v1.0; the pages name MXFP4 with
 * block 32 — model card §2 — and give no rounding rule): scale exponent
 * e = clamp(floor(log2(max|x|)) - 2 + 127, 0, 254); each x*2^(127-e) is
 * rounded to the nearest E2M1 value, ties to the even code, saturating at 6;
 * the code's sign bit is x's sign bit.  An all-zero block gets e = 0; a block
 * holding NaN or Inf gets e = 0xFF and zero codes.  Bit-exact and
 * deterministic.  Requires K % 32 == 0; rows, K >= 0.
 */
int mxfp4_pack(const void* x, int x_dtype, int64_t rows, int64_t K,
               uint8_t* codes, uint8_t* scales, void* stream);

/*
 * mxfp4_unpack — dequantise MXFP4 to f32 or bf16.
 *   codes [rows, K/2], scales [rows, K/32] as written by mxfp4_pack
 *   y     [rows, K] f32 or bf16 (y_dtype), written
 * y = E2M1(code) * 2^(e-127), computed exactly and rounded to the output type
 * (exact for every finite result, subnormals included; f32 overflows to Inf
 * only for e >= 253).  A scale byte 0xFF gives a quiet NaN for the block.
 * The pages store the experts in MXFP4 with block size 32
 * ("MiMo-V2.5-Pro-FP4-DFlash" model card, §2 "FP4 Quantization"; nxbn.cn
 * article, "量化策略的智能选择": store_dtype mxfp4, mxfp4_block_size 32); the
 * element and scale encodings are OCP MX v1.0's E2M1 and E8M0 (reading).
 */
int mxfp4_unpack(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                 int64_t K, void* y, int y_dtype, void* stream);

/*
 * moe_route_topk — choose k experts per token.
 *   logits  [T, E] f32, read (the router projection is upstream of this call)
 *   topk_ids[T, k] int32, written: experts by descending logit, the lower
 *           index first on equal logits; -0.0 equals +0.0; NaN ranks as -inf
 *   topk_w  [T, k] f32, written: softmax over all E experts renormalised over
 *           the k chosen, i.e. w_j = exp(l_j - l_1) / sum_j' exp(l_j' - l_1)
 * The pages give 384 experts and 8 active per token (nxbn.cn article,
 * "架构设计与配置详解") and no scoring rule; the rule above is the reading.
 * Ids are deterministic and bit-exact; a row with a +Inf logit or with no
 * finite logit has undefined weights.
 */
int moe_route_topk(const float* logits, int T, int E, int k,
                   int32_t* topk_ids, float* topk_w, void* stream);

/*
 * moe_router_topk — router projection, then moe_route_topk on its result.
 *   x_bf16   [T, H] bf16, read; 8-byte aligned
 *   w_router [E, H] f32, read (row e: expert e's router weights); 16-byte
 *            aligned
 *   bias     [E] f32 added to every token's logits, read; may be NULL
 *   logits   [T, E] f32, written: x_t . w_e accumulated in fp32 (the products
 *            of bf16 and fp32 values rounded by fused multiply-adds), plus
 *            bias_e
 *   topk_ids, topk_w: as moe_route_topk, computed from the written logits
 * The pages route each token to 8 of 384 experts (nxbn.cn article,
 * "架构设计与配置详解") with a hidden size of 6144 ("MiMo-V2.5-Pro-FP4-DFlash"
 * model card, §4 "Model Summary") and give no router form; a linear
 * projection of the bf16 hidden state with fp32 weights is the reading.
 * H must be a multiple of 4 (up to 2^20).  Ids and weights are exactly what
 * moe_route_topk gives for the written logits; the logits are deterministic
 * run to run (fixed summation order) and lie within fp32 accumulation error
 * of the exact sum.
 */
int moe_router_topk(const uint16_t* x_bf16, const float* w_router, const float* bias,
                    int T, int H, int E, int k, float* logits, int32_t* topk_ids,
                    float* topk_w, void* stream);

/* Workspace dflash_verify_accept needs (0 for invalid sizes). */
size_t dflash_verify_workspace_bytes(int B, int L, int V);

/*
 * dflash_verify_accept — rejection-sampling verification of B drafted blocks
 * of L tokens over a vocabulary of V.
 *   target_logits [B, L+1, V] f32, read: the backbone's logits at the L block
 *                 positions and the one after; 16-byte aligned
 *   draft_probs   [B, L, V] f32, read: the drafter's probabilities; 16-byte
 *                 aligned
 *   draft_tokens  [B, L] int32, read: the drafted tokens
 *   uniforms      [B, L+1] f32 in [0, 1), read: one per position, the last
 *                 for the draw
 *   accept_len    [B] int32, written: n, the leading positions accepted
 *   next_token    [B] int32, written: the token after the n accepted ones
 *   workspace     dflash_verify_workspace_bytes(B, L, V) bytes, 8-byte aligned
 * The pages verify a whole drafted block in one backbone step with
 * rejection sampling keeping the output lossless, blocks capped at 8
 * ("MiMo-V2.5-Pro-FP4-DFlash" model card, §3 "Block-Diffusion Speculative
 * Decoding (DFlash)").  The rule is the reading: with p_i = softmax of the
 * logits (temperature 1) and q_i the drafter's probabilities, position i is
 * accepted when u_i * q_i(d_i) < p_i(d_i); n counts the leading accepted
 * positions; the next token is drawn with u_L from max(0, p_n - q_n) when
 * n < L (from p_n if that is all zero) and from p_L when n = L, by inverse
 * CDF in vocabulary order.  A drafted token outside [0, V) is rejected.
 * 1 <= L <= 32, V a multiple of 4; a row with no finite logit is outside
 * the contract.  Computed in fp32 in fixed orders (deterministic); decisions
 * within fp32 rounding of a threshold may differ from exact arithmetic.
 */
int dflash_verify_accept(const float* target_logits, const float* draft_probs,
                         const int32_t* draft_tokens, const float* uniforms, int B, int L,
                         int V, int32_t* accept_len, int32_t* next_token, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Workspace moe_permute (and moe_route_permute, moe_mxfp4_layer) needs for
 * these sizes: 0 up to 8192 pairs (T*k), above that 4*E bytes per range of
 * 1024 pairs (at most 1024 ranges): per-range histograms, then per-range
 * bases.  0 for invalid sizes. */
size_t moe_permute_workspace_bytes(int T, int E, int k);

/*
 * moe_permute — group token-expert pairs by expert.
 *   topk_ids     [T, k] int32, read; each in [0, E)
 *   counts       [E]   int32, written: pairs routed to each expert
 *   offsets      [E+1] int32, written: exclusive prefix sum of counts
 *   sorted_pairs [T*k] int32, written: pair ids p = t*k + j, expert segments
 *                in expert order, ascending p within a segment
 *   pair_to_row  [T*k] int32, written: inverse of sorted_pairs
 *   workspace    device scratch of moe_permute_workspace_bytes(T, E, k)
 *                bytes, 4-byte aligned (may be NULL when that is 0); its
 *                contents need no initialisation and are overwritten
 * Bookkeeping the grouped expert contractions need; not on the pages.
 * Bit-exact and deterministic.  A pair whose id is outside [0, E) is
 * dropped: it is not counted, its pair_to_row entry is -1 and offsets[E]
 * then falls short of T*k.
 */
int moe_permute(const int32_t* topk_ids, int T, int E, int k,
                int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                int32_t* pair_to_row, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * moe_route_permute — moe_route_topk followed by moe_permute, in one call.
 *   arguments as those two calls (topk_ids and topk_w are written, then read)
 * Results are bit-identical to the two calls.  For T <= 16 (and E small
 * enough that the grouping tables fit 64 KB of LDS) both steps run in one
 * workgroup, the ids passing through LDS: one launch and one round trip to
 * memory fewer, which is most of their cost at decode sizes.  Errors as the
 * two calls; nothing is enqueued on a shape, null-pointer or alignment error.
 */
int moe_route_permute(const float* logits, int T, int E, int k, int32_t* topk_ids,
                      float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                      int32_t* pair_to_row, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * moe_mxfp4_gate_up_swiglu — first half of every chosen expert's FFN.
 *   x_bf16       [T, H] bf16 activations, read
 *   sorted_pairs [T*k], offsets [E+1] from moe_permute, read
 *   w13_codes    [E, 2I, H/2] uint8, w13_scales [E, 2I, H/32] uint8: per
 *                expert, rows 0..I-1 are the gate projection, rows I..2I-1
 *                the up projection (reading), MX blocks along H
 *   h_bf16       [T*k, I] bf16, written in sorted order: row r belongs to
 *                pair sorted_pairs[r] and its expert's segment
 * For row r of expert e with token t = sorted_pairs[r] / k:
 *   g = W_gate,e x_t, u = W_up,e x_t (fp32 accumulation),
 *   h_r = bf16_rne(silu(g) * u), silu(g) = g / (1 + exp(-g)).
 * The pages fix MXFP4 experts with block 32 and higher-precision activations
 * ("MiMo-V2.5-Pro-FP4-DFlash" model card, §2 "FP4 Quantization"; bf16 from
 * §5 "Deployment", --dtype bfloat16) and 384 experts with 8 active per token
 * (nxbn.cn article, "架构设计与配置详解"); the SwiGLU form without biases and
 * the gate-then-up row order are readings (the pages do not describe the
 * expert FFN).
 * Scale bytes must lie in 1..254 (2^-126 .. 2^127).  Byte 0 (2^-127, below
 * the normal fp32 range) is outside the contract: the kernels take it as
 * zero, which differs from mxfp4_unpack by at most 6*2^-127 per weight; byte
 * 255 (NaN) is outside it too.
 */
int moe_mxfp4_gate_up_swiglu(const uint16_t* x_bf16, const int32_t* sorted_pairs,
                             const int32_t* offsets, int T, int H, int I, int E,
                             int k, const uint8_t* w13_codes,
                             const uint8_t* w13_scales, uint16_t* h_bf16,
                             void* stream);

/*
 * moe_mxfp4_down — second half of every chosen expert's FFN.
 *   h_bf16     [T*k, I] bf16 from moe_mxfp4_gate_up_swiglu, read
 *   offsets    [E+1] from moe_permute, read
 *   w2_codes   [E, H, I/2] uint8, w2_scales [E, H, I/32] uint8, blocks along I
 *   y          [T*k, H] f32, written in sorted order: y_r = W_down,e h_r
 *              (fp32 accumulation of the bf16 h and the exactly dequantised
 *              weights)
 * Same sources and readings as moe_mxfp4_gate_up_swiglu (model card §2 for
 * the MXFP4 format and block size; the down projection completes the
 * reading's SwiGLU FFN); scale bytes in 1..254 as there.
 */
int moe_mxfp4_down(const uint16_t* h_bf16, const int32_t* offsets, int T, int H,
                   int I, int E, int k, const uint8_t* w2_codes,
                   const uint8_t* w2_scales, float* y, void* stream);

/*
 * moe_combine — mix each token's k expert outputs.
 *   y           [T*k, H] f32 from moe_mxfp4_down, read
 *   topk_w      [T, k] f32 from moe_route_topk, read
 *   pair_to_row [T*k] from moe_permute, read
 *   out         [T, H] f32, written: out_t = sum_{j=0..k-1} w_tj * y[row(t,j)],
 *               summed in slot order j (deterministic); a dropped pair
 *               (pair_to_row < 0) contributes nothing
 * Not on the pages: they name the routed experts (8 of 384, nxbn.cn
 * article, "架构设计与配置详解") but not how their outputs are mixed.  The
 * reading is the routing-weighted sum with the weights of moe_route_topk, in
 * fp32, with no shared expert and no routed scaling factor.
 */
int moe_combine(const float* y, const float* topk_w, const int32_t* pair_to_row,
                int T, int H, int k, float* out, void* stream);

/*
 * moe_mxfp4_layer — the whole layer: enqueues moe_route_permute (which
 * runs routing and grouping as one fused launch for T <= 16, else as
 * moe_route_topk then moe_permute), moe_mxfp4_gate_up_swiglu,
 * moe_mxfp4_down and moe_combine on `stream`, with the caller's intermediate
 * buffers (topk_ids [T,k], topk_w [T,k], counts [E], offsets [E+1],
 * sorted_pairs [T*k], pair_to_row [T*k], h [T*k, I] bf16, y [T*k, H] f32)
 * and grouping workspace (moe_permute_workspace_bytes).  Results are those of
 * the separate calls, bit for bit.  Sources and readings: those of each call.
 */
int moe_mxfp4_layer(const uint16_t* x_bf16, const float* logits, int T, int H,
                    int I, int E, int k, const uint8_t* w13_codes,
                    const uint8_t* w13_scales, const uint8_t* w2_codes,
                    const uint8_t* w2_scales, int32_t* topk_ids, float* topk_w,
                    int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                    int32_t* pair_to_row, uint16_t* h_bf16, float* y, float* out,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace moe_mxfp4_decode_layer needs for these sizes (0 when the
 * persistent kernel does not take them). */
size_t moe_mxfp4_decode_layer_workspace_bytes(int T, int H, int I, int E, int k);

/*
 * moe_mxfp4_decode_layer — the whole layer for a verify-sized batch as ONE
 * persistent kernel: routing, grouping, gate/up + SwiGLU, down and combine.
 *   arguments and results as moe_mxfp4_layer (results equal bit for bit),
 *   except the workspace:
 *   workspace  moe_mxfp4_decode_layer_workspace_bytes(...) bytes, 16-byte
 *              aligned, ZERO-FILLED by the caller before its first use; every
 *              call leaves it zero-filled for the next one, except 32-bit word
 *              2, which becomes nonzero (and stays so) if one of the kernel's
 *              bounded waits gave up, in which case the call's outputs are not
 *              valid.  Calls sharing a workspace must not overlap.
 * Taken shapes: 1 <= T <= 16, T*k <= 512, H and I multiples of 2048 up to
 * 8192, E <= 1024; other shapes return MXM_ERR_UNIMPLEMENTED (use
 * moe_mxfp4_layer).  The pages credit the decode speed of the serving
 * runtime to a persistent engine kernel that removes the gaps at operator
 * boundaries ("Xiaomi MiMo-V2.5-Pro-UltraSpeed" release notes, "TileRT
 * 執行模型", item 1); the verify block of 8 tokens per sequence is the
 * model card's §3 DFlash.  One workgroup per CU; each routes every token
 * itself, takes gate/up units from a queue in tile order, then down units
 * from a second queue once their tile's gate/up units are in, and the
 * workgroup that completes a column block combines it.  Every wait is for
 * units already claimed by running workgroups that never wait, so the grid
 * need not be resident all at once.  Errors as moe_mxfp4_layer.
 */
int moe_mxfp4_decode_layer(const uint16_t* x_bf16, const float* logits, int T, int H,
                           int I, int E, int k, const uint8_t* w13_codes,
                           const uint8_t* w13_scales, const uint8_t* w2_codes,
                           const uint8_t* w2_scales, int32_t* topk_ids, float* topk_w,
                           int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                           int32_t* pair_to_row, uint16_t* h_bf16, float* y, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_mxfp4_layer_noalloc — moe_mxfp4_layer for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and results.
 *   The grouping workspace (needed above 8192 token-expert pairs, see
 *   moe_permute_workspace_bytes) lives in a fixed 1 MiB device array of the
 *   library, one per GPU, held until the process ends; its address is looked
 *   up on the first call on each device.  Sizes whose workspace exceeds
 *   1 MiB return MXM_ERR_SCRATCH with nothing enqueued (E = 384 takes up to
 *   682 ranges of 1024 pairs, i.e. T*k up to 698,368).  The call allocates
 *   and frees nothing.  Every call on one GPU shares that array: calls that
 *   overlap on one GPU (two streams, or two host threads) race and must be
 *   ordered by the caller.  Inputs, outputs and intermediates are the
 *   caller's, as for moe_mxfp4_layer.
 */
int moe_mxfp4_layer_noalloc(const uint16_t* x_bf16, const float* logits, int T, int H,
                            int I, int E, int k, const uint8_t* w13_codes,
                            const uint8_t* w13_scales, const uint8_t* w2_codes,
                            const uint8_t* w2_scales, int32_t* topk_ids, float* topk_w,
                            int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                            int32_t* pair_to_row, uint16_t* h_bf16, float* y, float* out,
                            void* stream);

/*
 * mxm_stream_xor — measurement aid, not a step of the layer: a plain
 * streaming read of `bytes` bytes at `src` (16-byte aligned, bytes % 16 == 0)
 * that XORs every 32-bit word into *result (4-byte aligned; the caller sets
 * it beforehand, the call XORs into it).  The rate it reaches is the HBM read
 * ceiling the weight-streaming contractions are compared with; nontemporal
 * != 0 issues the loads with the non-temporal hint.
 */
int mxm_stream_xor(const void* src, int64_t bytes, int nontemporal, uint32_t* result,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4MOE_H */

/*
 * beam_moe.h -- C ABI of one Beam sparse-MoE layer forward on an MI355X (gfx950).
 *
 * The layer (Transformers "Beam" model page, Overview: sparse MoE item and the
 * FP32 numerics note; archdb "Beam-1.0-501B-A23B" fact sheet, MoE rows;
 * news.hamidun.com article on Beam, section on where it saves and where it pays
 * in memory):
 *   z = x . Wr (FP32), s = sigmoid(z), b = s + bias;
 *   group score = sum of the two largest b in each group of E/n_group experts;
 *   keep the topk_group best groups, then the top_k experts by b inside them;
 *   w_j = routed_scaling_factor * s_j / sum_j s_j   (plain S * s_j if norm_topk_prob = 0);
 *   y = sum_j w_j * Wd_e . bf16(silu(Wg_e . x) * (Wu_e . x)),   e = chosen expert j.
 * With the pre-MLP sandwich norm fused in (norm_w != NULL), x = bf16(RMSNorm(h) * norm_w)
 * first (Transformers "Beam" page, Overview: sandwich norms; BeamConfig: rms_norm_eps).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are caller-owned DEVICE memory, row-major, 16-byte aligned.
 *     bf16 tensors are raw bfloat16 bit patterns (uint16). The library never
 *     allocates, frees or synchronises; it keeps no global state and is re-entrant
 *     when callers use distinct workspaces.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every launch is queued
 *     on it; results are ready when that stream reaches the point after the call.
 *   - Outputs are fully overwritten, never accumulated into.
 *   - Arguments are validated on the host before anything is launched; a non-OK
 *     status means nothing was launched (except BEAM_MOE_ERR_HIP, which reports a
 *     failed launch and may follow earlier launches of the same call).
 *   - T = 0 returns BEAM_MOE_OK with no launch.
 *   - Weight layouts follow the (out_features, in_features) convention of linear
 *     layers: Wg, Wu [E, I, d]; Wd [E, d, I]; the router weight is Wr [d, E] FP32. The
 *     expert weights may instead be given in the packed layout of beam_moe_pack_weights,
 *     as beam_moe_shape.weight_layout says (same values, same results, faster streams).
 *
 * Supported shapes (else BEAM_MOE_ERR_UNSUPPORTED_SHAPE): d and I multiples of 64;
 * E <= 64, or E in {128, 256, 512, 1024}; E % n_group == 0; n_group <= 64; the
 * group size E/n_group >= 2 and, per 64-lane wavefront, a power-of-two number of
 * lanes per group; 1 <= topk_group <= n_group; 1 <= top_k <= min(16, topk_group *
 * E/n_group); T * top_k < 2^31.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer shape and constants (Transformers "Beam" page, BeamConfig: hidden_size = d,
 * num_experts = E, n_group, topk_group, num_experts_per_tok = top_k,
 * moe_intermediate_size = I, routed_scaling_factor, norm_topk_prob, rms_norm_eps). */
typedef struct beam_moe_shape {
    int64_t T;                    /* tokens in the batch */
    int32_t d;                    /* hidden size (5120 for Beam) */
    int32_t E;                    /* routed experts (256) */
    int32_t n_group;              /* expert groups (8) */
    int32_t topk_group;           /* groups kept per token (4) */
    int32_t top_k;                /* experts per token (8) */
    int32_t I;                    /* expert intermediate size (2560) */
    float routed_scaling_factor;  /* 2.5 */
    int32_t norm_topk_prob;       /* 1: renormalise the chosen weights to sum to 1 first */
    float rms_eps;                /* 1e-6; used only when a norm weight is given */
    int32_t weight_layout;        /* BEAM_MOE_WEIGHTS_ROW_MAJOR (0) or BEAM_MOE_WEIGHTS_PACKED (1) */
} beam_moe_shape;

/* Layout of the expert weights Wg, Wu [E, I, d] and Wd [E, d, I] that a call reads.
 * ROW_MAJOR: as written, row-major. PACKED: the same bf16 values rearranged by
 * beam_moe_pack_weights, once, when the weights are loaded; every entry point that takes a
 * shape and expert weights accepts either (for FP8 weights, see beam_moe_forward_fp8), with
 * bitwise-identical results. Packed, the decode weight streams read whole contiguous
 * kilobytes and run ~10% faster on MI355X. */
enum { BEAM_MOE_WEIGHTS_ROW_MAJOR = 0, BEAM_MOE_WEIGHTS_PACKED = 1 };

typedef enum beam_moe_status {
    BEAM_MOE_OK = 0,
    BEAM_MOE_ERR_INVALID_ARG = 1,        /* NULL required pointer, misaligned pointer, bad value */
    BEAM_MOE_ERR_UNSUPPORTED_SHAPE = 2,  /* shape outside the supported set above */
    BEAM_MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    BEAM_MOE_ERR_HIP = 4                 /* a kernel launch failed */
} beam_moe_status;

/* Bytes of device workspace that beam_moe_forward needs for this shape; it also
 * covers beam_moe_route and beam_moe_dispatch. Returns 0 for an invalid shape. */
size_t beam_moe_workspace_bytes(const beam_moe_shape* shape);

/* Router: the routing steps of the layer for T tokens.
 *   x         [T, d] bf16: hidden states (or, with norm_w, the pre-norm hidden states h)
 *   norm_w    [d] bf16 or NULL: pre-MLP RMSNorm weight; when given, x_normed must be given
 *   x_normed  [T, d] bf16 out, written iff norm_w != NULL: bf16((h * r) * norm_w),
 *             r = 1/sqrt(mean(h^2) + rms_eps), computed in FP64
 *   Wr        [d, E] FP32 router weight;  bias [E] FP32 per-expert selection bias
 *   topk_idx  [T, top_k] int32 out: chosen experts, by descending biased score,
 *             ties to the lower expert id
 *   topk_w    [T, top_k] FP32 out: routing weights aligned with topk_idx (unbiased
 *             scores, renormalised, times routed_scaling_factor)
 *   logits    [T, E] FP32 out or NULL: raw router logits z (before the sigmoid)
 *   workspace, ws_bytes: device scratch of at least beam_moe_workspace_bytes(shape). */
beam_moe_status beam_moe_route(const beam_moe_shape* shape, const void* x, const void* norm_w, void* x_normed,
                               const float* Wr, const float* bias, int32_t* topk_idx, float* topk_w,
                               float* logits, void* workspace, size_t ws_bytes, void* stream);

/* Dispatch: a stable counting sort of the T*top_k (token, slot) pairs by expert
 * (the single-GPU form of sending each token to the holder of its experts; "Use HF
 * Transformers" cookbook, Parallelism). Pair p = t*top_k + j.
 *   topk_idx        [T, top_k] int32: expert ids; each must lie in [0, E) and the ids of
 *                   one token must be distinct (as beam_moe_route produces). Pairs with an
 *                   id outside [0, E) are dropped (pair_rank = -1); repeated ids within a
 *                   token are not detected.
 *   expert_offsets  [E+1] int32 out: pairs of expert e occupy [offsets[e], offsets[e+1])
 *   sorted_pairs    [T*top_k] int32 out: pair ids in expert order, ascending p inside an expert
 *   pair_rank       [T*top_k] int32 out or NULL: position of pair p in sorted_pairs
 *   workspace, ws_bytes: as for beam_moe_route. */
beam_moe_status beam_moe_dispatch(const beam_moe_shape* shape, const int32_t* topk_idx, int32_t* expert_offsets,
                                  int32_t* sorted_pairs, int32_t* pair_rank, void* workspace, size_t ws_bytes,
                                  void* stream);

/* The whole layer: route, dispatch, the grouped SwiGLU expert GEMMs (BF16 MFMA,
 * FP32 accumulation, h rounded to bf16 once) and the weighted combine.
 *   x, norm_w, Wr, bias  as for beam_moe_route (the normed x is kept in the workspace)
 *   Wg, Wu    [E, I, d] bf16 gate and up projections;  Wd [E, d, I] bf16 down projection
 *   y         [T, d] FP32 out: sum over the token's experts of w_j * expert output, added
 *             in slot order j = 0..top_k-1 (bitwise deterministic run to run)
 *   topk_idx, topk_w, logits: optional copies of the routing (NULL to skip)
 *   workspace, ws_bytes: at least beam_moe_workspace_bytes(shape). */
beam_moe_status beam_moe_forward(const beam_moe_shape* shape, const void* x, const void* norm_w, const float* Wr,
                                 const float* bias, const void* Wg, const void* Wu, const void* Wd, float* y,
                                 int32_t* topk_idx, float* topk_w, float* logits, void* workspace, size_t ws_bytes,
                                 void* stream);

/* beam_moe_forward with stage timing, for measurement tools: identical work and results,
 * plus a hipEventRecord on `stream` of each non-NULL stage_events[i] (hipEvent_t, created
 * by the caller) at six points: [0] before the router, [1] after the router, [2] after
 * the dispatch, [3] after the gate/up SwiGLU GEMM, [4] after the down GEMM, [5] after the
 * combine. stage_events may be NULL (then this is beam_moe_forward). */
beam_moe_status beam_moe_forward_staged(const beam_moe_shape* shape, const void* x, const void* norm_w,
                                        const float* Wr, const float* bias, const void* Wg, const void* Wu,
                                        const void* Wd, float* y, int32_t* topk_idx, float* topk_w, float* logits,
                                        void* workspace, size_t ws_bytes, void* stream, void* const* stage_events);

/* Post-MLP half of the sandwich norm and the depth-scaled residual add (Transformers
 * "Beam" page, Overview: sandwich norms item and FP32 RMSNorm note; archdb fact sheet,
 * normalisation and residual rows: k = 2(i+1)+1 for the MLP of 0-indexed layer i, FP32
 * residual accumulation; news.hamidun.com article, section on the residual stream).
 * For every token t, in FP32:
 *   n[t]         = y[t] * (1 / sqrt(mean_j y[t,j]^2 + rms_eps)) * post_w
 *   resid_out[t] = resid[t] * sqrt((k-1)/k) + n[t] / sqrt(k),   k = 2 * (layer + 1) + 1
 *   shape      the layer's shape; only T, d and rms_eps are used (the rest is still validated)
 *   y          [T, d] FP32: the MoE output (as beam_moe_forward writes it)
 *   post_w     [d] bf16: the post-MLP RMSNorm weight
 *   layer      0-indexed decoder layer (>= 0, else BEAM_MOE_ERR_INVALID_ARG)
 *   resid      [T, d] FP32: the residual stream before this MLP's contribution
 *   resid_out  [T, d] FP32 out; may be the same buffer as resid (in place), must not
 *              otherwise overlap it
 * d up to 16384 (else BEAM_MOE_ERR_UNSUPPORTED_SHAPE). No workspace. */
beam_moe_status beam_moe_post_residual(const beam_moe_shape* shape, const float* y, const void* post_w, int32_t layer,
                                       const float* resid, float* resid_out, void* stream);

/* The whole layer with the post-MLP norm and residual add fused into the combine: the
 * same routing and expert work as beam_moe_forward_staged, then for each token the
 * slot-ordered sum y[t] feeds beam_moe_post_residual's formula in the same kernel, so y
 * need not make a round trip through HBM.
 *   post_w, layer, resid, resid_out: as for beam_moe_post_residual
 *   y          [T, d] FP32 out or NULL: the MoE output before the norm, bitwise equal to
 *              beam_moe_forward's y (NULL skips the write)
 *   stage_events: as for beam_moe_forward_staged ([5] follows the fused combine), or NULL
 * Other arguments as for beam_moe_forward. */
beam_moe_status beam_moe_forward_residual(const beam_moe_shape* shape, const void* x, const void* norm_w,
                                          const float* Wr, const float* bias, const void* Wg, const void* Wu,
                                          const void* Wd, const void* post_w, int32_t layer, const float* resid,
                                          float* resid_out, float* y, int32_t* topk_idx, float* topk_w,
                                          float* logits, void* workspace, size_t ws_bytes, void* stream,
                                          void* const* stage_events);

/* FP8 expert weights (decode-sized batches). The pages name FP8 checkpoints (news.hamidun.com
 * article and strelka.ai overview, FP8 weights) but no scaling recipe; the layout here is the
 * OCP Microscaling (MX) v1.0 FP8 one: E4M3 codes (OCP 8-bit floating point: bias 7, largest
 * finite 448) and one E8M0 scale byte per 32 consecutive values of a row, value =
 * 2^(scale - 127) * e4m3(code).
 *
 * beam_moe_quantize_fp8: w [rows, K] bf16 -> q [rows, K] codes and scales [rows, K/32] bytes.
 *   Shared exponent of a block = floor(log2(max |w|)) - 8, clamped to [-127, 127] (0 for a
 *   block of zeros); each w / 2^shared rounded to the nearest E4M3 value, ties to even,
 *   saturated to +-448. K % 32 == 0 (else BEAM_MOE_ERR_INVALID_ARG); w and q 16-byte aligned.
 *   For expert weights call it on Wg and Wu viewed as [E*I, d] and on Wd as [E*d, I]. */
beam_moe_status beam_moe_quantize_fp8(int64_t rows, int32_t K, const void* w, void* q, void* scales, void* stream);

/* beam_moe_forward_staged with FP8 expert weights: identical routing, dispatch and combine;
 * the gate/up and down GEMMs read the codes and scales from beam_moe_quantize_fp8 (Wg8, Wu8
 * [E, I, d], Wd8 [E, d, I], sg, su [E, I, d/32], sd [E, d, I/32]) and widen them exactly to bf16
 * in registers, so the result is the bf16 layer's on the dequantized weights. Decode-sized
 * batches only (T * top_k <= 16 * E) with d and I multiples of 512, else
 * BEAM_MOE_ERR_UNSUPPORTED_SHAPE. All pointers 16-byte aligned.
 * With weight_layout = BEAM_MOE_WEIGHTS_PACKED the codes are packed: each code matrix q
 * [rows, K] passed through beam_moe_pack_weights(rows, K / 2, q, q_packed) (two codes per
 * 16-bit unit), which gives 16-row blocks of 64-k steps of 1 KB; the scales stay as the
 * quantizer wrote them. The result is bitwise the row-major one. */
beam_moe_status beam_moe_forward_fp8(const beam_moe_shape* shape, const void* x, const void* norm_w, const float* Wr,
                                     const float* bias, const void* Wg8, const void* Wu8, const void* Wd8,
                                     const void* sg, const void* su, const void* sd, float* y, int32_t* topk_idx,
                                     float* topk_w, float* logits, void* workspace, size_t ws_bytes, void* stream,
                                     void* const* stage_events);

/* Dense SwiGLU MLP of the first decoder layers (Transformers "Beam" page, Overview: the
 * first 3 layers use a dense SwiGLU MLP; BeamConfig: intermediate_size, hidden_act):
 *   y = Wd . bf16(silu(Wg . x) * (Wu . x))   per token, BF16 MFMA with FP32 accumulation,
 * h rounded to bf16 once as in the experts; no routing, no scaling.
 *   T, d, I    tokens, hidden size (5120), intermediate size (20480); d and I multiples of
 *              128, I >= 2048, T*d, T*I and d*I below 2^31, else BEAM_MOE_ERR_UNSUPPORTED_SHAPE.
 *              (h is rounded to bf16 from FP32 sums; where the FP64 sum rounds to the other
 *              neighbour, one ulp of a large h moves y by about 2^-4 * 3.5 / sqrt(I), which
 *              reaches 1e-2 * rms(y) near I = 512 and stays near half of it from I = 2048.) T <= 64
 *              (decode): weight streams against the tokens, the reduction over k split in parts
 *              added in a fixed order. Larger T: the tiled GEMM.
 *   weight_layout  BEAM_MOE_WEIGHTS_ROW_MAJOR, or PACKED (Wg, Wu through beam_moe_pack_weights
 *              as [I, d], Wd as [d, I]); else BEAM_MOE_ERR_INVALID_ARG. Same results either way.
 *   x          [T, d] bf16
 *   Wg, Wu     [I, d] bf16;  Wd [d, I] bf16
 *   y          [T, d] FP32 out
 *   workspace  at least beam_moe_dense_workspace_bytes(T, d, I) bytes
 * T = 0 returns BEAM_MOE_OK with no launch. */
size_t beam_moe_dense_workspace_bytes(int64_t T, int32_t d, int32_t I);
beam_moe_status beam_moe_dense_mlp(int64_t T, int32_t d, int32_t I, int32_t weight_layout, const void* x,
                                   const void* Wg, const void* Wu, const void* Wd, float* y, void* workspace,
                                   size_t ws_bytes, void* stream);

/* Expert-parallel share of the layer: what one GPU computes when each GPU holds one
 * contiguous block of the experts and the tokens routed to them are sent to it ("Use HF
 * Transformers" cookbook, Parallelism: 32 of the 256 experts per GPU, which is one
 * routing group). Given the routing of T tokens (from beam_moe_route on any device),
 *   y_part[t] = sum over the slots j with e_begin <= topk_idx[t,j] < e_begin + e_count,
 *               in slot order, of topk_w[t,j] * expert(x_t)
 * (a row with no such slot is 0); summed over a partition of the experts into blocks, the
 * shares give beam_moe_forward's y up to FP32 rounding order. Same kernels as the layer,
 * on the local block only: dispatch of the local pairs, grouped SwiGLU GEMMs, combine.
 *   shape      the model shape (E = all experts; its routing fields are only validated)
 *              with T = number of tokens passed in
 *   e_begin, e_count  the local block of expert ids: 1 <= e_count, 0 <= e_begin,
 *              e_begin + e_count <= E, else BEAM_MOE_ERR_INVALID_ARG
 *   x          [T, d] bf16 (the normed hidden states if the layer uses the norm)
 *   topk_idx   [T, top_k] int32 global expert ids, distinct within a token; topk_w [T, top_k] FP32
 *   Wg, Wu     [e_count, I, d] bf16, Wd [e_count, d, I] bf16: the local experts, local id
 *              e - e_begin
 *   y_part     [T, d] FP32 out, fully overwritten
 *   workspace  at least beam_moe_share_workspace_bytes(shape, e_count) bytes
 *   stage_events  NULL, or 6 hipEvent_t recorded as in beam_moe_forward_staged ([0] and
 *              [1] together: there is no router step)
 * All pointers 16-byte aligned. T = 0 returns BEAM_MOE_OK with no launch.
 * beam_moe_share_workspace_bytes returns 0 for an invalid shape or e_count. */
size_t beam_moe_share_workspace_bytes(const beam_moe_shape* shape, int32_t e_count);
beam_moe_status beam_moe_experts_share(const beam_moe_shape* shape, int32_t e_begin, int32_t e_count, const void* x,
                                       const int32_t* topk_idx, const float* topk_w, const void* Wg, const void* Wu,
                                       const void* Wd, float* y_part, void* workspace, size_t ws_bytes, void* stream,
                                       void* const* stage_events);

/* Rearranges a bf16 weight matrix w [rows, K] (row-major) into the PACKED layout of the
 * expert weights: rows in blocks of 16; block b is a run of K/32 steps of 512 values, step
 * j holding, for lane l = 0..63, the 8 values w[16b + l % 16][32j + 8(l / 16) .. +8] (the
 * operand a wave of 64 lanes feeds one 16x16x32 MFMA). Pack Wg and Wu as [E*I, d] and Wd
 * as [E*d, I]; the expert blocks stay contiguous (expert e is rows [e*I, (e+1)*I)), so a
 * slice of experts of a packed tensor is the packed tensor of those experts.
 *   rows     a multiple of 16;  K  a multiple of 32  (else BEAM_MOE_ERR_INVALID_ARG)
 *   w        [rows, K] bf16 in;  packed  [rows * K] bf16 out, not overlapping w
 * Pointers 16-byte aligned; rows * K below 2^40. rows = 0 returns BEAM_MOE_OK. */
beam_moe_status beam_moe_pack_weights(int64_t rows, int32_t K, const void* w, void* packed, void* stream);

/* beam_moe_forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same validation, kernels and results (bitwise) as beam_moe_forward, with its workspace
 * taken from a fixed 64 MiB scratch array that the library holds on each GPU it runs on until
 * the process ends (enough for the Beam shape up to T = 192 tokens). The call allocates and
 * frees nothing. A shape whose beam_moe_workspace_bytes exceeds 64 MiB returns
 * BEAM_MOE_ERR_WORKSPACE_TOO_SMALL before any GPU work. Every call on one GPU shares that GPU's
 * scratch, which keeps the last call's contents (nothing in it has to start at zero): calls that
 * overlap on one GPU (on different streams, or from several threads) race, and the caller must
 * order them. */
beam_moe_status beam_moe_forward_noalloc(const beam_moe_shape* shape, const void* x, const void* norm_w,
                                         const float* Wr, const float* bias, const void* Wg, const void* Wu,
                                         const void* Wd, float* y, int32_t* topk_idx, float* topk_w, float* logits,
                                         void* stream);

/* Static, human-readable name of a status code; "unknown status" for any other value (the
 * argument is a plain int so that any value a caller passes is well defined). */
const char* beam_moe_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */

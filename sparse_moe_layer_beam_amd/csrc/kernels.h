// Host-side launchers of the MoE-layer kernels (internal to libbeam_moe.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

struct Shape {
    int64_t T;
    int d, E, G, KG, K, I;
    float S;
    int norm;
    float eps;
    int packed;     // expert weights in the packed layout of beam_moe_pack_weights
    int route_E;    // experts the routing spreads the pairs over (E, or all experts for a share)
};

// Router (router.hip)
void launch_rmsnorm(const Shape& s, const void* h, const void* w, void* x_out, hipStream_t st);
int router_ksplit(const Shape& s);
size_t router_split_bytes(const Shape& s);
size_t router_zp_floats(const Shape& s);
// Logits, sigmoid, bias, group-limited top-k and weights for T tokens. With norm_w the input h
// is first normed into x_normed (pre-MLP RMSNorm, in the launch that splits the router weight
// when the route has one), which the router then reads; without it h is x.
// wrs: scratch of router_split_bytes(s); z_part: scratch of router_zp_floats(s) floats.
void launch_router(const Shape& s, const void* h, const void* norm_w, void* x_normed, const float* Wr,
                   const float* bias, void* wrs, float* z_part, int32_t* idx, float* w, float* logits, hipStream_t st);

// Dispatch (dispatch.hip)
constexpr int kChunkPairs = 1024;
// The tile count that the dispatch writes for the grouped GEMMs is followed by their work-queue
// counters, one per XCD for each of the two GEMMs, which the same dispatch zeroes.
constexpr int kTileWords = 1 + 2 * 8;
void launch_dispatch(const Shape& s, const int32_t* idx, int32_t* offsets, int32_t* sorted_pairs,
                     int32_t* pair_rank, int32_t* chunk_counts, int32_t* rank_in_chunk, int32_t* tiles,
                     int32_t* n_tiles, int tile_m, hipStream_t st);

// Experts (experts.hip: path choice, streaming kernels, combine; grouped_gemm.hip: tiled GEMM)
int experts_tile_m(const Shape& s);
bool experts_tiled(const Shape& s);
int gemm_tile_m(const Shape& s);
// Router logits of large batches on the tiled GEMM (grouped_gemm.hip): zp[kb][t][pl*E + e]
// over k part kb of ks, for the three planes pl of the split router weight.
void launch_gemm_router(const Shape& s, const void* x, const void* WrS, float* zp, int ks, hipStream_t st);
int gemm_router_items(const Shape& s, int ks);
bool gemm_supports(const Shape& s);
void launch_gemm_swiglu(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                        const int32_t* tiles, int32_t* n_tiles, const void* Wg, const void* Wu, void* h,
                        hipStream_t st);
void launch_gemm_down(const Shape& s, const void* h, const int32_t* offsets, const int32_t* sorted_pairs,
                      const int32_t* tiles, int32_t* n_tiles, const void* Wd, float* y_perm, hipStream_t st);
void launch_swiglu(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                   const int32_t* tiles, int32_t* n_tiles, const void* Wg, const void* Wu, void* h,
                   hipStream_t st);
void launch_down(const Shape& s, const void* h, const int32_t* offsets, const int32_t* sorted_pairs,
                 const int32_t* tiles, int32_t* n_tiles, const void* Wd, float* y_perm, hipStream_t st);
void launch_combine(const Shape& s, const float* y_perm, const int32_t* pair_rank, const float* topk_w, float* y,
                    hipStream_t st);

// Weights [rows, K] -> the packed layout of beam_moe_pack_weights (rows % 16 == 0, K % 32 == 0).
void launch_pack_stream(const void* W, void* P, int64_t rows, int K, hipStream_t st);

// Expert ids -> local ids of the block [e_begin, e_begin + e_count), -1 outside (expert-parallel share).
void launch_share_idx(const int32_t* idx, int64_t P, int e_begin, int e_count, int32_t* idx_local, hipStream_t st);

// FP8 (OCP E4M3 + one E8M0 scale per 32 values) expert weights for decode (experts_fp8.hip).
void launch_fp8_quantize(int64_t rows, int K, const void* w, void* q, void* s, hipStream_t st);
bool fp8_supports(const Shape& s);
void launch_swiglu_fp8(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                       const void* Wg8, const void* Wu8, const void* sg, const void* su, void* h, hipStream_t st);
void launch_down_fp8(const Shape& s, const void* h, const int32_t* offsets, const void* Wd8, const void* sd,
                     float* y_perm, hipStream_t st);

// Dense SwiGLU MLP through the same GEMM (grouped_gemm.hip).
bool dense_supports(int64_t T, int d, int I);
// Dense MLP for decode-sized batches (T <= 64): weight streams against packed token tiles.
bool dense_stream_supports(int64_t T, int d, int I);
size_t dense_stream_workspace_bytes(int64_t T, int d, int I);
void launch_dense_stream(int64_t T, int d, int I, bool packed, const void* x, const void* Wg, const void* Wu,
                         const void* Wd, float* y, void* ws, hipStream_t st);
void launch_dense_swiglu(int64_t T, int d, int I, bool packed, const void* x, const void* Wg, const void* Wu, void* h,
                         hipStream_t st);
void launch_dense_down(int64_t T, int d, int I, bool packed, const void* h, const void* Wd, float* y, hipStream_t st);

// Post-MLP RMSNorm + depth-scaled residual (residual.hip); rows of up to kPostMaxD floats.
constexpr int kPostMaxD = 16384;
void launch_combine_post_residual(const Shape& s, const float* y_perm, const int32_t* pair_rank, const float* topk_w,
                                  const void* post_w, int layer, const float* resid, float* resid_out, float* y,
                                  hipStream_t st);
void launch_post_residual(const Shape& s, const float* y, const void* post_w, int layer, const float* resid,
                          float* resid_out, hipStream_t st);

}  // namespace beam

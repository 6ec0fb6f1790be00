// Tiled grouped GEMM for batches with many tokens per expert (prefill): the gate/up
// projection with SwiGLU fused in the epilogue, and the down projection with the routing
// weight fused in the epilogue. BF16 MFMA (v_mfma_f32_32x32x16_bf16), FP32 accumulation.
//
// Method: Transformers "Beam" model page (Overview: sparse MoE item, FP32 SwiGLU note;
// BeamConfig: moe_intermediate_size, hidden_act) and archdb "Beam-1.0-501B-A23B" fact
// sheet (FFN rows: SwiGLU without biases).
//
// Tile: 128 tokens of one expert x 256 weight rows (gate/up: 128 gate + the matching 128 up
// channels; down: 256 output channels), K staged through LDS 64 at a time, double-buffered.
// Eight waves (two per SIMD, so one wave's MFMAs cover the other's stalls), each a 64-token
// x 64-row register tile (4 MFMA tiles of 32x32, 64 FP32 accumulators per lane); a 4-wave
// variant with 64x128 wave tiles is kept behind BEAM_GEMM_WAVES. The weight rows are the MFMA A operand and the tokens the B
// operand, so each lane ends up holding 4 consecutive output channels of one token.
#include "common.h"
#include "kernels.h"

namespace beam {
namespace {

constexpr int GBM = 128;             // tokens per tile
constexpr int GBK = 64;              // k per LDS stage
constexpr int GBR = 256;             // weight rows per tile
constexpr int LROW = GBK + 8;        // padded LDS row (bf16): 144 B keeps ds_read_b128 conflict-free
constexpr int A_ELEMS = GBM * LROW;
constexpr int B_ELEMS = GBR * LROW;
constexpr int STAGE = A_ELEMS + B_ELEMS;
#ifndef BEAM_GEMM_WAVES
#define BEAM_GEMM_WAVES 8       // 8: two waves per SIMD, 64x64 wave tiles; 4: 64x128 wave tiles
#endif
constexpr int NW = BEAM_GEMM_WAVES;
constexpr int NT = 64 * NW;                 // threads per block
constexpr int LR = NT / 8;                  // rows covered by one 16-byte-per-thread sweep
constexpr int NQ = NW == 8 ? 2 : 4;         // 32-row weight subtiles per wave
constexpr int AL = GBM / LR, BL = GBR / LR; // 16-byte loads per thread per stage

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void gload(u32x4 (&ra)[AL], u32x4 (&rb)[BL], const u16* const (&a_src)[AL],
                                      const u16* const (&b_src)[BL], int k) {
#pragma unroll
    for (int i = 0; i < AL; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + k);
#pragma unroll
    for (int i = 0; i < BL; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + k);
}

__device__ __forceinline__ void lstore(u16* stage, const u32x4 (&ra)[AL], const u32x4 (&rb)[BL], int lrow,
                                       int lcol) {
    u16* B = stage + A_ELEMS;
#pragma unroll
    for (int i = 0; i < AL; ++i) *reinterpret_cast<u32x4*>(stage + (lrow + LR * i) * LROW + lcol) = ra[i];
#pragma unroll
    for (int i = 0; i < BL; ++i) *reinterpret_cast<u32x4*>(B + (lrow + LR * i) * LROW + lcol) = rb[i];
}

// MODE 0: out = h [P, I] bf16 = bf16(silu(act . Wg^T) * (act . Wu^T)), act = x rows gathered
//         through sorted_pairs (token = pair / top_k); W0 = Wg, W1 = Wu, both [E, Ndim, Kdim].
// MODE 1: out = y_perm [P, d] fp32 = w_pair * (act . Wd^T), act = h rows in sorted order;
//         W0 = Wd [E, Ndim, Kdim].
template <int MODE>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_kernel(
        const u16* __restrict__ act, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
        const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles_p, const u16* __restrict__ W0,
        const u16* __restrict__ W1, const float* __restrict__ topk_w, int top_k, void* __restrict__ out, int Kdim,
        int Ndim, int n_nb) {
    __shared__ __align__(16) u16 lds[2 * STAGE];

    // Work item -> (expert, n-block, m-tile). Blocks are dispatched to the 8 XCDs round-robin
    // (block b on XCD b % 8); XCD x takes the contiguous item range [x*per_xcd, (x+1)*per_xcd),
    // ordered expert, n-block, m-tile, so the m-tiles sharing one weight tile run together
    // on one XCD and the tile comes from HBM about once.
    const int n_items = *n_tiles_p * n_nb;
    const int per_xcd = (n_items + 7) / 8;
    const int slot = blockIdx.x >> 3;
    if (slot >= per_xcd) return;
    const int item = (blockIdx.x & 7) * per_xcd + slot;
    if (item >= n_items) return;
    const int j = item / n_nb;                 // a tile of the item's expert
    const int e = tiles[4 * j], first = tiles[4 * j + 2], cnt = tiles[4 * j + 3];
    const int local = item - first * n_nb;
    const int nb = local / cnt;
    const int mt = local - nb * cnt;
    const int beg = offsets[e];
    const int n_e = offsets[e + 1] - beg;
    const int m0 = mt * GBM;
    const int rows = min(GBM, n_e - m0);
    const int n0 = nb * (MODE == 0 ? GBR / 2 : GBR);

    // Global -> LDS roles: thread t moves 16 B at column (t%8)*8 of rows t/8 + LR*i.
    const int tid = threadIdx.x;
    const int lrow = tid >> 3, lcol = (tid & 7) * 8;
    const u16* a_src[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int m = m0 + min(lrow + LR * i, rows - 1);   // rows past the end repeat a valid row
        size_t row;
        if constexpr (MODE == 0) row = (size_t)(sorted_pairs[beg + m] / top_k);
        else row = (size_t)(beg + m);
        a_src[i] = act + row * Kdim + lcol;
    }
    const u16* b_src[BL];
#pragma unroll
    for (int i = 0; i < BL; ++i) {
        const int r = lrow + LR * i;
        if constexpr (MODE == 0) {
            const u16* W = r < GBR / 2 ? W0 : W1;
            const int ch = min(n0 + (r & (GBR / 2 - 1)), Ndim - 1);
            b_src[i] = W + ((size_t)e * Ndim + ch) * Kdim + lcol;
        } else {
            const int ch = min(n0 + r, Ndim - 1);
            b_src[i] = W0 + ((size_t)e * Ndim + ch) * Kdim + lcol;
        }
    }
    u32x4 ra0[AL], rb0[BL], ra1[AL], rb1[BL];
    // Wave tile: tokens [64*wm, +64) as 2 subtiles; NQ weight subtiles of 32 rows. For the
    // gate/up pass the first half of the subtiles are gate rows and the second half the up
    // rows of the same channels.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // wave id in an SGPR
    const int wm = wave & 1, wn = wave >> 1;
    constexpr int WROWS = NQ * 32;              // weight rows per wave
    int wrow[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if constexpr (MODE == 0) wrow[q] = (q < NQ / 2 ? 0 : GBR / 2) + (WROWS / 2) * wn + 32 * (q % (NQ / 2));
        else wrow[q] = WROWS * wn + 32 * q;
    }
    const int frag = (lane & 31) * LROW + (lane >> 5) * 8;
    f32x16 acc[2][NQ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][q][v] = 0.0f;

    // Token subtiles of this wave that hold at least one real token (the rest of a partial
    // tile is padding: its MFMAs are skipped).
    const int live = min(2, max(0, (rows - 64 * wm + 31) / 32));

    // Pipeline (Kdim is a multiple of 2*GBK): LDS holds stage kt (being multiplied) and receives stage kt+1 from registers
    // loaded one step earlier; the loads for stage kt+2 are in flight meanwhile. The last
    // prefetches re-read the final stage (in bounds, never consumed), so there is no branch.
    const int nk = Kdim / GBK;
    gload(ra0, rb0, a_src, b_src, 0);
    lstore(lds, ra0, rb0, lrow, lcol);
    gload(ra1, rb1, a_src, b_src, min(1, nk - 1) * GBK);
    __syncthreads();
    // One LDS stage: 4 sub-steps of k=16; the fragments of sub-step kk+1 are read from LDS
    // while the 8 MFMAs of sub-step kk run.
    auto mma_stage = [&](const u16* A) {
        const u16* B = A + A_ELEMS;
        bf16x8 w[2][NQ], x[2][2];
#pragma unroll
        for (int q = 0; q < NQ; ++q) w[0][q] = *reinterpret_cast<const bf16x8*>(B + wrow[q] * LROW + frag);
#pragma unroll
        for (int i = 0; i < 2; ++i) x[0][i] = *reinterpret_cast<const bf16x8*>(A + (64 * wm + 32 * i) * LROW + frag);
#pragma unroll
        for (int kk = 0; kk < GBK / 16; ++kk) {
            const int c = kk & 1, n = c ^ 1;
            if (kk + 1 < GBK / 16) {
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    w[n][q] = *reinterpret_cast<const bf16x8*>(B + wrow[q] * LROW + frag + 16 * (kk + 1));
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    x[n][i] = *reinterpret_cast<const bf16x8*>(A + (64 * wm + 32 * i) * LROW + frag + 16 * (kk + 1));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (i < live)
#pragma unroll
                    for (int q = 0; q < NQ; ++q) acc[i][q] = mfma32(w[c][q], x[c][i], acc[i][q]);
        }
    };
    for (int kt = 0; kt < nk; kt += 2) {
        gload(ra0, rb0, a_src, b_src, min(kt + 2, nk - 1) * GBK);
        mma_stage(lds);
        lstore(lds + STAGE, ra1, rb1, lrow, lcol);
        __syncthreads();
        gload(ra1, rb1, a_src, b_src, min(kt + 3, nk - 1) * GBK);
        mma_stage(lds + STAGE);
        lstore(lds, ra0, rb0, lrow, lcol);
        __syncthreads();
    }

    // Epilogue. acc[i][q][v]: token 64*wm + 32*i + lane%32 of the tile, weight row
    // wrow[q] + 8*(v/4) + 4*(lane/32) + v%4.
    const int tcol = lane & 31, rsub = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + tcol;
        if (r >= rows) continue;
        const size_t orow = (size_t)(beg + m0 + r);
        if constexpr (MODE == 0) {
            u16* h = reinterpret_cast<u16*>(out);
#pragma unroll
            for (int q = 0; q < NQ / 2; ++q)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int ch = n0 + (WROWS / 2) * wn + 32 * q + 8 * g4 + rsub;
                    if (ch >= Ndim) continue;
                    uint32_t pk[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int v = 4 * g4 + 2 * h2;
                        pk[h2] = (uint32_t)f32_to_bf16(silu_mul(acc[i][q][v], acc[i][q + NQ / 2][v])) |
                                 ((uint32_t)f32_to_bf16(silu_mul(acc[i][q][v + 1], acc[i][q + NQ / 2][v + 1]))
                                  << 16);
                    }
                    *reinterpret_cast<uint2*>(h + orow * Ndim + ch) = make_uint2(pk[0], pk[1]);
                }
        } else {
            float* y = reinterpret_cast<float*>(out);
            const float wt = topk_w[sorted_pairs[beg + m0 + r]];
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int ch = n0 + WROWS * wn + 32 * q + 8 * g4 + rsub;
                    if (ch >= Ndim) continue;
                    const int v = 4 * g4;
                    *reinterpret_cast<float4*>(y + orow * Ndim + ch) =
                        make_float4(wt * acc[i][q][v], wt * acc[i][q][v + 1], wt * acc[i][q][v + 2],
                                    wt * acc[i][q][v + 3]);
                }
        }
    }
}

int max_items(const Shape& s, int n_nb) {
    const int64_t P = s.T * s.K;
    const int64_t max_tiles = (P + GBM - 1) / GBM + s.E;
    return (int)(max_tiles * n_nb);
}

}  // namespace

int gemm_tile_m() { return GBM; }

bool gemm_supports(const Shape& s) { return s.d % (2 * GBK) == 0 && s.I % (2 * GBK) == 0; }

void launch_gemm_swiglu(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                        const int32_t* tiles, const int32_t* n_tiles, const void* Wg, const void* Wu, void* h,
                        hipStream_t st) {
    const int n_nb = (s.I + GBR / 2 - 1) / (GBR / 2);
    const int blocks = (max_items(s, n_nb) + 7) / 8 * 8;
    hipLaunchKernelGGL(grouped_gemm_kernel<0>, dim3((unsigned)blocks), dim3(NT), 0, st, (const u16*)x, offsets,
                       sorted_pairs, tiles, n_tiles, (const u16*)Wg, (const u16*)Wu, nullptr, s.K, h, s.d, s.I,
                       n_nb);
}

void launch_gemm_down(const Shape& s, const void* h, const int32_t* offsets, const int32_t* sorted_pairs,
                      const float* topk_w, const int32_t* tiles, const int32_t* n_tiles, const void* Wd,
                      float* y_perm, hipStream_t st) {
    const int n_nb = (s.d + GBR - 1) / GBR;
    const int blocks = (max_items(s, n_nb) + 7) / 8 * 8;
    hipLaunchKernelGGL(grouped_gemm_kernel<1>, dim3((unsigned)blocks), dim3(NT), 0, st, (const u16*)h, offsets,
                       sorted_pairs, tiles, n_tiles, (const u16*)Wd, nullptr, topk_w, s.K, y_perm, s.I, s.d,
                       n_nb);
}

}  // namespace beam

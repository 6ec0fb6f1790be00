// Tiled grouped GEMM for batches with many tokens per expert (prefill): the gate/up
// projection with SwiGLU fused in the epilogue, and the down projection with the routing
// weight fused in the epilogue. BF16 MFMA (v_mfma_f32_16x16x32_bf16), FP32 accumulation.
//
// Method: Transformers "Beam" model page (Overview: sparse MoE item, FP32 SwiGLU note;
// BeamConfig: moe_intermediate_size, hidden_act) and archdb "Beam-1.0-501B-A23B" fact
// sheet (FFN rows: SwiGLU without biases).
//
// Tile: up to 128 tokens of one expert x 256 weight rows (gate/up: 128 gate channels and
// the same 128 up channels; down: 256 output channels). Four waves, one per SIMD, each
// owning 64 weight rows (four 16-row MFMA subtiles) against all the tile's tokens: a
// 128 x 64 register tile, 128 FP32 accumulators per lane, so two blocks share a CU and
// one block's MFMAs run while the other waits on memory.
//
// Why this shape on gfx950:
//  * A weight row is used by one wave only, so weights skip LDS and stream from global
//    memory straight into registers in MFMA operand layout, one LDS stage ahead. Only the
//    tokens, which every wave needs, are staged through LDS (64 k at a time,
//    double-buffered, one barrier per stage). Per flop this needs half the LDS reads of a
//    both-operands-in-LDS tile with 64x64 wave tiles and a third of its LDS writes.
//  * The 16x16x32 operand layout gives four lanes to a row, so one weight load covers 16
//    rows x 64 contiguous bytes (in the 32x32x16 layout a load touches 32 rows x 32 bytes).
//  * Operands are buffer resources: base and size in scalar registers, one 32-bit offset
//    per row in a vector register, and loads past the end return zeros.
// What bounds it (measured on MI355X at T = 8192): removing every MFMA leaves the time
// unchanged, removing the weight loads halves it. The kernel is bound by the operand
// traffic from L2 into the CUs (each weight byte is read once per 128-token tile of its
// expert, tokens once per 256-row weight block), not by the MFMAs or LDS.
#include "common.h"
#include "kernels.h"

namespace beam {
namespace {

#ifndef BEAM_GEMM_M
#define BEAM_GEMM_M 128
#endif
constexpr int GM = BEAM_GEMM_M;      // tokens per tile
constexpr int kBlocksPerCU = GM == 128 ? 2 : 1;
constexpr int GN = 256;              // weight rows per tile (4 waves x 64)
constexpr int GK = 64;               // k per LDS stage (two MFMA k-steps of 32)
constexpr int LROW = GK + 8;         // padded LDS row (bf16): 144 B keeps ds_read_b128 conflict-free
constexpr int TILE = GM * LROW;      // one LDS stage
constexpr int NT = 256;              // threads per block
constexpr int PAIRS = GM / 32;       // 32-token groups per tile (the unit of partial-tile trimming)
constexpr int LOADS = GM * GK * 2 / (NT * 16);   // 16-byte token loads per thread per stage
constexpr int kFrag = 4;             // token fragments read ahead of the MFMAs
#ifndef BEAM_GEMM_RING
#define BEAM_GEMM_RING 2
#endif
constexpr int RW = BEAM_GEMM_RING;   // stages of weights held in registers (RW-1 in flight)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Global operands as buffer resources: the base and size live in scalar registers and each
// lane keeps one 32-bit byte offset per row, so the loads cost few vector registers (that
// is what lets the weight prefetch run several stages deep). A load past the resource's
// size returns zeros instead of faulting.
constexpr uint32_t kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

struct Operands {
    __amdgpu_buffer_rsrc_t w0, w1;   // weight subtiles 0,1 and 2,3 (gate/up: gate and up)
    __amdgpu_buffer_rsrc_t a;        // token rows
    uint32_t wv0, wv1;               // this lane's weight row offsets (subtile q even / odd), bytes
    uint32_t av[LOADS];              // this thread's token row offsets, bytes
};

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// Weight registers of one stage: [k-step j][subtile q]; lane holds row lane%16 of subtile q,
// k = 64*s + 32*j + 8*(lane/16) .. +8 (kbytes = 128*s). Subtiles 0,1 come from w0 and 2,3
// from w1, the odd one 16 rows after the even one.
__device__ __forceinline__ void load_weights(bf16x8 (&w)[2][4], const Operands& op, uint32_t kbytes) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            w[j][q] = __builtin_bit_cast(bf16x8, bload(q < 2 ? op.w0 : op.w1, (q & 1 ? op.wv1 : op.wv0) + 64 * j,
                                                       kbytes));
}

// One LDS stage s (k = 64*s .. +64) for a tile whose first 32*LIVE tokens hold the real
// ones. PAR = s % 2 picks the weight registers; both are template arguments so every
// register array index is a compile-time constant and the stage has no branches.
template <int PAR, int LIVE>
__device__ __forceinline__ void gemm_stage(int s, int nstages, const u16* cur, u16* next,
                                           f32x4 (&acc)[2 * LIVE][4], bf16x8 (&wr)[RW][2][4], const Operands& op,
                                           u32x4 (&stg)[LOADS], int st_off, int frag) {
    constexpr int NS = 2 * LIVE;     // 16-token subtiles
    // tokens of stage s+1 into registers (the last stage re-reads itself: in bounds, unused)
    const int kn = min(s + 1, nstages - 1) * GK;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) stg[i] = bload(op.a, op.av[i], 2 * kn);
    // Token fragments stream through a ring of kFrag registers over the (k-step, subtile)
    // sequence, so each ds_read is issued kFrag-1 fragments before it is needed.
    constexpr int NF = 2 * NS;
    bf16x8 xr[kFrag];
#pragma unroll
    for (int f = 0; f < kFrag; ++f)
        if (f < NF) xr[f] = *reinterpret_cast<const bf16x8*>(cur + 16 * (f % NS) * LROW + frag + 32 * (f / NS));
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int j = f / NS, i = f % NS;
        const bf16x8 x = xr[f % kFrag];
        if (f + kFrag < NF) {
            const int g = f + kFrag;
            xr[f % kFrag] = *reinterpret_cast<const bf16x8*>(cur + 16 * (g % NS) * LROW + frag + 32 * (g / NS));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = mfma16(wr[PAR][j][q], x, acc[i][q]);
        // keep the read-ahead where it is: left alone, the scheduler sinks each ds_read to
        // its MFMAs and the LDS latency is paid in full every time
        __builtin_amdgcn_sched_barrier(0);
    }
    // this stage's weight registers take stage s+RW (clamped: in bounds, unused)
    load_weights(wr[PAR], op, 2 * GK * min(s + RW, nstages - 1));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) *reinterpret_cast<u32x4*>(next + st_off + 32 * i * LROW) = stg[i];
    __syncthreads();
}

// Stages s+P .. s+RW-1 of one ring period; LDS buffers alternate (RW is even).
template <int P, int LIVE>
__device__ __forceinline__ void gemm_period(int s, int nstages, u16* lds, f32x4 (&acc)[2 * LIVE][4],
                                            bf16x8 (&wr)[RW][2][4], const Operands& op, u32x4 (&stg)[LOADS],
                                            int st_off, int frag) {
    if constexpr (P < RW) {
        gemm_stage<P, LIVE>(s + P, nstages, lds + (P & 1) * TILE, lds + ((P + 1) & 1) * TILE, acc, wr, op, stg,
                            st_off, frag);
        gemm_period<P + 1, LIVE>(s, nstages, lds, acc, wr, op, stg, st_off, frag);
    }
}

// Everything after the work-item decode, for a tile with LIVE live 32-token groups.
template <int MODE, int LIVE>
__device__ __forceinline__ void gemm_tile(u16* lds, const Operands& op, int Kdim, int Ndim, int rows,
                                          size_t orow0, int c0, int lane, const int32_t* __restrict__ pair_of_row,
                                          const float* __restrict__ topk_w, void* __restrict__ out) {
    constexpr int NS = 2 * LIVE;
    f32x4 acc[NS][4];
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nstages = Kdim / GK;   // Kdim is a multiple of RW*GK
    bf16x8 wr[RW][2][4];
#pragma unroll
    for (int r = 0; r < RW; ++r) load_weights(wr[r], op, 2 * GK * min(r, nstages - 1));
    const int tid = threadIdx.x;
    const int st_off = (tid >> 3) * LROW + (tid & 7) * 8;
    u32x4 stg[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) stg[i] = bload(op.a, op.av[i], 0);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) *reinterpret_cast<u32x4*>(lds + st_off + 32 * i * LROW) = stg[i];
    __syncthreads();

    // token operand (MFMA B: lane holds token lane%16 of a subtile, k 8*(lane/16) .. +8)
    const int frag = (lane & 15) * LROW + (lane >> 4) * 8;
    for (int s = 0; s < nstages; s += RW)
        gemm_period<0, LIVE>(s, nstages, lds, acc, wr, op, stg, st_off, frag);

    // Epilogue. acc[i][q][v]: token 16*i + lane%16 of the tile, row 4*(lane/16) + v of
    // subtile q, i.e. channel c0 + 16*q' + 4*(lane/16) + v with q' = q (down) or q % 2
    // (gate/up: q = 0,1 gate and q = 2,3 up of the same channels).
    const int tcol = lane & 15, rsub = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int r = 16 * i + tcol;
        if (r >= rows) continue;
        const size_t orow = orow0 + r;
        if constexpr (MODE == 0) {
            u16* h = reinterpret_cast<u16*>(out);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int ch = c0 + 16 * q + rsub;
                if (ch >= Ndim) continue;
                const uint32_t lo = (uint32_t)f32_to_bf16(silu_mul(acc[i][q][0], acc[i][q + 2][0])) |
                                    ((uint32_t)f32_to_bf16(silu_mul(acc[i][q][1], acc[i][q + 2][1])) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16(silu_mul(acc[i][q][2], acc[i][q + 2][2])) |
                                    ((uint32_t)f32_to_bf16(silu_mul(acc[i][q][3], acc[i][q + 2][3])) << 16);
                *reinterpret_cast<uint2*>(h + orow * Ndim + ch) = make_uint2(lo, hi);
            }
        } else {
            float* y = reinterpret_cast<float*>(out);
            const float wt = topk_w ? topk_w[pair_of_row[r]] : 1.0f;   // NULL: dense MLP, weight 1
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ch = c0 + 16 * q + rsub;
                if (ch >= Ndim) continue;
                *reinterpret_cast<float4*>(y + orow * Ndim + ch) =
                    make_float4(wt * acc[i][q][0], wt * acc[i][q][1], wt * acc[i][q][2], wt * acc[i][q][3]);
            }
        }
    }
}

// MODE 0: out = h [P, I] bf16 = bf16(silu(act . Wg^T) * (act . Wu^T)), act = x rows gathered
//         through sorted_pairs (token = pair / top_k); W0 = Wg, W1 = Wu, both [E, Ndim, Kdim].
// MODE 1: out = y_perm [P, d] fp32 = w_pair * (act . Wd^T), act = h rows in sorted order;
//         W0 = Wd [E, Ndim, Kdim].
// DENSE: one expert holding all act_rows tokens in order (the dense SwiGLU MLP): no tile
//         list, no gather, weight 1; MODE 1 then writes y [T, d] directly.
template <int MODE, bool DENSE>
__global__ __launch_bounds__(NT, kBlocksPerCU) void grouped_gemm_kernel(
        const u16* __restrict__ act, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
        const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles_p, const u16* __restrict__ W0,
        const u16* __restrict__ W1, const float* __restrict__ topk_w, int top_k, void* __restrict__ out, int Kdim,
        int Ndim, int n_nb, int act_rows) {
    __shared__ __align__(16) u16 lds[2 * TILE];

    // Work item -> (expert, n-block, m-tile). Blocks are dispatched to the 8 XCDs round-robin
    // (block b on XCD b % 8); XCD x takes the contiguous item range [x*per_xcd, (x+1)*per_xcd),
    // ordered expert, n-block, m-tile, so the m-tiles sharing one weight tile run together
    // on one XCD and the tile comes from HBM about once.
    const int n_mt_dense = (act_rows + GM - 1) / GM;
    const int n_items = DENSE ? n_mt_dense * n_nb : *n_tiles_p * n_nb;
    const int per_xcd = (n_items + 7) / 8;
    const int slot = blockIdx.x >> 3;
    if (slot >= per_xcd) return;
    const int item = (blockIdx.x & 7) * per_xcd + slot;
    if (item >= n_items) return;
    int e, nb, mt, beg, n_e;
    if constexpr (DENSE) {
        e = 0;
        nb = item / n_mt_dense;
        mt = item - nb * n_mt_dense;
        beg = 0;
        n_e = act_rows;
    } else {
        const int j = item / n_nb;                 // a tile of the item's expert
        e = tiles[4 * j];
        const int first = tiles[4 * j + 2], cnt = tiles[4 * j + 3];
        const int local = item - first * n_nb;
        nb = local / cnt;
        mt = local - nb * cnt;
        beg = offsets[e];
        n_e = offsets[e + 1] - beg;
    }
    const int m0 = mt * GM;
    const int rows = min(GM, n_e - m0);
    const int live = min(PAIRS, (rows + 31) / 32);   // 32-token groups holding real tokens

    // Token staging: thread t moves 16 B at column (t%8)*8 of tile rows t/8 + 32*i.
    // Rows past the end of the expert's segment repeat its last row.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = tid >> 3, lcol = (tid & 7) * 8;
    Operands op;
    op.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(act), (short)0, 2 * act_rows * Kdim, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {   // gemm_supports keeps these offsets below 2^32
        const int m = m0 + min(lrow + 32 * i, rows - 1);
        uint32_t row;
        if constexpr (MODE == 0 && !DENSE) row = (uint32_t)(sorted_pairs[beg + m] / top_k);
        else row = (uint32_t)(beg + m);
        op.av[i] = 2 * (row * (uint32_t)Kdim + lcol);
    }
    // Weight operand (MFMA A: lane holds row lane%16 of a 16-row subtile, k 8*(lane/16) .. +8
    // of each 32-wide k-step). The wave's channels start at c0; the expert's base pointers
    // stay in scalar registers.
    int c0;
    const u16* We0 = W0 + (size_t)e * Ndim * Kdim;
    const uint32_t wbytes = 2u * (uint32_t)Ndim * (uint32_t)Kdim;    // one expert's matrix
    if constexpr (MODE == 0) {
        c0 = nb * (GN / 2) + 32 * wave;                 // 32 channels: gate rows, then up rows
        op.w0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(We0), (short)0, wbytes, kRsrcWord3);
        op.w1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(W1 + (size_t)e * Ndim * Kdim), (short)0, wbytes,
                                                  kRsrcWord3);
    } else {
        c0 = nb * GN + 64 * wave;                       // 64 output channels
        op.w0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(We0), (short)0, wbytes, kRsrcWord3);
        op.w1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(We0 + 32 * (size_t)Kdim), (short)0,
                                                  wbytes - 64u * (uint32_t)Kdim, kRsrcWord3);
    }
    // rows past Ndim (a partial last n-block) are clamped in bounds; their results are dropped
    const int last = Ndim - (MODE == 0 ? 32 : 64);
    op.wv0 = 2 * ((uint32_t)(min(c0, last) + (lane & 15)) * Kdim + (lane >> 4) * 8);
    op.wv1 = op.wv0 + 32u * (uint32_t)Kdim;             // 16 rows further

    const size_t orow0 = (size_t)(beg + m0);
    const int32_t* pair_of_row = DENSE ? nullptr : sorted_pairs + beg + m0;
    switch (live) {
#define BEAM_GEMM_CASE(L)                                                                                       \
    case L:                                                                                                     \
        gemm_tile<MODE, L>(lds, op, Kdim, Ndim, rows, orow0, c0, lane, pair_of_row, topk_w, out);              \
        break;
        BEAM_GEMM_CASE(1) BEAM_GEMM_CASE(2) BEAM_GEMM_CASE(3) BEAM_GEMM_CASE(4)
#if BEAM_GEMM_M > 128
        BEAM_GEMM_CASE(5) BEAM_GEMM_CASE(6) BEAM_GEMM_CASE(7) BEAM_GEMM_CASE(8)
#endif
#undef BEAM_GEMM_CASE
    }
}

int max_items(const Shape& s, int n_nb) {
    const int64_t P = s.T * s.K;
    const int64_t max_tiles = (P + GM - 1) / GM + s.E;
    return (int)(max_tiles * n_nb);
}

}  // namespace

int gemm_tile_m() { return GM; }

bool gemm_supports(const Shape& s) {
    const int64_t P = s.T * s.K;
    return s.d % (RW * GK) == 0 && s.I % (RW * GK) == 0 && s.T * s.d < (int64_t)INT32_MAX &&
           P * s.I < (int64_t)INT32_MAX && (int64_t)s.d * s.I < (int64_t)INT32_MAX;   // byte sizes below 2^32
}

void launch_gemm_swiglu(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                        const int32_t* tiles, const int32_t* n_tiles, const void* Wg, const void* Wu, void* h,
                        hipStream_t st) {
    const int n_nb = (s.I + GN / 2 - 1) / (GN / 2);
    const int blocks = (max_items(s, n_nb) + 7) / 8 * 8;
    hipLaunchKernelGGL((grouped_gemm_kernel<0, false>), dim3((unsigned)blocks), dim3(NT), 0, st, (const u16*)x, offsets,
                       sorted_pairs, tiles, n_tiles, (const u16*)Wg, (const u16*)Wu, nullptr, s.K, h, s.d, s.I,
                       n_nb, (int)s.T);
}

void launch_gemm_down(const Shape& s, const void* h, const int32_t* offsets, const int32_t* sorted_pairs,
                      const float* topk_w, const int32_t* tiles, const int32_t* n_tiles, const void* Wd,
                      float* y_perm, hipStream_t st) {
    const int n_nb = (s.d + GN - 1) / GN;
    const int blocks = (max_items(s, n_nb) + 7) / 8 * 8;
    hipLaunchKernelGGL((grouped_gemm_kernel<1, false>), dim3((unsigned)blocks), dim3(NT), 0, st, (const u16*)h, offsets,
                       sorted_pairs, tiles, n_tiles, (const u16*)Wd, nullptr, topk_w, s.K, y_perm, s.I, s.d,
                       n_nb, (int)(s.T * s.K));
}

// Dense SwiGLU MLP (one expert, all T tokens in order): h = bf16(silu(x . Wg^T) * (x . Wu^T)),
// then y = h . Wd^T in FP32.
void launch_dense_swiglu(int64_t T, int d, int I, const void* x, const void* Wg, const void* Wu, void* h,
                         hipStream_t st) {
    const int n_nb = (I + GN / 2 - 1) / (GN / 2);
    const int items = (int)((T + GM - 1) / GM) * n_nb;
    hipLaunchKernelGGL((grouped_gemm_kernel<0, true>), dim3((unsigned)((items + 7) / 8 * 8)), dim3(NT), 0, st,
                       (const u16*)x, nullptr, nullptr, nullptr, nullptr, (const u16*)Wg, (const u16*)Wu, nullptr, 1,
                       h, d, I, n_nb, (int)T);
}

void launch_dense_down(int64_t T, int d, int I, const void* h, const void* Wd, float* y, hipStream_t st) {
    const int n_nb = (d + GN - 1) / GN;
    const int items = (int)((T + GM - 1) / GM) * n_nb;
    hipLaunchKernelGGL((grouped_gemm_kernel<1, true>), dim3((unsigned)((items + 7) / 8 * 8)), dim3(NT), 0, st,
                       (const u16*)h, nullptr, nullptr, nullptr, nullptr, (const u16*)Wd, nullptr, nullptr, 1, y, I, d,
                       n_nb, (int)T);
}

bool dense_supports(int64_t T, int d, int I) {
    Shape s{};
    s.T = T; s.d = d; s.I = I; s.K = 1; s.E = 1;
    return gemm_supports(s);
}

}  // namespace beam

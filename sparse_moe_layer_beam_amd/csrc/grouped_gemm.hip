// Tiled grouped GEMM for batches with many tokens per expert (prefill): the gate/up
// projection with SwiGLU fused in the epilogue, and the down projection with the routing
// weight fused in the epilogue. BF16 MFMA (v_mfma_f32_16x16x32_bf16), FP32 accumulation.
//
// Method: Transformers "Beam" model page (Overview: sparse MoE item, FP32 SwiGLU note;
// BeamConfig: moe_intermediate_size, hidden_act) and archdb "Beam-1.0-501B-A23B" fact
// sheet (FFN rows: SwiGLU without biases).
//
// Tile: up to 256 tokens of one expert x 256 weight rows (gate/up: 128 gate channels and
// the same 128 up channels; down: 256 output channels), k in stages of 64. Eight waves, two
// per SIMD, each a 128-token x 64-row register tile (128 FP32 accumulators per lane).
//
// Why this shape on gfx950:
//  * Both operands reach LDS through direct-to-LDS loads (global_load_lds_dwordx4): no
//    vector registers for staging and no LDS write instructions. Each load moves 8 rows x
//    128 contiguous bytes. Measured on MI355X, that shape streams L2-resident data into the
//    CUs at ~30 TB/s, while loads in the MFMA operand layout (16 rows x 64 bytes, what a
//    weights-straight-to-registers design needs) stop at ~10 TB/s, which bounded the
//    earlier versions of this kernel.
//  * A 256 x 256 tile reads 2/256 bytes of operands per flop.
//  * A stage is 256 token rows + 256 weight rows of 128 bytes. Token rows come mostly from
//    L2 and are double-buffered; weight rows come from HBM and are triple-buffered, their
//    loads issued two stages ahead (160 KB of LDS). The waits before each stage's barrier
//    are placed by hand: the barrier of __syncthreads would drain every load in flight.
//  * The direct loads write 1 KB per wave in lane order; each lane picks its source chunk
//    so that LDS row r holds global 16-byte chunk c at position c ^ (r % 8). The MFMA
//    fragment reads (16 rows x one chunk) then hit eight different positions per eight
//    lanes and stay free of bank conflicts without padding.
//  * Weights in the packed layout (beam_moe_pack_weights) arrive in MFMA fragment order:
//    each direct load copies one contiguous kilobyte (a 16-row block's 32-k step) and the
//    fragment reads index it directly, no swizzle. Same results, same speed here.
#include "common.h"
#include "kernels.h"

namespace beam {
namespace {

constexpr int GM = 256;                  // tokens per tile
constexpr int GN = 256;                  // weight rows per tile
constexpr int GK = 64;                   // k per stage
constexpr int NW = 8, NT = 64 * NW;      // waves, threads per block
constexpr int SROWS = GM + GN;           // rows per stage: tokens (loaded by waves 0-3), then weights (4-7)
constexpr int TELEMS = GM * GK;          // bf16 of one token buffer (32 KB)
constexpr int WELEMS = GN * GK;          // bf16 of one weight buffer (32 KB)
constexpr int NTB = 2, NWB = 3;          // token and weight buffers: 160 KB of LDS
constexpr int DMA = SROWS / (8 * NW);    // direct loads per wave per stage (8 rows each)
#ifndef BEAM_GEMM_KFRAG
#define BEAM_GEMM_KFRAG 2
#endif
// token fragments read from LDS ahead of their MFMAs (2: ~1% faster than 4 on MI355X, 6 and 8 slower)
constexpr int kFrag = BEAM_GEMM_KFRAG;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct loads of this wave's 64 rows of stage s into buffer buf (token waves: a token
// buffer; weight waves: a weight buffer): load i fills 1 KB of the wave's part (1 KB
// aligned), lane l writing 16 bytes at l*16; src[i] + s*step is this lane's source.
__device__ __forceinline__ void stage_load(const u16* const (&src)[DMA], int s, int step, u16* buf) {
#pragma unroll
    for (int i = 0; i < DMA; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(src[i] + s * step), (lds_void*)(buf + 8 * i * GK), 16, 0, 0);
}

// End of a stage: this wave's loads that the next stage needs have landed and its LDS reads
// are done, then every wave meets. Token waves keep nothing in flight; weight waves keep
// the loads of the stage after next (DMA instructions) in flight. Written as one asm block
// so that the compiler neither drains every load at the barrier nor moves memory
// operations across it.
__device__ __forceinline__ void stage_end(bool deep) {
    if (deep) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One stage: MFMAs of the wave's LIVE 16-token subtiles against its four 16-row weight
// subtiles, k = 64, from token buffer tb and weight buffer wb. Fragment of global k-chunk
// c (8 bf16) of a buffer row r sits at r*64 + 8*(c ^ (r % 8)); this lane's rows all have
// r % 8 == lane % 8. Packed weights arrive in fragment order instead (PK).
template <int LIVE, bool PK>
__device__ __forceinline__ void stage_mma(const u16* tb, const u16* wb, int tok0, const int (&wrow)[4], int lane,
                                          f32x4 (&acc)[8][4]) {
    const int lr = lane & 15, sw = lane & 7, c0 = lane >> 4;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int pos = ((4 * j + c0) ^ sw) * 8;
        bf16x8 w[4];
        // packed weights: 16-row block b, k-step j of the stage is the 1 KB at b*1024 + j*512,
        // already in fragment order
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = PK ? *reinterpret_cast<const bf16x8*>(wb + (wrow[q] / 16) * 1024 + j * 512 + lane * 8)
                      : *reinterpret_cast<const bf16x8*>(wb + (wrow[q] + lr) * GK + pos);
        if constexpr (LIVE > 0) {
            bf16x8 xr[kFrag];
#pragma unroll
            for (int f = 0; f < kFrag; ++f)
                if (f < LIVE) xr[f] = *reinterpret_cast<const bf16x8*>(tb + (tok0 + 16 * f + lr) * GK + pos);
#pragma unroll
            for (int i = 0; i < LIVE; ++i) {
                const bf16x8 x = xr[i % kFrag];
                if (i + kFrag < LIVE)
                    xr[i % kFrag] = *reinterpret_cast<const bf16x8*>(tb + (tok0 + 16 * (i + kFrag) + lr) * GK + pos);
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[i][q] = mfma16(w[q], x, acc[i][q]);
                // keep the read-ahead in place (the scheduler would sink it to its MFMAs)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// K loop and epilogue for a wave whose first LIVE 16-token subtiles hold real tokens.
template <int MODE, int LIVE, bool PK>
__device__ __forceinline__ void gemm_run(u16* lds, const u16* const (&src)[DMA], int nstages, int wave, int lane,
                                         int tok0, const int (&wrow)[4], int rows, size_t orow0, int c0, int Ndim,
                                         const int32_t* __restrict__ pair_of_row, const float* __restrict__ topk_w,
                                         void* __restrict__ out) {
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Token waves load stage s+1 during stage s (two token buffers); weight waves load stage
    // s+2 (three weight buffers), since weights come from HBM at its loaded latency. Every
    // wave issues the same number of loads per stage (clamped to the last stage at the end),
    // which is what the fixed wait counts in stage_end rely on.
    u16* const tbuf = lds;
    u16* const wbuf = lds + NTB * TELEMS;
    const bool weight_wave = wave >= NW / 2;
    const int part = (weight_wave ? wave - NW / 2 : wave) * 64 * GK;   // this wave's 64 rows of a buffer
    const int last = nstages - 1;
    // a wave's ring depth: the buffers of the operand it loads
    const int nb = weight_wave ? NWB : NTB;
    u16* const mine = (weight_wave ? wbuf : tbuf) + part;
    const int belems = weight_wave ? WELEMS : TELEMS;
    const bool deep = nb == 3;
    // source elements per stage: 64 k of a row-major row; packed, two 32-k steps of 512
    const int step = (PK && weight_wave) ? 1024 : GK;
    stage_load(src, 0, step, mine);
    if (deep) stage_load(src, min(1, last), step, mine + belems);
    stage_end(deep);
    for (int s = 0; s < nstages; ++s) {
        // the buffer loaded here was last read in stage s-1, which every wave has left
        const int ahead = nb - 1;
        stage_load(src, min(s + ahead, last), step, mine + ((s + ahead) % nb) * belems);
        stage_mma<LIVE, PK>(tbuf + (s % NTB) * TELEMS, wbuf + (s % NWB) * WELEMS, tok0, wrow, lane, acc);
        stage_end(deep);
    }
    // the weight waves' last (clamped, unused) loads must land before the block's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Epilogue. acc[i][q][v]: token tok0 + 16*i + lane%16 of the tile, channel
    // c0 + 16*q' + 4*(lane/16) + v with q' = q (down) or q % 2 (gate/up: q = 0,1 gate and
    // q = 2,3 up of the same channels).
    const int tcol = lane & 15, rsub = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < LIVE; ++i) {
        const int r = tok0 + 16 * i + tcol;
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

// The block's work item. Each XCD owns the contiguous range [x*per_xcd, (x+1)*per_xcd) of the
// item order and hands it out in order through its counter q[x]; a block whose XCD has spent
// its range takes the next item of the range with the most items left, so that the XCDs end
// together although their items differ in cost (tile fill). Returns -1 once every item has
// been claimed: a claim that fails means its range is spent for good, so at most nine tries
// are needed. Lane 0 of wave 0 claims; the result reaches the other waves through the first
// LDS word, before any load into LDS is issued.
__device__ __forceinline__ int claim_item(int32_t* q, int x, int per_xcd, int n_items, u16* lds) {
    int32_t* const word = reinterpret_cast<int32_t*>(lds);
    if (threadIdx.x == 0) {
        int got = -1, y = x;
        for (int tries = 0; tries < 16; ++tries) {
            const int len = min(per_xcd, n_items - y * per_xcd);
            if (len > 0) {
                const int v = atomicAdd(q + y, 1);
                if (v < len) {
                    got = y * per_xcd + v;
                    break;
                }
            }
            int most = 0;
            y = -1;
            for (int z = 0; z < 8; ++z) {
                const int left = min(per_xcd, n_items - z * per_xcd) -
                                 __hip_atomic_load(q + z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (left > most) {
                    most = left;
                    y = z;
                }
            }
            if (y < 0) break;
        }
        *word = got;
    }
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int32_t*>(word));
    __syncthreads();
    return item;
}

// MODE 0: out = h [P, I] bf16 = bf16(silu(act . Wg^T) * (act . Wu^T)), act = x rows gathered
//         through sorted_pairs (token = pair / top_k); W0 = Wg, W1 = Wu, both [E, Ndim, Kdim].
// MODE 1: out = y_perm [P, d] fp32 = w_pair * (act . Wd^T), act = h rows in sorted order;
//         W0 = Wd [E, Ndim, Kdim].
// DENSE: one expert holding all act_rows tokens in order (the dense SwiGLU MLP, the router
//         logits): no tile list, no gather, weight 1; MODE 1 then writes y [T, Ndim] directly.
//         k may be cut into kparts parts of Kdim (rows ldk long); part kb writes its partial
//         product to out + kb * act_rows * Ndim. Its items all cost
//         the same and map to blocks statically; the grouped GEMMs claim theirs (claim_item)
//         from the counters that follow the tile count in n_tiles_p.
template <int MODE, bool DENSE, bool PK>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_kernel(
        const u16* __restrict__ act, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
        const int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles_p, const u16* __restrict__ W0,
        const u16* __restrict__ W1, const float* __restrict__ topk_w, int top_k, void* __restrict__ out, int Kdim,
        int Ndim, int n_nb, int act_rows, int ldk, int kparts) {
    __shared__ __attribute__((aligned(1024))) u16 lds[NTB * TELEMS + NWB * WELEMS];

    // Work item -> (expert, n-block, m-tile). Blocks are dispatched to the 8 XCDs round-robin
    // (block b on XCD b % 8, checked on MI355X with the XCC_ID register); XCD x takes the
    // contiguous item range [x*per_xcd, (x+1)*per_xcd), expert-major, so the items sharing
    // one expert's weights and tokens run together on one XCD.
    const int n_mt_dense = (act_rows + GM - 1) / GM;
    const int n_items = DENSE ? n_mt_dense * n_nb * kparts : *n_tiles_p * n_nb;
    const int per_xcd = (n_items + 7) / 8;
    int item;
    if constexpr (DENSE) {
        const int slot = blockIdx.x >> 3;
        if (slot >= per_xcd) return;
        item = (blockIdx.x & 7) * per_xcd + slot;
        if (item >= n_items) return;
    } else {
        // The grid is sized for the largest possible tile list. A block runs one item, so an XCD
        // can take items from another only with blocks to spare: a quarter more blocks than items
        // claim (the XCDs' shares of the work differ by up to ~16% at T=8192), the rest leave at
        // once. A claim fails only once every item is claimed, so all items are taken.
        if ((int)blockIdx.x >= n_items + n_items / 4 + 64) return;
        item = claim_item(n_tiles_p + 1 + 8 * MODE, blockIdx.x & 7, per_xcd, n_items, lds);
        if (item < 0) return;
    }
    int e, local, cnt, beg, n_e, kb = 0;
    if constexpr (DENSE) {
        kb = item / (n_mt_dense * n_nb);
        e = 0;
        local = item - kb * (n_mt_dense * n_nb);
        cnt = n_mt_dense;
        beg = 0;
        n_e = act_rows;
    } else {
        const int j = item / n_nb;                 // a tile of the item's expert
        e = tiles[4 * j];
        const int first = tiles[4 * j + 2];
        cnt = tiles[4 * j + 3];
        local = item - first * n_nb;
        beg = offsets[e];
        n_e = offsets[e + 1] - beg;
    }
    // The expert's n_nb x cnt items in groups of GW n-blocks, m-tile-major inside a group, so
    // that a run of consecutive items (the blocks of one XCD running together) covers a few
    // n-blocks times a few m-tiles and shares both weight blocks and token tiles through L2.
    // Measured on MI355X: GW = 4 takes 5% off the dense MLP at T=8192, GW = 2 about 1% off
    // the grouped GEMMs; wider groups lose again.
    constexpr int GW = DENSE ? 4 : 2;
    const int grp = local / (GW * cnt);
    const int gw = min(GW, n_nb - grp * GW);
    const int in = local - grp * GW * cnt;
    const int mt = in / gw;
    const int nb = grp * GW + (in - mt * gw);
    const int m0 = mt * GM;
    const int rows = min(GM, n_e - m0);
    const int n0 = nb * (MODE == 0 ? GN / 2 : GN);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Sources of this lane's direct loads: row 64*wave + 8i + lane/8 of the stage (token rows
    // 0..255, weight rows 256..511), global chunk (lane % 8) ^ (lane / 8). Token rows past the
    // expert's segment repeat its last row; weight rows past Ndim repeat the last row.
    const u16* src[DMA];
    const int chunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
        const int row = 64 * wave + 8 * i + (lane >> 3);
        const u16* p;
        if (row < GM) {
            const int m = m0 + min(row, rows - 1);
            size_t tr;
            if constexpr (MODE == 0 && !DENSE) tr = (size_t)(sorted_pairs[beg + m] / top_k);
            else tr = (size_t)(beg + m);
            p = act + tr * ldk + (size_t)kb * Kdim;
        } else if constexpr (PK) {
            // weight wave ww loads 16-row blocks 4ww .. 4ww+3 of the tile, two 32-k steps each
            const int qb = 4 * (wave - NW / 2) + i / 2;
            int ch;
            const u16* W = W0;
            if constexpr (MODE == 0) {
                ch = n0 + 16 * (qb % (GN / 32));
                if (qb >= GN / 32) W = W1;
            } else {
                ch = n0 + 16 * qb;
            }
            const size_t blk = ((size_t)e * Ndim + min(ch, Ndim - 16)) / 16;   // past Ndim: the last block
            src[i] = W + (blk * (ldk / 32) * 64 + lane) * 8 + (size_t)kb * Kdim * 16 + (i % 2) * 512;
            continue;
        } else {
            const int wr = row - GM;
            int ch;
            const u16* W = W0;
            if constexpr (MODE == 0) {
                ch = n0 + (wr & (GN / 2 - 1));
                if (wr >= GN / 2) W = W1;
            } else {
                ch = n0 + wr;
            }
            p = W + ((size_t)e * Ndim + min(ch, Ndim - 1)) * ldk + (size_t)kb * Kdim;
        }
        src[i] = p + 8 * chunk;
    }

    // This wave's part of the tile: tokens 128*(wave % 2) .. +128, and four 16-row weight
    // subtiles (gate/up: 32 gate rows and the matching 32 up rows; down: 64 rows), as rows
    // of a weight buffer.
    const int wm = wave & 1, wn = wave >> 1;
    const int tok0 = 128 * wm;
    int wrow[4], c0;
    if constexpr (MODE == 0) {
        c0 = n0 + 32 * wn;
        wrow[0] = 32 * wn;
        wrow[1] = 32 * wn + 16;
        wrow[2] = GN / 2 + 32 * wn;
        wrow[3] = GN / 2 + 32 * wn + 16;
    } else {
        c0 = n0 + 64 * wn;
#pragma unroll
        for (int q = 0; q < 4; ++q) wrow[q] = 64 * wn + 16 * q;
    }
    const int real = rows - tok0;                   // real tokens in this wave's half (may be <= 0)
    const int live = real <= 0 ? 0 : min(8, 2 * ((real + 31) / 32));
    const int nstages = Kdim / GK;
    const size_t orow0 = (size_t)(beg + m0);
    const int32_t* pair_of_row = DENSE ? nullptr : sorted_pairs + beg + m0;
    if constexpr (MODE == 1 && DENSE) out = static_cast<float*>(out) + (size_t)kb * act_rows * Ndim;
    switch (live) {
#define BEAM_GEMM_CASE(L)                                                                                     \
    case L:                                                                                                   \
        gemm_run<MODE, L, PK>(lds, src, nstages, wave, lane, tok0, wrow, rows, orow0, c0, Ndim, pair_of_row,  \
                              topk_w, out);                                                                   \
        break;
        BEAM_GEMM_CASE(0) BEAM_GEMM_CASE(2) BEAM_GEMM_CASE(4) BEAM_GEMM_CASE(6) BEAM_GEMM_CASE(8)
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
    return s.d % (2 * GK) == 0 && s.I % (2 * GK) == 0 && s.d >= 64 && s.I >= 64;
}

void launch_gemm_swiglu(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                        const int32_t* tiles, int32_t* n_tiles, const void* Wg, const void* Wu, void* h,
                        hipStream_t st) {
    const int n_nb = (s.I + GN / 2 - 1) / (GN / 2);
    const int blocks = (max_items(s, n_nb) + 7) / 8 * 8;
#define BEAM_GU(PK)                                                                                           \
    hipLaunchKernelGGL((grouped_gemm_kernel<0, false, PK>), dim3((unsigned)blocks), dim3(NT), 0, st,           \
                       (const u16*)x, offsets, sorted_pairs, tiles, n_tiles, (const u16*)Wg, (const u16*)Wu,  \
                       nullptr, s.K, h, s.d, s.I, n_nb, (int)s.T, s.d, 1)
    if (s.packed) BEAM_GU(true); else BEAM_GU(false);
#undef BEAM_GU
}

void launch_gemm_down(const Shape& s, const void* h, const int32_t* offsets, const int32_t* sorted_pairs,
                      const float* topk_w, const int32_t* tiles, int32_t* n_tiles, const void* Wd,
                      float* y_perm, hipStream_t st) {
    const int n_nb = (s.d + GN - 1) / GN;
    const int blocks = (max_items(s, n_nb) + 7) / 8 * 8;
#define BEAM_DN(PK)                                                                                           \
    hipLaunchKernelGGL((grouped_gemm_kernel<1, false, PK>), dim3((unsigned)blocks), dim3(NT), 0, st,           \
                       (const u16*)h, offsets, sorted_pairs, tiles, n_tiles, (const u16*)Wd, nullptr, topk_w, \
                       s.K, y_perm, s.I, s.d, n_nb, (int)(s.T * s.K), s.I, 1)
    if (s.packed) BEAM_DN(true); else BEAM_DN(false);
#undef BEAM_DN
}

// Dense SwiGLU MLP (one expert, all T tokens in order): h = bf16(silu(x . Wg^T) * (x . Wu^T)),
// then y = h . Wd^T in FP32.
void launch_dense_swiglu(int64_t T, int d, int I, bool packed, const void* x, const void* Wg, const void* Wu, void* h,
                         hipStream_t st) {
    const int n_nb = (I + GN / 2 - 1) / (GN / 2);
    const int items = (int)((T + GM - 1) / GM) * n_nb;
#define BEAM_DGU(PK)                                                                                          \
    hipLaunchKernelGGL((grouped_gemm_kernel<0, true, PK>), dim3((unsigned)((items + 7) / 8 * 8)), dim3(NT), 0, st, \
                       (const u16*)x, nullptr, nullptr, nullptr, nullptr, (const u16*)Wg, (const u16*)Wu, nullptr, 1, \
                       h, d, I, n_nb, (int)T, d, 1)
    if (packed) BEAM_DGU(true); else BEAM_DGU(false);
#undef BEAM_DGU
}

void launch_dense_down(int64_t T, int d, int I, bool packed, const void* h, const void* Wd, float* y, hipStream_t st) {
    const int n_nb = (d + GN - 1) / GN;
    const int items = (int)((T + GM - 1) / GM) * n_nb;
#define BEAM_DDN(PK)                                                                                          \
    hipLaunchKernelGGL((grouped_gemm_kernel<1, true, PK>), dim3((unsigned)((items + 7) / 8 * 8)), dim3(NT), 0, st, \
                       (const u16*)h, nullptr, nullptr, nullptr, nullptr, (const u16*)Wd, nullptr, nullptr, 1, y, I, d, \
                       n_nb, (int)T, I, 1)
    if (packed) BEAM_DDN(true); else BEAM_DDN(false);
#undef BEAM_DDN
}

// Router logits on the GEMM: zp[kb][t][pl*E + e] = x_t . WrS[pl][e] over k part kb of ks, for
// the three bf16 planes pl of the split router weight ([3E, d], row-major).
void launch_gemm_router(const Shape& s, const void* x, const void* WrS, float* zp, int ks, hipStream_t st) {
    const int Ndim = 3 * s.E;
    const int n_nb = (Ndim + GN - 1) / GN;
    const int items = (int)((s.T + GM - 1) / GM) * n_nb * ks;
    hipLaunchKernelGGL((grouped_gemm_kernel<1, true, false>), dim3((unsigned)((items + 7) / 8 * 8)), dim3(NT), 0, st,
                       (const u16*)x, nullptr, nullptr, nullptr, nullptr, (const u16*)WrS, nullptr, nullptr, 1, zp,
                       s.d / ks, Ndim, n_nb, (int)s.T, s.d, ks);
}

int gemm_router_items(const Shape& s, int ks) {
    return (int)((s.T + GM - 1) / GM) * ((3 * s.E + GN - 1) / GN) * ks;
}

bool dense_supports(int64_t T, int d, int I) {
    Shape s{};
    s.T = T; s.d = d; s.I = I; s.K = 1; s.E = 1; s.route_E = 1;
    return gemm_supports(s);
}

}  // namespace beam

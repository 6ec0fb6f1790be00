// Tiled grouped GEMM for batches with many tokens per expert (prefill): the gate/up
// projection with SwiGLU fused in the epilogue, and the down projection (the combine applies
// the routing weights). BF16 MFMA (v_mfma_f32_16x16x32_bf16), FP32 accumulation.
//
// Method: Transformers "Beam" model page (Overview: sparse MoE item, FP32 SwiGLU note;
// BeamConfig: moe_intermediate_size, hidden_act) and archdb "Beam-1.0-501B-A23B" fact
// sheet (FFN rows: SwiGLU without biases).
//
// Two kernels: grouped_gemm_kernel (below; row-major weights, and shapes the second does not
// take) stages both operands through LDS; grouped_gemm_ws_kernel (further below; packed weights)
// streams the weights into registers. The first one's tile: up to 256 tokens of one expert x
// 256 weight rows (gate/up: 128 gate channels and the same 128 up channels; down: 256 output
// channels), k in stages of 64. Eight waves, two per SIMD, each a 128-token x 64-row register
// tile (128 FP32 accumulators per lane).
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
//
// Packed weights whose k runs are multiples of 512 take a second kernel instead
// (grouped_gemm_ws_kernel, below): the same items and arithmetic, weights streamed from
// memory straight into registers and only the tokens staged in LDS.
#include <atomic>

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
// token fragments read from LDS ahead of their MFMAs (2: ~1% faster than 4 on MI355X, 6 and 8 slower)
constexpr int kFrag = 2;

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
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ch = c0 + 16 * q + rsub;
                if (ch >= Ndim) continue;
                *reinterpret_cast<float4*>(y + orow * Ndim + ch) =
                    make_float4(acc[i][q][0], acc[i][q][1], acc[i][q][2], acc[i][q][3]);
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
    // an LDS-typed pointer: ds instructions (a volatile access through a generic pointer would be a
    // flat one, whose wait also counts every global load and store in flight)
    __attribute__((address_space(3))) volatile int32_t* const word =
        (__attribute__((address_space(3))) volatile int32_t*)(lds);
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
    const int item = __builtin_amdgcn_readfirstlane(*word);
    __syncthreads();
    return item;
}

// MODE 0: out = h [P, I] bf16 = bf16(silu(act . Wg^T) * (act . Wu^T)), act = x rows gathered
//         through sorted_pairs (token = pair / top_k); W0 = Wg, W1 = Wu, both [E, Ndim, Kdim].
// MODE 1: out = y_perm [P, d] fp32 = act . Wd^T, act = h rows in sorted order;
//         W0 = Wd [E, Ndim, Kdim].
// DENSE: one expert holding all act_rows tokens in order (the dense SwiGLU MLP, the router
//         logits): no tile list, no gather; MODE 1 then writes y [T, Ndim] directly.
//         k may be cut into kparts parts of Kdim (rows ldk long); part kb writes its partial
//         product to out + kb * act_rows * Ndim. Its items all cost
//         the same and map to blocks statically; the grouped GEMMs claim theirs (claim_item)
//         from the counters that follow the tile count in n_tiles_p.
template <int MODE, bool DENSE, bool PK>
__global__ __launch_bounds__(NT, 1) void grouped_gemm_kernel(
        const u16* __restrict__ act, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs,
        const int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles_p, const u16* __restrict__ W0,
        const u16* __restrict__ W1, int top_k, void* __restrict__ out, int Kdim,
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
    if constexpr (MODE == 1 && DENSE) out = static_cast<float*>(out) + (size_t)kb * act_rows * Ndim;
    switch (live) {
#define BEAM_GEMM_CASE(L)                                                                                     \
    case L:                                                                                                   \
        gemm_run<MODE, L, PK>(lds, src, nstages, wave, lane, tok0, wrow, rows, orow0, c0, Ndim, out);          \
        break;
        BEAM_GEMM_CASE(0) BEAM_GEMM_CASE(2) BEAM_GEMM_CASE(4) BEAM_GEMM_CASE(6) BEAM_GEMM_CASE(8)
#undef BEAM_GEMM_CASE
    }
}

// ---- packed weights: weights streamed into registers, tokens through LDS --------------------
//
// The same kind of work items as grouped_gemm_kernel (an expert's m-tile of up to 320 tokens, or
// 256 when the other expert GEMM runs grouped_gemm_kernel, or the dense MLP's m-tiles, x an n-block
// of 256 weight rows), the same arithmetic (16x16x32 bf16 MFMAs over k in order into FP32
// accumulators, the same epilogues), organised for packed weights:
//  * eight waves, two per SIMD: wave w owns two 16-row weight blocks (gate/up: the gate rows and
//    the up rows of channels n0 + 16 w .. +16; down: output channels n0 + 32 w .. +32) against
//    every live token of the tile: up to 20 x 2 x 4 = 160 FP32 accumulators per lane.
//  * each wave loads its weight fragments from memory straight into a ring of registers, WRW
//    stages ahead; in the packed layout every fragment is one contiguous kilobyte. Each weight
//    byte crosses the CU's vector memory path once: a stage moves 32 KB of weights and 32 KB of
//    tokens through it. That path delivers about 64 bytes per clock per CU (measured on MI355X
//    with L1-resident data), against 2048 MFMA clocks per full stage.
//  * only the tokens pass through LDS: the eight waves load the live rows (direct-to-LDS, WDT
//    stages ahead, the XOR swizzle of the kernel above) and every wave reads all of them: 256 KB
//    of fragment reads per full stage, which LDS serves at about 200 bytes per clock.
//  * every load is a buffer load (a per-lane offset fixed for the item, the stage in a scalar
//    offset) and runs on every path, so the compiler counts its own waits on the ring precisely.
//  * the grouped launches are persistent: one block per CU walks its XCD's items. The next item
//    is claimed one loop iteration before the current one ends (an atomic whose result is read
//    only after the k loop), and the next item starts right after the current item's epilogue
//    stores are issued, with no block launch and no claim latency in between. On MI355X, against
//    one block per item (same box, alternating builds, results bitwise the same): T=8192 layer
//    6.01 -> 5.89 ms (gate/up 3.52-3.55 -> 3.39-3.46 ms), T=4096 skewed 3.85-3.99 -> 3.80-3.82,
//    T=32768 18.73-18.80 -> 18.51-18.67. Issuing the next item's token loads before the stores
//    (so that the stores drain under its first stages) measured 13% slower for gate/up: with the
//    prologue's loads out of the steady state's order the compiler's waits on the weight ring
//    tighten in every stage.
constexpr int WM = 320;                   // tokens per tile at most
constexpr int WK = 64;                    // k per stage
constexpr int WNW = 8;                    // waves per block
constexpr int WTB = WM * WK;              // bf16 of one token buffer (40 KB)
constexpr int WNB = 4;                    // token buffers
constexpr int WDT = WNB - 1;              // token stages loaded ahead
// Token fragments read from LDS ahead of their MFMAs: four, but two in the down GEMM's 20-subtile
// tiles. With four there the allocator spilled 6 VGPRs, and each reload inside the k loop waited
// for vmcnt(0): every token and weight load in flight, twice per eight stages. With two the
// kernel has no scratch. On MI355X: down 2.12 -> 2.07-2.08 ms at T=8192, 6.59 -> 6.42 ms at
// T=32768, bitwise the same (only the read-ahead changes).
template <int MODE, int LH>
constexpr int ws_pf() {
    return MODE == 1 && LH >= 20 ? 2 : 4;
}
constexpr int WUN = 8;                    // stages per loop iteration (divides the stage count)
constexpr int kRsrcWord3 = 0x00020000;    // raw buffer, 32-bit data format (gfx9 V# word 3)

// Waits until this wave's loads older than its N most recent have landed (the token loads of the
// stage about to start among them) and its LDS reads are done, then meets the other waves.
template <int N>
__device__ __forceinline__ void ws_stage_wait() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Keeps memory operations in program order on both sides of it, for the optimizer (the memory
// clobber) and for the machine scheduler.
__device__ __forceinline__ void ws_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Claim state of a persistent launch: the per-XCD counters, this block's XCD and the item split.
struct ClaimQ {
    int32_t* q;
    int x, per_xcd, n_items;
};

// One claim from the block's own XCD range, issued ahead: the counter's old value. The caller
// reads it only after the k loop (claim_next), so no wait for it lands inside the loop. The
// address goes through a VGPR: for a uniform address the compiler would reduce the atomic over
// the wave and broadcast its result at once, waiting for it (and every load before it) there.
__device__ __forceinline__ int claim_own_raw(const ClaimQ& c) {
    int z = 0;
    asm volatile("" : "+v"(z));
    return atomicAdd(c.q + c.x + z, 1);
}

// The item that claim's counter value names, or -2 if the range was spent (for good).
__device__ __forceinline__ int claim_own_item(const ClaimQ& c, int v) {
    const int len = min(c.per_xcd, c.n_items - c.x * c.per_xcd);
    return v < len ? c.x * c.per_xcd + v : -2;
}

typedef __attribute__((address_space(3))) int32_t lds_i32;

// After an item: lane 0 of wave 0 holds the item claimed ahead (claim_own_item of claim_own_raw's
// value, resolved before the epilogue stores are issued); a spent range (-2) sends it to the other
// XCDs' ranges as in claim_item. The item reaches every wave through the first LDS word: the waves
// have finished reading the token buffers (first barrier) and read the word before any wave loads
// into LDS again (last barrier). The word is accessed through an LDS pointer (ds instructions,
// counted by lgkmcnt) and the barriers wait for LDS work only, so the epilogue stores issued before
// them keep draining: a volatile access through a generic pointer compiles to a flat access, and
// the wait for it (vmcnt(0)) would wait for every store.
__device__ __forceinline__ int claim_next(const ClaimQ& c, int got, u16* lds) {
    lds_i32* const word = (lds_i32*)(lds);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (threadIdx.x == 0) {
        if (got == -2) {
            got = -1;
            for (int tries = 0; tries < 16; ++tries) {
                int most = 0, y = -1;
                for (int z = 0; z < 8; ++z) {
                    const int left = min(c.per_xcd, c.n_items - z * c.per_xcd) -
                                     __hip_atomic_load(c.q + z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (left > most) {
                        most = left;
                        y = z;
                    }
                }
                if (y < 0) break;
                const int len = min(c.per_xcd, c.n_items - y * c.per_xcd);
                const int v = atomicAdd(c.q + y, 1);
                if (v < len) {
                    got = y * c.per_xcd + v;
                    break;
                }
            }
        }
        *word = got;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int item = __builtin_amdgcn_readfirstlane(*word);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    return item;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Direct loads per wave per stage for LH live 16-token subtiles: 2 LH groups of 8 rows over
// eight waves, the count rounded up (the spare loads repeat live rows into unread LDS rows).
template <int LH>
constexpr int ws_nt() {
    return (2 * LH + WNW - 1) / WNW;
}

// Weight stages held in registers: four (64 VGPRs) up to 14 live subtiles; from 16 (128 FP32
// accumulators) four would spill, so two.
template <int LH>
constexpr int ws_rw() {
    return LH <= 14 ? 4 : 2;
}

// K loop and epilogue of one wave of a tile with LH live 16-token subtiles (even, 2..20).
template <int MODE, int LH, int NTT>
__device__ __forceinline__ void ws_run(u16* lds, __amdgpu_buffer_rsrc_t trs, const uint32_t (&toff)[NTT],
                                       const __amdgpu_buffer_rsrc_t (&wrs)[2], int nstages, int wave, int lane,
                                       int rows, size_t orow0, const int (&chq)[2], int Ndim,
                                       void* __restrict__ out, const ClaimQ& cq, int& next) {
    constexpr int NT = ws_nt<LH>();           // token loads per stage
    static_assert(NTT == NT, "one token offset per token load");
    constexpr int NWL = 4;                    // weight loads per stage: 2 blocks x 2 k-halves
    constexpr int WRW = ws_rw<LH>();
    // loads issued after a stage's token loads, up to that stage: the weight refill issued with
    // them, then WDT - 1 further stages of token loads and weight refills
    constexpr int WAIT = NWL + (WDT - 1) * (NT + NWL);
    static_assert(WAIT <= 63, "vmcnt range");
    static_assert(WUN % WRW == 0, "ring slots repeat with the unrolled loop");
    // after the prologue, the loads issued after stage 0's token loads
    constexpr int WAIT0 = (WDT - 1) * NT + (WRW < WDT ? WRW : WDT) * NWL;
    constexpr int PRO = WRW > WDT ? WRW : WDT;
    f32x4 acc[LH][2];
#pragma unroll
    for (int i = 0; i < LH; ++i)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[i][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 wr[WRW][2][2];
    const int last = nstages - 1;
    const int lr = lane & 15, sw = lane & 7, c0 = lane >> 4;

    auto tload = [&](int s) {
        const int sc = min(s, last);
        u16* const buf = lds + (s % WNB) * WTB;
#pragma unroll
        for (int i = 0; i < NT; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(trs, (lds_void*)(buf + 8 * (WNW * i + wave) * WK), 16, toff[i],
                                                     sc * (WK * 2), 0, 0);
    };
    auto wload = [&](int s, int slot) {
        const int sc = min(s, last);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                wr[slot][q][j] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wrs[q], (uint32_t)lane * 16, (2 * sc + j) * 1024, 0));
    };

    // prologue, in the steady state's order: the loads of stages 0 .. PRO - 1 that run ahead
#pragma unroll
    for (int u = -PRO; u < 0; ++u) {
        if (u + WDT >= 0) tload(u + WDT);
        ws_fence();
        if (u + WRW >= 0) wload(u + WRW, u + WRW);
        ws_fence();
    }
    // fewer loads follow stage 0's tokens here than in the steady state: wait for them now
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WAIT0) : "memory");
    for (int s0 = 0; s0 < nstages; s0 += WUN) {
        // the next item's first claim, one loop iteration (WUN stages) before this item ends; an
        // extra load in flight only makes the counted waits below wait for more, never less
        if (cq.q && s0 + WUN >= nstages && threadIdx.x == 0) next = claim_own_raw(cq);
#pragma unroll
        for (int r = 0; r < WUN; ++r) {
            const int s = s0 + r;
            ws_stage_wait<WAIT>();
            // the buffer loaded here, (s + WDT) % WNB = (s - 1) % WNB, was last read in stage s - 1
            tload(s + WDT);
            ws_fence();
            const u16* const tb = lds + (s % WNB) * WTB;
            constexpr int WPF = ws_pf<MODE, LH>();
            bf16x8 xr[WPF];
#pragma unroll
            for (int f = 0; f < WPF; ++f)
                xr[f] = *reinterpret_cast<const bf16x8*>(tb + (16 * (f % LH) + lr) * WK + ((4 * (f / LH) + c0) ^ sw) * 8);
#pragma unroll
            for (int f = 0; f < 2 * LH; ++f) {
                const int i = f % LH, j = f / LH;
                const bf16x8 x = xr[f % WPF];
                const int g = f + WPF;
                if (g < 2 * LH)
                    xr[f % WPF] = *reinterpret_cast<const bf16x8*>(tb + (16 * (g % LH) + lr) * WK +
                                                                   ((4 * (g / LH) + c0) ^ sw) * 8);
#pragma unroll
                for (int q = 0; q < 2; ++q) acc[i][q] = mfma16(wr[r % WRW][q][j], x, acc[i][q]);
                ws_fence();
            }
            // slot r % WRW is free: the weights of stage s + WRW go there
            wload(s + WRW, r % WRW);
            ws_fence();
        }
    }
    // the last (clamped, unused) loads must land before the block's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // the claim made ahead has returned too: read it now, before any store is in flight
    if (cq.q && threadIdx.x == 0) next = claim_own_item(cq, next);

    // Epilogue. acc[i][q][v]: token 16*i + lane%16 of the tile, channel chq[q] + 4*(lane/16) + v
    // (gate/up: q = 0 gate and q = 1 up of the same channels).
    const int rsub = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < LH; ++i) {
        const int rr = 16 * i + lr;
        if (rr >= rows) continue;
        const size_t orow = orow0 + rr;
        if constexpr (MODE == 0) {
            u16* h = reinterpret_cast<u16*>(out);
            const int ch = chq[0] + rsub;
            if (ch >= Ndim) continue;
            const uint32_t lo = (uint32_t)f32_to_bf16(silu_mul(acc[i][0][0], acc[i][1][0])) |
                                ((uint32_t)f32_to_bf16(silu_mul(acc[i][0][1], acc[i][1][1])) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(silu_mul(acc[i][0][2], acc[i][1][2])) |
                                ((uint32_t)f32_to_bf16(silu_mul(acc[i][0][3], acc[i][1][3])) << 16);
            *reinterpret_cast<uint2*>(h + orow * Ndim + ch) = make_uint2(lo, hi);
        } else {
            float* y = reinterpret_cast<float*>(out);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int ch = chq[q] + rsub;
                if (ch >= Ndim) continue;
                *reinterpret_cast<float4*>(y + orow * Ndim + ch) =
                    make_float4(acc[i][q][0], acc[i][q][1], acc[i][q][2], acc[i][q][3]);
            }
        }
    }
}

template <int MODE, int LH>
__device__ __forceinline__ void ws_item(u16* lds, const u16* __restrict__ act, uint32_t act_bytes,
                                        const int32_t* __restrict__ sorted_pairs, int top_k, int beg, int m0, int rows,
                                        int e, int n0, const u16* W0, const u16* W1,
                                        void* __restrict__ out, int Kdim, int Ndim, int wave, int lane,
                                        const ClaimQ& cq, int& next) {
    // token offsets: load i of this wave covers rows 8(8i + wave) .. +8 of the tile, lane row
    // + lane/8, global chunk (lane % 8) ^ (lane / 8); rows past the expert's segment repeat its last
    constexpr int NT = ws_nt<LH>();
    uint32_t toff[NT];
    const int chunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int m = m0 + min(8 * (WNW * i + wave) + (lane >> 3), rows - 1);
        uint32_t tr;
        // gate/up gathers the tokens of its pairs; the dense MLP (no sorted_pairs) takes them in order
        if (MODE == 0 && sorted_pairs) tr = (uint32_t)(sorted_pairs[beg + m] / top_k);
        else tr = (uint32_t)(beg + m);
        toff[i] = (tr * (uint32_t)Kdim + 8u * chunk) * 2u;
    }
    const __amdgpu_buffer_rsrc_t trs = ws_rsrc(act, act_bytes);
    // weight blocks: this wave's two 16-row blocks (gate/up: the gate and the up rows of 16
    // channels; down: 32 output channels), each a resource of Kdim * 16 bf16; a block past Ndim
    // reads the last block (discarded)
    __amdgpu_buffer_rsrc_t wrs[2];
    int chq[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const u16* W = W0;
        int ch;
        if constexpr (MODE == 0) {
            ch = n0 + 16 * wave;
            if (q == 1) W = W1;
        } else {
            ch = n0 + 32 * wave + 16 * q;
        }
        chq[q] = ch;
        const size_t blk = ((size_t)e * Ndim + min(ch, Ndim - 16)) / 16;
        wrs[q] = ws_rsrc(W + blk * (size_t)Kdim * 16, (uint32_t)Kdim * 32u);
    }
    ws_run<MODE, LH>(lds, trs, toff, wrs, Kdim / WK, wave, lane, rows, (size_t)(beg + m0), chq, Ndim, out, cq, next);
}

// MODE 0: out = h [P, I] bf16 = bf16(silu(act . Wg^T) * (act . Wu^T)), act = x rows gathered
//         through sorted_pairs; W0 = Wg, W1 = Wu, packed [E*Ndim, Kdim].
// MODE 1: out = y_perm [P, d] fp32 = act . Wd^T, act = h rows in sorted order; W0 = Wd.
// act_bytes: the size of act (below 4 GiB: buffer offsets are 32-bit); Kdim a multiple of 512.
// Work items and their claim as in grouped_gemm_kernel (the tile list of the dispatch).
// DENSE: one expert holding all act_rows tokens in order (the dense SwiGLU MLP): items from
// act_rows directly, statically mapped XCD by XCD, no gather; MODE 1 then writes y [T, Ndim].
template <int MODE, bool DENSE>
__global__ __launch_bounds__(64 * WNW, 1) void grouped_gemm_ws_kernel(
        const u16* __restrict__ act, uint32_t act_bytes, const int32_t* __restrict__ offsets,
        const int32_t* __restrict__ sorted_pairs, const int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles_p,
        // no __restrict__: loads through restrict-qualified read-only pointers are free to move past
        // the fences that keep the weight and token loads in the order the waits count on
        const u16* W0, const u16* W1, int top_k, void* __restrict__ out, int Kdim,
        int Ndim, int n_nb, int tile_m, int act_rows) {
    __shared__ __attribute__((aligned(1024))) u16 lds[WNB * WTB];
    // one work item: an expert's m-tile x n-block (see below)
    auto run_item = [&](int e, int beg, int n_e, int cnt, int local, const ClaimQ& cq, int& next) {
        // the expert's n_nb x cnt items in groups of four n-blocks, m-tile-major inside a group (on
        // MI355X, against groups of two: T=8192 layer 6.32 -> 6.15 ms, T=32768 19.9 -> 19.75; eight: 6.26)
        constexpr int GW = 4;
        const int grp = local / (GW * cnt);
        const int gw = min(GW, n_nb - grp * GW);
        const int in = local - grp * GW * cnt;
        const int mt = in / gw;
        const int nb = grp * GW + (in - mt * gw);
        const int m0 = mt * tile_m;
        const int rows = min(tile_m, n_e - m0);
        const int n0 = nb * (MODE == 0 ? 128 : 256);
        // opaque per item, so that the compiler does not hoist the lane-derived addresses of all
        // ten tile forms out of the item loop (they would stay live across it and spill)
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        // live 16-token subtiles, in pairs
        const int lh = min(WM / 16, 2 * ((rows + 31) / 32));
        switch (lh) {
#define BEAM_WS_CASE(L)                                                                                         \
    case L:                                                                                                     \
        ws_item<MODE, L>(lds, act, act_bytes, sorted_pairs, top_k, beg, m0, rows, e, n0, W0, W1, out,          \
                         Kdim, Ndim, wave, lane, cq, next);                                                     \
        break;
            BEAM_WS_CASE(2) BEAM_WS_CASE(4) BEAM_WS_CASE(6) BEAM_WS_CASE(8)
            BEAM_WS_CASE(10) BEAM_WS_CASE(12) BEAM_WS_CASE(14) BEAM_WS_CASE(16) BEAM_WS_CASE(18) BEAM_WS_CASE(20)
#undef BEAM_WS_CASE
        }
    };
    if constexpr (DENSE) {
        const int n_mt = (act_rows + tile_m - 1) / tile_m;
        const int n_items = n_mt * n_nb;
        const int per_xcd = (n_items + 7) / 8;
        const int slot = blockIdx.x >> 3;
        if (slot >= per_xcd) return;
        const int local = (blockIdx.x & 7) * per_xcd + slot;
        if (local >= n_items) return;
        const ClaimQ none{nullptr, 0, 0, 0};
        int unused = -1;
        run_item(0, 0, act_rows, n_mt, local, none, unused);
    } else {
        // persistent: one block per CU walks items until every item is claimed; the claim of the
        // next item is made before the current one ends, and each item's epilogue stores drain
        // while the next item's loads start
        const int n_items = *n_tiles_p * n_nb;
        const ClaimQ cq{n_tiles_p + 1 + 8 * MODE, (int)(blockIdx.x & 7), (n_items + 7) / 8, n_items};
        int item = claim_item(cq.q, cq.x, cq.per_xcd, n_items, lds);
        while (item >= 0) {
            const int j = item / n_nb;
            const int e = tiles[4 * j];
            const int first = tiles[4 * j + 2];
            const int cnt = tiles[4 * j + 3];
            const int beg = offsets[e];
            int next = 0x7fffffff;    // the claim made ahead: a counter value (none: spent)
            run_item(e, beg, offsets[e + 1] - beg, cnt, item - first * n_nb, cq, next);
            item = claim_next(cq, next, lds);
        }
    }
}

// The weight-streaming form takes packed weights, stage counts that are multiples of WUN and
// activations that 32-bit buffer offsets reach.
bool ws_supports(const Shape& s, int Kdim, uint64_t act_bytes) {
    return s.packed && Kdim % (WK * WUN) == 0 && act_bytes < ((uint64_t)1 << 32);
}

// Blocks of a persistent weight-streaming launch: one per CU of the current device (a multiple of
// the 8 XCDs, so that every XCD's range has its share of blocks), looked up once per device.
int ws_grid() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
        cus = cus / 8 * 8;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

int max_items(const Shape& s, int n_nb, int tile_m) {
    const int64_t P = s.T * s.K;
    const int64_t max_tiles = (P + tile_m - 1) / tile_m + s.E;
    return (int)(max_tiles * n_nb);
}

// Both expert GEMMs in the weight-streaming form: the dispatch cuts each expert's tokens into
// tiles of WM. An expert's tile re-reads its weight slice, and the tokens per expert spread
// widely around T*K/E, so fewer, larger tiles save weight traffic: at T=8192 (256 experts,
// 2..745 tokens each) 414 tiles of 256 tokens against 363 of 320, which ran the gate/up GEMM
// in 3.61-3.65 ms against 3.68 on MI355X, bitwise the same. 320 is what the registers allow:
// 160 accumulators and a 2-stage weight ring come to 250 VGPRs.
bool ws_both(const Shape& s) {
    return ws_supports(s, s.d, (uint64_t)s.T * s.d * 2) && ws_supports(s, s.I, (uint64_t)s.T * s.K * s.I * 2);
}

}  // namespace

int gemm_tile_m(const Shape& s) { return ws_both(s) ? WM : GM; }

bool gemm_supports(const Shape& s) {
    return s.d % (2 * GK) == 0 && s.I % (2 * GK) == 0 && s.d >= 64 && s.I >= 64;
}

void launch_gemm_swiglu(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                        const int32_t* tiles, int32_t* n_tiles, const void* Wg, const void* Wu, void* h,
                        hipStream_t st) {
    const int n_nb = (s.I + GN / 2 - 1) / (GN / 2);
    const int tile_m = gemm_tile_m(s);
    const int blocks = (max_items(s, n_nb, tile_m) + 7) / 8 * 8;
    const uint64_t x_bytes = (uint64_t)s.T * s.d * 2;
    if (ws_supports(s, s.d, x_bytes)) {
        hipLaunchKernelGGL((grouped_gemm_ws_kernel<0, false>), dim3((unsigned)std::min(blocks, ws_grid())),
                           dim3(64 * WNW), 0, st,
                           (const u16*)x, (uint32_t)x_bytes, offsets, sorted_pairs, tiles, n_tiles, (const u16*)Wg,
                           (const u16*)Wu, s.K, h, s.d, s.I, n_nb, tile_m, 0);
        return;
    }
#define BEAM_GU(PK)                                                                                           \
    hipLaunchKernelGGL((grouped_gemm_kernel<0, false, PK>), dim3((unsigned)blocks), dim3(NT), 0, st,           \
                       (const u16*)x, offsets, sorted_pairs, tiles, n_tiles, (const u16*)Wg, (const u16*)Wu,  \
                       s.K, h, s.d, s.I, n_nb, (int)s.T, s.d, 1)
    if (s.packed) BEAM_GU(true); else BEAM_GU(false);
#undef BEAM_GU
}

void launch_gemm_down(const Shape& s, const void* h, const int32_t* offsets, const int32_t* sorted_pairs,
                      const int32_t* tiles, int32_t* n_tiles, const void* Wd,
                      float* y_perm, hipStream_t st) {
    const int n_nb = (s.d + GN - 1) / GN;
    const int tile_m = gemm_tile_m(s);
    const int blocks = (max_items(s, n_nb, tile_m) + 7) / 8 * 8;
    const uint64_t h_bytes = (uint64_t)s.T * s.K * s.I * 2;
    if (ws_supports(s, s.I, h_bytes)) {
        hipLaunchKernelGGL((grouped_gemm_ws_kernel<1, false>), dim3((unsigned)std::min(blocks, ws_grid())),
                           dim3(64 * WNW), 0, st,
                           (const u16*)h, (uint32_t)h_bytes, offsets, sorted_pairs, tiles, n_tiles, (const u16*)Wd,
                           nullptr, s.K, y_perm, s.I, s.d, n_nb, tile_m, 0);
        return;
    }
#define BEAM_DN(PK)                                                                                           \
    hipLaunchKernelGGL((grouped_gemm_kernel<1, false, PK>), dim3((unsigned)blocks), dim3(NT), 0, st,           \
                       (const u16*)h, offsets, sorted_pairs, tiles, n_tiles, (const u16*)Wd, nullptr, \
                       s.K, y_perm, s.I, s.d, n_nb, (int)(s.T * s.K), s.I, 1)
    if (s.packed) BEAM_DN(true); else BEAM_DN(false);
#undef BEAM_DN
}

// Dense SwiGLU MLP (one expert, all T tokens in order): h = bf16(silu(x . Wg^T) * (x . Wu^T)),
// then y = h . Wd^T in FP32.
void launch_dense_swiglu(int64_t T, int d, int I, bool packed, const void* x, const void* Wg, const void* Wu, void* h,
                         hipStream_t st) {
    const int n_nb = (I + GN / 2 - 1) / (GN / 2);
    const uint64_t x_bytes = (uint64_t)T * d * 2;
    if (packed && d % (WK * WUN) == 0 && x_bytes < ((uint64_t)1 << 32)) {
        const int ws_items = (int)((T + WM - 1) / WM) * n_nb;
        hipLaunchKernelGGL((grouped_gemm_ws_kernel<0, true>), dim3((unsigned)((ws_items + 7) / 8 * 8)),
                           dim3(64 * WNW), 0, st, (const u16*)x, (uint32_t)x_bytes, nullptr, nullptr, nullptr,
                           nullptr, (const u16*)Wg, (const u16*)Wu, 1, h, d, I, n_nb, WM, (int)T);
        return;
    }
    const int items = (int)((T + GM - 1) / GM) * n_nb;
#define BEAM_DGU(PK)                                                                                          \
    hipLaunchKernelGGL((grouped_gemm_kernel<0, true, PK>), dim3((unsigned)((items + 7) / 8 * 8)), dim3(NT), 0, st, \
                       (const u16*)x, nullptr, nullptr, nullptr, nullptr, (const u16*)Wg, (const u16*)Wu, 1,       \
                       h, d, I, n_nb, (int)T, d, 1)
    if (packed) BEAM_DGU(true); else BEAM_DGU(false);
#undef BEAM_DGU
}

void launch_dense_down(int64_t T, int d, int I, bool packed, const void* h, const void* Wd, float* y, hipStream_t st) {
    const int n_nb = (d + GN - 1) / GN;
    const uint64_t h_bytes = (uint64_t)T * I * 2;
    if (packed && I % (WK * WUN) == 0 && h_bytes < ((uint64_t)1 << 32)) {
        const int ws_items = (int)((T + GM - 1) / GM) * n_nb;
        hipLaunchKernelGGL((grouped_gemm_ws_kernel<1, true>), dim3((unsigned)((ws_items + 7) / 8 * 8)),
                           dim3(64 * WNW), 0, st, (const u16*)h, (uint32_t)h_bytes, nullptr, nullptr, nullptr,
                           nullptr, (const u16*)Wd, nullptr, 1, y, I, d, n_nb, GM, (int)T);
        return;
    }
    const int items = (int)((T + GM - 1) / GM) * n_nb;
#define BEAM_DDN(PK)                                                                                          \
    hipLaunchKernelGGL((grouped_gemm_kernel<1, true, PK>), dim3((unsigned)((items + 7) / 8 * 8)), dim3(NT), 0, st, \
                       (const u16*)h, nullptr, nullptr, nullptr, nullptr, (const u16*)Wd, nullptr, 1, y, I, d,          \
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
                       (const u16*)x, nullptr, nullptr, nullptr, nullptr, (const u16*)WrS, nullptr, 1, zp,
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

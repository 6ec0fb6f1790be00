// Routed experts of the Beam MoE layer: grouped SwiGLU (gate/up) GEMM with the
// activation fused, grouped down-projection GEMM (unweighted rows), and a deterministic
// combine that applies the routing weights. BF16 MFMA with FP32 accumulation; silu(g)*u in FP32; h is
// rounded to bf16 once, for the bf16 down GEMM.
//
// Method: Transformers "Beam" model page (Overview: sparse MoE item, FP32 SwiGLU note;
// BeamConfig: hidden_act silu, moe_intermediate_size) and archdb "Beam-1.0-501B-A23B"
// fact sheet (FFN rows: SwiGLU, no FFN biases; MoE rows: no shared expert, scaled sum).
//
// Weight-streaming form: the expert weights are the MFMA A operand (16 output channels x
// 32 k per v_mfma_f32_16x16x32_bf16) loaded straight from HBM into registers, the tokens
// of the expert are the B operand (16 tokens per tile). Each weight byte is read once per
// 16 tokens of its expert, which is once per call whenever an expert has <= 16 tokens.
//
// Weights come row-major ([E, I, d] gate/up, [E, d, I] down) or in the packed layout of
// beam_moe_pack_weights: 16-row blocks stored as runs of 32-k steps, each step the 1 KB a
// wave loads (lane l: row l % 16, k 8(l / 16) .. +8). Row-major, one load instruction reads
// 64 bytes from each of 16 rows; packed, it reads 1 KB that is contiguous and that nothing else
// in the call reads, so it takes the non-temporal hint, and the stream runs at 6.8-7.0 TB/s
// instead of 5.6 on MI355X (same values, bitwise-equal results).
//
// Also here: the packing kernel itself, and the dense SwiGLU MLP for decode-sized batches
// (Transformers "Beam" page, Overview: the first 3 layers use a dense MLP), which streams its
// weights the same way against packed 16-token tiles.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace beam {
namespace {

// Tuning of the weight streams, chosen by measurement on MI355X (the sweeps are summarized beside
// each kernel below).
constexpr int kGuDepth = 6;             // gate/up: k-steps of 32 prefetched ahead of the MFMAs
constexpr int kDnDepth = 6;             // down: the same
constexpr int kGuOcc = 3;               // gate/up: blocks of 4 waves per CU the registers must allow
constexpr int kDnOcc = 3;               // down: the same
constexpr int kStreamMT = 1;            // 16-token tiles per pass over an expert's weights
constexpr int kGuKsplit = 4;            // gate/up: waves sharing one 16-channel group, each a part of k
constexpr int kDnKsplit = 2;            // down: the same

constexpr int kWavesPerBlock = 4;
// a block's waves cover whole k-split groups
static_assert(kGuKsplit >= 1 && kWavesPerBlock % kGuKsplit == 0, "gate/up k split must divide 4 waves");
static_assert(kDnKsplit >= 1 && kWavesPerBlock % kDnKsplit == 0, "down k split must divide 4 waves");
constexpr int kDgu = kGuDepth;
constexpr int kDdn = kDnDepth;
constexpr int kMT = kStreamMT;
// Weight elements per unit of k: 1 row-major, 16 packed (a 32-k step of a 16-row block is 512
// contiguous elements).
template <bool PK>
constexpr int kWStep = PK ? 16 : 1;

__device__ __forceinline__ bf16x8 ld8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }
// Weight fragments. Packed, each load reads a whole kilobyte that nothing else reads in the
// call: the non-temporal hint (decode 2.29 -> 2.02-2.09 ms on MI355X). Row-major, a load reads
// 64 bytes of each of 16 rows and the next k-step the other half of the same 128-byte lines,
// which the hint would evict in between (measured 2.67 -> 3.4-3.5 ms): plain loads.
template <bool PK>
__device__ __forceinline__ bf16x8 ld8w(const u16* p) {
    if constexpr (PK) return __builtin_bit_cast(bf16x8, ld_once(p));
    else return ld8(p);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc[m][r] += A_r . B_m^T over k in [0, K): A_r = 16 weight rows (lane: row r16, k-chunk kq),
// B_m = 16 token rows (PK / PT: weights / token tiles in the packed layout). Weights and token fragments live in a ring of D register slots: slot s
// is consumed by its MFMAs and then refilled with the step D ahead, so every wave keeps
// D*(RB+MT) 16-byte loads in flight without register copies. Prefetch addresses past the end
// are clamped to the last step (a redundant, in-bounds load that is never consumed); the
// (K/32) % D leftover steps are taken from the ring after the main loop.
template <int RB, int MT, int D, bool PK, bool PT = false>
__device__ __forceinline__ void stream_core(const u16* const (&a)[RB], const u16* const (&b)[MT], int K,
                                            f32x4 (&acc)[MT][RB]) {
    bf16x8 wa[D][RB], xb[D][MT];
    const int last = K - 32;
    const int nsteps = K / 32;
    const int kfull = (nsteps - nsteps % D) * 32;
#pragma unroll
    for (int s = 0; s < D; ++s) {
        const int k = min(s * 32, last);
#pragma unroll
        for (int r = 0; r < RB; ++r) wa[s][r] = ld8w<PK>(a[r] + k * kWStep<PK>);
#pragma unroll
        for (int m = 0; m < MT; ++m) xb[s][m] = ld8(b[m] + k * kWStep<PT>);
    }
    for (int k0 = 0; k0 < kfull; k0 += 32 * D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < RB; ++r) acc[m][r] = mfma16(wa[s][r], xb[s][m], acc[m][r]);
            const int kn = min(k0 + (s + D) * 32, last);
#pragma unroll
            for (int r = 0; r < RB; ++r) wa[s][r] = ld8w<PK>(a[r] + kn * kWStep<PK>);
#pragma unroll
            for (int m = 0; m < MT; ++m) xb[s][m] = ld8(b[m] + kn * kWStep<PT>);
        }
    }
    const int rem = nsteps - kfull / 32;
#pragma unroll
    for (int s = 0; s < D; ++s)
        if (s < rem)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < RB; ++r) acc[m][r] = mfma16(wa[s][r], xb[s][m], acc[m][r]);
}

template <int MT>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[MT][1]) {
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m][0] = f32x4{0, 0, 0, 0};
}

// Sums the k-parts of a channel group: waves kp = 1..KS-1 of the group hand their partial
// accumulators to wave kp = 0 through LDS, which adds them in kp order (a fixed order, so
// the result does not depend on timing). Every wave of the block calls this.
template <int KS, int MT, int NA>
__device__ __forceinline__ void ksplit_reduce(f32x4 (&part)[kWavesPerBlock][NA][MT][64], int wave, int lane,
                                              f32x4 (&a)[NA][MT][1]) {
    if constexpr (KS > 1) {
        const int kp = wave % KS;
        if (kp != 0)
#pragma unroll
            for (int q = 0; q < NA; ++q)
#pragma unroll
                for (int m = 0; m < MT; ++m) part[wave][q][m][lane] = a[q][m][0];
        __syncthreads();
        if (kp == 0)
#pragma unroll
            for (int j = 1; j < KS; ++j)
#pragma unroll
                for (int q = 0; q < NA; ++q)
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const f32x4 v = part[wave + j][q][m][lane];
                        a[q][m][0] = f32x4{a[q][m][0][0] + v[0], a[q][m][0][1] + v[1], a[q][m][0][2] + v[2],
                                           a[q][m][0][3] + v[3]};
                    }
    }
}

// h[beg+m, n] = bf16(silu(x_m . Wg[e,n]) * (x_m . Wu[e,n])) for the tokens m of expert e.
// grid: (ceil(I / (16 * 4 / KS)), E); block: 4 waves. The KS waves of a 16-channel group
// each stream a 1/KS part of k for those 16 gate rows, then the 16 up rows; their sums meet
// in LDS. A wave streams one 16-row block at a time, which keeps the number of DRAM rows
// open across the chip low, which is what sets the achieved bandwidth here. Splitting k
// shortens each block, and with it the tail of the launch, where fewer and fewer blocks
// are left to keep the memory busy. Measured on MI355X with packed weights: k in 4 parts
// and a 6-deep ring at three waves per SIMD here, an 8-deep ring at three waves per SIMD
// for down, 1.5% faster than one part and depth 6 at four waves; an 8-deep gate/up ring
// at three waves per SIMD ran 6% slower.
template <int KS, bool PK>
__global__ __launch_bounds__(256, kGuOcc) void swiglu_stream_kernel(const u16* __restrict__ x,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ sorted_pairs, int K,
                                                            const u16* __restrict__ Wg, const u16* __restrict__ Wu,
                                                            u16* __restrict__ h, int d, int I) {
    __shared__ f32x4 part[kWavesPerBlock][2][kMT][64];
    const int e = blockIdx.y;
    const int beg = offsets[e];
    const int n_e = offsets[e + 1] - beg;
    if (n_e <= 0) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * (kWavesPerBlock / KS) + wave / KS) * 16;
    const bool writer = wave % KS == 0 && n0 < I;
    const int kl = d / KS;                                    // this wave's part of k
    const int r16 = lane & 15, kq = (lane >> 4) * 8 + (wave % KS) * kl;
    const int nb16 = min(n0, I - 16);                         // a group past I reads valid rows; discarded
    size_t wo;
    if constexpr (PK)
        wo = (((size_t)e * I + nb16) / 16 * (d / 32) * 64 + lane) * 8 + (size_t)(wave % KS) * kl * 16;
    else
        wo = ((size_t)e * I + nb16 + r16) * d + kq;
    const u16* const ag[1] = {Wg + wo};
    const u16* const au[1] = {Wu + wo};
    for (int mb = 0; mb < n_e; mb += 16 * kMT) {
        const int ntile = min(kMT, (n_e - mb + 15) / 16);
        const u16* xp[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int m = min(mb + 16 * mt + r16, n_e - 1);   // rows past the end read a valid row; discarded
            xp[mt] = x + (size_t)(sorted_pairs[beg + m] / K) * d + kq;
        }
        f32x4 gu[2][kMT][1];
        zero_acc<kMT>(gu[0]);
        zero_acc<kMT>(gu[1]);
        stream_core<1, kMT, kDgu, PK>(ag, xp, kl, gu[0]);
        stream_core<1, kMT, kDgu, PK>(au, xp, kl, gu[1]);
        ksplit_reduce<KS, kMT, 2>(part, wave, lane, gu);
        // lane holds channels n0 + 4*(lane/16) + i for token row mb + 16*mt + lane%16
        if (writer)
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
                const int m = mb + 16 * mt + r16;
                if (mt >= ntile || m >= n_e) continue;
                const int n = n0 + (lane >> 4) * 4;
                const f32x4 gv = gu[0][mt][0], uv = gu[1][mt][0];
                uint32_t lo = (uint32_t)f32_to_bf16(silu_mul(gv[0], uv[0])) |
                              ((uint32_t)f32_to_bf16(silu_mul(gv[1], uv[1])) << 16);
                uint32_t hi = (uint32_t)f32_to_bf16(silu_mul(gv[2], uv[2])) |
                              ((uint32_t)f32_to_bf16(silu_mul(gv[3], uv[3])) << 16);
                *reinterpret_cast<uint2*>(h + (size_t)(beg + m) * I + n) = make_uint2(lo, hi);
            }
        if constexpr (KS > 1) __syncthreads();                // part is reused by the next token tile
    }
}

// y_perm[beg+m, c] = h[beg+m] . Wd[e,c] for the tokens m of expert e (the combine applies the
// routing weight).
// grid: (ceil(d / (16 * 4 / KS)), E); block: 4 waves; the KS waves of a 16-row group of Wd
// each stream a 1/KS part of k, as in the gate/up kernel.
template <int KS, bool PK>
__global__ __launch_bounds__(256, kDnOcc) void down_stream_kernel(const u16* __restrict__ h,
                                                          const int32_t* __restrict__ offsets,
                                                          const u16* __restrict__ Wd, float* __restrict__ y_perm,
                                                          int d, int I) {
    __shared__ f32x4 part[kWavesPerBlock][1][kMT][64];
    const int e = blockIdx.y;
    const int beg = offsets[e];
    const int n_e = offsets[e + 1] - beg;
    if (n_e <= 0) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * (kWavesPerBlock / KS) + wave / KS) * 16;
    const bool writer = wave % KS == 0 && n0 < d;
    const int kl = I / KS;
    const int r16 = lane & 15, kq = (lane >> 4) * 8 + (wave % KS) * kl;
    size_t wo;
    if constexpr (PK)
        wo = (((size_t)e * d + min(n0, d - 16)) / 16 * (I / 32) * 64 + lane) * 8 + (size_t)(wave % KS) * kl * 16;
    else
        wo = ((size_t)e * d + min(n0, d - 16) + r16) * I + kq;
    const u16* const a[1] = {Wd + wo};
    for (int mb = 0; mb < n_e; mb += 16 * kMT) {
        const int ntile = min(kMT, (n_e - mb + 15) / 16);
        const u16* hp[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) hp[mt] = h + (size_t)(beg + min(mb + 16 * mt + r16, n_e - 1)) * I + kq;
        f32x4 acc[1][kMT][1];
        zero_acc<kMT>(acc[0]);
        stream_core<1, kMT, kDdn, PK>(a, hp, kl, acc[0]);
        ksplit_reduce<KS, kMT, 1>(part, wave, lane, acc);
        if (writer)
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
                const int m = mb + 16 * mt + r16;
                if (mt >= ntile || m >= n_e) continue;
                const int c = n0 + (lane >> 4) * 4;
                const f32x4 v = acc[0][mt][0];
                *reinterpret_cast<float4*>(y_perm + (size_t)(beg + m) * d + c) = make_float4(v[0], v[1], v[2], v[3]);
            }
        if constexpr (KS > 1) __syncthreads();
    }
}

// y[t] = sum over the slots j = 0..K-1, in that order, of topk_w[t, j] * y_perm[pair_rank[t*K + j]]
// (each product rounded to FP32 on its own: no contraction into FMA). Slots with pair_rank -1
// (an expert this call does not hold: expert-parallel share) add nothing, and a row with no slot
// left is 0. grid: (T, ceil(d / 1024)); each thread owns one float4 of the row.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ pair_rank,
                                                      const float* __restrict__ topk_w, int K, int d,
                                                      float* __restrict__ y) {
#pragma clang fp contract(off)
    const int64_t t = blockIdx.x;
    const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (c >= d) return;
    int rk[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) rk[j] = j < K ? pair_rank[t * K + j] : -1;
    float4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (rk[j] >= 0) {
            // each y_perm element is read once (non-temporal: T=8192 0.305 -> 0.267 ms on MI355X)
            const u32x4 r = ld_once(y_perm + (size_t)rk[j] * d + c);
            const float wt = topk_w[t * K + j];
            v[j] = make_float4(wt * __uint_as_float(r.x), wt * __uint_as_float(r.y), wt * __uint_as_float(r.z),
                               wt * __uint_as_float(r.w));
        }
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    bool first = true;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (rk[j] >= 0) {
            if (first) acc = v[j];
            else { acc.x += v[j].x; acc.y += v[j].y; acc.z += v[j].z; acc.w += v[j].w; }
            first = false;
        }
    *reinterpret_cast<float4*>(y + t * d + c) = acc;
}

// Packed layout of a matrix W [rows, K] (rows % 16 == 0, K % 32 == 0): 16-row blocks, each a
// run of K/32 steps of 64 lanes x 8 elements, lane l holding row l % 16, k = 32 j + 8 (l / 16)
// .. +8 of step j: the order in which a streaming wave loads it, so every 1 KB load is
// contiguous. Rows at or past valid_rows repeat row valid_rows - 1 (token tiles padded to 16).
// One thread per 8 elements.
__global__ __launch_bounds__(256) void pack_stream_kernel(const u16* __restrict__ W, u16* __restrict__ P,
                                                          int64_t rows, int64_t valid_rows, int K) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;    // output chunk of 8 elements
    const int64_t steps = K / 32;
    if (o >= (rows / 16) * steps * 64) return;                     // rows * K / 8 chunks
    const int l = (int)(o & 63);
    const int64_t bj = o >> 6;
    const int64_t b = bj / steps, j = bj - b * steps;
    const int64_t r = min(16 * b + (l & 15), valid_rows - 1);
    const int64_t k = 32 * j + 8 * (l >> 4);
    *reinterpret_cast<uint4*>(P + o * 8) = *reinterpret_cast<const uint4*>(W + r * K + k);
}

// ---- dense SwiGLU MLP, decode-sized batches (T <= 64) ------------------------------------
// All T tokens are one expert; every weight byte must serve all of them in one pass. The
// tokens go to packed 16-token tiles first (four tiles, padded with the last token), so each
// wave's token fragments are contiguous kilobytes like its weight fragments. In both kernels
// the waves that stream the same weight rows take four consecutive parts of k against the four
// tiles, and their sums meet in LDS, added in part order. Measured on MI355X at
// T = 64, d = 5120, I = 20480 (packed weights): 0.142-0.146 ms with each token fragment feeding four
// weight fragments (two gate and two up 16-row blocks; four 16-row blocks of Wd), a 3-deep ring
// and two blocks per CU, against 0.158 ms with two weight fragments per token fragment (1:1 -> 2:1
// token bytes per weight byte from L2); 0.149 ms at depth 2 and three blocks per CU, 0.213 ms with
// eight weight fragments (one wave per SIMD); 0.190 ms with every k part written out and added by a
// second kernel. Results are bitwise the same in every form (the k order of each sum is unchanged).
// With the down pass in one round (dense_rb_dn): 0.133 ms; gate/up 87 us for 419 MB, down 41 us,
// token packing 6 us, the k-part sum 5 us; with gate/up in one round too (dense_gu_stream8_kernel)
// 0.1245 ms. Tried on the gate/up pass without gain (before that): ring depth 4
// and 5 (0.140, 0.150 ms), each block starting its k walk at a different step (0.133), the
// unit's weight blocks read as if interleaved per k step (0.133), and the launch's last partial
// round split into k quarters added by the last block to finish (-1 us, not kept). A copy that
// skipped the token fragment reloads ran 0.115 ms (its shorter blocks also shrank the second
// round). Reading x rows directly (16 rows x 64 B per
// fragment, no packing launch) ran 0.163 ms against 0.136; the k-part sum folded into the down
// pass (the last block of a column group adds the parts) 0.1375 against 0.1355.
constexpr int kDT = 4;                   // token tiles (64 tokens)
constexpr int kDD = 3;                   // ring depth of the dense streams
constexpr int kDenseKsDN = 8;            // most k parts of the down pass across blocks
constexpr int kDenseOcc = 2;             // down: blocks of 4 waves per CU the registers must allow

// Adds the other waves' accumulators to wave 0's, in wave order. Returns true in wave 0.
template <int NA>
__device__ __forceinline__ bool dense_reduce(f32x4 (&red)[kWavesPerBlock - 1][kDT][NA][64], int wave, int lane,
                                             f32x4 (&acc)[kDT][NA]) {
    if (wave != 0)
#pragma unroll
        for (int m = 0; m < kDT; ++m)
#pragma unroll
            for (int q = 0; q < NA; ++q) red[wave - 1][m][q][lane] = acc[m][q];
    __syncthreads();
    if (wave != 0) return false;
#pragma unroll
    for (int j = 0; j < kWavesPerBlock - 1; ++j)
#pragma unroll
        for (int m = 0; m < kDT; ++m)
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const f32x4 v = red[j][m][q][lane];
                acc[m][q] = f32x4{acc[m][q][0] + v[0], acc[m][q][1] + v[1], acc[m][q][2] + v[2], acc[m][q][3] + v[3]};
            }
    return true;
}

// hp = bf16(silu(x . Wg[n]) * (x . Wu[n])) for all 64 token slots, written as packed token tiles
// for the down pass, with one block of 8 waves per CU so that the launch is one round of the CUs:
// wave w streams RBW 16-row blocks over k quarter w % 4 against the four token tiles, the gate rows
// of the block's RBW 16-channel groups (w < 4) or their up rows (w >= 4); the quarters of each are
// added in quarter order through LDS, then the up sums meet the gate sums for the SwiGLU.
// grid: ceil(I / (16 RBW)). At I = 20480 (1280 groups) RBW = 5 gives 256 blocks; the form before,
// 640 blocks of 4 waves (two 16-channel groups each) at two blocks per CU, ran its last 128 blocks
// as a second round on half the CUs: T=64 layer 0.1344 -> 0.1245 ms on MI355X, bitwise the same y.
template <bool PK, int RBW>
__global__ __launch_bounds__(512, 1) void dense_gu_stream8_kernel(const u16* __restrict__ xp,
                                                                  const u16* __restrict__ Wg,
                                                                  const u16* __restrict__ Wu,
                                                                  u16* __restrict__ hp, int d, int I) {
    __shared__ f32x4 red[2][kWavesPerBlock - 1][kDT][RBW][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int kq = wave & 3, half = wave >> 2;
    const int ngr = I / 16, g0 = blockIdx.x * RBW;
    const int kl = d / kWavesPerBlock, k0 = kq * kl;
    const u16* const W = half ? Wu : Wg;
    const u16* a[RBW];
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
        const int ng = min(g0 + r, ngr - 1) * 16;       // groups past I repeat the last (not stored)
        a[r] = W + (PK ? ((size_t)ng / 16 * (d / 32) * 64 + lane) * 8 + (size_t)k0 * 16
                       : (size_t)(ng + (lane & 15)) * d + (lane >> 4) * 8 + k0);
    }
    const u16* xb[kDT];
#pragma unroll
    for (int m = 0; m < kDT; ++m) xb[m] = xp + ((size_t)m * (d / 32) * 64 + lane) * 8 + (size_t)k0 * 16;
    f32x4 acc[kDT][RBW];
#pragma unroll
    for (int m = 0; m < kDT; ++m)
#pragma unroll
        for (int r = 0; r < RBW; ++r) acc[m][r] = f32x4{0, 0, 0, 0};
    stream_core<RBW, kDT, kDD, PK, true>(a, xb, kl, acc);
    if (kq != 0)
#pragma unroll
        for (int m = 0; m < kDT; ++m)
#pragma unroll
            for (int r = 0; r < RBW; ++r) red[half][kq - 1][m][r][lane] = acc[m][r];
    __syncthreads();
    if (kq == 0)
#pragma unroll
        for (int j = 0; j < kWavesPerBlock - 1; ++j)
#pragma unroll
            for (int m = 0; m < kDT; ++m)
#pragma unroll
                for (int r = 0; r < RBW; ++r) {
                    const f32x4 v = red[half][j][m][r][lane];
                    acc[m][r] = f32x4{acc[m][r][0] + v[0], acc[m][r][1] + v[1], acc[m][r][2] + v[2],
                                      acc[m][r][3] + v[3]};
                }
    __syncthreads();
    if (kq == 0 && half == 1)
#pragma unroll
        for (int m = 0; m < kDT; ++m)
#pragma unroll
            for (int r = 0; r < RBW; ++r) red[0][0][m][r][lane] = acc[m][r];
    __syncthreads();
    if (kq != 0 || half != 0) return;
    // lane holds channels c .. c+3 (c = 16 g + 4 (lane / 16)) of token slot 16 m + lane % 16; in the
    // packed tiles they are elements c % 8 .. +3 of the 8-element chunk of k-step c / 32, lane
    // (lane % 16) + 16 ((c % 32) / 8)
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
        if (g0 + r >= ngr) break;
        const int c = (g0 + r) * 16 + 4 * (lane >> 4);
        const int pl = (lane & 15) + 16 * ((c & 31) >> 3);
#pragma unroll
        for (int m = 0; m < kDT; ++m) {
            const f32x4 gv = acc[m][r], uv = red[0][0][m][r][lane];
            const uint32_t lo = (uint32_t)f32_to_bf16(silu_mul(gv[0], uv[0])) |
                                ((uint32_t)f32_to_bf16(silu_mul(gv[1], uv[1])) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(silu_mul(gv[2], uv[2])) |
                                ((uint32_t)f32_to_bf16(silu_mul(gv[3], uv[3])) << 16);
            *reinterpret_cast<uint2*>(hp + (((size_t)m * (I / 32) + c / 32) * 64 + pl) * 8 + (c & 7)) =
                make_uint2(lo, hi);
        }
    }
}

// part[kb][t][c] = sum over k part kb (of gridDim.y) of I for output channel c and token slot t.
// grid: (d / (16 RB), ks); block: 4 waves, wave w streaming the block's RB 16-row blocks of Wd
// (each token fragment feeding all of them) over quarter w of part kb.
template <bool PK, int RB>
__global__ __launch_bounds__(256, kDenseOcc) void dense_dn_stream_kernel(const u16* __restrict__ hp,
                                                                      const u16* __restrict__ Wd,
                                                                      float* __restrict__ part, int d, int I) {
    __shared__ f32x4 red[kWavesPerBlock - 1][kDT][RB][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * 16 * RB;
    const int kb = blockIdx.y, kl = I / (int)gridDim.y / kWavesPerBlock;
    const int k0 = (kb * kWavesPerBlock + wave) * kl;
    const u16* a[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int nr = n0 + 16 * r;
        a[r] = Wd + (PK ? ((size_t)nr / 16 * (I / 32) * 64 + lane) * 8 + (size_t)k0 * 16
                        : (size_t)(nr + (lane & 15)) * I + (lane >> 4) * 8 + k0);
    }
    const u16* xb[kDT];
#pragma unroll
    for (int m = 0; m < kDT; ++m) xb[m] = hp + ((size_t)m * (I / 32) * 64 + lane) * 8 + (size_t)k0 * 16;
    f32x4 acc[kDT][RB];
#pragma unroll
    for (int m = 0; m < kDT; ++m)
#pragma unroll
        for (int r = 0; r < RB; ++r) acc[m][r] = f32x4{0, 0, 0, 0};
    stream_core<RB, kDT, kDD, PK, true>(a, xb, kl, acc);
    if (!dense_reduce<RB>(red, wave, lane, acc)) return;
    const int tp = 16 * kDT;
#pragma unroll
    for (int m = 0; m < kDT; ++m)
#pragma unroll
        for (int r = 0; r < RB; ++r)
            *reinterpret_cast<f32x4*>(part + ((size_t)kb * tp + 16 * m + (lane & 15)) * d + n0 + 16 * r +
                                      4 * (lane >> 4)) = acc[m][r];
}

// y[t] = sum over kb, in order, of part[kb][t] for the T real tokens. One thread per float4.
__global__ __launch_bounds__(256) void dense_dn_finish_kernel(const float* __restrict__ part, int ks, int64_t T, int d,
                                                              float* __restrict__ y) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= T * (d / 4)) return;
    const int64_t t = o / (d / 4);
    const int c = (int)(o - t * (d / 4)) * 4;
    const int tp = 16 * kDT;
    float4 acc = *reinterpret_cast<const float4*>(part + (size_t)t * d + c);
    for (int kb = 1; kb < ks; ++kb) {
        const float4 v = *reinterpret_cast<const float4*>(part + ((size_t)kb * tp + t) * d + c);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4*>(y + t * d + c) = acc;
}

// k parts of the down pass across blocks: the most (up to kDenseKsDN) that leave every wave a
// whole number of 32-wide steps.
int dense_ks_dn(int I) {
    int ks = kDenseKsDN;
    while (ks > 1 && I % (32 * kWavesPerBlock * ks) != 0) ks /= 2;
    return ks;
}

// 16-row blocks of Wd per down block (each token fragment feeds them all): five when d allows,
// else four. At d = 5120 five give 64 x 8 = 512 blocks, one round at two blocks per CU on
// MI355X; four gave 640, whose last 128 ran as a second round: down pass 47.4 -> 40.9 us at
// T = 64, I = 20480 (bitwise the same y).
int dense_rb_dn(int d) { return d % (16 * 5) == 0 ? 5 : 4; }

}  // namespace

// Path choice from the average number of tokens per expert: up to 16 the weight-streaming
// kernels (each expert's weights read once per 16 of its tokens), above that the tiled
// grouped GEMM (weights read about once per call, tokens re-read from L2).
// An expert-parallel share decides on all experts (route_E), so that it takes the same path,
// with the same arithmetic, as the whole layer would.
bool experts_tiled(const Shape& s) { return gemm_supports(s) && s.T * (int64_t)s.K > 16 * (int64_t)s.route_E; }

int experts_tile_m(const Shape& s) { return experts_tiled(s) ? gemm_tile_m(s) : 16 * kMT; }

void launch_swiglu(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                   const int32_t* tiles, int32_t* n_tiles, const void* Wg, const void* Wu, void* h,
                   hipStream_t st) {
    if (experts_tiled(s)) {
        launch_gemm_swiglu(s, x, offsets, sorted_pairs, tiles, n_tiles, Wg, Wu, h, st);
        return;
    }
    // k parts must be whole 32-wide MFMA steps
    const int ks = s.d % (32 * kGuKsplit) == 0 ? kGuKsplit : 1;
    const int per_block = kWavesPerBlock / ks * 16;
    const dim3 grid((unsigned)((s.I + per_block - 1) / per_block), (unsigned)s.E);
#define BEAM_GU(KS, PK)                                                                                       \
    hipLaunchKernelGGL((swiglu_stream_kernel<KS, PK>), grid, dim3(256), 0, st, (const u16*)x, offsets,         \
                       sorted_pairs, s.K, (const u16*)Wg, (const u16*)Wu, (u16*)h, s.d, s.I)
    if (ks == kGuKsplit) {
        if (s.packed) BEAM_GU(kGuKsplit, true); else BEAM_GU(kGuKsplit, false);
    } else {
        if (s.packed) BEAM_GU(1, true); else BEAM_GU(1, false);
    }
#undef BEAM_GU
}

void launch_down(const Shape& s, const void* h, const int32_t* offsets, const int32_t* sorted_pairs,
                 const int32_t* tiles, int32_t* n_tiles, const void* Wd, float* y_perm, hipStream_t st) {
    if (experts_tiled(s)) {
        launch_gemm_down(s, h, offsets, sorted_pairs, tiles, n_tiles, Wd, y_perm, st);
        return;
    }
    const int ks = s.I % (32 * kDnKsplit) == 0 ? kDnKsplit : 1;
    const int per_block = kWavesPerBlock / ks * 16;
    const dim3 grid((unsigned)((s.d + per_block - 1) / per_block), (unsigned)s.E);
#define BEAM_DN(KS, PK)                                                                                       \
    hipLaunchKernelGGL((down_stream_kernel<KS, PK>), grid, dim3(256), 0, st, (const u16*)h, offsets,           \
                       (const u16*)Wd, y_perm, s.d, s.I)
    if (ks == kDnKsplit) {
        if (s.packed) BEAM_DN(kDnKsplit, true); else BEAM_DN(kDnKsplit, false);
    } else {
        if (s.packed) BEAM_DN(1, true); else BEAM_DN(1, false);
    }
#undef BEAM_DN
}

void launch_combine(const Shape& s, const float* y_perm, const int32_t* pair_rank, const float* topk_w, float* y,
                    hipStream_t st) {
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)s.T, (unsigned)((s.d + 1023) / 1024)), dim3(256), 0, st, y_perm,
                       pair_rank, topk_w, s.K, s.d, y);
}

void launch_pack_stream(const void* W, void* P, int64_t rows, int K, hipStream_t st) {
    const int64_t chunks = (rows / 16) * (K / 32) * 64;            // rows * K / 8
    hipLaunchKernelGGL(pack_stream_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, (const u16*)W,
                       (u16*)P, rows, rows, K);
}

// every wave of both passes streams a whole number of 32-wide k-steps: d, I multiples of 128
bool dense_stream_supports(int64_t T, int d, int I) {
    return T >= 1 && T <= 16 * kDT && d % 128 == 0 && I % 128 == 0;
}

size_t dense_stream_workspace_bytes(int64_t T, int d, int I) {
    (void)T;
    const size_t tp = 16 * kDT;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    return up(tp * d * 2) + up(tp * I * 2) + up((size_t)dense_ks_dn(I) * tp * d * 4);
}

void launch_dense_stream(int64_t T, int d, int I, bool packed, const void* x, const void* Wg, const void* Wu,
                         const void* Wd, float* y, void* ws, hipStream_t st) {
    const size_t tp = 16 * kDT;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const int ks_dn = dense_ks_dn(I), rb = dense_rb_dn(d);
    char* w = static_cast<char*>(ws);
    u16* xp = reinterpret_cast<u16*>(w);
    w += up(tp * d * 2);
    u16* hp = reinterpret_cast<u16*>(w);
    w += up(tp * I * 2);
    float* part_dn = reinterpret_cast<float*>(w);
    const int64_t xchunks = (int64_t)kDT * (d / 32) * 64;
    hipLaunchKernelGGL(pack_stream_kernel, dim3((unsigned)((xchunks + 255) / 256)), dim3(256), 0, st, (const u16*)x,
                       xp, (int64_t)tp, T, d);
    const dim3 gdn((unsigned)(d / (16 * rb)), (unsigned)ks_dn);
    // 16-channel groups per gate/up block: the fewest that cover I in one block per CU, at most 5
    const int ngr = I / 16, rbw = std::min(5, std::max(1, (ngr + 255) / 256));
    const dim3 ggu((unsigned)((ngr + rbw - 1) / rbw));
#define BEAM_DGU8(PK, R)                                                                                       \
    hipLaunchKernelGGL((dense_gu_stream8_kernel<PK, R>), ggu, dim3(512), 0, st, xp, (const u16*)Wg,          \
                       (const u16*)Wu, hp, d, I)
#define BEAM_DGU8_R(PK)                                                                                        \
    switch (rbw) {                                                                                             \
        case 1: BEAM_DGU8(PK, 1); break;                                                                       \
        case 2: BEAM_DGU8(PK, 2); break;                                                                       \
        case 3: BEAM_DGU8(PK, 3); break;                                                                       \
        case 4: BEAM_DGU8(PK, 4); break;                                                                       \
        default: BEAM_DGU8(PK, 5); break;                                                                      \
    }
    if (packed) { BEAM_DGU8_R(true) } else { BEAM_DGU8_R(false) }
#undef BEAM_DGU8_R
#undef BEAM_DGU8
#define BEAM_DDN(PK, RB)                                                                                       \
    hipLaunchKernelGGL((dense_dn_stream_kernel<PK, RB>), gdn, dim3(256), 0, st, hp, (const u16*)Wd, part_dn, d, I)
    if (rb == 5) {
        if (packed) BEAM_DDN(true, 5); else BEAM_DDN(false, 5);
    } else {
        if (packed) BEAM_DDN(true, 4); else BEAM_DDN(false, 4);
    }
#undef BEAM_DDN
    const int64_t ychunks = T * (d / 4);
    hipLaunchKernelGGL(dense_dn_finish_kernel, dim3((unsigned)((ychunks + 255) / 256)), dim3(256), 0, st, part_dn,
                       ks_dn, T, d, y);
}

}  // namespace beam

// Router of the Beam MoE layer: optional pre-MLP RMSNorm, FP32 router GEMM,
// sigmoid + bias, group-limited top-k and weight normalisation.
//
// Method: Transformers "Beam" model page (Overview: sparse MoE item, sandwich norms,
// FP32 numerics note; BeamConfig: n_group, topk_group, num_experts_per_tok,
// norm_topk_prob, routed_scaling_factor, rms_norm_eps) and archdb
// "Beam-1.0-501B-A23B" fact sheet (MoE: sigmoid gating, group score = sum of the
// top-2 biased scores, renormalised weights, 2.5 scaling).
#include "common.h"
#include "kernels.h"

namespace beam {
namespace {

// ---------------------------------------------------------------------------------------
// Pre-MLP RMSNorm, one 256-thread block per token. Done in FP64 (the pages ask for at
// least FP32): the bf16 rounding of x is then a function of h and w alone, independent
// of the reduction order, so every consumer of x sees the same bits.
// bf16((a * r) * w) as the FP64 products round it (f64_to_bf16), mostly without FP64: the FP32
// product p carries three roundings (r to FP32, then two products), so it lies within 3.0002 FP32
// ulps of the FP64 one, and when p is at least 8 ulps from a bf16 rounding midpoint both round to
// the same bf16. The rest (near a midpoint, zero or subnormal exponent field, inf) take FP64.
__device__ __forceinline__ u16 norm_to_bf16(u16 ab, u16 wb, float r32, double r) {
    const float a = bf16_to_f32(ab), w = bf16_to_f32(wb);
    const float p = (a * r32) * w;
    const uint32_t u = __float_as_uint(p);
    const uint32_t ex = (u >> 23) & 0xffu;
    const int dist = (int)(u & 0xffffu) - 0x8000;
    if (ex != 0u && ex != 0xffu && (dist >= 8 || dist <= -8)) return (u16)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    return f64_to_bf16(((double)a * r) * (double)w);
}

// Sum of the squares of the 8 bf16 values in v, in FP64 (exact products, rounded sums).
__device__ __forceinline__ double sumsq8(uint4 v, double ss) {
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double a = bf16_to_f32((u16)(p[i] & 0xffffu)), b = bf16_to_f32((u16)(p[i] >> 16));
        ss += a * a;
        ss += b * b;
    }
    return ss;
}

__device__ __forceinline__ uint4 norm8(uint4 v, uint4 g, float r32, double r) {
    const uint32_t p[4] = {v.x, v.y, v.z, v.w}, q[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u16 lo = norm_to_bf16((u16)(p[i] & 0xffffu), (u16)(q[i] & 0xffffu), r32, r);
        const u16 hi = norm_to_bf16((u16)(p[i] >> 16), (u16)(q[i] >> 16), r32, r);
        o[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

constexpr int kNormChunks = 16;    // 8-value chunks per lane loaded together for the sum of squares

// x[t] = bf16((h[t] * r) * w), r = 1 / sqrt(mean(h[t]^2) + eps), the sum of squares and r in FP64:
// one wave per token row. The first pass issues all its loads of a row (up to 64 * 8 * kNormChunks
// values at a time) before it adds; the second reads the row again, from cache.
__device__ __forceinline__ void rmsnorm_row(const u16* __restrict__ h, const u16* __restrict__ w,
                                            u16* __restrict__ x, int d, double eps, int64_t t) {
    const int lane = threadIdx.x & 63;
    const u16* hr = h + t * d;
    u16* xr = x + t * d;
    double ss = 0.0;
    for (int c0 = 0; c0 < d; c0 += 64 * 8 * kNormChunks) {
        uint4 v[kNormChunks];
#pragma unroll
        for (int i = 0; i < kNormChunks; ++i) {
            const int c = c0 + (lane + 64 * i) * 8;
            v[i] = c < d ? *reinterpret_cast<const uint4*>(hr + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kNormChunks; ++i) ss = sumsq8(v[i], ss);
    }
    ss = wave_sum_f64(ss);
    const double r = 1.0 / sqrt(ss / (double)d + eps);
    const float r32 = (float)r;
#pragma unroll 2
    for (int c = lane * 8; c < d; c += 64 * 8)
        *reinterpret_cast<uint4*>(xr + c) =
            norm8(*reinterpret_cast<const uint4*>(hr + c), *reinterpret_cast<const uint4*>(w + c), r32, r);
}

constexpr int kNormRows = 4;    // token rows per 256-thread block, one per wave

__global__ __launch_bounds__(256) void rmsnorm_kernel(const u16* __restrict__ h, const u16* __restrict__ w,
                                                      u16* __restrict__ x, int d, double eps, int64_t T) {
    const int64_t t = (int64_t)blockIdx.x * kNormRows + (threadIdx.x >> 6);
    if (t < T) rmsnorm_row(h, w, x, d, eps, t);
}

// ---------------------------------------------------------------------------------------
// Router GEMM z = x . Wr in FP32 on the vector ALUs. Block tile: 64 tokens x 64 experts,
// K staged through LDS in steps of 32; each thread owns a 4x4 register tile. blockIdx.z
// splits K so that a decode-sized batch still spreads the 5 MB of Wr over many CUs; the
// partial sums go to z_part[ks] and are added in fixed order by the top-k kernel.
constexpr int RT = 64, RE = 64, RK = 32;

__global__ __launch_bounds__(256) void router_logits_kernel(const u16* __restrict__ x, const float* __restrict__ Wr,
                                                            float* __restrict__ zp, int64_t T, int d, int E,
                                                            int kchunk) {
    __shared__ float xs[RK][RT + 4];
    __shared__ float ws[RK][RE + 4];
    const int64_t t0 = (int64_t)blockIdx.x * RT;
    const int e0 = blockIdx.y * RE;
    const int kb = blockIdx.z * kchunk, ke = kb + kchunk;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int k0 = kb; k0 < ke; k0 += RK) {
        {
            const int tok = threadIdx.x >> 2, kc = (threadIdx.x & 3) * 8;
            const int64_t t = t0 + tok;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < T) v = *reinterpret_cast<const uint4*>(x + t * d + k0 + kc);
            uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xs[kc + 2 * i][tok] = bf16_to_f32((u16)(p[i] & 0xffffu));
                xs[kc + 2 * i + 1][tok] = bf16_to_f32((u16)(p[i] >> 16));
            }
        }
        {
            const int kk = threadIdx.x >> 3, ec = (threadIdx.x & 7) * 8;
            const float* src = Wr + (int64_t)(k0 + kk) * E + e0 + ec;
            if ((E & 3) == 0 && e0 + ec + 8 <= E) {
                float4 a = *reinterpret_cast<const float4*>(src);
                float4 b = *reinterpret_cast<const float4*>(src + 4);
                ws[kk][ec + 0] = a.x; ws[kk][ec + 1] = a.y; ws[kk][ec + 2] = a.z; ws[kk][ec + 3] = a.w;
                ws[kk][ec + 4] = b.x; ws[kk][ec + 5] = b.y; ws[kk][ec + 6] = b.z; ws[kk][ec + 7] = b.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) ws[kk][ec + i] = (e0 + ec + i < E) ? src[i] : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll 8
        for (int k = 0; k < RK; ++k) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { a[i] = xs[k][4 * ty + i]; b[i] = ws[k][4 * tx + i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    float* out = zp + (int64_t)blockIdx.z * T * E;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 4 * ty + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + 4 * tx + j;
            if (e < E) out[t * E + e] = acc[i][j];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Selection for one token, by one whole wavefront. Lane l holds the logits of experts
// [l*EPL, (l+1)*EPL); a group of E/G experts spans LPG = E/(G*EPL) adjacent lanes (a power
// of two), so the group top-2 is an xor-butterfly inside aligned lane blocks. Ties go to
// the lower index everywhere. Writes idx/w rows (and the logits row when asked).
template <int EPL>
__device__ __forceinline__ void select_token(const float (&z)[EPL], int lane, int E, int G, int KG, int K, float S,
                                             int norm, const float* __restrict__ bias, int32_t* __restrict__ idx_row,
                                             float* __restrict__ w_row, float* __restrict__ logits_row) {
    const int e0 = lane * EPL;
    const bool live = e0 < E;
    const float NEG = -INFINITY;
    float s[EPL], b[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = e0 + i;
        s[i] = 0.0f;
        b[i] = NEG;
        if (e < E) {
            if (logits_row) logits_row[e] = z[i];
            s[i] = 1.0f / (1.0f + expf(-z[i]));
            b[i] = s[i] + bias[e];
        }
    }
    // Group score: sum of the two largest biased scores of the group.
    const int gsz = E / G;
    const int lpg = gsz / EPL;
    float v1 = NEG, v2 = NEG;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float v = b[i];
        if (v > v1) { v2 = v1; v1 = v; } else if (v > v2) { v2 = v; }
    }
    for (int m = 1; m < lpg; m <<= 1) {
        const float o1 = __shfl_xor(v1, m, kWave), o2 = __shfl_xor(v2, m, kWave);
        const float n2 = fmaxf(fminf(v1, o1), fmaxf(v2, o2));
        v1 = fmaxf(v1, o1);
        v2 = n2;
    }
    const float gs = v1 + v2;
    // Lane g < G takes group g's score, then its rank among the groups.
    const float gsl = __shfl(gs, (lane < G ? lane : 0) * lpg, kWave);
    int rank = 0;
    for (int g2 = 0; g2 < G; ++g2) {
        const float o = __shfl(gsl, g2, kWave);
        rank += (o > gsl) || (o == gsl && g2 < lane);
    }
    const uint64_t kept = __ballot(lane < G && rank < KG);
    const bool my_kept = live && ((kept >> (e0 / gsz)) & 1ull);
    // Top-K among experts of the kept groups: K rounds of a wave-wide argmax on a key
    // that orders by biased score, then by lower expert id.
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = e0 + i;
        key[i] = (my_kept && e < E) ? (((uint64_t)f32_order_key(b[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e))
                                    : 0ull;
    }
    float sum = 0.0f, my_s = 0.0f;
    int my_e = 0;
    for (int j = 0; j < K; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffu));
        float se = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (e0 + i == e) { se = s[i]; key[i] = 0ull; }
        se = __shfl(se, e / EPL, kWave);
        sum += se;
        if (lane == j) { my_e = e; my_s = se; }
    }
    if (lane < K) {
        idx_row[lane] = my_e;
        w_row[lane] = norm ? S * my_s / sum : S * my_s;
    }
}

// Selection from partial logits zp [ks][T][P*E] (P = 1, or 3 for the planes of the split
// weight, which the GEMM route keeps apart): one wavefront per token; the ks*P partial sums of
// each logit are added in ascending order of (k part, plane) (deterministic).
template <int EPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ zp, int ks, int64_t T, int E,
                                                          int G, int KG, int K, float S, int norm,
                                                          const float* __restrict__ bias, int32_t* __restrict__ idx,
                                                          float* __restrict__ wout, float* __restrict__ logits, int P) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int e0 = lane * EPL;
    float z[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) z[i] = 0.0f;
    if (e0 < E) {
        // part j = (k part, plane) of a logit row: j / P, j % P
        const int parts = ks * P;
        auto at = [&](int j) { return zp + ((int64_t)(j / P) * T + t) * (P * E) + (j % P) * E + e0; };
        if constexpr (EPL == 4) {
            // E is a multiple of 64 here, so each lane's 4 logits are one aligned float4
            int j = 0;
            for (; j + 8 <= parts; j += 8) {
                float4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(at(j + u));
#pragma unroll
                for (int u = 0; u < 8; ++u) { z[0] += v[u].x; z[1] += v[u].y; z[2] += v[u].z; z[3] += v[u].w; }
            }
            for (; j < parts; ++j) {
                const float4 v = *reinterpret_cast<const float4*>(at(j));
                z[0] += v.x; z[1] += v.y; z[2] += v.z; z[3] += v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (e0 + i < E)
                    for (int j = 0; j < parts; ++j) z[i] += at(j)[i];
        }
    }
    select_token<EPL>(z, lane, E, G, KG, K, S, norm, bias, idx + t * K, wout + t * K, logits ? logits + t * E : nullptr);
}

// The same selection for E = 256 when each logit has many partial sums and the tokens are few
// (decode): one token per block, the four waves each add a contiguous quarter of the parts
// (one batch of loads in flight each), then wave 0 adds the four quarter sums in order and
// selects. Deterministic; the sum is grouped by quarters instead of running left to right.
__global__ __launch_bounds__(256) void router_topk_quarters_kernel(const float* __restrict__ zp, int ks, int64_t T,
                                                                   int E, int G, int KG, int K, float S, int norm,
                                                                   const float* __restrict__ bias,
                                                                   int32_t* __restrict__ idx, float* __restrict__ wout,
                                                                   float* __restrict__ logits, int P) {
    constexpr int kBatch = 16;
    __shared__ float4 qsum[3][64];
    const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int64_t t = blockIdx.x;
    const int parts = ks * P, per = (parts + 3) / 4;
    const int j0 = q * per, j1 = min(parts, j0 + per);
    auto at = [&](int j) { return zp + ((int64_t)(j / P) * T + t) * (P * E) + (j % P) * E + 4 * lane; };
    float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int j = j0; j < j1; j += kBatch) {
        float4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (j + u < j1) v[u] = *reinterpret_cast<const float4*>(at(j + u));
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (j + u < j1) { z.x += v[u].x; z.y += v[u].y; z.z += v[u].z; z.w += v[u].w; }
    }
    if (q > 0) qsum[q - 1][lane] = z;
    __syncthreads();
    if (q != 0) return;
    float zz[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        const float4 o = qsum[r][lane];
        zz[0] += o.x; zz[1] += o.y; zz[2] += o.z; zz[3] += o.w;
    }
    select_token<4>(zz, lane, E, G, KG, K, S, norm, bias, idx + t * K, wout + t * K, logits ? logits + t * E : nullptr);
}

// ---------------------------------------------------------------------------------------
// Router GEMM on BF16 MFMA with FP32-exact products. Each FP32 router weight is split into
// three bf16 parts (hi + mid + lo = w exactly: 8 + 8 + 8 significant bits); x is bf16 already,
// so x*hi, x*mid and x*lo are exact and are accumulated in FP32 by the MFMA, the same FP32
// dot product the vector path computes, about 10x faster.

// w = hi + mid + lo exactly: hi and mid are w and its first remainder cut to bf16, lo the
// second remainder rounded to bf16 (bit patterns in the low 16 bits of each output).
__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const float h = __uint_as_float(__float_as_uint(w) & 0xffff0000u);
    const float r1 = w - h;
    const float m = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
    hi = __float_as_uint(h) >> 16;
    mid = __float_as_uint(m) >> 16;
    lo = (uint32_t)f32_to_bf16(r1 - m);
}

// Wr [d, E] fp32 -> WrS [3][E][d] bf16 (expert-major, k contiguous: the MFMA B-operand layout),
// the 64 x 64 tile (k0, e0).
__device__ __forceinline__ void split_tile(const float* __restrict__ Wr, u16* __restrict__ WrS, int d, int E,
                                           int k0, int e0) {
    __shared__ float tile[64][65];
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
        const int kk = i >> 4, ec = (i & 15) * 4;
        const float4 v = *reinterpret_cast<const float4*>(Wr + (size_t)(k0 + kk) * E + e0 + ec);
        tile[kk][ec] = v.x; tile[kk][ec + 1] = v.y; tile[kk][ec + 2] = v.z; tile[kk][ec + 3] = v.w;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 8; i += 256) {
        const int e = i >> 3, kc = (i & 7) * 8;
        uint32_t p[3][4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            uint32_t h2[3][2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) split3(tile[kc + j + jj][e], h2[0][jj], h2[1][jj], h2[2][jj]);
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) p[pl][j / 2] = h2[pl][0] | (h2[pl][1] << 16);
        }
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
            *reinterpret_cast<uint4*>(WrS + ((size_t)pl * E + e0 + e) * d + k0 + kc) =
                make_uint4(p[pl][0], p[pl][1], p[pl][2], p[pl][3]);
    }
}

__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ Wr, u16* __restrict__ WrS,
                                                           int d, int E) {
    split_tile(Wr, WrS, d, E, blockIdx.x * 64, blockIdx.y * 64);
}

// The two passes that precede the router product when the layer opens with the pre-MLP
// RMSNorm, in one launch: blocks [0, nbn) norm kNormRows tokens each (x = bf16(h * r * w), the x
// the router and the experts read), blocks [nbn, nbn + (d/64)(E/64)) split one 64 x 64 tile of Wr.
__global__ __launch_bounds__(256) void router_prep_kernel(const u16* __restrict__ h, const u16* __restrict__ w,
                                                          u16* __restrict__ x, double eps, int64_t T,
                                                          const float* __restrict__ Wr, u16* __restrict__ WrS,
                                                          int d, int E) {
    const int64_t b = blockIdx.x, nbn = (T + kNormRows - 1) / kNormRows;
    if (b < nbn) {
        const int64_t t = b * kNormRows + (threadIdx.x >> 6);
        if (t < T) rmsnorm_row(h, w, x, d, eps, t);
        return;
    }
    const int tile = (int)(b - nbn), nk = d / 64;
    split_tile(Wr, WrS, d, E, (tile % nk) * 64, (tile / nk) * 64);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Block: 64 tokens x E experts (4 waves of E/4 experts = NTW tiles of 16), k range
// [blockIdx.y*kc, +kc). FUSED (kc = d): logits go through LDS and the block selects the
// experts of its 64 tokens. Otherwise the partial logits go to zp[blockIdx.y].
// RAW: the weights come as the FP32 Wr [d, E] itself and are split in registers (few tokens:
// the split copy would cost a launch and more bytes than it saves).
template <int NTW, bool FUSED, bool RAW = false>
__global__ __launch_bounds__(256, 2) void router_mfma_kernel(const u16* __restrict__ x, const void* __restrict__ Wsrc,
                                                             float* __restrict__ zp, int64_t T, int d, int E, int kc,
                                                             int G, int KG, int K, float S, int norm,
                                                             const float* __restrict__ bias,
                                                             int32_t* __restrict__ idx, float* __restrict__ wout,
                                                             float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)blockIdx.x * 64;
    const int kb = blockIdx.y * kc;
    const int kq = (lane >> 4) * 8;
    const u16* ap[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = min(t0 + 16 * i + (lane & 15), T - 1);   // rows past the end repeat; not stored
        ap[i] = x + t * d + kb + kq;
    }
    const int ew = (blockIdx.z * 4 + wave) * (NTW * 16);     // blockIdx.z: a quarter-block of experts (small T)
    const u16* const WrS = reinterpret_cast<const u16*>(Wsrc);
    const float* const Wr = reinterpret_cast<const float*>(Wsrc);
    const u16* bp[NTW][3];
    const float* fp[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        if constexpr (RAW) fp[j] = Wr + (size_t)(kb + kq) * E + ew + 16 * j + (lane & 15);
        else
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) bp[j][pl] = WrS + ((size_t)pl * E + ew + 16 * j + (lane & 15)) * d + kb + kq;
    }
    f32x4 acc[4][NTW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
    bf16x8 a[2][4], bw[2][NTW][3];
    float raw[2][NTW][8];
    auto load = [&](int buf, int k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[buf][i] = *reinterpret_cast<const bf16x8*>(ap[i] + k);
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            if constexpr (RAW) {
#pragma unroll
                for (int u = 0; u < 8; ++u) raw[buf][j][u] = fp[j][(size_t)(k + u) * E];
            } else {
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) bw[buf][j][pl] = *reinterpret_cast<const bf16x8*>(bp[j][pl] + k);
            }
        }
    };
    auto mma = [&](int buf) {
        if constexpr (RAW) {
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                u32x4 p[3];
#pragma unroll
                for (int u = 0; u < 8; u += 2) {
                    uint32_t h0[3], h1[3];
                    split3(raw[buf][j][u], h0[0], h0[1], h0[2]);
                    split3(raw[buf][j][u + 1], h1[0], h1[1], h1[2]);
#pragma unroll
                    for (int pl = 0; pl < 3; ++pl) p[pl][u / 2] = h0[pl] | (h1[pl] << 16);
                }
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) bw[buf][j][pl] = __builtin_bit_cast(bf16x8, p[pl]);
            }
        }
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NTW; ++j) acc[i][j] = mfma16(a[buf][i], bw[buf][j][pl], acc[i][j]);
    };
    // two k-steps in flight; kc is a multiple of 64
    load(0, 0);
    for (int k = 0; k < kc; k += 64) {
        load(1, min(k + 32, kc - 32));
        mma(0);
        load(0, min(k + 64, kc - 32));
        mma(1);
    }
    // acc[i][j][v]: token 16*i + 4*(lane/16) + v, expert ew + 16*j + lane%16
    if constexpr (!FUSED) {
        float* out = zp + (size_t)blockIdx.y * T * E;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t t = t0 + 16 * i + 4 * (lane >> 4) + v;
                if (t >= T) continue;
#pragma unroll
                for (int j = 0; j < NTW; ++j) out[t * E + ew + 16 * j + (lane & 15)] = acc[i][j][v];
            }
    } else {
        __shared__ float zs[64][NTW * 64 + 4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int j = 0; j < NTW; ++j) zs[16 * i + 4 * (lane >> 4) + v][ew + 16 * j + (lane & 15)] = acc[i][j][v];
        __syncthreads();
        constexpr int EPL = NTW;   // E = 64 * NTW: NTW logits per lane
        for (int r = wave; r < 64; r += 4) {
            const int64_t t = t0 + r;
            if (t >= T) break;
            float z[EPL];
#pragma unroll
            for (int i = 0; i < EPL; ++i) z[i] = zs[r][lane * EPL + i];
            select_token<EPL>(z, lane, E, G, KG, K, S, norm, bias, idx + t * K, wout + t * K,
                              logits ? logits + t * E : nullptr);
        }
    }
}

}  // namespace

void launch_rmsnorm(const Shape& s, const void* h, const void* w, void* x_out, hipStream_t st) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)((s.T + kNormRows - 1) / kNormRows)), dim3(256), 0, st,
                       (const u16*)h, (const u16*)w, (u16*)x_out, s.d, (double)s.eps, s.T);
}

bool router_uses_mfma(const Shape& s) { return (s.E == 128 || s.E == 256) && s.d % 64 == 0; }

// The quarter-split selection (router_topk_quarters_kernel) takes E = 256 batches of at most
// this many tokens whose logits have at least this many partial sums.
constexpr int kQuartersMinParts = 16;
constexpr int64_t kQuartersMaxT = 1024;

// Blocks of 64 tokens; batches of 1024+ blocks run the fused full-K kernel, smaller ones split
// K so that about 1024 blocks share the work (and the 5 MB router weight).

int router_ksplit(const Shape& s) {
    const int64_t tb = (s.T + 63) / 64;
    if (router_uses_mfma(s)) {
        if (tb >= 1024) return 1;                   // enough blocks for the fused full-K kernel
        const int steps = s.d / 64;                 // 64-wide k chunks
        int want = (int)(1024 / tb);
        int ks = 1;
        for (int c = 1; c <= want && c <= 64; ++c)
            if (steps % c == 0 && steps / c >= 2) ks = c;
        return ks;
    }
    const int64_t tiles = (int64_t)((s.E + RE - 1) / RE) * tb;
    int64_t want = 512 / (tiles > 0 ? tiles : 1);
    if (want < 1) want = 1;
    if (want > 16) want = 16;
    const int steps = s.d / RK;
    int ks = 1;
    for (int c = 1; c <= want; ++c)
        if (steps % c == 0) ks = c;
    return ks;
}

size_t router_split_bytes(const Shape& s) { return router_uses_mfma(s) ? (size_t)3 * s.E * s.d * 2 : 0; }

// Large batches take the router product to the tiled GEMM (direct-to-LDS operand loads, 256 x
// 256 tiles): the 64-token blocks of router_mfma_kernel each reload all 3E rows of the split
// weight in MFMA operand layout, which bounds them by the L2-to-CU load rate. k is cut into the
// fewest parts (of 1, 2, 4, 8) that give at least two items per CU. 0: not this route.
constexpr int64_t kRouterGemmMinT = 2048;
constexpr int kRouterGemmItems = 512;
int router_gemm_ks(const Shape& s) {
    if (!router_uses_mfma(s) || s.T < kRouterGemmMinT || s.d % 128 != 0) return 0;
    int ks = 1;
    while (ks < 8 && gemm_router_items(s, ks) < kRouterGemmItems && s.d % (64 * 2 * ks) == 0) ks *= 2;
    return ks;
}

size_t router_zp_floats(const Shape& s) {
    const int gks = router_gemm_ks(s);
    if (gks) return (size_t)gks * s.T * 3 * s.E;
    return (size_t)router_ksplit(s) * s.T * s.E;
}

void launch_router(const Shape& s, const void* h, const void* norm_w, void* x_normed, const float* Wr,
                   const float* bias, void* wrs, float* z_part, int32_t* idx, float* w, float* logits, hipStream_t st) {
    const int gks = router_gemm_ks(s);
    const int ks = gks ? gks : router_ksplit(s);
    const int P = gks ? 3 : 1;
    const int epl = s.E <= 64 ? 1 : s.E / 64;
    const unsigned tb = (unsigned)((s.T + 63) / 64);
    const bool split = gks || (router_uses_mfma(s) && !((int64_t)tb * ks <= 256 && ks > 1));
    // the router reads x: the input itself, or the normed copy made here (with the weight split
    // when there is one, in the same launch)
    const void* x = norm_w ? x_normed : h;
    if (split && norm_w) {
        const unsigned nb = (unsigned)((s.T + kNormRows - 1) / kNormRows + (int64_t)(s.d / 64) * (s.E / 64));
        hipLaunchKernelGGL(router_prep_kernel, dim3(nb), dim3(256), 0, st, (const u16*)h, (const u16*)norm_w,
                           (u16*)x_normed, (double)s.eps, s.T, Wr, (u16*)wrs, s.d, s.E);
    } else if (split) {
        hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)(s.d / 64), (unsigned)(s.E / 64)), dim3(256), 0, st,
                           Wr, (u16*)wrs, s.d, s.E);
    } else if (norm_w) {
        launch_rmsnorm(s, h, norm_w, x_normed, st);
    }
    if (gks) {
        launch_gemm_router(s, x, wrs, z_part, gks, st);
    } else if (router_uses_mfma(s)) {
        const bool small = !split;
#define BEAM_RMMA(NTW, F)                                                                                        \
    hipLaunchKernelGGL((router_mfma_kernel<NTW, F>), dim3(tb, (unsigned)ks), dim3(256), 0, st, (const u16*)x,     \
                       (const u16*)wrs, z_part, s.T, s.d, s.E, s.d / ks, s.G, s.KG, s.K, s.S, s.norm, bias, idx, w, \
                       logits)
        if (ks == 1) {
            if (s.E == 256) BEAM_RMMA(4, true); else BEAM_RMMA(2, true);
            return;
        }
        if (small) {
            // few token blocks (decode): the experts of a block split over E/64 blocks, one 16-expert
            // tile per wave, for four times the blocks; each logit is summed in the same order
            hipLaunchKernelGGL((router_mfma_kernel<1, false, true>), dim3(tb, (unsigned)ks, (unsigned)(s.E / 64)),
                               dim3(256), 0, st, (const u16*)x, (const void*)Wr, z_part, s.T, s.d, s.E, s.d / ks, s.G,
                               s.KG, s.K, s.S, s.norm, bias, idx, w, logits);
        } else if (s.E == 256) {
            BEAM_RMMA(4, false);
        } else {
            BEAM_RMMA(2, false);
        }
#undef BEAM_RMMA
    } else {
        dim3 grid(tb, (unsigned)((s.E + RE - 1) / RE), (unsigned)ks);
        hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, st, (const u16*)x, Wr, z_part, s.T, s.d, s.E,
                           s.d / ks);
    }
    if (s.E == 256 && ks * P >= kQuartersMinParts && s.T <= kQuartersMaxT) {
        hipLaunchKernelGGL(router_topk_quarters_kernel, dim3((unsigned)s.T), dim3(256), 0, st, z_part, ks, s.T, s.E,
                           s.G, s.KG, s.K, s.S, s.norm, bias, idx, w, logits, P);
        return;
    }
    dim3 grid((unsigned)((s.T + 3) / 4));
#define BEAM_TOPK(N)                                                                                              \
    hipLaunchKernelGGL(router_topk_kernel<N>, grid, dim3(256), 0, st, z_part, ks, s.T, s.E, s.G, s.KG, s.K, s.S,  \
                       s.norm, bias, idx, w, logits, P)
    switch (epl) {
        case 1: BEAM_TOPK(1); break;
        case 2: BEAM_TOPK(2); break;
        case 4: BEAM_TOPK(4); break;
        case 8: BEAM_TOPK(8); break;
        default: BEAM_TOPK(16); break;
    }
#undef BEAM_TOPK
}

}  // namespace beam

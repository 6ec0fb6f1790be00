// FP8 expert weights for decode: OCP E4M3 elements with one power-of-two (E8M0) scale per
// 32 consecutive k of a weight row, the OCP Microscaling (MX) v1.0 FP8 layout. The pages
// name FP8 checkpoints (news.hamidun.com article, section on FP8 weights; strelka.ai
// overview of the release) but no scaling recipe; this layout is the published one gfx950's
// conversion and scaled-MFMA instructions are built around.
//
// Weights are stored as q [rows, K] bytes and s [rows, K/32] bytes; a value is
// 2^(s - 127) * e4m3(q). The codes may instead be in the packed layout (beam_moe_pack_weights
// on q viewed as [rows, K/2] 16-bit units): 16-row blocks of 64-k steps, each step the 1 KB
// one wave loads (lane l: row l % 16, bytes 64t + 16(l / 16) .. +16), so every load is
// contiguous; the scales stay row-major. The kernels stream q from HBM (half the bytes of bf16), widen it
// to bf16 in registers with v_cvt_scalef32_pk_bf16_fp8 (exact: an E4M3 value times a power
// of two has at most 4 significant bits) and run the same bf16 MFMAs with FP32
// accumulation as the bf16 path, so the layer computes exactly the bf16 layer on the
// dequantized weights.
#include "common.h"
#include "kernels.h"

namespace beam {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kD = 8;   // 64-k steps in flight per wave (8: one group of scale bytes)

// ---- quantization --------------------------------------------------------------------------

// Nearest E4M3 code to x, ties to the even mantissa, |x| >= 448 saturated to +-448.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t sgn = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fabsf(x);
    if (a >= 448.0f) return sgn | 0x7Eu;
    if (a < 0.015625f) return sgn | (uint32_t)rintf(a * 512.0f);     // multiples of 2^-9; 8 -> 2^-6
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;         // a is a normal float here
    int m = (int)rintf((ldexpf(a, -e) - 1.0f) * 8.0f);
    if (m == 8) {
        m = 0;
        ++e;
    }
    return sgn | (uint32_t)(((e + 7) << 3) | m);
}

// One thread per block of 32 values: shared exponent floor(log2(max |w|)) - 8 (clamped to
// the E8M0 range; 0 for a block of zeros), then every value divided by 2^shared is rounded.
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const u16* __restrict__ w, int64_t n_blocks,
                                                           uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= n_blocks) return;
    const u16* src = w + 32 * b;
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(src + 8 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * i + 2 * j] = __uint_as_float(raw[j] << 16);
            v[8 * i + 2 * j + 1] = __uint_as_float(raw[j] & 0xFFFF0000u);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    int shared = 0;
    if (amax > 0.0f) {
        int ex;
        frexpf(amax, &ex);                       // amax = f * 2^ex, f in [0.5, 1)
        shared = min(127, max(-127, ex - 1 - 8));
    }
    s[b] = (uint8_t)(shared + 127);
    u32x4 out[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) word |= e4m3_encode(ldexpf(v[4 * i + j], -shared)) << (8 * j);
        out[i / 4][i % 4] = word;
    }
    *reinterpret_cast<u32x4*>(q + 32 * b) = out[0];
    *reinterpret_cast<u32x4*>(q + 32 * b + 16) = out[1];
}

// ---- decode streaming --------------------------------------------------------------------

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 fp8 codes (two dwords) times the scale -> 8 bf16 (an MFMA operand).
__device__ __forceinline__ bf16x8 widen(uint32_t lo, uint32_t hi, float sc) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true);
    const u32x4 w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                     __builtin_bit_cast(uint32_t, d)};
    return __builtin_bit_cast(bf16x8, w);
}

// acc[m][b] += W_b . X_m^T over k in [0, K), K a multiple of 512, for RB blocks of 16 fp8
// weight rows and MT tiles of 16 tokens. In 64-k step t, lane (r = lane%16, c = lane/16)
// holds bytes 64t + 16c .. +16 of row r of each block and elements 64t + 16c .. +16 of its
// token rows, which feed two MFMAs (elements 0..7, then 8..15): the k order inside a step is
// the same for both operands, and each weight load covers 16 rows x 64 contiguous bytes.
// The token fragments of a step serve all RB blocks (for gate/up: the gate and up rows of
// the same channels), half the activation loads of one pass per block. Measured on MI355X
// at the decode workload it runs as fast as two passes (a second open row stream per wave
// costs what the saved loads gain); with 1-byte weights the activation loads, not the
// weights, hold these kernels below the bf16 kernels' share of HBM bandwidth.
// wq[b]: row r of block b + 16c bytes (packed: the lane's 16 bytes of step 0, steps 1 KB apart);
// ws[b]: its scale bytes; x: token rows + 16c elements.
template <int RB, int MT, bool PK>
__device__ __forceinline__ void stream_fp8(const uint8_t* const (&wq)[RB], const uint8_t* const (&ws)[RB],
                                           const u16* const (&x)[MT], int K, int c, f32x4 (&acc)[MT][RB]) {
    // weight bytes from one step to the next. Packed, a load reads a kilobyte that nothing else
    // reads in the call (non-temporal hint); row-major, consecutive steps read the two halves of
    // the same 128-byte lines (plain loads, which keep the line for the second half).
    constexpr int kWB = PK ? 1024 : 64;
    u32x4 wa[kD][RB];
    bf16x8 xa[kD][MT][2];
    const int nsteps = K / 64;
    const int last = nsteps - 1;
    // scale bytes of eight steps (16 blocks of 32) per 16-byte load; this lane needs block
    // 2t + c/2 of step t
    const int half = c >> 1;
    u32x4 sc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) sc[b] = *reinterpret_cast<const u32x4*>(ws[b]);
#pragma unroll
    for (int t = 0; t < kD; ++t) {
#pragma unroll
        for (int b = 0; b < RB; ++b)
            wa[t][b] = PK ? ld_once(wq[b] + kWB * t) : *reinterpret_cast<const u32x4*>(wq[b] + kWB * t);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            xa[t][m][0] = *reinterpret_cast<const bf16x8*>(x[m] + 64 * t);
            xa[t][m][1] = *reinterpret_cast<const bf16x8*>(x[m] + 64 * t + 8);
        }
    }
    for (int g = 0; g < nsteps; g += kD) {
        u32x4 sc_next[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b)
            sc_next[b] = *reinterpret_cast<const u32x4*>(ws[b] + 2 * min(g + kD, last - (kD - 1)));
#pragma unroll
        for (int t = 0; t < kD; ++t) {
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const uint32_t byte = (sc[b][t >> 1] >> (16 * (t & 1) + 8 * half)) & 0xFFu;
                const float s = __uint_as_float(byte << 23);       // 2^(byte - 127)
                const bf16x8 a0 = widen(wa[t][b][0], wa[t][b][1], s);
                const bf16x8 a1 = widen(wa[t][b][2], wa[t][b][3], s);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    acc[m][b] = mfma16(a0, xa[t][m][0], acc[m][b]);
                    acc[m][b] = mfma16(a1, xa[t][m][1], acc[m][b]);
                }
            }
            const int tn = min(g + kD + t, last);                  // clamped: in bounds, unused at the end
            const int kn = 64 * tn;
#pragma unroll
            for (int b = 0; b < RB; ++b)
                wa[t][b] = PK ? ld_once(wq[b] + (size_t)kWB * tn) : *reinterpret_cast<const u32x4*>(wq[b] + (size_t)kWB * tn);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                xa[t][m][0] = *reinterpret_cast<const bf16x8*>(x[m] + kn);
                xa[t][m][1] = *reinterpret_cast<const bf16x8*>(x[m] + kn + 8);
            }
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) sc[b] = sc_next[b];
    }
}

// h[beg+m, n] = bf16(silu(x_m . Wg[e,n]) * (x_m . Wu[e,n])) for the tokens m of expert e, fp8
// weights. grid: (ceil(I / 64), E); block: 4 waves of 16 output channels, each streaming its
// gate and up rows together.
template <bool PK>
__global__ __launch_bounds__(256) void swiglu_fp8_kernel(const u16* __restrict__ x, const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ sorted_pairs, int top_k,
                                                         const uint8_t* __restrict__ Wg, const uint8_t* __restrict__ Wu,
                                                         const uint8_t* __restrict__ sg, const uint8_t* __restrict__ su,
                                                         u16* __restrict__ h, int d, int I) {
    const int e = blockIdx.y;
    const int beg = offsets[e];
    const int n_e = offsets[e + 1] - beg;
    if (n_e <= 0) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * kWaves + wave) * 16;
    if (n0 >= I) return;
    const int r = lane & 15, c = lane >> 4;
    const size_t row = (size_t)e * I + n0 + r;
    for (int mb = 0; mb < n_e; mb += 16) {
        const int m = min(mb + r, n_e - 1);                         // rows past the end repeat a valid row
        const u16* const xp[1] = {x + (size_t)(sorted_pairs[beg + m] / top_k) * d + 16 * c};
        const size_t wo = PK ? (((size_t)e * I + n0) / 16 * (d / 64) * 64 + lane) * 16 : row * d + 16 * c;
        const uint8_t* const wq[2] = {Wg + wo, Wu + wo};
        const uint8_t* const ws[2] = {sg + row * (d / 32), su + row * (d / 32)};
        f32x4 acc[1][2] = {{{0, 0, 0, 0}, {0, 0, 0, 0}}};
        stream_fp8<2, 1, PK>(wq, ws, xp, d, c, acc);
        const f32x4 g = acc[0][0], u = acc[0][1];
        // lane holds channels n0 + 4c + i of token mb + r
        if (mb + r < n_e) {
            const uint32_t lo = (uint32_t)f32_to_bf16(silu_mul(g[0], u[0])) |
                                ((uint32_t)f32_to_bf16(silu_mul(g[1], u[1])) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(silu_mul(g[2], u[2])) |
                                ((uint32_t)f32_to_bf16(silu_mul(g[3], u[3])) << 16);
            *reinterpret_cast<uint2*>(h + (size_t)(beg + mb + r) * I + n0 + 4 * c) = make_uint2(lo, hi);
        }
    }
}

// y_perm[beg+m, n] = h[beg+m] . Wd[e,n] with fp8 Wd (the combine applies the routing weight).
// grid: (ceil(d / (64 * kDnRB)), E);
// block: 4 waves, each streaming kDnRB blocks of 16 output channels whose rows share the
// activation fragments (one 16-row block of 1-byte codes is only a 40 KB stream at I = 2560).
constexpr int kDnRB = 2;
template <bool PK>
__global__ __launch_bounds__(256) void down_fp8_kernel(const u16* __restrict__ h, const int32_t* __restrict__ offsets,
                                                       const uint8_t* __restrict__ Wd, const uint8_t* __restrict__ sd,
                                                       float* __restrict__ y_perm, int d, int I) {
    const int e = blockIdx.y;
    const int beg = offsets[e];
    const int n_e = offsets[e + 1] - beg;
    if (n_e <= 0) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * kWaves + wave) * 16 * kDnRB;
    if (n0 >= d) return;                                           // d % 512 == 0: all kDnRB blocks in range
    const int r = lane & 15, c = lane >> 4;
    for (int mb = 0; mb < n_e; mb += 16) {
        const u16* const hp[1] = {h + (size_t)(beg + min(mb + r, n_e - 1)) * I + 16 * c};
        const uint8_t* wq[kDnRB];
        const uint8_t* ws[kDnRB];
#pragma unroll
        for (int b = 0; b < kDnRB; ++b) {
            const size_t nb = (size_t)e * d + n0 + 16 * b, row = nb + r;
            wq[b] = Wd + (PK ? (nb / 16 * (I / 64) * 64 + lane) * 16 : row * I + 16 * c);
            ws[b] = sd + row * (I / 32);
        }
        f32x4 acc[1][kDnRB];
#pragma unroll
        for (int b = 0; b < kDnRB; ++b) acc[0][b] = f32x4{0, 0, 0, 0};
        stream_fp8<kDnRB, 1, PK>(wq, ws, hp, I, c, acc);
        if (mb + r < n_e) {
#pragma unroll
            for (int b = 0; b < kDnRB; ++b)
                *reinterpret_cast<float4*>(y_perm + (size_t)(beg + mb + r) * d + n0 + 16 * b + 4 * c) =
                    make_float4(acc[0][b][0], acc[0][b][1], acc[0][b][2], acc[0][b][3]);
        }
    }
}

}  // namespace

void launch_fp8_quantize(int64_t rows, int K, const void* w, void* q, void* s, hipStream_t st) {
    const int64_t n_blocks = rows * (K / 32);
    hipLaunchKernelGGL(fp8_quantize_kernel, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, st,
                       static_cast<const u16*>(w), n_blocks, static_cast<uint8_t*>(q), static_cast<uint8_t*>(s));
}

bool fp8_supports(const Shape& s) { return s.d % 512 == 0 && s.I % 512 == 0 && !experts_tiled(s); }

void launch_swiglu_fp8(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                       const void* Wg8, const void* Wu8, const void* sg, const void* su, void* h, hipStream_t st) {
#define BEAM_GU8(PK)                                                                                          \
    hipLaunchKernelGGL((swiglu_fp8_kernel<PK>), dim3((unsigned)((s.I + 63) / 64), (unsigned)s.E), dim3(256), 0, st, \
                       static_cast<const u16*>(x), offsets, sorted_pairs, s.K, static_cast<const uint8_t*>(Wg8),   \
                       static_cast<const uint8_t*>(Wu8), static_cast<const uint8_t*>(sg),                         \
                       static_cast<const uint8_t*>(su), static_cast<u16*>(h), s.d, s.I)
    if (s.packed) BEAM_GU8(true); else BEAM_GU8(false);
#undef BEAM_GU8
}

void launch_down_fp8(const Shape& s, const void* h, const int32_t* offsets, const void* Wd8, const void* sd,
                     float* y_perm, hipStream_t st) {
#define BEAM_DN8(PK)                                                                                          \
    hipLaunchKernelGGL((down_fp8_kernel<PK>), dim3((unsigned)((s.d + 64 * kDnRB - 1) / (64 * kDnRB)), (unsigned)s.E), \
                       dim3(256), 0, st,                                                                      \
                       static_cast<const u16*>(h), offsets, static_cast<const uint8_t*>(Wd8),                 \
                       static_cast<const uint8_t*>(sd), y_perm, s.d, s.I)
    if (s.packed) BEAM_DN8(true); else BEAM_DN8(false);
#undef BEAM_DN8
}

}  // namespace beam

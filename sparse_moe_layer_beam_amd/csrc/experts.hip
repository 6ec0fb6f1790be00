// Routed experts of the Beam MoE layer: grouped SwiGLU (gate/up) GEMM with the
// activation fused, grouped down-projection GEMM with the routing weight fused, and a
// deterministic combine. BF16 MFMA with FP32 accumulation; silu(g)*u in FP32; h is
// rounded to bf16 once, for the bf16 down GEMM.
//
// Method: Transformers "Beam" model page (Overview: sparse MoE item, FP32 SwiGLU note;
// BeamConfig: hidden_act silu, moe_intermediate_size) and archdb "Beam-1.0-501B-A23B"
// fact sheet (FFN rows: SwiGLU, no FFN biases; MoE rows: no shared expert, scaled sum).
//
// Weight-streaming form: the expert weights are the MFMA A operand (16 output channels x
// 32 k per v_mfma_f32_16x16x32_bf16) loaded straight from HBM into registers, the tokens
// of the expert are the B operand (16 tokens per tile). Each weight byte is read once per
// 64 tokens of its expert, which is once per call whenever an expert has <= 64 tokens.
#include "common.h"
#include "kernels.h"

namespace beam {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kChanPerWave = 32;   // two 16-channel MFMA tiles
constexpr int kMT = 4;             // 16-token tiles held in registers per pass

__device__ __forceinline__ bf16x8 ld8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// h[beg+m, n] = bf16(silu(x_m . Wg[e,n]) * (x_m . Wu[e,n])) for the tokens m of expert e.
// grid: (ceil(I / 128), E); block: 4 waves, each owning 32 output channels.
__global__ __launch_bounds__(256) void swiglu_stream_kernel(const u16* __restrict__ x,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ sorted_pairs, int K,
                                                            const u16* __restrict__ Wg, const u16* __restrict__ Wu,
                                                            u16* __restrict__ h, int d, int I) {
    const int e = blockIdx.y;
    const int beg = offsets[e];
    const int n_e = offsets[e + 1] - beg;
    if (n_e <= 0) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * kWavesPerBlock + wave) * kChanPerWave;
    if (n0 >= I) return;
    const int r16 = lane & 15, kq = (lane >> 4) * 8;
    const u16* g0 = Wg + ((size_t)e * I + n0 + r16) * d + kq;
    const u16* g1 = g0 + (size_t)16 * d;
    const u16* u0 = Wu + ((size_t)e * I + n0 + r16) * d + kq;
    const u16* u1 = u0 + (size_t)16 * d;
    for (int mb = 0; mb < n_e; mb += 16 * kMT) {
        const int ntile = min(kMT, (n_e - mb + 15) / 16);
        const u16* xp[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int m = min(mb + 16 * mt + r16, n_e - 1);   // rows past the end read a valid row; discarded
            xp[mt] = x + (size_t)(sorted_pairs[beg + m] / K) * d + kq;
        }
        f32x4 ag[kMT][2], au[kMT][2];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int r = 0; r < 2; ++r) { ag[mt][r] = f32x4{0, 0, 0, 0}; au[mt][r] = f32x4{0, 0, 0, 0}; }
#pragma unroll 2
        for (int k = 0; k < d; k += 32) {
            const bf16x8 wg0 = ld8(g0 + k), wg1 = ld8(g1 + k), wu0 = ld8(u0 + k), wu1 = ld8(u1 + k);
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
                if (mt < ntile) {
                    const bf16x8 xb = ld8(xp[mt] + k);
                    ag[mt][0] = mfma16(wg0, xb, ag[mt][0]);
                    ag[mt][1] = mfma16(wg1, xb, ag[mt][1]);
                    au[mt][0] = mfma16(wu0, xb, au[mt][0]);
                    au[mt][1] = mfma16(wu1, xb, au[mt][1]);
                }
            }
        }
        // lane holds channels n0 + 16r + 4*(lane/16) + i for token row mb + 16*mt + lane%16
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int m = mb + 16 * mt + r16;
            if (mt >= ntile || m >= n_e) continue;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int n = n0 + 16 * r + (lane >> 4) * 4;
                uint32_t lo = (uint32_t)f32_to_bf16(silu_mul(ag[mt][r][0], au[mt][r][0])) |
                              ((uint32_t)f32_to_bf16(silu_mul(ag[mt][r][1], au[mt][r][1])) << 16);
                uint32_t hi = (uint32_t)f32_to_bf16(silu_mul(ag[mt][r][2], au[mt][r][2])) |
                              ((uint32_t)f32_to_bf16(silu_mul(ag[mt][r][3], au[mt][r][3])) << 16);
                *reinterpret_cast<uint2*>(h + (size_t)(beg + m) * I + n) = make_uint2(lo, hi);
            }
        }
    }
}

// y_perm[beg+m, c] = w_pair * (h[beg+m] . Wd[e,c]) for the tokens m of expert e.
// grid: (ceil(d / 128), E).
__global__ __launch_bounds__(256) void down_stream_kernel(const u16* __restrict__ h,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_pairs,
                                                          const float* __restrict__ topk_w,
                                                          const u16* __restrict__ Wd, float* __restrict__ y_perm,
                                                          int d, int I) {
    const int e = blockIdx.y;
    const int beg = offsets[e];
    const int n_e = offsets[e + 1] - beg;
    if (n_e <= 0) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = (blockIdx.x * kWavesPerBlock + wave) * kChanPerWave;
    if (n0 >= d) return;
    const int r16 = lane & 15, kq = (lane >> 4) * 8;
    const u16* w0 = Wd + ((size_t)e * d + n0 + r16) * I + kq;
    const u16* w1 = w0 + (size_t)16 * I;
    for (int mb = 0; mb < n_e; mb += 16 * kMT) {
        const int ntile = min(kMT, (n_e - mb + 15) / 16);
        const u16* hp[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) hp[mt] = h + (size_t)(beg + min(mb + 16 * mt + r16, n_e - 1)) * I + kq;
        f32x4 acc[kMT][2];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) { acc[mt][0] = f32x4{0, 0, 0, 0}; acc[mt][1] = f32x4{0, 0, 0, 0}; }
#pragma unroll 2
        for (int k = 0; k < I; k += 32) {
            const bf16x8 a0 = ld8(w0 + k), a1 = ld8(w1 + k);
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
                if (mt < ntile) {
                    const bf16x8 hb = ld8(hp[mt] + k);
                    acc[mt][0] = mfma16(a0, hb, acc[mt][0]);
                    acc[mt][1] = mfma16(a1, hb, acc[mt][1]);
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int m = mb + 16 * mt + r16;
            if (mt >= ntile || m >= n_e) continue;
            const float wt = topk_w[sorted_pairs[beg + m]];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int c = n0 + 16 * r + (lane >> 4) * 4;
                float4 v = make_float4(wt * acc[mt][r][0], wt * acc[mt][r][1], wt * acc[mt][r][2], wt * acc[mt][r][3]);
                *reinterpret_cast<float4*>(y_perm + (size_t)(beg + m) * d + c) = v;
            }
        }
    }
}

// y[t] = sum over slots j = 0..K-1, in that order, of y_perm[pair_rank[t*K + j]].
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ pair_rank, int K, int d,
                                                      float* __restrict__ y) {
    const int64_t t = blockIdx.x;
    __shared__ int rk[16];
    if (threadIdx.x < K) rk[threadIdx.x] = pair_rank[t * K + threadIdx.x];
    __syncthreads();
    for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
        float4 acc = *reinterpret_cast<const float4*>(y_perm + (size_t)rk[0] * d + c);
        for (int j = 1; j < K; ++j) {
            const float4 v = *reinterpret_cast<const float4*>(y_perm + (size_t)rk[j] * d + c);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        *reinterpret_cast<float4*>(y + t * d + c) = acc;
    }
}

}  // namespace

int experts_tile_m(const Shape&) { return 64; }

void launch_swiglu(const Shape& s, const void* x, const int32_t* offsets, const int32_t* sorted_pairs,
                   const int32_t* /*tiles*/, const int32_t* /*n_tiles*/, const void* Wg, const void* Wu, void* h,
                   hipStream_t st) {
    const int per_block = kWavesPerBlock * kChanPerWave;
    hipLaunchKernelGGL(swiglu_stream_kernel, dim3((unsigned)((s.I + per_block - 1) / per_block), (unsigned)s.E),
                       dim3(256), 0, st, (const u16*)x, offsets, sorted_pairs, s.K, (const u16*)Wg, (const u16*)Wu,
                       (u16*)h, s.d, s.I);
}

void launch_down(const Shape& s, const void* h, const int32_t* offsets, const int32_t* sorted_pairs,
                 const float* topk_w, const int32_t* /*tiles*/, const int32_t* /*n_tiles*/, const void* Wd,
                 float* y_perm, hipStream_t st) {
    const int per_block = kWavesPerBlock * kChanPerWave;
    hipLaunchKernelGGL(down_stream_kernel, dim3((unsigned)((s.d + per_block - 1) / per_block), (unsigned)s.E),
                       dim3(256), 0, st, (const u16*)h, offsets, sorted_pairs, topk_w, (const u16*)Wd, y_perm, s.d,
                       s.I);
}

void launch_combine(const Shape& s, const float* y_perm, const int32_t* pair_rank, float* y, hipStream_t st) {
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)s.T), dim3(256), 0, st, y_perm, pair_rank, s.K, s.d, y);
}

}  // namespace beam

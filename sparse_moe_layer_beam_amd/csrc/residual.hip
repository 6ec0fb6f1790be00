// Post-MLP half of the sandwich norm and the depth-scaled FP32 residual add, fused into
// the combine of the expert outputs (Transformers "Beam" page, Overview: sandwich norms
// item and FP32 RMSNorm note; archdb "Beam-1.0-501B-A23B" fact sheet, normalisation and
// residual rows; news.hamidun.com article, section on the unusual residual stream).
//
// For token t, with y[t] = sum over its K slots of the weighted expert rows (slot order):
//   n[t]         = y[t] * rsqrt(mean_j y[t,j]^2 + eps) * w        (FP32, not rounded)
//   resid_out[t] = resid[t] * keep + n[t] * add,   keep = sqrt((k-1)/k), add = 1/sqrt(k)
// One block per token keeps the whole row in registers between the sum of squares and
// the output, so y is never written unless the caller asks for it: the combine's HBM
// traffic grows only by the residual read and write. Batches of fewer than 1024 tokens
// leave most CUs idle, so there a block has 1024 threads (one or two float4 of the row
// each) to keep more loads in flight per token; larger batches use 256.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace beam {
namespace {


__device__ __forceinline__ float4 add4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

// w * v rounded to FP32 on its own (never contracted with the add that follows into an FMA).
__device__ __forceinline__ float4 mul4(float w, float4 v) {
#pragma clang fp contract(off)
    return make_float4(w * v.x, w * v.y, w * v.z, w * v.w);
}

// A float4 of Y_perm, which the combine reads once (non-temporal).
__device__ __forceinline__ float4 ld4_once(const float* p) {
    const u32x4 r = ld_once(p);
    return make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w));
}

// COMBINE: src is Y_perm [T*K, d] read through pair_rank, slot j weighted by topk_w[t, j] (each
// product rounded to FP32 on its own, then added in slot order); else src is y [T, d].
template <bool COMBINE, int kThreads>
__global__ __launch_bounds__(kThreads) void post_residual_kernel(const float* __restrict__ src,
                                                                 const int32_t* __restrict__ pair_rank,
                                                                 const float* __restrict__ topk_w, int K,
                                                                 int d, const u16* __restrict__ w, float keep,
                                                                 float add, float eps,
                                                                 const float* resid, float* resid_out,
                                                                 float* __restrict__ y_out) {
    constexpr int kMaxV = kPostMaxD / (4 * kThreads);   // float4 chunks per thread
    __shared__ float red[kThreads / kWave];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int nq = d >> 2;
    float4 v[kMaxV];
    if constexpr (COMBINE) {
        int rk[16];
        float wt[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            rk[j] = j < K ? pair_rank[t * K + j] : 0;
            wt[j] = j < K ? topk_w[t * K + j] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kMaxV; ++i) {
            const int q = tid + i * kThreads;
            if (q < nq) {
                float4 acc = mul4(wt[0], ld4_once(src + (size_t)rk[0] * d + 4 * q));
#pragma unroll
                for (int j = 1; j < 16; ++j)
                    if (j < K) acc = add4(acc, mul4(wt[j], ld4_once(src + (size_t)rk[j] * d + 4 * q)));
                v[i] = acc;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kMaxV; ++i) {
            const int q = tid + i * kThreads;
            if (q < nq) v[i] = *reinterpret_cast<const float4*>(src + t * d + 4 * q);
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxV; ++i) {
        const int q = tid + i * kThreads;
        if (q < nq) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) tot += red[i];
    const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
    for (int i = 0; i < kMaxV; ++i) {
        const int q = tid + i * kThreads;
        if (q < nq) {
            const uint2 wb = *reinterpret_cast<const uint2*>(w + 4 * q);
            const float w0 = __uint_as_float(wb.x << 16), w1 = __uint_as_float(wb.x & 0xffff0000u);
            const float w2 = __uint_as_float(wb.y << 16), w3 = __uint_as_float(wb.y & 0xffff0000u);
            const size_t o = (size_t)t * d + 4 * q;
            const float4 rs = *reinterpret_cast<const float4*>(resid + o);
            float4 out;
            out.x = rs.x * keep + (v[i].x * r * w0) * add;
            out.y = rs.y * keep + (v[i].y * r * w1) * add;
            out.z = rs.z * keep + (v[i].z * r * w2) * add;
            out.w = rs.w * keep + (v[i].w * r * w3) * add;
            *reinterpret_cast<float4*>(resid_out + o) = out;
            if (y_out) *reinterpret_cast<float4*>(y_out + o) = v[i];
        }
    }
}

void residual_factors(int layer, float* keep, float* add) {
    const double k = 2.0 * (layer + 1) + 1.0;   // the MLP of 0-indexed layer i is contribution 2(i+1)+1
    *keep = (float)std::sqrt((k - 1.0) / k);
    *add = (float)(1.0 / std::sqrt(k));
}

constexpr int kSmallBatch = 1024;

}  // namespace

void launch_combine_post_residual(const Shape& s, const float* y_perm, const int32_t* pair_rank, const float* topk_w,
                                  const void* post_w, int layer, const float* resid, float* resid_out, float* y,
                                  hipStream_t st) {
    float keep, add;
    residual_factors(layer, &keep, &add);
    const u16* w = static_cast<const u16*>(post_w);
    if (s.T < kSmallBatch)
        hipLaunchKernelGGL((post_residual_kernel<true, 1024>), dim3((unsigned)s.T), dim3(1024), 0, st, y_perm,
                           pair_rank, topk_w, s.K, s.d, w, keep, add, s.eps, resid, resid_out, y);
    else
        hipLaunchKernelGGL((post_residual_kernel<true, 256>), dim3((unsigned)s.T), dim3(256), 0, st, y_perm,
                           pair_rank, topk_w, s.K, s.d, w, keep, add, s.eps, resid, resid_out, y);
}

void launch_post_residual(const Shape& s, const float* y, const void* post_w, int layer, const float* resid,
                          float* resid_out, hipStream_t st) {
    float keep, add;
    residual_factors(layer, &keep, &add);
    const u16* w = static_cast<const u16*>(post_w);
    if (s.T < kSmallBatch)
        hipLaunchKernelGGL((post_residual_kernel<false, 1024>), dim3((unsigned)s.T), dim3(1024), 0, st, y, nullptr,
                           nullptr, 0, s.d, w, keep, add, s.eps, resid, resid_out, nullptr);
    else
        hipLaunchKernelGGL((post_residual_kernel<false, 256>), dim3((unsigned)s.T), dim3(256), 0, st, y, nullptr,
                           nullptr, 0, s.d, w, keep, add, s.eps, resid, resid_out, nullptr);
}

}  // namespace beam

// Seeded synthetic inputs, device side: the same per-element definitions as
// synth_host.c (Philox4x32-10 of Salmon et al., SC'11; Box & Muller normals;
// double arithmetic with no contraction; one rounding to fp32, then RNE to bf16),
// written for gfx950 so that tens of GB of expert weights are produced in HBM
// directly. Holds no arithmetic of the MoE layer. Built with -ffp-contract=off.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;

__device__ __forceinline__ uint4 philox10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += kW0; k1 += kW1; }
        uint32_t lo0 = kM0 * c.x, hi0 = __umulhi(kM0, c.x);
        uint32_t lo1 = kM1 * c.z, hi1 = __umulhi(kM1, c.z);
        uint4 n;
        n.x = hi1 ^ c.y ^ k0;
        n.y = lo1;
        n.z = hi0 ^ c.w ^ k1;
        n.w = lo0;
        c = n;
    }
    return c;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

__device__ __forceinline__ double normal_value(uint64_t seed, uint32_t tid, int64_t i, double mean, double stdv) {
    uint64_t q = (uint64_t)i >> 1;
    uint4 w = philox10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), tid, 0u), (uint32_t)seed, (uint32_t)(seed >> 32));
    uint64_t a = (((uint64_t)w.y << 32) | w.x) >> 11;
    uint64_t b = (((uint64_t)w.w << 32) | w.z) >> 11;
    double u1 = ((double)a + 0.5) * 0x1p-53;
    double u2 = (double)b * 0x1p-53;
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586 * u2;
    double z = (i & 1) ? r * sin(th) : r * cos(th);
    double s = stdv * z;
    return mean + s;
}

__device__ __forceinline__ double uniform_value(uint64_t seed, uint32_t tid, int64_t i, double lo, double hi) {
    uint4 w = philox10(make_uint4((uint32_t)(uint64_t)i, (uint32_t)((uint64_t)i >> 32), tid, 1u),
                       (uint32_t)seed, (uint32_t)(seed >> 32));
    uint64_t a = (((uint64_t)w.y << 32) | w.x) >> 11;
    double u = (double)a * 0x1p-53;
    double span = hi - lo;
    double s = span * u;
    return lo + s;
}

__global__ void fill_kernel(void* dst, int dtype, int law, int64_t start, int64_t n, uint64_t seed,
                            uint32_t tid, double p0, double p1) {
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride) {
        int64_t i = start + k;
        double v = law == 0 ? normal_value(seed, tid, i, p0, p1) : uniform_value(seed, tid, i, p0, p1);
        float f = (float)v;
        if (dtype == 0) ((float*)dst)[k] = f;
        else ((uint16_t*)dst)[k] = f32_to_bf16_rne(f);
    }
}

int launch(void* dst, int dtype, int law, int64_t start, int64_t n, uint64_t seed, uint32_t tid,
           double p0, double p1, void* stream) {
    if (n <= 0) return 0;
    if (!dst || (dtype != 0 && dtype != 1)) return 1;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       dst, dtype, law, start, n, seed, tid, p0, p1);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace

extern "C" int synth_dev_fill_normal(void* dst, int dtype, int64_t start, int64_t n, uint64_t seed,
                                     uint32_t tid, double mean, double stdv, void* stream) {
    return launch(dst, dtype, 0, start, n, seed, tid, mean, stdv, stream);
}

extern "C" int synth_dev_fill_uniform(void* dst, int dtype, int64_t start, int64_t n, uint64_t seed,
                                      uint32_t tid, double lo, double hi, void* stream) {
    return launch(dst, dtype, 1, start, n, seed, tid, lo, hi, stream);
}

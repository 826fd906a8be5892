// pool.hip -- HISA block pooling on gfx950 (HISA abstract, stage (1): the
// pooled block representatives the coarse filter scores).
//
// pooled[b, j, d] = bf16_nearest_even(mean of k[b, s, d] over s in block j).
// The sum runs in fp64 in ascending key order, the order of the definition
// (exact for bf16 keys; for fp8 keys each scale * e4m3fn product is exact in
// fp64), so the fp64 mean is reproduced bit for bit and the rounding to bf16
// is the only one.  fp64 -> bf16 goes through a
// round-to-odd fp32 intermediate, which keeps that rounding single.
//
// A thread owns 4 consecutive dims of one block and walks its keys; a wave
// covers 64 / (D/4) blocks, and the kernel streams the key cache once: it
// is HBM-bound.
#include "tks_launch.hpp"

namespace tks {

namespace {

__device__ inline uint16_t f64_to_bf16_rne(double x) {
    // round-to-odd to fp32 (24 bits >= 8 + 2), then nearest-even to bf16
    float f = __double2float_rz(x);
    if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <bool FP8>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a, int64_t n_threads) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_threads) return;
    const int tpb = a.dim / 4;
    const int64_t nb = a.n_k / a.block;
    const int64_t bj = gid / tpb;  // b * nb + j
    const int d0 = (int)(gid % tpb) * 4;
    const int64_t b = bj / nb, j = bj % nb;
    const int64_t s0 = b * a.n_k + j * a.block;
    double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
    if (FP8) {
        const uint8_t* base = reinterpret_cast<const uint8_t*>(a.k) + s0 * a.dim + d0;
        const float* sc = a.k_scale + s0;
#pragma unroll 16
        for (int s = 0; s < a.block; ++s) {
            const uint32_t c = *reinterpret_cast<const uint32_t*>(base + (int64_t)s * a.dim);
            const double scale = (double)sc[s];
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);
            // scale * code is exact in fp64, so one fused rounding = add
            acc0 = fma(scale, (double)lo[0], acc0);
            acc1 = fma(scale, (double)lo[1], acc1);
            acc2 = fma(scale, (double)hi[0], acc2);
            acc3 = fma(scale, (double)hi[1], acc3);
        }
    } else {
        const uint16_t* base = reinterpret_cast<const uint16_t*>(a.k) + s0 * a.dim + d0;
#pragma unroll 16
        for (int s = 0; s < a.block; ++s) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(base + (int64_t)s * a.dim);
            acc0 += (double)__uint_as_float(v[0] << 16);
            acc1 += (double)__uint_as_float(v[0] & 0xFFFF0000u);
            acc2 += (double)__uint_as_float(v[1] << 16);
            acc3 += (double)__uint_as_float(v[1] & 0xFFFF0000u);
        }
    }
    const double n = (double)a.block;
    uint16_t* o = a.out + bj * a.dim + d0;
    const uint32_t p0 = (uint32_t)f64_to_bf16_rne(acc0 / n) |
                        ((uint32_t)f64_to_bf16_rne(acc1 / n) << 16);
    const uint32_t p1 = (uint32_t)f64_to_bf16_rne(acc2 / n) |
                        ((uint32_t)f64_to_bf16_rne(acc3 / n) << 16);
    *reinterpret_cast<u32x2*>(o) = u32x2{p0, p1};
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, bool fp8, hipStream_t stream) {
    const int64_t nb = a.n_k / a.block;
    const int64_t n_threads = (int64_t)a.batch * nb * (a.dim / 4);
    if (n_threads <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((n_threads + 255) / 256);
    if (fp8)
        hipLaunchKernelGGL(pool_kernel<true>, dim3(grid), dim3(256), 0, stream, a, n_threads);
    else
        hipLaunchKernelGGL(pool_kernel<false>, dim3(grid), dim3(256), 0, stream, a, n_threads);
    return hipGetLastError();
}

}  // namespace tks

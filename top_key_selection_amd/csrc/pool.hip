// pool.hip -- HISA block pooling on gfx950 (HISA abstract, stage (1): the
// pooled block representatives the coarse filter scores).
//
// pooled[b, j, d] = bf16_nearest_even(mean of k[b, s, d] over s in block j).
// The sum runs in fp64 in ascending key order, the order of the definition
// (exact for bf16 keys; for fp8 keys each scale * e4m3fn product is exact in
// fp64), so the fp64 mean is reproduced bit for bit and the rounding to bf16
// is the only one.  fp64 -> bf16 goes through a round-to-odd fp32
// intermediate, which keeps that rounding single.
//
// The kernel streams the key cache once and is HBM-bound.  A workgroup of
// 256 threads owns G = 256 / D consecutive blocks, one thread per (block,
// dim).  Keys are staged through LDS in chunks of up to 64 rows: the
// workgroup reads each block's chunk as one contiguous run with 16-byte
// loads, then every thread walks its column of the chunk in key order.
#include "tks_launch.hpp"

namespace tks {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;  // key rows staged per block and step

__device__ inline uint16_t f64_to_bf16_rne(double x) {
    // round-to-odd to fp32 (24 bits >= 8 + 2), then nearest-even to bf16
    float f = __double2float_rz(x);
    if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <bool FP8, int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(PoolArgs a, int64_t n_blocks) {
    constexpr int G = kThreads / D;              // blocks per workgroup
    constexpr int ROW = FP8 ? D : 2 * D;         // bytes per key row
    constexpr int STRIDE = kChunk * ROW;         // LDS bytes per block
    __shared__ __align__(16) uint8_t s_keys[G * STRIDE];
    __shared__ float s_scale[FP8 ? G * kChunk : 1];

    const int tid = threadIdx.x;
    const int g = tid / D, d = tid % D;
    const int64_t nb = a.n_k / a.block;
    const int64_t bj0 = (int64_t)blockIdx.x * G;
    const int64_t bj = bj0 + g;                  // this thread's block
    const int ch = a.block < kChunk ? a.block : kChunk;
    const int vec_per_block = ch * ROW / 16;
    double acc = 0.0;

    for (int c0 = 0; c0 < a.block; c0 += ch) {
        // stage rows c0 .. c0+ch-1 of every block of the workgroup
        for (int v = tid; v < G * vec_per_block; v += kThreads) {
            const int gg = v / vec_per_block, off = (v % vec_per_block) * 16;
            const int64_t b2 = bj0 + gg;
            if (b2 < n_blocks) {
                const int64_t row0 = (b2 / nb) * a.n_k + (b2 % nb) * a.block + c0;
                // each block chunk is contiguous: whole lines, streamed once
                const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                    reinterpret_cast<const uint8_t*>(a.k) + row0 * ROW + off));
                *reinterpret_cast<u32x4*>(&s_keys[gg * STRIDE + off]) = x;
            }
        }
        if (FP8) {
            for (int v = tid; v < G * ch; v += kThreads) {
                const int gg = v / ch, s = v % ch;
                const int64_t b2 = bj0 + gg;
                if (b2 < n_blocks)
                    s_scale[gg * kChunk + s] =
                        a.k_scale[(b2 / nb) * a.n_k + (b2 % nb) * a.block + c0 + s];
            }
        }
        __syncthreads();
        if (bj < n_blocks) {
            const uint8_t* col = &s_keys[g * STRIDE];
#pragma unroll 8
            for (int s = 0; s < ch; ++s) {
                if (FP8) {
                    const int code = col[s * ROW + d];
                    const float v = __builtin_amdgcn_cvt_f32_fp8(code, 0);
                    // scale * code is exact in fp64, so one fused rounding = add
                    acc = fma((double)s_scale[g * kChunk + s], (double)v, acc);
                } else {
                    const uint32_t h = *reinterpret_cast<const uint16_t*>(col + s * ROW + 2 * d);
                    acc += (double)__uint_as_float(h << 16);
                }
            }
        }
        __syncthreads();
    }
    if (bj < n_blocks) a.out[bj * D + d] = f64_to_bf16_rne(acc / (double)a.block);
}

template <bool FP8, int D>
void launch_d(const PoolArgs& a, int64_t n_blocks, hipStream_t stream) {
    constexpr int G = kThreads / D;
    const unsigned grid = (unsigned)((n_blocks + G - 1) / G);
    hipLaunchKernelGGL((pool_kernel<FP8, D>), dim3(grid), dim3(kThreads), 0, stream, a, n_blocks);
}

template <bool FP8>
void launch_fp(const PoolArgs& a, int64_t n_blocks, hipStream_t stream) {
    if (a.dim == 32)
        launch_d<FP8, 32>(a, n_blocks, stream);
    else if (a.dim == 64)
        launch_d<FP8, 64>(a, n_blocks, stream);
    else
        launch_d<FP8, 128>(a, n_blocks, stream);
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, bool fp8, hipStream_t stream) {
    const int64_t n_blocks = (int64_t)a.batch * (a.n_k / a.block);
    if (n_blocks <= 0) return hipSuccess;
    if (fp8)
        launch_fp<true>(a, n_blocks, stream);
    else
        launch_fp<false>(a, n_blocks, stream);
    return hipGetLastError();
}

}  // namespace tks

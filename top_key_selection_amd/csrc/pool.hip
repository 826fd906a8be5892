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
// The kernel streams the key cache once and is HBM-bound.  Each thread owns
// one 16-byte column piece of one block (16 fp8 or 8 bf16 dimensions) and
// walks the block's key rows in order, so every output keeps the sequential
// sum; two batches of four rows are in flight, one summed while the next
// loads (nontemporal 16-byte loads: every key byte is read exactly once).  The threads of a wave cover one row of
// several consecutive blocks, each as whole 128-byte lines.
#include "tks_launch.hpp"

namespace tks {

namespace {

constexpr int kThreads = 64;  // one wave per workgroup: many small workgroups spread best
constexpr int kAhead = 4;  // key rows per batch (two batches in flight)

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
    constexpr int EPT = FP8 ? 16 : 8;   // key elements per 16-byte piece
    constexpr int TPB = D / EPT;         // threads per block (pieces per row)
    constexpr int ROW = FP8 ? D : 2 * D; // bytes per key row
    const int64_t gt = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t bj = gt / TPB;         // pooled block over all sequences
    const int part = (int)(gt % TPB);
    if (bj >= n_blocks) return;
    const int64_t nb = a.n_k / a.block;
    const int64_t row0 = (bj / nb) * a.n_k + (bj % nb) * a.block;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.k) + row0 * ROW + part * 16;
    const float* scl = FP8 ? a.k_scale + row0 : nullptr;

    double acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.0;
    // two batches of kAhead rows: one is summed while the next is in flight
    u32x4 va[kAhead], vb[kAhead];
    float sa[kAhead], sb[kAhead];
    auto load = [&](u32x4* v, float* sc, int s0) {
#pragma unroll
        for (int i = 0; i < kAhead; ++i)
            v[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(src + (int64_t)(s0 + i) * ROW));
        if (FP8) {
#pragma unroll
            for (int i = 0; i < kAhead; ++i) sc[i] = scl[s0 + i];
        }
    };
    auto add = [&](const u32x4* v, const float* sc) {
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
            if constexpr (FP8) {
                // scale * code is exact in fp64, so the fma rounds once, like
                // the sum of the exact products
                const double sd = (double)sc[i];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i][w], false);
                    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[i][w], true);
                    acc[4 * w + 0] = fma(sd, (double)lo[0], acc[4 * w + 0]);
                    acc[4 * w + 1] = fma(sd, (double)lo[1], acc[4 * w + 1]);
                    acc[4 * w + 2] = fma(sd, (double)hi[0], acc[4 * w + 2]);
                    acc[4 * w + 3] = fma(sd, (double)hi[1], acc[4 * w + 3]);
                }
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    acc[2 * w + 0] += (double)__uint_as_float(v[i][w] << 16);
                    acc[2 * w + 1] += (double)__uint_as_float(v[i][w] & 0xFFFF0000u);
                }
            }
        }
    };
    // the block size is a multiple of 2 * kAhead (32 .. 256)
    load(va, sa, 0);
    for (int s0 = 0; s0 < a.block; s0 += 2 * kAhead) {
        load(vb, sb, s0 + kAhead);
        add(va, sa);
        if (s0 + 2 * kAhead < a.block) load(va, sa, s0 + 2 * kAhead);
        add(vb, sb);
    }
    // EPT bf16 results = 16 (bf16) or 32 (fp8) contiguous bytes
    uint32_t o[EPT / 2];
#pragma unroll
    for (int e = 0; e < EPT / 2; ++e)
        o[e] = (uint32_t)f64_to_bf16_rne(acc[2 * e] / (double)a.block) |
               ((uint32_t)f64_to_bf16_rne(acc[2 * e + 1] / (double)a.block) << 16);
    u32x4* dst = reinterpret_cast<u32x4*>(a.out + bj * D + part * EPT);
#pragma unroll
    for (int e = 0; e < EPT / 8; ++e) dst[e] = u32x4{o[4 * e], o[4 * e + 1], o[4 * e + 2], o[4 * e + 3]};
}

template <bool FP8, int D>
void launch_d(const PoolArgs& a, int64_t n_blocks, hipStream_t stream) {
    constexpr int TPB = D / (FP8 ? 16 : 8);
    const unsigned grid = (unsigned)((n_blocks * TPB + kThreads - 1) / kThreads);
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

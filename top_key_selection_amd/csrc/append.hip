// append.hip -- key-cache append on gfx950: key compression, fp8
// quantisation and HISA block pooling fused into one pass (StreamIndex
// abstract: the indexer reads keys compressed by a ratio m; HISA abstract,
// stage (1): pooled block representatives).
//
// A call appends n_new raw bf16 keys to every sequence of the batch, whose
// raw streams already hold raw_len keys.  Compressed key j, the mean of raw
// keys m*j .. m*j+m-1 (summed in fp64 in position order, rounded once to
// bf16), is complete when its last raw key arrives; it is written to the key
// cache, as bf16 or as e4m3fn codes of kc / scale with scale = max|kc| / 448.
// Pooled block J, the mean of compressed keys J*B .. J*B+B-1, is complete
// with its last compressed key and is written in the same pass from the
// values just produced, so keeping the pooled keys current never re-reads
// the cache.  Raw keys of a group still open at the end of the call wait in
// a caller-owned staging buffer (slot = raw position mod m).
//
// Work split: a job is (sequence, block J) over the groups of J this call
// completes.  D/8 threads each own 8 dimensions (one 16-byte bf16 piece) and
// walk the job's raw keys in position order, four 16-byte loads in flight,
// so each compressed key and each pooled sum keeps the order of its
// definition.  Compressed keys of J that earlier calls wrote are summed
// first, read back from the cache.  The job holding the first group of the
// call also moves the staging buffer: its threads read the old staged keys
// of that group before they stage the new ones, and no other thread touches
// a slot.
//
// A call that stays inside one block per sequence (a decode append) takes a
// workgroup per sequence instead: all its threads copy the block's earlier
// compressed keys to LDS at once (one memory round trip instead of one per
// few keys), then one thread per dimension sums them from LDS in key order
// and hands the sums to the D/8 owner threads.
#include "tks_launch.hpp"

namespace tks {

namespace {

constexpr int kThreads = 256;
constexpr int kAhead = 4;  // raw (or cached) key rows in flight per thread
constexpr int kStageMax = 255;  // earlier keys of a block staged in LDS (block <= 256)

// fp64 -> bf16, nearest-even: round-to-odd to fp32 (24 bits >= 8 + 2), then
// nearest-even to bf16, which keeps the rounding single.
__device__ inline uint32_t f64_to_bf16(double x) {
    float f = __double2float_rz(x);
    if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// OCP e4m3fn codes of four values (byte i = x[i]): nearest magnitude, ties
// to the even code, sign kept, saturated at 448 -- the clamp keeps every
// input inside the finite range, where v_cvt_pk_fp8_f32 rounds to nearest
// even.
__device__ inline uint32_t e4m3fn_x4(const float* x) {
    float c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_fmed3f(x[i], -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
    return (uint32_t)w;
}

__device__ inline void add_bf16x8(double* acc, const u32x4& v) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        acc[2 * w + 0] += (double)__uint_as_float(v[w] << 16);
        acc[2 * w + 1] += (double)__uint_as_float(v[w] & 0xFFFF0000u);
    }
}

// acc += scale * e4m3fn(codes) (8 codes); the product is exact in fp64, so
// the fma rounds once, like the sum of the exact products
__device__ inline void add_fp8x8(double* acc, uint32_t c0, uint32_t c1, float scale) {
    const double sd = (double)scale;
    const uint32_t c[2] = {c0, c1};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[w], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[w], true);
        acc[4 * w + 0] = fma(sd, (double)lo[0], acc[4 * w + 0]);
        acc[4 * w + 1] = fma(sd, (double)lo[1], acc[4 * w + 1]);
        acc[4 * w + 2] = fma(sd, (double)hi[0], acc[4 * w + 2]);
        acc[4 * w + 3] = fma(sd, (double)hi[1], acc[4 * w + 3]);
    }
}

template <bool FP8, int D, bool M1, bool STAGE>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
    constexpr int TPG = D / 8;  // threads per key (8 dims each)
    const int64_t gt = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    // STAGE: one job per workgroup; threads past TPG only help stage
    const int64_t job = STAGE ? (int64_t)blockIdx.x : gt / TPG;
    const int piece = STAGE ? (int)threadIdx.x : (int)(gt % TPG);
    if (job >= (int64_t)a.batch * a.n_jobs) return;
    const int32_t b = (int32_t)(job / a.n_jobs);
    const int32_t J = a.J0 + (int32_t)(job % a.n_jobs);
    const int32_t m = M1 ? 1 : a.m;
    const int32_t gs = max(a.g0, J * a.span);          // groups completed here
    const int32_t ge = min(a.g1, (J + 1) * a.span);
    const bool pool = a.pooled != nullptr && (J + 1) * a.span <= a.g1;
    const int64_t kbase = (int64_t)b * a.n_k;
    const int64_t raw_len = a.raw_len;

    double pacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pacc[e] = 0.0;

    // compressed keys of block J that earlier calls wrote, in key order
    if (STAGE && pool) {
        constexpr int KB = FP8 ? D : 2 * D;  // bytes per cached key
        __shared__ __align__(16) uint8_t s_k[STAGE ? kStageMax * KB : 16];
        __shared__ float s_s[STAGE ? kStageMax : 1];
        __shared__ double s_sum[STAGE ? D : 1];
        const int32_t n_back = gs - J * a.span;  // < block size <= 256
        const uint8_t* src = static_cast<const uint8_t*>(a.k) + (kbase + J * a.span) * KB;
        // four 16-byte loads per thread in flight before their stores
        const int32_t nb = n_back * KB;
        for (int32_t o0 = 0; o0 < nb; o0 += 4 * kThreads * 16) {
            u32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int32_t o = o0 + (u * kThreads + (int)threadIdx.x) * 16;
                if (o < nb) v[u] = *reinterpret_cast<const u32x4*>(src + o);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int32_t o = o0 + (u * kThreads + (int)threadIdx.x) * 16;
                if (o < nb) *reinterpret_cast<u32x4*>(s_k + o) = v[u];
            }
        }
        if (FP8)
            for (int i = threadIdx.x; i < n_back; i += kThreads) s_s[i] = a.k_scale[kbase + J * a.span + i];
        __syncthreads();
        // one thread per dimension sums the earlier keys in key order (the
        // same operations, in the same order, as the owner threads' sums)
        if (threadIdx.x < D) {
            const int d = threadIdx.x;
            double acc = 0.0;
            constexpr int U = 8;
            for (int32_t i0 = 0; i0 < n_back; i0 += U) {
                float x[U];
                float sc[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int32_t i = min(i0 + u, n_back - 1);
                    if constexpr (FP8) {
                        x[u] = __builtin_amdgcn_cvt_f32_fp8((int)s_k[i * KB + d], 0);
                        sc[u] = s_s[i];
                    } else {
                        x[u] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(s_k)[i * D + d] << 16);
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (i0 + u < n_back) {
                        if constexpr (FP8)
                            acc = fma((double)sc[u], (double)x[u], acc);
                        else
                            acc += (double)x[u];
                    }
                }
            }
            s_sum[d] = acc;
        }
        __syncthreads();
        if (piece >= TPG) return;
#pragma unroll
        for (int e = 0; e < 8; ++e) pacc[e] = s_sum[8 * piece + e];
    } else if (STAGE && piece >= TPG) {
        return;
    } else if (pool) {
        for (int32_t g = J * a.span; g < gs; g += kAhead) {
            if constexpr (FP8) {
                u32x2 c[kAhead];
                float s[kAhead];
#pragma unroll
                for (int u = 0; u < kAhead; ++u) {
                    const int32_t gg = min(g + u, gs - 1);
                    c[u] = *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(a.k) +
                                                           (kbase + gg) * D + 8 * piece);
                    s[u] = a.k_scale[kbase + gg];
                }
#pragma unroll
                for (int u = 0; u < kAhead; ++u)
                    if (g + u < gs) add_fp8x8(pacc, c[u][0], c[u][1], s[u]);
            } else {
                u32x4 v[kAhead];
#pragma unroll
                for (int u = 0; u < kAhead; ++u) {
                    const int32_t gg = min(g + u, gs - 1);
                    v[u] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.k) +
                                                           (kbase + gg) * D + 8 * piece);
                }
#pragma unroll
                for (int u = 0; u < kAhead; ++u)
                    if (g + u < gs) add_bf16x8(pacc, v[u]);
            }
        }
    }

    // raw row at position p: staged (p < raw_len, only in group g0, whose
    // slot is p mod m = p - m * g0) or new
    const int64_t tail0 = (int64_t)m * a.g0;
    auto raw_row = [&](int64_t p) -> const u32x4* {
        const uint16_t* src = p < raw_len ? a.tail + ((int64_t)b * m + (p - tail0)) * D
                                          : a.raw + ((int64_t)b * a.n_new + (p - raw_len)) * D;
        return reinterpret_cast<const u32x4*>(src + 8 * piece);
    };

    double gsum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) gsum[e] = 0.0;
    // the mean divides by m: for a power of two, multiplying by the exact
    // reciprocal is the same operation (no fp64 underflow at bf16 magnitudes)
    const bool m_pow2 = (m & (m - 1)) == 0;
    const double inv_m = 1.0 / (double)m;
    const int64_t p_end = (int64_t)m * ge;
    int32_t r = 0;       // position within the current group
    int32_t g = gs;      // current group
    // one raw row of the job, in position order
    auto consume = [&](const u32x4& row_in) {
        // kw: the compressed key's 8 bf16 values, packed in pairs
        u32x4 kw;
        if constexpr (M1) {
            // the mean of one bf16 key is that key, except that a sum
            // starting from +0 turns -0 into +0
            kw = row_in;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t z = kw[w];
                if ((z & 0x7FFFu) == 0) z &= ~0x8000u;
                if ((z & 0x7FFF0000u) == 0) z &= ~0x80000000u;
                kw[w] = z;
            }
        } else {
            add_bf16x8(gsum, row_in);
            if (++r < m) return;
            // group g complete: round the mean once to bf16
            uint32_t kc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kc[e] = f64_to_bf16(m_pow2 ? gsum[e] * inv_m : gsum[e] / (double)m);
                gsum[e] = 0.0;
            }
            kw = u32x4{kc[0] | (kc[1] << 16), kc[2] | (kc[3] << 16), kc[4] | (kc[5] << 16),
                       kc[6] | (kc[7] << 16)};
            r = 0;
        }
        const int64_t row = kbase + g;
        if constexpr (FP8) {
            float x[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                x[2 * w] = __uint_as_float(kw[w] << 16);
                x[2 * w + 1] = __uint_as_float(kw[w] & 0xFFFF0000u);
            }
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
            for (int o = 1; o < TPG; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, TPG));
            const float scale = amax / 448.0f;
            const float div = scale > 0.0f ? scale : 1.0f;
            if (div >= 0x1p-60f) {
                // x / div correctly rounded from the correctly rounded
                // reciprocal y: two fma residual corrections bring the
                // quotient within one ulp, and Markstein's theorem
                // (y = RN(1/div), residual exact) makes the last one
                // round correctly.  div >= 2^-60 keeps every residual
                // that can change a code in the normal range; the sign
                // is restored for -0.
                const float y = 1.0f / div;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float q0 = x[e] * y;
                    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, div, x[e]), y, q0);
                    const float q2 = __builtin_fmaf(__builtin_fmaf(-q1, div, x[e]), y, q1);
                    x[e] = __builtin_copysignf(q2, x[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = x[e] / div;
            }
            const uint32_t c0 = e4m3fn_x4(x), c1 = e4m3fn_x4(x + 4);
            *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(a.k) + row * D + 8 * piece) = u32x2{c0, c1};
            if (piece == 0) a.k_scale[row] = scale;
            if (pool) add_fp8x8(pacc, c0, c1, scale);
        } else {
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.k) + row * D + 8 * piece) = kw;
            if (pool) add_bf16x8(pacc, kw);
        }
        ++g;
    };
    // two batches of kAhead raw rows: one is consumed while the next loads
    const int64_t p0 = (int64_t)m * gs;
    u32x4 va[kAhead], vb[kAhead];
    auto load = [&](u32x4* v, int64_t p) {
#pragma unroll
        for (int u = 0; u < kAhead; ++u) v[u] = __builtin_nontemporal_load(raw_row(min(p + u, p_end - 1)));
    };
    auto take = [&](const u32x4* v, int64_t p) {
#pragma unroll
        for (int u = 0; u < kAhead; ++u)
            if (p + u < p_end) consume(v[u]);
    };
    if (p0 < p_end) load(va, p0);
    for (int64_t p = p0; p < p_end; p += 2 * kAhead) {
        if (p + kAhead < p_end) load(vb, p + kAhead);
        take(va, p);
        if (p + 2 * kAhead < p_end) load(va, p + 2 * kAhead);
        if (p + kAhead < p_end) take(vb, p + kAhead);
    }

    if (pool) {
        const double inv_span = 1.0 / (double)a.span;  // exact: the block size is a power of two
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = f64_to_bf16(pacc[2 * e] * inv_span) | (f64_to_bf16(pacc[2 * e + 1] * inv_span) << 16);
        const int64_t nb = a.n_k / a.span;
        *reinterpret_cast<u32x4*>(a.pooled + ((int64_t)b * nb + J) * D + 8 * piece) =
            u32x4{o[0], o[1], o[2], o[3]};
    }

    // stage the raw keys of the group left open (first job of the sequence,
    // after its own reads of the staged keys above)
    if (m > 1 && J == a.J0) {
        // the open group is g1: raw position p sits in slot p - m * g1
        const int64_t end = raw_len + a.n_new;
        const int64_t open0 = (int64_t)m * a.g1;
        for (int64_t p = max(raw_len, open0); p < end; ++p) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(
                a.raw + ((int64_t)b * a.n_new + (p - raw_len)) * D + 8 * piece);
            *reinterpret_cast<u32x4*>(a.tail + ((int64_t)b * m + (p - open0)) * D + 8 * piece) = v;
        }
    }
}

template <bool FP8, int D>
void launch_d(const AppendArgs& a, hipStream_t stream) {
    constexpr int TPG = D / 8;
    if (a.n_jobs == 1 && a.pooled != nullptr && a.span <= kStageMax + 1) {
        // one block per sequence (decode): a workgroup per sequence
        const dim3 grid((unsigned)a.batch);
        if (a.m == 1)
            hipLaunchKernelGGL((append_kernel<FP8, D, true, true>), grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((append_kernel<FP8, D, false, true>), grid, dim3(kThreads), 0, stream, a);
        return;
    }
    const int64_t threads = (int64_t)a.batch * a.n_jobs * TPG;
    const unsigned grid = (unsigned)((threads + kThreads - 1) / kThreads);
    if (a.m == 1)
        hipLaunchKernelGGL((append_kernel<FP8, D, true, false>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((append_kernel<FP8, D, false, false>), dim3(grid), dim3(kThreads), 0, stream, a);
}

template <bool FP8>
void launch_fp(const AppendArgs& a, int dim, hipStream_t stream) {
    if (dim == 32)
        launch_d<FP8, 32>(a, stream);
    else if (dim == 64)
        launch_d<FP8, 64>(a, stream);
    else
        launch_d<FP8, 128>(a, stream);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int dim, bool fp8, hipStream_t stream) {
    if ((int64_t)a.batch * a.n_jobs <= 0) return hipSuccess;
    if (fp8)
        launch_fp<true>(a, dim, stream);
    else
        launch_fp<false>(a, dim, stream);
    return hipGetLastError();
}

}  // namespace tks

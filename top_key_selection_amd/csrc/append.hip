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
#include "tks_launch.hpp"

namespace tks {

namespace {

constexpr int kThreads = 256;
constexpr int kAhead = 4;  // raw (or cached) key rows in flight per thread

// fp64 -> bf16, nearest-even: round-to-odd to fp32 (24 bits >= 8 + 2), then
// nearest-even to bf16, which keeps the rounding single.
__device__ inline uint32_t f64_to_bf16(double x) {
    float f = __double2float_rz(x);
    if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// OCP e4m3fn code of x: nearest magnitude, ties to the even code, saturated
// at 448, sign bit kept.  Below 2^-6 the grid is the subnormal step 2^-9;
// above, the 3-bit significand is rounded to nearest-even, and a carry out of
// it moves to the next binade's first code by plain addition.
__device__ inline uint32_t e4m3fn_code(float x) {
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fminf(fabsf(x), 448.0f);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        const uint32_t u = __float_as_uint(a);
        const uint32_t mant = u & 0x7FFFFFu;
        code = (((u >> 23) - 120u) << 3) + ((mant + 0x7FFFFu + ((mant >> 20) & 1u)) >> 20);
    }
    return sign | code;
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

template <bool FP8, int D>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
    constexpr int TPG = D / 8;  // threads per key (8 dims each)
    const int64_t gt = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t job = gt / TPG;
    const int piece = (int)(gt % TPG);
    if (job >= (int64_t)a.batch * a.n_jobs) return;
    const int32_t b = (int32_t)(job / a.n_jobs);
    const int32_t J = a.J0 + (int32_t)(job % a.n_jobs);
    const int32_t m = a.m;
    const int32_t gs = max(a.g0, J * a.span);          // groups completed here
    const int32_t ge = min(a.g1, (J + 1) * a.span);
    const bool pool = a.pooled != nullptr && (J + 1) * a.span <= a.g1;
    const int64_t kbase = (int64_t)b * a.n_k;
    const int64_t raw_len = a.raw_len;

    double pacc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pacc[e] = 0.0;

    // compressed keys of block J that earlier calls wrote, in key order
    if (pool) {
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

    // raw row at position p: staged (p < raw_len) or new
    auto raw_row = [&](int64_t p) -> const u32x4* {
        const uint16_t* src = p < raw_len ? a.tail + ((int64_t)b * m + p % m) * D
                                          : a.raw + ((int64_t)b * a.n_new + (p - raw_len)) * D;
        return reinterpret_cast<const u32x4*>(src + 8 * piece);
    };

    double gsum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) gsum[e] = 0.0;
    const int64_t p_end = (int64_t)m * ge;
    int32_t r = 0;       // position within the current group
    int32_t g = gs;      // current group
    for (int64_t p = (int64_t)m * gs; p < p_end; p += kAhead) {
        u32x4 v[kAhead];
#pragma unroll
        for (int u = 0; u < kAhead; ++u) v[u] = __builtin_nontemporal_load(raw_row(min(p + u, p_end - 1)));
#pragma unroll
        for (int u = 0; u < kAhead; ++u) {
            if (p + u >= p_end) break;
            add_bf16x8(gsum, v[u]);
            if (++r < m) continue;
            // group g complete: round the mean once to bf16
            uint32_t kc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kc[e] = f64_to_bf16(gsum[e] / (double)m);
                gsum[e] = 0.0;
            }
            const int64_t row = kbase + g;
            if constexpr (FP8) {
                float amax = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(__uint_as_float(kc[e] << 16)));
#pragma unroll
                for (int o = 1; o < TPG; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, TPG));
                const float scale = amax / 448.0f;
                const float div = scale > 0.0f ? scale : 1.0f;
                uint32_t c0 = 0, c1 = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    c0 |= e4m3fn_code(__uint_as_float(kc[e] << 16) / div) << (8 * e);
                    c1 |= e4m3fn_code(__uint_as_float(kc[4 + e] << 16) / div) << (8 * e);
                }
                *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(a.k) + row * D + 8 * piece) = u32x2{c0, c1};
                if (piece == 0) a.k_scale[row] = scale;
                if (pool) add_fp8x8(pacc, c0, c1, scale);
            } else {
                const u32x4 o = u32x4{kc[0] | (kc[1] << 16), kc[2] | (kc[3] << 16),
                                      kc[4] | (kc[5] << 16), kc[6] | (kc[7] << 16)};
                *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.k) + row * D + 8 * piece) = o;
                if (pool) add_bf16x8(pacc, o);
            }
            r = 0;
            ++g;
        }
    }

    if (pool) {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = f64_to_bf16(pacc[2 * e] / (double)a.span) |
                   (f64_to_bf16(pacc[2 * e + 1] / (double)a.span) << 16);
        const int64_t nb = a.n_k / a.span;
        *reinterpret_cast<u32x4*>(a.pooled + ((int64_t)b * nb + J) * D + 8 * piece) =
            u32x4{o[0], o[1], o[2], o[3]};
    }

    // stage the raw keys of the group left open (first job of the sequence,
    // after its own reads of the staged keys above)
    if (m > 1 && J == a.J0) {
        const int64_t end = raw_len + a.n_new;
        for (int64_t p = max(raw_len, (int64_t)m * a.g1); p < end; ++p) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(
                a.raw + ((int64_t)b * a.n_new + (p - raw_len)) * D + 8 * piece);
            *reinterpret_cast<u32x4*>(a.tail + ((int64_t)b * m + p % m) * D + 8 * piece) = v;
        }
    }
}

template <bool FP8, int D>
void launch_d(const AppendArgs& a, hipStream_t stream) {
    constexpr int TPG = D / 8;
    const int64_t threads = (int64_t)a.batch * a.n_jobs * TPG;
    const unsigned grid = (unsigned)((threads + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((append_kernel<FP8, D>), dim3(grid), dim3(kThreads), 0, stream, a);
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

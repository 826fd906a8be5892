// tks_device.hpp -- device-side building blocks shared by the gfx950 kernels
// of the indexer top-k library (visibility rule, score ordering keys,
// parameter blocks).  Host glue and kernels include it; nothing outside the
// library does.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tks {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Visibility (HISA abstract: the indexer scans the whole causal prefix):
// query t at position q_pos0 + t sees keys s <= floor((q_pos0 + t) / ratio),
// s < n_k.  With blk > 0 the rule counts the complete blocks strictly
// before the query's local block (the ones HISA block selection scores).
struct VisRule {
    int32_t q_pos0;
    int32_t ratio;
    int32_t n_k;
    int32_t blk;  // 0: tokens; else block size

    __host__ __device__ inline int32_t tokens(int32_t t) const {
        int64_t p = (int64_t)q_pos0 + t;
        // floor division (skipped for the common ratio 1)
        int64_t v = ratio == 1 ? p : p >= 0 ? p / ratio : -((-p + ratio - 1) / ratio);
        if (v < 0) return 0;
        return v + 1 < n_k ? (int32_t)(v + 1) : n_k;
    }
    // Number of visible candidates: tokens, or complete blocks before the
    // local block.
    __host__ __device__ inline int32_t count(int32_t t) const {
        int32_t n = tokens(t);
        if (blk == 0) return n;
        return n > 0 ? (n - 1) / blk : 0;
    }
};

// Orderable 32-bit key of a score: a larger float gives a larger key, -0
// maps to the key of +0.  NaN payload 0xFFFFFFFF maps to 0 (never a real
// score's key; used as "no candidate").
__device__ inline uint32_t score_key(float x) {
    uint32_t u = __float_as_uint(x + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float key_score(uint32_t key) {
    uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return __uint_as_float(u);
}

// Row addressing of the score kernels and the selection kernel: a launch
// covers output rows y = 0..n_rows-1 of a chunk that starts at global row
// y0; global row g maps to sequence b = g / rows_per_seq and query
// t = t_begin + g % rows_per_seq.
struct RowMap {
    int64_t y0;
    int32_t rows_per_seq;
    int32_t t_begin;
    int32_t n_q;  // queries per sequence in q / w
    __host__ __device__ inline int32_t seq(int64_t y) const {
        return (int32_t)((y0 + y) / rows_per_seq);
    }
    __host__ __device__ inline int32_t query(int64_t y) const {
        return t_begin + (int32_t)((y0 + y) % rows_per_seq);
    }
    // flat row of q / w
    __host__ __device__ inline int64_t qrow(int64_t y) const {
        return (int64_t)seq(y) * n_q + query(y);
    }
};

}  // namespace tks

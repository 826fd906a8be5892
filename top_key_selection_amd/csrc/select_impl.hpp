// select_impl.hpp -- device side of the exact per-query top-k (internal to
// the library): candidate visitors, histograms, the threshold prefilter,
// the counting top-k, the radix fallbacks and the row writer.  The
// selection kernels (select.hip) and the fused score-filter finish
// (fused.hip) both build on it.
//
// select.hip -- exact per-query top-k on gfx950.
//
// The per-query top-k of the HISA abstract (a per-query set of k token
// indices) and the partition-merge of the StreamIndex abstract (a partial
// top-k per key tile merged into a running list) both reduce to one
// operation: from a row's candidates -- the running list of earlier tiles
// plus this tile's scores -- keep the k best in the total order (score
// descending, key index ascending).
//
// Every candidate becomes the 64-bit composite (orderable score key << 32 |
// ~index); the k largest composites are exactly the answer, whatever order
// the candidates arrive in.  A row takes one of three routes:
//
//   * at most 2048 candidates: all of them are gathered into LDS and sorted;
//   * at least 4096 candidates (16384 for kept-block rows): a threshold
//     from a small sample of the row
//     (the Indexer-TopK abstract on the StreamIndex page: estimate the score
//     range from a sample, keep only candidates above a tight threshold,
//     stay exact) fills an LDS pool in one pass;
//   * otherwise a 4096-bin histogram of the top 12 bits of the score key
//     (LDS, wave-aggregated atomics) locates the bin b* that holds the k-th
//     score, and a second pass puts everything from b* up into the pool.
//
// The best k of a pool are placed in order by counting on the score (4096
// equal score bins, a scan of the bin counts, and each entry's rank inside
// its bin), so selection and the final sort are one pass.  Pools that do
// not fit, heavy exact ties and clustered scores keep the exact fallbacks:
// LDS radix selection over 12- and 8-bit digits, an 8-bit radix select with
// an ordered tie scan over the whole row (no buffer at all), and a bitonic /
// merge sort.  Row passes keep four 16-byte loads per thread in flight;
// when the rows are few (decode) a row gets a 1024-thread workgroup, and
// few long rows are spread over every CU by a three-kernel form.
//
// Block-select output mode writes the kept blocks in ascending block order
// with the forced first / local blocks added (score +inf).
#pragma once

#include <algorithm>

#include "tks_launch.hpp"

namespace tks {

namespace {


constexpr int kMaxThreads = 1024;
constexpr int kMaxWaves = kMaxThreads / kWave;
constexpr int kMaxK = 2048;
constexpr int kCap = 4096;          // LDS candidate list (entries of the threshold bin)
constexpr int kBins = 4096;         // 12-bit first digit
constexpr int kBinShift = 20;
constexpr int kSamples = 2048;      // candidates sampled for the prefilter threshold
constexpr int kSampleRun = 16;      // ... in evenly spaced runs of consecutive candidates
static_assert(kSamples % 256 == 0 && kSamples % 1024 == 0, "whole samples per thread");
constexpr int kPrefilterMin = 16384; // rows at least this long take the prefilter
constexpr int kPrefilterMinTok = 4096; // ... token rows (not block lists) from this long
constexpr int kMaxBlkEntries = 512;
constexpr int kBitmapWords = 4096;  // block-select bitmap (ids below 131072)

// LDS of the selection kernels: selected list [0, kMaxK), candidate list
// [kMaxK, kMaxK + kCap).  The histogram of pass 1 aliases the candidate
// list; the radix fallback uses the selected list and 4 KiB after it.
struct SelectLds {
    uint64_t u[kMaxK + kCap];
    uint32_t hist8[256];  // digit histogram of the candidate resolution
    int32_t blk[kMaxBlkEntries];
    int32_t wsum[kMaxWaves];
    int32_t pick[8];
    int32_t cnt[2];
};

__device__ __forceinline__ uint32_t* lds_hist(SelectLds& L) { return reinterpret_cast<uint32_t*>(&L.u[kMaxK]); }

struct RowCtx {
    int64_t y;
    int32_t t;
    int32_t lo, hi;          // valid score columns [lo, hi)
    int32_t n_tok;
    bool prior;
    const float* srow;
    const int32_t* blk_row;  // block mode: LDS copy of the row's block list
};

__device__ __forceinline__ uint64_t composite(uint32_t key, int32_t idx) {
    return ((uint64_t)key << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// Key index of score column j, or -1 when the slot holds no candidate.
__device__ __forceinline__ int32_t column_index(const SelectArgs& a, const RowCtx& r, int32_t j) {
    if (!a.blocks_mode) return a.col_key0 + j;
    const int32_t b = r.blk_row[j >> a.block_shift];
    if (b < 0 || r.n_tok <= 0 || b > ((r.n_tok - 1) >> a.block_shift)) return -1;
    const int32_t idx = (b << a.block_shift) + (j & ((1 << a.block_shift) - 1));
    return idx < r.n_tok ? idx : -1;
}

// Visit the candidates of columns [c_begin, c_end) of the row (subset of
// [lo, hi)), thread-strided in groups of 4 consecutive columns, with U
// groups loaded before any is processed.  Every thread calls f the same
// number of times (valid = false past the end), so f may use wave-wide
// ballots.
template <bool VEC, int NT, class F>
__device__ __forceinline__ void visit_columns(const SelectArgs& a, const RowCtx& r, int32_t c_begin,
                                     int32_t c_end, F&& f) {
    constexpr int U = VEC ? 4 : 2;  // (scalar loads need more registers)
    constexpr int32_t kStep = 4 * NT * U;
    const int tid = threadIdx.x;
    if (c_begin >= c_end) return;
    const int32_t base0 = c_begin & ~3;
    // aligned groups past the end re-read the last group (inside the row's
    // storage, whose stride is a multiple of 4): the vector loads need no
    // branch, so all U of them stay in flight together, and the next group
    // of U is loaded before the current one is processed
    const int32_t last = (c_end - 1) & ~3;
    auto load = [&](float (*v)[4], int32_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t j0 = base + 4 * (u * NT + tid);
            if (VEC) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(r.srow + min(j0, last));
                v[u][0] = x[0]; v[u][1] = x[1]; v[u][2] = x[2]; v[u][3] = x[3];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int32_t j = j0 + i;
                    v[u][i] = (j >= c_begin && j < c_end) ? r.srow[j] : 0.0f;
                }
            }
        }
    };
    auto visit = [&](float (*v)[4], int32_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t j = base + 4 * (u * NT + tid) + i;
                int32_t idx = -1;
                if (j >= c_begin && j < c_end) idx = column_index(a, r, j);
                f(idx >= 0, score_key(v[u][i]), idx);
            }
        }
    };
    float va[U][4], vb[U][4];
    load(va, base0);
    for (int32_t base = base0; base < c_end; base += 2 * kStep) {
        load(vb, base + kStep);
        visit(va, base);
        if (base + kStep >= c_end) break;
        load(va, base + 2 * kStep);
        visit(vb, base + kStep);
    }
}

// Append every candidate of columns [c_begin, c_end) whose key is at least
// tau to dst (slots past cap are counted but not written).  The same
// double-buffered loads as visit_columns; the appends are batched per
// thread group of U * 4 columns: each lane counts its hits, a bitwise
// ballot prefix gives every lane its offset, and one atomic per wave and
// group reserves the run.
template <bool VEC, int NT>
__device__ __forceinline__ void collect_ge(const SelectArgs& a, const RowCtx& r, int32_t c_begin,
                                           int32_t c_end, uint32_t tau, int32_t* counter,
                                           uint64_t* dst, int32_t cap) {
    constexpr int U = VEC ? 4 : 2;
    constexpr int E = U * 4;
    constexpr int32_t kStep = 4 * NT * U;
    const int tid = threadIdx.x, lane = tid & 63;
    if (c_begin >= c_end) return;
    const int32_t base0 = c_begin & ~3;
    const int32_t last = (c_end - 1) & ~3;
    auto load = [&](float (*v)[4], int32_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t j0 = base + 4 * (u * NT + tid);
            if (VEC) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(r.srow + min(j0, last));
                v[u][0] = x[0]; v[u][1] = x[1]; v[u][2] = x[2]; v[u][3] = x[3];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int32_t j = j0 + i;
                    v[u][i] = (j >= c_begin && j < c_end) ? r.srow[j] : 0.0f;
                }
            }
        }
    };
    const uint64_t lt = (1ull << lane) - 1ull;
    auto group = [&](float (*v)[4], int32_t base) {
        uint32_t key[E];
        int32_t idx[E];
        int32_t cnt = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t j = base + 4 * (u * NT + tid) + i;
                const int32_t id = (j >= c_begin && j < c_end) ? column_index(a, r, j) : -1;
                const uint32_t k = score_key(v[u][i]);
                const bool p = id >= 0 && k >= tau;
                key[u * 4 + i] = k;
                idx[u * 4 + i] = p ? id : -1;
                cnt += p ? 1 : 0;
            }
        }
        int32_t pre = 0, tot = 0;
#pragma unroll
        for (int b = 0; b < 5; ++b) {  // cnt <= 16
            const uint64_t bb = __ballot((cnt >> b) & 1);
            pre += __popcll(bb & lt) << b;
            tot += __popcll(bb) << b;
        }
        if (tot == 0) return;
        int32_t at = 0;
        if (lane == 0) at = atomicAdd(counter, tot);
        int32_t pos = __builtin_amdgcn_readlane(at, 0) + pre;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (idx[e] >= 0) {
                if (pos < cap) dst[pos] = composite(key[e], idx[e]);
                ++pos;
            }
        }
    };
    float va[U][4], vb[U][4];
    load(va, base0);
    for (int32_t base = base0; base < c_end; base += 2 * kStep) {
        load(vb, base + kStep);
        group(va, base);
        if (base + kStep >= c_end) break;
        load(va, base + 2 * kStep);
        group(vb, base + kStep);
    }
}

// Visit the prior list (running top-k of earlier key tiles).
__device__ __forceinline__ int32_t prior_len(const SelectArgs& a) { return a.topk; }

template <int NT, class F>
__device__ __forceinline__ void visit_prior(const SelectArgs& a, const RowCtx& r, F&& f) {
    const int tid = threadIdx.x;
    if (!r.prior) return;
    const int32_t n = prior_len(a);
    for (int32_t base = 0; base < n; base += NT) {
        const int32_t p = base + tid;
        int32_t idx = -1;
        float v = 0.0f;
        if (p < n) {
            idx = a.prior_idx[r.y * n + p];
            v = a.prior_val[r.y * n + p];
        }
        f(idx >= 0, score_key(v), idx);
    }
}

// Wave-aggregated LDS histogram increment.
__device__ __forceinline__ void hist_add(uint32_t* h, bool valid, uint32_t bin) {
    const uint64_t act = __ballot(valid);
    if (act == 0) return;
    const int leader = __builtin_ctzll(act);
    const uint32_t first = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const uint64_t same = __ballot(valid && bin == first);
    if (same == act) {
        if ((int)(threadIdx.x & 63) == leader) atomicAdd(&h[bin], (uint32_t)__popcll(act));
    } else if (valid) {
        atomicAdd(&h[bin], 1u);
    }
}

// Wave-aggregated append: returns this lane's slot (or -1 if !pred).
__device__ __forceinline__ int32_t wave_append(int32_t* counter, bool pred) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return -1;
    const int lane = threadIdx.x & 63;
    const int leader = __builtin_ctzll(m);
    int32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (int32_t)__popcll(m));
    base = __builtin_amdgcn_readlane(base, leader);
    return pred ? base + (int32_t)__popcll(m & ((1ull << lane) - 1ull)) : -1;
}

// Threshold of the k best from a histogram (bins in LDS or global memory,
// read through `get`): pick = {b*, count above b*, count in b*, total}.
template <int NT, int NB, class G>
__device__ __forceinline__ void find_threshold_n(G&& get, int32_t K, int32_t* pick, int32_t* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kWaves = NT / kWave;
    constexpr int per = NB >= NT ? NB / NT : 1;  // bins per thread, descending order
    const bool has = NB >= NT || tid < NB;
    int32_t c[per];
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        c[i] = has ? (int32_t)get(NB - 1 - (per * tid + i)) : 0;
        s += c[i];
    }
    int32_t inc = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int32_t off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        off += (w < wave) ? wsum[w] : 0;
        total += wsum[w];
    }
    inc += off;
    const int32_t excl = inc - s;
    if (tid == 0) {
        pick[3] = total;
        pick[0] = -1;
    }
    __syncthreads();
    if (total > K && excl < K && K <= inc) {
        int32_t cum = excl;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            if (cum < K && K <= cum + c[i]) {
                pick[0] = NB - 1 - (per * tid + i);
                pick[1] = cum;
                pick[2] = c[i];
            }
            cum += c[i];
        }
    }
    __syncthreads();
}

template <int NT, class G>
__device__ __forceinline__ void find_threshold(G&& get, int32_t K, int32_t* pick, int32_t* wsum) {
    find_threshold_n<NT, kBins>(static_cast<G&&>(get), K, pick, wsum);
}

// Value of lane ^ S, exchanged by the vector ALU (DPP quad permutes and row
// shifts, v_permlane16/32_swap) rather than through the LDS crossbar.
template <int S>
__device__ __forceinline__ uint32_t xchg32(uint32_t v) {
    const int lane = threadIdx.x & 63;
    if constexpr (S == 1) {
        return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (S == 2) {
        return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (S == 4 || S == 8) {
        // row_shl:S reads lane + S, row_shr:S reads lane - S
        const uint32_t up = __builtin_amdgcn_update_dpp(0u, v, 0x100 + S, 0xF, 0xF, false);
        const uint32_t dn = __builtin_amdgcn_update_dpp(0u, v, 0x110 + S, 0xF, 0xF, false);
        return (lane & S) ? dn : up;
    } else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        static_assert(S == 32, "exchange stride");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}

template <int S>
__device__ __forceinline__ uint64_t xchg64(uint64_t v) {
#if defined(__HIP_DEVICE_COMPILE__)
    return ((uint64_t)xchg32<S>((uint32_t)(v >> 32)) << 32) | xchg32<S>((uint32_t)v);
#else
    return v;  // the permlane builtins exist for the device pass only
#endif
}

// One compare-exchange stage at lane stride S (< 64) of a bitonic network
// over 128 entries (entry `lane` in a[c], `lane + 64` in b[c]).
template <int S, int N>
__device__ __forceinline__ void cx_lanes(uint64_t* a, uint64_t* b, int size) {
    const int lane = threadIdx.x & 63;
    const bool lower = (lane & S) == 0;  // same for lane + 64
    const bool keep_a = ((lane & size) == 0) == lower;
    const bool keep_b = (((lane + 64) & size) == 0) == lower;
    uint64_t pa[N], pb[N];
#pragma unroll
    for (int c = 0; c < N; ++c) {
        pa[c] = xchg64<S>(a[c]);
        pb[c] = xchg64<S>(b[c]);
    }
    // entries are distinct: take the partner's value when it is the larger
    // one and this position keeps the larger, or the smaller and keeps the
    // smaller
#pragma unroll
    for (int c = 0; c < N; ++c) {
        a[c] = ((pa[c] > a[c]) == keep_a) ? pa[c] : a[c];
        b[c] = ((pb[c] > b[c]) == keep_b) ? pb[c] : b[c];
    }
}

// Bitonic sort of N independent 128-entry chunks held by one wave, each
// descending; the chunks go through the network together.
template <int N>
__device__ __forceinline__ void wave_sort128(uint64_t* a, uint64_t* b) {
#pragma unroll
    for (int size = 2; size <= 128; size <<= 1) {
        if (size == 128) {
            // one descending block: a holds the lower index of each pair
#pragma unroll
            for (int c = 0; c < N; ++c) {
                const uint64_t hi = a[c] > b[c] ? a[c] : b[c];
                const uint64_t lo = a[c] > b[c] ? b[c] : a[c];
                a[c] = hi;
                b[c] = lo;
            }
        }
        if (size >= 64) cx_lanes<32, N>(a, b, size);
        if (size >= 32) cx_lanes<16, N>(a, b, size);
        if (size >= 16) cx_lanes<8, N>(a, b, size);
        if (size >= 8) cx_lanes<4, N>(a, b, size);
        if (size >= 4) cx_lanes<2, N>(a, b, size);
        cx_lanes<1, N>(a, b, size);
    }
}

// Sort u[0, n) descending, n <= kMaxK; the entries must be distinct (the
// composites are).  tmp has room for the padded size.  Waves sort 128-entry
// chunks in registers; the chunks are then merged pairwise, each entry
// finding its place in the partner run by binary search (its rank in the
// merged run is its own position plus the partner entries above it).  A
// thread's searches advance in lockstep so their LDS reads overlap.
template <int NT>
__device__ __forceinline__ void sort_desc(uint64_t* u, uint64_t* tmp, int32_t n) {
    constexpr int W = NT / kWave;
    constexpr int CPW = (kMaxK / 128 + W - 1) / W;  // chunks per wave
    constexpr int EPT = (kMaxK + NT - 1) / NT;      // merge entries per thread
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (n <= 1) return;
    int32_t P = 128;
    while (P < n) P <<= 1;
    // padding: distinct values below every real composite
    for (int i = n + tid; i < P; i += NT) u[i] = (uint64_t)(P - i);
    __syncthreads();
    {
        const int n_chunks = P / 128;
        uint64_t a[CPW], b[CPW];
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int ch = wave + c * W;
            a[c] = ch < n_chunks ? u[ch * 128 + lane] : 0;
            b[c] = ch < n_chunks ? u[ch * 128 + 64 + lane] : 0;
        }
        wave_sort128<CPW>(a, b);
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int ch = wave + c * W;
            if (ch < n_chunks) {
                u[ch * 128 + lane] = a[c];
                u[ch * 128 + 64 + lane] = b[c];
            }
        }
    }
    __syncthreads();
    uint64_t* src = u;
    uint64_t* dst = tmp;
    for (int32_t L = 128; L < P; L <<= 1) {
        uint64_t x[EPT];
        int32_t k[EPT], other[EPT], at[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int i = tid + e * NT;
            const int32_t run = i / L;
            const int32_t base = (run & ~1) * L;
            x[e] = i < P ? src[i] : 0;
            other[e] = base + ((run & 1) ? 0 : L);
            at[e] = base + (i & (L - 1));
            k[e] = 0;
        }
        for (int32_t step = L >> 1; step > 0; step >>= 1) {
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (tid + e * NT < P && src[other[e] + k[e] + step - 1] > x[e]) k[e] += step;
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            if (tid + e * NT < P) {
                if (src[other[e] + k[e]] > x[e]) ++k[e];
                dst[at[e] + k[e]] = x[e];
            }
        }
        __syncthreads();
        uint64_t* t = src;
        src = dst;
        dst = t;
    }
    if (src != u) {
        for (int i = tid; i < n; i += NT) u[i] = src[i];
        __syncthreads();
    }
}

// The best K of src[0, n) (distinct composites), sorted descending, into
// out[0, min(K, n)), by counting on the score: the score range [vmin, vmax]
// is cut into NB equal bins (fp32 (v - vmin) * scale, a non-decreasing map
// of the score; 4096 unless the list is short), each entry is scattered to its bin's run (bins in
// descending order, run starts from an exclusive scan of the bin counts),
// and inside a bin its place is the number of bin entries above it in the
// total order (independent LDS reads, no dependency chain); entries placed
// at K or beyond are dropped.  Scores spread the entries over many bins, a
// few per bin.  Every entry is first taken into registers, so tmp may alias
// src and bins may alias out.  Returns false with src untouched when
// counting does not apply: a non-finite score range, or a bin of more than
// kBinCap entries (heavy ties, clustered scores).
constexpr int kSortBins = 4096;
constexpr int kBinCap = 128;

template <int NT, int NMAX, int NB = kSortBins>
__device__ __forceinline__ bool counting_topk(SelectLds& L, const uint64_t* src, int32_t n, int32_t K,
                                              uint64_t* out, uint64_t* tmp, uint32_t* bins) {
    constexpr int W = NT / kWave;
    constexpr int EPT = (NMAX + NT - 1) / NT;
    constexpr int per = NB >= NT ? NB / NT : 1;  // bins per thread in the scan, descending
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool has = NB >= NT || tid < NB;
    uint64_t e[EPT];
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int j = tid + i * NT;
        e[i] = j < n ? src[j] : 0;
        if (j < n) {
            kmin = min(kmin, (uint32_t)(e[i] >> 32));
            kmax = max(kmax, (uint32_t)(e[i] >> 32));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    }
    if (lane == 0) {
        L.hist8[wave] = kmin;
        L.hist8[64 + wave] = kmax;
    }
    for (int i = tid; i < NB; i += NT) bins[i] = 0u;
    __syncthreads();
    kmin = L.hist8[0];
    kmax = L.hist8[64];
#pragma unroll
    for (int w = 1; w < W; ++w) {
        kmin = min(kmin, L.hist8[w]);
        kmax = max(kmax, L.hist8[64 + w]);
    }
    const float vmin = key_score(kmin), vspan = key_score(kmax) - vmin;
    if (!(vspan < __builtin_inff())) {  // a non-finite score or range
        __syncthreads();
        return false;
    }
    const float scale = vspan > 0.0f ? (float)(NB - 1) / vspan : 0.0f;
    uint32_t bin[EPT], rank[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const float v = key_score((uint32_t)(e[i] >> 32));
        bin[i] = min((uint32_t)((v - vmin) * scale), (uint32_t)(NB - 1));
        rank[i] = tid + i * NT < n ? atomicAdd(&bins[bin[i]], 1u) : 0u;
    }
    __syncthreads();
    // run starts: bins in descending order, exclusive scan of the counts
    uint32_t c[per];
    int32_t sum = 0;
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        c[i] = has ? bins[NB - 1 - (per * tid + i)] : 0u;
        sum += (int32_t)c[i];
        mx = max(mx, c[i]);
    }
    int32_t inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    if (lane == 63) L.wsum[wave] = inc;
    if (lane == 0) L.hist8[128 + wave] = mx;
    __syncthreads();
    int32_t run = inc - sum;
    uint32_t maxc = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        run += w < wave ? L.wsum[w] : 0;
        maxc = max(maxc, L.hist8[128 + w]);
    }
    if (maxc > (uint32_t)kBinCap) {
        __syncthreads();
        return false;
    }
#pragma unroll
    for (int i = 0; i < per; ++i) {
        if (has) bins[NB - 1 - (per * tid + i)] = (uint32_t)run;
        run += (int32_t)c[i];
    }
    __syncthreads();
    // scatter; bin[] now holds the run start, rank[] the run end
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        if (tid + i * NT >= n) continue;
        const uint32_t st = bins[bin[i]];
        const uint32_t en = bin[i] == 0 ? (uint32_t)n : bins[bin[i] - 1];
        tmp[st + rank[i]] = e[i];
        bin[i] = st;
        rank[i] = en;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        if (tid + i * NT >= n || bin[i] >= (uint32_t)K) continue;
        uint32_t r = 0;
        for (uint32_t t = bin[i]; t < rank[i]; ++t) r += tmp[t] > e[i] ? 1u : 0u;
        if (bin[i] + r < (uint32_t)K) out[bin[i] + r] = e[i];
    }
    __syncthreads();
    return true;
}

// Sort the selected list L.u[0, n) descending, n <= kMaxK: counting (the
// scattered copy and the 4096 counters use the candidate area after the
// list), else the bitonic / merge sort.
static_assert(kMaxK * 8 + kSortBins * 4 <= kCap * 8, "counting scratch fits the candidate area");

template <int NT>
__device__ __forceinline__ void sort_final(SelectLds& L, int32_t n) {
    if (n <= 1) return;
    uint32_t* bins = reinterpret_cast<uint32_t*>(&L.u[kMaxK + kMaxK]);
    // about two bins per entry: short lists (block selection) zero and
    // scan far fewer counters
    const bool ok = n <= 256    ? counting_topk<NT, kMaxK, 512>(L, L.u, n, n, L.u, &L.u[kMaxK], bins)
                    : n <= 1024 ? counting_topk<NT, kMaxK, 2048>(L, L.u, n, n, L.u, &L.u[kMaxK], bins)
                                : counting_topk<NT, kMaxK>(L, L.u, n, n, L.u, &L.u[kMaxK], bins);
    if (!ok) sort_desc<NT>(L.u, &L.u[kMaxK], n);
}

// Write a finished row: sel[0, n_sel) sorted descending on the composite.
template <int NT>
__device__ __forceinline__ void write_row(const SelectArgs& a, const RowCtx& r, SelectLds& L, int32_t n_sel,
                                 bool final_out) {
    const int tid = threadIdx.x;
    uint64_t* sel = L.u;
    if (a.blockselect) {
        // ascending block index.  The selected block ids are distinct and
        // small: mark them in an LDS bitmap, and each one's output slot is
        // the number of marked ids below it (word prefix sums + popcount),
        // so no sort is needed.  Very long block lists use a sort instead.
        const int32_t Lb = r.n_tok > 0 ? (r.n_tok - 1) / a.sel_block : -1;
        const bool f_first = (a.force_flags & 1u) && Lb > 0;
        const bool f_local = (a.force_flags & 2u) && Lb >= 0;
        const int64_t g = a.rows.y0 + r.y;
        int32_t* oi = a.out_idx + g * a.out_width;
        float* ov = a.out_val ? a.out_val + g * a.out_width : nullptr;
        const int32_t off = f_first ? 1 : 0;
        const int32_t n_words = (a.col_key0 + a.n_cols + 31) / 32;
        auto id_of = [](uint64_t c) { return (int32_t)(0xFFFFFFFFu - (uint32_t)c); };
        if (n_words <= kBitmapWords) {
            uint32_t* bits = reinterpret_cast<uint32_t*>(&L.u[kMaxK]);
            uint32_t* pre = bits + kBitmapWords;
            for (int i = tid; i < n_words; i += NT) bits[i] = 0u;
            __syncthreads();
            for (int i = tid; i < n_sel; i += NT) {
                const int32_t id = id_of(sel[i]);
                atomicOr(&bits[id >> 5], 1u << (id & 31));
            }
            __syncthreads();
            // exclusive prefix of the word popcounts, per thread a run of words
            const int per = (n_words + NT - 1) / NT;
            const int w0 = tid * per;
            int32_t local = 0;
            for (int i = 0; i < per; ++i)
                if (w0 + i < n_words) local += __popc(bits[w0 + i]);
            const int lane = tid & 63, wave = tid >> 6;
            int32_t inc = local;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int32_t v = __shfl_up(inc, o);
                if (lane >= o) inc += v;
            }
            if (lane == 63) L.wsum[wave] = inc;
            __syncthreads();
            int32_t run = inc - local;
            for (int w = 0; w < wave; ++w) run += L.wsum[w];
            for (int i = 0; i < per; ++i) {
                if (w0 + i < n_words) {
                    pre[w0 + i] = run;
                    run += __popc(bits[w0 + i]);
                }
            }
            __syncthreads();
            for (int i = tid; i < n_sel; i += NT) {
                const uint64_t c = sel[i];
                const int32_t id = id_of(c);
                const int32_t pos = pre[id >> 5] + __popc(bits[id >> 5] & ((1u << (id & 31)) - 1u));
                oi[off + pos] = id;
                if (ov) ov[off + pos] = key_score((uint32_t)(c >> 32));
            }
        } else {
            // re-key with the index on top and sort
            for (int i = tid; i < n_sel; i += NT) {
                const uint64_t c = sel[i];
                sel[i] = ((uint64_t)(uint32_t)c << 32) | (c >> 32);
            }
            __syncthreads();
            sort_desc<NT>(sel, &L.u[kMaxK], n_sel);
            for (int j = tid; j < n_sel; j += NT) {
                const uint64_t c = sel[j];
                oi[off + j] = (int32_t)(0xFFFFFFFFu - (uint32_t)(c >> 32));
                if (ov) ov[off + j] = key_score((uint32_t)c);
            }
        }
        // forced blocks and padding around the selected run
        for (int j = tid; j < a.out_width; j += NT) {
            if (j >= off && j < off + n_sel) continue;
            int32_t id = -1;
            float v = __builtin_nanf("");
            if (f_first && j == 0) {
                id = 0;
                v = __builtin_inff();
            } else if (f_local && j == off + n_sel) {
                id = Lb;
                v = __builtin_inff();
            }
            oi[j] = id;
            if (ov) ov[j] = v;
        }
        return;
    }
    int32_t* oi;
    float* ov;
    if (final_out) {
        const int64_t g = a.rows.y0 + r.y;
        oi = a.out_idx + g * a.out_width;
        ov = a.out_val ? a.out_val + g * a.out_width : nullptr;
    } else {
        oi = a.run_idx + r.y * a.topk;
        ov = a.run_val + r.y * a.topk;
    }
    for (int j = tid; j < a.topk; j += NT) {
        int32_t id = -1;
        float v = __builtin_nanf("");
        if (j < n_sel) {
            const uint64_t c = sel[j];
            id = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
            v = key_score((uint32_t)(c >> 32));
        }
        oi[j] = id;
        if (ov) ov[j] = v;
    }
}

// Exact fallback for a threshold bin larger than the LDS candidate list:
// 8-bit radix select over the whole row (prior list first, then columns in
// key-index order, so "first in scan order" is "lowest index" among equal
// scores), then an ordered scan that collects the winners.  Fills
// L.u[0, n) and returns n.
template <bool VEC, int NT>
__device__ __forceinline__ int32_t radix_fallback(const SelectArgs& a, const RowCtx& r, SelectLds& L, int32_t K) {
    constexpr int kWaves = NT / kWave;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t* hist = reinterpret_cast<uint32_t*>(&L.u[kMaxK]);  // [kWaves][256]
    uint32_t prefix = 0;
    int shift_done = 32;
    int32_t kr = K;
    bool take_all = false;
    int32_t total = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < kWaves * 256; i += NT) hist[i] = 0;
        __syncthreads();
        auto f = [&](bool valid, uint32_t key, int32_t) {
            valid = valid && (shift_done >= 32 || (key >> shift_done) == (prefix >> shift_done));
            if (valid) atomicAdd(&hist[wave * 256 + ((key >> shift) & 255u)], 1u);
        };
        visit_prior<NT>(a, r, f);
        visit_columns<VEC, NT>(a, r, r.lo, r.hi, f);
        __syncthreads();
        if (wave == 0) {
            int32_t c[4], lsum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int bin = 255 - (4 * lane + i);
                int32_t v = 0;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) v += (int32_t)hist[w * 256 + bin];
                c[i] = v;
                lsum += v;
            }
            int32_t inc = lsum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int32_t v = __shfl_up(inc, o);
                if (lane >= o) inc += v;
            }
            const int32_t excl = inc - lsum;
            if (lane == 63) L.pick[3] = inc;
            if (excl < kr && kr <= inc) {
                int32_t cum = excl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (cum < kr && kr <= cum + c[i]) {
                        L.pick[0] = 255 - (4 * lane + i);
                        L.pick[1] = cum;
                        L.pick[2] = c[i];
                    }
                    cum += c[i];
                }
            }
        }
        __syncthreads();
        const int32_t bucket_total = L.pick[3];
        if (shift == 24) total = bucket_total;
        if (bucket_total <= kr) {
            take_all = shift == 24;
            kr = bucket_total;
            break;
        }
        kr -= L.pick[1];
        prefix |= (uint32_t)L.pick[0] << shift;
        shift_done = shift;
        const int32_t in_bucket = L.pick[2];
        __syncthreads();
        if (in_bucket == kr) break;
    }
    const int32_t need = take_all ? 0 : kr;
    const int32_t n_gt = take_all ? total : K - kr;
    if (tid == 0) L.cnt[0] = 0;
    __syncthreads();
    const uint32_t pb = shift_done < 32 ? (prefix >> shift_done) : 0u;
    int32_t eq_base = 0;
    auto g = [&](bool valid, uint32_t key, int32_t idx) {
        bool gt = false, eq = false;
        if (valid) {
            if (take_all || shift_done >= 32) {
                gt = take_all;
            } else {
                const uint32_t hi = key >> shift_done;
                gt = hi > pb;
                eq = hi == pb;
            }
        }
        const int32_t pos = wave_append(&L.cnt[0], gt);
        if (gt && pos < K) L.u[pos] = composite(key, idx);
        // workgroup-wide ordered count of `eq`
        const uint64_t bal = __ballot(eq);
        const int32_t below = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) L.wsum[wave] = __popcll(bal);
        __syncthreads();
        int32_t off = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            off += (w < wave) ? L.wsum[w] : 0;
            tot += L.wsum[w];
        }
        if (eq) {
            const int32_t p = eq_base + off + below;
            if (p < need) L.u[n_gt + p] = composite(key, idx);
        }
        eq_base += tot;
        __syncthreads();
    };
    // The prior list holds keys below every column's index, but in no
    // particular order: its tied entries are gathered, and when they are
    // more than needed, the ones with the lowest indices are picked by a
    // sort (a composite of equal keys orders by index alone).
    if (r.prior) {
        uint64_t* tie = &L.u[kMaxK];  // the histograms are done with
        if (tid == 0) L.cnt[1] = 0;
        __syncthreads();
        auto gp = [&](bool valid, uint32_t key, int32_t idx) {
            bool gt = false, eq = false;
            if (valid) {
                if (take_all || shift_done >= 32) {
                    gt = take_all;
                } else {
                    const uint32_t hi = key >> shift_done;
                    gt = hi > pb;
                    eq = hi == pb;
                }
            }
            const int32_t pos = wave_append(&L.cnt[0], gt);
            if (gt && pos < K) L.u[pos] = composite(key, idx);
            const int32_t pe = wave_append(&L.cnt[1], eq);
            if (eq) tie[pe] = composite(key, idx);
        };
        visit_prior<NT>(a, r, gp);
        __syncthreads();
        const int32_t n_tie = L.cnt[1];
        if (n_tie > need) sort_desc<NT>(tie, &L.u[kMaxK + kMaxK], n_tie);
        const int32_t take = min(n_tie, need);
        for (int i = tid; i < take; i += NT) L.u[n_gt + i] = tie[i];
        eq_base = take;
        __syncthreads();
    }
    // ordered scan of the columns: one candidate per thread per round
    // (scalar) keeps index order
    {
        RowCtx rr = r;
        for (int32_t base = r.lo; base < r.hi; base += NT) {
            const int32_t j = base + tid;
            int32_t idx = -1;
            float v = 0.0f;
            if (j < r.hi) {
                idx = column_index(a, rr, j);
                v = r.srow[j];
            }
            g(idx >= 0, score_key(v), idx);
        }
    }
    __syncthreads();
    return n_gt + need;
}

// sel[0, n_gt) is filled; cand[0, n_cand) holds composites that agree on
// every bit above bit first_shift + 8.  The best `need` candidates are
// appended to sel by an exact radix select, 8-bit digits from bit
// first_shift down, entirely in LDS: each round histograms the digit of the
// candidates that match every digit fixed so far, appends those above the
// digit that holds the need-th best, and fixes that digit.  Returns the
// selected count.
//
// `fixed` / `prefix` name bits already decided (a candidate is live while it
// matches them) and `live` counts the live candidates.
template <int NT>
__device__ __forceinline__ int32_t finish_from_candidates(SelectLds& L, int32_t n_gt, int32_t n_cand,
                                                 int32_t need, int first_shift, uint64_t prefix = 0,
                                                 uint64_t fixed = 0, int32_t live = -1) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t* cand = &L.u[kMaxK];
    uint32_t* hist = L.hist8;
    if (tid == 0) L.cnt[0] = n_gt;
    __syncthreads();
    const uint64_t all_bits = fixed | (first_shift >= 56 ? ~0ull : (1ull << (first_shift + 8)) - 1);
    if (live < 0) live = n_cand;
    for (int shift = first_shift; need > 0; shift = shift >= 8 ? shift - 8 : 0) {
        auto is_live = [&](uint64_t e) { return ((e ^ prefix) & fixed) == 0; };
        if (live <= need || fixed == all_bits) {
            // every remaining candidate is selected
            for (int base = 0; base < n_cand; base += NT) {
                const int i = base + tid;
                const uint64_t e = i < n_cand ? cand[i] : 0;
                const bool p = i < n_cand && is_live(e);
                const int32_t pos = wave_append(&L.cnt[0], p);
                if (p) L.u[pos] = e;
            }
            break;
        }
        for (int i = tid; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < n_cand; i += NT) {
            const uint64_t e = cand[i];
            if (is_live(e)) atomicAdd(&hist[(uint32_t)(e >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            int32_t c[4], lsum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[i] = (int32_t)hist[255 - (4 * lane + i)];
                lsum += c[i];
            }
            int32_t inc = lsum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int32_t v = __shfl_up(inc, o);
                if (lane >= o) inc += v;
            }
            const int32_t excl = inc - lsum;
            if (excl < need && need <= inc) {
                int32_t cum = excl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (cum < need && need <= cum + c[i]) {
                        L.pick[0] = 255 - (4 * lane + i);
                        L.pick[1] = cum;
                        L.pick[2] = c[i];
                    }
                    cum += c[i];
                }
            }
        }
        __syncthreads();
        const uint32_t d = (uint32_t)L.pick[0];
        const int32_t above = L.pick[1], in = L.pick[2];
        for (int base = 0; base < n_cand; base += NT) {
            const int i = base + tid;
            const uint64_t e = i < n_cand ? cand[i] : 0;
            const bool p = i < n_cand && is_live(e) && ((uint32_t)(e >> shift) & 255u) > d;
            const int32_t pos = wave_append(&L.cnt[0], p);
            if (p) L.u[pos] = e;
        }
        need -= above;
        live = in;
        prefix |= (uint64_t)d << shift;
        fixed |= 255ull << shift;
        __syncthreads();
    }
    __syncthreads();
    return L.cnt[0];
}

template <int NT>
__device__ __forceinline__ void setup_row(const SelectArgs& a, RowCtx& r, SelectLds& L, int64_t y,
                                 int32_t& count) {
    const int tid = threadIdx.x;
    r.y = y;
    r.t = a.rows.query(y);
    r.n_tok = a.vis.tokens(r.t);
    count = a.row_len ? a.row_len[y] : a.vis.count(r.t);
    r.prior = a.prior_val != nullptr && a.tile_begin > 0;
    r.srow = a.scores + y * a.score_stride;
    if (a.blocks_mode) {
        r.lo = 0;
        r.hi = a.n_cols;
        const int32_t n_ent = a.n_cols >> a.block_shift;
        const int32_t* src = a.blk + (a.rows.y0 + y) * a.blk_stride;
        for (int i = tid; i < n_ent; i += NT) L.blk[i] = src[i];
        r.blk_row = L.blk;
    } else {
        r.lo = a.col_lo;
        r.hi = min(a.n_cols, max(0, count - a.col_key0));
        r.blk_row = nullptr;
    }
}

// ------------------------------------------------- one workgroup per row

template <int NT>
__device__ __forceinline__ int32_t pool_best(SelectLds& L, int32_t n_pool, int32_t K, bool& sorted);

// Exact selection by a full histogram of the row (the path that never
// fails): the row's top-K candidates into L.u[0, n) (unsorted); returns n.
template <bool VEC, int NT>
__device__ __forceinline__ int32_t select_hist(const SelectArgs& a, const RowCtx& r, SelectLds& L, int32_t K,
                                               bool& sorted) {
    const int tid = threadIdx.x;
    sorted = false;
    if (K <= 0) return 0;
    uint32_t* hist = lds_hist(L);
    // pass 1: 12-bit histogram
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    __syncthreads();
    auto h = [&](bool valid, uint32_t key, int32_t) { hist_add(hist, valid, key >> kBinShift); };
    visit_prior<NT>(a, r, h);
    visit_columns<VEC, NT>(a, r, r.lo, r.hi, h);
    __syncthreads();
    find_threshold<NT>([&](int b) { return hist[b]; }, K, L.pick, L.wsum);
    const int32_t bstar = L.pick[0];
    const int32_t above = L.pick[1], inbin = L.pick[2], total = L.pick[3];
    __syncthreads();
    if (bstar >= 0 && inbin > kCap && inbin != K - above) return radix_fallback<VEC, NT>(a, r, L, K);
    const bool all = bstar < 0;  // total <= K
    if (!all && above + inbin <= kCap) {
        // pass 2: everything from the threshold bin up into the pool, whose
        // best K are then placed in order
        if (tid == 0) L.cnt[1] = 0;
        __syncthreads();
        auto cp = [&](bool valid, uint32_t key, int32_t idx) {
            const bool p = valid && (int32_t)(key >> kBinShift) >= bstar;
            const int32_t pos = wave_append(&L.cnt[1], p);
            if (p) L.u[kMaxK + pos] = composite(key, idx);
        };
        visit_prior<NT>(a, r, cp);
        // (the columns with batched appends: one atomic per wave and group)
        collect_ge<VEC, NT>(a, r, r.lo, r.hi, (uint32_t)bstar << kBinShift, &L.cnt[1], &L.u[kMaxK], kCap);
        __syncthreads();
        return pool_best<NT>(L, above + inbin, K, sorted);
    }
    // pass 2: collect
    const bool whole_bin = !all && inbin == K - above;
    if (tid == 0) {
        L.cnt[0] = 0;
        L.cnt[1] = 0;
    }
    __syncthreads();
    auto c = [&](bool valid, uint32_t key, int32_t idx) {
        const uint32_t bin = key >> kBinShift;
        const bool to_sel =
            valid && (all || (int32_t)bin > bstar || (whole_bin && (int32_t)bin == bstar));
        const bool to_cand = valid && !all && !whole_bin && (int32_t)bin == bstar;
        const int32_t ps = wave_append(&L.cnt[0], to_sel);
        if (to_sel && ps < kMaxK) L.u[ps] = composite(key, idx);
        const int32_t pc = wave_append(&L.cnt[1], to_cand);
        if (to_cand && pc < kCap) L.u[kMaxK + pc] = composite(key, idx);
    };
    visit_prior<NT>(a, r, c);
    visit_columns<VEC, NT>(a, r, r.lo, r.hi, c);
    __syncthreads();
    if (all) return total;
    if (whole_bin) return K;
    return finish_from_candidates<NT>(L, above, inbin, K - above, 44);
}

// Key threshold that at least K of the row's n candidates (prior list, then
// columns) reach with high probability, estimated from kSamples candidates
// (evenly spaced runs of kSampleRun consecutive ones).  With sv valid
// samples, the expected sample rank of the K-th best candidate is
// m = K * sv / n; the threshold is the key of sample rank m + d, with a
// margin d of three standard deviations of that rank (sqrt(m)) plus 4,
// capped so that the expected pool stays within 90 % of kCap.  The key is
// resolved to 16 bits with two 256-bin LDS histograms.  n > kSamples.
// Returns false when the sample cannot place it.
template <int NT>
__device__ __forceinline__ bool sample_threshold(const SelectArgs& a, const RowCtx& r, SelectLds& L,
                                                 int32_t n, int32_t K, uint32_t& tau) {
    const int tid = threadIdx.x;
    const int32_t np = r.prior ? prior_len(a) : 0;
    uint32_t* keys = reinterpret_cast<uint32_t*>(&L.u[kMaxK]);  // kSamples keys (0: no candidate)
    uint32_t* hist = L.hist8;                                   // 256 bins
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    if (tid == 0) L.cnt[0] = 0;
    __syncthreads();
    // every sample load is issued before any is used
    constexpr int PER = kSamples / NT;
    bool v[PER];
    float x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int s = tid + i * NT;
        // run s / kSampleRun starts at an even spacing; a run covers 64
        // consecutive bytes, so the sample touches 1/8 of the row's lines
        // (single spaced samples would touch every line of a long row)
        const int32_t q = min(n - 1, (int32_t)(((int64_t)(s / kSampleRun) * n) / (kSamples / kSampleRun)) +
                                         s % kSampleRun);
        if (q < np) {
            v[i] = a.prior_idx[r.y * np + q] >= 0;
            x[i] = a.prior_val[r.y * np + q];
        } else {
            const int32_t j = r.lo + (q - np);
            v[i] = column_index(a, r, j) >= 0;
            x[i] = r.srow[j];
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint32_t key = v[i] ? score_key(x[i]) : 0u;
        keys[tid + i * NT] = key;
        hist_add(hist, v[i], key >> 24);
        const uint64_t m = __ballot(v[i]);
        if ((threadIdx.x & 63) == 0 && m) atomicAdd(&L.cnt[0], (int32_t)__popcll(m));
    }
    __syncthreads();
    const int32_t sv = L.cnt[0];
    const float m = (float)K * (float)sv / (float)n;
    const float dmax = (0.9f * kCap - (float)K) * (float)sv / (float)n;
    const float rsf = ceilf(m + fminf(3.0f * sqrtf(m) + 4.0f, dmax));
    if (!(rsf >= 1.0f) || rsf >= (float)sv) return false;
    const int32_t rs = (int32_t)rsf;
    find_threshold_n<NT, 256>([&](int b) { return hist[b]; }, rs, L.pick, L.wsum);
    const int32_t b1 = L.pick[0];
    const int32_t r2 = rs - L.pick[1];
    __syncthreads();
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int s = tid; s < kSamples; s += NT) {
        const uint32_t k = keys[s];
        hist_add(hist, k != 0u && (int32_t)(k >> 24) == b1, (k >> 16) & 255u);
    }
    __syncthreads();
    find_threshold_n<NT, 256>([&](int b) { return hist[b]; }, r2, L.pick, L.wsum);
    const int32_t b2 = L.pick[0];
    tau = ((uint32_t)b1 << 24) | (b2 >= 0 ? (uint32_t)b2 << 16 : 0u);
    __syncthreads();
    return true;
}

// The best K of the pool cand[0, n) (K <= n <= kCap) into L.u[0, K), exact:
// a 12-bit first digit (histogram in the still empty list), then the LDS
// radix select of finish_from_candidates.  Returns K.
template <int NT>
__device__ __forceinline__ int32_t resolve_pool(SelectLds& L, int32_t n_pool, int32_t K) {
    const int tid = threadIdx.x;
    const uint64_t* cand = &L.u[kMaxK];
    if (n_pool == K) {
        for (int i = tid; i < n_pool; i += NT) L.u[i] = cand[i];
        __syncthreads();
        return K;
    }
    uint32_t* hist = reinterpret_cast<uint32_t*>(L.u);
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    __syncthreads();
    for (int base = 0; base < n_pool; base += NT) {
        const int i = base + tid;
        hist_add(hist, i < n_pool, i < n_pool ? (uint32_t)(cand[i] >> 52) : 0u);
    }
    __syncthreads();
    find_threshold<NT>([&](int b) { return hist[b]; }, K, L.pick, L.wsum);
    const int32_t b = L.pick[0], above = L.pick[1], inbin = L.pick[2];
    __syncthreads();
    if (tid == 0) L.cnt[0] = 0;
    __syncthreads();
    for (int base = 0; base < n_pool; base += NT) {
        const int i = base + tid;
        const uint64_t e = i < n_pool ? cand[i] : 0;
        const bool p = i < n_pool && (int32_t)(e >> 52) > b;
        const int32_t pos = wave_append(&L.cnt[0], p);
        if (p) L.u[pos] = e;
    }
    __syncthreads();
    return finish_from_candidates<NT>(L, above, n_pool, K - above, 44, (uint64_t)b << 52,
                                      0xFFFull << 52, inbin);
}

// The best K of the pool L.u[kMaxK, kMaxK + n) (K <= n <= kCap) into
// L.u[0, K): sorted by counting when it applies (sorted = true), else by
// the radix select (unsorted).  Returns K.
template <int NT>
__device__ __forceinline__ int32_t pool_best(SelectLds& L, int32_t n_pool, int32_t K, bool& sorted) {
    uint64_t* cand = &L.u[kMaxK];
    sorted = counting_topk<NT, kCap>(L, cand, n_pool, K, L.u, cand, reinterpret_cast<uint32_t*>(L.u));
    return sorted ? K : resolve_pool<NT>(L, n_pool, K);
}

// Exact selection of the row's top-K candidates into L.u[0, n) (unsorted);
// returns n.
//
// Threshold prefilter (the threshold-based Indexer-TopK abstract listed on
// the StreamIndex page: bin the scores and keep only candidates above a
// tight threshold, the result staying exact): a row with more candidates
// than the LDS pool holds gets a key threshold from a sample, sized for
// about 1.4 K candidates; one pass keeps every candidate at or above it
// in the LDS pool.  If the pool holds at least K candidates, every
// candidate left out ranks below all of them, so the pool's best K are the
// answer; they are found by an LDS radix select.  A pool that is too small
// or overflows falls back to the full histogram path.
template <bool VEC, int NT>
__device__ __forceinline__ int32_t select_core(const SelectArgs& a, const RowCtx& r, SelectLds& L, int32_t K,
                                               bool& sorted) {
    const int tid = threadIdx.x;
    sorted = false;
    if (K <= 0) return 0;
    const int32_t n_cols = max(0, r.hi - r.lo);
    const int32_t n_total = n_cols + (r.prior ? prior_len(a) : 0);
    uint64_t* cand = &L.u[kMaxK];
    uint32_t tau = 0;
    if (n_total > K && n_total <= kMaxK) {
        // few candidates: gather them all and sort them; the best K lead
        if (tid == 0) L.cnt[1] = 0;
        __syncthreads();
        auto c = [&](bool valid, uint32_t key, int32_t idx) {
            const int32_t pos = wave_append(&L.cnt[1], valid);
            if (valid) L.u[pos] = composite(key, idx);
        };
        visit_prior<NT>(a, r, c);
        collect_ge<VEC, NT>(a, r, r.lo, r.hi, 0u, &L.cnt[1], L.u, kMaxK);
        __syncthreads();
        const int32_t n = L.cnt[1];
        sort_final<NT>(L, n);
        sorted = true;
        return min(K, n);
    }
    // (the refinement rows of kept blocks keep the histogram route below
    // 16384: there the sampled threshold was measured slower)
    if (n_total > K && n_total < (a.blocks_mode ? kPrefilterMin : kPrefilterMinTok))
        return select_hist<VEC, NT>(a, r, L, K, sorted);
    if (n_total > kCap) {
        if (!sample_threshold<NT>(a, r, L, n_total, K, tau)) return select_hist<VEC, NT>(a, r, L, K, sorted);
    }
    // one pass: the pool of candidates with key >= tau (all of them when
    // tau = 0); a row that fits the answer goes straight to the list
    const bool direct = n_total <= K;
    uint64_t* dst = direct ? L.u : cand;
    const int32_t cap = direct ? kMaxK : kCap;
    if (tid == 0) L.cnt[1] = 0;
    __syncthreads();
    auto c = [&](bool valid, uint32_t key, int32_t idx) {
        const bool p = valid && key >= tau;
        const int32_t pos = wave_append(&L.cnt[1], p);
        if (p && pos < cap) dst[pos] = composite(key, idx);
    };
    visit_prior<NT>(a, r, c);
    collect_ge<VEC, NT>(a, r, r.lo, r.hi, tau, &L.cnt[1], dst, cap);
    __syncthreads();
    const int32_t n_pool = L.cnt[1];
    if (direct) return n_pool;
    if (tau == 0u && n_pool <= K) {
        // fewer valid candidates than K (block slots without a key)
        for (int i = tid; i < n_pool; i += NT) L.u[i] = cand[i];
        __syncthreads();
        return n_pool;
    }
    if (n_pool < K || n_pool > kCap) {
        __syncthreads();
        return select_hist<VEC, NT>(a, r, L, K, sorted);
    }
    return pool_best<NT>(L, n_pool, K, sorted);
}

}  // namespace

}  // namespace tks

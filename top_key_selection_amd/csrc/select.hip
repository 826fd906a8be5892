// select.hip -- exact per-query top-k on gfx950 (one workgroup per row).
//
// The per-query top-k of the HISA abstract (a per-query set of k token
// indices) and the partition-merge of the StreamIndex abstract (a partial
// top-k per key tile merged into a running list) both reduce to one
// operation: from a row's candidates -- the running list of earlier tiles
// followed by this tile's scores, in key-index order -- keep the k best in
// the total order (score descending, key index ascending).
//
//   1. Radix select on the orderable 32-bit key of each score, 8 bits per
//      pass from the top, finds the k-th key's bucket; per-wave LDS
//      histograms keep atomic contention inside a wave.  A pass that finds a
//      bucket whose entries are all needed stops early.
//   2. One ordered pass collects every candidate above the bucket (atomic
//      append) and the first `need` candidates inside it in key-index order
//      (a workgroup prefix count), which is exactly the tie rule.
//   3. A bitonic sort in LDS orders the <= k survivors on the 64-bit
//      composite (key << 32 | ~index); the row is written with -1 / NaN
//      padding.
//
// Block-select output mode writes the kept blocks in ascending block order
// with the forced first / local blocks added (score +inf).
#include "tks_launch.hpp"

namespace tks {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxK = 2048;
constexpr int kMaxBlkEntries = 512;

struct RowCtx {
    int64_t y;
    int32_t t;
    int32_t lo, hi;        // valid score columns [lo, hi)
    int32_t n_tok;
    bool prior;
    const float* srow;
    const int32_t* blk_row;  // LDS copy in block mode
};

// Visit candidate p of the row's index space (prior list first, then score
// columns lo..hi-1).  Returns false for an empty / invalid slot.
__device__ inline bool candidate(const SelectArgs& a, const RowCtx& r, int32_t p, uint32_t& key,
                                 int32_t& idx) {
    const int32_t np = r.prior ? a.topk : 0;
    if (p < np) {
        idx = a.prior_idx[r.y * a.topk + p];
        if (idx < 0) return false;
        key = score_key(a.prior_val[r.y * a.topk + p]);
        return true;
    }
    const int32_t j = r.lo + (p - np);
    if (j >= r.hi) return false;
    if (a.blocks_mode) {
        const int32_t b = r.blk_row[j >> a.block_shift];
        if (b < 0 || r.n_tok <= 0 || b > ((r.n_tok - 1) >> a.block_shift)) return false;
        idx = (b << a.block_shift) + (j & ((1 << a.block_shift) - 1));
        if (idx >= r.n_tok) return false;
    } else {
        idx = a.col_key0 + j;
    }
    key = score_key(r.srow[j]);
    return true;
}

__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a, int64_t n_rows) {
    __shared__ uint64_t s_sel[kMaxK];
    __shared__ uint32_t s_hist[kWaves][256];
    __shared__ int32_t s_blk[kMaxBlkEntries];
    __shared__ int32_t s_wsum[kWaves];
    __shared__ int32_t s_pick[4];
    __shared__ int32_t s_cgt;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    RowCtx r;
    r.y = blockIdx.x;
    if (r.y >= n_rows) return;
    r.t = a.rows.query(r.y);
    r.n_tok = a.vis.tokens(r.t);
    const int32_t count = a.row_len ? a.row_len[r.y] : a.vis.count(r.t);

    // Rows whose visible keys all lie before this tile finished earlier.
    if (!a.always_final && a.tile_begin > 0 && count <= a.tile_begin) return;
    const bool final_out = a.always_final || count <= a.tile_end;
    r.prior = a.prior_val != nullptr && a.tile_begin > 0;

    r.srow = a.scores + r.y * a.score_stride;
    if (a.blocks_mode) {
        r.lo = 0;
        r.hi = a.n_cols;
        const int32_t n_ent = a.n_cols >> a.block_shift;
        const int32_t* src = a.blk + (a.rows.y0 + r.y) * a.blk_stride;
        for (int i = tid; i < n_ent; i += kThreads) s_blk[i] = src[i];
        r.blk_row = s_blk;
    } else {
        r.lo = a.col_lo;
        r.hi = min(a.n_cols, max(0, count - a.col_key0));
        r.blk_row = nullptr;
    }
    const int32_t n_slots = (r.prior ? a.topk : 0) + max(0, r.hi - r.lo);
    const int32_t K = a.topk;

    // ---- 1. radix select -------------------------------------------------
    uint32_t prefix = 0;     // selected high bits
    int shift_done = 32;     // bits >= shift_done are fixed in `prefix`
    int32_t kr = K;          // rank still to place inside the current bucket
    bool take_all = false;
    int32_t total = 0;
    for (int shift = 24; shift >= 0 && K > 0; shift -= 8) {
        for (int i = tid; i < kWaves * 256; i += kThreads) (&s_hist[0][0])[i] = 0;
        __syncthreads();
        for (int32_t p = tid; p < n_slots; p += kThreads) {
            uint32_t key;
            int32_t idx;
            if (!candidate(a, r, p, key, idx)) continue;
            if (shift_done < 32 && (key >> shift_done) != (prefix >> shift_done)) continue;
            atomicAdd(&s_hist[wave][(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // bins in descending order: position 4*lane + i is bin 255 - 4*lane - i
            int32_t c[4];
            int32_t lsum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int bin = 255 - (4 * lane + i);
                int32_t v = 0;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) v += (int32_t)s_hist[w][bin];
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
            if (lane == 63) s_pick[3] = inc;  // candidates in the current bucket
            if (excl < kr && kr <= inc) {
                int32_t cum = excl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (cum < kr && kr <= cum + c[i]) {
                        s_pick[0] = 255 - (4 * lane + i);
                        s_pick[1] = cum;
                        s_pick[2] = c[i];
                    }
                    cum += c[i];
                }
            }
        }
        __syncthreads();
        const int32_t bucket_total = s_pick[3];
        if (shift == 24) total = bucket_total;
        if (bucket_total <= kr) {  // every candidate of the bucket is kept
            take_all = shift == 24;
            kr = bucket_total;
            break;
        }
        const int32_t d = s_pick[0];
        kr -= s_pick[1];
        prefix |= (uint32_t)d << shift;
        shift_done = shift;
        const int32_t in_bucket = s_pick[2];
        __syncthreads();
        if (in_bucket == kr) break;  // the whole bucket is needed
    }
    if (K == 0) {
        take_all = false;
        kr = 0;
        total = 0;
    }

    // ---- 2. ordered collection ------------------------------------------
    // Selected = candidates whose bits above shift_done exceed the bucket
    // prefix, plus the first `need` candidates inside the bucket.
    int32_t need, n_gt;
    if (take_all) {
        need = 0;
        n_gt = total;
    } else {
        need = kr;
        n_gt = K - kr;
    }
    if (K == 0) n_gt = 0;
    if (tid == 0) s_cgt = 0;
    __syncthreads();
    const uint32_t pb = shift_done < 32 ? (prefix >> shift_done) : 0u;
    int32_t eq_base = 0;
    for (int32_t base = 0; base < n_slots && K > 0; base += kThreads) {
        const int32_t p = base + tid;
        uint32_t key = 0;
        int32_t idx = -1;
        bool gt = false, eq = false;
        if (p < n_slots && candidate(a, r, p, key, idx)) {
            if (take_all || shift_done >= 32) {
                gt = take_all;
                eq = !take_all;
            } else {
                const uint32_t hi = key >> shift_done;
                gt = hi > pb;
                eq = hi == pb;
            }
        }
        const uint64_t comp = ((uint64_t)key << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
        if (gt) {
            const int32_t pos = atomicAdd(&s_cgt, 1);
            if (pos < K) s_sel[pos] = comp;
        }
        // workgroup-wide exclusive count of `eq` in slot order
        const uint64_t bal = __ballot(eq);
        const int32_t below = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) s_wsum[wave] = __popcll(bal);
        __syncthreads();
        int32_t off = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int32_t c = s_wsum[w];
            off += (w < wave) ? c : 0;
            tot += c;
        }
        if (eq) {
            const int32_t pos = eq_base + off + below;
            if (pos < need) s_sel[n_gt + pos] = comp;
        }
        eq_base += tot;
        __syncthreads();
    }
    const int32_t n_sel = n_gt + need;

    // ---- 3. sort survivors ------------------------------------------------
    if (a.blockselect) {
        // ascending block index: composite with the index on top
        for (int i = tid; i < n_sel; i += kThreads) {
            const uint64_t c = s_sel[i];
            const uint32_t key = (uint32_t)(c >> 32);
            const uint32_t nidx = (uint32_t)c;  // 0xFFFFFFFF - idx
            s_sel[i] = ((uint64_t)nidx << 32) | key;
        }
    }
    int32_t P2 = 1;
    while (P2 < n_sel) P2 <<= 1;
    for (int i = n_sel + tid; i < P2; i += kThreads) s_sel[i] = 0;
    __syncthreads();
    for (int size = 2; size <= P2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (P2 >> 1); i += kThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t x = s_sel[lo], z = s_sel[hi];
                if ((x < z) == desc) {
                    s_sel[lo] = z;
                    s_sel[hi] = x;
                }
            }
            __syncthreads();
        }
    }

    // ---- 4. write ---------------------------------------------------------
    if (a.blockselect) {
        const int32_t L = r.n_tok > 0 ? (r.n_tok - 1) / a.sel_block : -1;
        const bool f_first = (a.force_flags & 1u) && L > 0;
        const bool f_local = (a.force_flags & 2u) && L >= 0;
        const int64_t g = a.rows.y0 + r.y;
        int32_t* oi = a.out_idx + g * a.out_width;
        float* ov = a.out_val ? a.out_val + g * a.out_width : nullptr;
        const int32_t off = f_first ? 1 : 0;
        for (int j = tid; j < a.out_width; j += kThreads) {
            int32_t id = -1;
            float v = __builtin_nanf("");
            if (f_first && j == 0) {
                id = 0;
                v = __builtin_inff();
            } else if (j - off < n_sel) {
                const uint64_t c = s_sel[j - off];
                id = (int32_t)(0xFFFFFFFFu - (uint32_t)(c >> 32));
                v = key_score((uint32_t)c);
            } else if (f_local && j == off + n_sel) {
                id = L;
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
    for (int j = tid; j < K; j += kThreads) {
        int32_t id = -1;
        float v = __builtin_nanf("");
        if (j < n_sel) {
            const uint64_t c = s_sel[j];
            id = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
            v = key_score((uint32_t)(c >> 32));
        }
        oi[j] = id;
        if (ov) ov[j] = v;
    }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, int64_t n_rows, hipStream_t stream) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)n_rows), dim3(kThreads), 0, stream, a,
                       n_rows);
    return hipGetLastError();
}

}  // namespace tks

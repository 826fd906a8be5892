// select.hip -- exact per-query top-k kernels on gfx950 and their launchers
// (the device building blocks are in select_impl.hpp).  Block-select rows of
// at most 2048 blocks take a wave each, with no LDS (below).
#include "select_impl.hpp"

namespace tks {

namespace {

template <bool VEC, int NT>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a, int64_t n_rows) {
    __shared__ SelectLds L;
    if ((int64_t)blockIdx.x >= n_rows) return;
    RowCtx r;
    int32_t count;
    setup_row<NT>(a, r, L, blockIdx.x, count);
    if (!a.always_final && a.tile_begin > 0 && count <= a.tile_begin) return;
    const bool final_out = a.always_final || count <= a.tile_end;
    const int32_t K = a.topk;
    bool sorted;
    const int32_t n_sel = select_core<VEC, NT>(a, r, L, K, sorted);
    __syncthreads();
    // (block-select output is ordered by block index: write_row does that;
    // the running list of a non-final tile needs no order)
    if (!a.blockselect && final_out && !sorted) sort_final<NT>(L, n_sel);
    write_row<NT>(a, r, L, n_sel, final_out);
}

// ------------------------------------------- few long rows over every CU
//
// With fewer rows than CUs, one workgroup per row leaves most of the chip
// idle.  The prefilter then runs as three kernels: (1) one workgroup per
// row draws the sample and stores the row's key threshold; (2) workgroups
// over (row, column partition) append every candidate at or above it to
// the row's pool in global memory (gathered in LDS first, then one atomic
// per workgroup on the row's counter reserves their run); (3) one workgroup per row loads the pool and resolves it
// exactly in LDS -- or, when the pool came out too small or overflowed,
// selects from the whole row with the full histogram path.  Only rows
// without a prior list take this path.

constexpr uint32_t kNoTau = 0xFFFFFFFFu;  // no usable threshold: stage 3 scans the row
constexpr int32_t kFilterSpan = 4096;     // columns per filter workgroup

struct PrefilterWs {
    uint32_t* tau;    // [rows]
    int32_t* count;   // [rows]
    uint64_t* pool;   // [rows, kCap]
};

__host__ __device__ inline PrefilterWs prefilter_ws(void* ws, int64_t n_rows) {
    char* p = static_cast<char*>(ws);
    PrefilterWs w;
    w.pool = reinterpret_cast<uint64_t*>(p);
    w.tau = reinterpret_cast<uint32_t*>(p + n_rows * kCap * 8);
    w.count = reinterpret_cast<int32_t*>(p + n_rows * kCap * 8 + n_rows * 4);
    return w;
}

template <int NT>
__global__ __launch_bounds__(NT) void prefilter_sample_kernel(SelectArgs a, int64_t n_rows, PrefilterWs w) {
    __shared__ SelectLds L;
    if ((int64_t)blockIdx.x >= n_rows) return;
    RowCtx r;
    int32_t count;
    setup_row<NT>(a, r, L, blockIdx.x, count);
    const int32_t n = max(0, r.hi - r.lo);
    uint32_t tau = 0;  // a row that fits the pool keeps every candidate
    if (n > kCap) {
        const int32_t K = a.topk;
        if (!sample_threshold<NT>(a, r, L, n, K, tau)) tau = kNoTau;
    }
    if (threadIdx.x == 0) {
        w.tau[r.y] = tau;
        w.count[r.y] = 0;
    }
}

template <bool VEC>
__global__ __launch_bounds__(256) void prefilter_filter_kernel(SelectArgs a, int64_t n_rows, int32_t span,
                                                               PrefilterWs w) {
    const int64_t y = blockIdx.x;
    if (y >= n_rows) return;
    // (kNoTau passes no finite score, so such a row appends nothing; the
    // score loads need not wait for the threshold)
    const uint32_t tau = w.tau[y];
    RowCtx r;
    r.y = y;
    r.t = a.rows.query(y);
    r.n_tok = a.vis.tokens(r.t);
    const int32_t count = a.row_len ? a.row_len[y] : a.vis.count(r.t);
    r.prior = false;
    r.srow = a.scores + y * a.score_stride;
    r.blk_row = nullptr;
    const int32_t lo = a.col_lo, hi = min(a.n_cols, max(0, count - a.col_key0));
    r.lo = lo + (int32_t)blockIdx.y * span;
    r.hi = min(hi, r.lo + span);
    if (r.lo >= r.hi) return;
    // gather the partition's hits in LDS, then reserve their run of the
    // row's pool with one global atomic
    __shared__ uint64_t buf[kFilterSpan];
    __shared__ int32_t n_hit, base;
    if (threadIdx.x == 0) n_hit = 0;
    __syncthreads();
    collect_ge<VEC, 256>(a, r, r.lo, r.hi, tau, &n_hit, buf, kFilterSpan);
    __syncthreads();
    if (threadIdx.x == 0) base = atomicAdd(w.count + y, n_hit);
    __syncthreads();
    uint64_t* pool = w.pool + y * kCap;
    for (int i = threadIdx.x; i < n_hit; i += 256)
        if (base + i < kCap) pool[base + i] = buf[i];
}

template <bool VEC, int NT>
__global__ __launch_bounds__(NT) void prefilter_finish_kernel(SelectArgs a, int64_t n_rows, PrefilterWs w) {
    __shared__ SelectLds L;
    const int tid = threadIdx.x;
    if ((int64_t)blockIdx.x >= n_rows) return;
    RowCtx r;
    int32_t count;
    setup_row<NT>(a, r, L, blockIdx.x, count);
    const bool final_out = a.always_final || count <= a.tile_end;
    const int32_t K = a.topk;
    const uint32_t tau = w.tau[r.y];
    const int32_t n_pool = w.count[r.y];
    int32_t n_sel;
    bool sorted = false;
    if (tau != kNoTau && ((tau == 0u && n_pool <= K) || (n_pool >= K && n_pool <= kCap))) {
        const uint64_t* src = w.pool + r.y * kCap;
        uint64_t* dst = n_pool <= K ? L.u : &L.u[kMaxK];
        for (int i = tid; i < n_pool; i += NT) dst[i] = src[i];
        __syncthreads();
        n_sel = n_pool <= K ? n_pool : pool_best<NT>(L, n_pool, K, sorted);
    } else {
        n_sel = select_hist<VEC, NT>(a, r, L, K, sorted);
    }
    __syncthreads();
    if (!sorted) sort_final<NT>(L, n_sel);
    write_row<NT>(a, r, L, n_sel, final_out);
}

// ------------------------------------------- block selection, a wave per row
//
// A block-select row is short (one score per pooled block: 512 for 65,536
// keys in blocks of 128) and keeps few blocks, so one wave holds the whole
// row in registers -- lane l the columns [l E, l E + E) -- and needs neither
// LDS nor barriers:
//   * the k-th largest score key T is built bit by bit from the top: a bit
//     stays set when at least k keys reach the value so far (one count over
//     the wave per bit; bits that every valid key shares are taken as they
//     are), stopping as soon as exactly k keys reach it;
//   * the kept columns are the keys above T and, of the keys equal to T,
//     those with the lowest block indices (the composite order);
//   * lane order is column order, so a kept block's output slot is the
//     number of kept blocks in lower columns (a prefix over the wave), and
//     the list comes out in ascending block order without a sort.

// Sum over the wave of a per-lane count below 2^BITS (ballots of its bits).
template <int BITS>
__device__ __forceinline__ int32_t wave_count_sum(uint32_t c) {
    int32_t s = 0;
#pragma unroll
    for (int b = 0; b < BITS; ++b) s += __popcll(__ballot((c >> b) & 1u)) << b;
    return s;
}

// ... of the lanes below this one.
template <int BITS>
__device__ __forceinline__ int32_t wave_count_prefix(uint32_t c, uint64_t below) {
    int32_t s = 0;
#pragma unroll
    for (int b = 0; b < BITS; ++b) s += __popcll(__ballot((c >> b) & 1u) & below) << b;
    return s;
}

// Row y of a block-select launch by one wave, from the row's scores srow
// (16-byte aligned when VEC).  Columns at or past the row's candidate range
// are not read.
template <int E, bool VEC>
__device__ __forceinline__ void wave_block_select(const SelectArgs& a, int64_t y, const float* srow) {
    constexpr int BITS = E <= 8 ? 4 : E <= 16 ? 5 : 6;  // bits of a lane's count 0..E
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    const int32_t t = a.rows.query(y);
    const int32_t n_tok = a.vis.tokens(t);
    const int32_t count = a.row_len ? a.row_len[y] : a.vis.count(t);
    const int32_t lo = a.col_lo;
    const int32_t hi = min(a.n_cols, max(0, count - a.col_key0));
    const int32_t j0 = lane * E;

    // the lane's columns; nothing at or past hi is read
    uint32_t key[E];
    uint32_t valid = 0u;  // bit e: column j0 + e is a candidate
#pragma unroll
    for (int g = 0; g < E; g += 4) {
        float v[4];
        if (VEC && j0 + g + 3 < hi) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(srow + j0 + g);
            v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = j0 + g + i < hi ? srow[j0 + g + i] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int32_t j = j0 + g + i;
            key[g + i] = score_key(v[i]);
            if (j >= lo && j < hi) valid |= 1u << (g + i);
        }
    }
    const int32_t n_valid = wave_count_sum<BITS>((uint32_t)__popc(valid));
    const int32_t K = a.topk;
    uint32_t sel = valid;  // every candidate when there are at most K
    if (n_valid > K) {
        sel = 0u;
        if (K > 0) {
            // the bits shared by every valid key: the common prefix of the
            // smallest and the largest one
            uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if ((valid >> e) & 1u) {
                    kmin = min(kmin, key[e]);
                    kmax = max(kmax, key[e]);
                }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
                kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
            }
            const uint32_t diff = kmin ^ kmax;
            uint32_t T = kmin;
            if (diff != 0u) {
                const int top = 31 - __builtin_clz(diff);
                T = kmin & ~(uint32_t)((2ull << top) - 1ull);
                // every valid key is >= T: the count starts at n_valid > K.
                // The search ends early once exactly K keys reach T: those
                // K are the answer whatever the lower bits.  (Keys of
                // non-candidates are 0 here, below every c >= 1.)
                uint32_t vk[E];
#pragma unroll
                for (int e = 0; e < E; ++e) vk[e] = ((valid >> e) & 1u) ? key[e] : 0u;
                for (int b = top; b >= 0; --b) {
                    const uint32_t c = T | (1u << b);
                    int32_t n = 0;
#pragma unroll
                    for (int e = 0; e < E; ++e) n += __popcll(__ballot(vk[e] >= c));
                    if (n >= K) {
                        T = c;
                        if (n == K) break;
                    }
                }
            }
            // keys above T, then the lowest columns among the keys equal to T
            uint32_t n_gt = 0, n_eq = 0, gt = 0u, eq = 0u;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool v = (valid >> e) & 1u;
                if (v && key[e] > T) {
                    gt |= 1u << e;
                    ++n_gt;
                }
                if (v && key[e] == T) {
                    eq |= 1u << e;
                    ++n_eq;
                }
            }
            const int32_t need = K - wave_count_sum<BITS>(n_gt);
            int32_t r = wave_count_prefix<BITS>(n_eq, below);
            sel = gt;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if ((eq >> e) & 1u) {
                    if (r < need) sel |= 1u << e;
                    ++r;
                }
        }
    }
    const int32_t n_sel = min(K, n_valid);

    // output: [first block] kept blocks ascending [local block], padding
    const int32_t Lb = n_tok > 0 ? (n_tok - 1) / a.sel_block : -1;
    const bool f_first = (a.force_flags & 1u) && Lb > 0;
    const bool f_local = (a.force_flags & 2u) && Lb >= 0;
    const int64_t gr = a.rows.y0 + y;
    int32_t* oi = a.out_idx + gr * a.out_width;
    float* ov = a.out_val ? a.out_val + gr * a.out_width : nullptr;
    const int32_t off = f_first ? 1 : 0;
    int32_t pos = off + wave_count_prefix<BITS>((uint32_t)__popc(sel), below);
#pragma unroll
    for (int e = 0; e < E; ++e)
        if ((sel >> e) & 1u) {
            oi[pos] = a.col_key0 + j0 + e;
            if (ov) ov[pos] = key_score(key[e]);
            ++pos;
        }
    for (int j = lane; j < a.out_width; j += 64) {
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
}

// A block-select row per wave (wave_block_select), scores in global memory.
template <int E, bool VEC>
__global__ __launch_bounds__(256) void block_select_wave_kernel(SelectArgs a, int64_t n_rows) {
    const int64_t y = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (y >= n_rows) return;
    wave_block_select<E, VEC>(a, y, a.scores + y * a.score_stride);
}

bool vec_ok(const SelectArgs& a) {
    return (reinterpret_cast<uintptr_t>(a.scores) % 16 == 0) && (a.score_stride % 4 == 0);
}

template <int NT>
void launch_nt(const SelectArgs& a, int64_t n_rows, dim3 grid, hipStream_t stream) {
    if (vec_ok(a))
        hipLaunchKernelGGL((select_kernel<true, NT>), grid, dim3(NT), 0, stream, a, n_rows);
    else
        hipLaunchKernelGGL((select_kernel<false, NT>), grid, dim3(NT), 0, stream, a, n_rows);
}

template <int E>
void launch_block_wave(const SelectArgs& a, int64_t n_rows, hipStream_t stream) {
    // few rows: a wave per workgroup, spread over the CUs; else 4 rows each
    const int rpw = n_rows < 1024 ? 1 : 4;
    const dim3 grid((unsigned)((n_rows + rpw - 1) / rpw));
    if (vec_ok(a))
        hipLaunchKernelGGL((block_select_wave_kernel<E, true>), grid, dim3(64 * rpw), 0, stream, a, n_rows);
    else
        hipLaunchKernelGGL((block_select_wave_kernel<E, false>), grid, dim3(64 * rpw), 0, stream, a, n_rows);
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, int64_t n_rows, hipStream_t stream) {
    if (n_rows <= 0) return hipSuccess;
    if (a.blockselect && !a.prior_val && a.n_cols <= 2048) {
        if (a.n_cols <= 512)
            launch_block_wave<8>(a, n_rows, stream);
        else if (a.n_cols <= 1024)
            launch_block_wave<16>(a, n_rows, stream);
        else
            launch_block_wave<32>(a, n_rows, stream);
        return hipGetLastError();
    }
    // few rows: a wide workgroup per row; many long rows: 512-thread ones
    // (two per CU at 95 VGPRs), which keep more loads in flight per row and
    // let one row's sampling and final sort overlap the other's streaming
    // pass; many short rows (block lists): 256 threads, whose barriers cost
    // less
    if (n_rows < 512)
        launch_nt<1024>(a, n_rows, dim3((unsigned)n_rows), stream);
    else if (a.n_cols > 2048)
        launch_nt<512>(a, n_rows, dim3((unsigned)n_rows), stream);
    else
        launch_nt<256>(a, n_rows, dim3((unsigned)n_rows), stream);
    return hipGetLastError();
}

SelectSplit select_split(int64_t n_rows, int32_t n_cols, int32_t topk) {
    SelectSplit sp{0, 0};
    constexpr int32_t span = kFilterSpan;
    // fewer rows than CUs and rows long enough for the prefilter
    if (n_rows <= 0 || n_rows >= 256 || n_cols < kPrefilterMin || topk > kMaxK) return sp;
    sp.parts = (n_cols + span - 1) / span;
    sp.span = span;
    return sp;
}

size_t select_split_workspace(int64_t n_rows, const SelectSplit& sp) {
    if (sp.parts == 0) return 0;
    return (size_t)((n_rows * (kCap * 8 + 8) + 255) / 256 * 256);
}

hipError_t launch_select_split(const SelectArgs& a, int64_t n_rows, const SelectSplit& sp,
                               void* ws, hipStream_t stream) {
    if (n_rows <= 0) return hipSuccess;
    if (a.blocks_mode || (a.prior_val && a.tile_begin > 0))
        return hipErrorInvalidValue;  // planned for contiguous rows without a prior list only
    const PrefilterWs w = prefilter_ws(ws, n_rows);
    hipLaunchKernelGGL((prefilter_sample_kernel<1024>), dim3((unsigned)n_rows), dim3(1024), 0, stream, a,
                       n_rows, w);
    const dim3 g2((unsigned)n_rows, (unsigned)sp.parts);
    if (vec_ok(a)) {
        hipLaunchKernelGGL((prefilter_filter_kernel<true>), g2, dim3(256), 0, stream, a, n_rows, sp.span, w);
        hipLaunchKernelGGL((prefilter_finish_kernel<true, 1024>), dim3((unsigned)n_rows), dim3(1024), 0,
                           stream, a, n_rows, w);
    } else {
        hipLaunchKernelGGL((prefilter_filter_kernel<false>), g2, dim3(256), 0, stream, a, n_rows, sp.span, w);
        hipLaunchKernelGGL((prefilter_finish_kernel<false, 1024>), dim3((unsigned)n_rows), dim3(1024), 0,
                           stream, a, n_rows, w);
    }
    return hipGetLastError();
}

}  // namespace tks

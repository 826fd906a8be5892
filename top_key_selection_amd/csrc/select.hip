// select.hip -- exact per-query top-k kernels on gfx950 and their launchers
// (the device building blocks are in select_impl.hpp).
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

}  // namespace

hipError_t launch_select(const SelectArgs& a, int64_t n_rows, hipStream_t stream) {
    if (n_rows <= 0) return hipSuccess;
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

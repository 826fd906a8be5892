// gather.hip -- re-layout of the selected key / value rows on gfx950 (the
// LongCat Sparse Attention abstract, strategy (1): scattered KV entries that
// the top-k selects are copied into a contiguous, aligned layout, so the
// attention that consumes them reads with coalesced loads).
//
// out[b, t, j, :] = kv[b, idx[b, t, j], :] (row_bytes bytes), zeros where
// idx[b, t, j] is -1 or outside [0, n_kv).  The copy is HBM-bound: one
// 16-byte piece per thread task, consecutive threads on consecutive pieces
// of a row (whole cache lines on both sides), four tasks in flight per
// thread, nontemporal stores (the output is read once, later).
#include <algorithm>

#include "tks_launch.hpp"

namespace tks {

namespace {

constexpr int kThreads = 256;
constexpr int kTasks = 4;  // 16-byte pieces in flight per thread

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a, int64_t n_pieces) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int32_t pr = a.row_bytes / 16;  // pieces per row
    for (int64_t base = t0; base < n_pieces; base += kTasks * stride) {
        u32x4 v[kTasks];
        int64_t dst[kTasks];
#pragma unroll
        for (int u = 0; u < kTasks; ++u) {
            const int64_t task = base + u * stride;
            v[u] = u32x4{0, 0, 0, 0};
            dst[u] = -1;
            if (task < n_pieces) {
                const int64_t row = task / pr;          // output row (b, t, j)
                const int32_t piece = (int32_t)(task - row * pr);
                const int64_t bq = row / a.topk;        // query row (b, t)
                const int32_t b = (int32_t)(bq / a.n_q);
                const int32_t s = a.idx[row];
                if (s >= 0 && s < a.n_kv)
                    v[u] = *reinterpret_cast<const u32x4*>(
                        static_cast<const uint8_t*>(a.kv) + ((int64_t)b * a.n_kv + s) * a.row_bytes + piece * 16);
                dst[u] = row * a.row_bytes + piece * 16;
            }
        }
#pragma unroll
        for (int u = 0; u < kTasks; ++u)
            if (dst[u] >= 0)
                __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.out) + dst[u]));
    }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, int64_t n_rows, hipStream_t stream) {
    const int64_t n_pieces = n_rows * (a.row_bytes / 16);
    if (n_pieces <= 0) return hipSuccess;
    // enough workgroups to fill the chip several times over, each thread
    // then loops over its tasks
    const int64_t want = (n_pieces + kThreads * kTasks - 1) / (kThreads * kTasks);
    const unsigned grid = (unsigned)std::min<int64_t>(want, 256 * 32);
    hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(kThreads), 0, stream, a, n_pieces);
    return hipGetLastError();
}

}  // namespace tks

// fused.hip -- finish of the fused flat indexer top-k on gfx950.
//
// The fused scoring pass (score.hip) never writes a row's scores: every
// segment of kFusedSeg keys keeps at most r_cap candidates (those at or
// above a threshold T of its own) in the row's survivor pool.  This is the
// StreamIndex abstract's partition-merge that never materialises the score
// tensor, with the write-back of only the promising candidates from the
// threshold-based Indexer-TopK abstract listed on the same page.
//
// The finish selects the row's top-k from the pool (the counting top-k of
// the selection kernels) and proves it exact: a dropped candidate of
// segment g has a score key below T_g, so when the k-th best survivor's key
// is at least max_g T_g, every dropped candidate ranks below k survivors.
// With fewer than k survivors the result is exact only if nothing was
// dropped.  A row that fails the proof (clustered or heavily tied scores)
// is redone exactly: its keys are rescored tile by tile with the same MFMA
// sequence as the streaming kernels (so the same fp32 scores) into an arena
// slice, and each tile is merged into a running list by the exact selection
// of the tiled path.
#include "score_common.hpp"
#include "select_impl.hpp"

namespace tks {

namespace {

constexpr int kFinishMaxSeg = kFusedMaxPoolSeg;  // segments per row (4 per lane of one wave)
static_assert(kFusedPoolCap == kCap, "the pool of a row fits the selection's candidate list");

// Arena words per finish workgroup: a score tile and the running list
// (values, indices), rounded so every slice stays 256-byte aligned.
__host__ __device__ inline int64_t arena_stride(int32_t topk) {
    return ((int64_t)kFusedSeg + 2 * (int64_t)topk + 63) / 64 * 64;
}

// The row's q (heads padded to 64, rows padded by 16 bytes so the fragment
// reads spread over the banks) and head weights, staged in LDS.
constexpr int kQS = 128 + 8;
struct RescoreLds {
    uint16_t q[64 * kQS];
    float w[64];
};
static_assert(sizeof(RescoreLds) <= sizeof(uint64_t) * (kMaxK + kCap), "staging fits the selection LDS");

template <int NT>
__device__ void stage_row(const FusedFinishArgs& a, RescoreLds& R, int64_t qr) {
    constexpr int D = 128;
    const int hq = a.heads * D;
    const uint16_t* src = a.q + qr * hq;
    for (int e = threadIdx.x * 8; e < 64 * D; e += NT * 8) {
        u32x4 v = u32x4{0, 0, 0, 0};
        if (e < hq) v = *reinterpret_cast<const u32x4*>(src + e);
        *reinterpret_cast<u32x4*>(&R.q[(e / D) * kQS + e % D]) = v;
    }
    for (int h = threadIdx.x; h < 64; h += NT) R.w[h] = h < a.heads ? a.w[qr * a.heads + h] : 0.0f;
}

// Scores of keys [tb, tb + n) of one sequence into dst[0, n): each wave
// walks 32-key sub-blocks with the instruction sequence of the streaming
// kernels (D = 128, heads padded to 64), one fragment at a time, reading
// the q fragments and weights from LDS.
template <bool FP8, int NT>
__device__ void rescore_tile(const FusedFinishArgs& a, const RescoreLds& R, int64_t kseq,
                             int32_t tb, int32_t n, float* dst) {
    constexpr int D = 128, KS = 8, MB = 2, NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, m = lane & 31, hf = lane >> 5;
    for (int32_t j = wave * 32; j < n; j += NW * 32) {
        const bool valid = j + m < n;
        const int64_t row = kseq + (valid ? tb + j + m : 0);
        KeyFrag<D, FP8> f;
        load_key<D, FP8>(f, a.k, row, hf);
        const float scale = FP8 ? a.k_scale[row] : 1.0f;
        f32x16 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kb = key_operand<D, FP8>(f, ks);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const bf16x8 qa = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(&R.q[(mb * 32 + m) * kQS + hf * (D / 2) + ks * 8]));
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb, acc[mb], 0, 0, 0);
            }
        }
        float sc = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sc = fmaf(R.w[mb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3)], relu_bits(acc[mb][i]), sc);
        sc += __shfl_xor(sc, 32);
        if (FP8) sc *= scale;
        if (hf == 0 && valid) dst[j + m] = sc;
    }
}

// Exact top-k of row y by rescoring (the path that never fails).
template <bool FP8, int NT>
__device__ void redo_row(const FusedFinishArgs& a, SelectLds& L, float* arena, int64_t y,
                         int32_t n_vis) {
    const int32_t K = a.sel.topk;
    const int64_t qr = a.sel.rows.qrow(y);
    const int64_t kseq = (int64_t)a.sel.rows.seq(y) * a.k_seq_len;
    RescoreLds& R = *reinterpret_cast<RescoreLds*>(L.u);
    float* tile = arena;
    float* run_val = arena + kFusedSeg;
    int32_t* run_idx = reinterpret_cast<int32_t*>(arena + kFusedSeg + K);
    // the tiled exact selection of one row (chunk of one row at global row
    // y), the running list in the arena
    auto tile_args = [&](int32_t tb, int32_t te) {
        SelectArgs t = a.sel;
        t.scores = tile;
        t.score_stride = kFusedSeg;
        t.n_cols = te - tb;
        t.rows = RowMap{a.sel.rows.y0 + y, a.sel.rows.rows_per_seq, a.sel.rows.t_begin, a.sel.rows.n_q};
        t.col_key0 = tb;
        t.col_lo = 0;
        t.row_len = nullptr;
        t.blocks_mode = 0;
        t.prior_val = run_val;
        t.prior_idx = run_idx;
        t.run_val = run_val;
        t.run_idx = run_idx;
        t.tile_begin = tb;
        t.tile_end = te >= n_vis ? INT32_MAX : te;
        t.always_final = 0;
        t.blockselect = 0;
        return t;
    };
    for (int32_t tb = 0; tb < n_vis; tb += kFusedSeg) {
        const int32_t te = min(n_vis, tb + kFusedSeg);
        // (the selection of the previous tile is done with L)
        stage_row<NT>(a, R, qr);
        __syncthreads();
        rescore_tile<FP8, NT>(a, R, kseq, tb, te - tb, tile);
        __threadfence();
        __syncthreads();
        const SelectArgs s = tile_args(tb, te);
        RowCtx r;
        int32_t count;
        setup_row<NT>(s, r, L, 0, count);
        const bool final_out = count <= s.tile_end;
        bool sorted;
        const int32_t n_sel = select_core<true, NT>(s, r, L, K, sorted);
        __syncthreads();
        if (final_out && !sorted) sort_final<NT>(L, n_sel);
        write_row<NT>(s, r, L, n_sel, final_out);
        __threadfence();
        __syncthreads();
    }
}

template <int NT>
__global__ __launch_bounds__(NT) void fused_finish_kernel(FusedFinishArgs a) {
    __shared__ SelectLds L;
    __shared__ int32_t s_off[kFinishMaxSeg];
    __shared__ int32_t s_cnt[kFinishMaxSeg];
    __shared__ int32_t s_total;
    __shared__ uint32_t s_tau, s_kth;
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t K = a.sel.topk;
    const FusedPool& P = a.pool;
    for (int64_t y = blockIdx.x; y < a.n_rows; y += gridDim.x) {
        const int32_t n_vis = a.sel.vis.tokens(a.sel.rows.query(y));
        const int32_t n_seg = (n_vis + kFusedSeg - 1) / kFusedSeg * P.split;
        // survivor counts -> offsets, and the largest threshold (one wave)
        if (wave == 0) {
            constexpr int PER = kFinishMaxSeg / 64;
            int32_t c[PER];
            int32_t sum = 0;
            uint32_t tmax = 0u;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int g = lane * PER + i;
                c[i] = g < n_seg ? P.count[y * P.n_seg + g] : 0;
                tmax = max(tmax, g < n_seg ? P.tau[y * P.n_seg + g] : 0u);
                sum += c[i];
            }
            int32_t inc = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int32_t v = __shfl_up(inc, o);
                if (lane >= o) inc += v;
                tmax = max(tmax, (uint32_t)__shfl_xor((int)tmax, o));
            }
            int32_t run = inc - sum;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int g = lane * PER + i;
                if (g < n_seg) {
                    s_off[g] = run;
                    s_cnt[g] = c[i];
                }
                run += c[i];
            }
            if (lane == 63) s_total = inc;
            if (lane == 0) s_tau = tmax;
        }
        __syncthreads();
        const int32_t total = s_total;
        const uint32_t tau_max = s_tau;
        bool ok = total <= kCap;
        if (ok) {
            // the pool, compacted into the candidate list (a wave per
            // segment, four loads per lane issued before any is stored)
            for (int g = wave; g < n_seg; g += NW) {
                const uint64_t* src = P.cand + (y * P.n_seg + g) * (int64_t)P.r_cap;
                const int32_t o = s_off[g], c = s_cnt[g];
                for (int b = 0; b < c; b += 256) {
                    uint64_t v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = b + j * 64 + lane;
                        v[j] = i < c ? src[i] : 0ull;
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = b + j * 64 + lane;
                        if (i < c) L.u[kMaxK + o + i] = v[j];
                    }
                }
            }
        }
        __syncthreads();
        int32_t n_sel = 0;
        bool sorted = false;
        if (ok && total <= K) {
            ok = tau_max == 0u;  // fewer than k survivors: exact only if none was dropped
            if (ok) {
                for (int i = tid; i < total; i += NT) L.u[i] = L.u[kMaxK + i];
                n_sel = total;
            }
            __syncthreads();
        } else if (ok) {
            n_sel = pool_best<NT>(L, total, K, sorted);
            // the k-th best survivor's key: the smallest selected key
            uint32_t kmin = 0xFFFFFFFFu;
            for (int i = tid; i < K; i += NT) kmin = min(kmin, (uint32_t)(L.u[i] >> 32));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
            if (tid == 0) s_kth = 0xFFFFFFFFu;
            __syncthreads();
            if (lane == 0) atomicMin(&s_kth, kmin);
            __syncthreads();
            ok = s_kth >= tau_max;
        }
        if (ok) {
            if (!sorted) sort_final<NT>(L, n_sel);
            RowCtx r{};
            r.y = y;
            write_row<NT>(a.sel, r, L, n_sel, true);
        } else if (tid == 0) {
            a.failed[atomicAdd(a.n_failed, 1)] = (int32_t)y;  // redone by the repair kernel
        }
        __syncthreads();
    }
}

// The rows whose survivors could not prove the result, redone exactly
// (rescoring + tiled exact selection).  The failed-row counter is cleared
// by the fused scoring pass that precedes the finish.
template <bool FP8, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void fused_repair_kernel(
    FusedFinishArgs a) {
    __shared__ SelectLds L;
    const int32_t n = *a.n_failed;
    float* arena = a.arena + (int64_t)blockIdx.x * arena_stride(a.sel.topk);
    for (int32_t i = blockIdx.x; i < n; i += gridDim.x) {
        const int64_t y = a.failed[i];
        redo_row<FP8, NT>(a, L, arena, y, a.sel.vis.tokens(a.sel.rows.query(y)));
        __syncthreads();
    }
}

// Repair workgroups: a small persistent grid (rows that fail the proof are
// rare; a launch that finds none should cost little).
constexpr int32_t kFinishGridMax = 16;

}  // namespace

int32_t fused_finish_grid(int64_t n_rows) {
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>(n_rows, kFinishGridMax));
}

size_t fused_arena_bytes(int64_t n_rows, int32_t topk) {
    return (size_t)fused_finish_grid(n_rows) * (size_t)arena_stride(topk) * 4;
}

hipError_t launch_fused_finish(const FusedFinishArgs& a, bool fp8, hipStream_t stream) {
    if (a.n_rows <= 0) return hipSuccess;
    if (a.pool.n_seg > kFinishMaxSeg || a.pool.n_seg * (int64_t)a.pool.r_cap > kCap ||
        a.sel.topk > kMaxK)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)std::min<int64_t>(a.n_rows, 65535));
    // few rows: a wide workgroup per row (as the selection kernels do)
    if (a.n_rows < 512)
        hipLaunchKernelGGL((fused_finish_kernel<1024>), grid, dim3(1024), 0, stream, a);
    else
        hipLaunchKernelGGL((fused_finish_kernel<256>), grid, dim3(256), 0, stream, a);
    const dim3 rgrid((unsigned)fused_finish_grid(a.n_rows));
    if (fp8)
        hipLaunchKernelGGL((fused_repair_kernel<true, 256>), rgrid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((fused_repair_kernel<false, 256>), rgrid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tks

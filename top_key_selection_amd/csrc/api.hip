// api.hip -- the C ABI of include/tks.h: argument checks, workspace
// planning and the chunk x tile partition-merge driver (StreamIndex
// abstract: chunked partition-merge top-k that never materialises the full
// score tensor).  Every check runs before the first launch; no device
// memory is allocated here.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tks.h"

#include "tks_launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(TKS_EHIP, "%s: %s", where, hipGetErrorString(e));
}

// TKS_DEBUG_SYNC=1 in the environment: every launch is followed by a
// synchronisation of its stream (not while the stream is being captured into
// a graph), so a failure inside a kernel is reported by the call that made
// the launch instead of by some later HIP call.
bool debug_sync_on() {
    static const bool on = [] {
        const char* v = getenv("TKS_DEBUG_SYNC");
        return v != nullptr && v[0] == '1';
    }();
    return on;
}

hipError_t after_launch(hipError_t e, hipStream_t s) {
    if (e != hipSuccess || !debug_sync_on()) return e;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(s, &cs)) != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusNone) return hipSuccess;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    return hipGetLastError();
}

// ---------------------------------------------------------- instrumentation

struct TimedLaunch {
    std::string role;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<TimedLaunch> g_prof;

// Brackets one launch with events on its stream while profiling is enabled.
class Timed {
  public:
    Timed(const char* role, hipStream_t s) : s_(s) {
        std::lock_guard<std::mutex> g(g_prof_mu);
        if (!g_prof_on) return;
        on_ = hipEventCreate(&rec_.start) == hipSuccess && hipEventCreate(&rec_.stop) == hipSuccess &&
              hipEventRecord(rec_.start, s_) == hipSuccess;
        rec_.role = role;
    }
    ~Timed() {
        if (!on_) return;
        if (hipEventRecord(rec_.stop, s_) != hipSuccess) return;
        std::lock_guard<std::mutex> g(g_prof_mu);
        g_prof.push_back(rec_);
    }

  private:
    hipStream_t s_;
    bool on_ = false;
    TimedLaunch rec_;
};

void prof_clear() {
    for (auto& r : g_prof) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    g_prof.clear();
}

constexpr int kMaxTopk = 2048;
constexpr int kMaxBlkEntries = 512;
// Score-buffer budget used when a chunk / tile size is left to the library.
constexpr int64_t kScoreBudget = 256ll << 20;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int check_shape(const tks_shape* s, bool need_keys) {
    if (!s) return fail(TKS_EINVAL, "shape is NULL");
    if (s->batch < 0 || s->n_q < 0 || s->n_k < 0)
        return fail(TKS_EINVAL, "negative size (batch %d, n_q %d, n_k %d)", s->batch, s->n_q, s->n_k);
    if (s->heads < 1 || s->heads > 64)
        return fail(TKS_EUNSUPPORTED, "heads = %d (supported 1..64)", s->heads);
    if (s->dim != 32 && s->dim != 64 && s->dim != 128)
        return fail(TKS_EUNSUPPORTED, "dim = %d (supported 32, 64, 128)", s->dim);
    if (s->causal_ratio < 1) return fail(TKS_EINVAL, "causal_ratio = %d (must be >= 1)", s->causal_ratio);
    if (s->key_dtype != TKS_KEY_BF16 && s->key_dtype != TKS_KEY_FP8_E4M3FN)
        return fail(TKS_EINVAL, "key_dtype = %d", s->key_dtype);
    if ((int64_t)s->batch * s->n_q > INT32_MAX || (int64_t)s->batch * s->n_k > INT32_MAX)
        return fail(TKS_EUNSUPPORTED, "batch * n_q or batch * n_k exceeds 2^31 - 1");
    (void)need_keys;
    return TKS_OK;
}

int check_qwk(const tks_shape* s, const void* q, const float* w, const void* k,
              const float* k_scale) {
    const bool rows = (int64_t)s->batch * s->n_q > 0;
    const bool keys = (int64_t)s->batch * s->n_k > 0;
    if (rows && (!q || !w)) return fail(TKS_EINVAL, "q or w is NULL");
    if (keys && !k) return fail(TKS_EINVAL, "k is NULL");
    if (keys && s->key_dtype == TKS_KEY_FP8_E4M3FN && !k_scale)
        return fail(TKS_EINVAL, "fp8 keys need k_scale");
    if ((q && !aligned(q, 16)) || (k && !aligned(k, 16)))
        return fail(TKS_EINVAL, "q and k must be 16-byte aligned");
    if ((w && !aligned(w, 4)) || (k_scale && !aligned(k_scale, 4)))
        return fail(TKS_EINVAL, "w and k_scale must be 4-byte aligned");
    return TKS_OK;
}

tks::VisRule vis_tokens(const tks_shape* s) { return tks::VisRule{s->q_pos0, s->causal_ratio, s->n_k, 0}; }

// Largest visible-key count over queries t in [t0, t1] (count is monotone in t).
int32_t max_visible(const tks_shape* s, int64_t g0, int64_t g1) {
    // global rows g0..g1-1; if they span a sequence boundary the last query of
    // a sequence is included
    const int64_t t_last = (g0 / s->n_q != (g1 - 1) / s->n_q) ? s->n_q - 1 : (g1 - 1) % s->n_q;
    return vis_tokens(s).tokens((int32_t)t_last);
}

int block_shift_of(int32_t block) {
    switch (block) {
        case 32: return 5;
        case 64: return 6;
        case 128: return 7;
        case 256: return 8;
        default: return -1;
    }
}

// ------------------------------------------------------------- flat planning
//
// Two forms, neither of which holds the scores of every row and key:
//   * fused (one query per sequence, D = 128, chunk and tile left to the
//     library): segments of kFusedSeg keys are scored and filtered in one
//     pass; the workspace holds at most kFusedPoolCap survivors per row plus
//     the rescoring arena of the exact fallback;
//   * tiled: a [q_chunk, k_tile] fp32 score tile and the running top-k lists
//     of a chunk; the automatic sizes stay within kScoreBudget and never let
//     one tile cover every row and every visible key.

constexpr int32_t kFusedMaxSeg = 256;

struct FlatPlan {
    bool fused;
    int64_t rows;
    int32_t q_chunk;
    int32_t k_tile;
    int64_t score_stride;
    tks::SelectSplit split;  // few long rows over every CU (single tile only)
    size_t off_scores, off_run_val, off_run_idx, off_split;
    int32_t n_seg, r_cap;    // fused: key segments of kFusedSeg, survivors per pool segment
    int32_t pool_split;      // fused: pool segments per key segment
    size_t off_cand, off_count, off_tau, off_failed, off_arena;
    size_t bytes;
};

FlatPlan plan_flat(const tks_shape* s, int32_t topk, int32_t q_chunk, int32_t k_tile) {
    FlatPlan p{};
    p.rows = (int64_t)s->batch * s->n_q;
    const int32_t maxvis = p.rows > 0 ? max_visible(s, 0, p.rows) : 0;
    const int64_t n_seg = ((int64_t)maxvis + tks::kFusedSeg - 1) / tks::kFusedSeg;
    if (q_chunk == 0 && k_tile == 0 && s->n_q == 1 && s->dim == 128 && n_seg >= 1 &&
        n_seg <= kFusedMaxSeg) {
        p.fused = true;
        p.n_seg = (int32_t)n_seg;
        // fp8 keys: every wave of a scoring workgroup filters its own keys of
        // a segment (no workgroup barrier), while the finish can take the
        // segments
        p.pool_split = s->key_dtype == TKS_KEY_FP8_E4M3FN && n_seg * tks::kFusedWaves <= tks::kFusedMaxPoolSeg
                           ? tks::kFusedWaves : 1;
        const int64_t pseg = n_seg * p.pool_split;
        p.r_cap = std::min<int32_t>(tks::kFusedSeg / p.pool_split, tks::kFusedPoolCap / (int32_t)pseg);
        size_t off = 0;
        p.off_cand = off;
        off += round_up(p.rows * pseg * p.r_cap * 8, 256);
        p.off_count = off;
        off += round_up(p.rows * pseg * 4, 256);
        p.off_tau = off;
        off += round_up(p.rows * pseg * 4, 256);
        p.off_failed = off;  // failed-row list, then its counter
        off += round_up((p.rows + 1) * 4, 256);
        p.off_arena = off;
        off += round_up((int64_t)tks::fused_arena_bytes(p.rows, topk), 256);
        p.bytes = off;
        return p;
    }
    int64_t kt = k_tile > 0 ? k_tile : round_up(std::max<int32_t>(maxvis, 1), 32);
    int64_t qc;
    if (q_chunk > 0) {
        qc = q_chunk;
    } else {
        qc = std::max<int64_t>(1, kScoreBudget / (kt * 4));
        if (k_tile <= 0 && qc < std::min<int64_t>(p.rows, 1024)) {
            kt = 16384;
            qc = std::max<int64_t>(1, kScoreBudget / (kt * 4));
        }
        // one tile would hold every row's scores of every visible key:
        // split the rows into two chunks, so at most half of them are held
        // at once (a single row: two key tiles).  (Four chunks measured 7 %
        // slower at 8K prefill: the early chunks of the causal triangle are
        // too small to fill the GPU.)
        if (qc >= p.rows && kt >= maxvis) {
            if (p.rows > 1)
                qc = (p.rows + 1) / 2;
            else if (k_tile <= 0 && maxvis > 32)
                kt = round_up((maxvis + 1) / 2, 32);
        }
    }
    qc = std::max<int64_t>(1, std::min<int64_t>(qc, std::max<int64_t>(p.rows, 1)));
    p.q_chunk = (int32_t)qc;
    p.k_tile = (int32_t)kt;
    p.score_stride = round_up(kt, 4);
    const bool tiled = kt < maxvis;
    size_t off = 0;
    p.off_scores = off;
    off += round_up(qc * p.score_stride * 4, 256);
    p.off_run_val = off;
    if (tiled) off += round_up(qc * (int64_t)topk * 4, 256);
    p.off_run_idx = off;
    if (tiled) off += round_up(qc * (int64_t)topk * 4, 256);
    p.split = tiled ? tks::SelectSplit{0, 0}
                    : tks::select_split(qc, (int32_t)std::min<int64_t>(kt, maxvis), topk);
    p.off_split = off;
    off += tks::select_split_workspace(qc, p.split);
    p.bytes = off;
    return p;
}

}  // namespace

extern "C" {

int tks_version(void) { return 100; }

const char* tks_last_error(void) { return g_err; }

int tks_indexer_scores(const tks_shape* s, const void* q, const float* w, const void* k,
                       const float* k_scale, int32_t q_begin, int32_t q_count, int32_t k_begin,
                       int32_t k_count, float* scores, hipStream_t stream) {
    int rc = check_shape(s, true);
    if (rc) return rc;
    if (q_begin < 0 || q_count < 0 || k_begin < 0 || k_count < 0 ||
        (int64_t)q_begin + q_count > s->n_q || (int64_t)k_begin + k_count > s->n_k)
        return fail(TKS_EINVAL, "rectangle [%d,+%d) x [%d,+%d) outside n_q %d / n_k %d", q_begin,
                    q_count, k_begin, k_count, s->n_q, s->n_k);
    const int64_t n_rows = (int64_t)s->batch * q_count;
    if (n_rows == 0 || k_count == 0) return TKS_OK;
    if ((rc = check_qwk(s, q, w, k, k_scale))) return rc;
    if (!scores || !aligned(scores, 4)) return fail(TKS_EINVAL, "scores is NULL or misaligned");
    tks::ScoreArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.w = w;
    a.k = k;
    a.k_scale = k_scale;
    a.k_seq_len = s->n_k;
    a.heads = s->heads;
    a.rows = tks::RowMap{0, q_count, q_begin, s->n_q};
    a.vis = vis_tokens(s);
    a.col_key0 = k_begin;
    a.n_cols = k_count;
    a.out = scores;
    a.out_stride = k_count;
    a.write_masked = 1;
    hipError_t e;
    {
        Timed tm("score_flat", stream);
        e = tks::launch_score(a, n_rows, s->dim, s->key_dtype == TKS_KEY_FP8_E4M3FN, false,
                              stream);
    }
    if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "score launch");
    return TKS_OK;
}

size_t tks_topk_flat_workspace(const tks_shape* s, int32_t topk, int32_t q_chunk, int32_t k_tile) {
    if (check_shape(s, true) || topk < 1 || topk > kMaxTopk || q_chunk < 0 || k_tile < 0)
        return 0;
    return plan_flat(s, topk, q_chunk, k_tile).bytes;
}

}  // extern "C"

namespace {

// Argument checks of the flat top-k (shared by both entry points); sets
// *rows and *plan.  rows == 0 means nothing to do.
int flat_checks(const tks_shape* s, const void* q, const float* w, const void* k,
                const float* k_scale, int32_t topk, int32_t q_chunk, int32_t k_tile,
                const int32_t* idx, const float* vals, int64_t* rows, FlatPlan* plan) {
    int rc = check_shape(s, true);
    if (rc) return rc;
    if (topk < 1 || topk > kMaxTopk)
        return fail(TKS_EUNSUPPORTED, "topk = %d (supported 1..%d)", topk, kMaxTopk);
    if (q_chunk < 0 || k_tile < 0) return fail(TKS_EINVAL, "negative q_chunk or k_tile");
    if (k_tile > 0 && k_tile % 32 != 0)
        return fail(TKS_EINVAL, "k_tile = %d (must be a multiple of 32)", k_tile);
    *rows = (int64_t)s->batch * s->n_q;
    if (*rows == 0) return TKS_OK;
    if ((rc = check_qwk(s, q, w, k, k_scale))) return rc;
    if (!idx || !aligned(idx, 4) || (vals && !aligned(vals, 4)))
        return fail(TKS_EINVAL, "idx is NULL, or idx / vals misaligned");
    *plan = plan_flat(s, topk, q_chunk, k_tile);
    return TKS_OK;
}

int topk_flat_run(const tks_shape* s, const void* q, const float* w, const void* k,
                  const float* k_scale, int32_t topk, int32_t* idx, float* vals, const FlatPlan& p,
                  char* ws, hipStream_t stream);

}  // namespace

extern "C" {

int tks_topk_flat(const tks_shape* s, const void* q, const float* w, const void* k,
                  const float* k_scale, int32_t topk, int32_t q_chunk, int32_t k_tile,
                  int32_t* idx, float* vals, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
    int64_t rows = 0;
    FlatPlan p{};
    int rc = flat_checks(s, q, w, k, k_scale, topk, q_chunk, k_tile, idx, vals, &rows, &p);
    if (rc || rows == 0) return rc;
    if (!workspace || workspace_bytes < p.bytes)
        return fail(TKS_EWORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                    p.bytes);
    if (!aligned(workspace, 256)) return fail(TKS_EINVAL, "workspace must be 256-byte aligned");
    return topk_flat_run(s, q, w, k, k_scale, topk, idx, vals, p, static_cast<char*>(workspace),
                         stream);
}

}  // extern "C"

namespace {

int topk_flat_run(const tks_shape* s, const void* q, const float* w, const void* k,
                  const float* k_scale, int32_t topk, int32_t* idx, float* vals, const FlatPlan& p,
                  char* ws, hipStream_t stream) {
    const int64_t rows = p.rows;
    if (p.fused) {
        const bool fp8k = s->key_dtype == TKS_KEY_FP8_E4M3FN;
        const tks::FusedPool pool{reinterpret_cast<uint64_t*>(ws + p.off_cand),
                                  reinterpret_cast<int32_t*>(ws + p.off_count),
                                  reinterpret_cast<uint32_t*>(ws + p.off_tau), p.n_seg * p.pool_split,
                                  p.r_cap, p.pool_split};
        const tks::RowMap rm{0, s->n_q, 0, s->n_q};
        tks::ScoreArgs a{};
        a.q = static_cast<const uint16_t*>(q);
        a.w = w;
        a.k = k;
        a.k_scale = k_scale;
        a.k_seq_len = s->n_k;
        a.heads = s->heads;
        a.rows = rm;
        a.vis = vis_tokens(s);
        a.col_key0 = 0;
        a.n_cols = p.n_seg * tks::kFusedSeg;
        a.stream_keys = 1;
        a.fuse = pool;
        a.fuse_clear = reinterpret_cast<int32_t*>(ws + p.off_failed) + rows;
        hipError_t e;
        {
            Timed tm("score_flat", stream);
            e = tks::launch_score_fused(a, rows, p.n_seg, fp8k, stream);
        }
        if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "fused score launch");
        tks::FusedFinishArgs f{};
        f.pool = pool;
        f.sel.rows = rm;
        f.sel.vis = vis_tokens(s);
        f.sel.topk = topk;
        f.sel.out_val = vals;
        f.sel.out_idx = idx;
        f.sel.out_width = topk;
        f.sel.always_final = 1;
        f.q = static_cast<const uint16_t*>(q);
        f.w = w;
        f.k = k;
        f.k_scale = k_scale;
        f.k_seq_len = s->n_k;
        f.heads = s->heads;
        f.arena = reinterpret_cast<float*>(ws + p.off_arena);
        f.failed = reinterpret_cast<int32_t*>(ws + p.off_failed);
        f.n_failed = f.failed + rows;
        f.n_rows = rows;
        {
            Timed tm("select_flat", stream);
            e = tks::launch_fused_finish(f, fp8k, stream);
        }
        if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "fused finish launch");
        return TKS_OK;
    }
    float* sbuf = reinterpret_cast<float*>(ws + p.off_scores);
    float* run_val = reinterpret_cast<float*>(ws + p.off_run_val);
    int32_t* run_idx = reinterpret_cast<int32_t*>(ws + p.off_run_idx);
    const bool fp8 = s->key_dtype == TKS_KEY_FP8_E4M3FN;

    for (int64_t g0 = 0; g0 < rows; g0 += p.q_chunk) {
        const int64_t n = std::min<int64_t>(p.q_chunk, rows - g0);
        const int32_t maxvis = max_visible(s, g0, g0 + n);
        const int32_t n_tiles = std::max<int32_t>(1, (maxvis + p.k_tile - 1) / p.k_tile);
        const tks::RowMap rm{g0, s->n_q, 0, s->n_q};
        for (int32_t ti = 0; ti < n_tiles; ++ti) {
            const int32_t tb = ti * p.k_tile;
            const int32_t te = std::min<int32_t>(tb + p.k_tile, maxvis);
            tks::ScoreArgs a{};
            a.q = static_cast<const uint16_t*>(q);
            a.w = w;
            a.k = k;
            a.k_scale = k_scale;
            a.k_seq_len = s->n_k;
            a.heads = s->heads;
            a.rows = rm;
            a.vis = vis_tokens(s);
            a.col_key0 = tb;
            a.n_cols = std::max(0, te - tb);
            a.out = sbuf;
            a.out_stride = p.score_stride;
            a.stream_keys = s->n_q == 1;
            hipError_t e;
            {
                Timed tm("score_flat", stream);
                e = tks::launch_score(a, n, s->dim, fp8, false, stream);
            }
            if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "score launch");

            tks::SelectArgs sa{};
            sa.scores = sbuf;
            sa.score_stride = p.score_stride;
            sa.n_cols = a.n_cols;
            sa.rows = rm;
            sa.vis = vis_tokens(s);
            sa.col_key0 = tb;
            sa.col_lo = 0;
            sa.prior_val = n_tiles > 1 ? run_val : nullptr;
            sa.prior_idx = n_tiles > 1 ? run_idx : nullptr;
            sa.topk = topk;
            sa.run_val = run_val;
            sa.run_idx = run_idx;
            sa.out_val = vals;
            sa.out_idx = idx;
            sa.out_width = topk;
            sa.tile_begin = tb;
            sa.tile_end = ti + 1 == n_tiles ? INT32_MAX : te;
            {
                Timed tm("select_flat", stream);
                if (p.split.parts > 0 && n_tiles == 1)
                    e = tks::launch_select_split(sa, n, p.split, ws + p.off_split, stream);
                else
                    e = tks::launch_select(sa, n, stream);
            }
            if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "select launch");
        }
    }
    return TKS_OK;
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

// The allocation-free flat top-k keeps its workspace in this device array,
// one per GPU, held until the process ends.  In host code the name is only
// a stand-in: the array's device address comes from hipGetSymbolAddress,
// once per device, and only that address is ever passed on.
constexpr size_t kStaticScratchBytes = (size_t)TKS_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// device's first call, with that device current).
int static_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(TKS_EUNSUPPORTED, "device %d (supported 0..%d)", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr || !aligned(ptr, 256)) return fail(TKS_EHIP, "scratch array has no usable device address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return TKS_OK;
}

}  // namespace

extern "C" {

int tks_topk_flat_static(const tks_shape* s, const void* q, const float* w, const void* k,
                         const float* k_scale, int32_t topk, int32_t q_chunk, int32_t k_tile,
                         int32_t* idx, float* vals, hipStream_t stream) {
    int64_t rows = 0;
    FlatPlan p{};
    int rc = flat_checks(s, q, w, k, k_scale, topk, q_chunk, k_tile, idx, vals, &rows, &p);
    if (rc || rows == 0) return rc;
    if (p.bytes > kStaticScratchBytes)
        return fail(TKS_EWORKSPACE,
                    "the call needs %zu bytes of workspace; the static scratch holds %zu "
                    "(use tks_topk_flat with a caller workspace)",
                    p.bytes, kStaticScratchBytes);
    void* ws = nullptr;
    if ((rc = static_scratch(&ws))) return rc;
    return topk_flat_run(s, q, w, k, k_scale, topk, idx, vals, p, static_cast<char*>(ws), stream);
}

int tks_topk_flat_redone(const tks_shape* s, int32_t topk, int32_t q_chunk, int32_t k_tile,
                         const void* workspace, int32_t* n_redone, hipStream_t stream) {
    int rc = check_shape(s, true);
    if (rc) return rc;
    if (topk < 1 || topk > kMaxTopk || q_chunk < 0 || k_tile < 0 || !n_redone)
        return fail(TKS_EINVAL, "bad topk / q_chunk / k_tile, or n_redone is NULL");
    const FlatPlan p = plan_flat(s, topk, q_chunk, k_tile);
    *n_redone = 0;
    if (!p.fused) return TKS_OK;
    if (!workspace) return fail(TKS_EINVAL, "workspace is NULL");
    const char* cnt = static_cast<const char*>(workspace) + p.off_failed + p.rows * 4;
    hipError_t e = hipMemcpyAsync(n_redone, cnt, 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "reading the redone-row count");
    return TKS_OK;
}

size_t tks_topk_scores_workspace(int32_t n_rows, int32_t n_cols, int32_t topk) {
    if (n_rows < 0 || n_cols < 0 || topk < 1 || topk > kMaxTopk) return 0;
    return tks::select_split_workspace(n_rows, tks::select_split(n_rows, n_cols, topk));
}

int tks_topk_scores(const float* scores, int32_t n_rows, int32_t n_cols, int64_t row_stride,
                    const int32_t* row_len, int32_t topk, int32_t* idx, float* vals,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (n_rows < 0 || n_cols < 0) return fail(TKS_EINVAL, "negative n_rows / n_cols");
    if (topk < 1 || topk > kMaxTopk)
        return fail(TKS_EUNSUPPORTED, "topk = %d (supported 1..%d)", topk, kMaxTopk);
    if (n_rows == 0) return TKS_OK;
    if (row_stride < n_cols) return fail(TKS_EINVAL, "row_stride %lld < n_cols %d", (long long)row_stride, n_cols);
    if ((!scores && n_cols > 0) || !idx) return fail(TKS_EINVAL, "scores or idx is NULL");
    if ((scores && !aligned(scores, 4)) || !aligned(idx, 4) || (vals && !aligned(vals, 4)) ||
        (row_len && !aligned(row_len, 4)))
        return fail(TKS_EINVAL, "misaligned pointer");
    tks::SelectArgs sa{};
    sa.scores = scores;
    sa.score_stride = row_stride;
    sa.n_cols = n_cols;
    sa.rows = tks::RowMap{0, n_rows, 0, n_rows};
    sa.vis = tks::VisRule{INT32_MAX / 2, 1, n_cols, 0};  // every column visible
    sa.row_len = row_len;
    sa.topk = topk;
    sa.out_val = vals;
    sa.out_idx = idx;
    sa.out_width = topk;
    sa.always_final = 1;
    const tks::SelectSplit sp = tks::select_split(n_rows, n_cols, topk);
    const size_t need = tks::select_split_workspace(n_rows, sp);
    if (need && (!workspace || workspace_bytes < need))
        return fail(TKS_EWORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                    need);
    if (need && !aligned(workspace, 256)) return fail(TKS_EINVAL, "workspace must be 256-byte aligned");
    hipError_t e;
    {
        Timed tm("select_scores", stream);
        e = sp.parts > 0 ? tks::launch_select_split(sa, n_rows, sp, workspace, stream)
                         : tks::launch_select(sa, n_rows, stream);
    }
    if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "select launch");
    return TKS_OK;
}

int tks_hisa_pool_keys(const tks_shape* s, const void* k, const float* k_scale, int32_t block,
                       void* pooled, hipStream_t stream) {
    int rc = check_shape(s, true);
    if (rc) return rc;
    if (block_shift_of(block) < 0)
        return fail(TKS_EUNSUPPORTED, "block = %d (supported 32, 64, 128, 256)", block);
    const int64_t nb = s->n_k / block;
    if ((int64_t)s->batch * nb == 0) return TKS_OK;
    if (!k || !aligned(k, 16)) return fail(TKS_EINVAL, "k is NULL or not 16-byte aligned");
    if (s->key_dtype == TKS_KEY_FP8_E4M3FN && (!k_scale || !aligned(k_scale, 4)))
        return fail(TKS_EINVAL, "fp8 keys need a 4-byte aligned k_scale");
    if (!pooled || !aligned(pooled, 16)) return fail(TKS_EINVAL, "pooled is NULL or not 16-byte aligned");
    tks::PoolArgs a{k, k_scale, s->batch, s->n_k, s->dim, block, static_cast<uint16_t*>(pooled)};
    hipError_t e;
    {
        Timed tm("pool", stream);
        e = tks::launch_pool(a, s->key_dtype == TKS_KEY_FP8_E4M3FN, stream);
    }
    if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "pool launch");
    return TKS_OK;
}

int tks_kv_append(const tks_shape* s, const void* raw, int32_t n_new, int32_t raw_len,
                  void* raw_tail, void* k, float* k_scale, int32_t block, void* pooled,
                  hipStream_t stream) {
    int rc = check_shape(s, true);
    if (rc) return rc;
    if (raw_len < 0 || n_new < 0) return fail(TKS_EINVAL, "raw_len %d / n_new %d negative", raw_len, n_new);
    const int64_t m = s->causal_ratio;
    const int64_t total = (int64_t)raw_len + n_new;
    if (total / m > s->n_k)
        return fail(TKS_EINVAL, "append of %d raw keys after %d overflows the cache (%d keys at ratio %d)",
                    n_new, raw_len, s->n_k, s->causal_ratio);
    if (block != 0 && block_shift_of(block) < 0)
        return fail(TKS_EUNSUPPORTED, "block = %d (supported 0, 32, 64, 128, 256)", block);
    if (s->batch == 0 || n_new == 0) return TKS_OK;
    if (!raw || !aligned(raw, 16)) return fail(TKS_EINVAL, "raw is NULL or not 16-byte aligned");
    if (m > 1 && (!raw_tail || !aligned(raw_tail, 16)))
        return fail(TKS_EINVAL, "raw_tail is NULL or not 16-byte aligned (ratio %d)", s->causal_ratio);
    if (!k || !aligned(k, 16)) return fail(TKS_EINVAL, "k is NULL or not 16-byte aligned");
    if (s->key_dtype == TKS_KEY_FP8_E4M3FN && (!k_scale || !aligned(k_scale, 4)))
        return fail(TKS_EINVAL, "fp8 keys need a 4-byte aligned k_scale");
    if (block > 0 && (!pooled || !aligned(pooled, 16)))
        return fail(TKS_EINVAL, "pooled is NULL or not 16-byte aligned");
    tks::AppendArgs a{};
    a.raw = static_cast<const uint16_t*>(raw);
    a.tail = static_cast<uint16_t*>(raw_tail);
    a.k = k;
    a.k_scale = k_scale;
    a.pooled = block > 0 ? static_cast<uint16_t*>(pooled) : nullptr;
    a.batch = s->batch;
    a.n_k = s->n_k;
    a.n_new = n_new;
    a.m = (int32_t)m;
    a.raw_len = raw_len;
    a.g0 = (int32_t)(raw_len / m);
    a.g1 = (int32_t)(total / m);
    a.span = block > 0 ? block : 64;
    a.J0 = a.g0 / a.span;
    a.n_jobs = std::max<int32_t>(1, (a.g1 + a.span - 1) / a.span - a.J0);
    hipError_t e;
    {
        Timed tm("append", stream);
        e = tks::launch_append(a, s->dim, s->key_dtype == TKS_KEY_FP8_E4M3FN, stream);
    }
    if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "append launch");
    return TKS_OK;
}

namespace {

struct BlockPlan {
    int64_t rows;
    int32_t nb;
    int32_t chunk;
    int64_t stride;
    size_t bytes;
};

BlockPlan plan_blocks(const tks_shape* s, int32_t block) {
    BlockPlan p{};
    p.rows = (int64_t)s->batch * s->n_q;
    p.nb = s->n_k / block;
    p.stride = round_up(std::max<int32_t>(p.nb, 1), 4);
    p.chunk = (int32_t)std::max<int64_t>(1, std::min<int64_t>(std::max<int64_t>(p.rows, 1),
                                                               kScoreBudget / (p.stride * 4)));
    p.bytes = round_up((int64_t)p.chunk * p.stride * 4, 256);
    return p;
}

int popcount2(uint32_t f) { return (int)((f & 1u) + ((f >> 1) & 1u)); }

}  // namespace

size_t tks_hisa_block_select_workspace(const tks_shape* s, int32_t block, int32_t m_scored) {
    if (check_shape(s, true) || block_shift_of(block) < 0 || m_scored < 0) return 0;
    return plan_blocks(s, block).bytes;
}

int tks_hisa_block_select(const tks_shape* s, const void* q, const float* w, const void* pooled,
                          int32_t block, int32_t m_scored, uint32_t force_flags, int32_t* blk,
                          float* blk_vals, int32_t m_total, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    int rc = check_shape(s, true);
    if (rc) return rc;
    if (block_shift_of(block) < 0)
        return fail(TKS_EUNSUPPORTED, "block = %d (supported 32, 64, 128, 256)", block);
    if (force_flags & ~3u) return fail(TKS_EINVAL, "force_flags = %u", force_flags);
    if (m_scored < 0 || m_scored > kMaxTopk)
        return fail(TKS_EUNSUPPORTED, "m_scored = %d (supported 0..%d)", m_scored, kMaxTopk);
    if (m_total != m_scored + popcount2(force_flags))
        return fail(TKS_EINVAL, "m_total = %d, expected m_scored + forced = %d", m_total,
                    m_scored + popcount2(force_flags));
    if (m_total < 1 || m_total > kMaxBlkEntries)
        return fail(TKS_EUNSUPPORTED, "m_total = %d (supported 1..%d)", m_total, kMaxBlkEntries);
    const BlockPlan p = plan_blocks(s, block);
    if (p.rows == 0) return TKS_OK;
    if (!q || !w || !aligned(q, 16) || !aligned(w, 4))
        return fail(TKS_EINVAL, "q / w NULL or misaligned");
    if (p.nb > 0 && (!pooled || !aligned(pooled, 16)))
        return fail(TKS_EINVAL, "pooled is NULL or not 16-byte aligned");
    if (!blk || !aligned(blk, 4) || (blk_vals && !aligned(blk_vals, 4)))
        return fail(TKS_EINVAL, "blk is NULL, or blk / blk_vals misaligned");
    if (!workspace || workspace_bytes < p.bytes)
        return fail(TKS_EWORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                    p.bytes);
    if (!aligned(workspace, 256)) return fail(TKS_EINVAL, "workspace must be 256-byte aligned");

    float* sbuf = static_cast<float*>(workspace);
    const tks::VisRule vb{s->q_pos0, s->causal_ratio, s->n_k, block};
    for (int64_t g0 = 0; g0 < p.rows; g0 += p.chunk) {
        const int64_t n = std::min<int64_t>(p.chunk, p.rows - g0);
        const tks::RowMap rm{g0, s->n_q, 0, s->n_q};
        tks::ScoreArgs a{};
        a.q = static_cast<const uint16_t*>(q);
        a.w = w;
        a.k = pooled;
        a.k_scale = nullptr;
        a.k_seq_len = p.nb;
        a.heads = s->heads;
        a.rows = rm;
        a.vis = vb;
        a.col_key0 = 0;
        a.n_cols = p.nb;
        a.out = sbuf;
        a.out_stride = p.stride;
        hipError_t e;
        {
            Timed tm("score_pooled", stream);
            e = tks::launch_score(a, n, s->dim, false, false, stream);
        }
        if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "block score launch");

        tks::SelectArgs sa{};
        sa.scores = sbuf;
        sa.score_stride = p.stride;
        sa.n_cols = p.nb;
        sa.rows = rm;
        sa.vis = vb;
        sa.col_key0 = 0;
        sa.col_lo = (force_flags & TKS_FORCE_FIRST) ? 1 : 0;
        sa.topk = m_scored;
        sa.out_val = blk_vals;
        sa.out_idx = blk;
        sa.out_width = m_total;
        sa.always_final = 1;
        sa.blockselect = 1;
        sa.force_flags = force_flags;
        sa.sel_block = block;
        {
            Timed tm("select_pooled", stream);
            e = tks::launch_select(sa, n, stream);
        }
        if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "block select launch");
    }
    return TKS_OK;
}

namespace {

// the refinement plans of every group are made in one launch when their
// arrays take at most this many bytes (else chunk by chunk)
constexpr int64_t kPlanAllBytes = (int64_t)64 << 20;

struct RefinePlan {
    int64_t rows;
    int32_t slots;
    int32_t chunk;
    int64_t stride;
    bool shared;        // prefill rows, bf16 keys, dim 128: the shared-key ring
    bool sched;         // ... with a plan per group of rows (bounded sizes)
    bool plan_all;      // one plan launch for every group of the call
    int32_t sched_stride;
    int32_t sched_blocks;
    int64_t groups;     // plan slots: every group, or a chunk's groups at most
    size_t off_n, off_blk, off_rank;  // plan arrays in the workspace
    size_t bytes;
};

RefinePlan plan_refine(const tks_shape* s, int32_t block, int32_t m_total, int32_t q_chunk) {
    RefinePlan p{};
    p.rows = (int64_t)s->batch * s->n_q;
    p.slots = block * m_total;
    p.stride = round_up(p.slots, 4);
    p.shared = s->key_dtype == TKS_KEY_BF16 && s->dim == 128 && s->n_q > 1;
    int64_t c = q_chunk > 0 ? q_chunk : kScoreBudget / (p.stride * 4);
    p.chunk = (int32_t)std::max<int64_t>(1, std::min<int64_t>(c, std::max<int64_t>(p.rows, 1)));
    p.bytes = round_up((int64_t)p.chunk * p.stride * 4, 256);
    // the plan of a group holds its union of kept blocks: at most every
    // block of the cache, and at most every list entry of its rows
    const int64_t nb_all = ((int64_t)s->n_k + block - 1) / block;
    const int64_t pu = std::min<int64_t>(nb_all, (int64_t)tks::kSchedRows * m_total);
    p.sched = p.shared && nb_all >= 1 && nb_all <= tks::kSchedMaxBlocks && pu <= tks::kSchedMaxPos;
    if (p.sched) {
        p.sched_stride = (int32_t)round_up(pu, 4);
        p.sched_blocks = (int32_t)nb_all;
        // groups of kSchedRows queries of a sequence; a chunk of c rows
        // touches at most c / kSchedRows + 1 of them per sequence it starts
        // or ends in, and enters at most c / n_q + 2 sequences
        const int64_t all = (int64_t)s->batch * ((s->n_q + tks::kSchedRows - 1) / tks::kSchedRows);
        const int64_t per_chunk = std::min<int64_t>(
            all, (p.chunk + tks::kSchedRows - 1) / tks::kSchedRows + (p.chunk + s->n_q - 1) / s->n_q + 3);
        p.plan_all = all * p.sched_stride * (4 + 2 * tks::kSchedRows) <= kPlanAllBytes;
        p.groups = p.plan_all ? all : per_chunk;
        p.off_n = p.bytes;
        p.off_blk = p.off_n + round_up(p.groups * 4, 256);
        p.off_rank = p.off_blk + round_up(p.groups * p.sched_stride * 4, 256);
        p.bytes = p.off_rank + round_up(p.groups * p.sched_stride * tks::kSchedRows * 2, 256);
    }
    return p;
}

}  // namespace

size_t tks_hisa_refine_workspace(const tks_shape* s, int32_t block, int32_t m_total, int32_t topk,
                                 int32_t q_chunk) {
    if (check_shape(s, true) || block_shift_of(block) < 0 || m_total < 1 ||
        m_total > kMaxBlkEntries || topk < 1 || topk > kMaxTopk || q_chunk < 0)
        return 0;
    return plan_refine(s, block, m_total, q_chunk).bytes;
}

int tks_hisa_refine_topk(const tks_shape* s, const void* q, const float* w, const void* k,
                         const float* k_scale, int32_t block, const int32_t* blk,
                         int32_t m_total, int32_t topk, int32_t q_chunk, int32_t* idx,
                         float* vals, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    int rc = check_shape(s, true);
    if (rc) return rc;
    const int bs = block_shift_of(block);
    if (bs < 0) return fail(TKS_EUNSUPPORTED, "block = %d (supported 32, 64, 128, 256)", block);
    if (m_total < 1 || m_total > kMaxBlkEntries)
        return fail(TKS_EUNSUPPORTED, "m_total = %d (supported 1..%d)", m_total, kMaxBlkEntries);
    if (topk < 1 || topk > kMaxTopk)
        return fail(TKS_EUNSUPPORTED, "topk = %d (supported 1..%d)", topk, kMaxTopk);
    if (q_chunk < 0) return fail(TKS_EINVAL, "negative q_chunk");
    const RefinePlan p = plan_refine(s, block, m_total, q_chunk);
    if (p.rows == 0) return TKS_OK;
    if ((rc = check_qwk(s, q, w, k, k_scale))) return rc;
    if (!blk || !aligned(blk, 4)) return fail(TKS_EINVAL, "blk is NULL or misaligned");
    if (!idx || !aligned(idx, 4) || (vals && !aligned(vals, 4)))
        return fail(TKS_EINVAL, "idx is NULL, or idx / vals misaligned");
    if (!workspace || workspace_bytes < p.bytes)
        return fail(TKS_EWORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0,
                    p.bytes);
    if (!aligned(workspace, 256)) return fail(TKS_EINVAL, "workspace must be 256-byte aligned");

    float* sbuf = static_cast<float*>(workspace);
    const bool fp8 = s->key_dtype == TKS_KEY_FP8_E4M3FN;
    for (int64_t g0 = 0; g0 < p.rows; g0 += p.chunk) {
        const int64_t n = std::min<int64_t>(p.chunk, p.rows - g0);
        const tks::RowMap rm{g0, s->n_q, 0, s->n_q};
        tks::ScoreArgs a{};
        a.q = static_cast<const uint16_t*>(q);
        a.w = w;
        a.k = k;
        a.k_scale = k_scale;
        a.k_seq_len = s->n_k;
        a.heads = s->heads;
        a.rows = rm;
        a.vis = vis_tokens(s);
        a.n_cols = p.slots;
        a.blk = blk;
        a.blk_stride = m_total;
        a.block_shift = bs;
        a.out = sbuf;
        a.out_stride = p.stride;
        a.stream_keys = s->n_q == 1;
        hipError_t e;
        {
            Timed tm("score_refine", stream);
            if (p.sched) {
                uint8_t* base = static_cast<uint8_t*>(workspace);
                a.sched.n_pos = reinterpret_cast<int32_t*>(base + p.off_n);
                a.sched.blocks = reinterpret_cast<int32_t*>(base + p.off_blk);
                a.sched.ranks = reinterpret_cast<int16_t*>(base + p.off_rank);
                a.sched.stride = p.sched_stride;
                a.sched.max_blocks = p.sched_blocks;
                int64_t g_lo, g_hi;
                tks::refine_sched_groups(rm, n, g_lo, g_hi);
                // the plans: every group with the first chunk, or this chunk's
                e = hipSuccess;
                if (p.plan_all) {
                    a.sched.group0 = 0;
                    if (g0 == 0) e = tks::launch_refine_plan(a, 0, p.groups, stream);
                } else {
                    a.sched.group0 = g_lo;
                    e = g_hi - g_lo > p.groups ? hipErrorInvalidValue
                                               : tks::launch_refine_plan(a, g_lo, g_hi, stream);
                }
                if (e == hipSuccess) e = tks::launch_score_refine_sched(a, n, stream);
            } else if (p.shared) {
                // keys of the run: up to the last visible key of the chunk
                a.n_cols = max_visible(s, g0, g0 + n);
                a.col_key0 = 0;
                e = tks::launch_score_refine_shared(a, n, stream);
            } else {
                e = tks::launch_score(a, n, s->dim, fp8, true, stream);
            }
        }
        if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "refine score launch");

        tks::SelectArgs sa{};
        sa.scores = sbuf;
        sa.score_stride = p.stride;
        sa.n_cols = p.slots;
        sa.rows = rm;
        sa.vis = vis_tokens(s);
        sa.blk = blk;
        sa.blk_stride = m_total;
        sa.block_shift = bs;
        sa.blocks_mode = 1;
        sa.topk = topk;
        sa.out_val = vals;
        sa.out_idx = idx;
        sa.out_width = topk;
        sa.always_final = 1;
        {
            Timed tm("select_refine", stream);
            e = tks::launch_select(sa, n, stream);
        }
        if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "refine select launch");
    }
    return TKS_OK;
}

int tks_gather_selected(const void* kv, int32_t batch, int32_t n_kv, int32_t row_bytes,
                        const int32_t* idx, int32_t n_q, int32_t topk, void* out,
                        hipStream_t stream) {
    if (batch < 0 || n_kv < 0 || n_q < 0 || topk < 0)
        return fail(TKS_EINVAL, "negative size (batch %d, n_kv %d, n_q %d, topk %d)", batch, n_kv, n_q, topk);
    if (row_bytes <= 0 || row_bytes % 16 != 0 || row_bytes > 65536)
        return fail(TKS_EUNSUPPORTED, "row_bytes = %d (a multiple of 16, 16..65536)", row_bytes);
    const int64_t rows = (int64_t)batch * n_q * topk;
    if (rows == 0) return TKS_OK;
    if ((int64_t)batch * n_q > INT32_MAX || rows * (row_bytes / 16) > ((int64_t)1 << 40))
        return fail(TKS_EUNSUPPORTED, "output too large");
    if (!idx || !aligned(idx, 4)) return fail(TKS_EINVAL, "idx is NULL or misaligned");
    if (!out || !aligned(out, 16)) return fail(TKS_EINVAL, "out is NULL or not 16-byte aligned");
    if (n_kv > 0 && (!kv || !aligned(kv, 16))) return fail(TKS_EINVAL, "kv is NULL or not 16-byte aligned");
    tks::GatherArgs a{kv, idx, out, n_kv, n_q, topk, row_bytes};
    hipError_t e;
    {
        Timed tm("gather", stream);
        e = tks::launch_gather(a, rows, stream);
    }
    if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "gather launch");
    return TKS_OK;
}

size_t tks_sparse_attention_workspace(int32_t batch, int32_t n_q, int32_t heads, int32_t topk) {
    if (batch < 0 || n_q < 0 || heads < 16 || heads > 128 || heads % 16 || topk < 1 || topk > kMaxTopk)
        return 0;
    return tks::attend_workspace((int64_t)batch * n_q, heads, topk);
}

int tks_sparse_attention(const void* q, const void* k, const void* v, int32_t batch, int32_t n_q,
                         int32_t heads, int32_t dim, int32_t n_kv, const int32_t* idx,
                         int32_t topk, float scale, float* out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    if (batch < 0 || n_q < 0 || n_kv < 0)
        return fail(TKS_EINVAL, "negative size (batch %d, n_q %d, n_kv %d)", batch, n_q, n_kv);
    if (heads < 16 || heads > 128 || heads % 16)
        return fail(TKS_EUNSUPPORTED, "heads = %d (a multiple of 16, 16..128)", heads);
    if (dim != 128) return fail(TKS_EUNSUPPORTED, "dim = %d (supported 128)", dim);
    if (topk < 1 || topk > kMaxTopk) return fail(TKS_EUNSUPPORTED, "topk = %d (supported 1..%d)", topk, kMaxTopk);
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return fail(TKS_EINVAL, "scale is not finite");
    const int64_t rows = (int64_t)batch * n_q;
    if (rows == 0) return TKS_OK;
    if (rows > INT32_MAX / heads) return fail(TKS_EUNSUPPORTED, "batch * n_q * heads exceeds 2^31 - 1");
    if (!q || !aligned(q, 16)) return fail(TKS_EINVAL, "q is NULL or not 16-byte aligned");
    if (n_kv > 0 && (!k || !v || !aligned(k, 16) || !aligned(v, 16)))
        return fail(TKS_EINVAL, "k / v NULL or not 16-byte aligned");
    if (!idx || !aligned(idx, 4)) return fail(TKS_EINVAL, "idx is NULL or misaligned");
    if (!out || !aligned(out, 4)) return fail(TKS_EINVAL, "out is NULL or misaligned");
    const size_t need = tks::attend_workspace(rows, heads, topk);
    if (!workspace || workspace_bytes < need)
        return fail(TKS_EWORKSPACE, "workspace %zu bytes, need %zu", workspace ? workspace_bytes : 0, need);
    if (!aligned(workspace, 256)) return fail(TKS_EINVAL, "workspace must be 256-byte aligned");
    tks::AttnArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.idx = idx;
    a.n_split = tks::attend_splits(topk);
    const int64_t part = rows * a.n_split * heads;
    a.o_part = static_cast<float*>(workspace);
    a.ml_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up(part * 128 * 4, 256));
    a.out = out;
    a.n_q = n_q;
    a.heads = heads;
    a.n_kv = n_kv;
    a.topk = topk;
    a.scale = scale;
    hipError_t e;
    {
        Timed tm("attend", stream);
        e = tks::launch_attend(a, rows, stream);
    }
    if ((e = after_launch(e, stream)) != hipSuccess) return hip_fail(e, "attention launch");
    return TKS_OK;
}

int tks_profile_enable(int on) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (on) prof_clear();
    g_prof_on = on != 0;
    return TKS_OK;
}

int tks_profile_read(const char* role, double* total_ms, int64_t* launches) {
    static const char* kRoles[] = {"score_flat",   "score_pooled",  "score_refine", "select_flat",
                                   "select_pooled", "select_refine", "select_scores", "pool",
                                   "append",       "gather",        "attend"};
    if (!role || !total_ms || !launches) return fail(TKS_EINVAL, "NULL argument");
    bool known = false;
    for (const char* r : kRoles) known = known || strcmp(r, role) == 0;
    if (!known) return fail(TKS_EINVAL, "unknown kernel role '%s'", role);
    std::lock_guard<std::mutex> g(g_prof_mu);
    double sum = 0.0;
    int64_t n = 0;
    for (auto& r : g_prof) {
        if (r.role != role) continue;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_fail(e, "profile event");
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) return hip_fail(e, "profile event");
        sum += ms;
        ++n;
    }
    *total_ms = sum;
    *launches = n;
    return TKS_OK;
}

}  // extern "C"

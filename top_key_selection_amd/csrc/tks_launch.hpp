// tks_launch.hpp -- kernel parameter blocks and host-side launchers of the
// gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tks_device.hpp"

namespace tks {

// Fused flat scoring (score.hip): a workgroup scores one segment of
// kFusedSeg consecutive keys of a row, keeps its best candidates (at most
// r_cap: every candidate whose score key is at least a threshold T of its
// own) and writes them, with T, to the row's survivor pool.  Every dropped
// candidate of the segment has a score key below T (T = 0: none dropped).
// With split = kFusedWaves (fp8 keys) every wave of the workgroup does this
// for the keys it scored, as a pool segment of its own, so the waves never
// wait for each other.
// The finish (fused.hip) selects the row's top-k from the pool; the result
// is exact when its k-th best survivor's key is at least every segment's T.
constexpr int kFusedSeg = 4096;
constexpr int kFusedPoolCap = 4096;  // survivors of one row, all segments together
constexpr int kFusedMaxPoolSeg = 256;  // pool segments of one row the finish takes
constexpr int kFusedWaves = 4;       // waves of an fp8 scoring workgroup
struct FusedPool {
    uint64_t* cand;    // [rows, n_seg, r_cap] composites (score key << 32 | ~index)
    int32_t* count;    // [rows, n_seg]
    uint32_t* tau;     // [rows, n_seg]
    int32_t n_seg;     // segments per row in the pool's layout
    int32_t r_cap;     // survivors per segment at most
    int32_t split;     // pool segments per kFusedSeg keys: 1, or one per wave
                       // of the scoring workgroup (each filtered on its own)
};

// Refinement schedule (score.hip): for each group of kSchedRows consecutive
// queries of one sequence (group g of the call: sequence g / G, queries
// kSchedRows * (g % G) on, G = ceil(n_q / kSchedRows)), the blocks any of
// them kept, in the order the scheduled refinement copies them, with each
// row's position of the block in its own list (-1: not kept).  Plan slot
// g - group0 holds group g.
constexpr int kSchedRows = 8;
constexpr int kSchedMaxPos = 1024;     // blocks of a group's union at most
constexpr int kSchedMaxBlocks = 8192;  // visible blocks of a row at most
struct RefineSched {
    int32_t* n_pos;      // [slots]
    int32_t* blocks;     // [slots, stride]
    int16_t* ranks;      // [slots, stride, kSchedRows]
    int32_t stride;      // positions per group in the layout: a multiple of 4, <= kSchedMaxPos
    int32_t max_blocks;  // visible blocks of any row at most, <= kSchedMaxBlocks
    int64_t group0;      // group of plan slot 0
};

// Scoring of one row chunk against a run of key slots (score.hip).
//   contiguous mode: slot j is key col_key0 + j of the row's sequence;
//   block mode:      slot j is key blk[row][j / B] * B + j % B.
// A slot is valid when its key is visible (VisRule) and, in block mode,
// its block entry is not -1.  Only valid slots are written, unless
// write_masked is set (then masked slots get -inf).
struct ScoreArgs {
    const uint16_t* q;      // bf16 bits [*, n_q, heads, dim]
    const float* w;         // [*, n_q, heads]
    const void* k;          // bf16 bits or e4m3fn codes [batch, k_seq_len, dim]
    const float* k_scale;   // [batch, k_seq_len] (fp8 keys) or null
    int64_t k_seq_len;      // keys per sequence in `k`
    int32_t heads;
    RowMap rows;
    VisRule vis;
    int32_t col_key0;
    int32_t n_cols;
    const int32_t* blk;     // block mode: kept blocks of global row g at blk + g * blk_stride
    int32_t blk_stride;
    int32_t block_shift;
    float* out;             // chunk-relative rows
    int64_t out_stride;
    int32_t write_masked;
    int32_t stream_keys;    // each key row is read by one query row only (decode)
    FusedPool fuse;         // fused mode (fuse.cand != null): survivors instead of `out`
    int32_t* fuse_clear;    // fused mode: a counter the first workgroup sets to 0
    RefineSched sched;      // scheduled refinement: the plan (written, then read)
};

// Exact top-k of row candidates (select.hip).  Candidates of a row are the
// optional prior list (running top-k of earlier key tiles) followed by the
// valid slots of its score-buffer row, in key-index order.
struct SelectArgs {
    const float* scores;
    int64_t score_stride;
    int32_t n_cols;
    RowMap rows;
    VisRule vis;
    int32_t col_key0;     // contiguous mode: key of column 0
    int32_t col_lo;       // contiguous mode: first eligible column
    const int32_t* row_len;  // explicit valid length per chunk row (overrides vis)
    const int32_t* blk;   // block mode (as in ScoreArgs)
    int32_t blk_stride;
    int32_t block_shift;
    int32_t blocks_mode;
    const float* prior_val;   // chunk-relative [n_rows, topk] or null
    const int32_t* prior_idx;
    int32_t topk;
    float* run_val;           // chunk-relative [n_rows, topk]
    int32_t* run_idx;
    float* out_val;           // global rows [*, out_width] (may be null)
    int32_t* out_idx;
    int32_t out_width;        // topk, or m_total in block-select output mode
    int32_t tile_begin;       // key range [tile_begin, tile_end) of this pass
    int32_t tile_end;
    int32_t always_final;
    // block-select output mode: kept blocks ascending with forced blocks
    int32_t blockselect;
    uint32_t force_flags;
    int32_t sel_block;        // block size (local block = (tokens - 1) / sel_block)
};

struct PoolArgs {
    const void* k;
    const float* k_scale;
    int32_t batch, n_k, dim, block;
    uint16_t* out;
};

// Key-cache append (append.hip): compressed keys g0 .. g1-1 of every
// sequence are completed by this call; jobs are the blocks J0 .. J0+n_jobs-1
// of `span` compressed keys (the pooled block size, or a job size when
// pooled is null).
struct AppendArgs {
    const uint16_t* raw;  // bf16 [batch, n_new, D]
    uint16_t* tail;       // bf16 [batch, m, D] staging (m > 1)
    void* k;              // [batch, n_k, D] bf16 or e4m3fn codes
    float* k_scale;       // [batch, n_k] (fp8)
    uint16_t* pooled;     // bf16 [batch, n_k / span, D] or null
    int32_t batch, n_k, n_new, m;
    int32_t raw_len;
    int32_t g0, g1;
    int32_t span;
    int32_t J0, n_jobs;
};

// Re-layout of selected rows (gather.hip): see tks_gather_selected.
struct GatherArgs {
    const void* kv;       // [batch, n_kv, row_bytes]
    const int32_t* idx;   // [batch, n_q, topk]
    void* out;            // [batch, n_q, topk, row_bytes]
    int32_t n_kv, n_q, topk, row_bytes;
};

// Sparse attention over selected keys (attend.hip): see tks_sparse_attention.
struct AttnArgs {
    const uint16_t* q;    // bf16 [rows, heads, 128]
    const uint16_t* k;    // bf16 [batch, n_kv, 128]
    const uint16_t* v;    // bf16 [batch, n_kv, 128]
    const int32_t* idx;   // [rows, topk]
    float* o_part;        // [rows, n_split, heads, 128]
    float* ml_part;       // [rows, n_split, heads, 2]
    float* out;           // [rows, heads, 128]
    int32_t n_q, heads, n_kv, topk, n_split;
    float scale;
};

hipError_t launch_score(const ScoreArgs& a, int64_t n_rows, int dim, bool fp8, bool blocks,
                        hipStream_t stream);
// Fused flat scoring of every row's segments (D = 128; heads padded to 64).
hipError_t launch_score_fused(const ScoreArgs& a, int64_t n_rows, int32_t n_seg, bool fp8,
                              hipStream_t stream);

// Finish of the fused flat path (fused.hip): one workgroup per row selects
// the row's top-k from its survivor pool and checks exactness; a row that
// fails the check is listed, and a repair kernel redoes it exactly: its
// keys are rescored tile by tile (kFusedSeg keys, the same MFMA order, so
// the same scores) into an arena slice and merged by the exact selection
// with a running list.
struct FusedFinishArgs {
    FusedPool pool;
    SelectArgs sel;        // rows, vis, topk, out_idx / out_val
    const uint16_t* q;     // (rescoring)
    const float* w;
    const void* k;
    const float* k_scale;
    int64_t k_seq_len;
    int32_t heads;
    float* arena;          // [repair grid, kFusedSeg + 2 * topk] words
    int32_t* failed;       // [n_rows] rows the finish could not prove
    int32_t* n_failed;     // cleared by the fused scoring pass
    int64_t n_rows;
};
int32_t fused_finish_grid(int64_t n_rows);
size_t fused_arena_bytes(int64_t n_rows, int32_t topk);
hipError_t launch_fused_finish(const FusedFinishArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_select(const SelectArgs& a, int64_t n_rows, hipStream_t stream);
// Selection plan for few long rows (parts = 0: one workgroup per row).
// parts > 0: a sampled threshold per row, a filter over parts x span column
// partitions into a per-row pool, and an exact finish per row.
struct SelectSplit {
    int32_t parts, span;
};
SelectSplit select_split(int64_t n_rows, int32_t n_cols, int32_t topk);
size_t select_split_workspace(int64_t n_rows, const SelectSplit& sp);
// Launch the three kernels; `ws` holds select_split_workspace bytes.
hipError_t launch_select_split(const SelectArgs& a, int64_t n_rows, const SelectSplit& sp,
                               void* ws, hipStream_t stream);
hipError_t launch_pool(const PoolArgs& a, bool fp8, hipStream_t stream);
// HISA refinement scoring of prefill rows (bf16 keys, D = 128; keys shared
// by position through the shared-key ring; a.n_cols = keys of the run,
// a.blk / a.blk_stride = block lists, a.out = [rows, blk_stride << shift])
hipError_t launch_score_refine_shared(const ScoreArgs& a, int64_t n_rows, hipStream_t stream);
// Scheduled refinement (bf16 keys, D = 128): the groups [g_lo, g_hi) that
// chunk rows [0, n_rows) touch; the plan of groups [g_lo, g_hi) (a.sched
// written, a.rows only for n_q); and the refinement of the chunk rows, each
// group's union of kept blocks scored in plan order through the shared-key
// ring (a.out as above; rows of a group outside the chunk are left out).
void refine_sched_groups(const RowMap& rows, int64_t n_rows, int64_t& g_lo, int64_t& g_hi);
hipError_t launch_refine_plan(const ScoreArgs& a, int64_t g_lo, int64_t g_hi, hipStream_t stream);
hipError_t launch_score_refine_sched(const ScoreArgs& a, int64_t n_rows, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, int dim, bool fp8, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, int64_t n_rows, hipStream_t stream);
size_t attend_workspace(int64_t rows, int32_t heads, int32_t topk);
int32_t attend_splits(int32_t topk);
hipError_t launch_attend(const AttnArgs& a, int64_t rows, hipStream_t stream);

}  // namespace tks

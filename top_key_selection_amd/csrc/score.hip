// score.hip -- indexer scoring on gfx950 matrix cores.
//
// Computes I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]) (HISA abstract:
// the lightweight token indexer; StreamIndex abstract: H_I indexer heads)
// for one query row against 32-key sub-blocks:
//
//   * the q.k contraction runs on v_mfma_f32_32x32x16_bf16 with the query's
//     heads as the 32-row M dimension and 32 keys as the N dimension, so one
//     query's 64 heads are two M blocks and its q fragment (64 x D bf16)
//     stays in VGPRs for the whole row;
//   * the 16 k elements one MFMA consumes are split between the two lane
//     halves: lanes 0-31 take dim [ks*8, ks*8+8), lanes 32-63 take
//     [D/2 + ks*8, ...), so each lane streams one contiguous D/2 run of a key
//     row (128 B for bf16, 64 B for fp8) with 16-byte loads;
//   * the ReLU * w head reduction is fused into the MFMA epilogue: each lane
//     holds 32 of the 64 heads of one key in its accumulators, reduces them
//     with FMAs and adds the other half with one lane swap;
//   * fp8 e4m3fn keys are widened exactly to bf16 in registers
//     (v_cvt_scalef32_pk_bf16_fp8, scale 1) and the per-token scale is applied
//     to the reduced score (scale >= 0 commutes with the ReLU).

#include <algorithm>

#include "score_common.hpp"

namespace tks {

namespace {

// Block-list entries of one row (HISA kept blocks, forced ones included).
constexpr int kMaxBlkEntries = 512;


// ------------------------------------------------------------------------
// Fused segment filter.  A workgroup that scored one segment of a row holds
// the segment's score keys in LDS (key 0: no candidate) and the range of
// its valid keys (tracked while scoring).  It keeps at most r_cap of them
// without sorting: the segment's score range [vmin, vmax] is cut into 256
// equal bins (a non-decreasing function of the score), and the kept keys
// are those of the top bins that together hold at most r_cap.  Every
// dropped key lies in a lower bin, so it is below every kept key: the
// segment's threshold T (the smallest kept key, or above vmax when none is
// kept) bounds every dropped key from above, which is all the finish needs
// to prove its result exact.  A segment that fits keeps everything (T = 0).

constexpr int kFilterScratch = 256 + 32;  // words of a 256-thread filter: bins, wave sums, results

__device__ __forceinline__ uint64_t fz_composite(uint32_t key, int32_t idx) {
    return ((uint64_t)key << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// key_score of tks_device.hpp, for the bin of a key
__device__ __forceinline__ float fz_value(uint32_t key) {
    const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return __uint_as_float(u);
}

// Filter stash[0, n) (n_valid valid keys, whose smallest and largest keys
// this thread saw are lo / hi) of segment `seg` of pool row `row`; the key
// index of stash slot i is key0 + i.  NT threads call it (NT bins, one per
// thread in the scan); n <= kFusedSeg; scratch holds NT + 32 words.
template <int NT>
__device__ __forceinline__ void fused_filter(const uint32_t* stash, int32_t n, int32_t n_valid,
                                             int32_t key0, uint32_t* scratch, const FusedPool& P,
                                             int64_t row, int32_t seg, uint32_t lo, uint32_t hi) {
    constexpr int NB = NT, PER = kFusedSeg / NT;
    static_assert(PER % 4 == 0, "16-byte stash reads");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t* hist = scratch;
    int32_t* wsum = reinterpret_cast<int32_t*>(scratch + NB);
    uint32_t* misc = scratch + NB + 16;  // kmin, kmax, kept, kept min, keep-from bin
    // this thread's keys: slots c * 4 NT + 4 * tid + j (16-byte LDS reads)
    uint32_t key[PER];
#pragma unroll
    for (int c = 0; c < PER / 4; ++c) {
        const int i0 = c * (4 * NT) + 4 * tid;
        const u32x4 v = i0 < n ? *reinterpret_cast<const u32x4*>(stash + i0) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) key[4 * c + j] = i0 + j < n ? v[j] : 0u;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
    }
    if (tid == 0) {
        misc[0] = 0xFFFFFFFFu;
        misc[1] = 0u;
        misc[2] = 0u;
        misc[3] = 0xFFFFFFFFu;
        misc[4] = 0u;  // keep from bin 0: every valid key
    }
    hist[tid] = 0u;
    __syncthreads();
    if (lane == 0) {
        atomicMin(&misc[0], lo);
        atomicMax(&misc[1], hi);
    }
    __syncthreads();
    const uint32_t kmin = misc[0], kmax = misc[1];
    const float vmin = fz_value(kmin);
    const float range = fz_value(kmax) - vmin;
    // (a range that overflows, or so narrow that the bin scale overflows,
    // keeps no key; the finish then rescores the row)
    float scale = range > 0.0f && range < __builtin_inff() ? (float)NB / range : 0.0f;
    if (!(scale < __builtin_inff())) scale = 0.0f;
    const bool filter = n_valid > P.r_cap;
    auto bin_of = [&](uint32_t k) {
        return (int32_t)fminf((fz_value(k) - vmin) * scale, (float)(NB - 1));
    };
    if (filter && scale > 0.0f) {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            if (key[e]) atomicAdd(&hist[bin_of(key[e])], 1u);
        __syncthreads();
        // bins from the top: the first bin at which the count passes r_cap
        // is the boundary; keep the bins above it
        const int32_t c = (int32_t)hist[NB - 1 - tid];
        int32_t inc = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t v = __shfl_up(inc, o);
            if (lane >= o) inc += v;
        }
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) inc += w < wave ? wsum[w] : 0;
        if (inc - c <= P.r_cap && inc > P.r_cap) misc[4] = (uint32_t)(NB - tid);
    } else if (filter) {
        if (tid == 0) misc[4] = NB;  // keep none
    }
    __syncthreads();
    const int32_t keep_from = (int32_t)misc[4];
    // emit the kept keys (wave-aggregated slots in the segment's pool run)
    uint64_t* dst = P.cand + (row * P.n_seg + seg) * (int64_t)P.r_cap;
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t kept_min = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const uint32_t k = key[e];
        const bool p = k != 0u && (!filter || (keep_from < NB && scale > 0.0f && bin_of(k) >= keep_from));
        const uint64_t m = __ballot(p);
        if (m == 0) continue;
        if (p) kept_min = min(kept_min, k);
        uint32_t at = 0;
        if (lane == 0) at = atomicAdd(&misc[2], (uint32_t)__popcll(m));
        const int32_t pos = (int32_t)__builtin_amdgcn_readlane((int)at, 0) + (int32_t)__popcll(m & lt);
        const int i = (e >> 2) * (4 * NT) + 4 * tid + (e & 3);
        if (p && pos < P.r_cap) dst[pos] = fz_composite(k, key0 + i);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) kept_min = min(kept_min, (uint32_t)__shfl_xor((int)kept_min, o));
    if (lane == 0) atomicMin(&misc[3], kept_min);
    __syncthreads();
    if (tid == 0) {
        const uint32_t kept = misc[2];
        P.count[row * P.n_seg + seg] = min((int32_t)kept, P.r_cap);
        // every dropped key is below the smallest kept one (or above none)
        P.tau[row * P.n_seg + seg] = !filter ? 0u : kept > 0 ? misc[3] : kmax + 1u;
    }
}

// One wave's filter of the keys it scored in a segment, as pool segment
// `seg` of row `row` (the waves of a workgroup then never wait for each
// other): key[e] of each lane (0: no candidate) has key index idx_of(e);
// lo / hi are the smallest and largest valid key the lane saw.  The rule
// of fused_filter over 256 value bins, with wave-level reductions only;
// hist is the wave's own 256 words of LDS (one wave's LDS instructions run
// in program order, so no barrier orders its phases).  Survivors are
// placed by a bitwise ballot prefix of the lanes' counts.
template <int PER, class IDX>
__device__ __forceinline__ void fused_filter_wave(const uint32_t (&key)[PER], IDX&& idx_of, uint32_t* hist,
                                                  const FusedPool& P, int64_t row, int32_t seg,
                                                  uint32_t lo, uint32_t hi) {
    constexpr int NB = 256;
    static_assert(PER < 32, "per-lane counts fit five bits");
    const int lane = threadIdx.x & 63;
    const uint64_t lt = (1ull << lane) - 1ull;
    int32_t n_valid = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) n_valid += __popcll(__ballot(key[e] != 0u));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
    }
    const uint32_t kmin = lo, kmax = hi;
    const float vmin = fz_value(kmin);
    const float range = fz_value(kmax) - vmin;
    float scale = range > 0.0f && range < __builtin_inff() ? (float)NB / range : 0.0f;
    if (!(scale < __builtin_inff())) scale = 0.0f;
    const bool filter = n_valid > P.r_cap;
    auto bin_of = [&](uint32_t k) {
        return (int32_t)fminf((fz_value(k) - vmin) * scale, (float)(NB - 1));
    };
    int32_t keep_from = 0;  // every valid key
    if (filter) {
        keep_from = NB;  // none, unless the bins place the boundary
        if (scale > 0.0f) {
#pragma unroll
            for (int i = 0; i < NB / 64; ++i) hist[lane * (NB / 64) + i] = 0u;
            // (the adds as inline LDS instructions: the bins never share LDS
            // with the key ring, and a compiler atomic would first wait for
            // every ring copy in flight)
            const uint32_t hbase = (uint32_t)(uintptr_t)hist;
#pragma unroll
            for (int e = 0; e < PER; ++e)
                if (key[e]) asm volatile("ds_add_u32 %0, %1" ::"v"(hbase + 4u * (uint32_t)bin_of(key[e])), "v"(1u) : "memory");
            // lane l holds bins NB-1-4l .. NB-4-4l (descending); the first bin
            // at which the count from the top passes r_cap is the boundary,
            // and the bins above it are kept
            constexpr int BPL = NB / 64;
            int32_t c[BPL];
            int32_t sum = 0;
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                c[i] = (int32_t)hist[NB - 1 - (BPL * lane + i)];
                sum += c[i];
            }
            int32_t inc = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int32_t v = __shfl_up(inc, o);
                if (lane >= o) inc += v;
            }
            int32_t cum = inc - sum, kf = 0;
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                if (cum <= P.r_cap && cum + c[i] > P.r_cap) kf = NB - (BPL * lane + i);
                cum += c[i];
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) kf = max(kf, __shfl_xor(kf, o));
            if (kf > 0) keep_from = kf;
        }
    }
    uint64_t* dst = P.cand + (row * P.n_seg + seg) * (int64_t)P.r_cap;
    uint32_t kept_min = 0xFFFFFFFFu;
    bool keep[PER];
    int32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const uint32_t k = key[e];
        keep[e] = k != 0u && (!filter || (keep_from < NB && scale > 0.0f && bin_of(k) >= keep_from));
        cnt += keep[e] ? 1 : 0;
        if (keep[e]) kept_min = min(kept_min, k);
    }
    int32_t pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
        const uint64_t bb = __ballot((cnt >> b) & 1);
        pre += __popcll(bb & lt) << b;
        tot += __popcll(bb) << b;
    }
    int32_t pos = pre;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        if (keep[e]) {
            if (pos < P.r_cap) dst[pos] = fz_composite(key[e], idx_of(e));
            ++pos;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) kept_min = min(kept_min, (uint32_t)__shfl_xor((int)kept_min, o));
    if (lane == 0) {
        P.count[row * P.n_seg + seg] = min(tot, P.r_cap);
        // every dropped key is below the smallest kept one (or above none)
        P.tau[row * P.n_seg + seg] = !filter ? 0u : tot > 0 ? kept_min : kmax + 1u;
    }
}

// WPR (wave per row): each wave owns one row and walks all its slots;
// otherwise a workgroup owns one row segment and its 4 waves interleave
// 32-slot sub-blocks.
template <int D, int MB, bool FP8, bool BLOCKS, bool WPR, bool FUSE = false>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a, int64_t n_rows,
                                                    int32_t seg_slots) {
    static_assert(!FUSE || (!BLOCKS && !WPR), "fused mode: contiguous row segments");
    constexpr int KS = D / 16;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m = lane & 31;
    const int hf = lane >> 5;
    if (FUSE && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.fuse_clear = 0;

    const int64_t y = WPR ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
    if (y >= n_rows) return;
    const int32_t seq = a.rows.seq(y);
    const int32_t t = a.rows.query(y);
    const int64_t qr = a.rows.qrow(y);
    const int32_t n_tok = a.vis.tokens(t);

    int32_t slot_begin, slot_end, step, first;
    if (WPR) {
        slot_begin = 0;
        slot_end = a.n_cols;
        first = 0;
        step = 32;
    } else {
        slot_begin = blockIdx.y * seg_slots;
        slot_end = min(a.n_cols, slot_begin + seg_slots);
        first = wave * 32;
        step = 128;
    }
    // Slots past `limit` are certainly masked.
    int32_t limit = slot_end;
    if (!BLOCKS) limit = min(slot_end, max(0, a.vis.count(t) - a.col_key0));
    int32_t work_end = a.write_masked ? slot_end : limit;
    if (slot_begin >= work_end) return;

    // q fragment: A operand rows = heads (mb*32 + m), k elements as above.
    bf16x8 qa[MB][KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int h = mb * 32 + m;
        if (h < a.heads) {
            const u32x4* p = reinterpret_cast<const u32x4*>(a.q + (qr * a.heads + h) * D + hf * (D / 2));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = __builtin_bit_cast(bf16x8, p[ks]);
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        }
    }
    // head weights of this lane's accumulator rows: mb*32 + 8*(j/4) + 4*hf + j%4
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int h = mb * 32 + 8 * (j >> 2) + 4 * hf + (j & 3);
            wv[mb][j] = h < a.heads ? a.w[qr * a.heads + h] : 0.0f;
        }

    const int64_t kseq = (int64_t)seq * a.k_seq_len;
    const int32_t bmask = (1 << a.block_shift) - 1;
    // the row's block list, staged in LDS: a key address then never waits on
    // a global load that the key loads already in flight would hold up
    __shared__ int32_t s_blk[BLOCKS ? kMaxBlkEntries : 1];
    __shared__ int32_t s_last[4];
    // fused mode: the segment's score keys, then the filter's scratch; the
    // smallest / largest valid key this lane stored
    __shared__ __align__(16) uint32_t s_stash[FUSE ? kFusedSeg : 4];
    __shared__ uint32_t s_scr[FUSE ? kFilterScratch : 1];
    uint32_t f_lo = 0xFFFFFFFFu, f_hi = 0u;
    if constexpr (BLOCKS) {
        const int32_t* blk_row = a.blk + (a.rows.y0 + y) * a.blk_stride;
        const int32_t n_ent = (a.n_cols + bmask) >> a.block_shift;
        int32_t last = -1;  // last list entry holding a block
        for (int i = threadIdx.x; i < n_ent; i += 256) {
            const int32_t bb = blk_row[i];
            s_blk[i] = bb;
            if (bb >= 0) last = i;
        }
        if constexpr (!WPR) {
            // slots after the last kept block (the -1 padding of rows with
            // fewer eligible blocks than the list holds) need no work
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o));
            if (lane == 0) s_last[wave] = last;
        }
        __syncthreads();
        if constexpr (!WPR) {
            last = max(max(s_last[0], s_last[1]), max(s_last[2], s_last[3]));
            limit = min(limit, (last + 1) << a.block_shift);
            if (!a.write_masked) work_end = limit;
            if (slot_begin >= work_end) return;
        }
    }

    auto key_of = [&](int32_t slot, bool& valid) -> int32_t {
        int32_t key;
        if (BLOCKS) {
            // the block list is only read for slots inside the row
            const int32_t b = slot < limit ? s_blk[slot >> a.block_shift] : -1;
            // blocks past the last visible key are skipped before the shift
            const bool ok = b >= 0 && b <= ((n_tok - 1) >> a.block_shift);
            key = ok ? (b << a.block_shift) + (slot & bmask) : 0;
            valid = ok && key < n_tok;
        } else {
            key = a.col_key0 + slot;
            valid = slot < limit;
        }
        return key;
    };

    // One 32-slot sub-block: MFMA over the key fragment, fused ReLU * w head
    // reduction, store.  `scale` is the key's fp8 scale (1 for bf16).
    auto process = [&](const KeyFrag<D, FP8>& f, int32_t j, bool valid, float scale) {
        f32x16 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kb = key_operand<D, FP8>(f, ks);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
        }
        float sc = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc = fmaf(wv[mb][i], relu_bits(acc[mb][i]), sc);
        sc += __shfl_xor(sc, 32);
        if (FP8) sc *= scale;
        const int32_t slot = j + m;
        if constexpr (FUSE) {
            const uint32_t key = valid ? score_key(sc) : 0u;
            if (hf == 0 && slot < slot_end) s_stash[slot - slot_begin] = key;
            if (valid) {
                f_lo = min(f_lo, key);
                f_hi = max(f_hi, key);
            }
        } else if (hf == 0 && slot < slot_end) {
            if (valid)
                a.out[y * a.out_stride + slot] = sc;
            else if (a.write_masked)
                a.out[y * a.out_stride + slot] = -__builtin_inff();
        }
    };
    // Fetch the fragment (and fp8 scale) of this lane's key of sub-block j;
    // slots without a key read key 0 of the sequence and are never stored.
    auto fetch = [&](KeyFrag<D, FP8>& f, int32_t j, bool& valid, float& scale) {
        const int32_t key = key_of(j + m, valid);
        valid = valid && j < work_end;
        const int64_t row = kseq + (valid ? key : 0);
        load_key<D, FP8>(f, a.k, row, hf);
        if (FP8) scale = a.k_scale[row];
    };

    // Ring of fragments in flight, unrolled so that no register is rotated
    // and the loop body has no early exit: a sub-block past the end is
    // computed on a clamped address and never stored.
    int32_t j0 = slot_begin + first;
    if constexpr (FP8) {
        // fp8 fragments are 16 VGPRs: three sub-blocks in flight
        KeyFrag<D, FP8> f0, f1, f2;
        bool v0, v1, v2;
        float s0 = 1.0f, s1 = 1.0f, s2 = 1.0f;
        fetch(f0, j0, v0, s0);
        fetch(f1, j0 + step, v1, s1);
        fetch(f2, j0 + 2 * step, v2, s2);
        for (; j0 < work_end; j0 += 3 * step) {
            process(f0, j0, v0, s0);
            fetch(f0, j0 + 3 * step, v0, s0);
            process(f1, j0 + step, v1, s1);
            fetch(f1, j0 + 4 * step, v1, s1);
            process(f2, j0 + 2 * step, v2, s2);
            fetch(f2, j0 + 5 * step, v2, s2);
        }
    } else {
        KeyFrag<D, FP8> f0, f1;
        bool v0, v1;
        float s0 = 1.0f, s1 = 1.0f;
        fetch(f0, j0, v0, s0);
        fetch(f1, j0 + step, v1, s1);
        for (; j0 < work_end; j0 += 2 * step) {
            process(f0, j0, v0, s0);
            fetch(f0, j0 + 2 * step, v0, s0);
            process(f1, j0 + step, v1, s1);
            fetch(f1, j0 + 3 * step, v1, s1);
        }
    }
    if constexpr (FUSE) {
        // every 32-slot sub-block that starts below work_end was stored
        __syncthreads();
        const int32_t n_fill = min(slot_end, work_end) - slot_begin;
        fused_filter<256>(s_stash, n_fill, limit - slot_begin, a.col_key0 + slot_begin, s_scr, a.fuse,
                          y, blockIdx.y, f_lo, f_hi);
    }
}

// ------------------------------------------------------------------------
// fp8 keys streamed once (decode, gathered refinement): every wave keeps a
// ring of R sub-blocks in flight through LDS.  Each lane copies its own key
// fragment (and the key's scale) with direct global->LDS loads that hold no
// VGPRs while in flight and bypass the caches' reuse policy (nontemporal);
// the lane reads the fragment back itself, so the ring needs no barrier.
// The compiler cannot see which LDS slot a copy lands in, so the ring is
// read with inline-asm LDS loads and the wait for stage t is an explicit
// vmcnt: after stage t's copies the wave issues the copies of the R - 1
// later stages (CH + 1 each) and possibly stores, which only raise the
// count, so vmcnt((R - 1) * (CH + 1)) guarantees stage t has landed.

template <int D, int NR>
struct Fp8Ring {
    static constexpr int R = NR;                      // ring stages per wave
    static constexpr int CH = D / 32;                 // 16-byte chunks per lane and key
    static constexpr int STAGE = CH * 1024 + 256;     // chunk slabs + per-lane scales
    static constexpr int WAVE = R * STAGE;
};

// Read one ring stage (CH 16-byte chunks at base + off[c], and the scale)
// with a single wait; early-clobber outputs keep every address register
// intact while the reads are in flight.
template <int CH>
__device__ __forceinline__ void lds_read_stage(uint32_t base, const uint32_t* off, uint32_t saddr,
                                               u32x4* raw, float& scale) {
    if constexpr (CH == 4) {
        asm volatile(
            "ds_read_b128 %0, %5\n\t"
            "ds_read_b128 %1, %6\n\t"
            "ds_read_b128 %2, %7\n\t"
            "ds_read_b128 %3, %8\n\t"
            "ds_read_b32 %4, %9\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(raw[0]), "=&v"(raw[1]), "=&v"(raw[2]), "=&v"(raw[3]), "=&v"(scale)
            : "v"(base + off[0]), "v"(base + off[1]), "v"(base + off[2]), "v"(base + off[3]),
              "v"(saddr));
    } else if constexpr (CH == 2) {
        asm volatile(
            "ds_read_b128 %0, %3\n\t"
            "ds_read_b128 %1, %4\n\t"
            "ds_read_b32 %2, %5\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(raw[0]), "=&v"(raw[1]), "=&v"(scale)
            : "v"(base + off[0]), "v"(base + off[1]), "v"(saddr));
    } else {
        asm volatile(
            "ds_read_b128 %0, %2\n\t"
            "ds_read_b32 %1, %3\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(raw[0]), "=&v"(scale)
            : "v"(base + off[0]), "v"(saddr));
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// NW waves per workgroup, NR ring stages per wave (every launch takes four
// waves with three stages: two workgroups per CU).
template <int D, int MB, bool BLOCKS, bool FUSE = false, int NW = 4, int NR = 3, bool WAVEF = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void score_fp8_kernel(
    ScoreArgs a, int64_t n_rows, int32_t seg_slots) {
    static_assert(!FUSE || !BLOCKS, "fused mode: contiguous row segments");
    static_assert(!WAVEF || (FUSE && NW == kFusedWaves), "a pool segment per wave of a fused workgroup");
    constexpr int NT = NW * 64;
    constexpr int SB = NW * 32;  // slots per sub-block round of the workgroup
    using RG = Fp8Ring<D, NR>;
    if (FUSE && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.fuse_clear = 0;
    constexpr int KS = D / 16;
    __shared__ __align__(16) uint8_t ring[NW * RG::WAVE];
    // the row's q, zero-padded heads; rows padded by 16 bytes so that the
    // fragment reads (32 head rows, one column) spread over the banks
    constexpr int QS = D + 8;
    // (fused mode: after the q fragments are built, the segment's score
    // keys take this space)
    constexpr int QN = FUSE && MB * 32 * QS < 2 * kFusedSeg ? 2 * kFusedSeg : MB * 32 * QS;
    __shared__ __align__(16) uint16_t s_q[QN];
    uint32_t* stash = reinterpret_cast<uint32_t*>(s_q);
    // filter scratch: the workgroup's (kFilterScratch words), or 256 bins per
    // wave when every wave filters its own keys (WAVEF)
    __shared__ uint32_t s_fscr[!FUSE ? 1 : WAVEF ? NW * 256 : NT + 32];
    uint32_t f_lo = 0xFFFFFFFFu, f_hi = 0u;  // fused mode: range of this lane's valid keys
    __shared__ float s_w[MB * 32];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // (uniform: scalar addressing)
    const int m = lane & 31;
    const int hf = lane >> 5;

    const int64_t y = blockIdx.x;
    if (y >= n_rows) return;
    const int32_t seq = a.rows.seq(y);
    const int32_t t = a.rows.query(y);
    const int64_t qr = a.rows.qrow(y);
    const int32_t n_tok = a.vis.tokens(t);
    const int32_t slot_begin = blockIdx.y * seg_slots;
    const int32_t slot_end = min(a.n_cols, slot_begin + seg_slots);
    const int32_t limit = BLOCKS ? slot_end : min(slot_end, max(0, a.vis.count(t) - a.col_key0));
    const int32_t work_end = a.write_masked ? slot_end : limit;
    if (slot_begin >= work_end) return;

    bf16x8 qa[MB][KS];  // loaded after the first ring copies are issued
    float wv[MB][16];
    const int64_t kseq = (int64_t)seq * a.k_seq_len;
    const int32_t bmask = (1 << a.block_shift) - 1;
    // the row's block list in LDS (see score_kernel); staged before the first
    // key copies, which need it for their addresses
    __shared__ int32_t s_blk[BLOCKS ? kMaxBlkEntries : 1];
    if constexpr (BLOCKS) {
        const int32_t* blk_row = a.blk + (a.rows.y0 + y) * a.blk_stride;
        const int32_t n_ent = (a.n_cols + bmask) >> a.block_shift;
        for (int i = threadIdx.x; i < n_ent; i += NT) s_blk[i] = blk_row[i];
        __syncthreads();
    }
    auto key_of = [&](int32_t slot, bool& valid) -> int32_t {
        if (BLOCKS) {
            const int32_t b = slot < limit ? s_blk[slot >> a.block_shift] : -1;
            const bool ok = b >= 0 && b <= ((n_tok - 1) >> a.block_shift);
            const int32_t key = ok ? (b << a.block_shift) + (slot & bmask) : 0;
            valid = ok && key < n_tok;
            return key;
        }
        valid = slot < limit;
        return a.col_key0 + slot;
    };

    uint8_t* wring = ring + wave * RG::WAVE;
    const uint32_t wring_addr = (uint32_t)(uintptr_t)wring;
    // sub-block u of this wave covers slots first + u * SB .. + 31
    const int32_t first = slot_begin + wave * 32;
    const int32_t nsub = first < work_end ? (work_end - first + SB - 1) / SB : 0;

    // D = 128: copy instruction c reads key rows 8c .. 8c+7 of the sub-block
    // as one contiguous KiB (full cache lines, nontemporal): lane j = 8r + q
    // takes chunk (q - r - c) mod 8 of row 8c + r.  The read-back below
    // inverts the rotation, which spreads every 16-lane group of a read over
    // all LDS banks.  Other dims copy each lane's own half row.
    constexpr bool ROT = D == 128;
    const int rr = lane >> 3, qq = lane & 7;
    // byte offset of this lane's copy c from the sub-block's first key row
    uint32_t loff[RG::CH];
#pragma unroll
    for (int c = 0; c < RG::CH; ++c) {
        if constexpr (ROT)
            loff[c] = (uint32_t)((8 * c + rr) * D + ((qq - rr - c) & 7) * 16);
        else
            loff[c] = (uint32_t)(m * D + hf * (D / 2) + c * 16);
    }
    auto fetch = [&](int32_t u) {
        uint8_t* st = wring + (u % RG::R) * RG::STAGE;
        // a sub-block whose 32 slots all hold visible keys is one run of key
        // rows (a block holds whole sub-blocks): a uniform base and each
        // lane's fixed offset, with no per-key checks (the same copies)
#if defined(__HIP_DEVICE_COMPILE__)  // (device code only; the host pass skips it)
        const int32_t s0 = first + u * SB;
        int32_t kb0 = 0;
        bool whole;
        if constexpr (BLOCKS) {
            const int32_t b = s0 + 32 <= limit ? __builtin_amdgcn_readfirstlane(s_blk[s0 >> a.block_shift]) : -1;
            kb0 = (b << a.block_shift) + (s0 & bmask);
            whole = b >= 0 && kb0 + 32 <= n_tok;
        } else {
            kb0 = a.col_key0 + s0;
            whole = s0 + 32 <= limit;
        }
        if (whole) {
            const uint8_t* sb = reinterpret_cast<const uint8_t*>(a.k) + (kseq + kb0) * D;
#pragma unroll
            for (int c = 0; c < RG::CH; ++c) {
                if constexpr (ROT)
                    __builtin_amdgcn_global_load_lds(sb + loff[c], st + c * 1024, 16, 0, 2);
                else
                    __builtin_amdgcn_global_load_lds(sb + loff[c], st + c * 1024, 16, 0, 0);
            }
            __builtin_amdgcn_global_load_lds(a.k_scale + kseq + kb0 + m, st + RG::CH * 1024, 4, 0, 0);
            return;
        }
#endif
        if constexpr (ROT) {
#pragma unroll
            for (int c = 0; c < RG::CH; ++c) {
                bool valid;
                const int32_t key = key_of(first + u * SB + 8 * c + rr, valid);
                const int64_t row = kseq + (valid && first + u * SB < work_end ? key : 0);
                const int chunk = (qq - rr - c) & 7;
                __builtin_amdgcn_global_load_lds(
                    reinterpret_cast<const uint8_t*>(a.k) + row * D + chunk * 16, st + c * 1024,
                    16, 0, 2);
            }
            bool valid;
            const int32_t key = key_of(first + u * SB + m, valid);
            const int64_t row = kseq + (valid && first + u * SB < work_end ? key : 0);
            __builtin_amdgcn_global_load_lds(a.k_scale + row, st + RG::CH * 1024, 4, 0, 0);
        } else {
            bool valid;
            const int32_t key = key_of(first + u * SB + m, valid);
            const int64_t row = kseq + (valid && first + u * SB < work_end ? key : 0);
            const uint8_t* src = reinterpret_cast<const uint8_t*>(a.k) + row * D + hf * (D / 2);
#pragma unroll
            for (int c = 0; c < RG::CH; ++c)
                __builtin_amdgcn_global_load_lds(src + c * 16, st + c * 1024, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(a.k_scale + row, st + RG::CH * 1024, 4, 0, 0);
        }
    };
    // read-back offsets of this lane's four chunks (key m, half hf)
    uint32_t roff[RG::CH];
#pragma unroll
    for (int c = 0; c < RG::CH; ++c) {
        if constexpr (ROT) {
            const int i = m >> 3, r = m & 7, cc = hf * 4 + c;
            roff[c] = i * 1024 + (8 * r + ((cc + r + i) & 7)) * 16;
        } else {
            roff[c] = c * 1024 + lane * 16;
        }
    }

    // MFMAs of sub-block u, from the ring slot it occupies
    auto mfma_stage = [&](int32_t u, f32x16* acc, float& scale) {
        wait_vmcnt<(RG::R - 1) * (RG::CH + 1)>();
        const uint32_t st = wring_addr + (u % RG::R) * RG::STAGE;
        u32x4 raw[RG::CH];
        lds_read_stage<RG::CH>(st, roff, st + RG::CH * 1024 + lane * 4, raw, scale);
        fetch(u + RG::R);  // refill the slot just read
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4& v = raw[ks >> 1];
            const uint32_t d0 = (ks & 1) ? v[2] : v[0];
            const uint32_t d1 = (ks & 1) ? v[3] : v[1];
            const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, false);
            const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, true);
            const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, false);
            const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, true);
            bf16x8 kb;
            kb[0] = p0[0]; kb[1] = p0[1]; kb[2] = p1[0]; kb[3] = p1[1];
            kb[4] = p2[0]; kb[5] = p2[1]; kb[6] = p3[0]; kb[7] = p3[1];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
        }
    };
    // ReLU * w head reduction and store of sub-block u (WAVEF: returns the
    // score key of slot first + u * SB + m, 0 when not visible)
    auto epilogue = [&](int32_t u, const f32x16* acc, float scale) -> uint32_t {
        float sc = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc = fmaf(wv[mb][i], relu_bits(acc[mb][i]), sc);
        sc += __shfl_xor(sc, 32);
        sc *= scale;
        const int32_t j = first + u * SB;
        bool valid;
        key_of(j + m, valid);
        const int32_t slot = j + m;
        if constexpr (FUSE) {
            const uint32_t key = valid ? score_key(sc) : 0u;
            // (the second half reuses the stash after the first is filtered)
            if (hf == 0 && slot < slot_end) stash[(slot - slot_begin) & (kFusedSeg - 1)] = key;
            if (valid) {
                f_lo = min(f_lo, key);
                f_hi = max(f_hi, key);
            }
            return key;
        } else {
            if (hf == 0 && slot < slot_end) {
                if (valid)
                    a.out[y * a.out_stride + slot] = sc;
                else if (a.write_masked)
                    a.out[y * a.out_stride + slot] = -__builtin_inff();
            }
            return 0u;
        }
    };

#pragma unroll
    for (int u = 0; u < RG::R; ++u) fetch(u);
    // q / w: read once per workgroup into LDS (overlapping the first ring
    // copies), then every wave builds its fragments from there
    {
        const int hq = a.heads * D;  // bf16 elements of the row's q
        const uint16_t* qsrc = a.q + qr * hq;
        for (int e = threadIdx.x * 8; e < MB * 32 * D; e += NT * 8) {
            u32x4 v = u32x4{0, 0, 0, 0};
            if (e < hq) v = *reinterpret_cast<const u32x4*>(qsrc + e);
            *reinterpret_cast<u32x4*>(&s_q[(e / D) * QS + e % D]) = v;
        }
        for (int h = threadIdx.x; h < MB * 32; h += NT) s_w[h] = h < a.heads ? a.w[qr * a.heads + h] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int h = mb * 32 + m;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qa[mb][ks] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(&s_q[h * QS + hf * (D / 2) + ks * 8]));
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) wv[mb][j] = s_w[mb * 32 + 8 * (j >> 2) + 4 * hf + (j & 3)];
    // (fused mode: every wave has its fragments before the stash overwrites q)
    if constexpr (FUSE) __syncthreads();

    // two accumulator sets: the MFMAs of sub-block u + 1 are issued before the
    // VALU epilogue of sub-block u, so the matrix and vector pipes overlap
    f32x16 acc0[MB], acc1[MB];
    float sc0 = 1.0f, sc1 = 1.0f;
    auto run = [&](int32_t u0, int32_t u1) {  // this wave's sub-blocks [u0, u1)
        if (u0 >= u1) return;
        mfma_stage(u0, acc0, sc0);
        for (int32_t u = u0; u < u1; u += 2) {
            if (u + 1 < u1) mfma_stage(u + 1, acc1, sc1);
            epilogue(u, acc0, sc0);
            if (u + 1 >= u1) break;
            if (u + 2 < u1) mfma_stage(u + 2, acc0, sc0);
            epilogue(u + 1, acc1, sc1);
        }
    };
    if constexpr (!FUSE) {
        run(0, nsub);
        // drain the copies still in flight before the wave's LDS is released
        wait_vmcnt<0>();
    } else {
        // fused mode: the segment is parts of kFusedSeg keys (sub-blocks
        // [p * kPart, (p + 1) * kPart) of every wave hold part p), each one
        // pool segment, or with WAVEF one pool segment per wave.  A part is
        // filtered while the ring copies of the next part's first stages
        // are in flight; the filter scratch is its own LDS.
        constexpr int32_t kPart = kFusedSeg / SB;
        static_assert(kPart * SB == kFusedSeg, "whole sub-block rounds per part");
        const int32_t parts = seg_slots / kFusedSeg;
        for (int32_t p = 0; p < parts; ++p) {
            const int32_t h = slot_begin + p * kFusedSeg;  // (uniform)
            if (h >= work_end) break;
            if (p > 0) {
                f_lo = 0xFFFFFFFFu;
                f_hi = 0u;
                // the stage waits count on copies completing in issue
                // order; the filter's stores could complete out of order
                // with them, so a later part starts with nothing in flight
                // (its first stages have been landing during the filter)
                wait_vmcnt<0>();
                if constexpr (!WAVEF) __syncthreads();  // (and the filter has read the stash)
            }
            if constexpr (WAVEF) {
                // this wave's keys of the part, read back from the stash,
                // where only this wave wrote them (its own LDS writes, in
                // program order: no barrier): lane (m, hf) takes sub-blocks
                // u0 + 2e + hf; sub-blocks the wave did not reach hold none
                constexpr int PER = kPart / 2;
                const int32_t u0 = p * kPart, u1 = min(nsub, (p + 1) * kPart);
                run(u0, u1);
                uint32_t key[PER];
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    key[e] = u0 + 2 * e + hf < u1 ? stash[wave * 32 + (2 * e + hf) * SB + m] : 0u;
                const int32_t i0 = a.col_key0 + first + (u0 + hf) * SB + m;
                fused_filter_wave<PER>(key, [&](int e) { return i0 + e * (2 * SB); }, s_fscr + wave * 256,
                                       a.fuse, y, ((int32_t)blockIdx.y * parts + p) * NW + wave, f_lo, f_hi);
            } else {
                run(p * kPart, min(nsub, (p + 1) * kPart));
                __syncthreads();
                fused_filter<NT>(stash, min(min(slot_end, work_end) - h, kFusedSeg), min(limit - h, kFusedSeg),
                                 a.col_key0 + h, s_fscr, a.fuse, y, (int32_t)blockIdx.y * parts + p, f_lo, f_hi);
            }
        }
        wait_vmcnt<0>();
    }
}

// ------------------------------------------------------------------------
// Keys shared by a block of queries (prefill: contiguous key runs, bf16
// keys, D = 128).  A workgroup of NW waves owns NW consecutive query rows
// of one sequence, one row per wave, and a run of key slots.  The run is
// staged through an LDS ring of 128-key stages that all waves fill together
// with direct global->LDS copies; every staged key feeds the MFMAs of all NW
// queries, so a key crosses the L2 once per NW queries instead of once per
// query, and the copies run NS - 1 stages ahead of the MFMAs.  The loop
// walks one stage per barrier with its four sub-blocks unrolled, so every
// sub-block's LDS reads carry its offset as an immediate; the waves raise
// their issue priority while they feed the matrix pipe.
//
// Stage layout: key row r (256 bytes = 16 chunks of 16 bytes) keeps logical
// chunk c at physical chunk c ^ (r & 15).  A copy writes LDS linearly (lane
// i lands at base + 16 i), so each lane fetches the global chunk that
// belongs at its position; one copy still covers 4 whole key rows (1 KiB
// contiguous in memory).  When the lanes holding keys 0..31 read logical
// chunk c, every 16 consecutive lanes touch 16 distinct chunk columns, so
// the reads are free of bank conflicts.
struct SharedRing {
    static constexpr int D = 128;
    static constexpr int SK = 128;            // keys per stage
    static constexpr int SPS = SK / 32;       // 32-key sub-blocks per stage
    static constexpr int STAGE = SK * D * 2;  // 32 KiB
    static constexpr int NS = 3;              // stages in flight
};
constexpr int kSharedRows = 8;  // query rows (waves) per workgroup

template <int MB, int NW>
__global__ __launch_bounds__(NW * 64) void score_shared_kernel(ScoreArgs a, int64_t n_rows,
                                                               int32_t blocks_per_seq,
                                                               int32_t seg_slots) {
    using RG = SharedRing;
    constexpr int D = RG::D;
    constexpr int KS = D / 16;
    constexpr int CPW = RG::STAGE / (NW * 64 * 16);  // copies per wave and stage
    static_assert(CPW * NW * 64 * 16 == RG::STAGE, "stage split");
    __shared__ __align__(16) uint8_t ring[RG::NS * RG::STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m = lane & 31;
    const int hf = lane >> 5;

    // chunk rows [r_lo, r_hi) of one sequence
    const int64_t R = a.rows.rows_per_seq;
    const int64_t seq = a.rows.y0 / R + blockIdx.x / blocks_per_seq;
    const int64_t s_lo = seq * R - a.rows.y0;
    const int64_t lo = s_lo > 0 ? s_lo : 0;
    const int64_t hi = s_lo + R < n_rows ? s_lo + R : n_rows;
    const int64_t r_lo = lo + (int64_t)(blockIdx.x % blocks_per_seq) * NW;
    if (r_lo >= hi) return;
    const int64_t r_hi = r_lo + NW < hi ? r_lo + NW : hi;
    const bool active = r_lo + wave < r_hi;
    const int64_t y = active ? r_lo + wave : r_hi - 1;  // idle waves shadow the last row
    // (the RowMap helpers without their 64-bit divisions: seq is known)
    const int32_t t = a.rows.t_begin + (int32_t)(y - s_lo);
    const int64_t qr = seq * a.rows.n_q + t;

    const int32_t slot_begin = blockIdx.y * seg_slots;
    const int32_t slot_end = min(a.n_cols, slot_begin + seg_slots);
    // visibility grows with the query: the block's last row sees the most
    const int32_t blk_limit =
        min(slot_end, max(0, a.vis.count(a.rows.t_begin + (int32_t)(r_hi - 1 - s_lo)) - a.col_key0));
    const int32_t work_end = a.write_masked ? slot_end : blk_limit;
    if (slot_begin >= work_end) return;
    const int32_t limit = min(slot_end, max(0, a.vis.count(t) - a.col_key0));
    const int32_t n_st = (work_end - slot_begin + RG::SK - 1) / RG::SK;
    const int32_t nsub = (work_end - slot_begin + 31) / 32;

    // q fragment and head weights (as in score_kernel)
    bf16x8 qa[MB][KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int h = mb * 32 + m;
        if (h < a.heads) {
            const u32x4* p = reinterpret_cast<const u32x4*>(a.q + (qr * a.heads + h) * D + hf * (D / 2));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = __builtin_bit_cast(bf16x8, p[ks]);
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        }
    }
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int h = mb * 32 + 8 * (j >> 2) + 4 * hf + (j & 3);
            wv[mb][j] = h < a.heads ? a.w[qr * a.heads + h] : 0.0f;
        }

    // copies: chunk p = (i * NW + wave) * 64 + lane of a stage is row p / 16,
    // physical chunk p % 16, logical chunk (p % 16) ^ (row & 15)
    const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.k) + seq * a.k_seq_len * (2 * D);
    const int32_t kmax = (int32_t)(a.k_seq_len - 1);
    int32_t crow[CPW];
    uint32_t cchunk[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int p = (i * NW + wave) * 64 + lane;
        crow[i] = p >> 4;
        cchunk[i] = (uint32_t)(((p & 15) ^ ((p >> 4) & 15)) * 16);
    }
    auto fetch = [&](int32_t s) {
        uint8_t* st = ring + (s % RG::NS) * RG::STAGE;
        const int32_t key0 = a.col_key0 + slot_begin + s * RG::SK;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int32_t key = min(key0 + crow[i], kmax);
            // (one 64-bit offset: with two separate additions the host pass
            // of this compiler drops the kernel's launch stub)
            __builtin_amdgcn_global_load_lds(kseq + ((int64_t)key * (2 * D) + (int64_t)cchunk[i]),
                                             st + (i * NW + wave) * 1024, 16, 0, 0);
        }
    };
    // Stage s is ready once this wave's copies of it have landed (copies of
    // one wave complete in order; the later stages already issued, and any
    // stores, only raise the count) and every wave has passed the barrier,
    // which also means all waves are done reading stage s - 1, whose slot
    // the next copy reuses.
    auto sync = [&](int32_t s) {
        if (s + 1 < n_st)
            wait_vmcnt<CPW * (RG::NS - 2)>();
        else
            wait_vmcnt<0>();
        asm volatile("s_barrier" ::: "memory");
        if (s + RG::NS - 1 < n_st) fetch(s + RG::NS - 1);
    };
    static_assert(RG::NS == 3, "sync() counts one later stage");
    static_assert(RG::SPS % 2 == 0, "a sub-block's accumulator set (u % 2) follows from its place in the stage");

    uint32_t roff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[ks] = m * (2 * D) + (((hf * 8 + ks) ^ (m & 15)) * 16);
    // this lane's chunk pointers into the current stage; a sub-block adds a
    // compile-time offset, which the LDS reads carry as an immediate
    const uint8_t* sp[KS];
    auto stage_ptrs = [&](int32_t st) {
        const uint8_t* b = ring + (st % RG::NS) * RG::STAGE;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sp[ks] = b + roff[ks];
    };
    auto read_sub = [&](int j, u32x4* raw) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            raw[ks] = *reinterpret_cast<const u32x4*>(sp[ks] + j * 32 * (2 * D));
    };
    auto mfma_sub = [&](int j, f32x16* acc) {
        u32x4 raw[KS];
        read_sub(j, raw);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kb = __builtin_bit_cast(bf16x8, raw[ks]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
        }
    };
    auto reduce = [&](const f32x16* acc) {
        float sc = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc = fmaf(wv[mb][i], relu_bits(acc[mb][i]), sc);
        return add_upper_half(sc);
    };
    auto mfma_reduce = [&](int j, f32x16* acc, const f32x16* prev) {
        constexpr int PER = MB * 16 / KS;  // reduced elements per k-step
        u32x4 raw[KS];
        read_sub(j, raw);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
        float sc = 0.0f;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kb = __builtin_bit_cast(bf16x8, raw[ks]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = ks * PER; e < (ks + 1) * PER; ++e)
                sc = fmaf(wv[e >> 4][e & 15], relu_bits(prev[e >> 4][e & 15]), sc);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        return add_upper_half(sc);
    };
    float* orow = a.out + y * a.out_stride;
    auto store = [&](int32_t u, float sc) {
        const int32_t slot = slot_begin + u * 32 + m;
        const bool vis = slot < limit;
        if (active && hf == 0 && slot < slot_end && (vis || a.write_masked))
            orow[slot] = vis ? sc : -__builtin_inff();
    };

#pragma unroll
    for (int s = 0; s < RG::NS - 1; ++s)
        if (s < n_st) fetch(s);
    // Sub-block u is part u % SPS of stage u / SPS.  The MFMAs of u are
    // issued together with the VALU reduction of u - 1 (two accumulator
    // sets, acc[u % 2]); a stage's first sub-block follows its barrier, and
    // the store of the sub-block before it comes after that barrier so that
    // the stage waits never cover a store just issued.
    f32x16 acc0[MB], acc1[MB];
    sync(0);
    stage_ptrs(0);
    mfma_sub(0, acc0);
    for (int32_t st = 0;; ++st) {
        if (st > 0) {
            if (st * RG::SPS >= nsub) break;
            sync(st);
            stage_ptrs(st);
        }
        bool end = false;
#pragma unroll
        for (int j = 0; j < RG::SPS; ++j) {
            const int32_t u = st * RG::SPS + j;
            if (!end && u > 0) {
                if (u >= nsub) {
                    end = true;
                } else {
                    const float sv = (j & 1) ? mfma_reduce(j, acc1, acc0) : mfma_reduce(j, acc0, acc1);
                    store(u - 1, sv);
                }
            }
        }
        if (end) break;
    }
    // the last sub-block's reduction
    store(nsub - 1, ((nsub - 1) & 1) ? reduce(acc1) : reduce(acc0));
    wait_vmcnt<0>();
}

// ------------------------------------------------------------------------
// HISA refinement for prefill (HISA abstract: the token indexer again, only
// inside each query's kept blocks).  The keys are shared by position: the
// workgroup is the shared-key one (consecutive queries of one sequence, one
// per wave, a ring of key stages), and a wave runs the MFMAs and head
// reduction of a 32-key sub-block only when its row kept the sub-block's
// block, writing the scores to the row's slots e * B + (key mod B) for list
// entry e.  The arithmetic is the flat kernel's, so the scores are the same
// fp32 values.
//
// Refinement over a shared key ring with producer and consumer waves.
// NW consumer waves (one query row each) walk the ring at their own pace:
// a wave skips the sub-blocks its row did not keep and may run up to NS - 1
// stages ahead of the slowest, so the rows' different block lists average
// out instead of every stage costing the slowest row's work (as it would
// with a barrier per stage).  NP producer waves only copy, each whole
// stages in turn: a producer waits until every consumer is done with the
// stage its slot held, copies the new one, waits for its own loads and
// publishes it, so NP stages are in flight at once.  Each slot counts the
// consumers done with it over all its stages (the stage in slot x % NS may
// be overwritten by stage x once the count reaches NW * (x / NS)), and holds
// the number of the stage it has.  Waits are sleep loops: a consumer waits
// only for a producer, which waits only for consumers finishing an earlier
// stage, so every loop ends; the bound keeps a kernel from hanging forever
// should that reasoning fail, and then the failure shows in the output: the
// wave raises the workgroup's flag and consumers store NaN scores from then
// on, which no selection passes as a correct result.
constexpr int32_t kRingSpinMax = 1 << 22;

template <typename F>
__device__ __forceinline__ void spin_until(F&& ok, int32_t* fail) {
    for (int32_t spin = 0; spin < kRingSpinMax; ++spin) {
        if (ok()) return;
        __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_store(fail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// NW rows per workgroup, NS ring stages of 128 keys (32 KiB), NP producers.
template <int MB, int NW, int NS, int NP>
__global__ __launch_bounds__((NW + NP) * 64) void refine_shared_kernel(ScoreArgs a, int64_t n_rows,
                                                                       int32_t blocks_per_seq,
                                                                       int32_t seg_slots) {
    using RG = SharedRing;
    constexpr int D = RG::D;
    constexpr int KS = D / 16;
    constexpr int PIECES = RG::STAGE / (64 * 16);   // 16-byte copies of a stage per lane
    constexpr int CPW = PIECES / NW;                // ... per consumer in the first stages
    static_assert(CPW * NW == PIECES, "stage split");
    static_assert(NS > NP && NP >= 1, "ring depth");
    __shared__ __align__(16) uint8_t ring[NS * RG::STAGE];
    __shared__ int32_t s_ready[NS];                 // stage held by each slot
    __shared__ int32_t s_done[NS];                  // consumers done, all stages of the slot
    __shared__ int32_t s_fail;                      // a bounded wait ran out
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m = lane & 31;
    const int hf = lane >> 5;

    // chunk rows [r_lo, r_hi) of one sequence (as in score_shared_kernel)
    const int64_t R = a.rows.rows_per_seq;
    const int64_t seq = a.rows.y0 / R + blockIdx.x / blocks_per_seq;
    const int64_t s_lo = seq * R - a.rows.y0;
    const int64_t lo = s_lo > 0 ? s_lo : 0;
    const int64_t hi = s_lo + R < n_rows ? s_lo + R : n_rows;
    const int64_t r_lo = lo + (int64_t)(blockIdx.x % blocks_per_seq) * NW;
    if (r_lo >= hi) return;
    const int64_t r_hi = r_lo + NW < hi ? r_lo + NW : hi;
    const bool consumer = wave < NW;
    const bool active = consumer && r_lo + wave < r_hi;
    const int64_t y = active ? r_lo + wave : r_hi - 1;
    const int32_t t = a.rows.t_begin + (int32_t)(y - s_lo);
    const int64_t qr = seq * a.rows.n_q + t;
    const int32_t n_tok = a.vis.tokens(t);

    const int32_t slot_begin = blockIdx.y * seg_slots;  // key slots (key = slot)
    const int32_t work_end =
        min(min(a.n_cols, slot_begin + seg_slots), a.vis.tokens(a.rows.t_begin + (int32_t)(r_hi - 1 - s_lo)));
    if (slot_begin >= work_end) return;
    const int32_t n_st = (work_end - slot_begin + RG::SK - 1) / RG::SK;
    const int32_t nsub = (work_end - slot_begin + 31) / 32;

    const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.k) + seq * a.k_seq_len * (2 * D);
    const int32_t kmax = (int32_t)(a.k_seq_len - 1);
    // piece p (16 bytes at slot offset 16 p) of a stage is key row p / 16,
    // physical chunk p % 16, logical chunk (p % 16) ^ (row % 16); p - lane is
    // the same for the whole wave (the copy's LDS base)
    auto copy_piece = [&](uint8_t* sp, int32_t key0, int p) {
        const int32_t key = min(key0 + (p >> 4), kmax);
        const uint32_t chunk = (uint32_t)(((p & 15) ^ ((p >> 4) & 15)) * 16);
        __builtin_amdgcn_global_load_lds(kseq + ((int64_t)key * (2 * D) + (int64_t)chunk),
                                         sp + (p - lane) * 16, 16, 0, 0);
    };

    // the row's kept blocks of the segment as a mask (bit i: block b0 + i; a
    // segment starts on a block boundary and spans at most 64 blocks) and
    // the list position of the first of them (the list is ascending)
    const int32_t bshift = a.block_shift;
    const int32_t b0 = slot_begin >> bshift;
    uint32_t kmask_lo = 0, kmask_hi = 0;
    int32_t before = 0;
    if (active) {
        const int32_t* lst = a.blk + (a.rows.y0 + y) * a.blk_stride;
        for (int i = lane; i < a.blk_stride; i += 64) {
            const int32_t e = lst[i];
            if (e >= 0 && e < b0) {
                ++before;
            } else if (e >= b0 && e < b0 + 64) {
                if (e - b0 < 32)
                    kmask_lo |= 1u << (e - b0);
                else
                    kmask_hi |= 1u << (e - b0 - 32);
            }
        }
    }
    // first NS stages: copied by the consumers together
    if (consumer) {
#pragma unroll 1
        for (int st = 0; st < NS; ++st) {
            if (st < n_st) {
                uint8_t* sp = ring + st * RG::STAGE;
#pragma unroll
                for (int i = 0; i < CPW; ++i) copy_piece(sp, slot_begin + st * RG::SK, (i * NW + wave) * 64 + lane);
            }
        }
    }
    if (threadIdx.x < NS) {
        s_ready[threadIdx.x] = threadIdx.x < n_st ? (int32_t)threadIdx.x : -1;
        s_done[threadIdx.x] = 0;
        if (threadIdx.x == 0) s_fail = 0;
    }
    wait_vmcnt<0>();
    __syncthreads();  // the first stages and the slot states

    if (!consumer) {
#pragma unroll 1
        for (int32_t x = NS + (wave - NW); x < n_st; x += NP) {
            const int sl = x % NS;
            const int32_t freed = NW * (x / NS);
            spin_until(
                [&] {
                    return __hip_atomic_load(&s_done[sl], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= freed;
                },
                &s_fail);
            uint8_t* sp = ring + sl * RG::STAGE;
#pragma unroll
            for (int i = 0; i < PIECES; ++i) copy_piece(sp, slot_begin + x * RG::SK, i * 64 + lane);
            wait_vmcnt<0>();
            if (lane == 0) __hip_atomic_store(&s_ready[sl], x, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        return;
    }

    bf16x8 qa[MB][KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int h = mb * 32 + m;
        if (h < a.heads) {
            const u32x4* p = reinterpret_cast<const u32x4*>(a.q + (qr * a.heads + h) * D + hf * (D / 2));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = __builtin_bit_cast(bf16x8, p[ks]);
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        }
    }
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int h = mb * 32 + 8 * (j >> 2) + 4 * hf + (j & 3);
            wv[mb][j] = h < a.heads ? a.w[qr * a.heads + h] : 0.0f;
        }
    uint32_t roff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[ks] = m * (2 * D) + (((hf * 8 + ks) ^ (m & 15)) * 16);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        kmask_lo |= __shfl_xor(kmask_lo, o);
        kmask_hi |= __shfl_xor(kmask_hi, o);
        before += __shfl_xor(before, o);
    }
    // (the builtin returns a signed int: widen through uint32_t, or a set bit
    // 31 of the low word would sign-extend over the high word)
    const uint64_t kmask = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)kmask_hi) << 32) |
                           (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)kmask_lo);
    before = __builtin_amdgcn_readfirstlane(before);
    const int32_t bmask = (1 << bshift) - 1;
    float* orow = a.out + y * a.out_stride;

#pragma unroll 1
    for (int32_t st = 0; st < n_st; ++st) {
        const int slot = st % NS;
        // every stage is waited for, also one this row skips: a wave is then
        // never more than NS - 1 stages ahead of the slowest, which is what
        // makes the slot counts exact
        spin_until(
            [&] {
                return __hip_atomic_load(&s_ready[slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == st;
            },
            &s_fail);
        const uint8_t* sb = ring + slot * RG::STAGE;
#pragma unroll
        for (int j = 0; j < RG::SPS; ++j) {
            const int32_t u = st * RG::SPS + j;
            if (u >= nsub) break;
            const int32_t key0 = slot_begin + u * 32;
            const int32_t bi = (key0 >> bshift) - b0;  // 0 .. 63
            if (!((kmask >> bi) & 1) || key0 >= n_tok) continue;
            const int32_t ptr = before + __builtin_popcountll(kmask & ((1ull << bi) - 1));
            f32x16 acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 kb = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(sb + j * 32 * (2 * D) + roff[ks]));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
            }
            float sc = 0.0f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sc = fmaf(wv[mb][i], relu_bits(acc[mb][i]), sc);
            sc = add_upper_half(sc);
            const int32_t key = key0 + m;
            if (__hip_atomic_load(&s_fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) sc = __builtin_nanf("");
            if (hf == 0 && key < n_tok) orow[ptr * (bmask + 1) + (key & bmask)] = sc;
        }
        // done with the slot: its keys were read into registers above
        if (lane == 0) __hip_atomic_fetch_add(&s_done[slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

template <int MB, int NW, int NS, int NP>
hipError_t launch_refine_shared(const ScoreArgs& a, int64_t n_rows, hipStream_t stream) {
    const int64_t R = a.rows.rows_per_seq;
    const int64_t n_seq = (a.rows.y0 + n_rows - 1) / R - a.rows.y0 / R + 1;
    const int64_t per_seq = (std::min<int64_t>(n_rows, R) + NW - 1) / NW;
    // segments: whole blocks and whole stages, at most 64 blocks (the
    // kernel's kept-block mask), sized for a few workgroups per CU (each
    // computes about a quarter of what a flat one would)
    const int64_t unit = std::max<int64_t>(SharedRing::SK, int64_t(1) << a.block_shift);
    const int64_t cap = int64_t(64) << a.block_shift;
    const int64_t want = n_rows * (int64_t)a.n_cols / (NW * 8192);
    const int64_t seg = std::min<int64_t>(cap, std::max<int64_t>(2048, (want + unit - 1) / unit * unit));
    if ((a.n_cols + seg - 1) / seg > 65535) return hipErrorInvalidValue;
    dim3 grid((unsigned)(n_seq * per_seq), (unsigned)((a.n_cols + seg - 1) / seg));
    hipLaunchKernelGGL((refine_shared_kernel<MB, NW, NS, NP>), grid, dim3((NW + NP) * 64), 0, stream, a, n_rows,
                       (int32_t)per_seq, (int32_t)seg);
    return hipGetLastError();
}

// ------------------------------------------------------------------------
// Scheduled refinement.  In the segment ring above, a workgroup's time is
// set by the row of its 8 that kept the most blocks of the segment, and
// rows keep their blocks very unevenly along the keys, though each row
// keeps the same number in all (the scored blocks plus the forced ones).  So
// a group of 8 rows takes its whole visible range at once, and a plan orders
// the blocks any of them kept so that every row's work is spread evenly
// along the order: then the consumers run at about the same pace and the
// ring's few stages of slack suffice.  Blocks that no row kept are not
// copied at all.
//
// The plan (one wave per group) is greedy.  Blocks that the same rows kept
// (the same 8-bit pattern) are interchangeable, so each step picks a pattern:
// the one whose rows are furthest behind an even pace, score(p) = sum over
// rows j in p of (s + 1) * n_j / n - done_j, scaled by n to stay integer
// (n blocks in all, n_j of them kept by row j, done_j scheduled so far);
// ties go to the smaller pattern, and a pattern's blocks go in ascending
// order, so the plan is a function of the block lists alone.

// Group g of a call: queries [t0, t0 + nr) of sequence seq.
struct SchedGroup {
    int64_t seq;
    int32_t t0, nr;
};

__device__ __forceinline__ SchedGroup sched_group(int32_t n_q, int64_t g) {
    const int64_t per = (n_q + kSchedRows - 1) / kSchedRows;
    SchedGroup G;
    G.seq = g / per;
    G.t0 = (int32_t)(g % per) * kSchedRows;
    G.nr = min(kSchedRows, n_q - G.t0);
    return G;
}

// LDS of the plan kernel for `nb` (a multiple of 64) visible blocks and a
// layout stride `P` (a multiple of 4): pattern words, block -> union index,
// union blocks, union ranks, pattern counts and offsets, union patterns,
// pattern of each plan position, union indices by pattern
__host__ __device__ constexpr size_t plan_lds_bytes(int32_t nb, int32_t P) {
    return 3 * (size_t)nb + 24 * (size_t)P + 2048;
}

// Largest value over the wave (gfx9 DPP: shifts within rows of 16 lanes,
// then the row broadcasts; lane 63 ends with the maximum).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Lanes of the wave whose 8-bit value equals this lane's (one ballot per bit).
__device__ __forceinline__ uint64_t match8(uint32_t v) {
    uint64_t eq = ~0ull;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint64_t b = __ballot((v >> j) & 1u);
        eq &= ((v >> j) & 1u) ? b : ~b;
    }
    return eq;
}

__global__ __launch_bounds__(64) void refine_plan_kernel(ScoreArgs a, int64_t g_lo, int32_t lds_blocks) {
    extern __shared__ __align__(16) uint8_t plan_lds[];
    const int lane = threadIdx.x;
    const RefineSched P = a.sched;
    const int64_t gid = g_lo + blockIdx.x;
    const int64_t slot = gid - P.group0;
    const SchedGroup G = sched_group(a.rows.n_q, gid);
    const int nr = G.nr;
    const int64_t row0 = G.seq * a.rows.n_q + G.t0;  // global row of the group's first query
    const int32_t bshift = a.block_shift;
    const int32_t m_total = a.blk_stride;
    // blocks with a visible key, per row and for the group
    int32_t nbv_row[kSchedRows];
    int32_t nbv = 0;
#pragma unroll
    for (int j = 0; j < kSchedRows; ++j) {
        const int32_t n_tok = j < nr ? a.vis.tokens(G.t0 + j) : 0;
        nbv_row[j] = n_tok > 0 ? min(((n_tok - 1) >> bshift) + 1, lds_blocks) : 0;
        nbv = max(nbv, nbv_row[j]);
    }
    uint32_t* pw = reinterpret_cast<uint32_t*>(plan_lds);                 // [lds_blocks / 4]
    int16_t* umap = reinterpret_cast<int16_t*>(plan_lds + lds_blocks);    // [lds_blocks]
    int32_t* ublk = reinterpret_cast<int32_t*>(plan_lds + 3 * (size_t)lds_blocks);  // [P]
    int16_t* urank = reinterpret_cast<int16_t*>(ublk + P.stride);        // [P, kSchedRows]
    int32_t* pcnt = reinterpret_cast<int32_t*>(urank + (size_t)P.stride * kSchedRows);  // [256]
    int32_t* poff = pcnt + 256;                                          // [256]
    uint8_t* upat = reinterpret_cast<uint8_t*>(poff + 256);              // [P]
    uint8_t* seq = upat + P.stride;                                      // [P]
    int16_t* bucket = reinterpret_cast<int16_t*>(seq + P.stride);        // [P]

    const int nw = (nbv + 3) >> 2;
    for (int i = lane; i < nw; i += 64) pw[i] = 0u;
    for (int i = lane; i < 256; i += 64) pcnt[i] = 0;
    __syncthreads();
    // patterns: bit j of block b's byte = row j kept b
    for (int j = 0; j < nr; ++j) {
        const int32_t* lst = a.blk + (row0 + j) * (int64_t)m_total;
        for (int i = lane; i < m_total; i += 64) {
            const int32_t e = lst[i];
            if (e >= 0 && e < nbv_row[j]) atomicOr(&pw[e >> 2], 1u << (8 * (e & 3) + j));
        }
    }
    __syncthreads();
    // the union in ascending block order: lane owns words [w0, w1)
    const int cw = (nw + 63) >> 6;
    const int w0 = min(nw, lane * cw);
    const int w1 = min(nw, w0 + cw);
    int32_t cnt = 0;
    for (int w = w0; w < w1; ++w) {
        const uint32_t v = pw[w];
        cnt += ((v & 0xFFu) != 0u) + ((v & 0xFF00u) != 0u) + ((v & 0xFF0000u) != 0u) + ((v >> 24) != 0u);
    }
    int32_t inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    const int32_t n_u = __shfl(inc, 63);  // <= min(nbv, nr * m_total) <= P.stride
    int32_t u = inc - cnt;
    for (int w = w0; w < w1; ++w) {
        const uint32_t v = pw[w];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t pat = (v >> (8 * b)) & 0xFFu;
            if (pat != 0u) {
                ublk[u] = 4 * w + b;
                upat[u] = (uint8_t)pat;
                umap[4 * w + b] = (int16_t)u;
                ++u;
            }
        }
    }
    for (int i = lane; i < n_u * kSchedRows; i += 64) urank[i] = -1;
    __syncthreads();
    int32_t tot[kSchedRows];
#pragma unroll
    for (int j = 0; j < kSchedRows; ++j) tot[j] = 0;
    for (int i = lane; i < n_u; i += 64) {
        const uint32_t pat = upat[i];
        atomicAdd(&pcnt[pat], 1);
#pragma unroll
        for (int j = 0; j < kSchedRows; ++j) tot[j] += (pat >> j) & 1u;
    }
    for (int j = 0; j < nr; ++j) {
        const int32_t* lst = a.blk + (row0 + j) * (int64_t)m_total;
        for (int i = lane; i < m_total; i += 64) {
            const int32_t e = lst[i];
            if (e >= 0 && e < nbv_row[j]) urank[umap[e] * kSchedRows + j] = (int16_t)i;
        }
    }
#pragma unroll
    for (int j = 0; j < kSchedRows; ++j)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) tot[j] += __shfl_xor(tot[j], o);
    __syncthreads();

    // phase 1, the greedy over patterns (registers only): lane owns
    // patterns 4 lane .. 4 lane + 3; a pattern's key is its score shifted to
    // be non-negative (|score| < 2^22: n <= 1024 blocks, row totals <= 512)
    // with 255 - pattern below it, so the wave's largest key is the
    // pattern to take (ties: the smaller one)
    int32_t T[4], Dn[4], C[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = lane * 4 + k;
        T[k] = 0;
#pragma unroll
        for (int j = 0; j < kSchedRows; ++j) T[k] += ((p >> j) & 1) * tot[j];
        Dn[k] = 0;
        C[k] = p == 0 ? 0 : pcnt[p];
    }
    for (int32_t st = 0; st < n_u; ++st) {
        uint32_t key = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int32_t sc = (st + 1) * T[k] - n_u * Dn[k];
            const uint32_t kk = ((uint32_t)(sc + (1 << 22)) << 8) | (uint32_t)(255 - (lane * 4 + k));
            key = C[k] > 0 ? max(key, kk) : key;
        }
        const int32_t ps = 255 - (int32_t)(wave_max_u32(key) & 255u);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            Dn[k] += __builtin_popcount((uint32_t)((lane * 4 + k) & ps));
            C[k] -= (lane * 4 + k) == ps ? 1 : 0;
        }
        if (lane == 0) seq[st] = (uint8_t)ps;
    }
    // each pattern's union entries in ascending order: offsets, then a rank
    // among equal patterns for every entry (64 entries at a time)
    {
        int32_t c4[4], s4 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c4[k] = pcnt[lane * 4 + k];
            s4 += c4[k];
        }
        int32_t inc4 = s4;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t t = __shfl_up(inc4, o);
            if (lane >= o) inc4 += t;
        }
        int32_t run = inc4 - s4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            poff[lane * 4 + k] = run;
            run += c4[k];
        }
    }
    __syncthreads();
    for (int i = lane; i < 256; i += 64) pcnt[i] = 0;  // running counts per pattern
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
    for (int32_t c = 0; c < n_u; c += 64) {
        const int32_t u = c + lane;
        const uint32_t pu = u < n_u ? (uint32_t)upat[u] : 0u;  // 0: no entry
        const uint64_t eq = match8(pu) & __ballot(u < n_u);
        if (u < n_u) bucket[poff[pu] + pcnt[pu] + __popcll(eq & below)] = (int16_t)u;
        __syncthreads();
        if (u < n_u && (eq & below) == 0ull) pcnt[pu] += __popcll(eq);  // the group's first lane
        __syncthreads();
    }
    for (int i = lane; i < 256; i += 64) pcnt[i] = 0;
    __syncthreads();
    // phase 2: position st takes the next block of its pattern
    int32_t* out_blk = P.blocks + slot * P.stride;
    int16_t* out_rank = P.ranks + slot * P.stride * kSchedRows;
    for (int32_t c = 0; c < n_u; c += 64) {
        const int32_t st = c + lane;
        const uint32_t ps = st < n_u ? (uint32_t)seq[st] : 0u;
        const uint64_t eq = match8(ps) & __ballot(st < n_u);
        int32_t uu = 0;
        if (st < n_u) {
            uu = bucket[poff[ps] + pcnt[ps] + __popcll(eq & below)];
            out_blk[st] = ublk[uu];
            const uint64_t rk = *reinterpret_cast<const uint64_t*>(urank + uu * kSchedRows);
            const uint64_t rk2 = *reinterpret_cast<const uint64_t*>(urank + uu * kSchedRows + 4);
            reinterpret_cast<uint64_t*>(out_rank + (int64_t)st * kSchedRows)[0] = rk;
            reinterpret_cast<uint64_t*>(out_rank + (int64_t)st * kSchedRows)[1] = rk2;
        }
        __syncthreads();
        if (st < n_u && (eq & below) == 0ull) pcnt[ps] += __popcll(eq);
        __syncthreads();
    }
    if (lane == 0) P.n_pos[slot] = n_u;
}

// One workgroup per group: kSchedRows consumer waves (one row each) and NP
// producer waves over the plan's blocks, through an NS-stage ring of 128 key
// slots (with blocks of 32 or 64 keys a stage holds several plan positions,
// with 256-key blocks a position spans two stages).  Producers copy every
// stage (the first ones too, into free slots) and read a stage's block ids
// before issuing its copies; consumers issue no copies at all.
template <int MB, int NS, int NP>
__global__ __launch_bounds__((kSchedRows + NP) * 64) void refine_sched_kernel(ScoreArgs a, int64_t n_rows,
                                                                            int64_t g_lo) {
    using RG = SharedRing;
    constexpr int NW = kSchedRows;
    constexpr int D = RG::D;
    constexpr int KS = D / 16;
    constexpr int PIECES = RG::STAGE / (64 * 16);  // 16-byte copies of a stage per lane
    static_assert(NS > NP && NP >= 1, "ring depth");
    __shared__ __align__(16) uint8_t ring[NS * RG::STAGE];
    __shared__ int32_t s_blk[kSchedMaxPos];
    __shared__ __align__(16) int16_t s_rank[kSchedMaxPos * NW];
    __shared__ int32_t s_ready[NS];  // stage held by each slot
    __shared__ int32_t s_done[NS];   // consumers done, all stages of the slot
    __shared__ int32_t s_fail;       // a bounded wait ran out
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m = lane & 31;
    const int hf = lane >> 5;

    const int64_t gid = g_lo + blockIdx.x;
    const int64_t slot_g = gid - a.sched.group0;
    const SchedGroup G = sched_group(a.rows.n_q, gid);
    const int32_t n_pos = min(a.sched.n_pos[slot_g], kSchedMaxPos);
    if (n_pos <= 0) return;
    const bool consumer = wave < NW;
    // this wave's query and its chunk row (rows of the group outside the
    // chunk are left out)
    const int32_t t = G.t0 + min(wave, G.nr - 1);
    const int64_t qr = G.seq * a.rows.n_q + t;
    const int64_t yc = qr - a.rows.y0;
    const bool active = consumer && wave < G.nr && yc >= 0 && yc < n_rows;
    const int64_t y = active ? yc : 0;
    const int32_t n_tok = a.vis.tokens(t);

    // the plan into LDS (a position's ranks are 16 bytes)
    {
        const int32_t* pb = a.sched.blocks + slot_g * a.sched.stride;
        const u32x4* pr = reinterpret_cast<const u32x4*>(a.sched.ranks + slot_g * a.sched.stride * NW);
        for (int i = threadIdx.x; i < n_pos; i += (NW + NP) * 64) {
            s_blk[i] = pb[i];
            reinterpret_cast<u32x4*>(s_rank)[i] = pr[i];
        }
    }
    if (threadIdx.x < NS) {
        s_ready[threadIdx.x] = -1;
        s_done[threadIdx.x] = 0;
        if (threadIdx.x == 0) s_fail = 0;
    }
    __syncthreads();

    const int32_t bshift = a.block_shift;
    const int32_t bmask = (1 << bshift) - 1;
    const int32_t n_st = (int32_t)((((int64_t)n_pos << bshift) + RG::SK - 1) / RG::SK);
    const uint8_t* kseq = reinterpret_cast<const uint8_t*>(a.k) + G.seq * a.k_seq_len * (2 * D);
    const int32_t kmax = (int32_t)(a.k_seq_len - 1);

    if (!consumer) {
#pragma unroll 1
        for (int32_t x = wave - NW; x < n_st; x += NP) {
            const int sl = x % NS;
            const int32_t z0 = x * RG::SK;  // first slot of the stage
            const int32_t pos0 = z0 >> bshift;
            int32_t bk[4];  // blocks of the stage's positions (4 with 32-key blocks)
#pragma unroll
            for (int i = 0; i < 4; ++i) bk[i] = pos0 + i < n_pos ? s_blk[pos0 + i] : -1;
            const int32_t freed = NW * (x / NS);
            spin_until(
                [&] {
                    return __hip_atomic_load(&s_done[sl], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= freed;
                },
                &s_fail);
            uint8_t* sp = ring + sl * RG::STAGE;
#pragma unroll
            for (int i = 0; i < PIECES; ++i) {
                // piece p: slot z0 + p / 16 (row of the stage), physical chunk
                // p % 16, logical chunk (p % 16) ^ (row % 16)
                const int p = i * 64 + lane;
                const int32_t z = z0 + (p >> 4);
                const int32_t pi = (z >> bshift) - pos0;
                const int32_t b = pi == 0 ? bk[0] : pi == 1 ? bk[1] : pi == 2 ? bk[2] : bk[3];
                const int32_t key = b >= 0 ? min((b << bshift) + (z & bmask), kmax) : kmax;
                const uint32_t chunk = (uint32_t)(((p & 15) ^ ((p >> 4) & 15)) * 16);
                __builtin_amdgcn_global_load_lds(kseq + ((int64_t)key * (2 * D) + (int64_t)chunk),
                                                 sp + i * 1024, 16, 0, 0);
            }
            wait_vmcnt<0>();
            if (lane == 0) __hip_atomic_store(&s_ready[sl], x, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        return;
    }

    bf16x8 qa[MB][KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int h = mb * 32 + m;
        if (h < a.heads) {
            const u32x4* p = reinterpret_cast<const u32x4*>(a.q + (qr * a.heads + h) * D + hf * (D / 2));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = __builtin_bit_cast(bf16x8, p[ks]);
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[mb][ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
        }
    }
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int h = mb * 32 + 8 * (j >> 2) + 4 * hf + (j & 3);
            wv[mb][j] = h < a.heads ? a.w[qr * a.heads + h] : 0.0f;
        }
    uint32_t roff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[ks] = m * (2 * D) + (((hf * 8 + ks) ^ (m & 15)) * 16);
    float* orow = a.out + y * a.out_stride;

#pragma unroll 1
    for (int32_t st = 0; st < n_st; ++st) {
        const int slot = st % NS;
        // every stage is waited for, also one this row skips: a wave is then
        // never more than NS - 1 stages ahead of the slowest, which is what
        // makes the slot counts exact
        spin_until(
            [&] {
                return __hip_atomic_load(&s_ready[slot], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == st;
            },
            &s_fail);
        const uint8_t* sb = ring + slot * RG::STAGE;
#pragma unroll
        for (int j = 0; j < RG::SPS; ++j) {
            const int32_t z = st * RG::SK + j * 32;  // slot of the sub-block's first key
            const int32_t pos = z >> bshift;
            if (pos >= n_pos) break;
            const int32_t rank = s_rank[pos * NW + wave];
            if (!active || rank < 0) continue;
            const int32_t off = z & bmask;
            const int32_t key0 = (s_blk[pos] << bshift) + off;
            if (key0 >= n_tok) continue;
            f32x16 acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mb][i] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 kb = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(sb + j * 32 * (2 * D) + roff[ks]));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
            }
            float sc = 0.0f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sc = fmaf(wv[mb][i], relu_bits(acc[mb][i]), sc);
            sc = add_upper_half(sc);
            if (__hip_atomic_load(&s_fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) sc = __builtin_nanf("");
            if (hf == 0 && key0 + m < n_tok) orow[(rank << bshift) + off + m] = sc;
        }
        // done with the slot: its keys were read into registers above
        if (lane == 0) __hip_atomic_fetch_add(&s_done[slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

template <int MB, int NW>
hipError_t launch_shared(const ScoreArgs& a, int64_t n_rows, hipStream_t stream) {
    const int64_t R = a.rows.rows_per_seq;
    const int64_t n_seq = (a.rows.y0 + n_rows - 1) / R - a.rows.y0 / R + 1;
    const int64_t per_seq = (std::min<int64_t>(n_rows, R) + NW - 1) / NW;
    // segments: a multiple of the stage, sized for a few workgroups per CU
    const int64_t want = n_rows * (int64_t)a.n_cols / (NW * 2048);
    int64_t seg = std::min<int64_t>(4096, std::max<int64_t>(512, (want + 127) / 128 * 128));
    while ((a.n_cols + seg - 1) / seg > 65535) seg *= 2;
    dim3 grid((unsigned)(n_seq * per_seq), (unsigned)((a.n_cols + seg - 1) / seg));
    hipLaunchKernelGGL((score_shared_kernel<MB, NW>), grid, dim3(NW * 64), 0, stream, a, n_rows,
                       (int32_t)per_seq, (int32_t)seg);
    return hipGetLastError();
}

template <int D, int MB, bool FP8, bool BLOCKS>
hipError_t launch_t(const ScoreArgs& a, int64_t n_rows, hipStream_t stream) {
    if (n_rows <= 0 || a.n_cols <= 0) return hipSuccess;
    // several queries of one sequence per workgroup share each key tile
    if (D == 128 && !FP8 && !BLOCKS && !a.stream_keys && a.k_seq_len > 0 &&
        std::min<int64_t>(n_rows, a.rows.rows_per_seq) >= kSharedRows)
        return launch_shared<MB, kSharedRows>(a, n_rows, stream);
    if (FP8 && a.stream_keys) {
        // keys read once: fp8 LDS-ring streaming kernel, >= ~2048 workgroups
        // about two long-lived workgroups per CU, each loading its row's q / w
        // once and streaming a long run of keys
        const int64_t want = (n_rows * (int64_t)a.n_cols + 511) / 512;
        int64_t seg = std::min<int64_t>(16384, std::max<int64_t>(128, (want + 127) / 128 * 128));
        while ((a.n_cols + seg - 1) / seg > 65535) seg *= 2;
        dim3 grid((unsigned)n_rows, (unsigned)((a.n_cols + seg - 1) / seg));
        hipLaunchKernelGGL((score_fp8_kernel<D, MB, BLOCKS>), grid, dim3(256), 0, stream, a, n_rows,
                           (int32_t)seg);
        return hipGetLastError();
    }
    if (a.n_cols <= 1024 && !BLOCKS && n_rows >= 8192) {
        // many short rows: one wave per row
        dim3 grid((unsigned)((n_rows + 3) / 4));
        hipLaunchKernelGGL((score_kernel<D, MB, FP8, BLOCKS, true>), grid, dim3(256), 0, stream,
                           a, n_rows, 0);
    } else {
        // a workgroup per row segment; segments sized for >= ~2048 workgroups
        const int64_t want = (n_rows * (int64_t)a.n_cols + 2047) / 2048;
        int64_t seg = std::min<int64_t>(4096, std::max<int64_t>(128, (want + 127) / 128 * 128));
        while ((a.n_cols + seg - 1) / seg > 65535) seg *= 2;
        dim3 grid((unsigned)n_rows, (unsigned)((a.n_cols + seg - 1) / seg));
        hipLaunchKernelGGL((score_kernel<D, MB, FP8, BLOCKS, false>), grid, dim3(256), 0, stream,
                           a, n_rows, (int32_t)seg);
    }
    return hipGetLastError();
}

template <int D, int MB>
hipError_t launch_d(const ScoreArgs& a, int64_t n_rows, bool fp8, bool blocks, hipStream_t s) {
    if (fp8)
        return blocks ? launch_t<D, MB, true, true>(a, n_rows, s)
                      : launch_t<D, MB, true, false>(a, n_rows, s);
    return blocks ? launch_t<D, MB, false, true>(a, n_rows, s)
                  : launch_t<D, MB, false, false>(a, n_rows, s);
}

}  // namespace

void refine_sched_groups(const RowMap& rows, int64_t n_rows, int64_t& g_lo, int64_t& g_hi) {
    g_lo = g_hi = 0;
    if (n_rows <= 0 || rows.n_q <= 0) return;
    const int64_t per = (rows.n_q + kSchedRows - 1) / kSchedRows;
    auto group_of = [&](int64_t global_row) {
        return (global_row / rows.n_q) * per + (global_row % rows.n_q) / kSchedRows;
    };
    g_lo = group_of(rows.y0);
    g_hi = group_of(rows.y0 + n_rows - 1) + 1;
}

hipError_t launch_refine_plan(const ScoreArgs& a, int64_t g_lo, int64_t g_hi, hipStream_t stream) {
    const RefineSched& P = a.sched;
    if (g_hi <= g_lo) return hipSuccess;
    if (P.stride < 4 || P.stride > kSchedMaxPos || P.stride % 4 || P.max_blocks < 1 ||
        P.max_blocks > kSchedMaxBlocks || a.blk_stride < 1 || a.blk_stride > kMaxBlkEntries ||
        g_lo < P.group0 || a.rows.rows_per_seq != a.rows.n_q || a.rows.t_begin != 0 || g_hi - g_lo > INT32_MAX)
        return hipErrorInvalidValue;
    const int32_t lds_blocks = (P.max_blocks + 63) / 64 * 64;
    hipLaunchKernelGGL(refine_plan_kernel, dim3((unsigned)(g_hi - g_lo)), dim3(64),
                       plan_lds_bytes(lds_blocks, P.stride), stream, a, g_lo, lds_blocks);
    return hipGetLastError();
}

hipError_t launch_score_refine_sched(const ScoreArgs& a, int64_t n_rows, hipStream_t stream) {
    if (n_rows <= 0) return hipSuccess;
    if (a.rows.rows_per_seq != a.rows.n_q || a.rows.t_begin != 0) return hipErrorInvalidValue;
    int64_t g_lo, g_hi;
    refine_sched_groups(a.rows, n_rows, g_lo, g_hi);
    if (g_lo < a.sched.group0 || g_hi - g_lo > INT32_MAX) return hipErrorInvalidValue;
    if (a.heads > 32)
        hipLaunchKernelGGL((refine_sched_kernel<2, 4, 3>), dim3((unsigned)(g_hi - g_lo)),
                           dim3((kSchedRows + 3) * 64), 0, stream, a, n_rows, g_lo);
    else
        hipLaunchKernelGGL((refine_sched_kernel<1, 4, 3>), dim3((unsigned)(g_hi - g_lo)),
                           dim3((kSchedRows + 3) * 64), 0, stream, a, n_rows, g_lo);
    return hipGetLastError();
}

hipError_t launch_score_refine_shared(const ScoreArgs& a, int64_t n_rows, hipStream_t stream) {
    if (n_rows <= 0 || a.n_cols <= 0) return hipSuccess;
    return a.heads > 32 ? launch_refine_shared<2, kSharedRows, 4, 3>(a, n_rows, stream)
                        : launch_refine_shared<1, kSharedRows, 4, 3>(a, n_rows, stream);
}

hipError_t launch_score_fused(const ScoreArgs& a, int64_t n_rows, int32_t n_seg, bool fp8,
                              hipStream_t stream) {
    if (n_rows <= 0 || n_seg <= 0) return hipSuccess;
    if (n_seg > 65535 || a.fuse.cand == nullptr) return hipErrorInvalidValue;
    // heads padded to 64 (zero q rows and weights add exactly nothing), so
    // the finish's rescoring uses the same instruction sequence
    if (fp8) {
        // four-wave workgroups, two per CU, each taking two pool segments of
        // a row (one when that would leave fewer workgroups than CU slots).
        // (Eight-wave workgroups with four ring stages, one per CU, measured
        // slower: every part boundary stalls the CU's only workgroup.)
        const int32_t parts = n_rows * ((n_seg + 1) / 2) >= 512 ? 2 : 1;
        const dim3 grid((unsigned)n_rows, (unsigned)((n_seg + parts - 1) / parts));
        // (a pool split per wave: every wave filters its own keys)
        if (a.fuse.split == kFusedWaves)
            hipLaunchKernelGGL((score_fp8_kernel<128, 2, false, true, 4, 3, true>), grid, dim3(256), 0, stream, a,
                               n_rows, (int32_t)(parts * kFusedSeg));
        else if (a.fuse.split == 1)
            hipLaunchKernelGGL((score_fp8_kernel<128, 2, false, true, 4, 3>), grid, dim3(256), 0, stream, a,
                               n_rows, (int32_t)(parts * kFusedSeg));
        else
            return hipErrorInvalidValue;
    } else {
        if (a.fuse.split != 1) return hipErrorInvalidValue;  // (one filter per workgroup)
        hipLaunchKernelGGL((score_kernel<128, 2, false, false, false, true>),
                           dim3((unsigned)n_rows, (unsigned)n_seg), dim3(256), 0, stream, a, n_rows,
                           (int32_t)kFusedSeg);
    }
    return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, int64_t n_rows, int dim, bool fp8, bool blocks,
                        hipStream_t stream) {
    const bool two = a.heads > 32;
    switch (dim) {
        case 32:
            return two ? launch_d<32, 2>(a, n_rows, fp8, blocks, stream)
                       : launch_d<32, 1>(a, n_rows, fp8, blocks, stream);
        case 64:
            return two ? launch_d<64, 2>(a, n_rows, fp8, blocks, stream)
                       : launch_d<64, 1>(a, n_rows, fp8, blocks, stream);
        case 128:
            return two ? launch_d<128, 2>(a, n_rows, fp8, blocks, stream)
                       : launch_d<128, 1>(a, n_rows, fp8, blocks, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace tks

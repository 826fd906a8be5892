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

#include "tks_launch.hpp"

namespace tks {

namespace {

template <int D, bool FP8>
struct KeyFrag {
    // bf16: D/2 bf16 = D bytes per lane; fp8: D/2 bytes per lane.
    static constexpr int kBytes = FP8 ? D / 2 : D;
    static constexpr int kVec = kBytes / 16;
    u32x4 v[kVec];
};

// Branch-free fragment load (the caller clamps `row` into the key tensor for
// slots that hold no key), so the compiler can keep several loads in
// flight and wait for each one by count.
template <int D, bool FP8>
__device__ inline void load_key(KeyFrag<D, FP8>& f, const void* k, int64_t row, int hf) {
    constexpr int KB = KeyFrag<D, FP8>::kBytes;
    const u32x4* p = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint8_t*>(k) + row * (int64_t)(FP8 ? D : 2 * D) + hf * KB);
#pragma unroll
    for (int i = 0; i < KeyFrag<D, FP8>::kVec; ++i) f.v[i] = p[i];
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Block-list entries of one row (HISA kept blocks, forced ones included).
constexpr int kMaxBlkEntries = 512;

// max(0, x) in one integer max on the bit pattern: negative floats (and -0)
// are negative integers, non-negative floats keep their order.  Inputs are
// finite, so no NaN handling is needed.
__device__ __forceinline__ float relu_bits(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// B operand of k-step ks from a key fragment.
template <int D, bool FP8>
__device__ inline bf16x8 key_operand(const KeyFrag<D, FP8>& f, int ks) {
    if constexpr (!FP8) {
        return __builtin_bit_cast(bf16x8, f.v[ks]);
    } else {
        // 8 fp8 codes = 2 dwords of vector ks/2
        const u32x4& v = f.v[ks >> 1];
        uint32_t d0 = (ks & 1) ? v[2] : v[0];
        uint32_t d1 = (ks & 1) ? v[3] : v[1];
        bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, false);
        bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, true);
        bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, false);
        bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, true);
        bf16x8 r;
        r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
        r[4] = c[0]; r[5] = c[1]; r[6] = e[0]; r[7] = e[1];
        return r;
    }
}

// WPR (wave per row): each wave owns one row and walks all its slots;
// otherwise a workgroup owns one row segment and its 4 waves interleave
// 32-slot sub-blocks.
template <int D, int MB, bool FP8, bool BLOCKS, bool WPR>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a, int64_t n_rows,
                                                    int32_t seg_slots) {
    constexpr int KS = D / 16;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m = lane & 31;
    const int hf = lane >> 5;

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
        if (hf == 0 && slot < slot_end) {
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

template <int D>
struct Fp8Ring {
    static constexpr int R = 3;                       // stages in flight per wave
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

template <int D, int MB, bool BLOCKS>
__global__ __launch_bounds__(256) void score_fp8_kernel(ScoreArgs a, int64_t n_rows,
                                                        int32_t seg_slots) {
    using RG = Fp8Ring<D>;
    constexpr int KS = D / 16;
    __shared__ __align__(16) uint8_t ring[4 * RG::WAVE];
    // the row's q, zero-padded heads; rows padded by 16 bytes so that the
    // fragment reads (32 head rows, one column) spread over the banks
    constexpr int QS = D + 8;
    __shared__ __align__(16) uint16_t s_q[MB * 32 * QS];
    __shared__ float s_w[MB * 32];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
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
        for (int i = threadIdx.x; i < n_ent; i += 256) s_blk[i] = blk_row[i];
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
    // sub-block u of this wave covers slots first + u * 128 .. + 31
    const int32_t first = slot_begin + wave * 32;
    const int32_t nsub = first < work_end ? (work_end - first + 127) / 128 : 0;

    // D = 128: copy instruction c reads key rows 8c .. 8c+7 of the sub-block
    // as one contiguous KiB (full cache lines, nontemporal): lane j = 8r + q
    // takes chunk (q - r - c) mod 8 of row 8c + r.  The read-back below
    // inverts the rotation, which spreads every 16-lane group of a read over
    // all LDS banks.  Other dims copy each lane's own half row.
    constexpr bool ROT = D == 128;
    const int rr = lane >> 3, qq = lane & 7;
    auto fetch = [&](int32_t u) {
        uint8_t* st = wring + (u % RG::R) * RG::STAGE;
        if constexpr (ROT) {
#pragma unroll
            for (int c = 0; c < RG::CH; ++c) {
                bool valid;
                const int32_t key = key_of(first + u * 128 + 8 * c + rr, valid);
                const int64_t row = kseq + (valid && first + u * 128 < work_end ? key : 0);
                const int chunk = (qq - rr - c) & 7;
                __builtin_amdgcn_global_load_lds(
                    reinterpret_cast<const uint8_t*>(a.k) + row * D + chunk * 16, st + c * 1024,
                    16, 0, 2);
            }
            bool valid;
            const int32_t key = key_of(first + u * 128 + m, valid);
            const int64_t row = kseq + (valid && first + u * 128 < work_end ? key : 0);
            __builtin_amdgcn_global_load_lds(a.k_scale + row, st + RG::CH * 1024, 4, 0, 0);
        } else {
            bool valid;
            const int32_t key = key_of(first + u * 128 + m, valid);
            const int64_t row = kseq + (valid && first + u * 128 < work_end ? key : 0);
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
    // ReLU * w head reduction and store of sub-block u
    auto epilogue = [&](int32_t u, const f32x16* acc, float scale) {
        float sc = 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc = fmaf(wv[mb][i], relu_bits(acc[mb][i]), sc);
        sc += __shfl_xor(sc, 32);
        sc *= scale;
        const int32_t j = first + u * 128;
        bool valid;
        key_of(j + m, valid);
        const int32_t slot = j + m;
        if (hf == 0 && slot < slot_end) {
            if (valid)
                a.out[y * a.out_stride + slot] = sc;
            else if (a.write_masked)
                a.out[y * a.out_stride + slot] = -__builtin_inff();
        }
    };

#pragma unroll
    for (int u = 0; u < RG::R; ++u) fetch(u);
    // q / w: read once per workgroup into LDS (overlapping the first ring
    // copies), then every wave builds its fragments from there
    {
        const int hq = a.heads * D;  // bf16 elements of the row's q
        const uint16_t* qsrc = a.q + qr * hq;
        for (int e = threadIdx.x * 8; e < MB * 32 * D; e += 256 * 8) {
            u32x4 v = u32x4{0, 0, 0, 0};
            if (e < hq) v = *reinterpret_cast<const u32x4*>(qsrc + e);
            *reinterpret_cast<u32x4*>(&s_q[(e / D) * QS + e % D]) = v;
        }
        for (int h = threadIdx.x; h < MB * 32; h += 256) s_w[h] = h < a.heads ? a.w[qr * a.heads + h] : 0.0f;
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

    // two accumulator sets: the MFMAs of sub-block u + 1 are issued before the
    // VALU epilogue of sub-block u, so the matrix and vector pipes overlap
    f32x16 acc0[MB], acc1[MB];
    float sc0 = 1.0f, sc1 = 1.0f;
    if (nsub > 0) mfma_stage(0, acc0, sc0);
    for (int32_t u = 0; u < nsub; u += 2) {
        if (u + 1 < nsub) mfma_stage(u + 1, acc1, sc1);
        epilogue(u, acc0, sc0);
        if (u + 1 >= nsub) break;
        if (u + 2 < nsub) mfma_stage(u + 2, acc0, sc0);
        epilogue(u + 1, acc1, sc1);
    }
    // drain the copies still in flight before the wave's LDS is released
    wait_vmcnt<0>();
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

// Lanes 0-31 get x + x[lane + 32] (v_permlane32_swap: its second result
// holds the upper half's values in the lower half).  The builtin exists for
// the device pass only.
__device__ __forceinline__ float add_upper_half(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                     false);
    return x + __uint_as_float(sw[1]);
#else
    return x;
#endif
}

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

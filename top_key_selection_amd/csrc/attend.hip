// attend.hip -- sparse attention over the selected keys on gfx950 (HISA
// abstract: the sparse attention reads only the entries the indexer keeps).
// The pages give no attention shapes; the form here has one shared K / V
// head of width 128 and H query heads:
//     p_j = softmax over valid slots j of scale * q[h] . k[idx_j]
//     o[h] = sum_j p_j v[idx_j]
//
// Split-K decoding: a workgroup owns one query row, 128 heads (16 per wave,
// so every gathered row is loaded once for all heads) and one split of 256
// slots, walked in chunks of 32 slots (the rows of the next two chunks load
// into registers while the current one is computed).  A chunk's key
// rows go to LDS (16-byte pieces, XOR-swizzled by row so the MFMA operand
// reads are conflict free) and its value rows to a transposed LDS tile
// (padded rows), which makes the value operand of P.V two 8-byte reads.
// Per wave and chunk:
//   S^T = K . Q^T   v_mfma_f32_16x16x32_bf16, keys as rows, heads as columns,
//                   so a head's scores sit in one lane column and its max /
//                   sum need two lane exchanges;
//   online softmax  exp2 against a reference moved only when a score exceeds
//                   it by more than 8 (O, l rescaled then), so most chunks
//                   skip the rescale;
//   O += P . V      P (bf16) is already in the A-operand layout once the
//                   key order of a 32-key step is permuted, and V is read in
//                   that order.
// The split's unnormalised O, running max and sum go to a workspace; a
// second kernel merges the splits.
#include <algorithm>

#include "tks_launch.hpp"

namespace tks {

namespace {

constexpr int kD = 128;          // key / value width
constexpr int kChunk = 32;       // slots per LDS chunk
constexpr int kSplit = 256;      // slots per workgroup
constexpr int kVtStride = kChunk + 8;  // bf16 per transposed value row (padded)

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;                 // 16 heads per wave
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsWg = kWaves * 16;

__global__ __launch_bounds__(kThreads, 2) void attend_split_kernel(AttnArgs a) {
    __shared__ __align__(16) uint8_t s_k[kChunk * kD * 2];          // swizzled key rows
    __shared__ __align__(16) __bf16 s_vt[kD * kVtStride];          // transposed value rows
    __shared__ int32_t s_valid[kChunk];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t row = blockIdx.x;
    const int32_t split = blockIdx.y;
    const int32_t head0 = blockIdx.z * kHeadsWg + wave * 16;
    const bool active = head0 < a.heads;
    const int32_t b = (int32_t)(row / a.n_q);
    const int32_t* idx_row = a.idx + row * a.topk;
    const int32_t slot0 = split * kSplit;
    const int32_t slot_end = min(a.topk, slot0 + kSplit);

    // Q^T fragments (B operand): head head0 + c16, dims ks * 32 + 8 g .. + 8
    bf16x8 qb[kD / 32];
    {
        const int h = active ? head0 + c16 : 0;
        const u32x4* p = reinterpret_cast<const u32x4*>(a.q + (row * a.heads + h) * kD + 8 * g);
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks) qb[ks] = __builtin_bit_cast(bf16x8, p[ks * 4]);
    }
    f32x4 o[kD / 16];
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt) o[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -__builtin_inff(), l_run = 0.0f;  // of head head0 + c16

    const float sl2 = a.scale * 1.4426950408889634f;  // scale * log2(e)
    // A chunk is kChunk rows x 16 pieces for K and for V: one K and one V
    // piece per thread, loaded into registers two chunks ahead of their use
    // (two register sets).  Wave w takes pieces 4 (w % 4) .. + 3 of rows
    // 16 (w / 4) .. + 15, 16 rows per instruction: the transposed value
    // writes then spread over 16 banks (4-way), the key writes over all.
    static_assert(kChunk * 16 == kThreads, "one piece per thread and chunk");
    const int lr = 16 * (wave >> 2) + (lane & 15), lc = 4 * (wave & 3) + (lane >> 4);
    struct Stage {
        u32x4 k, v;
        bool ok;
    };
    auto load_chunk = [&](Stage& sg, int32_t c0) {
        const int32_t slot = c0 + lr;
        const int32_t key = slot < slot_end ? idx_row[slot] : -1;
        sg.ok = key >= 0 && key < a.n_kv;
        // an empty slot reads key 0 (branch-free): its score is masked,
        // so its weight is 0 and its (finite) value row adds nothing
        const int64_t base = ((int64_t)b * a.n_kv + (sg.ok ? key : 0)) * kD + lc * 8;
        sg.k = *reinterpret_cast<const u32x4*>(a.k + base);
        sg.v = *reinterpret_cast<const u32x4*>(a.v + base);
    };
    auto compute_chunk = [&]() {
        // S^T: keys 16 mt + 4 g + i (rows) x heads c16 (columns)
        f32x4 s[kChunk / 16];
#pragma unroll
        for (int mt = 0; mt < kChunk / 16; ++mt) {
            s[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const int r = mt * 16 + c16;
#pragma unroll
            for (int ks = 0; ks < kD / 32; ++ks) {
                const int c = ks * 4 + g;
                const bf16x8 ka =
                    *reinterpret_cast<const bf16x8*>(s_k + r * (kD * 2) + ((c ^ (r & 15)) * 16));
                s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[ks], s[mt], 0, 0, 0);
            }
        }
        // online softmax of head c16 over this chunk, with a lazily moved
        // reference: the weights are 2^(s - m_run), and m_run (and O, l with
        // it) is only moved when a score exceeds it by more than 8, so the
        // weights stay below 2^8 and most chunks need no rescaling.  The
        // final normalisation makes the result independent of m_run.
        float cmax = -__builtin_inff();
#pragma unroll
        for (int mt = 0; mt < kChunk / 16; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = s_valid[mt * 16 + 4 * g + i] != 0;
                s[mt][i] = ok ? s[mt][i] * sl2 : -__builtin_inff();
                cmax = fmaxf(cmax, s[mt][i]);
            }
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        // a chunk without a valid key (the same for every head) adds nothing
        if (cmax == -__builtin_inff()) return;
        // the wave moves its references together (one branch for all heads)
        const bool move = cmax > m_run + 8.0f;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
            const float m_new = move ? cmax : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // m_run = -inf: 0
            l_run *= alpha;
            m_run = m_new;
            // O rows are heads 4 g + i: their alpha sits in lane column 4 g + i
            float al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
            for (int dt = 0; dt < kD / 16; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[dt][i] *= al[i];
        }
        float psum = 0.0f;
        bf16x8 pa[kChunk / 32];
#pragma unroll
        for (int mt = 0; mt < kChunk / 16; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(s[mt][i] - m_run);
                psum += (float)pb;  // the sum of the weights P.V uses
                pa[mt >> 1][(mt & 1) * 4 + i] = pb;
            }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        l_run += psum;
        // O += P . V; step kk covers keys 32 kk .. + 31, lane group g holding
        // keys 32 kk + 4 g + 0..3 and 32 kk + 16 + 4 g + 0..3
#pragma unroll
        for (int kk = 0; kk < kChunk / 32; ++kk) {
#pragma unroll
            for (int dt = 0; dt < kD / 16; ++dt) {
                const __bf16* vr = s_vt + (dt * 16 + c16) * kVtStride + 32 * kk + 4 * g;
                const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
                const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 16);
                bf16x8 vb;
                vb[0] = lo[0]; vb[1] = lo[1]; vb[2] = lo[2]; vb[3] = lo[3];
                vb[4] = hi[0]; vb[5] = hi[1]; vb[6] = hi[2]; vb[7] = hi[3];
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[kk], vb, o[dt], 0, 0, 0);
            }
        }
    };
    // chunk c0 from register set sg to LDS, the set refilled with chunk
    // c0 + 2 kChunk, then the chunk computed
    auto step = [&](Stage& sg, int32_t c0) {
        __syncthreads();  // the previous chunk's operands have been read
        *reinterpret_cast<u32x4*>(s_k + lr * (kD * 2) + ((lc ^ (lr & 15)) * 16)) = sg.k;
        const bf16x8 vb = __builtin_bit_cast(bf16x8, sg.v);
#pragma unroll
        for (int j = 0; j < 8; ++j) s_vt[(lc * 8 + j) * kVtStride + lr] = vb[j];
        if (lc == 0) s_valid[lr] = sg.ok ? 1 : 0;
        __syncthreads();
        if (c0 + 2 * kChunk < slot_end) load_chunk(sg, c0 + 2 * kChunk);  // in flight meanwhile
        if (active) compute_chunk();
    };
    if (a.n_kv > 0) {
        Stage s0, s1;
        if (slot0 < slot_end) load_chunk(s0, slot0);
        if (slot0 + kChunk < slot_end) load_chunk(s1, slot0 + kChunk);
        for (int32_t c0 = slot0; c0 < slot_end; c0 += 2 * kChunk) {
            step(s0, c0);
            if (c0 + kChunk >= slot_end) break;
            step(s1, c0 + kChunk);
        }
    }
    if (!active) return;
    // the split's partial: unnormalised O (heads 4 g + i, dims 16 dt + c16),
    // running max and sum (lane column c16, group 0)
    const int64_t part = (row * a.n_split + split) * a.heads;
#pragma unroll
    for (int dt = 0; dt < kD / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = head0 + 4 * g + i;
            if (h < a.heads) a.o_part[(part + h) * kD + dt * 16 + c16] = o[dt][i];
        }
    if (g == 0 && head0 + c16 < a.heads) {
        a.ml_part[(part + head0 + c16) * 2] = m_run;
        a.ml_part[(part + head0 + c16) * 2 + 1] = l_run;
    }
}

// o = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s with m the largest
// running max; zeros for a row without a valid key.  A workgroup merges
// four (row, head) pairs, 32 threads each with four dims; every split's
// partial is loaded before any is used (n_split <= kMaxSplits).
constexpr int kMaxSplits = 2048 / kSplit;
constexpr int kMergeHeads = 4;

__global__ __launch_bounds__(128) void attend_merge_kernel(AttnArgs a, int64_t n_rh) {
    const int64_t rh = (int64_t)blockIdx.x * kMergeHeads + (threadIdx.x >> 5);  // row * heads + h
    if (rh >= n_rh) return;
    const int d = (threadIdx.x & 31) * 4;
    const int64_t row = rh / a.heads;
    const int h = (int)(rh % a.heads);
    float ms[kMaxSplits], ls[kMaxSplits];
    f32x4 os[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        ms[s] = -__builtin_inff();
        ls[s] = 0.0f;
        os[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (s < a.n_split) {
            const int64_t p = (row * a.n_split + s) * a.heads + h;
            ms[s] = a.ml_part[p * 2];
            ls[s] = a.ml_part[p * 2 + 1];
            os[s] = *reinterpret_cast<const f32x4*>(a.o_part + p * kD + d);
        }
    }
    float m = -__builtin_inff();
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) m = fmaxf(m, ms[s]);
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float l = 0.0f;
    if (m != -__builtin_inff()) {
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s) {
            if (ms[s] == -__builtin_inff()) continue;
            const float f = exp2f(ms[s] - m);
            l += f * ls[s];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += f * os[s][i];
        }
    }
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = l > 0.0f ? acc[i] / l : 0.0f;
    float* op = a.out + rh * kD + d;
    if ((reinterpret_cast<uintptr_t>(a.out) & 15u) == 0) {
        *reinterpret_cast<f32x4*>(op) = o;
    } else {  // out need only be 4-byte aligned
#pragma unroll
        for (int i = 0; i < 4; ++i) op[i] = o[i];
    }
}

}  // namespace

size_t attend_workspace(int64_t rows, int32_t heads, int32_t topk) {
    const int64_t n_split = (topk + kSplit - 1) / kSplit;
    const int64_t part = rows * n_split * heads;
    return (size_t)((part * kD * 4 + 255) / 256 * 256 + (part * 2 * 4 + 255) / 256 * 256);
}

int32_t attend_splits(int32_t topk) { return (topk + kSplit - 1) / kSplit; }

hipError_t launch_attend(const AttnArgs& a, int64_t rows, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const dim3 g1((unsigned)rows, (unsigned)a.n_split, (unsigned)((a.heads + kHeadsWg - 1) / kHeadsWg));
    hipLaunchKernelGGL(attend_split_kernel, g1, dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(attend_merge_kernel, dim3((unsigned)((rows * a.heads + kMergeHeads - 1) / kMergeHeads)),
                       dim3(128), 0, stream, a, rows * (int64_t)a.heads);
    return hipGetLastError();
}

}  // namespace tks

// score_common.hpp -- device helpers of the MFMA indexer scoring (internal
// to the library): key fragments in the B-operand lane layout of
// v_mfma_f32_32x32x16_bf16, exact fp8 e4m3fn -> bf16 widening, the ReLU on
// the bit pattern and the lane-half sum.  Every scoring path uses these, so
// a (query, key) pair gets the same fp32 score whichever kernel computes it.
#pragma once

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

}  // namespace

}  // namespace tks

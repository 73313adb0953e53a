// fa_mfma.h -- matrix-core and LDS helpers shared by the tiled kernels
// (prefill, and the matrix-core decode of grouped query heads).
#pragma once

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <typename ST>
struct Mfma;
template <>
struct Mfma<BF16> {
    typedef bf16x8 V8;
    typedef __bf16 E;
    static __device__ __forceinline__ f32x16 mm(V8 a, V8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mfma<F16> {
    typedef f16x8 V8;
    typedef _Float16 E;
    static __device__ __forceinline__ f32x16 mm(V8 a, V8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// Two fp32 values -> one word of the 16-bit type (element 0 in the low
// half), rounded to nearest even, built as a two-element vector so the
// compiler emits one packed conversion where the target has it.
template <typename ST>
__device__ __forceinline__ uint32_t cvt_pair(float a, float b) {
    using E = typename Mfma<ST>::E;
    typedef E E2 __attribute__((ext_vector_type(2)));
    E2 v;
    v[0] = (E)a;
    v[1] = (E)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Logical work index for a launch slot.  Consecutive slots are dealt round
// robin to the 8 XCDs (each with its own L2); this remap gives every XCD a
// contiguous range of logical tiles, so the query tiles that read the same
// K/V head run on the same L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t slot, int64_t total) {
    const int64_t full = total & ~int64_t(7);
    if (slot >= full) return slot;
    return (slot & 7) * (full >> 3) + (slot >> 3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i%4 of the 8-byte pieces addressed by lanes
// i/4, i/4+4, i/4+8 and i/4+12 of its group.
__device__ __forceinline__ s16x4 lds_read_tr(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// 16-byte-chunk swizzle of the unpadded LDS rows (period 16 rows).  For both
// read patterns of the kernel the lanes served together hit distinct banks:
// 16 consecutive rows at one logical chunk (the K reads) and four consecutive
// rows x four consecutive chunks (the transposing V reads).
template <int D>
__device__ __forceinline__ int swz(int r) {
    // Rows of 256 and 512 bytes both start at bank 0, so D = 256 shares the
    // D = 128 pattern (it only permutes the low four chunk bits).
    if constexpr (D == 128 || D == 256) {
        return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    }
}

}  // namespace fa

// fa_device.h -- device helpers shared by the gfx950 attention kernels:
// 16-bit storage <-> fp32, wavefront reductions on DPP, exp2 with the log2(e)
// folded into the scale, 128-bit loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// Storage tags: the 16-bit type the tensors hold.
struct BF16 {
    static constexpr bool is_bf16 = true;
};
struct F16 {
    static constexpr bool is_bf16 = false;
};

// Low / high 16-bit halves of a packed word -> fp32 (exact for both types).
template <typename ST>
__device__ __forceinline__ float lo_f32(uint32_t w) {
    if constexpr (ST::is_bf16) {
        return __uint_as_float(w << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    }
}
template <typename ST>
__device__ __forceinline__ float hi_f32(uint32_t w) {
    if constexpr (ST::is_bf16) {
        return __uint_as_float(w & 0xffff0000u);
    } else {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
}

// Eight packed 16-bit values -> fp32[8].
template <typename ST>
__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = lo_f32<ST>(w[i]);
        f[2 * i + 1] = hi_f32<ST>(w[i]);
    }
}

// Dot product of eight packed 16-bit values with fp32 accumulation
// (v_dot2c_f32_{bf16,f16}: each step adds two exact products).
template <typename ST>
__device__ __forceinline__ float dot8(const u32x4 a, const u32x4 b) {
    // The pairs are taken with vector shuffles of the whole 8-element value:
    // bit-casting single 32-bit lanes of the 128-bit vector has been seen to
    // make the compiler read the first register of the tuple for every pair.
    float r = 0.f;
    if constexpr (ST::is_bf16) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 0, 1), __builtin_shufflevector(bv, bv, 0, 1), r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 2, 3), __builtin_shufflevector(bv, bv, 2, 3), r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 4, 5), __builtin_shufflevector(bv, bv, 4, 5), r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 6, 7), __builtin_shufflevector(bv, bv, 6, 7), r, false);
    } else {
        const f16x8 av = __builtin_bit_cast(f16x8, a), bv = __builtin_bit_cast(f16x8, b);
        r = __builtin_amdgcn_fdot2(__builtin_shufflevector(av, av, 0, 1), __builtin_shufflevector(bv, bv, 0, 1), r, false);
        r = __builtin_amdgcn_fdot2(__builtin_shufflevector(av, av, 2, 3), __builtin_shufflevector(bv, bv, 2, 3), r, false);
        r = __builtin_amdgcn_fdot2(__builtin_shufflevector(av, av, 4, 5), __builtin_shufflevector(bv, bv, 4, 5), r, false);
        r = __builtin_amdgcn_fdot2(__builtin_shufflevector(av, av, 6, 7), __builtin_shufflevector(bv, bv, 6, 7), r, false);
    }
    return r;
}

// fp32 -> 16-bit storage bits, round to nearest even.
template <typename ST>
__device__ __forceinline__ uint16_t to_bits(float x) {
    if constexpr (ST::is_bf16) {
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
}
template <typename ST>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)to_bits<ST>(a) | ((uint32_t)to_bits<ST>(b) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// DPP lane moves inside rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// Sum over aligned groups of N lanes (N in {8, 16, 32}); every lane gets the
// sum.  Inside 16-lane rows the steps are DPP moves; the step between two
// rows goes through a lane permute.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16 || N == 32, "group of 8, 16 or 32 lanes");
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppMirror>(x);
    if constexpr (N == 32) x += shfl_xor(x, 16);
    return x;
}

// x as a wave-uniform value (lane 0's): for values every lane computes alike
// that the compiler cannot prove uniform.
__device__ __forceinline__ int64_t uni64(int64_t x) {
    const uint64_t u = (uint64_t)x;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld128(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// The same load with the non-temporal hint, for data streamed once (kStreamAux).
__device__ __forceinline__ u32x4 ld128_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// x from lane (lane ^ 32): v_permlane32_swap exchanges the upper half-wave of
// its first operand with the lower half-wave of its second, without LDS.
__device__ __forceinline__ float xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Decode streams the KV cache once per call: its loads carry the
// non-temporal hint (cache policy bit "nt"), so the lines they bring in are
// the first the caches give up and the stream does not crowd out what is
// reused.  Measured on the 128K-token decode: 358 -> 324 us.
constexpr int kStreamAux = 2;

// Buffer resources: a base address and a byte range; a load at or past the
// range returns zeros.  The resource type exists only in the device pass.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, int nrec) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld128(buf_rsrc r, int voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kStreamAux));
}
#else
struct buf_rsrc {};
__device__ buf_rsrc make_rsrc(const void*, int);
__device__ u32x4 buf_ld128(buf_rsrc, int);
#endif

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS (buffer_load ... lds):
// lane i of the wave writes dst + 16*i (dst is wave-uniform).  Byte offsets at
// or past nrec read as zero through the buffer resource's range check.  The
// resource type exists only in the device compilation pass.  Used by the
// decode (streamed once: non-temporal, as buf_ld128).
__device__ __forceinline__ void lds_dma16(const void* base, int nrec, lds_void* dst, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, kStreamAux);
#endif
}

// The same load issued from inline assembly, for loops that order their tile
// loads themselves (an explicit vmcnt wait and a barrier before a tile is
// read).  Through the builtin the compiler sees an LDS write and, where it
// cannot prove that a later LDS read touches another buffer (or at a barrier's
// fence), waits for every load in flight, which stalls the next tile's
// prefetch behind the current tile's work.  Here the resource (built once per
// tile by make_dma_rsrc) and the LDS address are wave-uniform, and M0 carries
// the LDS address as the instruction requires.
typedef uint32_t dma_rsrc __attribute__((ext_vector_type(4)));
__device__ __forceinline__ dma_rsrc make_dma_rsrc(const void* base, int nrec) {
    const uint64_t p = (uint64_t)base;
    dma_rsrc r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) & 0xffffu;  // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((uint32_t)nrec);
    r[3] = 0x00020000u;
    return r;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16_unordered(dma_rsrc r, lds_void* dst, int voff) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m), "v"(voff), "s"(r)
                 : "memory", "m0");
}
// The same load with M0 given as a wave-uniform LDS byte address computed
// beforehand (see lds_address), so a loop issuing tile loads spends only the
// M0 write on it.
__device__ __forceinline__ void lds_dma16_m0(dma_rsrc r, uint32_t m0, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "memory", "m0");
}
// The same as lds_dma16_unordered for data read once (non-temporal), as the
// decode's K/V stream: nothing the compiler tracks, so it places no wait on it.
__device__ __forceinline__ void lds_dma16_stream(dma_rsrc r, lds_void* dst, int voff) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(m), "v"(voff), "s"(r)
                 : "memory", "m0");
}
// Four bytes per lane (lane i's dword lands at M0 + 4i).
__device__ __forceinline__ void lds_dma4_m0(dma_rsrc r, uint32_t m0, int voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a __shared__ object, as a wave-uniform value.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)p);
}

}  // namespace fa

// dtype.hpp -- element types of the pools: raw storage words, conversions to
// and from fp32 (round to nearest even), quiet NaN, and the gfx950 MFMA
// 16x16x32 instruction for the 16-bit types.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lora {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT>
struct Elem;

template <>
struct Elem<DT_F32> {
    using raw = uint32_t;
    static constexpr raw qnan = 0x7FC00000u;
    static __device__ __forceinline__ float to_f(raw b) { return __uint_as_float(b); }
    static __device__ __forceinline__ raw from_f(float f) { return __float_as_uint(f); }
};

template <>
struct Elem<DT_F16> {
    using raw = uint16_t;
    using vec8 = f16x8_t;
    static constexpr raw qnan = 0x7E00u;
    static __device__ __forceinline__ float to_f(raw b) {
        return static_cast<float>(__builtin_bit_cast(_Float16, b));
    }
    static __device__ __forceinline__ raw from_f(float f) {
        return __builtin_bit_cast(raw, static_cast<_Float16>(f));
    }
    static __device__ __forceinline__ f32x4_t mfma(vec8 a, vec8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Elem<DT_BF16> {
    using raw = uint16_t;
    using vec8 = bf16x8_t;
    static constexpr raw qnan = 0x7FC0u;
    static __device__ __forceinline__ float to_f(raw b) {
        return __uint_as_float(static_cast<uint32_t>(b) << 16);
    }
    static __device__ __forceinline__ raw from_f(float f) {
        uint32_t u = __float_as_uint(f);
        if ((u & 0x7FFFFFFFu) > 0x7F800000u) return qnan;
        u += 0x7FFFu + ((u >> 16) & 1u);
        return static_cast<raw>(u >> 16);
    }
    static __device__ __forceinline__ f32x4_t mfma(vec8 a, vec8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// A value every lane of the wave holds, moved to a scalar register so that
// the compiler sees it as uniform: branches on it become scalar branches.
// Control flow around MFMA must be uniform in that sense -- MFMA does not
// honour EXEC, so an MFMA in a lane-masked block still executes.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 16-byte load of eight 16-bit elements as an MFMA operand.
template <typename V>
__device__ __forceinline__ V load8(const uint16_t *p) {
    return __builtin_bit_cast(V, *reinterpret_cast<const u32x4_t *>(p));
}

// Raw buffer resource over [base, base + bytes) (gfx9 family descriptor,
// word 3 = 0x00020000).  Loads through it address base + soffset + voffset +
// immediate; voffset + immediate at or past `bytes` read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}

// Cache-policy operand of the buffer memory intrinsics on gfx950: bit 4
// (sc1) makes a load or store coherent at agent scope -- a store is written
// through to the device's coherence point, a load does not use a copy that
// another XCD's writes could have made stale.
constexpr int CPOL_SC1 = 16;

// 16-byte buffer load as an MFMA operand (byte offsets).
template <typename V>
__device__ __forceinline__ V bload8(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(voff),
                                                                        static_cast<int>(soff), 0));
}

template <typename V>
__device__ __forceinline__ V zero8() {
    return __builtin_bit_cast(V, u32x4_t{0u, 0u, 0u, 0u});
}

}  // namespace lora

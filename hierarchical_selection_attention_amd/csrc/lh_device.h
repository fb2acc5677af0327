// Device-side helpers for the gfx950 kernels: vector types, bf16 conversion,
// wavefront shuffles.  Wave size is 64 on CDNA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lh {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// bf16 bits -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 8 consecutive elements of a row as fp32.  bf16: one 16-byte load; fp32: two.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&x)[8]) {
    if constexpr (DT == 0) {
        u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w[i]);
            x[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem);
        f32x4 a = p[0], b = p[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = a[i];
            x[4 + i] = b[i];
        }
    }
}

// Same as load8 with non-temporal loads: streamed inputs that are read once.
template <int DT>
__device__ __forceinline__ void load8_nt(const void* base, int64_t elem, float (&x)[8]) {
    if constexpr (DT == 0) {
        u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w[i]);
            x[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem);
        f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = a[i];
            x[4 + i] = b[i];
        }
    }
}

// Raw buffer resource over `bytes` bytes from `base` (no stride; dword3 value
// for the gfx9 family).  Loads through it take a scalar base, a per-lane 32-bit
// offset and a uniform scalar offset, so per-token addresses cost no VGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16-byte non-temporal load (cache policy bit 1 = nt) at lane offset + uniform offset.
__device__ __forceinline__ u32x4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
}

// Store of 8 elements in the I/O dtype; NT selects non-temporal stores.
template <int DT, bool NT = false>
__device__ __forceinline__ void store8(void* base, int64_t elem, const float (&x)[8]) {
    if constexpr (DT == 0) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        u32x4* p = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + elem);
        if constexpr (NT) __builtin_nontemporal_store(w, p);
        else *p = w;
    } else {
        f32x4* p = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + elem);
        const f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
        if constexpr (NT) {
            __builtin_nontemporal_store(a, p);
            __builtin_nontemporal_store(b, p + 1);
        } else {
            p[0] = a;
            p[1] = b;
        }
    }
}

__device__ __forceinline__ void load8f(const float* base, int64_t elem, float (&x)[8]) {
    const f32x4* p = reinterpret_cast<const f32x4*>(base + elem);
    f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
    }
}
__device__ __forceinline__ void store8f(float* base, int64_t elem, const float (&x)[8]) {
    f32x4* p = reinterpret_cast<f32x4*>(base + elem);
    p[0] = f32x4{x[0], x[1], x[2], x[3]};
    p[1] = f32x4{x[4], x[5], x[6], x[7]};
}

// 8 fp32 values with non-temporal stores
__device__ __forceinline__ void store8f_nt(float* base, int64_t elem, const float (&x)[8]) {
    f32x4* p = reinterpret_cast<f32x4*>(base + elem);
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, p);
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, p + 1);
}

// 8 bf16 values packed in 4 dwords -> fp32, exact.
__device__ __forceinline__ void unpack8(const u32x4& w, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(w[i]);
        x[2 * i + 1] = bf16_hi(w[i]);
    }
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// Value of lane (lane ^ OFF) for OFF in {1, 2, 4, 8, 16}: DPP quad permutes for
// 1 and 2, ds_swizzle (bit mode, xor mask) for 4..16.  Exact moves.
template <int OFF>
__device__ __forceinline__ float xor_lane(float v) {
    const int b = __float_as_int(v);
    int r;
    if constexpr (OFF == 1) r = __builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, false);       // [1,0,3,2]
    else if constexpr (OFF == 2) r = __builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
    else r = __builtin_amdgcn_ds_swizzle(b, (OFF << 10) | 0x1F);
    return __int_as_float(r);
}

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48),
// with the gfx950 row-swap permutes: permlane16_swap(v, v) yields the values of
// lanes l & ~16 and l | 16, permlane32_swap(v, v) those of l & ~32 and l | 32.
// Every lane receives the result; the pairing is the same on all lanes.
__device__ __forceinline__ float rows4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x with the hardware instruction (no denormal rescaling: results below the
// normal range flush to zero, which softmax weights tolerate).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace lh

// gdn_device.h -- device helpers shared by the libgdn kernels (gfx950 only).
//
// bf16 <-> fp32 conversion, 16-byte vector loads for fp32 / bf16 tensors, and
// cross-lane sums over aligned groups of 4..64 lanes of a 64-wide wavefront
// built from DPP row permutes and ds_swizzle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef uint16_t bf16_t;

struct alignas(16) f4 {
    float x, y, z, w;
};

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest, ties to even; NaN stays NaN (the hardware conversion,
// one instruction)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// ---- element-type traits -------------------------------------------------
template <typename T> struct io;

template <> struct io<float> {
    static __device__ __forceinline__ float ld(const float* p) { return *p; }
    static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
    // four consecutive elements (16-byte aligned)
    static __device__ __forceinline__ f4 ld4(const float* p) {
        return *reinterpret_cast<const f4*>(p);
    }
    static __device__ __forceinline__ void st4(float* p, f4 v) {
        *reinterpret_cast<f4*>(p) = v;
    }
};

template <> struct io<bf16_t> {
    static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
    // four consecutive elements (8-byte aligned)
    static __device__ __forceinline__ f4 ld4(const bf16_t* p) {
        uint2 u = *reinterpret_cast<const uint2*>(p);
        f4 r;
        r.x = __uint_as_float(u.x << 16);
        r.y = __uint_as_float(u.x & 0xffff0000u);
        r.z = __uint_as_float(u.y << 16);
        r.w = __uint_as_float(u.y & 0xffff0000u);
        return r;
    }
    static __device__ __forceinline__ void st4(bf16_t* p, f4 v) {
        uint2 u;
        u.x = static_cast<uint32_t>(f32_to_bf16(v.x)) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
        u.y = static_cast<uint32_t>(f32_to_bf16(v.z)) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
        *reinterpret_cast<uint2*>(p) = u;
    }
};

// explicit fused multiply-adds: every kernel that uses it rounds the same way,
// whatever the compiler would contract in its context
__device__ __forceinline__ float dot4(f4 a, f4 b) {
    return __builtin_fmaf(a.w, b.w, __builtin_fmaf(a.z, b.z, __builtin_fmaf(a.y, b.y, a.x * b.x)));
}

// ---- cross-lane sums -------------------------------------------------------
// DPP control codes (GFX9 encoding)
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// lane i <- lane i ^ 16 within each half-wave (ds_swizzle, bitmask mode)
__device__ __forceinline__ float swz_xor16(float x) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

__device__ __forceinline__ float xor32(float x) {
    return __shfl_xor(x, 32, 64);
}

// Sum over each aligned group of W lanes; every lane of the group gets the sum.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "W");
    if constexpr (W >= 2) x += dpp<kDppQuadXor1>(x);
    if constexpr (W >= 4) x += dpp<kDppQuadXor2>(x);
    if constexpr (W >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (W >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (W >= 32) x += swz_xor16(x);
    if constexpr (W >= 64) x += xor32(x);
    return x;
}

}  // namespace gdn

// gdn_prefill_common.h -- device helpers shared by the chunked-prefill
// kernels on MFMA (gfx950): LDS and buffer-resource loads and stores, the
// hardware exp2 of log2-unit decays, and the sequence / chunk lookups of a
// packed batch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_device.h"
#include "gdn_mfma.h"

namespace gdn {

__device__ __forceinline__ bf8_t lds8(const __bf16* p) {
    return *reinterpret_cast<const bf8_t*>(p);
}

__device__ __forceinline__ bf8_t gld8(const uint16_t* p) {
    return __builtin_bit_cast(bf8_t, *reinterpret_cast<const uint4*>(p));
}

// Raw buffer stores: an offset at or past num_records is dropped by the
// hardware, which masks rows past a sequence's end without a branch (a branch
// around a store would make the compiler wait for every outstanding load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void out_store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v, float*) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)(off * 4), 0, 0);
}
__device__ __forceinline__ void out_store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v, bf16_t*) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, (int)(off * 2), 0, 0);
}

__device__ __forceinline__ void out_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v, float*) {
    typedef unsigned u4_t __attribute__((ext_vector_type(4)));
    const u4_t d = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(d, r, (int)(off * 4), 0, 0);
}
// (bf16: the hardware's packed round-to-nearest-even conversion, the same
// result as f32_to_bf16 for every number, a quiet NaN for a NaN)
__device__ __forceinline__ void out_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v, bf16_t*) {
    typedef unsigned u2_t __attribute__((ext_vector_type(2)));
    const u2_t d = {__builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{v[0], v[1]}, bf2_t)),
                    __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{v[2], v[3]}, bf2_t))};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, (int)(off * 2), 0, 0);
}

// exponentials of log-decay differences: G is kept in log2 units (g log2 e),
// so e^{G_t - G_s} is one hardware exp2
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2f_(float x) { return __builtin_amdgcn_exp2f(x); }


__device__ __forceinline__ void seq_bounds_m(const int32_t* cu, int n, int T, int& s, int& e) {
    int a = cu[n], b = cu[n + 1];
    a = min(max(a, 0), T);
    b = min(max(b, a), T);
    s = a;
    e = b;
}

__device__ __forceinline__ int find_seq_m(const int32_t* chunk_off, int N, int c) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= c) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ float4 in_load4(__amdgpu_buffer_rsrc_t r, uint32_t off_elems) {
    typedef unsigned u4_t __attribute__((ext_vector_type(4)));
    const u4_t u = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off_elems * 4), 0, 0));
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}
__device__ __forceinline__ void load4_any(__amdgpu_buffer_rsrc_t r, uint32_t off, float* v, float*) {
    const float4 x = in_load4(r, off);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
__device__ __forceinline__ void load4_any(__amdgpu_buffer_rsrc_t r, uint32_t off, float* v, bf16_t*) {
    typedef unsigned u2_t __attribute__((ext_vector_type(2)));
    const u2_t u = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)(off * 2), 0, 0));
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
}

}  // namespace gdn

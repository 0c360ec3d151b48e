// gdn_mfma.h -- bf16 MFMA helpers shared by the prefill and attention kernels
// (gfx950).
//
// v_mfma_f32_16x16x32_bf16: lane l of a wavefront holds, for the A operand,
// row (l % 16) and the 8 consecutive k at 8 (l / 16); for B, column (l % 16)
// and the same 8 k; the 4 accumulators are rows 4 (l / 16) + r, column l % 16.
// fp32 operands enter as hi + lo bf16 pairs (x = hi + lo to 2^-16 relative).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f4_t mfma(bf8_t a, bf8_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// two floats -> packed hi and lo bf16 words: hi = bf16(x) (one packed
// conversion); x - hi in fp32 straight from the packed hi, as a bf16 dot
// product with (-1, 0) or (0, -1) accumulated onto x (one v_dot2c per value:
// x - bf16(x) is exact in fp32, so the dot's rounding never acts); lo =
// bf16(x - hi) (one conversion).  Four instructions per pair, against six
// when hi is widened back to fp32 by a shift and a mask and subtracted.  The
// two bf16 pairs are moved into scalar registers by hand: given as constants,
// the compiler folds (-1, 0) into an inline immediate that the hardware reads
// as (0, -1) (an in-bounds probe on gfx950: every lane wrong with the folded
// constant, every lane equal to the subtraction with the register).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    uint32_t m0, m1;
    asm("s_mov_b32 %0, 0xbf80" : "=s"(m0));      // bf16 (-1, 0)
    asm("s_mov_b32 %0, 0xbf800000" : "=s"(m1));  // bf16 (0, -1)
    const bf2_t h = __builtin_convertvector(f2_t{x0, x1}, bf2_t);
    const float d0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf2_t, m0), x0, false);
    const float d1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf2_t, m1), x1, false);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{d0, d1}, bf2_t));
}
// fp32 x -> (hi, lo) with hi = bf16(x), lo = bf16(x - hi): 4 or 8 values
__device__ __forceinline__ void split4(const float* x, uint2& hi, uint2& lo) {
    split2(x[0], x[1], hi.x, lo.x);
    split2(x[2], x[3], hi.y, lo.y);
}
__device__ __forceinline__ void split8(const float* x, bf8_t& hi, bf8_t& lo) {
    uint4 h, o;
    split2(x[0], x[1], h.x, o.x);
    split2(x[2], x[3], h.y, o.y);
    split2(x[4], x[5], h.z, o.z);
    split2(x[6], x[7], h.w, o.w);
    hi = __builtin_bit_cast(bf8_t, h);
    lo = __builtin_bit_cast(bf8_t, o);
}

// Raw buffer loads: a resource that covers exactly the valid rows makes rows
// past the end read as zero without a clamp or a select.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t in_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ bf8_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf8_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

}  // namespace gdn

// gdn_rmsnorm.hip -- RMSNormGated (gfx950).
//
// The norm that closes each DeltaNet layer (Qwen3.5-0.8B chat guide,
// section "Architektur"), per (row, head) group of dv values:
//
//     y = x / sqrt(mean(x^2) + eps) * w * silu(z),   silu(z) = z / (1 + e^-z)
//
// A group is spread over dv/4 lanes holding four consecutive values each; the
// sum of squares is a DPP / swizzle group sum.  A workgroup takes two runs of
// consecutive groups and loads both before it computes and stores either;
// x, z and y are each touched once, so their loads and stores are
// non-temporal (measured at the 0.8B prefill output shape, 16384 x 16 groups
// of 128: 61-64 us with one run and ordinary accesses, 56 us like this; four
// runs 59 us).  Each lane reads its x before it writes y, so y may alias x.
// Bound by HBM (read x and z, write y).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef float nv4f __attribute__((ext_vector_type(4)));
typedef unsigned nv2u __attribute__((ext_vector_type(2)));

// four consecutive elements, non-temporal (16-byte aligned fp32, 8-byte bf16)
__device__ __forceinline__ f4 ld4_nt(const float* p) {
    const nv4f v = __builtin_nontemporal_load(reinterpret_cast<const nv4f*>(p));
    return f4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ f4 ld4_nt(const bf16_t* p) {
    const nv2u u = __builtin_nontemporal_load(reinterpret_cast<const nv2u*>(p));
    return f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
              __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ void st4_nt(float* p, f4 v) {
    __builtin_nontemporal_store(nv4f{v.x, v.y, v.z, v.w}, reinterpret_cast<nv4f*>(p));
}
__device__ __forceinline__ void st4_nt(bf16_t* p, f4 v) {
    const nv2u u = {static_cast<uint32_t>(f32_to_bf16(v.x)) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16),
                    static_cast<uint32_t>(f32_to_bf16(v.z)) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16)};
    __builtin_nontemporal_store(u, reinterpret_cast<nv2u*>(p));
}
__device__ __forceinline__ f4 ld4_any_nt(const void* p, size_t i, bool bf16) {
    return bf16 ? ld4_nt(static_cast<const bf16_t*>(p) + i) : ld4_nt(static_cast<const float*>(p) + i);
}
__device__ __forceinline__ f4 ld4_any(const void* p, size_t i, bool bf16) {
    return bf16 ? io<bf16_t>::ld4(static_cast<const bf16_t*>(p) + i)
                : io<float>::ld4(static_cast<const float*>(p) + i);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

constexpr int kNormPasses = 2;

template <int DV, typename Tx, typename Ty>
__global__ __launch_bounds__(256) void rmsnorm_gated_kernel(const Tx* x, const void* z,
                                                            const void* w, Ty* y, long groups,
                                                            float eps, int z_bf16, int w_bf16) {
    constexpr int LPG = DV / 4;       // lanes per group
    constexpr int GPB = 256 / LPG;    // groups per pass of a block
    constexpr int P = kNormPasses;
    const long g0 = (long)blockIdx.x * (GPB * P) + threadIdx.x / LPG;
    const int c = 4 * (threadIdx.x % LPG);
    f4 xv[P], zv[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const long gi = g0 + (long)p * GPB;
        const size_t off = (size_t)(gi < groups ? gi : 0) * DV + c;
        xv[p] = ld4_nt(x + off);
        zv[p] = ld4_any_nt(z, off, z_bf16 != 0);
    }
    const f4 wv = ld4_any(w, c, w_bf16 != 0);
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const long gi = g0 + (long)p * GPB;
        const float ss = group_sum<LPG>(dot4(xv[p], xv[p]));
        const float inv = 1.0f / sqrtf(ss * (1.0f / DV) + eps);
        f4 yv;
        yv.x = xv[p].x * inv * wv.x * silu(zv[p].x);
        yv.y = xv[p].y * inv * wv.y * silu(zv[p].y);
        yv.z = xv[p].z * inv * wv.z * silu(zv[p].z);
        yv.w = xv[p].w * inv * wv.w * silu(zv[p].w);
        if (gi < groups) st4_nt(y + (size_t)gi * DV + c, yv);
    }
}

template <int DV, typename Tx, typename Ty>
static hipError_t launch_norm_t(const NormArgs& A) {
    constexpr int GPB = 256 / (DV / 4) * kNormPasses;
    const size_t blocks = ((size_t)A.groups + GPB - 1) / GPB;
    hipLaunchKernelGGL((rmsnorm_gated_kernel<DV, Tx, Ty>), dim3((unsigned)blocks), dim3(256), 0,
                       A.stream, static_cast<const Tx*>(A.x), A.z, A.w, static_cast<Ty*>(A.y),
                       A.groups, A.eps, (int)A.z_bf16, (int)A.w_bf16);
    return hipGetLastError();
}

template <typename Tx, typename Ty>
static hipError_t launch_norm_io(const NormArgs& A) {
    switch (A.dv) {
        case 16: return launch_norm_t<16, Tx, Ty>(A);
        case 32: return launch_norm_t<32, Tx, Ty>(A);
        case 64: return launch_norm_t<64, Tx, Ty>(A);
        default: return launch_norm_t<128, Tx, Ty>(A);
    }
}

hipError_t launch_rmsnorm_gated(const NormArgs& A) {
    if (A.x_bf16) return A.y_bf16 ? launch_norm_io<bf16_t, bf16_t>(A) : launch_norm_io<bf16_t, float>(A);
    return A.y_bf16 ? launch_norm_io<float, bf16_t>(A) : launch_norm_io<float, float>(A);
}

}  // namespace gdn

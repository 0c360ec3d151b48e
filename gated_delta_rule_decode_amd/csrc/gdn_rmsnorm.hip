// gdn_rmsnorm.hip -- RMSNormGated (gfx950).
//
// The norm that closes each DeltaNet layer (Qwen3.5-0.8B chat guide,
// section "Architektur"), per (row, head) group of dv values:
//
//     y = x / sqrt(mean(x^2) + eps) * w * silu(z),   silu(z) = z / (1 + e^-z)
//
// A group is spread over dv/4 lanes holding four consecutive values each; the
// sum of squares is a DPP / swizzle group sum.  Each lane reads its x before it
// writes y, so y may alias x.  Bound by HBM (read x and z, write y).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <typename T>
__device__ __forceinline__ f4 ld4_any(const void* p, size_t i, bool bf16) {
    return bf16 ? io<bf16_t>::ld4(static_cast<const bf16_t*>(p) + i)
                : io<float>::ld4(static_cast<const float*>(p) + i);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

template <int DV, typename Tx, typename Ty>
__global__ __launch_bounds__(256) void rmsnorm_gated_kernel(const Tx* x, const void* z,
                                                            const void* w, Ty* y, long groups,
                                                            float eps, int z_bf16, int w_bf16) {
    constexpr int LPG = DV / 4;       // lanes per group
    constexpr int GPB = 256 / LPG;    // groups per block
    const long gi = (long)blockIdx.x * GPB + threadIdx.x / LPG;
    const int c = 4 * (threadIdx.x % LPG);
    const bool ok = gi < groups;
    const size_t off = (size_t)(ok ? gi : 0) * DV + c;
    f4 xv = io<Tx>::ld4(x + off);
    f4 zv = ld4_any<float>(z, off, z_bf16 != 0);
    f4 wv = ld4_any<float>(w, c, w_bf16 != 0);
    const float ss = group_sum<LPG>(dot4(xv, xv));
    const float inv = 1.0f / sqrtf(ss * (1.0f / DV) + eps);
    f4 yv;
    yv.x = xv.x * inv * wv.x * silu(zv.x);
    yv.y = xv.y * inv * wv.y * silu(zv.y);
    yv.z = xv.z * inv * wv.z * silu(zv.z);
    yv.w = xv.w * inv * wv.w * silu(zv.w);
    if (ok) io<Ty>::st4(y + off, yv);
}

template <int DV, typename Tx, typename Ty>
static hipError_t launch_norm_t(const NormArgs& A) {
    constexpr int GPB = 256 / (DV / 4);
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

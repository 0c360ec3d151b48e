// gdn_decode.hip -- one-token decode of the gated delta rule (gfx950).
//
// Per (sequence n, value head h) the state S (dv x dk fp32, row-major in k) is
// advanced by one token (Gated Delta Networks, Yang et al., ICLR 2025; the
// single-step, state-owning decoder of the Qwen3.5-0.8B Core ML card, section
// "Model"):
//
//     S' = a S (I - b k k^T) + b v k^T,     o = scale * S' q
//
// Rows of S are independent once k, q, a, b are known.  With u = S k and
// r = S q taken from the OLD state in one read:
//
//     delta = b (v - a u)          (per row)
//     S'    = a S + delta k^T
//     o     = scale (a r + (k.q) delta)      since S' q = a S q + delta (k^T q)
//
// so each state element is read once and written once, by the same lane.
//
// Mapping.  A workgroup owns BV consecutive rows of one (n, h) state (a tile
// of BV * dk * 4 bytes).  A row is spread over LPR = dk/4 lanes holding four
// consecutive floats each, so one wavefront load instruction covers 256
// contiguous floats (1 KiB, fully coalesced).  The workgroup loads its whole
// tile (PASSES loads per lane) before any arithmetic, reduces u and r across
// the LPR lanes of a row with DPP / swizzle sums, and stores the tile back.
// The kernel is bound by HBM: 8 * dk * dv bytes of state traffic per
// (sequence, head) against ~6 * dk * dv flops.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef float v4f __attribute__((ext_vector_type(4)));

template <int DK, int BV, int NT, typename Tin, typename Tout>
__global__ __launch_bounds__(NT) void decode_kernel(const Tin* __restrict__ q,
                                                    const Tin* __restrict__ k,
                                                    const Tin* __restrict__ v,
                                                    const float* __restrict__ g,
                                                    const float* __restrict__ beta,
                                                    float* __restrict__ state,
                                                    Tout* __restrict__ o, int H, int HV, int dv,
                                                    float scale) {
    constexpr int LPR = DK / 4;       // lanes per state row
    constexpr int RPP = NT / LPR;     // rows per pass of the workgroup
    constexpr int PASSES = BV / RPP;  // 16-byte loads per lane
    static_assert(RPP * PASSES == BV && NT % 64 == 0, "tile shape");

    const int tiles = dv / BV;
    const int bid = blockIdx.x;
    const int tile = bid % tiles;
    const int nh = bid / tiles;  // n * HV + h
    const int n = nh / HV;
    const int h = nh - n * HV;
    const int hk = h / (HV / H);
    const int lc = threadIdx.x % LPR;  // column group: columns 4*lc .. 4*lc+3
    const int lr = threadIdx.x / LPR;  // row within a pass

    float* S = state + ((size_t)nh * dv + (size_t)tile * BV) * DK + 4 * lc;

    // the whole tile first: PASSES independent 16-byte loads in flight per lane
    v4f s[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        s[p] = *reinterpret_cast<const v4f*>(S + (size_t)(p * RPP + lr) * DK);

    const size_t qk = ((size_t)n * H + hk) * DK + 4 * lc;
    const f4 k4 = io<Tin>::ld4(k + qk);
    const f4 q4 = io<Tin>::ld4(q + qk);
    const Tin* vrow = v + (size_t)nh * dv + (size_t)tile * BV + lr;
    float vv[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) vv[p] = io<Tin>::ld(vrow + p * RPP);
    const float a = expf(g[nh]);
    const float b = beta[nh];

    const float kq = group_sum<LPR>(dot4(k4, q4));

    float u[PASSES], r[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        u[p] = s[p].x * k4.x + s[p].y * k4.y + s[p].z * k4.z + s[p].w * k4.w;
        r[p] = s[p].x * q4.x + s[p].y * q4.y + s[p].z * q4.z + s[p].w * q4.w;
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        u[p] = group_sum<LPR>(u[p]);
        r[p] = group_sum<LPR>(r[p]);
    }

    Tout* orow = o + (size_t)nh * dv + (size_t)tile * BV + lr;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const float delta = b * (vv[p] - a * u[p]);
        v4f sn;
        sn.x = a * s[p].x + delta * k4.x;
        sn.y = a * s[p].y + delta * k4.y;
        sn.z = a * s[p].z + delta * k4.z;
        sn.w = a * s[p].w + delta * k4.w;
        *reinterpret_cast<v4f*>(S + (size_t)(p * RPP + lr) * DK) = sn;
        if (lc == 0) io<Tout>::st(orow + p * RPP, scale * (a * r[p] + kq * delta));
    }
}

template <int DK, int BV, typename Tin, typename Tout>
static hipError_t launch_decode_t(const DecodeArgs& A) {
    constexpr int LPR = DK / 4;
    constexpr int PASSES = (BV * LPR > 256) ? (BV * LPR / 256) : 1;
    constexpr int NT = BV * LPR / PASSES;
    const int tiles = A.dv / BV;
    const size_t blocks = (size_t)A.N * A.HV * tiles;
    hipLaunchKernelGGL((decode_kernel<DK, BV, NT, Tin, Tout>), dim3((unsigned)blocks), dim3(NT),
                       0, A.stream, static_cast<const Tin*>(A.q), static_cast<const Tin*>(A.k),
                       static_cast<const Tin*>(A.v), A.g, A.beta, A.state,
                       static_cast<Tout*>(A.o), A.H, A.HV, A.dv, A.scale);
    return hipGetLastError();
}

template <int DK, typename Tin, typename Tout>
static hipError_t launch_decode_dk(const DecodeArgs& A) {
    if (A.dv == 16) return launch_decode_t<DK, 16, Tin, Tout>(A);
    return launch_decode_t<DK, 32, Tin, Tout>(A);
}

template <typename Tin, typename Tout>
static hipError_t launch_decode_io(const DecodeArgs& A) {
    switch (A.dk) {
        case 16: return launch_decode_dk<16, Tin, Tout>(A);
        case 32: return launch_decode_dk<32, Tin, Tout>(A);
        case 64: return launch_decode_dk<64, Tin, Tout>(A);
        default: return launch_decode_dk<128, Tin, Tout>(A);
    }
}

hipError_t launch_decode(const DecodeArgs& A) {
    if (A.in_bf16) {
        return A.o_bf16 ? launch_decode_io<bf16_t, bf16_t>(A) : launch_decode_io<bf16_t, float>(A);
    }
    return A.o_bf16 ? launch_decode_io<float, bf16_t>(A) : launch_decode_io<float, float>(A);
}

}  // namespace gdn

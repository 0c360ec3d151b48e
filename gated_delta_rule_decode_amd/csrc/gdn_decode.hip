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
// Mapping.  A workgroup owns BV consecutive rows of one (n, h) state.  A row is
// spread over LPR = dk/4 lanes holding four consecutive floats each, so one
// wavefront load covers 256 contiguous floats (1 KiB).  The workgroup loads its
// whole tile (PASSES 16-byte loads per lane) before any arithmetic, reduces u
// and r across the LPR lanes of a row with DPP / swizzle sums, and stores the
// tile back.  State loads and stores are non-temporal: the state of a layer
// is touched once per token, so it should not displace other data from the
// L2 and the Infinity Cache (measured: 4.6 -> 5.4 TB/s on the 0.8B shape).
// The kernel is bound by HBM: 8 dk dv bytes of state traffic per (sequence,
// head) against about 6 dk dv flops.
//
// The fused variant owns a whole head (BV = dv) so that it can finish with
// RMSNormGated (Qwen3.5-0.8B chat guide, section "Architektur") over the dv
// outputs of the head: y = o / sqrt(mean(o^2) + eps) * w * silu(z).
//
// The layer variant (EXT) is the serving form of the same step: the state of
// sequence n lives in slot slots[n] of a pool (a slot outside the pool skips
// the sequence and writes zero outputs), the gates may arrive as raw
// projections (g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b), the
// Gated DeltaNet layer's parameterisation) and q, k may be L2-normalised in
// the kernel: x / sqrt(sum x^2 + eps), one cross-lane sum per vector.  The
// extras touch only per-head scalars and the q/k vectors, so the state sweep
// is unchanged.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f ld_state(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
}
__device__ __forceinline__ void st_state(float* p, v4f v) {
    __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p));
}

// The streamed schedule addresses the tile through a buffer resource and
// writes with sc0 sc1 nt (streaming, written through to memory): measured
// about 3% faster than nt global stores on grids of several rounds.
constexpr int kCpolNt = 2, kCpolSc0Sc1Nt = 19;
__device__ __forceinline__ v4f ld_state_rs(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNt));
}
__device__ __forceinline__ void st_state_rs(__amdgpu_buffer_rsrc_t r, int off, v4f v) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, off, 0, kCpolSc0Sc1Nt);
}

// s . x for a row piece, as explicit fused multiply-adds (the same rounding in
// every variant of the kernel, so the fused and plain steps agree bit for bit)
__device__ __forceinline__ float dot4s(v4f s, f4 x) {
    return __builtin_fmaf(s.w, x.w, __builtin_fmaf(s.z, x.z, __builtin_fmaf(s.y, x.y, s.x * x.x)));
}

template <typename T>
__device__ __forceinline__ float ld_any(const void* p, size_t i, bool bf16) {
    return bf16 ? bf16_to_f32(static_cast<const bf16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// Element i of an fp32 or bf16 array with one 4-byte load and no branch: the
// aligned dword that holds the element (in bounds for arrays of even length;
// z and w have dv, an even count, per row).
__device__ __forceinline__ float ld_any_nb(const void* p, size_t i, bool bf16) {
    const size_t byte = bf16 ? i * 2 : i * 4;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(p) + (byte & ~size_t(3)));
    const uint32_t hi = (byte & 2) ? (w & 0xffff0000u) : (w << 16);
    return __uint_as_float(bf16 ? hi : w);
}

// Per-head scalars (uniform over the workgroup, never written by the kernel):
// read through the constant address space so they come in by scalar loads,
// which the vector-memory counter does not wait for.
typedef const __attribute__((address_space(4))) float cfloat_t;
typedef const __attribute__((address_space(4))) uint32_t cu32_t;
__device__ __forceinline__ float ld_uniform(const float* p, size_t i) {
    return ((cfloat_t*)(uintptr_t)p)[i];
}
// Element i of an element-aligned fp32 or bf16 array of n elements.  A bf16
// element comes from a scalar load of the dword that holds it, its half chosen
// by the element's address (a bf16 array need only be 2-byte aligned, e.g. a
// per-step slice of an odd-length buffer), when that dword lies inside the
// array; the first or last element of an array whose ends are not
// dword-aligned takes a 16-bit vector load instead.
__device__ __forceinline__ float ld_gate(const void* p, size_t i, size_t n, bool bf16) {
    if (!bf16) return ld_uniform(static_cast<const float*>(p), i);
    const uintptr_t base = (uintptr_t)p, a = base + 2 * i;
    const uintptr_t a4 = a & ~(uintptr_t)3;
    if (a4 >= base && a4 + 4 <= base + 2 * n) {
        const uint32_t w = *(cu32_t*)a4;
        return __uint_as_float((a & 2) ? (w & 0xffff0000u) : (w << 16));
    }
    return bf16_to_f32(static_cast<const bf16_t*>(p)[i]);
}
template <typename T>
__device__ __forceinline__ void st_any(void* p, size_t i, float v, bool bf16) {
    if (bf16) static_cast<bf16_t*>(p)[i] = f32_to_bf16(v);
    else static_cast<float*>(p)[i] = v;
}

// FUSE:   finish with RMSNormGated over the head (requires BV == dv).
// EXT:    slot table, raw gates, q/k L2 norm.
// STREAM: store each pass as soon as it is computed (grids of several rounds
//         of workgroups); otherwise read the whole tile before the first store
//         (a single round: HBM then serves the reads and the writes of the
//         launch in two phases instead of mixing them).
template <int DK, int BV, int NT, typename Tin, bool FUSE, bool EXT, bool STREAM>
__global__ __launch_bounds__(NT) void decode_kernel(const DecodeArgs A) {
    constexpr int LPR = DK / 4;       // lanes per state row
    constexpr int RPP = NT / LPR;     // rows per pass of the workgroup
    constexpr int PASSES = BV / RPP;  // 16-byte loads per lane
    static_assert(RPP * PASSES == BV && NT % 64 == 0, "tile shape");
    const Tin* __restrict__ q = static_cast<const Tin*>(A.q);
    const Tin* __restrict__ k = static_cast<const Tin*>(A.k);
    const Tin* __restrict__ v = static_cast<const Tin*>(A.v);
    const int dv = A.dv, H = A.H, HV = A.HV;

    const int tiles = dv / BV;
    const int bid = blockIdx.x;
    const int tile = bid % tiles;
    const int nh = bid / tiles;  // n * HV + h
    const int n = nh / HV;
    const int h = nh - n * HV;
    const int hk = h / (HV / H);
    const int lc = threadIdx.x % LPR;  // column group: columns 4*lc .. 4*lc+3
    const int lr = threadIdx.x / LPR;  // row within a pass

    const size_t row0 = (size_t)nh * dv + (size_t)tile * BV + lr;  // this lane's first row
    // per-row inputs: lane lc < PASSES of a row group loads the values of its
    // row group's pass lc (one memory instruction for all passes); v is then
    // broadcast to the whole row group, z and w stay with that lane, which
    // also finishes the row (o, y) for pass lc.
    const bool owner = lc < PASSES;
    const size_t myrow = row0 + (size_t)(owner ? lc : 0) * RPP;

    int slot = n;
    if constexpr (EXT) {
        if (A.slots) slot = A.slots[n];
        if ((unsigned)slot >= (unsigned)A.num_slots) {  // skipped sequence: zero outputs
            if (owner) {
                if (A.o) st_any<float>(A.o, myrow, 0.f, A.o_bf16);
                if constexpr (FUSE) st_any<float>(A.y, myrow, 0.f, A.y_bf16);
            }
            return;  // uniform over the workgroup
        }
    }
    const size_t sh = EXT ? (size_t)slot * HV + h : (size_t)nh;  // state head in the pool
    float* S = A.state + (sh * dv + (size_t)tile * BV) * DK + 4 * lc;
    // streamed schedule: the tile as a buffer (BV rows of DK floats)
    __amdgpu_buffer_rsrc_t rs;
    if constexpr (STREAM)
        rs = __builtin_amdgcn_make_buffer_rsrc(A.state + (sh * dv + (size_t)tile * BV) * DK,
                                               (short)0, BV * DK * 4, 0x00020000);

    v4f s[PASSES];
    f4 k4, q4;
    float vmine, zmine = 0.f, wmine = 0.f, graw, braw;
    if constexpr (STREAM) {
        // per-token inputs first, so that waiting for them does not wait for
        // the state tile (vector-memory loads complete in issue order); the
        // per-head scalars come in by scalar loads
        const size_t qk = ((size_t)n * H + hk) * DK + 4 * lc;
        k4 = io<Tin>::ld4(k + qk);
        q4 = io<Tin>::ld4(q + qk);
        vmine = io<Tin>::ld(v + myrow);
        if constexpr (FUSE) {
            zmine = ld_any_nb(A.z, myrow, A.z_bf16);
            wmine = ld_any_nb(A.w, (size_t)lr + (owner ? lc : 0) * RPP, A.w_bf16);
        }
        if (EXT && A.a_raw) {
            const size_t ngate = (size_t)A.N * HV;
            graw = ld_gate(A.a_raw, nh, ngate, A.gate_bf16) +
                   (A.dt_bias ? ld_uniform(A.dt_bias, h) : 0.f);
            braw = ld_gate(A.b_raw, nh, ngate, A.gate_bf16);
        } else {
            graw = ld_uniform(A.g, nh);
            braw = ld_uniform(A.beta, nh);
        }
        // then the whole state tile: PASSES independent 16-byte loads per lane
#pragma unroll
        for (int p = 0; p < PASSES; ++p) s[p] = ld_state_rs(rs, (16 * lc) + (p * RPP + lr) * DK * 4);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads together, ahead of the arithmetic
    } else {
        // the whole state tile first: PASSES independent 16-byte loads per lane
#pragma unroll
        for (int p = 0; p < PASSES; ++p) s[p] = ld_state(S + (size_t)(p * RPP + lr) * DK);
        const size_t qk = ((size_t)n * H + hk) * DK + 4 * lc;
        k4 = io<Tin>::ld4(k + qk);
        q4 = io<Tin>::ld4(q + qk);
        vmine = io<Tin>::ld(v + myrow);
        if constexpr (FUSE) {
            zmine = ld_any<float>(A.z, myrow, A.z_bf16);
            wmine = ld_any<float>(A.w, (size_t)lr + (owner ? lc : 0) * RPP, A.w_bf16);
        }
        if (EXT && A.a_raw) {
            graw = ld_any<float>(A.a_raw, nh, A.gate_bf16) + (A.dt_bias ? A.dt_bias[h] : 0.f);
            braw = ld_any<float>(A.b_raw, nh, A.gate_bf16);
        } else {
            graw = A.g[nh];
            braw = A.beta[nh];
        }
    }

    float a, b;
    if (EXT && A.a_raw) {
        const float sp = fmaxf(graw, 0.f) + log1pf(expf(-fabsf(graw)));  // softplus
        a = expf(-expf(STREAM ? ld_uniform(A.A_log, h) : A.A_log[h]) * sp);
        b = 1.0f / (1.0f + expf(-braw));
    } else {
        a = expf(graw);
        b = braw;
    }
    if (EXT && A.l2norm) {
        const float kn = 1.0f / sqrtf(group_sum<LPR>(dot4(k4, k4)) + A.l2_eps);
        const float qn = 1.0f / sqrtf(group_sum<LPR>(dot4(q4, q4)) + A.l2_eps);
        k4.x *= kn; k4.y *= kn; k4.z *= kn; k4.w *= kn;
        q4.x *= qn; q4.y *= qn; q4.z *= qn; q4.w *= qn;
    }
    const int gbase = (threadIdx.x & 63) & ~(LPR - 1);  // first lane of this row group in the wave
    float vv[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) vv[p] = __shfl(vmine, gbase + p, 64);

    const float kq = group_sum<LPR>(dot4(k4, q4));

    // STREAM: each pass is finished and stored as soon as its rows arrive.
    // Otherwise every row's reductions come first, so the workgroup stores
    // nothing before its whole tile has been read.
    float u[PASSES], r[PASSES];
    if constexpr (!STREAM) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            u[p] = dot4s(s[p], k4);
            r[p] = dot4s(s[p], q4);
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            u[p] = group_sum<LPR>(u[p]);
            r[p] = group_sum<LPR>(r[p]);
        }
        // every row's sums before the first store: the wavefront's stores then
        // leave as one burst (measured 12.3 -> 11.9 us per launch on the
        // 0.8B job, where the compiler had spread them over the sums)
        __builtin_amdgcn_sched_barrier(0);
    }
    float ov[PASSES];
    float omine = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        if constexpr (STREAM) {
            u[p] = group_sum<LPR>(dot4s(s[p], k4));
            r[p] = group_sum<LPR>(dot4s(s[p], q4));
        }
        const float delta = b * __builtin_fmaf(-a, u[p], vv[p]);
        v4f sn;
        sn.x = __builtin_fmaf(delta, k4.x, a * s[p].x);
        sn.y = __builtin_fmaf(delta, k4.y, a * s[p].y);
        sn.z = __builtin_fmaf(delta, k4.z, a * s[p].z);
        sn.w = __builtin_fmaf(delta, k4.w, a * s[p].w);
        if constexpr (STREAM)
            st_state_rs(rs, (16 * lc) + (p * RPP + lr) * DK * 4, sn);
        else
            st_state(S + (size_t)(p * RPP + lr) * DK, sn);
        ov[p] = A.scale * __builtin_fmaf(kq, delta, a * r[p]);
        omine = (lc == p) ? ov[p] : omine;
    }
    if (A.o && owner) st_any<float>(A.o, myrow, omine, A.o_bf16);
    if constexpr (FUSE) {
        // sum of o^2 over the head's dv rows: every lane of a row group holds
        // the same PASSES outputs; take one lane per row group
        __shared__ float part[NT / 64];
        float ss = 0.f;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) ss += ov[p] * ov[p];
        ss = (lc == 0) ? ss : 0.f;
        ss = group_sum<64>(ss);
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) tot += part[i];
        const float inv = 1.0f / sqrtf(tot * (1.0f / BV) + A.eps);
        if (owner) {
            const float y = omine * inv * wmine * (zmine / (1.0f + expf(-zmine)));
            st_any<float>(A.y, myrow, y, A.y_bf16);
        }
    }
}

// The fused kernel (eight 16-byte state loads per lane) streams its stores
// from this many workgroups on (several rounds on the 256 CUs; measured 2-4%
// faster there, 5-10% slower on a single round).  The unfused kernel, two
// loads per lane, keeps the two-phase schedule at every size.
constexpr size_t kStreamMinBlocks = 1024;

template <int DK, int BV, typename Tin, bool FUSE, bool EXT>
static hipError_t launch_decode_t(const DecodeArgs& A) {
    constexpr int LPR = DK / 4;
    constexpr int LIMIT = FUSE ? 512 : 256;  // threads per workgroup
    constexpr int PASSES = (BV * LPR > LIMIT) ? (BV * LPR / LIMIT) : 1;
    constexpr int NT = BV * LPR / PASSES;
    const int tiles = A.dv / BV;
    const size_t blocks = (size_t)A.N * A.HV * tiles;
    if (FUSE && blocks >= kStreamMinBlocks)
        hipLaunchKernelGGL((decode_kernel<DK, BV, NT, Tin, FUSE, EXT, true>), dim3((unsigned)blocks),
                           dim3(NT), 0, A.stream, A);
    else
        hipLaunchKernelGGL((decode_kernel<DK, BV, NT, Tin, FUSE, EXT, false>), dim3((unsigned)blocks),
                           dim3(NT), 0, A.stream, A);
    return hipGetLastError();
}

template <int DK, typename Tin, bool EXT>
static hipError_t launch_decode_dk(const DecodeArgs& A) {
    if (A.fuse_norm) {
        switch (A.dv) {
            case 16: return launch_decode_t<DK, 16, Tin, true, EXT>(A);
            case 32: return launch_decode_t<DK, 32, Tin, true, EXT>(A);
            case 64: return launch_decode_t<DK, 64, Tin, true, EXT>(A);
            default: return launch_decode_t<DK, 128, Tin, true, EXT>(A);
        }
    }
    return launch_decode_t<DK, 16, Tin, false, EXT>(A);
}

template <typename Tin, bool EXT>
static hipError_t launch_decode_in(const DecodeArgs& A) {
    switch (A.dk) {
        case 16: return launch_decode_dk<16, Tin, EXT>(A);
        case 32: return launch_decode_dk<32, Tin, EXT>(A);
        case 64: return launch_decode_dk<64, Tin, EXT>(A);
        default: return launch_decode_dk<128, Tin, EXT>(A);
    }
}

hipError_t launch_decode(const DecodeArgs& A) {
    if (A.ext)
        return A.in_bf16 ? launch_decode_in<bf16_t, true>(A) : launch_decode_in<float, true>(A);
    return A.in_bf16 ? launch_decode_in<bf16_t, false>(A) : launch_decode_in<float, false>(A);
}

}  // namespace gdn

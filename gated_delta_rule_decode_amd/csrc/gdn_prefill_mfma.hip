// gdn_prefill_mfma.hip -- chunked prefill on bf16 MFMA (gfx950, bf16 inputs).
//
// Same chunkwise form as gdn_prefill.hip (gated delta rule, Yang et al., ICLR
// 2025): per chunk of C = 64 tokens with cumulative log-decays G,
//
//     A_ts = b_t e^{G_t - G_s} k_t.k_s (s < t),   T' = (I + A)^-1 diag(b)
//     P_ts = e^{G_t - G_s} q_t.k_s (s <= t)
//     X    = V - diag(e^G) K S^T                  U  = T' X
//     O    = scale (diag(e^G) Q S^T + P U)
//     S'   = e^{G_n} S + U'^T K,                  U' = diag(e^{G_n - G}) U
//
// Every contraction runs on v_mfma_f32_16x16x32_bf16 (16 x 16 output tile,
// K = 32).  Lane l of a wavefront holds, for the A operand, row (l % 16) and
// the 8 consecutive k at 8 (l / 16); for B, column (l % 16) and the same 8 k;
// the 4 accumulators are rows 4 (l / 16) + r, column (l % 16).
//
// Precision.  q, k, v arrive as bf16 and enter the products exactly.  Every
// fp32 operand (S, X, U, U', P, T') is split into hi + lo bf16 (x = hi + lo up
// to 2^-16 relative); a product with an exact bf16 operand takes two MFMAs
// (hi, lo), a product of two split operands three (hi.hi + hi.lo + lo.hi).
// Accumulation is fp32 and the state between chunks stays fp32 in the
// accumulators of the update product.
//
// Work split.  What does not depend on the state runs chunk-parallel in
// prep_mfma, one workgroup per (chunk, value head): G, K K^T, Q K^T, the
// triangular inverse T' and the two state-free products R = P T' and
// Z^T = K^T diag(e^{G_n - G}) T', stored pre-split as hi/lo bf16 in the
// scan's operand order.  The sequential scan_mfma runs the rest:
// K S^T, Q S^T, X = V - diag(gamma) K S^T, O = scale (diag(gamma) Q S^T + R X)
// and S' = gamma_n S + Z^T X, with the state in MFMA accumulators.
#include <algorithm>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_prefill_common.h"

namespace gdn {


// ---------------------------------------------------------------------------
// prep: everything that does not depend on the state, chunk-parallel
// ---------------------------------------------------------------------------
// One workgroup (4 wavefronts) per (chunk, value head).  Wave w owns row block
// w (tokens 16 w .. 16 w + 15).  It produces
//   G   in-chunk cumulative log-decay (log2 units)
//   R   = P T'                          64 x 64, row t, column c   (hi / lo bf16)
//   Z^T = K^T diag(e^{G_n - G}) T'      dk x 64, row j, column c   (hi / lo bf16)
// with P = lower(Q K^T o Gamma) and T' = (I + A)^-1 diag(b), so that the scan
// only needs O = scale (diag(gamma) Q S^T + R X) and S' = gamma_n S + Z^T X.
// Rows and columns past the sequence end come out as exact zeros (K, Q and b
// read as zero there, so T' vanishes outside the valid block).  R and Z^T are
// stored in the scan's operand order: fragment f of a 64 x 64 (or dk x 64)
// plane is 1 KiB, lane l of the consuming wavefront reads bytes 16 l .. 16 l + 15,
// which hold row 16 (f / 2) + l % 16, columns 32 (f % 2) + 8 (l / 16) .. + 7.

// One workgroup per (chunk, value head): K K^T and Q K^T are computed again for
// every value head of a key head.  That costs a few MFMAs and an L2 re-read of
// K and Q, and nothing lives across value heads, so the kernel needs 70 VGPRs
// (196 when a workgroup looped over the value heads of its key head) and LDS
// alone sets the occupancy at three workgroups per CU.
template <int DK>
__global__ __launch_bounds__(256) void prep_mfma_kernel(const PrefillArgs A) {
    constexpr int C = kChunk;
    constexpr int KP = DK + 8;   // padded bf16 row of the K and Q tiles
    constexpr int AP = C + 4;    // padded fp32 row (16-byte aligned rows)
    constexpr int NKK = DK / 32;
    constexpr int PPR = DK / 8;         // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;       // rows per coalesced 1 KiB load
    constexpr int NLD = 16 / RPI;       // loads per wavefront per tile
    // LDS, 35,584 bytes at d_k = 128 (four workgroups per CU).  Beside K, one
    // 64 x 64 fp32 buffer holds in turn Q (needed only for the first
    // products), A, T = (I + A)^-1 written over A block by block (every block
    // of A is read before its place is written), and T'^T (T staged through
    // registers first).  The 32-block merge's X lives in the upper-right block,
    // which neither A nor T (lower triangular) uses.  G, b and e^{G_n - G}
    // are held for the value head.
    static_assert(C * KP * 2 <= C * AP * 4, "Q fits in the buffer of A and T");
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * KP];
    __shared__ __attribute__((aligned(16))) float Bf[C * AP];  // Q, A, T, then T'^T
    __shared__ __attribute__((aligned(16))) float Gs[C];
    __shared__ __attribute__((aligned(16))) float Bs[C];
    __shared__ __attribute__((aligned(16))) float Ds[C];
    __bf16* const Qs = reinterpret_cast<__bf16*>(Bf);
    float* const Am = Bf;        // A (lower blocks), later T'^T
    float* const Tm = Bf;        // T, rows 0 .. 63, lower triangle
    float* const Xm = Bf + 32;   // X [32 x 32], rows 0 .. 31, columns 32 .. 63

    const int H = A.H, HV = A.HV;
    const int c = blockIdx.x, tid = threadIdx.x;
    const int hv = blockIdx.y, hk = hv / (A.HV / A.H);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(w >= 0 && w < 4);
    const int l = tid & 63, lr = l & 15, lg = l >> 4;
    const int total = min(A.chunk_off[A.N], A.max_chunks);
    if (c >= total) return;
    const int n = find_seq_m(A.chunk_off, A.N, c);
    int s0, e0;
    seq_bounds_m(A.cu_seqlens, n, A.T, s0, e0);
    const int t0 = s0 + (c - A.chunk_off[n]) * C;
    const int L = min(C, e0 - t0);

    // ---- every global load first: K and Q rows of this wave (coalesced), g and b ----
    const uint32_t qk_row = (uint32_t)H * DK * 2;
    const __amdgpu_buffer_rsrc_t rk =
        in_rsrc(static_cast<const bf16_t*>(A.k) + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
    const __amdgpu_buffer_rsrc_t rq =
        in_rsrc(static_cast<const bf16_t*>(A.q) + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
    bf8_t kst[NLD], qst[NLD];
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
        const int row = 16 * w + RPI * p + l / PPR;
        const uint32_t off = ((uint32_t)row * H + hk) * DK * 2 + 16 * (l % PPR);
        kst[p] = bload8(rk, off);
        qst[p] = bload8(rq, off);
    }
    // wave 0: g and b of the value head for token l (zero past the end)
    float gv = 0.f, bv = 0.f;
    if (w == 0) {
        const __amdgpu_buffer_rsrc_t rg = in_rsrc(A.g + (size_t)t0 * HV, (uint32_t)L * HV * 4);
        const __amdgpu_buffer_rsrc_t rb = in_rsrc(A.beta + (size_t)t0 * HV, (uint32_t)L * HV * 4);
        gv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, (int)((l * HV + hv) * 4), 0, 0));
        bv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (int)((l * HV + hv) * 4), 0, 0));
    }
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
        const int at = (16 * w + RPI * p + l / PPR) * KP + 8 * (l % PPR);
        *reinterpret_cast<bf8_t*>(&Ks[at]) = kst[p];
        *reinterpret_cast<bf8_t*>(&Qs[at]) = qst[p];
    }
    // G (log2 units, inclusive in-chunk prefix sum) and the end decays e^{G_n - G}
    if (w == 0) {
        float gs = gv * kLog2e;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(gs, off, 64);
            if (l >= off) gs += up;
        }
        const float gn = __shfl(gs, L - 1, 64);
        Gs[l] = gs;
        Bs[l] = bv;
        Ds[l] = exp2f_(gn - gs);
        A.ws_G[((size_t)c * HV + hv) * C + l] = gs;
    }
    __syncthreads();

    // K K^T (row block w against column blocks sb <= w) and the raw P^T tiles
    //   kk[sb][r] = (K K^T)[t = 16 w + 4 lg + r][s = 16 sb + lr]
    //   pq[sb][r] = (Q K^T)[t = 16 w + lr][s = 16 sb + 4 lg + r]
    f4_t kk[4], pq[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        kk[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
        pq[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < NKK; ++ks) {
        const int col = 32 * ks + 8 * lg;
        bf8_t kb[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) kb[sb] = lds8(&Ks[(16 * sb + lr) * KP + col]);
        const bf8_t ka = lds8(&Ks[(16 * w + lr) * KP + col]);
        const bf8_t qa = lds8(&Qs[(16 * w + lr) * KP + col]);
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if (sb <= w) {
                kk[sb] = mfma(ka, kb[sb], kk[sb]);
                pq[sb] = mfma(kb[sb], qa, pq[sb]);
            }
        }
    }
    // selectors for K^T fragments: (K I)[s][j] picks column j of K exactly;
    // sel[h] holds the 32 x 16 identity block for the column half h of a k-step
    bf8_t sel[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int y = 0; y < 8; ++y)
            sel[h][y] = static_cast<__bf16>((8 * lg + y == 16 * h + lr) ? 1.f : 0.f);

    __syncthreads();  // every wavefront has read Q: A takes its place
    {
        const float* G = Gs;
        // A = strictly lower part of diag(b) (K K^T o e^{G_t - G_s}); branch-free: the
        // exponent is clamped at 0 (only s < t is kept, where it is <= 0 anyway)
        // and the mask multiplies
        {
            const float4 g4 = *reinterpret_cast<const float4*>(&G[16 * w + 4 * lg]);
            const float4 b4 = *reinterpret_cast<const float4*>(&Bs[16 * w + 4 * lg]);
            const float gt[4] = {g4.x, g4.y, g4.z, g4.w};
            const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (sb <= w) {
                    const float Gsb = G[16 * sb + lr];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * w + 4 * lg + r, s = 16 * sb + lr;
                        const float keep = (s < t) ? 1.f : 0.f;
                        Am[t * AP + s] = keep * bt[r] * exp2f_(fminf(gt[r] - Gsb, 0.f)) * kk[sb][r];
                    }
                }
            }
        }
        __syncthreads();
        // diagonal blocks T_bb = (I + A_bb)^-1 by forward substitution:
        // wave b, lane j < 16 owns column j, rows of A_bb preloaded
        if (l < 16) {
            const int o = 16 * w;
            float col[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float arow[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    if (4 * q4 < t) {
                        const float4 a4 = *reinterpret_cast<const float4*>(&Am[(o + t) * AP + o + 4 * q4]);
                        arow[4 * q4] = a4.x; arow[4 * q4 + 1] = a4.y;
                        arow[4 * q4 + 2] = a4.z; arow[4 * q4 + 3] = a4.w;
                    }
                }
                float v = (t == l) ? 1.f : 0.f;
#pragma unroll
                for (int x = 0; x < t; ++x) v -= arow[x] * col[x];
                col[t] = v;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) Tm[(o + t) * AP + o + l] = col[t];
        }
        __syncthreads();
        // 16-block merges on MFMA, one per wavefront (0 and 1):
        //   T_{ii,j} = -T_{ii,ii} (A_{ii,j} T_{jj}),  (ii, j) = (1, 0), (3, 2).
        // The 16-long contraction fills slots 0..3 of each lane group (slots 4..7
        // are zero), so the first product's accumulators (rows 4 lg + r, column
        // lr) are exactly the second product's B operand.
        if (w < 2) {
            const int j = 2 * w, ii = j + 1;
            const float4 a4 = *reinterpret_cast<const float4*>(&Am[(16 * ii + lr) * AP + 16 * j + 4 * lg]);
            float av[8] = {a4.x, a4.y, a4.z, a4.w, 0.f, 0.f, 0.f, 0.f};
            float bv8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int y = 0; y < 4; ++y) bv8[y] = Tm[(16 * j + 4 * lg + y) * AP + 16 * j + lr];
            bf8_t ah, al, bh, bl;
            split8(av, ah, al);
            split8(bv8, bh, bl);
            f4_t xa = f4_t{0.f, 0.f, 0.f, 0.f};  // xa[r] = (A_{ii,j} T_{jj})[4 lg + r][lr]
            xa = mfma(ah, bh, xa);
            xa = mfma(ah, bl, xa);
            xa = mfma(al, bh, xa);
            const float4 t4 = *reinterpret_cast<const float4*>(&Tm[(16 * ii + lr) * AP + 16 * ii + 4 * lg]);
            float tv[8] = {t4.x, t4.y, t4.z, t4.w, 0.f, 0.f, 0.f, 0.f};
            float xv[8] = {xa[0], xa[1], xa[2], xa[3], 0.f, 0.f, 0.f, 0.f};
            split8(tv, ah, al);
            split8(xv, bh, bl);
            f4_t ta = f4_t{0.f, 0.f, 0.f, 0.f};
            ta = mfma(ah, bh, ta);
            ta = mfma(ah, bl, ta);
            ta = mfma(al, bh, ta);
#pragma unroll
            for (int r = 0; r < 4; ++r) Tm[(16 * ii + 4 * lg + r) * AP + 16 * j + lr] = -ta[r];
        }
        __syncthreads();
        // 32-block merge on MFMA: X = A[32:64, 0:32] T[0:32, 0:32]; T[32:64, 0:32] = -T_B X
        {
            const int tbm = w >> 1, jb = w & 1;
            float av[8], bv8[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                av[x] = Am[(32 + 16 * tbm + lr) * AP + 8 * lg + x];
                const int xr = 8 * lg + x, cc = 16 * jb + lr;
                bv8[x] = (xr >= cc) ? Tm[xr * AP + cc] : 0.f;
            }
            bf8_t ah, al, bh, bl;
            split8(av, ah, al);
            split8(bv8, bh, bl);
            f4_t xa = f4_t{0.f, 0.f, 0.f, 0.f};
            xa = mfma(ah, bh, xa);
            xa = mfma(ah, bl, xa);
            xa = mfma(al, bh, xa);
#pragma unroll
            for (int r = 0; r < 4; ++r) Xm[(16 * tbm + 4 * lg + r) * AP + 16 * jb + lr] = xa[r];
        }
        __syncthreads();
        {
            const int tbm = w >> 1, jb = w & 1;
            float av[8], bv8[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const int rr = 16 * tbm + lr, xc = 8 * lg + x;  // T_B row rr, column xc (lower)
                av[x] = (xc <= rr) ? Tm[(32 + rr) * AP + 32 + xc] : 0.f;
                bv8[x] = Xm[(8 * lg + x) * AP + 16 * jb + lr];
            }
            bf8_t ah, al, bh, bl;
            split8(av, ah, al);
            split8(bv8, bh, bl);
            f4_t ta = f4_t{0.f, 0.f, 0.f, 0.f};
            ta = mfma(ah, bh, ta);
            ta = mfma(ah, bl, ta);
            ta = mfma(al, bh, ta);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Tm[(32 + 16 * tbm + 4 * lg + r) * AP + 16 * jb + lr] = -ta[r];
        }
        __syncthreads();
        // T'^T[c][s] = T[s][c] b_c (zero for s < c) in T's place: each thread
        // reads its pieces of T (row s, columns c4 .. c4 + 3), then, after a
        // barrier, writes their transposes
        constexpr int NTP = C * C / 4 / 256;
        float4 tq[NTP];
#pragma unroll
        for (int it = 0; it < NTP; ++it) {
            const int idx = tid + 256 * it, s_ = idx & 63, c4 = 4 * (idx >> 6);
            tq[it] = *reinterpret_cast<const float4*>(&Tm[s_ * AP + c4]);
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < NTP; ++it) {
            const int idx = tid + 256 * it, s_ = idx & 63, c4 = 4 * (idx >> 6);
            const float tv[4] = {tq[it].x, tq[it].y, tq[it].z, tq[it].w};
            const float4 b4 = *reinterpret_cast<const float4*>(&Bs[c4]);
            const float bc[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)  // a select, not a 0/1 factor: T's upper blocks hold other data
                Am[(c4 + r) * AP + s_] = (s_ >= c4 + r) ? tv[r] * bc[r] : 0.f;
        }
        __syncthreads();

        // R^T tiles (c block cb, t block w) = T'^T P^T: A = T'^T rows in the slot
        // order of the P^T fragments, B = decayed and masked P^T (this wave's t)
        {
            const size_t rbase = ((size_t)c * HV + hv) * C * C;
            const int t = 16 * w + lr;
            const float Gt = G[t];
            bf8_t ph[2], pl[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                float pv[8];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int sb = 2 * k2 + half;
                    const float4 g4 = *reinterpret_cast<const float4*>(&G[16 * sb + 4 * lg]);
                    const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int s_ = 16 * sb + 4 * lg + r;
                        const float keep = (s_ <= t) ? 1.f : 0.f;
                        pv[4 * half + r] = keep * pq[sb][r] * exp2f_(fminf(Gt - gs[r], 0.f));
                    }
                }
                split8(pv, ph[k2], pl[k2]);
            }
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                f4_t ra = f4_t{0.f, 0.f, 0.f, 0.f};
                if (cb <= w) {
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) {
                        if (2 * k2 <= w) {
                            const float* arow = &Am[(16 * cb + lr) * AP + 32 * k2 + 4 * lg];
                            const float4 a0 = *reinterpret_cast<const float4*>(arow);
                            const float4 a1 = *reinterpret_cast<const float4*>(arow + 16);
                            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                            bf8_t ah, al;
                            split8(av, ah, al);
                            ra = mfma(ah, ph[k2], ra);
                            ra = mfma(ah, pl[k2], ra);
                            ra = mfma(al, ph[k2], ra);
                        }
                    }
                }
                // ra[r] = R[t = 16 w + lr][c = 16 cb + 4 lg + r]: fragment (w, cb / 2),
                // lane 16 (2 (cb & 1) + lg / 2) + lr, elements 4 (lg & 1) .. + 3
                const float rv[4] = {ra[0], ra[1], ra[2], ra[3]};
                uint2 hi, lo;
                split4(rv, hi, lo);
                const size_t off = rbase + (size_t)((2 * w + (cb >> 1)) * 64 +
                                                    16 * (2 * (cb & 1) + (lg >> 1)) + lr) * 8 +
                                   4 * (lg & 1);
                *reinterpret_cast<uint2*>(A.ws_Rh + off) = hi;
                *reinterpret_cast<uint2*>(A.ws_Rl + off) = lo;
            }
        }
        // Z tiles (c block w, j block jb) = (T'^T diag(e^{G_n - G})) K with the
        // contraction over s in the slot order s = 32 k2 + 4 lg + (0..3) and
        // 32 k2 + 16 + 4 lg + (0..3); the K operand in that order comes from
        // selection products (K I) of two K row blocks.  T'^T row 16 w + lr is zero
        // before column 16 w, so k-steps start at w / 2.
        {
            const size_t zbase = ((size_t)c * HV + hv) * DK * C;
            bf8_t ah[2], al[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const float* arow = &Am[(16 * w + lr) * AP + 32 * k2 + 4 * lg];
                const float* drow = &Ds[32 * k2 + 4 * lg];
                const float4 a0 = *reinterpret_cast<const float4*>(arow);
                const float4 a1 = *reinterpret_cast<const float4*>(arow + 16);
                const float4 d0 = *reinterpret_cast<const float4*>(drow);
                const float4 d1 = *reinterpret_cast<const float4*>(drow + 16);
                const float av[8] = {a0.x * d0.x, a0.y * d0.y, a0.z * d0.z, a0.w * d0.w,
                                     a1.x * d1.x, a1.y * d1.y, a1.z * d1.z, a1.w * d1.w};
                split8(av, ah[k2], al[k2]);
            }
#pragma unroll
            for (int jb = 0; jb < DK / 16; ++jb) {
                f4_t za = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    if (k2 >= (w >> 1)) {
                        bf8_t kb;
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const int sb = 2 * k2 + half;
                            const bf8_t krow = lds8(&Ks[(16 * sb + lr) * KP + 32 * (jb >> 1) + 8 * lg]);
                            // tr[r] = K[16 sb + 4 lg + r][16 jb + lr] (exact)
                            const f4_t tr = mfma(krow, sel[jb & 1], f4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                            for (int r = 0; r < 4; ++r) kb[4 * half + r] = static_cast<__bf16>(tr[r]);
                        }
                        za = mfma(ah[k2], kb, za);
                        za = mfma(al[k2], kb, za);
                    }
                }
                // za[r] = Z[c = 16 w + 4 lg + r][j = 16 jb + lr] = Z^T[j][c]: fragment
                // (jb, w / 2), lane 16 (2 (w & 1) + lg / 2) + lr, elements 4 (lg & 1) .. + 3
                const float zv[4] = {za[0], za[1], za[2], za[3]};
                uint2 hi, lo;
                split4(zv, hi, lo);
                const size_t off = zbase + (size_t)((2 * jb + (w >> 1)) * 64 +
                                                    16 * (2 * (w & 1) + (lg >> 1)) + lr) * 8 +
                                   4 * (lg & 1);
                *reinterpret_cast<uint2*>(A.ws_Zh + off) = hi;
                *reinterpret_cast<uint2*>(A.ws_Zl + off) = lo;
            }
        }
        __syncthreads();  // Am and Tm are rewritten for the next value head
    }
}

// ---------------------------------------------------------------------------
// scan: sequential over chunks, state tile in MFMA accumulators
// ---------------------------------------------------------------------------
// 4 wavefronts, one per SIMD.  Wave w owns the chunk's row block tb = w
// (tokens 16 w .. 16 w + 15) of K S^T, Q S^T, X and O for both 16-column
// halves ib = 0, 1 of the state tile's 32 rows, and the state tiles
// S^T[16 jb .. +15][16 ibS .. +15] for its DK/64 column blocks jb.
// Per chunk, one exchange through LDS:
//   (A) K S^T, Q S^T from the state tile in LDS; X = V - diag(gamma) K S^T -> LDS
//   (B) O = scale (diag(gamma) Q S^T + R X) to memory (computed transposed,
//       so that each lane stores 16 contiguous bytes); S' = gamma_n S + Z^T X
//       in the accumulators; S' -> LDS as hi / lo for the next chunk
// Memory traffic is shaped for the vector-memory pipeline, which costs about
// one cycle per touched 128-byte line and so dominates once the products are
// cheap: R and Z^T arrive in operand order (one coalesced 1 KiB load per
// fragment); K and Q rows of a wave's row block are loaded as whole lines into
// that wave's own LDS area one chunk ahead and read back as fragments (only
// the wave itself touches the area, so no barrier is involved).  Every group
// is reloaded right after its last use.  Loads go through buffer resources
// that end at the chunk's last valid row: rows past a sequence end read as
// zero, which masks K, Q, V and X without selects, and output rows past the
// end are dropped by the store's resource.
template <int DK, typename Tout>
__device__ __forceinline__ void scan_mfma_item(const PrefillArgs& A, const int b) {
    constexpr int C = kChunk;
    constexpr int BV = 32;
    constexpr int KP = DK + 8;   // padded row of the state tile (bf16)
    constexpr int TP = C + 8;    // padded row of the X tile (bf16)
    constexpr int NKK = DK / 32;
    constexpr int NJB = DK / 64;  // state column blocks per wave

    __shared__ __attribute__((aligned(16))) __bf16 Sh[BV * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Sl[BV * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Xh[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Xl[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Kw[4][16 * KP];  // per-wave K rows
    __shared__ __attribute__((aligned(16))) __bf16 Qw[4][16 * KP];  // per-wave Q rows
    constexpr int PPR = DK / 8;    // 16-byte pieces per K / Q row
    constexpr int RPI = 64 / PPR;  // rows per coalesced 1 KiB load
    constexpr int NLD = 16 / RPI;  // loads per row block and tile

    const int H = A.H, HV = A.HV, dv = A.dv;
    const int tid = threadIdx.x;
    const int tb = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index = row block
    __builtin_assume(tb >= 0 && tb < 4);
    const int l = tid & 63, lr = l & 15, lg = l >> 4;
    // Work items.  The first part of the grid holds the value-state items
    // (segment, value head, 32-row tile of S); the second the transition
    // items of segments after a sequence's first (segment, value head, 32-row
    // tile of Phi: the same scan from the identity with V = 0, writing
    // w = scale Phi_t q_t instead of o).  Without segmentation a segment is a
    // sequence and every transition item exits at once.
    // XCD-aware mapping: workgroup b runs on XCD b % 8; all tiles of a chain
    // get the same b % 8 and neighbouring dispatch slots.
    const int TV = dv / BV;
    const int nb1 = ((A.seg_bound * HV + 7) / 8) * 8 * TV;
    const bool trans = b >= nb1;
    const int bb = trans ? b - nb1 : b;
    const int TT = trans ? DK / BV : TV;
    const int slot = bb >> 3;
    const int tile = slot % TT;
    const int chain = (slot / TT) * 8 + (bb & 7);
    const int nseg = __builtin_amdgcn_readfirstlane(A.plan[0]);
    if (chain >= nseg * HV) return;
    const int sg = chain / HV, h = chain - sg * HV;
    const int n = __builtin_amdgcn_readfirstlane(A.seg_seq[sg]);
    const int sidx = __builtin_amdgcn_readfirstlane(A.seg_idx[sg]);
    if (trans && sidx == 0) return;
    const int hk = h / (HV / H);
    const bf16_t* kp = static_cast<const bf16_t*>(A.k);
    const bf16_t* qp = static_cast<const bf16_t*>(A.q);
    const bf16_t* vp = static_cast<const bf16_t*>(A.v);
    Tout* op = static_cast<Tout*>(A.o);
    // where the item's state starts and ends (row-major, DK columns)
    const float* init = nullptr;  // null: zero state (or the identity for a transition item)
    float* fin;
    size_t ibase = 0, fbase;
    if (trans) {
        fin = A.ws_Phi;
        fbase = ((size_t)(sg * HV + h) * DK + (size_t)tile * BV) * DK;
    } else if (sidx == 0) {
        init = A.s0;
        ibase = ((size_t)(n * HV + h) * dv + (size_t)tile * BV) * DK;
        const bool whole = __builtin_amdgcn_readfirstlane(A.seq_nseg[n]) == 1;
        fin = whole ? A.s_final : A.ws_E;
        fbase = whole ? ibase : ((size_t)(sg * HV + h) * dv + (size_t)tile * BV) * DK;
    } else {
        fin = A.ws_E;
        fbase = ((size_t)(sg * HV + h) * dv + (size_t)tile * BV) * DK;
    }

    // state: sacc[x][ibS][r] = S[i = 16 ibS + lr][j = 16 (NJB tb + x) + 4 lg + r]
    f4_t sacc[NJB][2];
#pragma unroll
    for (int x = 0; x < NJB; ++x)
#pragma unroll
        for (int ibS = 0; ibS < 2; ++ibS) {
            const int i = 16 * ibS + lr, j = 16 * (NJB * tb + x) + 4 * lg;
            if (init) {
                const float4 v4 = *reinterpret_cast<const float4*>(init + ibase + (size_t)i * DK + j);
                sacc[x][ibS] = f4_t{v4.x, v4.y, v4.z, v4.w};
            } else if (trans) {
                const int d = tile * BV + i - j;  // identity: 1 where row == column
                sacc[x][ibS] = f4_t{d == 0 ? 1.f : 0.f, d == 1 ? 1.f : 0.f, d == 2 ? 1.f : 0.f,
                                    d == 3 ? 1.f : 0.f};
            } else {
                sacc[x][ibS] = f4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    auto store_state = [&](float* dst) {
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ibS = 0; ibS < 2; ++ibS) {
                const int i = 16 * ibS + lr, j = 16 * (NJB * tb + x) + 4 * lg;
                if (trans) {
                    // Phi is stored transposed (Phi^T[j][i]): the combine pass
                    // reads it as an MFMA B operand, 8 consecutive i per lane
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        dst[(size_t)(sg * HV + h) * DK * DK + (size_t)(j + r) * DK + tile * BV + i] =
                            sacc[x][ibS][r];
                } else {
                    *reinterpret_cast<float4*>(dst + fbase + (size_t)i * DK + j) =
                        make_float4(sacc[x][ibS][0], sacc[x][ibS][1], sacc[x][ibS][2], sacc[x][ibS][3]);
                }
            }
    };
    auto store_state_lds = [&]() {
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ibS = 0; ibS < 2; ++ibS) {
                const int off = (16 * ibS + lr) * KP + 16 * (NJB * tb + x) + 4 * lg;
                float sv[4] = {sacc[x][ibS][0], sacc[x][ibS][1], sacc[x][ibS][2], sacc[x][ibS][3]};
                uint2 hi, lo;
                split4(sv, hi, lo);
                *reinterpret_cast<uint2*>(&Sh[off]) = hi;
                *reinterpret_cast<uint2*>(&Sl[off]) = lo;
            }
    };

    int sq, eq;
    seq_bounds_m(A.cu_seqlens, n, A.T, sq, eq);
    const int c_first = __builtin_amdgcn_readfirstlane(A.seg_c0[sg]);
    int nch = __builtin_amdgcn_readfirstlane(A.seg_nch[sg]);
    sq += (c_first - min(A.chunk_off[n], A.max_chunks)) * C;  // the segment's first token
    if (c_first + nch > A.max_chunks) nch = max(0, A.max_chunks - c_first);
    if (nch <= 0) {
        if (fin) store_state(fin);
        return;
    }

    // byte offsets of this lane's data inside a chunk (the same for every chunk)
    const uint32_t qk_row = (uint32_t)H * DK * 2;  // bytes per token of q, k
    const uint32_t v_row = (uint32_t)HV * dv * 2;  // bytes per token of v
    uint32_t kq_off[NLD];                          // coalesced rows of the row block
#pragma unroll
    for (int p = 0; p < NLD; ++p)
        kq_off[p] = ((uint32_t)(16 * tb + RPI * p + l / PPR) * H + hk) * DK * 2 + 16 * (l % PPR);
    uint32_t v_off[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        v_off[r] = ((uint32_t)(16 * tb + 4 * lg + r) * HV + h) * dv * 2 + (tile * BV + lr) * 2;
    const uint32_t v_on = trans ? 0u : 1u;  // a transition item reads V as zero
    const uint32_t r_off = (2 * tb * 64 + l) * 16;  // fragment (tb, kk): + 1 KiB kk
    uint32_t z_off[NJB];                             // fragment (jb, kk): + 1 KiB kk
#pragma unroll
    for (int x = 0; x < NJB; ++x) z_off[x] = (2 * (NJB * tb + x) * 64 + l) * 16;

    // ---- operand data (one set; groups reloaded after their last use) ----
    bf8_t kst[NLD], qst[NLD];      // K, Q rows of the next chunk, as loaded
    bf8_t rH[2], rL[2];            // R fragments of row block tb
    bf8_t zH[NJB][2], zL[NJB][2];  // Z^T fragments of column blocks NJB tb + x
    uint32_t vr[2][4];             // V[t = 16 tb + 4 lg + r][i = 16 ib + lr], raw bf16 bits
    float4 gR;                     // G[16 tb + 4 lg + r]  (log2 units)
    float gT;                      // G[16 tb + lr]
    float gN;                      // G[L - 1]

    auto chunk_t0 = [&](int jc) { return sq + jc * C; };
    auto chunk_L = [&](int jc) { return min(C, eq - (sq + jc * C)); };
    auto load_kq = [&](int jc) {
        const int t0 = chunk_t0(jc), L = chunk_L(jc);
        const __amdgpu_buffer_rsrc_t rk = in_rsrc(kp + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
        const __amdgpu_buffer_rsrc_t rq = in_rsrc(qp + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
#pragma unroll
        for (int p = 0; p < NLD; ++p) {
            kst[p] = bload8(rk, kq_off[p]);
            qst[p] = bload8(rq, kq_off[p]);
        }
    };
    // loaded rows -> this wave's LDS area (after its fragment reads of the previous chunk)
    auto stage_kq = [&]() {
#pragma unroll
        for (int p = 0; p < NLD; ++p) {
            const int at = (RPI * p + l / PPR) * KP + 8 * (l % PPR);
            *reinterpret_cast<bf8_t*>(&Kw[tb][at]) = kst[p];
            *reinterpret_cast<bf8_t*>(&Qw[tb][at]) = qst[p];
        }
    };
    auto load_g = [&](int jc) {
        const float* G = A.ws_G + ((size_t)(c_first + jc) * HV + h) * C;
        gR = *reinterpret_cast<const float4*>(G + 16 * tb + 4 * lg);
        gT = G[16 * tb + lr];
        gN = G[chunk_L(jc) - 1];
    };
    auto load_v = [&](int jc) {
        const int t0 = chunk_t0(jc), L = chunk_L(jc);
        const __amdgpu_buffer_rsrc_t rv = in_rsrc(vp + (size_t)t0 * HV * dv, v_on * L * v_row);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vr[ib][r] = __builtin_amdgcn_raw_buffer_load_b16(rv, (int)(v_off[r] + 32 * ib), 0, 0);
    };
    auto load_rz = [&](int jc) {
        const size_t cc = (size_t)(c_first + jc) * HV + h;
        const __amdgpu_buffer_rsrc_t rh = in_rsrc(A.ws_Rh + cc * C * C, C * C * 2);
        const __amdgpu_buffer_rsrc_t rl = in_rsrc(A.ws_Rl + cc * C * C, C * C * 2);
        const __amdgpu_buffer_rsrc_t zh = in_rsrc(A.ws_Zh + cc * DK * C, DK * C * 2);
        const __amdgpu_buffer_rsrc_t zl = in_rsrc(A.ws_Zl + cc * DK * C, DK * C * 2);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            rH[kk] = bload8(rh, r_off + 1024 * kk);
            rL[kk] = bload8(rl, r_off + 1024 * kk);
#pragma unroll
            for (int x = 0; x < NJB; ++x) {
                zH[x][kk] = bload8(zh, z_off[x] + 1024 * kk);
                zL[x][kk] = bload8(zl, z_off[x] + 1024 * kk);
            }
        }
    };

    load_kq(0);
    stage_kq();
    load_kq(min(1, nch - 1));
    load_g(0);
    load_v(0);
    load_rz(0);
    store_state_lds();
    __syncthreads();

    for (int jc = 0; jc < nch; ++jc) {
        const int nj = min(jc + 1, nch - 1);   // the last chunk re-reads itself
        const int nj2 = min(jc + 2, nch - 1);
        const int t0 = chunk_t0(jc);
        const int L = chunk_L(jc);
        // decays of this chunk, taken before the next chunk's G overwrites them
        const float gr[4] = {gR.x, gR.y, gR.z, gR.w};
        float gn = exp2f_(gN);
        float gt = exp2f_(gT);
        float gam[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) gam[r] = exp2f_(gr[r]);
        // keep the exponentials here: computed at their use, they would hold
        // the old G live across its reload and stall on the new load
        asm volatile("" : "+v"(gn), "+v"(gt), "+v"(gam[0]), "+v"(gam[1]), "+v"(gam[2]),
                     "+v"(gam[3]));

        // (A) K S^T, Q S^T for row block tb, both column halves; the state
        // fragments of two k-steps are read before their products
        bf8_t kA[NKK], qA[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            kA[kk] = lds8(&Kw[tb][lr * KP + 32 * kk + 8 * lg]);
            qA[kk] = lds8(&Qw[tb][lr * KP + 32 * kk + 8 * lg]);
        }
        // the next chunk's rows replace them (same wavefront, after the reads)
        stage_kq();
        load_kq(nj2);
        f4_t ksa[2], qsa[2];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            ksa[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
            qsa[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k2 = 0; k2 < NKK; k2 += 2) {
            bf8_t sh[2][2], sl[2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int col = 32 * (k2 + u) + 8 * lg;
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    sh[u][ib] = lds8(&Sh[(16 * ib + lr) * KP + col]);
                    sl[u][ib] = lds8(&Sl[(16 * ib + lr) * KP + col]);
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int kk = k2 + u;
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    ksa[ib] = mfma(kA[kk], sh[u][ib], ksa[ib]);
                    qsa[ib] = mfma(sh[u][ib], qA[kk], qsa[ib]);
                }
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    ksa[ib] = mfma(kA[kk], sl[u][ib], ksa[ib]);
                    qsa[ib] = mfma(sl[u][ib], qA[kk], qsa[ib]);
                }
            }
        }
        load_g(nj);
        float vf[2][4];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) vf[ib][r] = __uint_as_float(vr[ib][r] << 16);
        load_v(nj);
        // X = V - diag(gamma) K S^T (zero in rows past the end: V and K read as zero)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            float xv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) xv[r] = vf[ib][r] - gam[r] * ksa[ib][r];
            uint2 hi, lo;
            split4(xv, hi, lo);
            const int off = (16 * ib + lr) * TP + 16 * tb + 4 * lg;
            *reinterpret_cast<uint2*>(&Xh[off]) = hi;
            *reinterpret_cast<uint2*>(&Xl[off]) = lo;
        }
        __syncthreads();

        // (B) X fragments (token k-steps kk, state-row halves ib) serve both products
        bf8_t xh[2][2], xl[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                xh[kk][ib] = lds8(&Xh[(16 * ib + lr) * TP + 32 * kk + 8 * lg]);
                xl[kk][ib] = lds8(&Xl[(16 * ib + lr) * TP + 32 * kk + 8 * lg]);
            }
        // O^T = scale (S Q^T diag(gamma) + X^T R^T), transposed so that a lane
        // holds four consecutive outputs of one token; R is lower triangular,
        // so row block tb needs the k-steps up to tb / 2
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) qsa[ib][r] *= gt;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk <= (tb >> 1)) {
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    qsa[ib] = mfma(xh[kk][ib], rH[kk], qsa[ib]);
                    qsa[ib] = mfma(xl[kk][ib], rH[kk], qsa[ib]);
                    qsa[ib] = mfma(xh[kk][ib], rL[kk], qsa[ib]);
                }
            }
        }
        // S'^T = gamma_n S^T + Z^T X for the wave's state tiles
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ibS = 0; ibS < 2; ++ibS) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[x][ibS][r] *= gn;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    sacc[x][ibS] = mfma(zH[x][kk], xh[kk][ibS], sacc[x][ibS]);
                    sacc[x][ibS] = mfma(zH[x][kk], xl[kk][ibS], sacc[x][ibS]);
                    sacc[x][ibS] = mfma(zL[x][kk], xh[kk][ibS], sacc[x][ibS]);
                }
            }
        load_rz(nj);
        {
            // qsa[ib][r] = O[t = 16 tb + lr][i = 16 ib + 4 lg + r]; rows t >= L land
            // at or past the resource end and are dropped.  A transition item
            // writes w (fp32, dk per token and head) instead of o.
            const int t = 16 * tb + lr;
            if (trans) {
                float* wp = A.ws_W + (size_t)t0 * HV * DK;
                const __amdgpu_buffer_rsrc_t wr = out_rsrc(wp, (uint32_t)(L * HV * DK * 4));
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const float ov[4] = {A.scale * qsa[ib][0], A.scale * qsa[ib][1],
                                         A.scale * qsa[ib][2], A.scale * qsa[ib][3]};
                    out_store4(wr, (uint32_t)((t * HV + h) * DK + tile * BV + 16 * ib + 4 * lg), ov,
                               wp);
                }
            } else {
                const __amdgpu_buffer_rsrc_t orsrc =
                    out_rsrc(op + (size_t)t0 * HV * dv, (uint32_t)(L * HV * dv * sizeof(Tout)));
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const float ov[4] = {A.scale * qsa[ib][0], A.scale * qsa[ib][1],
                                         A.scale * qsa[ib][2], A.scale * qsa[ib][3]};
                    out_store4(orsrc, (uint32_t)((t * HV + h) * dv + tile * BV + 16 * ib + 4 * lg),
                               ov, op);
                }
            }
        }
        // the state tile in LDS is read only in (A), which every wave has left
        store_state_lds();
        __syncthreads();
    }

    if (fin) store_state(fin);
}

// Persistent over work items: workgroup blockIdx.x takes items blockIdx.x,
// blockIdx.x + gridDim.x, ...  (the grid is a multiple of 8, so an item keeps
// its XCD).  The host sizes the grid to the work it can see: the unsegmented
// items when they already fill the CUs, otherwise every possible item.
template <int DK, typename Tout>
__global__ __launch_bounds__(256) void scan_mfma_kernel(const PrefillArgs A, int items) {
    for (int b = blockIdx.x; b < items; b += gridDim.x) scan_mfma_item<DK, Tout>(A, b);
}

// ---------------------------------------------------------------------------
// segment-parallel scan: plan, combine, correction
// ---------------------------------------------------------------------------
// The chunk map of a segment is affine in the state entering it:
//     S_end = S_in Phi + E,   o_t = scale S_t q_t = o0_t + S_in w_t,
// with Phi the product of the segment's token transitions a (I - b k k^T),
// E and o0 the end state and outputs of the segment's own pass from a zero
// state, and w_t = scale Phi_t q_t.  So every segment after a sequence's first
// runs twice in parallel with the other segments (the value pass from zero,
// giving E and o0, and the transition pass from the identity with V = 0,
// giving Phi and w), a short per-sequence pass chains
// S_in(j+1) = S_in(j) Phi_j + E_j, and a parallel pass adds S_in w_t to o.

// Exclusive prefix sum of count(i) over i < n; emit(i, position, count) is
// called once for every i.  Returns the total.  All 256 threads take part.
template <typename F, typename G>
__device__ int block_exclusive_scan(int n, F count, G emit, int* buf) {
    int carry = 0;
    for (int base = 0; base < n; base += 256) {
        const int i = base + (int)threadIdx.x;
        const int c = i < n ? count(i) : 0;
        buf[threadIdx.x] = c;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int add = (int)threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
            __syncthreads();
            buf[threadIdx.x] += add;
            __syncthreads();
        }
        if (i < n) emit(i, carry + buf[threadIdx.x] - c, c);
        carry += buf[255];
        __syncthreads();
    }
    return carry;
}

// Segment length candidates (chunks; 0: do not segment) and the cost model
// that picks one, in microseconds, fitted to measurements of the scan on the
// MI355X: with a workgroup per 32 state rows, a chain step takes about 2.2 us
// while at most 64 workgroups run, 2.6 us up to 256 (one per CU) and 4.5 us
// where two share a CU, and the whole launch sustains about 110 chain steps
// per us; with a workgroup per chain, a step takes about 5.6 us (one per CU)
// and the launch sustains about 46 steps per us; a segmented run moves
// about 8 (dk + dv) more bytes per token and head of every later segment (w
// written and read, o read and written again) at about 5 TB/s, plus about
// 3 us per segment of the combine pass.  A launch that already gives every
// CU a workgroup is segmented only when its longest chain takes more than
// twice as long as the launch's throughput allows (one long prompt among
// short ones): then the segments of that chain run beside the other work.
constexpr int kSegCand[7] = {0, 1024, 512, 256, 128, 64, 32};
constexpr int kNCand = 7;

// One workgroup: the chunk table (chunk_off, the first global chunk of every
// sequence), then the choice of the segment length, the segments of every
// sequence and the work lists of the combine and correction passes.
// plan = {segments, correction items, segment length (0: none), sequences
// with more than one segment}.  Chunk counts of the first kPlanCache
// sequences stay in LDS.
constexpr int kPlanCache = 2048;

__global__ __launch_bounds__(256) void plan_segments_kernel(const PrefillArgs A, int TV, int TK,
                                                            int tp) {
    __shared__ int ibuf[256];
    __shared__ int cnt_sh[kPlanCache], off_sh[kPlanCache];
    __shared__ float acc[3][kNCand];  // items, chain steps, tokens of later segments
    __shared__ int s_cmax;
    __shared__ int s_len;
    const int N = A.N, HV = A.HV;
    int32_t* co = A.chunk_off;
    auto count = [&](int n) {
        int s, e;
        seq_bounds_m(A.cu_seqlens, n, A.T, s, e);
        return (e - s + kChunk - 1) / kChunk;
    };
    const int total = block_exclusive_scan(
        N, count,
        [&](int n, int pos, int c) {
            co[n] = pos;
            if (n < kPlanCache) {
                cnt_sh[n] = c;
                off_sh[n] = pos;
            }
        },
        ibuf);
    if (threadIdx.x == 0) co[N] = total;
    __syncthreads();
    auto first_chunk = [&](int n) { return min(n < kPlanCache ? off_sh[n] : co[n], A.max_chunks); };
    auto nchunks = [&](int n) {
        const int o = n < kPlanCache ? off_sh[n] : co[n];
        const int c = n < kPlanCache ? cnt_sh[n] : co[n + 1] - co[n];
        return max(0, min(o + c, A.max_chunks) - min(o, A.max_chunks));
    };

    if (A.seg_req != 0 && A.seg_req != kSegAutoSkewed) {
        if (threadIdx.x == 0) s_len = A.seg_req < 0 ? 0 : A.seg_req;
    } else {
        if (threadIdx.x < 3 * kNCand) (&acc[0][0])[threadIdx.x] = 0.f;
        if (threadIdx.x == 0) s_cmax = 0;
        __syncthreads();
        float items[kNCand] = {}, steps[kNCand] = {}, later[kNCand] = {};
        int cmax = 0;
        for (int n = threadIdx.x; n < N; n += 256) {
            const int c = nchunks(n);
            cmax = max(cmax, c);
#pragma unroll
            for (int k = 0; k < kNCand; ++k) {
                const int L = kSegCand[k] ? kSegCand[k] : (1 << 30);
                const int m = c > 0 ? (c + L - 1) / L : 1;
                const int first = min(c, L);
                items[k] += (float)HV * TV + (float)(m - 1) * HV * (TV + TK);
                steps[k] += (float)first * HV * TV + (float)(c - first) * HV * (TV + TK);
                later[k] += (float)(c - first) * kChunk;
            }
        }
        // wavefront sums first, then one shared-memory atomic per wavefront
        auto wsum = [](float x) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
            return x;
        };
#pragma unroll
        for (int k = 0; k < kNCand; ++k) {
            items[k] = wsum(items[k]);
            steps[k] = wsum(steps[k]);
            later[k] = wsum(later[k]);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) cmax = max(cmax, __shfl_xor(cmax, o, 64));
        if ((threadIdx.x & 63) == 0) {
#pragma unroll
            for (int k = 0; k < kNCand; ++k) {
                atomicAdd(&acc[0][k], items[k]);
                atomicAdd(&acc[1][k], steps[k]);
                atomicAdd(&acc[2][k], later[k]);
            }
            atomicMax(&s_cmax, cmax);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            const int cm = s_cmax;
            const float dk = (float)A.dk, dv = (float)A.dv;
            float best = 0.f;
            int bestL = 0;
            // chain steps per microsecond over the whole GPU, and the time of one
            // chain step (us) for a number of items; the d_k = 128 scan holds one
            // workgroup per CU, so its step does not grow with the items
            const float thr = tp ? 120.f : 110.f;
            auto step_of = [&](float items) {
                return tp ? 2.1f : (items <= 64.f ? 2.2f : (items <= 256.f ? 2.6f : 4.5f));
            };
            const bool skewed = (float)cm * step_of(acc[0][0]) > 2.f * acc[1][0] / thr;
            for (int k = 0; k < (acc[0][0] < 256.f || skewed ? kNCand : 1); ++k) {
                const int L = kSegCand[k] ? kSegCand[k] : (1 << 30);
                const bool seg = cm > L;
                const float step = step_of(acc[0][k]);
                float cost = fmaxf(acc[1][k] / thr, (float)min(cm, L) * step);
                if (seg)
                    cost += acc[2][k] * HV * 8.f * (dk + dv) / 5.0e6f + 3.f * ((cm + L - 1) / L) + 5.f;
                if (k == 0 || cost < best) {
                    best = cost;
                    bestL = seg ? L : 0;
                }
            }
            s_len = bestL;
        }
    }
    __syncthreads();
    const int Ls = s_len;
    if (Ls == 0) {
        // one segment per sequence: the tables need no scans, and there are
        // no later segments, hence no combine or correction work
        for (int n = threadIdx.x; n < N; n += 256) {
            A.seq_seg0[n] = n;
            A.seq_nseg[n] = 1;
            A.seg_seq[n] = n;
            A.seg_c0[n] = first_chunk(n);
            A.seg_nch[n] = nchunks(n);
            A.seg_idx[n] = 0;
        }
        if (threadIdx.x == 0) {
            A.plan[0] = N;
            A.plan[1] = 0;
            A.plan[2] = 0;
            A.plan[3] = 0;
        }
        return;
    }
    auto nseg_of = [&](int n) {
        const int c = nchunks(n);
        return (Ls > 0 && c > 0) ? (c + Ls - 1) / Ls : 1;
    };
    // segments of every sequence
    const int nseg = block_exclusive_scan(
        N, nseg_of,
        [&](int n, int pos, int m) {
            const int c = nchunks(n);
            const int len = Ls > 0 ? Ls : c;
            A.seq_seg0[n] = pos;
            A.seq_nseg[n] = m;
            for (int j = 0; j < m; ++j) {
                A.seg_seq[pos + j] = n;
                A.seg_c0[pos + j] = first_chunk(n) + j * len;
                A.seg_nch[pos + j] = max(0, min(len, c - j * len));
                A.seg_idx[pos + j] = j;
            }
        },
        ibuf);
    // sequences with more than one segment
    const int nmulti = block_exclusive_scan(
        N, [&](int n) { return nseg_of(n) > 1 ? 1 : 0; },
        [&](int n, int pos, int c) {
            if (c) A.multi_seq[pos] = n;
        },
        ibuf);
    __syncthreads();  // the segment tables are complete
    // correction items: groups of kCorrChunks chunks of every later segment
    const int ncorr = block_exclusive_scan(
        nseg,
        [&](int sg) {
            return A.seg_idx[sg] > 0 ? (A.seg_nch[sg] + kCorrChunks - 1) / kCorrChunks : 0;
        },
        [&](int sg, int pos, int c) {
            for (int g = 0; g < c; ++g) {
                A.corr_seg[pos + g] = sg;
                A.corr_c0[pos + g] = A.seg_c0[sg] + g * kCorrChunks;
            }
        },
        ibuf);
    if (threadIdx.x == 0) {
        A.plan[0] = nseg;
        A.plan[1] = ncorr;
        A.plan[2] = Ls;
        A.plan[3] = nmulti;
    }
}

// Combine: per (sequence with several segments, value head, 32-row tile of
// S) walk the segments in order, S_in(j+1) = S_in(j) Phi_j + E_j; S_in of
// every later segment is kept for the correction, and the last product is the
// sequence's final state.  The product runs on MFMA with both operands split
// into hi + lo bf16 (fp32 accumulation), S_in staying in LDS as fp32 between
// steps; Phi^T and E of the next segment are loaded during the current step.
// Wave w computes output column blocks NCB w .. NCB w + NCB - 1, both row
// blocks.  Persistent over items.
template <int DK>
__global__ __launch_bounds__(256) void combine_kernel(const PrefillArgs A) {
    constexpr int BV = 32;
    constexpr int SP = DK + 4;        // padded fp32 row in LDS
    constexpr int NKK = DK / 32;      // k-steps
    constexpr int NCB = DK / 16 / 4;  // column blocks per wave
    __shared__ __attribute__((aligned(16))) float Sc[BV * SP];
    const int HV = A.HV, dv = A.dv, TV = dv / BV;
    const int nmulti = A.plan[3];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, lg = l >> 4;
    for (int item = blockIdx.x; item < nmulti * HV * TV; item += gridDim.x) {
        const int m = item / (HV * TV);
        const int h = (item / TV) % HV, tile = item % TV;
        const int n = A.multi_seq[m];
        const int s0 = A.seq_seg0[n], ns = A.seq_nseg[n];
        auto rows = [&](float* base, int sgi) {  // this tile's 32 rows of a value state
            return base + ((size_t)(sgi * HV + h) * dv + (size_t)tile * BV) * DK;
        };
        // B fragments (Phi^T rows = output columns) and E at the output positions
        bf8_t bh[NCB][NKK], bl[NCB][NKK];
        float ev[NCB][2][4];
        auto load_next = [&](int sgi) {
            const float* pt = A.ws_Phi + (size_t)(sgi * HV + h) * DK * DK;
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const float* p = pt + (size_t)(16 * (NCB * w + c) + lr) * DK + 32 * kk + 8 * lg;
                    const float4 x0 = *reinterpret_cast<const float4*>(p);
                    const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
                    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    split8(x, bh[c][kk], bl[c][kk]);
                }
            const float* e = rows(A.ws_E, sgi);
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ev[c][rb][r] = e[(size_t)(16 * rb + 4 * lg + r) * DK + 16 * (NCB * w + c) + lr];
        };
        __syncthreads();  // the previous item has finished with Sc
        {
            const float* e0 = rows(A.ws_E, s0);
            for (int x = tid; x < BV * DK / 4; x += 256) {
                const int r = x / (DK / 4), c = 4 * (x % (DK / 4));
                *reinterpret_cast<float4*>(&Sc[r * SP + c]) = *reinterpret_cast<const float4*>(e0 + (size_t)r * DK + c);
            }
        }
        if (ns > 1) load_next(s0 + 1);
        __syncthreads();
        for (int j = 1; j < ns; ++j) {
            const int sgi = s0 + j;
            // S_in of this segment, for the correction
            {
                float* dst = rows(A.ws_Sin, sgi);
                for (int x = tid; x < BV * DK / 4; x += 256) {
                    const int r = x / (DK / 4), c = 4 * (x % (DK / 4));
                    *reinterpret_cast<float4*>(dst + (size_t)r * DK + c) = *reinterpret_cast<const float4*>(&Sc[r * SP + c]);
                }
            }
            f4_t d[NCB][2];
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    d[c][rb] = f4_t{ev[c][rb][0], ev[c][rb][1], ev[c][rb][2], ev[c][rb][3]};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const float* p = &Sc[(16 * rb + lr) * SP + 32 * kk + 8 * lg];
                    const float4 x0 = *reinterpret_cast<const float4*>(p);
                    const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
                    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    bf8_t ah, al;
                    split8(x, ah, al);
#pragma unroll
                    for (int c = 0; c < NCB; ++c) {
                        d[c][rb] = mfma(ah, bh[c][kk], d[c][rb]);
                        d[c][rb] = mfma(al, bh[c][kk], d[c][rb]);
                        d[c][rb] = mfma(ah, bl[c][kk], d[c][rb]);
                    }
                }
            if (j + 1 < ns) load_next(sgi + 1);
            __syncthreads();  // every wave has read S_in
#pragma unroll
            for (int c = 0; c < NCB; ++c)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Sc[(16 * rb + 4 * lg + r) * SP + 16 * (NCB * w + c) + lr] = d[c][rb][r];
            __syncthreads();
        }
        if (A.s_final) {
            float* dst = A.s_final + ((size_t)(n * HV + h) * dv + (size_t)tile * BV) * DK;
            for (int x = tid; x < BV * DK / 4; x += 256) {
                const int r = x / (DK / 4), c = 4 * (x % (DK / 4));
                *reinterpret_cast<float4*>(dst + (size_t)r * DK + c) = *reinterpret_cast<const float4*>(&Sc[r * SP + c]);
            }
        }
    }
}

// Correction: o_t += S_in w_t for the tokens of every later segment, as
// O^T = S_in W^T on MFMA with both operands split into hi + lo bf16.  An item
// is (group of kCorrChunks chunks of one segment, value head); S_in of the
// item is staged in LDS once, wavefront w takes tokens 16 w .. 16 w + 15 of
// each chunk.  Persistent over items.
template <int DK, typename Tout>
__global__ __launch_bounds__(256) void correct_kernel(const PrefillArgs A) {
    constexpr int C = kChunk;
    constexpr int KP = DK + 8;
    constexpr int NKK = DK / 32;
    __shared__ __attribute__((aligned(16))) __bf16 Sh[128 * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Sl[128 * KP];
    const int HV = A.HV, dv = A.dv;
    const int ncorr = A.plan[1];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, lg = l >> 4;
    Tout* op = static_cast<Tout*>(A.o);
    for (int item = blockIdx.x; item < ncorr * HV; item += gridDim.x) {
        const int ci = item / HV, h = item - ci * HV;
        const int sg = A.corr_seg[ci];
        const int cfirst = A.corr_c0[ci];
        const int n = A.seg_seq[sg];
        const int cend = min(A.seg_c0[sg] + A.seg_nch[sg], cfirst + kCorrChunks);
        int sq, eq;
        seq_bounds_m(A.cu_seqlens, n, A.T, sq, eq);
        const int cseq = min(A.chunk_off[n], A.max_chunks);
        // S_in (dv x DK, fp32) -> hi / lo bf16 rows in LDS
        const float* sin = A.ws_Sin + (size_t)(sg * HV + h) * dv * DK;
        __syncthreads();  // the previous item has finished reading Sh, Sl
        for (int e = tid; e < dv * DK / 8; e += 256) {
            const int row = e / (DK / 8), col = 8 * (e % (DK / 8));
            const float4 a = *reinterpret_cast<const float4*>(sin + (size_t)row * DK + col);
            const float4 b = *reinterpret_cast<const float4*>(sin + (size_t)row * DK + col + 4);
            const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            bf8_t hi, lo;
            split8(x, hi, lo);
            *reinterpret_cast<bf8_t*>(&Sh[row * KP + col]) = hi;
            *reinterpret_cast<bf8_t*>(&Sl[row * KP + col]) = lo;
        }
        __syncthreads();
        for (int c = cfirst; c < cend; ++c) {
            const int t0 = sq + (c - cseq) * C;
            const int L = min(C, eq - t0);
            // W^T fragments: column = token 16 w + lr, k = 32 kk + 8 lg .. + 7
            const __amdgpu_buffer_rsrc_t wr = in_rsrc(A.ws_W + (size_t)t0 * HV * DK, (uint32_t)(L * HV * DK * 4));
            const uint32_t wrow = (uint32_t)((16 * w + lr) * HV + h) * DK;
            bf8_t wh[NKK], wl[NKK];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const float4 a = in_load4(wr, wrow + 32 * kk + 8 * lg);
                const float4 b = in_load4(wr, wrow + 32 * kk + 8 * lg + 4);
                const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                split8(x, wh[kk], wl[kk]);
            }
            const __amdgpu_buffer_rsrc_t orr = out_rsrc(op + (size_t)t0 * HV * dv, (uint32_t)(L * HV * dv * sizeof(Tout)));
            for (int nb = 0; nb < dv / 16; ++nb) {
                f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const bf8_t ah = lds8(&Sh[(16 * nb + lr) * KP + 32 * kk + 8 * lg]);
                    const bf8_t al = lds8(&Sl[(16 * nb + lr) * KP + 32 * kk + 8 * lg]);
                    d = mfma(ah, wh[kk], d);
                    d = mfma(al, wh[kk], d);
                    d = mfma(ah, wl[kk], d);
                }
                // d[r] = (S_in W^T)[i = 16 nb + 4 lg + r][t = 16 w + lr]
                const uint32_t off = (uint32_t)((16 * w + lr) * HV + h) * dv + 16 * nb + 4 * lg;
                float ov[4];
                load4_any(orr, off, ov, op);
#pragma unroll
                for (int r = 0; r < 4; ++r) ov[r] += d[r];
                out_store4(orr, off, ov, op);
            }
        }
    }
}

// Segmentation is possible when asked for; automatically (seg_req 0) when
// the unsegmented scan leaves CUs idle and some sequence may be longer than
// one segment; and with kSegAutoSkewed whenever
// some sequence may be longer than one segment (one long prompt among short
// ones, whose chains already fill the CUs: the planner decides from the
// lengths).  Otherwise the plan is fixed to one segment per sequence and the
// later passes are not launched: a possible plan costs their two launches
// even when it turns out to be unsegmented.
// "Idle" is fewer than 256 items for the per-tile scan (d_k = 64), and fewer
// than 128 for the d_k = 128 scan: it holds one workgroup per CU, and a later
// segment's value and transition items double its work, which paid only while
// most CUs would otherwise idle (one 32768-token prompt, 64 items: 1.10 ->
// 0.86 ms segmented; 128 items: 1.13 -> 1.37 ms).
static bool may_segment(const PrefillArgs& A) {
    const size_t TV = (size_t)A.dv / 32;
    const size_t idle = A.dk == 128 ? 128 : 256;
    const bool longer = (A.T + kChunk - 1) / kChunk > kSegMinChunks;
    return A.seg_req > 0 || (A.seg_req == kSegAutoSkewed && longer) ||
           (A.seg_req == 0 && longer && (size_t)A.N * A.HV * TV < idle);
}

// plan -> prep -> scan (value and transition items) -> combine -> correction.
// Without segmentation the last two find no work and exit.
template <int DK, typename Tout>
static hipError_t launch_mfma_t(const PrefillArgs& A0) {
    const int TV = A0.dv / 32, TK = DK / 32;
    PrefillArgs A = A0;
    const bool may = may_segment(A0);
    if (!may) A.seg_req = -1;
    // d_k = 128: the T'-only prep and the four-role scan (gdn_prefill_tp.hip);
    // d_k = 64: the prep with R and Z^T and the per-tile scan
    const bool tp = DK == 128;
    hipLaunchKernelGGL(plan_segments_kernel, dim3(1), dim3(256), 0, A.stream, A, TV, TK, tp ? 1 : 0);
    hipError_t err = tp ? launch_prep_tp(A) : hipSuccess;
    if (!tp)
        hipLaunchKernelGGL((prep_mfma_kernel<DK>), dim3(A.max_chunks, A.HV), dim3(256), 0,
                           A.stream, A);
    if (err == hipSuccess) err = hipGetLastError();
    if (err != hipSuccess) return err;
    // value items of up to seg_bound segments (N without segmentation), then
    // the transition items; the kernel splits the grid at seg_bound.  The grid
    // takes every possible item when the unsegmented items leave CUs idle,
    // otherwise just the unsegmented items (any segments' items are then taken
    // by the same workgroups in turn, and when there are none no workgroup is
    // launched only to exit)
    // (the four-role scan counts chains by key head, R value heads each)
    const size_t R = tp ? (size_t)(A.HV / A.H) : 1;
    const size_t CH = tp ? (size_t)A.H : (size_t)A.HV;
    const size_t chains8 = (size_t)(((may ? A.seg_bound : A.N) * CH + 7) / 8) * 8 * R;
    const size_t items = may ? chains8 * (TV + TK) : chains8 * TV;
    const size_t unseg = (size_t)((A.N * CH + 7) / 8) * 8 * R * TV;
    const size_t grid = (may && (size_t)A.N * A.HV * TV < 256) ? items : unseg;
    if (tp) {
        err = launch_scan_tp(A, grid, (int)items);
        if (err != hipSuccess) return err;
    } else {
        hipLaunchKernelGGL((scan_mfma_kernel<DK, Tout>), dim3((unsigned)grid), dim3(256), 0,
                           A.stream, A, (int)items);
    }
    if (may) {
        const int cgrid = (int)std::min<size_t>((size_t)A.N * A.HV * TV, 512);
        hipLaunchKernelGGL((combine_kernel<DK>), dim3(cgrid), dim3(256), 0, A.stream, A);
        const int rgrid = (int)std::min<size_t>((size_t)A.corr_bound * A.HV, 512);
        hipLaunchKernelGGL((correct_kernel<DK, Tout>), dim3(rgrid), dim3(256), 0, A.stream, A);
    }
    return hipGetLastError();
}

bool prefill_mfma_eligible(const PrefillArgs& A) {
    return A.in_bf16 && (A.dk == 64 || A.dk == 128) && (A.dv % 32 == 0);
}

bool prefill_may_segment(int N, int T, int HV, int dk, int dv, bool in_bf16, int seg_req) {
    PrefillArgs A{};
    A.N = N; A.T = T; A.HV = HV; A.dk = dk; A.dv = dv; A.in_bf16 = in_bf16; A.seg_req = seg_req;
    return prefill_mfma_eligible(A) && may_segment(A);
}

hipError_t launch_prefill_mfma(const PrefillArgs& A) {
    if (A.dk == 64) return A.o_bf16 ? launch_mfma_t<64, bf16_t>(A) : launch_mfma_t<64, float>(A);
    return A.o_bf16 ? launch_mfma_t<128, bf16_t>(A) : launch_mfma_t<128, float>(A);
}

}  // namespace gdn

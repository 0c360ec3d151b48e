// gdn_prefill_mfma.hip -- chunked prefill on bf16 MFMA (gfx950, bf16 inputs).
//
// Same chunkwise form as gdn_prefill.hip (gated delta rule, Yang et al., ICLR
// 2025): per chunk of C = 64 tokens with cumulative log-decays G,
//
//     A_ts = b_t e^{G_t - G_s} k_t.k_s (s < t),   T' = (I + A)^-1 diag(b)
//     X    = V - diag(e^G) K S^T                  U  = T' X
//     O    = scale (diag(e^G) Q S^T + P U),       P_ts = e^{G_t - G_s} q_t.k_s (s <= t)
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
// Kernels:
//   prep_mfma  one workgroup per (chunk, key head): K K^T once on MFMA, then
//              for each value head sharing that key head: G, A, the blocked
//              triangular inverse (16 x 16 diagonal blocks by substitution,
//              off-diagonal blocks by T_ij = -T_ii sum_k A_ik T_kj), and
//              T' = T diag(b) to the workspace.
//   scan_mfma  one workgroup per (sequence, value head, 32-row tile of S),
//              sequential over the sequence's chunks, with the next chunk's
//              K, Q, V, T', G prefetched into registers.  The tiles of one
//              (sequence, head) run on one XCD so that their shared K, Q and
//              T' reads hit the same L2.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4_t mfma(bf8_t a, bf8_t b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf8_t lds8(const __bf16* p) {
    return *reinterpret_cast<const bf8_t*>(p);
}

// fp32 x -> (hi, lo) with hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split8(const float* x, bf8_t& hi, bf8_t& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = static_cast<__bf16>(x[j]);
        hi[j] = h;
        lo[j] = static_cast<__bf16>(x[j] - static_cast<float>(h));
    }
}

__device__ __forceinline__ void split1(float x, __bf16& hi, __bf16& lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

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

// ---------------------------------------------------------------------------
// prep: K K^T, A, T' = (I + A)^-1 diag(b), G
// ---------------------------------------------------------------------------
template <int DK>
__global__ __launch_bounds__(256) void prep_mfma_kernel(
    const bf16_t* __restrict__ k, const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, int N, int T, int H,
    int HV, int max_chunks, float* __restrict__ wsT, float* __restrict__ wsG) {
    constexpr int C = kChunk;
    constexpr int KP = DK + 8;  // padded bf16 row
    constexpr int AP = C + 4;   // padded fp32 row (16-byte aligned rows)
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * KP];
    __shared__ __attribute__((aligned(16))) float Am[C * AP];
    __shared__ __attribute__((aligned(16))) float Tm[C * AP];
    __shared__ __attribute__((aligned(16))) float Xm[32 * 36];
    __shared__ float Gs[C], Bs[C];

    const int c = blockIdx.x, hk = blockIdx.y, tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int total = min(chunk_off[N], max_chunks);
    if (c >= total) return;
    const int n = find_seq_m(chunk_off, N, c);
    int s0, e0;
    seq_bounds_m(cu, n, T, s0, e0);
    const int t0 = s0 + (c - chunk_off[n]) * C;
    const int L = min(C, e0 - t0);
    const int ratio = HV / H;

    // K chunk -> LDS (rows past the sequence end are zero)
    for (int idx = tid; idx < C * DK / 8; idx += 256) {
        const int t = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
        uint4 val = *reinterpret_cast<const uint4*>(
            k + ((size_t)(t0 + min(t, L - 1)) * H + hk) * DK + c8);
        if (t >= L) val = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(&Ks[t * KP + c8]) = val;
    }
    __syncthreads();

    // K K^T for row block w and column blocks sb <= w
    f4_t kk[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) kk[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        const bf8_t a = lds8(&Ks[(16 * w + lr) * KP + 32 * ks + 8 * lg]);
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if (sb <= w) {
                const bf8_t b = lds8(&Ks[(16 * sb + lr) * KP + 32 * ks + 8 * lg]);
                kk[sb] = mfma(a, b, kk[sb]);
            }
        }
    }

    for (int hv = hk * ratio; hv < (hk + 1) * ratio; ++hv) {
        // G = in-chunk inclusive cumsum of g (wave 0), beta
        if (w == 0) {
            float gv = g[(size_t)(t0 + min(l, L - 1)) * HV + hv];
            float bv = beta[(size_t)(t0 + min(l, L - 1)) * HV + hv];
            if (l >= L) gv = 0.f, bv = 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float up = __shfl_up(gv, off, 64);
                if (l >= off) gv += up;
            }
            Gs[l] = gv;
            Bs[l] = bv;
        }
        __syncthreads();
        // A = strictly lower part of diag(b) (K K^T o e^{G_t - G_s})
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if (sb <= w) {
                const float Gsb = Gs[16 * sb + lr];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + 4 * lg + r, s = 16 * sb + lr;
                    Am[t * AP + s] = (s < t) ? Bs[t] * __expf(Gs[t] - Gsb) * kk[sb][r] : 0.f;
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
        // 16-block merges: T_10 = -T_11 (A_10 T_00), T_32 = -T_33 (A_32 T_22)
        {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int e = tid + 256 * half;
                const int j = (e >> 8) * 2, i = j + 1;  // (1,0) or (3,2)
                const int rho = (e >> 4) & 15, kap = e & 15;
                float acc = 0.f;
#pragma unroll
                for (int x = 0; x < 16; ++x)
                    acc += (x >= kap) ? Am[(16 * i + rho) * AP + 16 * j + x] *
                                            Tm[(16 * j + x) * AP + 16 * j + kap]
                                      : 0.f;
                Xm[(16 * (e >> 8) + rho) * 36 + kap] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int e = tid + 256 * half;
            const int j = (e >> 8) * 2, i = j + 1;
            const int rho = (e >> 4) & 15, kap = e & 15;
            float acc = 0.f;
#pragma unroll
            for (int x = 0; x < 16; ++x)
                acc += (x <= rho) ? Tm[(16 * i + rho) * AP + 16 * i + x] *
                                        Xm[(16 * (e >> 8) + x) * 36 + kap]
                                  : 0.f;
            Tm[(16 * i + rho) * AP + 16 * j + kap] = -acc;
        }
        __syncthreads();
        // 32-block merge on MFMA: X = A[32:64, 0:32] T[0:32, 0:32]; T[32:64, 0:32] = -T_B X
        {
            const int tb = w >> 1, jb = w & 1;
            float av[8], bv[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                av[x] = Am[(32 + 16 * tb + lr) * AP + 8 * lg + x];
                const int xr = 8 * lg + x, cc = 16 * jb + lr;
                bv[x] = (xr >= cc || (xr >> 4) > (cc >> 4)) ? Tm[xr * AP + cc] : 0.f;
            }
            bf8_t ah, al, bh, bl;
            split8(av, ah, al);
            split8(bv, bh, bl);
            f4_t xa = f4_t{0.f, 0.f, 0.f, 0.f};
            xa = mfma(ah, bh, xa);
            xa = mfma(ah, bl, xa);
            xa = mfma(al, bh, xa);
#pragma unroll
            for (int r = 0; r < 4; ++r) Xm[(16 * tb + 4 * lg + r) * 36 + 16 * jb + lr] = xa[r];
        }
        __syncthreads();
        {
            const int tb = w >> 1, jb = w & 1;
            float av[8], bv[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const int rr = 16 * tb + lr, xc = 8 * lg + x;  // T_B row rr, column xc (lower)
                av[x] = (xc <= rr) ? Tm[(32 + rr) * AP + 32 + xc] : 0.f;
                bv[x] = Xm[(8 * lg + x) * 36 + 16 * jb + lr];
            }
            bf8_t ah, al, bh, bl;
            split8(av, ah, al);
            split8(bv, bh, bl);
            f4_t ta = f4_t{0.f, 0.f, 0.f, 0.f};
            ta = mfma(ah, bh, ta);
            ta = mfma(ah, bl, ta);
            ta = mfma(al, bh, ta);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Tm[(32 + 16 * tb + 4 * lg + r) * AP + 16 * jb + lr] = -ta[r];
        }
        __syncthreads();
        // T' = T diag(b) (lower triangle; zeros above), and G
        float* To = wsT + ((size_t)c * HV + hv) * C * C;
        for (int idx = tid; idx < C * C / 4; idx += 256) {
            const int t = idx >> 4, s4 = 4 * (idx & 15);
            float4 out;
            out.x = (s4 + 0 <= t) ? Tm[t * AP + s4 + 0] * Bs[s4 + 0] : 0.f;
            out.y = (s4 + 1 <= t) ? Tm[t * AP + s4 + 1] * Bs[s4 + 1] : 0.f;
            out.z = (s4 + 2 <= t) ? Tm[t * AP + s4 + 2] * Bs[s4 + 2] : 0.f;
            out.w = (s4 + 3 <= t) ? Tm[t * AP + s4 + 3] * Bs[s4 + 3] : 0.f;
            *reinterpret_cast<float4*>(To + t * C + s4) = out;
        }
        if (tid < C) wsG[((size_t)c * HV + hv) * C + tid] = Gs[tid];
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// scan: sequential over chunks, state tile in MFMA accumulators
// ---------------------------------------------------------------------------
// 8 wavefronts.  Wave w owns output tile (tb = w / 2, ib = w % 2): rows
// 16 tb .. 16 tb + 15 of the chunk (tokens) and columns 16 ib .. 16 ib + 15
// of the state tile's 32 rows (value dims) in K S^T, Q S^T, X, U and O, and
// state tiles S^T[16 jb .. +15][16 ibS .. +15] for (jb, ibS) in its share.
// Products whose accumulators are written to LDS are taken in the
// orientation that gives each lane 4 consecutive elements of the stored
// layout (P^T = K Q^T, S'^T = K^T U'), so every LDS store is 8 bytes.
template <int DK, typename Tout>
__global__ __launch_bounds__(512) void scan_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, int N, int T, int H,
    int HV, int dv, int max_chunks, const float* __restrict__ wsT, const float* __restrict__ wsG,
    const float* s0, float* sfin, Tout* __restrict__ o, float scale) {
    constexpr int C = kChunk;
    constexpr int BV = 32;
    constexpr int KP = DK + 8;   // padded row of K, Q, S (bf16)
    constexpr int TP = C + 8;    // padded row of the [*, C] tiles (bf16)
    constexpr int KQ_LOADS = DK / 64;   // uint4 per lane for K (and for Q)
    constexpr int NST = DK / 64;        // state tiles per wave

    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Qs[C * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Kt[DK * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Sh[BV * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Sl[BV * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Xh[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Xl[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Uh[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Ul[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Wh[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Wl[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Ph[C * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Pl[C * TP];
    __shared__ float Gs[C];

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int tb = w >> 1, ib = w & 1;
    const int tiles = dv / BV;
    // XCD-aware mapping: workgroup b runs on XCD b % 8; all tiles of a chain
    // get the same b % 8 and neighbouring dispatch slots
    const int b = blockIdx.x;
    const int slot = b >> 3;
    const int tile = slot % tiles;
    const int chain = (slot / tiles) * 8 + (b & 7);
    if (chain >= N * HV) return;
    const int n = chain / HV, h = chain - n * HV;
    const int hk = h / (HV / H);
    const size_t sbase = ((size_t)chain * dv + (size_t)tile * BV) * DK;

    // state: sacc[x][r] = S[i = 16 ibS + lr][j = 16 jb + 4 lg + r], tile index w + 8 x
    f4_t sacc[NST];
#pragma unroll
    for (int x = 0; x < NST; ++x) {
        const int ti = w + 8 * x, jb = ti >> 1, ibS = ti & 1;
        const size_t off = sbase + (size_t)(16 * ibS + lr) * DK + 16 * jb + 4 * lg;
        if (s0) {
            const float4 v4 = *reinterpret_cast<const float4*>(s0 + off);
            sacc[x] = f4_t{v4.x, v4.y, v4.z, v4.w};
        } else {
            sacc[x] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    auto store_state_lds = [&]() {
#pragma unroll
        for (int x = 0; x < NST; ++x) {
            const int ti = w + 8 * x, jb = ti >> 1, ibS = ti & 1;
            const int off = (16 * ibS + lr) * KP + 16 * jb + 4 * lg;
            __bf16 hi[4], lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) split1(sacc[x][r], hi[r], lo[r]);
            *reinterpret_cast<uint2*>(&Sh[off]) = *reinterpret_cast<const uint2*>(hi);
            *reinterpret_cast<uint2*>(&Sl[off]) = *reinterpret_cast<const uint2*>(lo);
        }
    };
    store_state_lds();

    int sq, eq;
    seq_bounds_m(cu, n, T, sq, eq);
    const int c_first = chunk_off[n];
    int nch = chunk_off[n + 1] - c_first;
    if (c_first + nch > max_chunks) nch = max(0, max_chunks - c_first);

    // ---- prefetch registers (branch-free: rows past the end are clamped on
    //      load and zeroed on use, so no load waits for another) ----
    uint4 pk[KQ_LOADS], pq[KQ_LOADS];
    float pT[2][8];     // T' row 16 tb + lr, columns 32 kk + 8 lg .. +7
    uint16_t pV[4];     // V[t = 16 tb + 4 lg + r][i = 16 ib + lr], raw bf16
    float pG = 0.f;     // G[l]
    auto prefetch = [&](int jc) {
        const int c = c_first + jc;
        const int t0 = sq + jc * C;
        const int L = min(C, eq - t0);
        const size_t row = (size_t)(t0 + min(l, L - 1)) * H + hk;
#pragma unroll
        for (int m = 0; m < KQ_LOADS; ++m) {
            const size_t off = row * DK + 8 * (w + 8 * m);
            pk[m] = *reinterpret_cast<const uint4*>(k + off);
            pq[m] = *reinterpret_cast<const uint4*>(q + off);
        }
        const float* Tp = wsT + (((size_t)c * HV + h) * C + 16 * tb + lr) * C + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float4 x0 = *reinterpret_cast<const float4*>(Tp + 32 * kk);
            const float4 x1 = *reinterpret_cast<const float4*>(Tp + 32 * kk + 4);
            pT[kk][0] = x0.x; pT[kk][1] = x0.y; pT[kk][2] = x0.z; pT[kk][3] = x0.w;
            pT[kk][4] = x1.x; pT[kk][5] = x1.y; pT[kk][6] = x1.z; pT[kk][7] = x1.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = min(16 * tb + 4 * lg + r, L - 1);
            pV[r] = v[((size_t)(t0 + t) * HV + h) * dv + tile * BV + 16 * ib + lr];
        }
        pG = wsG[((size_t)c * HV + h) * C + l];
    };
    if (nch > 0) prefetch(0);

    for (int jc = 0; jc < nch; ++jc) {
        const int t0 = sq + jc * C;
        const int L = min(C, eq - t0);
        // (1) chunk -> LDS: K, Q (row-major), K^T (token pairs packed per dword), G.
        // Lane l holds token l; its partner l ^ 1 holds the neighbouring token.
        const bool live = l < L;
#pragma unroll
        for (int m = 0; m < KQ_LOADS; ++m) {
            const int c8 = 8 * (w + 8 * m);
            const uint4 kv = live ? pk[m] : make_uint4(0, 0, 0, 0);
            const uint4 qv = live ? pq[m] : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(&Ks[l * KP + c8]) = kv;
            *reinterpret_cast<uint4*>(&Qs[l * KP + c8]) = qv;
            const uint32_t own[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t par = (uint32_t)__builtin_amdgcn_update_dpp(
                    0, (int)own[p], kDppQuadXor1, 0xF, 0xF, false);
                const bool even = (l & 1) == 0;
                const uint32_t word = even ? ((own[p] & 0xFFFFu) | (par << 16))
                                           : ((par >> 16) | (own[p] & 0xFFFF0000u));
                const int j = c8 + 2 * p + (even ? 0 : 1);
                *reinterpret_cast<uint32_t*>(&Kt[j * TP + (l & ~1)]) = word;
            }
        }
        if (tid < C) Gs[tid] = pG;
        float cT[2][8], cV[4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int x = 0; x < 8; ++x) cT[kk][x] = pT[kk][x];
#pragma unroll
        for (int r = 0; r < 4; ++r) cV[r] = (16 * tb + 4 * lg + r < L) ? bf16_to_f32(pV[r]) : 0.f;
        __syncthreads();
        if (jc + 1 < nch) prefetch(jc + 1);

        // (2) K S^T and Q S^T for tile (tb, ib); P^T tiles; X = V - diag(gamma) K S^T
        f4_t ksa = f4_t{0.f, 0.f, 0.f, 0.f}, qsa = f4_t{0.f, 0.f, 0.f, 0.f};
        f4_t pa[2] = {f4_t{0.f, 0.f, 0.f, 0.f}, f4_t{0.f, 0.f, 0.f, 0.f}};
        // P^T tiles (sb, tb) handled here: sb = ib and sb = ib + 2, when sb <= tb
        const bool p0 = ib <= tb, p1 = ib + 2 <= tb;
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const int col = 32 * kk + 8 * lg;
            const bf8_t ak = lds8(&Ks[(16 * tb + lr) * KP + col]);
            const bf8_t aq = lds8(&Qs[(16 * tb + lr) * KP + col]);
            const bf8_t bh = lds8(&Sh[(16 * ib + lr) * KP + col]);
            const bf8_t bl = lds8(&Sl[(16 * ib + lr) * KP + col]);
            ksa = mfma(ak, bh, ksa);
            ksa = mfma(ak, bl, ksa);
            qsa = mfma(aq, bh, qsa);
            qsa = mfma(aq, bl, qsa);
            if (p0) pa[0] = mfma(lds8(&Ks[(16 * ib + lr) * KP + col]), aq, pa[0]);
            if (p1) pa[1] = mfma(lds8(&Ks[(16 * (ib + 2) + lr) * KP + col]), aq, pa[1]);
        }
        // pa[x][r] = P^T[s = 16 sb + 4 lg + r][t = 16 tb + lr]
        {
            const int t = 16 * tb + lr;
            const float Gt = Gs[t];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int sb = ib + 2 * x;
                // tiles inside the k-range that the O product reads must be stored (zeros
                // above the diagonal); others are never read
                if ((sb >> 1) <= (tb >> 1)) {
                    const bool comp = sb <= tb;
                    __bf16 hi[4], lo[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int s = 16 * sb + 4 * lg + r;
                        const float pv = (comp && s <= t) ? pa[x][r] * __expf(Gt - Gs[s]) : 0.f;
                        split1(pv, hi[r], lo[r]);
                    }
                    const int off = t * TP + 16 * sb + 4 * lg;
                    *reinterpret_cast<uint2*>(&Ph[off]) = *reinterpret_cast<const uint2*>(hi);
                    *reinterpret_cast<uint2*>(&Pl[off]) = *reinterpret_cast<const uint2*>(lo);
                }
            }
        }
        float Gt4[4], gam[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            Gt4[r] = Gs[16 * tb + 4 * lg + r];
            gam[r] = __expf(Gt4[r]);
        }
        {
            __bf16 hi[4], lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) split1(cV[r] - gam[r] * ksa[r], hi[r], lo[r]);
            const int off = (16 * ib + lr) * TP + 16 * tb + 4 * lg;
            *reinterpret_cast<uint2*>(&Xh[off]) = *reinterpret_cast<const uint2*>(hi);
            *reinterpret_cast<uint2*>(&Xl[off]) = *reinterpret_cast<const uint2*>(lo);
        }
        __syncthreads();

        // (3) U = T' X for tile (tb, ib) (T' lower triangular: k-steps up to tb / 2)
        f4_t ua = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk <= (tb >> 1)) {
                bf8_t ah, al;
                split8(cT[kk], ah, al);
                const int col = 32 * kk + 8 * lg;
                const bf8_t bh = lds8(&Xh[(16 * ib + lr) * TP + col]);
                const bf8_t bl = lds8(&Xl[(16 * ib + lr) * TP + col]);
                ua = mfma(ah, bh, ua);
                ua = mfma(ah, bl, ua);
                ua = mfma(al, bh, ua);
            }
        }
        const float Gn = Gs[L - 1];
        {
            __bf16 hi[4], lo[4], whi[4], wlo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                split1(ua[r], hi[r], lo[r]);
                split1(ua[r] * __expf(Gn - Gt4[r]), whi[r], wlo[r]);
            }
            const int off = (16 * ib + lr) * TP + 16 * tb + 4 * lg;
            *reinterpret_cast<uint2*>(&Uh[off]) = *reinterpret_cast<const uint2*>(hi);
            *reinterpret_cast<uint2*>(&Ul[off]) = *reinterpret_cast<const uint2*>(lo);
            *reinterpret_cast<uint2*>(&Wh[off]) = *reinterpret_cast<const uint2*>(whi);
            *reinterpret_cast<uint2*>(&Wl[off]) = *reinterpret_cast<const uint2*>(wlo);
        }
        __syncthreads();

        // (4a) O = scale (diag(gamma) Q S^T + P U) for tile (tb, ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) qsa[r] *= gam[r];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk <= (tb >> 1)) {
                const int col = 32 * kk + 8 * lg;
                const bf8_t ah = lds8(&Ph[(16 * tb + lr) * TP + col]);
                const bf8_t al = lds8(&Pl[(16 * tb + lr) * TP + col]);
                const bf8_t bh = lds8(&Uh[(16 * ib + lr) * TP + col]);
                const bf8_t bl = lds8(&Ul[(16 * ib + lr) * TP + col]);
                qsa = mfma(ah, bh, qsa);
                qsa = mfma(ah, bl, qsa);
                qsa = mfma(al, bh, qsa);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tb + 4 * lg + r;
            if (t < L)
                io<Tout>::st(o + ((size_t)(t0 + t) * HV + h) * dv + tile * BV + 16 * ib + lr,
                             scale * qsa[r]);
        }

        // (4b) S'^T = gamma_n S^T + K^T U' for the wave's state tiles
        const float gn = __expf(Gn);
#pragma unroll
        for (int x = 0; x < NST; ++x) {
            const int ti = w + 8 * x, jb = ti >> 1, ibS = ti & 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[x][r] *= gn;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int col = 32 * kk + 8 * lg;
                const bf8_t ak = lds8(&Kt[(16 * jb + lr) * TP + col]);
                const bf8_t bh = lds8(&Wh[(16 * ibS + lr) * TP + col]);
                const bf8_t bl = lds8(&Wl[(16 * ibS + lr) * TP + col]);
                sacc[x] = mfma(ak, bh, sacc[x]);
                sacc[x] = mfma(ak, bl, sacc[x]);
            }
        }
        // Sh / Sl are read only in (2): each wave can refresh its part now
        store_state_lds();
        __syncthreads();
    }

    if (sfin) {
#pragma unroll
        for (int x = 0; x < NST; ++x) {
            const int ti = w + 8 * x, jb = ti >> 1, ibS = ti & 1;
            const size_t off = sbase + (size_t)(16 * ibS + lr) * DK + 16 * jb + 4 * lg;
            *reinterpret_cast<float4*>(sfin + off) =
                make_float4(sacc[x][0], sacc[x][1], sacc[x][2], sacc[x][3]);
        }
    }
}

template <int DK, typename Tout>
static hipError_t launch_mfma_t(const PrefillArgs& A) {
    hipLaunchKernelGGL((prep_mfma_kernel<DK>), dim3(A.max_chunks, A.H), dim3(256), 0, A.stream,
                       static_cast<const bf16_t*>(A.k), A.g, A.beta, A.cu_seqlens, A.chunk_off,
                       A.N, A.T, A.H, A.HV, A.max_chunks, A.ws_T, A.ws_G);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int tiles = A.dv / 32;
    const int chains = A.N * A.HV;
    const size_t blocks = (size_t)((chains + 7) / 8) * 8 * tiles;
    hipLaunchKernelGGL((scan_mfma_kernel<DK, Tout>), dim3((unsigned)blocks), dim3(512), 0,
                       A.stream, static_cast<const bf16_t*>(A.q), static_cast<const bf16_t*>(A.k),
                       static_cast<const bf16_t*>(A.v), A.cu_seqlens, A.chunk_off, A.N, A.T, A.H,
                       A.HV, A.dv, A.max_chunks, A.ws_T, A.ws_G, A.s0, A.s_final,
                       static_cast<Tout*>(A.o), A.scale);
    return hipGetLastError();
}

bool prefill_mfma_eligible(const PrefillArgs& A) {
    return A.in_bf16 && (A.dk == 64 || A.dk == 128) && (A.dv % 32 == 0);
}

hipError_t launch_prefill_mfma(const PrefillArgs& A) {
    if (A.dk == 64) return A.o_bf16 ? launch_mfma_t<64, bf16_t>(A) : launch_mfma_t<64, float>(A);
    return A.o_bf16 ? launch_mfma_t<128, bf16_t>(A) : launch_mfma_t<128, float>(A);
}

}  // namespace gdn

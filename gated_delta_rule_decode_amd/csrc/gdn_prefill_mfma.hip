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
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * KP];
    __shared__ float Am[C][C + 1];
    __shared__ float Tm[C][C + 1];
    __shared__ float Xb[3][16][17];
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

    // K chunk -> LDS (zero rows past the sequence end)
    for (int idx = tid; idx < C * DK / 8; idx += 256) {
        const int t = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
        uint4 val = make_uint4(0, 0, 0, 0);
        if (t < L) val = *reinterpret_cast<const uint4*>(k + ((size_t)(t0 + t) * H + hk) * DK + c8);
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
            float gv = l < L ? g[(size_t)(t0 + l) * HV + hv] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float up = __shfl_up(gv, off, 64);
                if (l >= off) gv += up;
            }
            Gs[l] = gv;
            Bs[l] = l < L ? beta[(size_t)(t0 + l) * HV + hv] : 0.f;
        }
        __syncthreads();
        // A (strictly lower part of the blocks this wave computed)
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if (sb <= w) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + 4 * lg + r, s = 16 * sb + lr;
                    Am[t][s] = (s < t) ? Bs[t] * __expf(Gs[t] - Gs[s]) * kk[sb][r] : 0.f;
                }
            }
        }
        __syncthreads();
        // diagonal 16 x 16 blocks by forward substitution: wave b, lane j = column
        if (lr == l) {  // lanes 0..15 of every wave
            const int b = w;
            float col[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float v = (t == lr) ? 1.f : 0.f;
#pragma unroll
                for (int x = 0; x < t; ++x) v -= Am[16 * b + t][16 * b + x] * col[x];
                col[t] = v;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) Tm[16 * b + t][16 * b + lr] = col[t];
        }
        __syncthreads();
        // off-diagonal blocks, block row by block row
        for (int i = 1; i < 4; ++i) {
            // X_j = sum_{k=j}^{i-1} A_ik T_kj for j < i
            for (int e = tid; e < i * 256; e += 256) {
                const int j = e >> 8, rho = (e >> 4) & 15, kap = e & 15;
                float acc = 0.f;
                for (int kb = j; kb < i; ++kb) {
#pragma unroll
                    for (int x = 0; x < 16; ++x)
                        acc += Am[16 * i + rho][16 * kb + x] * Tm[16 * kb + x][16 * j + kap];
                }
                Xb[j][rho][kap] = acc;
            }
            __syncthreads();
            // T_ij = -T_ii X_j
            for (int e = tid; e < i * 256; e += 256) {
                const int j = e >> 8, rho = (e >> 4) & 15, kap = e & 15;
                float acc = 0.f;
                for (int x = 0; x <= rho; ++x) acc += Tm[16 * i + rho][16 * i + x] * Xb[j][x][kap];
                Tm[16 * i + rho][16 * j + kap] = -acc;
            }
            __syncthreads();
        }
        // T' = T diag(b) (lower triangle; zeros above), and G
        float* To = wsT + ((size_t)c * HV + hv) * C * C;
        for (int idx = tid; idx < C * C; idx += 256) {
            const int t = idx >> 6, s = idx & 63;
            To[idx] = (s <= t) ? Tm[t][s] * Bs[s] : 0.f;
        }
        if (tid < C) wsG[((size_t)c * HV + hv) * C + tid] = Gs[tid];
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// scan: sequential over chunks, state tile in MFMA accumulators
// ---------------------------------------------------------------------------
template <int DK, typename Tout>
__global__ __launch_bounds__(256) void scan_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, int N, int T, int H,
    int HV, int dv, int max_chunks, const float* __restrict__ wsT, const float* __restrict__ wsG,
    const float* s0, float* sfin, Tout* __restrict__ o, float scale) {
    constexpr int C = kChunk;
    constexpr int BV = 32;
    constexpr int KP = DK + 8;   // padded row of K, Q, S (bf16)
    constexpr int TP = C + 8;    // padded row of transposed [*, C] tiles (bf16)
    constexpr int NJB = DK / 16 / 4;  // 16-column blocks of S per wave
    constexpr int KQ_LOADS = C * DK / 8 / 256;  // uint4 per thread for K (and for Q)

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

    // state tiles owned by this wave: rows 16 ib + 4 lg + r, columns 16 (NJB w + jj) + lr
    f4_t sacc[2][NJB];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jj = 0; jj < NJB; ++jj) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ib + 4 * lg + r, j = 16 * (NJB * w + jj) + lr;
                sacc[ib][jj][r] = s0 ? s0[sbase + (size_t)i * DK + j] : 0.f;
            }
        }
    auto store_state_lds = [&]() {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int jj = 0; jj < NJB; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * ib + 4 * lg + r, j = 16 * (NJB * w + jj) + lr;
                    __bf16 hi, lo;
                    split1(sacc[ib][jj][r], hi, lo);
                    Sh[i * KP + j] = hi;
                    Sl[i * KP + j] = lo;
                }
    };
    store_state_lds();

    int sq, eq;
    seq_bounds_m(cu, n, T, sq, eq);
    const int c_first = chunk_off[n];
    int nch = chunk_off[n + 1] - c_first;
    if (c_first + nch > max_chunks) nch = max(0, max_chunks - c_first);

    // ---- prefetch registers ----
    uint4 pk[KQ_LOADS], pq[KQ_LOADS];
    float pT[2][8];     // T' row 16 w + lr, columns 32 kk + 8 lg .. +7
    float pV[2][4];     // V[t = 16 w + 4 lg + r][i = 16 ib + lr]
    float pG = 0.f;
    auto prefetch = [&](int jc) {
        const int c = c_first + jc;
        const int t0 = sq + jc * C;
        const int L = min(C, eq - t0);
#pragma unroll
        for (int m = 0; m < KQ_LOADS; ++m) {
            const int idx = tid + 256 * m;
            const int t = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
            if (t < L) {
                const size_t off = ((size_t)(t0 + t) * H + hk) * DK + c8;
                pk[m] = *reinterpret_cast<const uint4*>(k + off);
                pq[m] = *reinterpret_cast<const uint4*>(q + off);
            } else {
                pk[m] = make_uint4(0, 0, 0, 0);
                pq[m] = make_uint4(0, 0, 0, 0);
            }
        }
        const float* Tp = wsT + (((size_t)c * HV + h) * C + 16 * w + lr) * C + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float4 x0 = *reinterpret_cast<const float4*>(Tp + 32 * kk);
            const float4 x1 = *reinterpret_cast<const float4*>(Tp + 32 * kk + 4);
            pT[kk][0] = x0.x; pT[kk][1] = x0.y; pT[kk][2] = x0.z; pT[kk][3] = x0.w;
            pT[kk][4] = x1.x; pT[kk][5] = x1.y; pT[kk][6] = x1.z; pT[kk][7] = x1.w;
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * lg + r;
                pV[ib][r] = t < L ? bf16_to_f32(v[((size_t)(t0 + t) * HV + h) * dv + tile * BV +
                                                  16 * ib + lr])
                                  : 0.f;
            }
        if (tid < C) pG = wsG[((size_t)c * HV + h) * C + tid];
    };
    if (nch > 0) prefetch(0);

    for (int jc = 0; jc < nch; ++jc) {
        const int t0 = sq + jc * C;
        const int L = min(C, eq - t0);
        // (1) chunk -> LDS: K, Q (row-major), K^T, G
#pragma unroll
        for (int m = 0; m < KQ_LOADS; ++m) {
            const int idx = tid + 256 * m;
            const int t = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
            *reinterpret_cast<uint4*>(&Ks[t * KP + c8]) = pk[m];
            *reinterpret_cast<uint4*>(&Qs[t * KP + c8]) = pq[m];
            const uint32_t wds[4] = {pk[m].x, pk[m].y, pk[m].z, pk[m].w};
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const uint16_t bits = static_cast<uint16_t>(wds[x >> 1] >> (16 * (x & 1)));
                Kt[(c8 + x) * TP + t] = __builtin_bit_cast(__bf16, bits);
            }
        }
        if (tid < C) Gs[tid] = pG;
        float cT[2][8], cV[2][4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int x = 0; x < 8; ++x) cT[kk][x] = pT[kk][x];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) cV[ib][r] = pV[ib][r];
        __syncthreads();
        if (jc + 1 < nch) prefetch(jc + 1);

        // (2) K S^T, Q S^T (row block w), Q K^T -> P, X = V - diag(gamma) K S^T
        f4_t ksa[2], qsa[2], pa[4];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            ksa[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
            qsa[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) pa[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const int col = 32 * kk + 8 * lg;
            const bf8_t ak = lds8(&Ks[(16 * w + lr) * KP + col]);
            const bf8_t aq = lds8(&Qs[(16 * w + lr) * KP + col]);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const bf8_t bh = lds8(&Sh[(16 * ib + lr) * KP + col]);
                const bf8_t bl = lds8(&Sl[(16 * ib + lr) * KP + col]);
                ksa[ib] = mfma(ak, bh, ksa[ib]);
                ksa[ib] = mfma(ak, bl, ksa[ib]);
                qsa[ib] = mfma(aq, bh, qsa[ib]);
                qsa[ib] = mfma(aq, bl, qsa[ib]);
            }
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (sb <= w) {
                    const bf8_t bk = lds8(&Ks[(16 * sb + lr) * KP + col]);
                    pa[sb] = mfma(aq, bk, pa[sb]);
                }
            }
        }
        float Gt[4], gam[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            Gt[r] = Gs[16 * w + 4 * lg + r];
            gam[r] = __expf(Gt[r]);
        }
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const float Gsb = Gs[16 * sb + lr];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * lg + r, s = 16 * sb + lr;
                const float p = (sb <= w && s <= t) ? pa[sb][r] * __expf(Gt[r] - Gsb) : 0.f;
                __bf16 hi, lo;
                split1(p, hi, lo);
                Ph[t * TP + s] = hi;
                Pl[t * TP + s] = lo;
            }
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * lg + r, i = 16 * ib + lr;
                const float x = cV[ib][r] - gam[r] * ksa[ib][r];
                __bf16 hi, lo;
                split1(x, hi, lo);
                Xh[i * TP + t] = hi;
                Xl[i * TP + t] = lo;
            }
        __syncthreads();

        // (3) U = T' X for row block w (T' is lower triangular: k-steps up to w / 2)
        f4_t ua[2];
        ua[0] = f4_t{0.f, 0.f, 0.f, 0.f};
        ua[1] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk <= (w >> 1)) {
                bf8_t ah, al;
                split8(cT[kk], ah, al);
                const int col = 32 * kk + 8 * lg;
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const bf8_t bh = lds8(&Xh[(16 * ib + lr) * TP + col]);
                    const bf8_t bl = lds8(&Xl[(16 * ib + lr) * TP + col]);
                    ua[ib] = mfma(ah, bh, ua[ib]);
                    ua[ib] = mfma(ah, bl, ua[ib]);
                    ua[ib] = mfma(al, bh, ua[ib]);
                }
            }
        }
        const float Gn = Gs[L - 1];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * lg + r, i = 16 * ib + lr;
                __bf16 hi, lo;
                split1(ua[ib][r], hi, lo);
                Uh[i * TP + t] = hi;
                Ul[i * TP + t] = lo;
                split1(ua[ib][r] * __expf(Gn - Gt[r]), hi, lo);
                Wh[i * TP + t] = hi;
                Wl[i * TP + t] = lo;
            }
        __syncthreads();

        // (4a) O = scale (diag(gamma) Q S^T + P U) for row block w
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) qsa[ib][r] *= gam[r];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk <= (w >> 1)) {
                const int col = 32 * kk + 8 * lg;
                const bf8_t ah = lds8(&Ph[(16 * w + lr) * TP + col]);
                const bf8_t al = lds8(&Pl[(16 * w + lr) * TP + col]);
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const bf8_t bh = lds8(&Uh[(16 * ib + lr) * TP + col]);
                    const bf8_t bl = lds8(&Ul[(16 * ib + lr) * TP + col]);
                    qsa[ib] = mfma(ah, bh, qsa[ib]);
                    qsa[ib] = mfma(ah, bl, qsa[ib]);
                    qsa[ib] = mfma(al, bh, qsa[ib]);
                }
            }
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * lg + r;
                if (t < L)
                    io<Tout>::st(o + ((size_t)(t0 + t) * HV + h) * dv + tile * BV + 16 * ib + lr,
                                 scale * qsa[ib][r]);
            }

        // (4b) S' = gamma_n S + U'^T K for the wave's state tiles
        const float gn = __expf(Gn);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int jj = 0; jj < NJB; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[ib][jj][r] *= gn;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int col = 32 * kk + 8 * lg;
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const bf8_t ah = lds8(&Wh[(16 * ib + lr) * TP + col]);
                const bf8_t al = lds8(&Wl[(16 * ib + lr) * TP + col]);
#pragma unroll
                for (int jj = 0; jj < NJB; ++jj) {
                    const bf8_t bk = lds8(&Kt[(16 * (NJB * w + jj) + lr) * TP + col]);
                    sacc[ib][jj] = mfma(ah, bk, sacc[ib][jj]);
                    sacc[ib][jj] = mfma(al, bk, sacc[ib][jj]);
                }
            }
        }
        __syncthreads();
        store_state_lds();
    }

    if (sfin) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int jj = 0; jj < NJB; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * ib + 4 * lg + r, j = 16 * (NJB * w + jj) + lr;
                    sfin[sbase + (size_t)i * DK + j] = sacc[ib][jj][r];
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
    hipLaunchKernelGGL((scan_mfma_kernel<DK, Tout>), dim3((unsigned)blocks), dim3(256), 0,
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

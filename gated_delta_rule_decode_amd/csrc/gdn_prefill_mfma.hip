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
// Work split.  Everything that does not depend on the state runs
// chunk-parallel in prep_mfma: per (chunk, key head) K K^T and Q K^T, and per
// value head of that key head G, the triangular inverse, T' and P, stored
// pre-split as hi/lo bf16 row-major tiles, plus K^T of the chunk.  The
// sequential scan_mfma then only runs the state-dependent products, reading
// its T', P, K, Q and K^T fragments straight from memory into registers one
// chunk ahead; LDS holds just the state tile and the X, U, U' exchange tiles.
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

__device__ __forceinline__ bf8_t zero8() { return __builtin_bit_cast(bf8_t, make_uint4(0, 0, 0, 0)); }

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

// 4 consecutive floats -> 8-byte hi and lo words
__device__ __forceinline__ void split4(const float* x, uint2& hi, uint2& lo) {
    __bf16 h[4], o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) split1(x[r], h[r], o[r]);
    hi = *reinterpret_cast<const uint2*>(h);
    lo = *reinterpret_cast<const uint2*>(o);
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
// prep: everything that does not depend on the state, chunk-parallel
// ---------------------------------------------------------------------------
// One workgroup (4 wavefronts) per (chunk, key head).  Wave w owns row block
// w (tokens 16 w .. 16 w + 15) of K K^T and of P.  Outputs per value head:
// T' and P as hi/lo bf16 row-major 64 x 64 tiles (zeros above the diagonal and
// in rows / columns past the sequence end) and G; per key head: K^T (dk x 64).
template <int DK>
__global__ __launch_bounds__(256) void prep_mfma_kernel(const PrefillArgs A) {
    constexpr int C = kChunk;
    constexpr int KP = DK + 8;  // padded bf16 row
    constexpr int AP = C + 4;   // padded fp32 row (16-byte aligned rows)
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Qs[C * KP];
    __shared__ __attribute__((aligned(16))) float Am[C * AP];
    __shared__ __attribute__((aligned(16))) float Tm[C * AP];
    __shared__ __attribute__((aligned(16))) float Xm[32 * 36];
    __shared__ float Gs[C], Bs[C];

    const int H = A.H, HV = A.HV;
    const int c = blockIdx.x, hk = blockIdx.y, tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int total = min(A.chunk_off[A.N], A.max_chunks);
    if (c >= total) return;
    const int n = find_seq_m(A.chunk_off, A.N, c);
    int s0, e0;
    seq_bounds_m(A.cu_seqlens, n, A.T, s0, e0);
    const int t0 = s0 + (c - A.chunk_off[n]) * C;
    const int L = min(C, e0 - t0);
    const int ratio = HV / H;
    const bf16_t* k = static_cast<const bf16_t*>(A.k);
    const bf16_t* q = static_cast<const bf16_t*>(A.q);

    // K and Q chunk -> LDS (rows past the sequence end are zero)
    for (int idx = tid; idx < C * DK / 8; idx += 256) {
        const int t = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
        const size_t off = ((size_t)(t0 + min(t, L - 1)) * H + hk) * DK + c8;
        uint4 kv = *reinterpret_cast<const uint4*>(k + off);
        uint4 qv = *reinterpret_cast<const uint4*>(q + off);
        if (t >= L) kv = qv = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(&Ks[t * KP + c8]) = kv;
        *reinterpret_cast<uint4*>(&Qs[t * KP + c8]) = qv;
    }
    __syncthreads();

    // K^T of the chunk -> workspace, [dk][64] bf16
    {
        uint16_t* Kt = A.ws_Kt + ((size_t)c * H + hk) * DK * C;
        const uint16_t* Kr = reinterpret_cast<const uint16_t*>(Ks);
        for (int idx = tid; idx < DK * C / 8; idx += 256) {
            const int t8 = 8 * (idx % (C / 8)), j = idx / (C / 8);
            uint32_t wd[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                wd[x] = (uint32_t)Kr[(t8 + 2 * x) * KP + j] |
                        ((uint32_t)Kr[(t8 + 2 * x + 1) * KP + j] << 16);
            *reinterpret_cast<uint4*>(Kt + (size_t)j * C + t8) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        }
    }

    // K K^T (row block w, column blocks sb <= w) and P^T = K Q^T (column block w)
    f4_t kk[4], pq[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        kk[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
        pq[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        const int col = 32 * ks + 8 * lg;
        const bf8_t ka = lds8(&Ks[(16 * w + lr) * KP + col]);
        const bf8_t qa = lds8(&Qs[(16 * w + lr) * KP + col]);
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if (sb <= w) {
                const bf8_t kb = lds8(&Ks[(16 * sb + lr) * KP + col]);
                kk[sb] = mfma(ka, kb, kk[sb]);
                pq[sb] = mfma(kb, qa, pq[sb]);
            }
        }
    }
    // kk[sb][r] = (K K^T)[t = 16 w + 4 lg + r][s = 16 sb + lr]
    // pq[sb][r] = (Q K^T)[t = 16 w + lr][s = 16 sb + 4 lg + r]

    for (int hv = hk * ratio; hv < (hk + 1) * ratio; ++hv) {
        const size_t tileoff = ((size_t)c * HV + hv) * C * C;
        // G = in-chunk inclusive cumsum of g (wave 0), beta
        if (w == 0) {
            float gv = A.g[(size_t)(t0 + min(l, L - 1)) * HV + hv];
            float bv = A.beta[(size_t)(t0 + min(l, L - 1)) * HV + hv];
            if (l >= L) gv = 0.f, bv = 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float up = __shfl_up(gv, off, 64);
                if (l >= off) gv += up;
            }
            Gs[l] = gv;
            Bs[l] = bv;
            A.ws_G[((size_t)c * HV + hv) * C + l] = gv;
        }
        __syncthreads();
        // P = tril(Q K^T) o e^{G_t - G_s}: row block w, all column blocks, hi / lo
        {
            const int t = 16 * w + lr;
            const float Gt = Gs[t];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                float pv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * sb + 4 * lg + r;
                    pv[r] = (sb <= w && s <= t) ? pq[sb][r] * __expf(Gt - Gs[s]) : 0.f;
                }
                uint2 hi, lo;
                split4(pv, hi, lo);
                const size_t off = tileoff + (size_t)t * C + 16 * sb + 4 * lg;
                *reinterpret_cast<uint2*>(A.ws_Ph + off) = hi;
                *reinterpret_cast<uint2*>(A.ws_Pl + off) = lo;
            }
        }
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
                bv[x] = (xr >= cc) ? Tm[xr * AP + cc] : 0.f;
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
        // T' = T diag(b) (lower triangle; zeros above) as hi / lo
        for (int idx = tid; idx < C * C / 4; idx += 256) {
            const int t = idx >> 4, s4 = 4 * (idx & 15);
            float tv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                tv[r] = (s4 + r <= t) ? Tm[t * AP + s4 + r] * Bs[s4 + r] : 0.f;
            uint2 hi, lo;
            split4(tv, hi, lo);
            *reinterpret_cast<uint2*>(A.ws_Th + tileoff + t * C + s4) = hi;
            *reinterpret_cast<uint2*>(A.ws_Tl + tileoff + t * C + s4) = lo;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// scan: sequential over chunks, state tile in MFMA accumulators
// ---------------------------------------------------------------------------
// 4 wavefronts, one per SIMD.  Wave w owns the chunk's row block tb = w
// (tokens 16 w .. 16 w + 15) in K S^T, Q S^T, X, U and O for both 16-column
// halves ib = 0, 1 of the state tile's 32 rows, so its K, Q, T', P row
// fragments are loaded once; and the state tiles S^T[16 jb .. +15][16 ibS ..]
// for its DK/64 column blocks jb and both halves ibS.
// Per chunk: (A) K S^T, Q S^T, X -> LDS; (B) U = T' X, U and U' -> LDS;
// (C) O = gamma Q S^T + P U to memory and S' = gamma_n S + U'^T K -> LDS.
// Operand fragments that come from memory are held in one register set: each
// group is reloaded for the next chunk right after its last use in this one
// (K, Q and G after (A), T' after (B), P after the output product, K^T after
// the state update), so every load has a full chunk to arrive and the loads
// are spread over the chunk instead of queueing at its start.  No branch
// surrounds a load or store (masked rows use clamped loads and out-of-range
// buffer stores), so the compiler waits for exactly the group it needs.
template <int DK, typename Tout>
__global__ __launch_bounds__(256) void scan_mfma_kernel(const PrefillArgs A) {
    constexpr int C = kChunk;
    constexpr int BV = 32;
    constexpr int KP = DK + 8;   // padded row of S (bf16)
    constexpr int TP = C + 8;    // padded row of the [*, C] tiles (bf16)
    constexpr int NKK = DK / 32;
    constexpr int NJB = DK / 64;  // state column blocks per wave

    __shared__ __attribute__((aligned(16))) __bf16 Sh[BV * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Sl[BV * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Xh[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Xl[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Uh[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Ul[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Wh[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Wl[BV * TP];

    const int H = A.H, HV = A.HV, dv = A.dv, N = A.N;
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int tb = w;
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
    const bf16_t* kp = static_cast<const bf16_t*>(A.k);
    const bf16_t* qp = static_cast<const bf16_t*>(A.q);
    const bf16_t* vp = static_cast<const bf16_t*>(A.v);
    Tout* op = static_cast<Tout*>(A.o);

    // state: sacc[x][ibS][r] = S[i = 16 ibS + lr][j = 16 (NJB w + x) + 4 lg + r]
    f4_t sacc[NJB][2];
#pragma unroll
    for (int x = 0; x < NJB; ++x)
#pragma unroll
        for (int ibS = 0; ibS < 2; ++ibS) {
            const size_t off = sbase + (size_t)(16 * ibS + lr) * DK + 16 * (NJB * w + x) + 4 * lg;
            if (A.s0) {
                const float4 v4 = *reinterpret_cast<const float4*>(A.s0 + off);
                sacc[x][ibS] = f4_t{v4.x, v4.y, v4.z, v4.w};
            } else {
                sacc[x][ibS] = f4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    auto store_state_lds = [&]() {
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ibS = 0; ibS < 2; ++ibS) {
                const int off = (16 * ibS + lr) * KP + 16 * (NJB * w + x) + 4 * lg;
                float sv[4] = {sacc[x][ibS][0], sacc[x][ibS][1], sacc[x][ibS][2], sacc[x][ibS][3]};
                uint2 hi, lo;
                split4(sv, hi, lo);
                *reinterpret_cast<uint2*>(&Sh[off]) = hi;
                *reinterpret_cast<uint2*>(&Sl[off]) = lo;
            }
    };
    store_state_lds();

    int sq, eq;
    seq_bounds_m(A.cu_seqlens, n, A.T, sq, eq);
    const int c_first = A.chunk_off[n];
    int nch = A.chunk_off[n + 1] - c_first;
    if (c_first + nch > A.max_chunks) nch = max(0, A.max_chunks - c_first);
    if (nch <= 0) {
        if (A.s_final) {
#pragma unroll
            for (int x = 0; x < NJB; ++x)
#pragma unroll
                for (int ibS = 0; ibS < 2; ++ibS) {
                    const size_t off = sbase + (size_t)(16 * ibS + lr) * DK + 16 * (NJB * w + x) + 4 * lg;
                    *reinterpret_cast<float4*>(A.s_final + off) =
                        make_float4(sacc[x][ibS][0], sacc[x][ibS][1], sacc[x][ibS][2], sacc[x][ibS][3]);
                }
        }
        return;
    }

    // ---- operand fragments (one set; groups reloaded after their last use) ----
    bf8_t kA[NKK], qA[NKK];      // K, Q row 16 tb + lr, k-step kk
    bf8_t tH[2], tL[2];          // T' row 16 tb + lr, columns 32 kk + 8 lg ..
    bf8_t pH[2], pL[2];          // P row 16 tb + lr
    bf8_t ktA[NJB][2];           // K^T row 16 jb + lr, tokens 32 kk + 8 lg ..
    uint32_t vr[2][4];           // V[t = 16 tb + 4 lg + r][i = 16 ib + lr], raw bf16 bits
    float4 gR;                   // G[16 tb + 4 lg + r]
    float gN;                    // G[L - 1]

    auto chunk_t0 = [&](int jc) { return sq + jc * C; };
    auto chunk_L = [&](int jc) { return min(C, eq - (sq + jc * C)); };
    auto load_kq_g = [&](int jc) {
        const int t0 = chunk_t0(jc), L = chunk_L(jc);
        const size_t krow = ((size_t)(t0 + min(16 * tb + lr, L - 1)) * H + hk) * DK + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            kA[kk] = __builtin_bit_cast(bf8_t, *reinterpret_cast<const uint4*>(kp + krow + 32 * kk));
            qA[kk] = __builtin_bit_cast(bf8_t, *reinterpret_cast<const uint4*>(qp + krow + 32 * kk));
        }
        const float* G = A.ws_G + ((size_t)(c_first + jc) * HV + h) * C;
        gR = *reinterpret_cast<const float4*>(G + 16 * tb + 4 * lg);
        gN = G[L - 1];
    };
    auto load_v = [&](int jc) {
        const int t0 = chunk_t0(jc), L = chunk_L(jc);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = min(16 * tb + 4 * lg + r, L - 1);
                vr[ib][r] = vp[((size_t)(t0 + t) * HV + h) * dv + tile * BV + 16 * ib + lr];
            }
    };
    auto tile_off = [&](int jc) {
        return (((size_t)(c_first + jc) * HV + h) * C + 16 * tb + lr) * C + 8 * lg;
    };
    auto load_t = [&](int jc) {
        const size_t toff = tile_off(jc);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            tH[kk] = gld8(A.ws_Th + toff + 32 * kk);
            tL[kk] = gld8(A.ws_Tl + toff + 32 * kk);
        }
    };
    auto load_p = [&](int jc) {
        const size_t toff = tile_off(jc);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            pH[kk] = gld8(A.ws_Ph + toff + 32 * kk);
            pL[kk] = gld8(A.ws_Pl + toff + 32 * kk);
        }
    };
    auto load_kt = [&](int jc) {
        const uint16_t* Kt = A.ws_Kt + ((size_t)(c_first + jc) * H + hk) * DK * C;
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                ktA[x][kk] = gld8(Kt + (size_t)(16 * (NJB * w + x) + lr) * C + 32 * kk + 8 * lg);
    };
    load_kq_g(0);
    load_v(0);
    load_t(0);
    load_p(0);
    load_kt(0);

    for (int jc = 0; jc < nch; ++jc) {
        const int nj = min(jc + 1, nch - 1);  // the last chunk re-reads itself
        const int t0 = chunk_t0(jc);
        const int L = chunk_L(jc);
        const bool rowlive = 16 * tb + lr < L;  // K / Q row of this lane's A fragments
        const float gr[4] = {gR.x, gR.y, gR.z, gR.w};
        const float gNc = gN;
        float gam[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) gam[r] = __expf(gr[r]);

        // (A) K S^T and Q S^T for row block tb, both column halves; X = V - diag(gamma) K S^T
        f4_t ksa[2], qsa[2];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            ksa[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
            qsa[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int col = 32 * kk + 8 * lg;
            const bf8_t ak = rowlive ? kA[kk] : zero8();
            const bf8_t aq = rowlive ? qA[kk] : zero8();
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const bf8_t bh = lds8(&Sh[(16 * ib + lr) * KP + col]);
                const bf8_t bl = lds8(&Sl[(16 * ib + lr) * KP + col]);
                ksa[ib] = mfma(ak, bh, ksa[ib]);
                qsa[ib] = mfma(aq, bh, qsa[ib]);
                ksa[ib] = mfma(ak, bl, ksa[ib]);
                qsa[ib] = mfma(aq, bl, qsa[ib]);
            }
        }
        load_kq_g(nj);
        float vf[2][4];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) vf[ib][r] = __uint_as_float(vr[ib][r] << 16);
        load_v(nj);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            float xv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                xv[r] = (16 * tb + 4 * lg + r < L) ? vf[ib][r] - gam[r] * ksa[ib][r] : 0.f;
            uint2 hi, lo;
            split4(xv, hi, lo);
            const int off = (16 * ib + lr) * TP + 16 * tb + 4 * lg;
            *reinterpret_cast<uint2*>(&Xh[off]) = hi;
            *reinterpret_cast<uint2*>(&Xl[off]) = lo;
        }
        __syncthreads();

        // (B) U = T' X for row block tb (T' is lower triangular: k-steps up to tb / 2)
        f4_t ua[2] = {f4_t{0.f, 0.f, 0.f, 0.f}, f4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk <= (tb >> 1)) {
                const int col = 32 * kk + 8 * lg;
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const bf8_t bh = lds8(&Xh[(16 * ib + lr) * TP + col]);
                    const bf8_t bl = lds8(&Xl[(16 * ib + lr) * TP + col]);
                    ua[ib] = mfma(tH[kk], bh, ua[ib]);
                    ua[ib] = mfma(tH[kk], bl, ua[ib]);
                    ua[ib] = mfma(tL[kk], bh, ua[ib]);
                }
            }
        }
        load_t(nj);
        {
            float dec[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) dec[r] = __expf(gNc - gr[r]);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                float uv[4], wv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uv[r] = ua[ib][r];
                    wv[r] = ua[ib][r] * dec[r];
                }
                uint2 hi, lo;
                const int off = (16 * ib + lr) * TP + 16 * tb + 4 * lg;
                split4(uv, hi, lo);
                *reinterpret_cast<uint2*>(&Uh[off]) = hi;
                *reinterpret_cast<uint2*>(&Ul[off]) = lo;
                split4(wv, hi, lo);
                *reinterpret_cast<uint2*>(&Wh[off]) = hi;
                *reinterpret_cast<uint2*>(&Wl[off]) = lo;
            }
        }
        __syncthreads();

        // (C1) O = scale (diag(gamma) Q S^T + P U) for row block tb
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) qsa[ib][r] *= gam[r];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk <= (tb >> 1)) {
                const int col = 32 * kk + 8 * lg;
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const bf8_t bh = lds8(&Uh[(16 * ib + lr) * TP + col]);
                    const bf8_t bl = lds8(&Ul[(16 * ib + lr) * TP + col]);
                    qsa[ib] = mfma(pH[kk], bh, qsa[ib]);
                    qsa[ib] = mfma(pH[kk], bl, qsa[ib]);
                    qsa[ib] = mfma(pL[kk], bh, qsa[ib]);
                }
            }
        }
        load_p(nj);
        {
            // rows t >= L land at or past the resource end and are dropped
            const __amdgpu_buffer_rsrc_t orsrc =
                out_rsrc(op + (size_t)t0 * HV * dv, (uint32_t)(L * HV * dv * sizeof(Tout)));
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tb + 4 * lg + r;
                    out_store(orsrc, (uint32_t)((t * HV + h) * dv + tile * BV + 16 * ib + lr),
                              A.scale * qsa[ib][r], op);
                }
        }
        // (C2) S'^T = gamma_n S^T + K^T U' for the wave's state tiles
        const float gn = __expf(gNc);
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ibS = 0; ibS < 2; ++ibS) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[x][ibS][r] *= gn;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int col = 32 * kk + 8 * lg;
                    const bf8_t bh = lds8(&Wh[(16 * ibS + lr) * TP + col]);
                    const bf8_t bl = lds8(&Wl[(16 * ibS + lr) * TP + col]);
                    sacc[x][ibS] = mfma(ktA[x][kk], bh, sacc[x][ibS]);
                    sacc[x][ibS] = mfma(ktA[x][kk], bl, sacc[x][ibS]);
                }
            }
        load_kt(nj);
        // Sh / Sl are read only in (A): each wave refreshes its part now
        store_state_lds();
        __syncthreads();
    }

    if (A.s_final) {
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ibS = 0; ibS < 2; ++ibS) {
                const size_t off = sbase + (size_t)(16 * ibS + lr) * DK + 16 * (NJB * w + x) + 4 * lg;
                *reinterpret_cast<float4*>(A.s_final + off) =
                    make_float4(sacc[x][ibS][0], sacc[x][ibS][1], sacc[x][ibS][2], sacc[x][ibS][3]);
            }
    }
}

template <int DK, typename Tout>
static hipError_t launch_mfma_t(const PrefillArgs& A) {
    hipLaunchKernelGGL((prep_mfma_kernel<DK>), dim3(A.max_chunks, A.H), dim3(256), 0, A.stream, A);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int tiles = A.dv / 32;
    const int chains = A.N * A.HV;
    const size_t blocks = (size_t)((chains + 7) / 8) * 8 * tiles;
    hipLaunchKernelGGL((scan_mfma_kernel<DK, Tout>), dim3((unsigned)blocks), dim3(256), 0,
                       A.stream, A);
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

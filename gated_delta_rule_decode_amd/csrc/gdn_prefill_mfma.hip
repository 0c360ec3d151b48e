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
// prep_mfma: per (chunk, key head) K K^T, and per value head of that key head
// G, the triangular inverse and T', stored pre-split as hi/lo bf16 row-major
// tiles.  The sequential scan_mfma runs the rest: K S^T, Q S^T, the causal
// Q K^T (computed again per chunk: it costs less MFMA time than the HBM bytes
// of storing P), U = T' X, O and the state update.  It reads K, Q, V, G and T'
// fragments straight from memory into registers one chunk ahead; LDS holds
// the state tile, the X, U, U' exchange tiles and the chunk's K rows.
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

// exponentials of log-decay differences: G is kept in log2 units (g log2 e),
// so e^{G_t - G_s} is one hardware exp2
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2f_(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

// two floats -> packed hi and lo bf16 words (one conversion per word)
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{x0, x1}, bf2_t));
    const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{x0 - h0, x1 - h1}, bf2_t));
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

// Raw buffer loads: the resource covers exactly the valid rows of a chunk, so
// rows past a sequence end read as zero without a clamp or a select.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t in_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ bf8_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf8_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
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
// w (tokens 16 w .. 16 w + 15) of K K^T.  Outputs per value head: T' as hi/lo
// bf16 row-major 64 x 64 tiles (zeros above the diagonal and in rows /
// columns past the sequence end) and G.
template <int DK>
__global__ __launch_bounds__(256) void prep_mfma_kernel(const PrefillArgs A) {
    constexpr int C = kChunk;
    constexpr int KP = DK + 8;  // padded bf16 row
    constexpr int AP = C + 4;   // padded fp32 row (16-byte aligned rows)
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * KP];
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

    // K chunk -> LDS (rows past the sequence end are zero)
    for (int idx = tid; idx < C * DK / 8; idx += 256) {
        const int t = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
        const size_t off = ((size_t)(t0 + min(t, L - 1)) * H + hk) * DK + c8;
        uint4 kv = *reinterpret_cast<const uint4*>(k + off);
        if (t >= L) kv = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(&Ks[t * KP + c8]) = kv;
    }
    __syncthreads();

    // K K^T (row block w, column blocks sb <= w)
    f4_t kk[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) kk[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        const int col = 32 * ks + 8 * lg;
        const bf8_t ka = lds8(&Ks[(16 * w + lr) * KP + col]);
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if (sb <= w) {
                const bf8_t kb = lds8(&Ks[(16 * sb + lr) * KP + col]);
                kk[sb] = mfma(ka, kb, kk[sb]);
            }
        }
    }
    // kk[sb][r] = (K K^T)[t = 16 w + 4 lg + r][s = 16 sb + lr]

    for (int hv = hk * ratio; hv < (hk + 1) * ratio; ++hv) {
        const size_t tileoff = ((size_t)c * HV + hv) * C * C;
        // G = in-chunk inclusive cumsum of g (wave 0), beta
        if (w == 0) {
            float gv = A.g[(size_t)(t0 + min(l, L - 1)) * HV + hv] * kLog2e;
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
        // A = strictly lower part of diag(b) (K K^T o e^{G_t - G_s})
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if (sb <= w) {
                const float Gsb = Gs[16 * sb + lr];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + 4 * lg + r, s = 16 * sb + lr;
                    Am[t * AP + s] = (s < t) ? Bs[t] * exp2f_(Gs[t] - Gsb) * kk[sb][r] : 0.f;
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
// (tokens 16 w .. 16 w + 15) in K S^T, Q S^T, P, X, U and O for both 16-column
// halves ib = 0, 1 of the state tile's 32 rows, and the state tiles
// S^T[16 jb .. +15][16 ibS .. +15] for its DK/64 column blocks jb.
// Per chunk:
//   (A) K S^T, Q S^T, P^T = K Q^T (row block tb against column blocks <= tb);
//       X = V - diag(gamma) K S^T -> LDS
//   (B) U = T' X; U and U' -> LDS
//   (C) O = gamma Q S^T + P U to memory, with P taken straight from the P^T
//       accumulators (the contraction slots are ordered so that a lane's four
//       accumulator values of two P^T tiles are its eight A-operand values,
//       and U is read in the same order); S' = gamma_n S + K^T U' -> LDS;
//       the next chunk's K rows and G go to the other half of a double buffer.
// Operand fragments from memory (K, Q rows, G, V, T') are held in one register
// set: each group is reloaded for the next chunk right after its last use, so
// every load has about a chunk to arrive.  Loads go through buffer resources
// that end at the chunk's last valid row: rows past a sequence end read as
// zero, which masks K, Q, V, X and U without selects, and output rows past
// the end are dropped by the store's resource.  No branch surrounds a memory
// operation whose count differs between paths, so the compiler waits for
// exactly the group it needs.
template <int DK, typename Tout>
__global__ __launch_bounds__(256) void scan_mfma_kernel(const PrefillArgs A) {
    constexpr int C = kChunk;
    constexpr int BV = 32;
    constexpr int KP = DK + 8;   // padded row of S and K (bf16)
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
    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][C * KP];
    __shared__ __attribute__((aligned(16))) float Gs[2][C];

    const int H = A.H, HV = A.HV, dv = A.dv, N = A.N;
    const int tid = threadIdx.x;
    const int tb = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index = row block
    __builtin_assume(tb >= 0 && tb < 4);
    const int l = tid & 63, lr = l & 15, lg = l >> 4;
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

    // state: sacc[x][ibS][r] = S[i = 16 ibS + lr][j = 16 (NJB tb + x) + 4 lg + r]
    f4_t sacc[NJB][2];
#pragma unroll
    for (int x = 0; x < NJB; ++x)
#pragma unroll
        for (int ibS = 0; ibS < 2; ++ibS) {
            const size_t off = sbase + (size_t)(16 * ibS + lr) * DK + 16 * (NJB * tb + x) + 4 * lg;
            if (A.s0) {
                const float4 v4 = *reinterpret_cast<const float4*>(A.s0 + off);
                sacc[x][ibS] = f4_t{v4.x, v4.y, v4.z, v4.w};
            } else {
                sacc[x][ibS] = f4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    auto store_state = [&](float* dst) {
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ibS = 0; ibS < 2; ++ibS) {
                const size_t off = sbase + (size_t)(16 * ibS + lr) * DK + 16 * (NJB * tb + x) + 4 * lg;
                *reinterpret_cast<float4*>(dst + off) =
                    make_float4(sacc[x][ibS][0], sacc[x][ibS][1], sacc[x][ibS][2], sacc[x][ibS][3]);
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
    const int c_first = A.chunk_off[n];
    int nch = A.chunk_off[n + 1] - c_first;
    if (c_first + nch > A.max_chunks) nch = max(0, A.max_chunks - c_first);
    if (nch <= 0) {
        if (A.s_final) store_state(A.s_final);
        return;
    }

    // byte offsets of this lane's fragments inside a chunk (the same for every chunk)
    const uint32_t qk_row = (uint32_t)H * DK * 2;  // bytes per token of q, k
    const uint32_t v_row = (uint32_t)HV * dv * 2;  // bytes per token of v
    const uint32_t kq_off = ((uint32_t)(16 * tb + lr) * H + hk) * DK * 2 + 16 * lg;
    uint32_t v_off[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        v_off[r] = ((uint32_t)(16 * tb + 4 * lg + r) * HV + h) * dv * 2 + (tile * BV + lr) * 2;
    const uint32_t t_off = ((16 * tb + lr) * C + 8 * lg) * 2;

    // ---- operand fragments (one set; groups reloaded after their last use) ----
    bf8_t kA[NKK], qA[NKK];      // K, Q row 16 tb + lr, k-step kk
    bf8_t tH[2], tL[2];          // T' row 16 tb + lr, columns 32 kk + 8 lg ..
    uint32_t vr[2][4];           // V[t = 16 tb + 4 lg + r][i = 16 ib + lr], raw bf16 bits
    float4 gR;                   // G[16 tb + 4 lg + r]  (log2 units)
    float gN;                    // G[L - 1]

    auto chunk_t0 = [&](int jc) { return sq + jc * C; };
    auto chunk_L = [&](int jc) { return min(C, eq - (sq + jc * C)); };
    auto load_kq_g = [&](int jc) {
        const int t0 = chunk_t0(jc), L = chunk_L(jc);
        const __amdgpu_buffer_rsrc_t rk = in_rsrc(kp + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
        const __amdgpu_buffer_rsrc_t rq = in_rsrc(qp + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            kA[kk] = bload8(rk, kq_off + 64 * kk);
            qA[kk] = bload8(rq, kq_off + 64 * kk);
        }
        const float* G = A.ws_G + ((size_t)(c_first + jc) * HV + h) * C;
        gR = *reinterpret_cast<const float4*>(G + 16 * tb + 4 * lg);
        gN = G[L - 1];
    };
    auto load_v = [&](int jc) {
        const int t0 = chunk_t0(jc), L = chunk_L(jc);
        const __amdgpu_buffer_rsrc_t rv = in_rsrc(vp + (size_t)t0 * HV * dv, (uint32_t)L * v_row);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vr[ib][r] = __builtin_amdgcn_raw_buffer_load_b16(rv, (int)(v_off[r] + 32 * ib), 0, 0);
    };
    auto load_t = [&](int jc) {
        const size_t tt = ((size_t)(c_first + jc) * HV + h) * C * C;
        const __amdgpu_buffer_rsrc_t rh = in_rsrc(A.ws_Th + tt, C * C * 2);
        const __amdgpu_buffer_rsrc_t rl = in_rsrc(A.ws_Tl + tt, C * C * 2);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            tH[kk] = bload8(rh, t_off + 64 * kk);
            tL[kk] = bload8(rl, t_off + 64 * kk);
        }
    };
    // K rows of row block tb and G of the chunk whose fragments are loaded -> LDS
    auto stage_k_g = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            *reinterpret_cast<bf8_t*>(&Ks[buf][(16 * tb + lr) * KP + 32 * kk + 8 * lg]) = kA[kk];
        if (lr == 0) *reinterpret_cast<float4*>(&Gs[buf][16 * tb + 4 * lg]) = gR;
    };

    load_kq_g(0);
    load_v(0);
    load_t(0);
    store_state_lds();
    stage_k_g(0);
    __syncthreads();

    for (int jc = 0; jc < nch; ++jc) {
        const int nj = min(jc + 1, nch - 1);  // the last chunk re-reads itself
        const int buf = jc & 1;
        const __bf16* Kc = Ks[buf];
        const float* Gc = Gs[buf];
        const int t0 = chunk_t0(jc);
        const int L = chunk_L(jc);
        const float gr[4] = {gR.x, gR.y, gR.z, gR.w};
        const float gNc = gN;
        float gam[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) gam[r] = exp2f_(gr[r]);

        // (A) K S^T, Q S^T (row block tb, both column halves) and P^T tiles
        f4_t ksa[2], qsa[2], pa[4];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
            ksa[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
            qsa[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) pa[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int col = 32 * kk + 8 * lg;
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const bf8_t bh = lds8(&Sh[(16 * ib + lr) * KP + col]);
                const bf8_t bl = lds8(&Sl[(16 * ib + lr) * KP + col]);
                ksa[ib] = mfma(kA[kk], bh, ksa[ib]);
                qsa[ib] = mfma(qA[kk], bh, qsa[ib]);
                ksa[ib] = mfma(kA[kk], bl, ksa[ib]);
                qsa[ib] = mfma(qA[kk], bl, qsa[ib]);
            }
            // pa[sb][r] = (Q K^T)[t = 16 tb + lr][s = 16 sb + 4 lg + r]
#pragma unroll
            for (int sb = 0; sb < 4; ++sb)
                if (sb <= tb) pa[sb] = mfma(lds8(&Kc[(16 * sb + lr) * KP + col]), qA[kk], pa[sb]);
        }
        load_kq_g(nj);
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
        // P = P^T values masked to s <= t and decayed, split into hi / lo: the
        // A operand of k-step kk holds s = 32 kk + 4 lg + (0..3) from tile 2 kk
        // and s = 32 kk + 16 + 4 lg + (0..3) from tile 2 kk + 1.  Tiles below
        // the diagonal block need no mask; tiles above it are zero.
        uint4 pHw[2], pLw[2];
        {
            const int t = 16 * tb + lr;
            const float Gt = Gc[t];
            float pv[4][4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const float4 g4 = *reinterpret_cast<const float4*>(&Gc[16 * sb + 4 * lg]);
                const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
                if (sb < tb) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) pv[sb][r] = pa[sb][r] * exp2f_(Gt - gs[r]);
                } else if (sb == tb) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pv[sb][r] = (4 * lg + r <= lr) ? pa[sb][r] * exp2f_(Gt - gs[r]) : 0.f;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) pv[sb][r] = 0.f;
                }
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                split2(pv[2 * kk][0], pv[2 * kk][1], pHw[kk].x, pLw[kk].x);
                split2(pv[2 * kk][2], pv[2 * kk][3], pHw[kk].y, pLw[kk].y);
                split2(pv[2 * kk + 1][0], pv[2 * kk + 1][1], pHw[kk].z, pLw[kk].z);
                split2(pv[2 * kk + 1][2], pv[2 * kk + 1][3], pHw[kk].w, pLw[kk].w);
            }
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
            for (int r = 0; r < 4; ++r) dec[r] = exp2f_(gNc - gr[r]);
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

        // (C1) O = scale (diag(gamma) Q S^T + P U) for row block tb; U is read in
        // the slot order of the P operand (two 8-byte pieces per k-step)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) qsa[ib][r] *= gam[r];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk <= (tb >> 1)) {
                const int col = 32 * kk + 4 * lg;
                const bf8_t ph = __builtin_bit_cast(bf8_t, pHw[kk]);
                const bf8_t pl = __builtin_bit_cast(bf8_t, pLw[kk]);
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const int row = (16 * ib + lr) * TP;
                    const uint2 h0 = *reinterpret_cast<const uint2*>(&Uh[row + col]);
                    const uint2 h1 = *reinterpret_cast<const uint2*>(&Uh[row + col + 16]);
                    const uint2 l0 = *reinterpret_cast<const uint2*>(&Ul[row + col]);
                    const uint2 l1 = *reinterpret_cast<const uint2*>(&Ul[row + col + 16]);
                    const bf8_t bh = __builtin_bit_cast(bf8_t, make_uint4(h0.x, h0.y, h1.x, h1.y));
                    const bf8_t bl = __builtin_bit_cast(bf8_t, make_uint4(l0.x, l0.y, l1.x, l1.y));
                    qsa[ib] = mfma(ph, bh, qsa[ib]);
                    qsa[ib] = mfma(ph, bl, qsa[ib]);
                    qsa[ib] = mfma(pl, bh, qsa[ib]);
                }
            }
        }
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
        // (C2) S'^T = gamma_n S^T + K^T U' for the wave's state tiles; the K^T
        // fragment (column j, tokens 32 kk + 8 lg .. +7) is gathered from the
        // row-major K tile
        const float gn = exp2f_(gNc);
#pragma unroll
        for (int x = 0; x < NJB; ++x) {
            const int j = 16 * (NJB * tb + x) + lr;
            bf8_t ka[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int y = 0; y < 8; ++y) ka[kk][y] = Kc[(32 * kk + 8 * lg + y) * KP + j];
#pragma unroll
            for (int ibS = 0; ibS < 2; ++ibS) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[x][ibS][r] *= gn;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int col = 32 * kk + 8 * lg;
                    const bf8_t bh = lds8(&Wh[(16 * ibS + lr) * TP + col]);
                    const bf8_t bl = lds8(&Wl[(16 * ibS + lr) * TP + col]);
                    sacc[x][ibS] = mfma(ka[kk], bh, sacc[x][ibS]);
                    sacc[x][ibS] = mfma(ka[kk], bl, sacc[x][ibS]);
                }
            }
        }
        // Sh / Sl are read only in (A), and the other K / G buffer was last
        // read in the previous chunk: both can be written before the barrier
        store_state_lds();
        stage_k_g(buf ^ 1);
        __syncthreads();
    }

    if (A.s_final) store_state(A.s_final);
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

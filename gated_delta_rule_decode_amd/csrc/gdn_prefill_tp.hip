// gdn_prefill_tp.hip -- chunked prefill with a state-free pass that keeps only
// the triangular factor T' and a scan that forms every other chunk product
// itself (gfx950, bf16 inputs, d_k = 128).
//
// Per chunk of C = 64 tokens with in-chunk cumulative log-decays G
// (gamma_t = e^{G_t}), the chunkwise form of the gated delta rule (Yang,
// Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025):
//
//     A_ts = b_t e^{G_t - G_s} k_t.k_s  (s < t)      T' = (I + A)^-1 diag(b)
//     X    = V - diag(gamma) K S^T                   U  = T' X
//     O    = scale (diag(gamma) Q S^T + P U)         P_ts = e^{G_t - G_s} q_t.k_s (s <= t)
//     S'   = gamma_n S + U'^T K                      U' = diag(e^{G_n - G}) U
//
// prep_tp_kernel (chunk-parallel, one workgroup per (chunk, key head), its
// value heads in turn) writes G and T' -- 10 KiB per (chunk, value head), the
// ten 16 x 16 blocks of T' on or below the diagonal, split into hi and lo
// bf16 in the order the scan's MFMA operands read them -- and nothing else.
// scan_tp_kernel (sequential over chunks) forms P, K^T, Q S^T and the rest
// on the chip from K, Q and V, so no product of the chunk makes a round trip
// through memory.
//
// The scan splits a workgroup's eight wavefronts into two roles.  The four
// chain wavefronts carry only the state's dependency chain,
//     S -> K S^T -> X -> U = T' X -> S' = gamma_n S + U'^T K,
// with the state in MFMA accumulators; the K^T operand of the last product is
// read from the row-major K tile with the LDS transpose read
// (ds_read_b64_tr_b16).  The four helper wavefronts do what the chain does not
// wait for: they stage the next chunk's K, Q, V, G and T' into LDS (loads
// issued a chunk ahead), form P of the next chunk and Q S^T, and finish and
// store the outputs.  A chain and a helper wavefront share each SIMD, so the
// helpers' products, loads and stores fill the issue slots the chain leaves
// while it waits on its own dependences.  Three barriers per chunk separate
// the phases A (K S^T, X; Q S^T), U (U = T' X; staging of the next chunk) and
// S (S'; O = scale (gamma Q S^T + P U), stores, P of the next chunk).
//
// Precision as in the other MFMA kernels: q, k, v enter the products
// exactly; every fp32 operand (S, X, U, U', P, T') is split into hi + lo
// bf16; accumulation is fp32 and the state between chunks stays fp32.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_prefill_common.h"

namespace gdn {

// T' of one (chunk, value head): block (tb, sb), sb <= tb, at index
// tb (tb + 1) / 2 + sb; a block is 1 KiB, 512 bytes of hi then 512 of lo.
// Inside a block, the 16 bytes at lane-in-block lb = row + 16 half hold
// columns 8 half .. 8 half + 7 of that row: an MFMA A operand for rows
// 16 tb .. + 15 and contraction slots 32 kk .. + 31 reads, in lane
// l = lr + 16 lg, block (tb, 2 kk + lg / 2) at lb = lr + 16 (lg % 2).
constexpr int kTpBlocks = 10;
constexpr int kTpBlockElems = 512;                          // uint16 per block (hi + lo)
constexpr int kTpElems = kTpBlocks * kTpBlockElems;         // per (chunk, value head)
__host__ __device__ constexpr int tp_block(int tb, int sb) { return tb * (tb + 1) / 2 + sb; }

template <int V>
struct TokenBlock {
    static constexpr int value = V;
};
// Runs f(TokenBlock<tb>{}) for a wavefront-uniform tb in 0..3, so that the
// triangular loops of a token block unroll with compile-time bounds: no
// branch splits their LDS reads from one another.
template <typename F>
__device__ __forceinline__ void with_token_block(int tb, F&& f) {
    switch (tb) {
    case 0: f(TokenBlock<0>{}); break;
    case 1: f(TokenBlock<1>{}); break;
    case 2: f(TokenBlock<2>{}); break;
    default: f(TokenBlock<3>{}); break;
    }
}

// ---------------------------------------------------------------------------
// prep: G and T' per (chunk, value head)
// ---------------------------------------------------------------------------
// One workgroup (4 wavefronts) per (chunk, key head): the chunk's K rows are
// read once and serve every value head of the key head in turn.  Per value
// head: G (a wave prefix sum, log2 units), A = strictly lower
// diag(b) (K K^T o e^{G_t - G_s}) from K K^T on MFMA (row block w per
// wavefront), T = (I + A)^-1 by forward substitution on the 16 x 16 diagonal
// blocks and block merges on split-bf16 MFMA, then T' = T diag(b) written out
// as hi / lo blocks.  Rows past a sequence end read K, g and b as zero, so
// T' has zero rows there and its valid block is the inverse of the valid
// part alone.
template <int DK>
__global__ __launch_bounds__(256) void prep_tp_kernel(const PrefillArgs A) {
    constexpr int C = kChunk;
    constexpr int KP = DK + 8;   // padded bf16 row of the K tile
    constexpr int AP = C + 4;    // padded fp32 row (16-byte aligned rows)
    constexpr int NKK = DK / 32;
    constexpr int PPR = DK / 8;  // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;
    constexpr int NLD = 16 / RPI;
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * KP];
    __shared__ __attribute__((aligned(16))) float Tm[C * AP];  // A, then T written over it
    __shared__ __attribute__((aligned(16))) float Gs[C];
    __shared__ __attribute__((aligned(16))) float Bs[C];
    float* const Am = Tm;
    float* const Xm = Tm + 32;  // 32-block merge: X [32 x 32] in the upper-right block

    const int H = A.H, HV = A.HV, R = HV / H;
    const int c = blockIdx.x, hk = blockIdx.y, tid = threadIdx.x;
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

    // K rows of the key head (coalesced 16-byte pieces), g and b of the first
    // value head for token l (wave 0; zero past the end)
    const uint32_t qk_row = (uint32_t)H * DK * 2;
    const __amdgpu_buffer_rsrc_t rk =
        in_rsrc(static_cast<const bf16_t*>(A.k) + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
    bf8_t kst[NLD];
#pragma unroll
    for (int p = 0; p < NLD; ++p) {
        const int row = 16 * w + RPI * p + l / PPR;
        kst[p] = bload8(rk, ((uint32_t)row * H + hk) * DK * 2 + 16 * (l % PPR));
    }
    const __amdgpu_buffer_rsrc_t rg = in_rsrc(A.g + (size_t)t0 * HV, (uint32_t)L * HV * 4);
    const __amdgpu_buffer_rsrc_t rb = in_rsrc(A.beta + (size_t)t0 * HV, (uint32_t)L * HV * 4);
    auto load_gb = [&](int hv, float& gv, float& bv) {
        gv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, (int)((l * HV + hv) * 4), 0, 0));
        bv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (int)((l * HV + hv) * 4), 0, 0));
    };
    float gnext = 0.f, bnext = 0.f;
    if (w == 0) load_gb(hk * R, gnext, bnext);
#pragma unroll
    for (int p = 0; p < NLD; ++p)
        *reinterpret_cast<bf8_t*>(&Ks[(16 * w + RPI * p + l / PPR) * KP + 8 * (l % PPR)]) = kst[p];

    for (int v = 0; v < R; ++v) {
        const int hv = hk * R + v;
        if (w == 0) {
            // G (log2 units, inclusive in-chunk prefix sum) and b of this value head
            float gs = gnext * kLog2e;
            const float bv = bnext;
            if (v + 1 < R) load_gb(hv + 1, gnext, bnext);  // the next value head's, in flight
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float up = __shfl_up(gs, off, 64);
                if (l >= off) gs += up;
            }
            Gs[l] = gs;
            Bs[l] = bv;
            A.ws_G[((size_t)c * HV + hv) * C + l] = gs;
        }
        __syncthreads();  // K (first value head), G and b are in LDS

        // A = strictly lower part of diag(b) (K K^T o e^{G_t - G_s}), row block w
        {
            f4_t kk[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) kk[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKK; ++ks) {
                const int col = 32 * ks + 8 * lg;
                const bf8_t ka = lds8(&Ks[(16 * w + lr) * KP + col]);
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
                    if (sb <= w) kk[sb] = mfma(ka, lds8(&Ks[(16 * sb + lr) * KP + col]), kk[sb]);
            }
            // kk[sb][r] = (K K^T)[t = 16 w + 4 lg + r][s = 16 sb + lr]
            const float4 g4 = *reinterpret_cast<const float4*>(&Gs[16 * w + 4 * lg]);
            const float4 b4 = *reinterpret_cast<const float4*>(&Bs[16 * w + 4 * lg]);
            const float gt[4] = {g4.x, g4.y, g4.z, g4.w};
            const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (sb <= w) {
                    const float Gsb = Gs[16 * sb + lr];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * w + 4 * lg + r, s = 16 * sb + lr;
                        // only s < t is kept, where the exponent is <= 0 anyway
                        const float keep = (s < t) ? 1.f : 0.f;
                        Am[t * AP + s] = keep * bt[r] * exp2f_(fminf(gt[r] - Gsb, 0.f)) * kk[sb][r];
                    }
                }
            }
        }
        __syncthreads();
        // diagonal blocks T_bb = (I + A_bb)^-1 by forward substitution: wave b,
        // lane j < 16 owns column j
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
                float v_ = (t == l) ? 1.f : 0.f;
#pragma unroll
                for (int x = 0; x < t; ++x) v_ -= arow[x] * col[x];
                col[t] = v_;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) Tm[(o + t) * AP + o + l] = col[t];
        }
        __syncthreads();
        // 16-block merges, one per wavefront 0 and 1:
        //   T_{ii,j} = -T_{ii,ii} (A_{ii,j} T_{jj}),  (ii, j) = (1, 0), (3, 2)
        // (the 16-long contraction fills slots 0..3 of each lane group, slots
        // 4..7 are zero, so the first product's accumulators are the second
        // product's B operand)
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
            f4_t xa = f4_t{0.f, 0.f, 0.f, 0.f};
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
        // 32-block merge: X = A[32:64, 0:32] T[0:32, 0:32]; T[32:64, 0:32] = -T_B X
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
        // T' = T diag(b), the ten blocks on or below the diagonal, hi / lo in
        // operand order: unit u = (block, lane-in-block), 8 columns each.  A
        // select, not a 0/1 factor, keeps the zero upper half of a diagonal
        // block (T's other upper blocks hold scratch data and are not read).
        uint16_t* const tp = A.ws_Tp + ((size_t)c * HV + hv) * kTpElems;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int u = tid + 256 * q;
            if (u < kTpBlocks * 32) {
                const int blk = u >> 5, lb = u & 31;
                const int tb = blk >= 6 ? 3 : (blk >= 3 ? 2 : (blk >= 1 ? 1 : 0));
                const int sb = blk - tp_block(tb, 0);
                const int t = 16 * tb + (lb & 15), s = 16 * sb + 8 * (lb >> 4);
                const float4 x0 = *reinterpret_cast<const float4*>(&Tm[t * AP + s]);
                const float4 x1 = *reinterpret_cast<const float4*>(&Tm[t * AP + s + 4]);
                const float4 b0 = *reinterpret_cast<const float4*>(&Bs[s]);
                const float4 b1 = *reinterpret_cast<const float4*>(&Bs[s + 4]);
                const float tv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = (s + e <= t) ? tv[e] * bb[e] : 0.f;
                bf8_t hi, lo;
                split8(pv, hi, lo);
                *reinterpret_cast<bf8_t*>(tp + blk * kTpBlockElems + lb * 8) = hi;
                *reinterpret_cast<bf8_t*>(tp + blk * kTpBlockElems + 256 + lb * 8) = lo;
            }
        }
        __syncthreads();  // Tm, Gs and Bs are rewritten for the next value head
    }
}

// ---------------------------------------------------------------------------
// scan: sequential over chunks, chain and helper wavefronts
// ---------------------------------------------------------------------------
// Work items as in the per-tile scan: (segment, value head, 32-row tile of
// S) value items first, then the transition items of later segments (the same
// scan from the identity with V read as zero: d_k rows, writing
// w = scale Phi_t q_t instead of o and Phi^T instead of the state).  All tiles
// of a chain get the same b % 8 and neighbouring dispatch slots (workgroup b
// runs on XCD b % 8), so their shared K, Q reads meet in one L2.
//
// Chain wavefront c (0..3): token block tb = c in phases A and U (K S^T,
// Q S^T, X; U = T' X), state columns j in 32 c .. 32 c + 31 in phase S; its
// accumulators hold
//   sacc[x][ib][r] = S'^T[j = 16 (2 c + x) + 4 lg + r][i = 16 ib + lr].
// Helper wavefront 4 + c: token block tb = 3 - c of P and O (so that the
// triangular work of a chain and a helper on one SIMD adds up to about the
// same on every SIMD), and a quarter of every staging copy.
// Chunk c's K, Q, G, V and T' sit in the buffers of parity c % 2 from
// phase A of step c - 1 (staged) to phase S of step c (last read).
template <int DK, typename Tout>
__device__ __forceinline__ void scan_tp_item(const PrefillArgs& A, const int b) {
    static_assert(DK == 128, "the chain / helper scan is written for d_k = 128");
    constexpr int C = kChunk;
    constexpr int BV = 32;       // state rows per workgroup
    constexpr int KP = DK + 8;   // padded bf16 row: state, K and Q tiles
    constexpr int TP = C + 8;    // padded bf16 row of the transposed tiles (X^T, U^T, U'^T)
    constexpr int VP = BV + 16;  // padded bf16 row of V: the four rows of a transpose read fall in disjoint banks
    constexpr int NKK = DK / 32;
    constexpr int NJB = DK / 64;  // state column blocks per chain wavefront
    __shared__ __attribute__((aligned(16))) __bf16 Sh[BV * KP];   // S, hi / lo
    __shared__ __attribute__((aligned(16))) __bf16 Sl[BV * KP];
    __shared__ __attribute__((aligned(16))) __bf16 Xh[BV * TP];   // X^T [i][t]
    __shared__ __attribute__((aligned(16))) __bf16 Xl[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Uh[BV * TP];   // U^T [i][t]
    __shared__ __attribute__((aligned(16))) __bf16 Ul[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Wh[BV * TP];   // U'^T [i][t]
    __shared__ __attribute__((aligned(16))) __bf16 Wl[BV * TP];
    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][C * KP]; // K [t][j], by chunk parity
    __shared__ __attribute__((aligned(16))) __bf16 Qs[2][C * KP]; // Q [t][j]
    __shared__ __attribute__((aligned(16))) __bf16 Vs[2][C * VP];   // V [t][i] of the tile
    __shared__ __attribute__((aligned(16))) uint16_t Tp[2][kTpElems];
    __shared__ __attribute__((aligned(16))) float Gs[2][C];
    __shared__ __attribute__((aligned(16))) f4_t QSs[4][2][64];   // gamma (S Q^T) per token block, O^T lane order
    typedef short v4s_t __attribute__((ext_vector_type(4)));

    const int H = A.H, HV = A.HV, dv = A.dv;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(w >= 0 && w < 8);
    const bool is_chain = w < 4;
    const int tb = is_chain ? w : 7 - w;  // token block of the wavefront
    const int l = tid & 63, lr = l & 15, lg = l >> 4;
    const int hp = tid & 255;  // a helper's lane among the 256 helper lanes

    const int TV = dv / BV;
    const int nb1 = ((A.seg_bound * HV + 7) / 8) * 8 * TV;
    const bool trans = b >= nb1;
    const int bb = trans ? b - nb1 : b;
    const int TT = trans ? DK / BV : TV;
    const int slot = bb >> 3;
    const int tile = slot % TT;
    const int chn = (slot / TT) * 8 + (bb & 7);
    const int nseg = __builtin_amdgcn_readfirstlane(A.plan[0]);
    if (chn >= nseg * HV) return;
    const int sg = chn / HV, h = chn - sg * HV;
    const int n = __builtin_amdgcn_readfirstlane(A.seg_seq[sg]);
    const int sidx = __builtin_amdgcn_readfirstlane(A.seg_idx[sg]);
    if (trans && sidx == 0) return;
    const int hk = h / (HV / H);
    Tout* op = static_cast<Tout*>(A.o);
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

    // chain: the state of its column blocks
    f4_t sacc[NJB][2];
    if (is_chain) {
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int i = 16 * ib + lr, j = 16 * (NJB * tb + x) + 4 * lg;
                if (init) {
                    const float4 v4 = *reinterpret_cast<const float4*>(init + ibase + (size_t)i * DK + j);
                    sacc[x][ib] = f4_t{v4.x, v4.y, v4.z, v4.w};
                } else if (trans) {
                    const int d = tile * BV + i - j;  // identity: 1 where row == column
                    sacc[x][ib] = f4_t{d == 0 ? 1.f : 0.f, d == 1 ? 1.f : 0.f, d == 2 ? 1.f : 0.f,
                                       d == 3 ? 1.f : 0.f};
                } else {
                    sacc[x][ib] = f4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
    }
    auto store_state = [&]() {
        if (!fin) return;
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int i = 16 * ib + lr, j = 16 * (NJB * tb + x) + 4 * lg;
                if (trans) {
                    // Phi is stored transposed (Phi^T[j][i]): the combine pass
                    // reads it as an MFMA B operand, 8 consecutive i per lane
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        fin[(size_t)(sg * HV + h) * DK * DK + (size_t)(j + r) * DK + tile * BV + i] =
                            sacc[x][ib][r];
                } else {
                    *reinterpret_cast<float4*>(fin + fbase + (size_t)i * DK + j) =
                        make_float4(sacc[x][ib][0], sacc[x][ib][1], sacc[x][ib][2], sacc[x][ib][3]);
                }
            }
    };
    auto state_to_lds = [&]() {
#pragma unroll
        for (int x = 0; x < NJB; ++x)
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int off = (16 * ib + lr) * KP + 16 * (NJB * tb + x) + 4 * lg;
                float sv[4] = {sacc[x][ib][0], sacc[x][ib][1], sacc[x][ib][2], sacc[x][ib][3]};
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
        if (is_chain) store_state();
        return;
    }

    // ---- helpers: loads of a chunk (into registers) and their staging ----
    const uint32_t qk_row = (uint32_t)H * DK * 2;  // bytes per token of q, k
    const uint32_t v_row = (uint32_t)HV * dv * 2;  // bytes per token of v
    const uint32_t v_on = trans ? 0u : 1u;         // a transition item reads V as zero
    // K and Q: piece pi = hp + 256 q of the 64 x 256-byte tile (row pi / 16)
    uint32_t kq_off[4];
    int kq_st[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int pi = hp + 256 * q, row = pi >> 4, c16 = pi & 15;
        kq_off[q] = ((uint32_t)row * H + hk) * DK * 2 + 16 * c16;
        kq_st[q] = row * KP + 8 * c16;
    }
    // V: token hp / 4, rows 8 (hp % 4) .. + 7 of the tile
    const int v_tok = hp >> 2, v_row0 = 8 * (hp & 3);
    const uint32_t v_off = ((uint32_t)v_tok * HV + h) * (uint32_t)dv * 2 + (uint32_t)(tile * BV + v_row0) * 2;
    bf8_t kst[4], qst[4], vst, tst[3];
    float gst = 0.f;
    auto chunk_t0 = [&](int jc) { return sq + jc * C; };
    auto chunk_L = [&](int jc) { return min(C, eq - (sq + jc * C)); };
    auto load_chunk = [&](int jc) {
        const int t0 = chunk_t0(jc), L = chunk_L(jc);
        const __amdgpu_buffer_rsrc_t rk =
            in_rsrc(static_cast<const bf16_t*>(A.k) + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
        const __amdgpu_buffer_rsrc_t rq =
            in_rsrc(static_cast<const bf16_t*>(A.q) + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
        const __amdgpu_buffer_rsrc_t rv =
            in_rsrc(static_cast<const bf16_t*>(A.v) + (size_t)t0 * HV * dv, v_on * L * v_row);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            kst[q] = bload8(rk, kq_off[q]);
            qst[q] = bload8(rq, kq_off[q]);
        }
        vst = bload8(rv, v_off);
        const uint16_t* tp = A.ws_Tp + ((size_t)(c_first + jc) * HV + h) * kTpElems;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const int pi = hp + 256 * q;
            if (pi < kTpElems / 8) tst[q] = gld8(tp + 8 * pi);
        }
        if (hp < C) gst = A.ws_G[((size_t)(c_first + jc) * HV + h) * C + hp];
    };
    auto stage_chunk = [&](int jc) {
        const int pb = jc & 1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            *reinterpret_cast<bf8_t*>(&Ks[pb][kq_st[q]]) = kst[q];
            *reinterpret_cast<bf8_t*>(&Qs[pb][kq_st[q]]) = qst[q];
        }
        *reinterpret_cast<bf8_t*>(&Vs[pb][v_tok * VP + v_row0]) = vst;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const int pi = hp + 256 * q;
            if (pi < kTpElems / 8) *reinterpret_cast<bf8_t*>(&Tp[pb][8 * pi]) = tst[q];
        }
        if (hp < C) Gs[pb][hp] = gst;
    };

    // The chain and the helpers run separate loops with the same three
    // barriers per chunk, so that neither role's registers are held live
    // across the other's code.
    if (is_chain) {
        state_to_lds();
        __syncthreads();  // B0: the state and chunk 0 in LDS
        for (int jc = 0; jc < nch; ++jc) {
            const int L = chunk_L(jc);
            const int pb = jc & 1;
            const float* Gc = Gs[pb];
            // ===== phase A =====
            // K S^T (tokens of block tb, both 16-row halves) and S Q^T (its
            // transposed O^T layout), sharing the state fragments; the hi and
            // lo parts accumulate separately (four independent chains each)
            f4_t kh[2], kl[2], qh[2], ql[2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                kh[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
                kl[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
                qh[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
                ql[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
            }
            // every fragment is read before the first product
            bf8_t ka[NKK], qa[NKK], sh[NKK][2], sl[NKK][2];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int col = 32 * kk + 8 * lg;
                ka[kk] = lds8(&Ks[pb][(16 * tb + lr) * KP + col]);
                qa[kk] = lds8(&Qs[pb][(16 * tb + lr) * KP + col]);
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    sh[kk][ib] = lds8(&Sh[(16 * ib + lr) * KP + col]);
                    sl[kk][ib] = lds8(&Sl[(16 * ib + lr) * KP + col]);
                }
            }
            // V[t = 16 tb + 4 lg + r][i = 16 ib + lr], r = 0..3, by transpose
            // reads: lane m of each 16-lane group points at row 16 tb + 4 lg + m / 4,
            // columns 16 ib + 4 (m % 4) ..
            v4s_t vr[2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
                vr[ib] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(
                    &Vs[pb][(16 * tb + 4 * lg + (lr >> 2)) * VP + 16 * ib + 4 * (lr & 3)]));
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    kh[ib] = mfma(ka[kk], sh[kk][ib], kh[ib]);
                    kl[ib] = mfma(ka[kk], sl[kk][ib], kl[ib]);
                    qh[ib] = mfma(sh[kk][ib], qa[kk], qh[ib]);
                    ql[ib] = mfma(sl[kk][ib], qa[kk], ql[ib]);
                }
            const float4 g4 = *reinterpret_cast<const float4*>(&Gc[16 * tb + 4 * lg]);
            const float gam[4] = {exp2f_(g4.x), exp2f_(g4.y), exp2f_(g4.z), exp2f_(g4.w)};
            // X = V - diag(gamma) K S^T, rows [i][t] hi / lo
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int off = (16 * ib + lr) * TP + 16 * tb + 4 * lg;
                float vf[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) vf[r] = __uint_as_float((uint32_t)(uint16_t)vr[ib][r] << 16);
                float xv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) xv[r] = vf[r] - gam[r] * (kh[ib][r] + kl[ib][r]);
                uint2 hi, lo;
                split4(xv, hi, lo);
                *reinterpret_cast<uint2*>(&Xh[off]) = hi;
                *reinterpret_cast<uint2*>(&Xl[off]) = lo;
            }
            // gamma_t (S Q^T)[i][t], t = 16 tb + lr: the O^T tiles' first part
            const float gt = exp2f_(Gc[16 * tb + lr]);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                f4_t v_;
#pragma unroll
                for (int r = 0; r < 4; ++r) v_[r] = gt * (qh[ib][r] + ql[ib][r]);
                QSs[tb][ib][l] = v_;
            }
            __syncthreads();  // B1: X, gamma S Q^T of the chunk in LDS; the next chunk staged
            // ===== phase U =====
            // U = T' X for token block tb (T' lower: k-steps kk <= tb / 2)
            f4_t ua[2];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) ua[ib] = f4_t{0.f, 0.f, 0.f, 0.f};
            with_token_block(tb, [&](auto TB) {
                constexpr int tbc = decltype(TB)::value;
                bf8_t th[2], tl[2], xh[2][2], xl[2][2];
#pragma unroll
                for (int kk = 0; kk <= (tbc >> 1); ++kk) {
                    // lanes of the upper half-step (sb = tb + 1) read block 0
                    // and are zeroed below
                    const int sb = 2 * kk + (lg >> 1);
                    const int bi = (sb <= tbc) ? tp_block(tbc, sb) : 0;
                    const int at = bi * kTpBlockElems + (lr + 16 * (lg & 1)) * 8;
                    th[kk] = *reinterpret_cast<const bf8_t*>(&Tp[pb][at]);
                    tl[kk] = *reinterpret_cast<const bf8_t*>(&Tp[pb][at + 256]);
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        xh[kk][ib] = lds8(&Xh[(16 * ib + lr) * TP + 32 * kk + 8 * lg]);
                        xl[kk][ib] = lds8(&Xl[(16 * ib + lr) * TP + 32 * kk + 8 * lg]);
                    }
                }
#pragma unroll
                for (int kk = 0; kk <= (tbc >> 1); ++kk) {
                    if ((tbc & 1) == 0 && kk == (tbc >> 1) && (lg >> 1)) {  // an upper block: zero
                        th[kk] = zero8();
                        tl[kk] = zero8();
                    }
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        ua[ib] = mfma(th[kk], xh[kk][ib], ua[ib]);
                        ua[ib] = mfma(th[kk], xl[kk][ib], ua[ib]);
                        ua[ib] = mfma(tl[kk], xh[kk][ib], ua[ib]);
                    }
                }
            });
            // ua[ib][r] = U[t = 16 tb + 4 lg + r][i = 16 ib + lr]; U' = diag(e^{G_n - G}) U
            const float Gn = Gc[L - 1];  // g4: G of the wavefront's tokens, read in phase A
            const float dd[4] = {exp2f_(Gn - g4.x), exp2f_(Gn - g4.y), exp2f_(Gn - g4.z),
                                 exp2f_(Gn - g4.w)};
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                const int off = (16 * ib + lr) * TP + 16 * tb + 4 * lg;
                float uv[4] = {ua[ib][0], ua[ib][1], ua[ib][2], ua[ib][3]};
                uint2 hi, lo;
                split4(uv, hi, lo);
                *reinterpret_cast<uint2*>(&Uh[off]) = hi;
                *reinterpret_cast<uint2*>(&Ul[off]) = lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) uv[r] *= dd[r];
                split4(uv, hi, lo);
                *reinterpret_cast<uint2*>(&Wh[off]) = hi;
                *reinterpret_cast<uint2*>(&Wl[off]) = lo;
            }
            __syncthreads();  // B2: U, U' of the chunk in LDS
            // ===== phase S =====
            // S'^T = gamma_n S^T + K^T U' for the wavefront's column blocks
            const float gn = exp2f_(Gc[L - 1]);
#pragma unroll
            for (int x = 0; x < NJB; ++x)
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sacc[x][ib][r] *= gn;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf8_t wh[2], wl[2];
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    wh[ib] = lds8(&Wh[(16 * ib + lr) * TP + 32 * kk + 8 * lg]);
                    wl[ib] = lds8(&Wl[(16 * ib + lr) * TP + 32 * kk + 8 * lg]);
                }
#pragma unroll
                for (int x = 0; x < NJB; ++x) {
                    const int jb = NJB * tb + x;
                    // K^T rows j = 16 jb + lr, tokens 32 kk + 8 lg .. + 7: two
                    // transpose reads; lane m of each 16-lane group points at
                    // row 32 kk + 8 lg + m / 4 (+ 4), columns 16 jb + 4 (m % 4) ..
                    const __bf16* kp_ = &Ks[pb][(32 * kk + 8 * lg + (lr >> 2)) * KP + 16 * jb + 4 * (lr & 3)];
                    const v4s_t k0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s_t*)(kp_));
                    const v4s_t k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s_t*)(kp_ + 4 * KP));
                    const bf8_t kt = __builtin_bit_cast(bf8_t, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        sacc[x][ib] = mfma(kt, wh[ib], sacc[x][ib]);
                        sacc[x][ib] = mfma(kt, wl[ib], sacc[x][ib]);
                    }
                }
            }
            // the next chunk's state (S of this chunk was last read in phase A)
            state_to_lds();
            __syncthreads();  // B3: the next chunk's state in LDS; U, gamma S Q^T read
        }
        store_state();
    } else {
        load_chunk(0);
        stage_chunk(0);
        if (nch > 1) load_chunk(1);
        __syncthreads();  // B0
        bf8_t ph[2], pl[2];  // P fragments of the chunk (B operand, slot order)
        for (int jc = 0; jc < nch; ++jc) {
            const int t0 = chunk_t0(jc), L = chunk_L(jc);
            const int pb = jc & 1;
            const float* Gc = Gs[pb];
            // ===== phase A =====
            // the next chunk into the other buffers; the one after it in flight
            if (jc + 1 < nch) stage_chunk(jc + 1);
            if (jc + 2 < nch) load_chunk(jc + 2);
            __syncthreads();  // B1
            // ===== phase U =====
            // P of this chunk for token block tb, decayed and masked, as B
            // operands in the slot order s = 32 k2 + 16 half + 4 lg + r (slot
            // 4 half + r): pq[sb][r] = (K Q^T)[s = 16 sb + 4 lg + r][t = 16 tb + lr]
            // (blocks sb > tb are zero: their fragments stay unset and unread)
            with_token_block(tb, [&](auto TB) {
                constexpr int tbc = decltype(TB)::value;
                f4_t pq[tbc + 1];
#pragma unroll
                for (int sb = 0; sb <= tbc; ++sb) pq[sb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const bf8_t qb = lds8(&Qs[pb][(16 * tbc + lr) * KP + 32 * kk + 8 * lg]);
                    bf8_t kb[tbc + 1];
#pragma unroll
                    for (int sb = 0; sb <= tbc; ++sb) kb[sb] = lds8(&Ks[pb][(16 * sb + lr) * KP + 32 * kk + 8 * lg]);
#pragma unroll
                    for (int sb = 0; sb <= tbc; ++sb) pq[sb] = mfma(kb[sb], qb, pq[sb]);
                }
                const int t = 16 * tbc + lr;
                const float Gt = Gc[t];
#pragma unroll
                for (int k2 = 0; k2 <= (tbc >> 1); ++k2) {
                    float pv[8];
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int sb = 2 * k2 + half;
                        if (sb > tbc) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) pv[4 * half + r] = 0.f;
                            continue;
                        }
                        const float4 g4 = *reinterpret_cast<const float4*>(&Gc[16 * sb + 4 * lg]);
                        const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            // Gt - gs <= 0 for s <= t, so the factor is at most 1; the
                            // diagonal block masks s > t by a 0 / 1 factor
                            float f = exp2f_(fminf(Gt - gs[r], 0.f));
                            if (sb == tbc) f *= (4 * lg + r <= lr) ? 1.f : 0.f;
                            pv[4 * half + r] = pq[sb][r] * f;
                        }
                    }
                    split8(pv, ph[k2], pl[k2]);
                }
            });
            __syncthreads();  // B2
            // ===== phase S =====
            // O^T = gamma S Q^T + U^T P^T (P lower: k-steps kk <= tb / 2); U^T
            // read in the slot order of the P fragments
            f4_t oacc[2] = {QSs[tb][0][l], QSs[tb][1][l]};
            with_token_block(tb, [&](auto TB) {
                constexpr int tbc = decltype(TB)::value;
                bf8_t uh[2][2], ul[2][2];
#pragma unroll
                for (int kk = 0; kk <= (tbc >> 1); ++kk)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        const int off = (16 * ib + lr) * TP + 32 * kk + 4 * lg;
                        const uint2 h0 = *reinterpret_cast<const uint2*>(&Uh[off]);
                        const uint2 h1 = *reinterpret_cast<const uint2*>(&Uh[off + 16]);
                        const uint2 l0 = *reinterpret_cast<const uint2*>(&Ul[off]);
                        const uint2 l1 = *reinterpret_cast<const uint2*>(&Ul[off + 16]);
                        uh[kk][ib] = __builtin_bit_cast(bf8_t, make_uint4(h0.x, h0.y, h1.x, h1.y));
                        ul[kk][ib] = __builtin_bit_cast(bf8_t, make_uint4(l0.x, l0.y, l1.x, l1.y));
                    }
#pragma unroll
                for (int kk = 0; kk <= (tbc >> 1); ++kk)
#pragma unroll
                    for (int ib = 0; ib < 2; ++ib) {
                        oacc[ib] = mfma(uh[kk][ib], ph[kk], oacc[ib]);
                        oacc[ib] = mfma(ul[kk][ib], ph[kk], oacc[ib]);
                        oacc[ib] = mfma(uh[kk][ib], pl[kk], oacc[ib]);
                    }
            });
            // oacc[ib][r] = O[t = 16 tb + lr][i = 16 ib + 4 lg + r]; rows t >= L land
            // at or past the resource end and are dropped.  A transition item
            // writes w (fp32, d_k per token and head) instead of o.
            const int t = 16 * tb + lr;
            if (trans) {
                float* wp = A.ws_W + (size_t)t0 * HV * DK;
                const __amdgpu_buffer_rsrc_t wr = out_rsrc(wp, (uint32_t)(L * HV * DK * 4));
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const float ov[4] = {A.scale * oacc[ib][0], A.scale * oacc[ib][1],
                                         A.scale * oacc[ib][2], A.scale * oacc[ib][3]};
                    out_store4(wr, (uint32_t)((t * HV + h) * DK + tile * BV + 16 * ib + 4 * lg), ov, wp);
                }
            } else {
                const __amdgpu_buffer_rsrc_t orsrc =
                    out_rsrc(op + (size_t)t0 * HV * dv, (uint32_t)(L * HV * dv * sizeof(Tout)));
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    const float ov[4] = {A.scale * oacc[ib][0], A.scale * oacc[ib][1],
                                         A.scale * oacc[ib][2], A.scale * oacc[ib][3]};
                    out_store4(orsrc, (uint32_t)((t * HV + h) * dv + tile * BV + 16 * ib + 4 * lg), ov, op);
                }
            }
            __syncthreads();  // B3
        }
    }
}

// Persistent over work items, as the per-tile scan: workgroup blockIdx.x takes
// items blockIdx.x, blockIdx.x + gridDim.x, ... (the grid is a multiple of 8,
// so an item keeps its XCD).
template <int DK, typename Tout>
__global__ __launch_bounds__(512) void scan_tp_kernel(const PrefillArgs A, int items) {
    for (int b = blockIdx.x; b < items; b += gridDim.x) {
        __syncthreads();  // the previous item has finished with the LDS
        scan_tp_item<DK, Tout>(A, b);
    }
}

hipError_t launch_prep_tp(const PrefillArgs& A) {
    hipLaunchKernelGGL((prep_tp_kernel<128>), dim3(A.max_chunks, A.H), dim3(256), 0, A.stream, A);
    return hipGetLastError();
}

hipError_t launch_scan_tp(const PrefillArgs& A, size_t grid, int items) {
    if (A.o_bf16)
        hipLaunchKernelGGL((scan_tp_kernel<128, bf16_t>), dim3((unsigned)grid), dim3(512), 0,
                           A.stream, A, items);
    else
        hipLaunchKernelGGL((scan_tp_kernel<128, float>), dim3((unsigned)grid), dim3(512), 0,
                           A.stream, A, items);
    return hipGetLastError();
}

}  // namespace gdn

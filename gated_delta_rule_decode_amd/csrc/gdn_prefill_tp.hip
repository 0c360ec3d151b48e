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
// value heads in turn) writes G and T' -- 12 KiB per (chunk, value head): the
// lower part of T' as six 16 x 32 tiles, split into hi and lo bf16 in the
// order the scan's MFMA operands read them -- and nothing else.
// scan_tp_kernel (sequential over chunks) forms P, Q S^T and every other
// product on the chip from K, Q and V, so no product of the chunk makes a
// round trip through memory.
//
// The scan gives a workgroup's six wavefronts three roles.  Two chain
// wavefronts carry only the state's dependency chain,
//     S -> K S^T -> X -> U = T' X -> S' = gamma_n S + U'^T K,
// for 16 state rows each, with the state in MFMA accumulators; the K^T
// operand of the last product is read from the row-major K tile with the LDS
// transpose read (ds_read_b64_tr_b16).  Two output wavefronts form P and
// Q S^T and finish and store the outputs.  Two staging wavefronts stage the
// next chunk's K, Q, V, G and T' into LDS (loads issued a chunk ahead, and
// the workgroup's next item's first chunk during an item's last steps).  The
// chain and output wavefronts run on different SIMDs; two barriers per chunk
// separate phase 1 (K S^T, X, U; Q S^T and P) from phase 2 (S'; U P and the
// stores).
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

// Contraction slots.  The state, X, U and P enter the MFMAs straight from
// the accumulators of the products that made them: an accumulator lane
// (lg, lr) holds rows 4 lg .. 4 lg + 3 of a 16-row block.  So a 32-long
// contraction step kk gives the lane of group lg the eight slots
//   e = 0..7  ->  index 32 kk + 16 (e / 4) + 4 lg + e % 4,
// the lane's own rows of two adjacent 16-blocks, and every operand read
// from memory (K, Q, T') is laid out in that order too.
__host__ __device__ constexpr int slot_index(int kk, int lg, int e) { return 32 * kk + 16 * (e >> 2) + 4 * lg + (e & 3); }

// T' of one (chunk, value head) in A-operand order: one tile per (token
// block tb, contraction step kk <= tb / 2), tile tp_tile(tb, kk); a tile is
// 512 bf16 of hi then 512 of lo, lane l's 8 slots at 8 l: row t = 16 tb + l % 16,
// columns slot_index(kk, l / 16, e).  Columns past the diagonal hold zeros.
constexpr int kTpTiles = 6;
constexpr int kTpTileElems = 1024;                       // uint16 per tile (hi + lo)
constexpr int kTpElems = kTpTiles * kTpTileElems;        // per (chunk, value head)
__host__ __device__ constexpr int tp_tile(int tb, int kk) { return (tb < 3 ? tb : 4) + kk; }

// A token block as a compile-time constant (triangular loops over token
// blocks unroll with fixed bounds).
template <int V>
struct TokenBlock {
    static constexpr int value = V;
};

// ---------------------------------------------------------------------------
// prep: G and T' per (chunk, value head)
// ---------------------------------------------------------------------------
// One workgroup (4 wavefronts) per (chunk, key head): the chunk's K rows are
// read once and K K^T is formed once on MFMA (row block w per wavefront, kept
// in registers) for every value head of the key head; the K tile's LDS then
// holds A and T.  Per value head: G (a wave prefix sum, log2 units), A =
// strictly lower diag(b) (K K^T o e^{G_t - G_s}), T = (I + A)^-1 by forward
// substitution on the 16 x 16 diagonal blocks and block merges on split-bf16
// MFMA, then T' = T diag(b) written out as hi / lo blocks.  P value heads go
// through these steps together, each in its own A / T buffer (P = 2 when a
// key head has an even number of value heads): the diagonal blocks of value
// head p take lanes 16 p .. 16 p + 15 of each wavefront, its 16-block merges
// wavefronts 2 p and 2 p + 1, and every wavefront does its 32-block merge
// products for each of them, so a pair costs about one value head's
// latency.  Rows past a sequence end read K, g and b as zero, so T' has zero
// rows there and its valid block is the inverse of the valid part alone.  At
// most 128 VGPRs keep four workgroups on a CU (a tighter bound spills and
// measured slower).
template <int DK, int P>
__global__ __launch_bounds__(256, 4) void prep_tp_kernel(const PrefillArgs A) {
    constexpr int C = kChunk;
    constexpr int KP = DK + 8;   // padded bf16 row of the K tile
    constexpr int AP = C + 4;    // padded fp32 row (16-byte aligned rows)
    constexpr int NKK = DK / 32;
    constexpr int PPR = DK / 8;  // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;
    constexpr int NLD = 16 / RPI;
    static_assert(P == 1 || P == 2, "one or two value heads at a time");
    static_assert(C * KP * 2 <= C * AP * 4, "the K tile fits the A / T buffer");
    // per value head in flight: A, then T written over it; buffer 0 first holds K
    __shared__ __attribute__((aligned(16))) float Tm[P][C * AP];
    __bf16* const Ks = reinterpret_cast<__bf16*>(Tm[0]);
    __shared__ __attribute__((aligned(16))) float Gs[P][C];
    __shared__ __attribute__((aligned(16))) float Bs[P][C];

    const int H = A.H, HV = A.HV, R = HV / H;
    // workgroup id -> (chunk, key head): the key heads of a chunk on one XCD
    // (id % 8) in neighbouring slots, so the cache lines of g and beta that
    // they share (every value head of a token in one line) come from one L2
    const int id = blockIdx.x, slot = id >> 3;
    const int c = (slot / H) * 8 + (id & 7), hk = slot - (slot / H) * H, tid = threadIdx.x;
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

    // K rows of the key head (coalesced 16-byte pieces); g and b of value
    // head p for token l on wavefront p (zero past the end)
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
    if (w < P) load_gb(hk * R + w, gnext, bnext);
#pragma unroll
    for (int p = 0; p < NLD; ++p)
        *reinterpret_cast<bf8_t*>(&Ks[(16 * w + RPI * p + l / PPR) * KP + 8 * (l % PPR)]) = kst[p];
    __syncthreads();  // K is in LDS
    // K K^T of row block w, once for all value heads of the key head:
    // kk[sb][r] = (K K^T)[t = 16 w + 4 lg + r][s = 16 sb + lr]
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
    __syncthreads();  // every wavefront has read K: its buffer holds A and T from here

    for (int v0 = 0; v0 < R; v0 += P) {
        if (w < P) {
            // G (log2 units, inclusive in-chunk prefix sum) and b of value head v0 + w
            const int hv = hk * R + v0 + w;
            float gs = gnext * kLog2e;
            const float bv = bnext;
            if (v0 + P < R) load_gb(hv + P, gnext, bnext);  // the next pass's, in flight
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float up = __shfl_up(gs, off, 64);
                if (l >= off) gs += up;
            }
            Gs[w][l] = gs;
            Bs[w][l] = bv;
            A.ws_G[((size_t)c * HV + hv) * C + l] = gs;
        }
        __syncthreads();  // G and b are in LDS

        // A = strictly lower part of diag(b) (K K^T o e^{G_t - G_s}), row block w
#pragma unroll
        for (int p = 0; p < P; ++p) {
            float* const Am = Tm[p];
            const float4 g4 = *reinterpret_cast<const float4*>(&Gs[p][16 * w + 4 * lg]);
            const float4 b4 = *reinterpret_cast<const float4*>(&Bs[p][16 * w + 4 * lg]);
            const float gt[4] = {g4.x, g4.y, g4.z, g4.w};
            const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if (sb <= w) {
                    const float Gsb = Gs[p][16 * sb + lr];
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
        // diagonal blocks T_bb = (I + A_bb)^-1 by forward substitution:
        // wavefront b, lane 16 p + j of value head p owns column j
        if (l < 16 * P) {
            const int o = 16 * w;
            float* const Am = Tm[P == 1 ? 0 : (l >> 4)];
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
                float v_ = (t == lr) ? 1.f : 0.f;
#pragma unroll
                for (int x = 0; x < t; ++x) v_ -= arow[x] * col[x];
                col[t] = v_;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) Am[(o + t) * AP + o + lr] = col[t];
        }
        __syncthreads();
        // 16-block merges, value head p on wavefronts 2 p and 2 p + 1:
        //   T_{ii,j} = -T_{ii,ii} (A_{ii,j} T_{jj}),  (ii, j) = (1, 0), (3, 2)
        // (the 16-long contraction fills slots 0..3 of each lane group, slots
        // 4..7 are zero, so the first product's accumulators are the second
        // product's B operand)
        if (w < 2 * P) {
            float* const Tb = Tm[P == 1 ? 0 : (w >> 1)];
            const int j = 2 * (w & 1), ii = j + 1;
            const float4 a4 = *reinterpret_cast<const float4*>(&Tb[(16 * ii + lr) * AP + 16 * j + 4 * lg]);
            float av[8] = {a4.x, a4.y, a4.z, a4.w, 0.f, 0.f, 0.f, 0.f};
            float bv8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int y = 0; y < 4; ++y) bv8[y] = Tb[(16 * j + 4 * lg + y) * AP + 16 * j + lr];
            bf8_t ah, al, bh, bl;
            split8(av, ah, al);
            split8(bv8, bh, bl);
            f4_t xa = f4_t{0.f, 0.f, 0.f, 0.f};
            xa = mfma(ah, bh, xa);
            xa = mfma(ah, bl, xa);
            xa = mfma(al, bh, xa);
            const float4 t4 = *reinterpret_cast<const float4*>(&Tb[(16 * ii + lr) * AP + 16 * ii + 4 * lg]);
            float tv[8] = {t4.x, t4.y, t4.z, t4.w, 0.f, 0.f, 0.f, 0.f};
            float xv[8] = {xa[0], xa[1], xa[2], xa[3], 0.f, 0.f, 0.f, 0.f};
            split8(tv, ah, al);
            split8(xv, bh, bl);
            f4_t ta = f4_t{0.f, 0.f, 0.f, 0.f};
            ta = mfma(ah, bh, ta);
            ta = mfma(ah, bl, ta);
            ta = mfma(al, bh, ta);
#pragma unroll
            for (int r = 0; r < 4; ++r) Tb[(16 * ii + 4 * lg + r) * AP + 16 * j + lr] = -ta[r];
        }
        __syncthreads();
        // 32-block merge: X = A[32:64, 0:32] T[0:32, 0:32] into the upper-right
        // block; T[32:64, 0:32] = -T_B X.  Wavefront w: row block w >> 1,
        // column block w & 1, for each value head in flight.
        const int tbm = w >> 1, jb = w & 1;
        {
            f4_t xa[P];
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const float* const Tb = Tm[p];
                float av[8], bv8[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    av[x] = Tb[(32 + 16 * tbm + lr) * AP + 8 * lg + x];
                    const int xr = 8 * lg + x, cc = 16 * jb + lr;
                    bv8[x] = (xr >= cc) ? Tb[xr * AP + cc] : 0.f;
                }
                bf8_t ah, al, bh, bl;
                split8(av, ah, al);
                split8(bv8, bh, bl);
                xa[p] = f4_t{0.f, 0.f, 0.f, 0.f};
                xa[p] = mfma(ah, bh, xa[p]);
                xa[p] = mfma(ah, bl, xa[p]);
                xa[p] = mfma(al, bh, xa[p]);
            }
#pragma unroll
            for (int p = 0; p < P; ++p) {
                float* const Xm = Tm[p] + 32;
#pragma unroll
                for (int r = 0; r < 4; ++r) Xm[(16 * tbm + 4 * lg + r) * AP + 16 * jb + lr] = xa[p][r];
            }
        }
        __syncthreads();
        {
            f4_t ta[P];
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const float* const Tb = Tm[p];
                const float* const Xm = Tb + 32;
                float av[8], bv8[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const int rr = 16 * tbm + lr, xc = 8 * lg + x;  // T_B row rr, column xc (lower)
                    av[x] = (xc <= rr) ? Tb[(32 + rr) * AP + 32 + xc] : 0.f;
                    bv8[x] = Xm[(8 * lg + x) * AP + 16 * jb + lr];
                }
                bf8_t ah, al, bh, bl;
                split8(av, ah, al);
                split8(bv8, bh, bl);
                ta[p] = f4_t{0.f, 0.f, 0.f, 0.f};
                ta[p] = mfma(ah, bh, ta[p]);
                ta[p] = mfma(ah, bl, ta[p]);
                ta[p] = mfma(al, bh, ta[p]);
            }
#pragma unroll
            for (int p = 0; p < P; ++p) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Tm[p][(32 + 16 * tbm + 4 * lg + r) * AP + 16 * jb + lr] = -ta[p][r];
            }
        }
        __syncthreads();
        // T' = T diag(b) in tile order (unit u = (value head, tile, lane)), hi /
        // lo.  A select, not a 0/1 factor, zeroes the slots past the diagonal
        // (T's upper blocks hold scratch data).
        constexpr int kUnits = kTpTiles * 64;
#pragma unroll
        for (int q = 0; q < (P * kUnits + 255) / 256; ++q) {
            const int u = tid + 256 * q;
            if (u < P * kUnits) {
                const int p = P == 1 ? 0 : u / kUnits, uu = u - p * kUnits;
                const int ti = uu >> 6, ul = uu & 63, ulr = ul & 15, ulg = ul >> 4;
                const int tb = ti < 2 ? ti : (ti < 4 ? 2 : 3);
                const int kk = ti - tp_tile(tb, 0);
                const int t = 16 * tb + ulr;
                const float* const Tb = Tm[p];
                float pv[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int s0 = slot_index(kk, ulg, 4 * hh);
                    const float4 x4 = *reinterpret_cast<const float4*>(&Tb[t * AP + s0]);
                    const float4 b4 = *reinterpret_cast<const float4*>(&Bs[p][s0]);
                    const float tv[4] = {x4.x, x4.y, x4.z, x4.w};
                    const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) pv[4 * hh + r] = (s0 + r <= t) ? tv[r] * bb[r] : 0.f;
                }
                bf8_t hi, lo;
                split8(pv, hi, lo);
                uint16_t* const tp = A.ws_Tp + ((size_t)c * HV + hk * R + v0 + p) * kTpElems;
                *reinterpret_cast<bf8_t*>(tp + ti * kTpTileElems + ul * 8) = hi;
                *reinterpret_cast<bf8_t*>(tp + ti * kTpTileElems + 512 + ul * 8) = lo;
            }
        }
        __syncthreads();  // Tm, Gs and Bs are rewritten for the next pass
    }
}

// ---------------------------------------------------------------------------
// scan: sequential over chunks; state rows split over chain wavefronts, the
// output over output wavefronts
// ---------------------------------------------------------------------------
// The scan workgroup's LDS, declared once in the kernel: the chain and output
// wavefronts and the staging wavefronts run separate item loops over it.
template <int DK>
struct ScanLds {
    static constexpr int C = kChunk, KR = DK + 16, VR = 32 + 16;
    __attribute__((aligned(16))) __bf16 Ks[2][C * KR];  // K [t][slot order], by chunk parity
    __attribute__((aligned(16))) __bf16 Qs[2][C * KR];  // Q [t][slot order]
    __attribute__((aligned(16))) __bf16 Vs[2][C * VR];  // V [t][i] of the tile
    __attribute__((aligned(16))) uint16_t Tp[2][kTpElems];
    __attribute__((aligned(16))) float Gs[2][3][C];     // G, e^{G}, e^{G_n - G}
    __attribute__((aligned(16))) bf8_t Sx[2][4][2][64]; // chain S operands [a][kk][hi, lo][lane]
    __attribute__((aligned(16))) float4 Uf[2][2][2][64];  // chain U, fp32 [a][kk][half][lane]
    __attribute__((aligned(16))) bf8_t Px[kTpTiles][2][64];  // P tiles [tile][hi, lo][lane]
};

// Work items: (segment, value head, 32-row tile of S) value items first, then
// the transition items of later segments (the same scan from the identity
// with V read as zero: d_k rows, writing w = scale Phi_t q_t instead of o and
// Phi^T instead of the state).  Items are numbered by key chain (segment, key
// head): every tile of every value head of a key head gets the same b % 8 and
// neighbouring dispatch slots (workgroup b runs on XCD b % 8), so their shared
// K, Q reads meet in one L2.
//
// One work item's coordinates, every field wavefront-uniform; valid 0: an
// item with nothing to do (a key chain past the plan's segments, or the
// transition item of a first segment); live: valid with chunks to scan.
struct ScanItem {
    int valid, live, trans, sg, hk, h, tile, n, sidx, whole, c_first, nch, sq, eq;
};

// Item b's coordinates.  The table reads take two dependent rounds: the segment's entries (its index
// clamped into the tables, so that an item past the plan reads in bounds),
// then its sequence's; an item's validity is decided after both.
template <int DK>
__device__ __forceinline__ ScanItem scan_item(const PrefillArgs& A, const int b) {
    constexpr int C = kChunk, BV = 32;
    const int H = A.H, HV = A.HV, dv = A.dv;
    const int R = HV / H;
    const int TV = dv / BV;
    const int nb1 = ((A.seg_bound * H + 7) / 8) * 8 * R * TV;
    const bool trans = b >= nb1;
    const int bb = trans ? b - nb1 : b;
    const int TT = trans ? DK / BV : TV;
    const int slot = bb >> 3;
    const int per = R * TT;
    const int kc = (slot / per) * 8 + (bb & 7);
    const int rem = slot - (slot / per) * per;
    const int sg = kc / H;
    const int sgc = min(sg, A.seg_bound - 1);
    const int nseg = __builtin_amdgcn_readfirstlane(A.plan[0]);
    const int n0 = __builtin_amdgcn_readfirstlane(A.seg_seq[sgc]);
    const int sidx = __builtin_amdgcn_readfirstlane(A.seg_idx[sgc]);
    const int c_first = __builtin_amdgcn_readfirstlane(A.seg_c0[sgc]);
    int nch = __builtin_amdgcn_readfirstlane(A.seg_nch[sgc]);
    const int n = min(max(n0, 0), A.N - 1);
    int sq, eq;
    seq_bounds_m(A.cu_seqlens, n, A.T, sq, eq);
    const int coff = __builtin_amdgcn_readfirstlane(A.chunk_off[n]);
    const int nsq = __builtin_amdgcn_readfirstlane(A.seq_nseg[n]);
    sq += (c_first - min(coff, A.max_chunks)) * C;  // the segment's first token
    if (c_first + nch > A.max_chunks) nch = max(0, A.max_chunks - c_first);
    ScanItem it;
    it.valid = (kc < nseg * H && !(trans && sidx == 0)) ? 1 : 0;
    it.live = (it.valid && nch > 0) ? 1 : 0;
    it.trans = trans ? 1 : 0;
    it.sg = sg;
    it.hk = kc - sg * H;
    it.h = it.hk * R + rem / TT;
    it.tile = rem % TT;
    it.n = n;
    it.sidx = sidx;
    it.whole = nsq == 1 ? 1 : 0;
    it.c_first = c_first;
    it.nch = nch;
    it.sq = __builtin_amdgcn_readfirstlane(sq);
    it.eq = __builtin_amdgcn_readfirstlane(eq);
    return it;
}

// The rows of S evolve independently.  Chain wavefront a (0, 1) owns rows
// i = 16 a .. 16 a + 15 of the tile:
//   sacc[jb][r] = S^T[j = 16 jb + 4 lg + r][i = 16 a + lr]
// are the B operand of K S^T, and K S^T, X, U and U' come out of one product
// in the lane layout the next one takes (the contraction slots above), so the
// chain step needs nothing from other wavefronts.  Per chunk, with
// gamma_t = e^{G_t}:
//   X = V - diag(gamma) K S^T,  U = T' X,  U' = diag(e^{G_n - G}) U,
//   S'^T = gamma_n S^T + K^T U'.
// Output wavefront 2 + a takes the chain's S operands and U from LDS and forms
//   O^T = scale (S Q^T diag(gamma) + U^T P^T),  P = (Q K^T) o e^{G_t - G_s} [s <= t],
// each output wavefront computing the P tiles of two token blocks for both.
// Wavefronts 4 and 5 stage the next chunk's K, Q, V, T' and G into the other
// LDS buffers.  A chunk step has two phases:
//   1: chain K S^T, X, U = T' X, U to LDS;  output S Q^T, its P tiles to LDS;
//   2: chain S' and its operands to LDS;     output U^T P^T and the stores.
// K and Q rows are stored with their columns in slot order (an operand read
// is 16 contiguous bytes); a K^T operand is two transpose reads.
template <int DK, typename Tout>
__device__ __forceinline__ void scan_tp_item(const PrefillArgs& A, const int b, ScanLds<DK>& S) {
    static_assert(DK == 128, "the row-split scan is written for d_k = 128");
    constexpr int C = kChunk;
    constexpr int BV = 32;        // state rows per workgroup
    constexpr int KR = DK + 16;   // bf16 per K / Q row in LDS (288 bytes)
    constexpr int VR = BV + 16;   // bf16 per V row in LDS (96 bytes)
    constexpr int NJB = DK / 16;  // 16-column blocks of the state
    auto& Ks = S.Ks;
    auto& Qs = S.Qs;
    auto& Vs = S.Vs;
    auto& Tp = S.Tp;
    auto& Gs = S.Gs;
    auto& Sx = S.Sx;
    auto& Uf = S.Uf;
    auto& Px = S.Px;
    typedef short v4s_t __attribute__((ext_vector_type(4)));

    const int HV = A.HV, dv = A.dv;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(w >= 0 && w < 4);
    const int l = tid & 63, lr = l & 15, lg = l >> 4;

    const ScanItem it = scan_item<DK>(A, b);
    if (!it.valid) return;
    const bool trans = it.trans != 0;
    const int sg = it.sg, h = it.h, tile = it.tile, n = it.n, sidx = it.sidx;
    const int nch = it.nch, sq = it.sq, eq = it.eq;
    auto chunk_t0 = [&](int jc) { return sq + jc * C; };
    auto chunk_L = [&](int jc) { return min(C, eq - (sq + jc * C)); };

    if (w < 2) {
        // ===================== chain wavefront =====================
        const float* init = nullptr;  // null: zero state (or the identity for a transition item)
        float* fin;
        size_t ibase = 0, fbase;
        if (trans) {
            fin = A.ws_Phi;
            fbase = ((size_t)(sg * HV + h) * DK + (size_t)tile * BV) * DK;
        } else if (sidx == 0) {
            init = A.s0;
            ibase = ((size_t)(n * HV + h) * dv + (size_t)tile * BV) * DK;
            const bool whole = it.whole != 0;
            fin = whole ? A.s_final : A.ws_E;
            fbase = whole ? ibase : ((size_t)(sg * HV + h) * dv + (size_t)tile * BV) * DK;
        } else {
            fin = A.ws_E;
            fbase = ((size_t)(sg * HV + h) * dv + (size_t)tile * BV) * DK;
        }
        const int il = 16 * w + lr;  // the lane's state row in the tile
        f4_t sacc[NJB];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            const int j = 16 * jb + 4 * lg;
            if (init) {
                const float4 v4 = *reinterpret_cast<const float4*>(init + ibase + (size_t)il * DK + j);
                sacc[jb] = f4_t{v4.x, v4.y, v4.z, v4.w};
            } else if (trans) {
                const int d = tile * BV + il - j;  // identity: 1 where row == column
                sacc[jb] = f4_t{d == 0 ? 1.f : 0.f, d == 1 ? 1.f : 0.f, d == 2 ? 1.f : 0.f, d == 3 ? 1.f : 0.f};
            } else {
                sacc[jb] = f4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
        // the state as split-bf16 operands, one per contraction step; also
        // handed to the output wavefront of these rows
        bf8_t sh[4], sl[4];
        auto state_operands = [&]() {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                float sv[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sv[r] = sacc[2 * kk][r];
                    sv[4 + r] = sacc[2 * kk + 1][r];
                }
                split8(sv, sh[kk], sl[kk]);
                Sx[w][kk][0][l] = sh[kk];
                Sx[w][kk][1][l] = sl[kk];
            }
        };
        if (nch > 0) {
            state_operands();
            __syncthreads();  // B0: chunk 0 staged, the state operands in LDS
        }
        for (int jc = 0; jc < nch; ++jc) {
            const int pb = jc & 1;
            const int L = chunk_L(jc);
            const float* G1 = Gs[pb][1];
            const float* G2 = Gs[pb][2];
            // the LDS operands of X, U' and phase 2 first, so that their latency
            // passes under the K S^T products (pinned here: the scheduler would
            // otherwise sink each read to its first use)
            v4s_t vv[4];
            float4 g1v[4], g2v[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                vv[tb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(
                    &Vs[pb][(16 * tb + 4 * lg + (lr >> 2)) * VR + 16 * w + 4 * (lr & 3)]));
                g1v[tb] = *reinterpret_cast<const float4*>(&G1[16 * tb + 4 * lg]);
                g2v[tb] = *reinterpret_cast<const float4*>(&G2[16 * tb + 4 * lg]);
            }
            const float gn = G1[L - 1];
            __builtin_amdgcn_sched_barrier(0);
            // ---- phase 1: K S^T [t][i] ----
            f4_t aks[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) aks[x] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf8_t kf[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) kf[x] = lds8(&Ks[pb][(16 * x + lr) * KR + 32 * kk + 8 * lg]);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    aks[tb] = mfma(kf[tb], sh[kk], aks[tb]);
                    aks[tb] = mfma(kf[tb], sl[kk], aks[tb]);
                }
            }
            // T' read before X is formed, so that its latency passes under the
            // X arithmetic (pinned as above)
            bf8_t tph[kTpTiles], tpl[kTpTiles];
#pragma unroll
            for (int ti = 0; ti < kTpTiles; ++ti) {
                tph[ti] = *reinterpret_cast<const bf8_t*>(&Tp[pb][ti * kTpTileElems + 8 * l]);
                tpl[ti] = *reinterpret_cast<const bf8_t*>(&Tp[pb][ti * kTpTileElems + 512 + 8 * l]);
            }
            __builtin_amdgcn_sched_barrier(0);
            // X = V - diag(gamma) K S^T: V[t = 16 tb + 4 lg + r][i] by a transpose
            // read (lane m of a 16-lane group points at row 16 tb + 4 lg + m / 4,
            // columns 16 a + 4 (m % 4) ..)
            float xv[4][4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float gam[4] = {g1v[tb].x, g1v[tb].y, g1v[tb].z, g1v[tb].w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    xv[tb][r] = __uint_as_float((uint32_t)(uint16_t)vv[tb][r] << 16) - gam[r] * aks[tb][r];
            }
            bf8_t xh[2], xl[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                float v8[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v8[r] = xv[2 * kk][r];
                    v8[4 + r] = xv[2 * kk + 1][r];
                }
                split8(v8, xh[kk], xl[kk]);
            }
            // U = T' X (T' lower: steps kk <= tb / 2)
            f4_t ua[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                ua[tb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk <= (tb >> 1); ++kk) {
                    const bf8_t th = tph[tp_tile(tb, kk)];
                    const bf8_t tl = tpl[tp_tile(tb, kk)];
                    ua[tb] = mfma(th, xh[kk], ua[tb]);
                    ua[tb] = mfma(th, xl[kk], ua[tb]);
                    ua[tb] = mfma(tl, xh[kk], ua[tb]);
                }
            }
            // U to the output wavefront (fp32: it splits U itself); U' =
            // diag(e^{G_n - G}) U kept
            bf8_t wh[2], wl[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                float wv[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int tb = 2 * kk + hh;
                    const float dd[4] = {g2v[tb].x, g2v[tb].y, g2v[tb].z, g2v[tb].w};
                    Uf[w][kk][hh][l] = make_float4(ua[tb][0], ua[tb][1], ua[tb][2], ua[tb][3]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) wv[4 * hh + r] = ua[tb][r] * dd[r];
                }
                split8(wv, wh[kk], wl[kk]);
            }
            // the K^T operands of phase 2, read while the barrier waits: K^T rows
            // j = 16 jb + lr over the step's token slots, two transpose reads
            // (tokens 32 kk + 4 lg + m / 4 and 16 more), lane m pointing at the
            // stored column of j-group 16 jb + 4 (m % 4)
            bf8_t ktp[2][NJB];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    const int col = 32 * (jb >> 1) + 8 * (lr & 3) + 4 * (jb & 1);
                    const __bf16* kp = &Ks[pb][(32 * kk + 4 * lg + (lr >> 2)) * KR + col];
                    const v4s_t k0 =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(kp));
                    const v4s_t k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s_t*)(kp + 16 * KR));
                    ktp[kk][jb] = __builtin_bit_cast(bf8_t, __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            }
            __syncthreads();  // B1
            // ---- phase 2: S'^T = gamma_n S^T + K^T U' ----
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[jb][r] *= gn;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    sacc[jb] = mfma(ktp[kk][jb], wh[kk], sacc[jb]);
                    sacc[jb] = mfma(ktp[kk][jb], wl[kk], sacc[jb]);
                }
            }
            // (after the last chunk too, where nothing reads them: no branch
            // between the products and the split)
            state_operands();
            __syncthreads();  // B2
        }
        // the final state (Phi^T for a transition item), from one base
        // address per lane so that the stores issue back to back
        if (fin && trans) {
            // Phi is stored transposed (Phi^T[j][i]): the combine pass reads
            // it as an MFMA B operand, 8 consecutive i per lane
            float* const fp = fin + (size_t)(sg * HV + h) * DK * DK + (size_t)(4 * lg) * DK + tile * BV + il;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r) fp[(size_t)(16 * jb + r) * DK] = sacc[jb][r];
        } else if (fin) {
            float* const fp = fin + fbase + (size_t)il * DK + 4 * lg;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
                *reinterpret_cast<float4*>(fp + 16 * jb) = make_float4(sacc[jb][0], sacc[jb][1], sacc[jb][2], sacc[jb][3]);
        }
        return;
    }

    if (nch <= 0) return;
    if (w < 4) {
        // ===================== output wavefront =====================
        const int a = w - 2;  // the chain (rows 16 a ..) whose output this is
        Tout* op = static_cast<Tout*>(A.o);
        __syncthreads();  // B0
        // P tiles of token blocks T0 and T1 (compile-time), from the
        // (K Q^T)^T blocks pq[x][sb][r] = (K Q^T)^T[s = 16 sb + 4 lg + r][t = 16 T + lr]
        auto output_step = [&](auto T0c, auto T1c, int jc) {
            constexpr int T0 = decltype(T0c)::value, T1 = decltype(T1c)::value;
            const int pb = jc & 1;
            const int t0 = chunk_t0(jc), L = chunk_L(jc);
            const float* G0 = Gs[pb][0];
            const float* G1 = Gs[pb][1];
            // ---- phase 1: S Q^T [i][t] and the P tiles ----
            bf8_t sh[4], sl[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                sh[kk] = Sx[a][kk][0][l];
                sl[kk] = Sx[a][kk][1][l];
            }
            f4_t aqs[4], pq0[T0 + 1], pq1[T1 + 1];
#pragma unroll
            for (int x = 0; x < 4; ++x) aqs[x] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x <= T0; ++x) pq0[x] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x <= T1; ++x) pq1[x] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf8_t qf[4], kf[T1 + 1];
#pragma unroll
                for (int x = 0; x < 4; ++x) qf[x] = lds8(&Qs[pb][(16 * x + lr) * KR + 32 * kk + 8 * lg]);
#pragma unroll
                for (int x = 0; x <= T1; ++x) kf[x] = lds8(&Ks[pb][(16 * x + lr) * KR + 32 * kk + 8 * lg]);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    aqs[tb] = mfma(sh[kk], qf[tb], aqs[tb]);
                    aqs[tb] = mfma(sl[kk], qf[tb], aqs[tb]);
                }
#pragma unroll
                for (int sb = 0; sb <= T0; ++sb) pq0[sb] = mfma(kf[sb], qf[T0], pq0[sb]);
#pragma unroll
                for (int sb = 0; sb <= T1; ++sb) pq1[sb] = mfma(kf[sb], qf[T1], pq1[sb]);
            }
            auto p_tiles = [&](auto Tc, const f4_t* pq) {
                constexpr int tb = decltype(Tc)::value;
                const int t = 16 * tb + lr;
                const float Gt = G0[t];
#pragma unroll
                for (int kk = 0; kk <= (tb >> 1); ++kk) {
                    float pv[8];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int sb = 2 * kk + hh;
                        if (sb > tb) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) pv[4 * hh + r] = 0.f;
                            continue;
                        }
                        const float4 g4 = *reinterpret_cast<const float4*>(&G0[16 * sb + 4 * lg]);
                        const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            // G_t - G_s <= 0 for s <= t; the diagonal block masks
                            // s > t by a 0 / 1 factor (the factor is finite)
                            float f = exp2f_(fminf(Gt - gs[r], 0.f));
                            if (sb == tb) f *= (4 * lg + r <= lr) ? 1.f : 0.f;
                            pv[4 * hh + r] = pq[sb][r] * f;
                        }
                    }
                    bf8_t ph, pl;
                    split8(pv, ph, pl);
                    Px[tp_tile(tb, kk)][0][l] = ph;
                    Px[tp_tile(tb, kk)][1][l] = pl;
                }
            };
            p_tiles(T0c, pq0);
            p_tiles(T1c, pq1);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float gt = G1[16 * tb + lr];
#pragma unroll
                for (int r = 0; r < 4; ++r) aqs[tb][r] *= gt;
            }
            __syncthreads();  // B1
            // ---- phase 2: + U^T P^T, then stored: aqs[tb][r] =
            // O[t = 16 tb + lr][i = 16 a + 4 lg + r]; rows t >= L land at or past
            // the resource end and are dropped.  A transition item writes w
            // (fp32, d_k per token and head) instead of o. ----
            bf8_t uh[2], ul[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float4 u0 = Uf[a][kk][0][l], u1 = Uf[a][kk][1][l];
                float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
                split8(uv, uh[kk], ul[kk]);
            }
            const __amdgpu_buffer_rsrc_t orsrc =
                trans ? out_rsrc(A.ws_W + (size_t)t0 * HV * DK, (uint32_t)(L * HV * DK * 4))
                      : out_rsrc(op + (size_t)t0 * HV * dv, (uint32_t)(L * HV * dv * sizeof(Tout)));
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                for (int kk = 0; kk <= (tb >> 1); ++kk) {
                    const bf8_t ph = Px[tp_tile(tb, kk)][0][l];
                    const bf8_t pl = Px[tp_tile(tb, kk)][1][l];
                    aqs[tb] = mfma(uh[kk], ph, aqs[tb]);
                    aqs[tb] = mfma(ul[kk], ph, aqs[tb]);
                    aqs[tb] = mfma(uh[kk], pl, aqs[tb]);
                }
                const int t = 16 * tb + lr;
                const float ov[4] = {A.scale * aqs[tb][0], A.scale * aqs[tb][1], A.scale * aqs[tb][2],
                                     A.scale * aqs[tb][3]};
                if (trans)
                    out_store4(orsrc, (uint32_t)((t * HV + h) * DK + tile * BV + 16 * a + 4 * lg), ov, A.ws_W);
                else
                    out_store4(orsrc, (uint32_t)((t * HV + h) * dv + tile * BV + 16 * a + 4 * lg), ov, op);
            }
            __syncthreads();  // B2
        };
        for (int jc = 0; jc < nch; ++jc) {
            if (a == 0)
                output_step(TokenBlock<0>{}, TokenBlock<3>{}, jc);
            else
                output_step(TokenBlock<1>{}, TokenBlock<2>{}, jc);
        }
        return;
    }
}

// The staging wavefronts' own item loop.  They stage each item's chunks one
// step ahead and keep the chunk after it in flight, as in one item; during an
// item's last steps they load the first chunk of the workgroup's next item,
// so that item's first barrier does not wait on memory.  Per item they pass
// the same barriers as the other roles: one at the item's top, then, for an
// item with chunks, B0 and two per chunk.
template <int DK>
__device__ __forceinline__ void scan_tp_stage(const PrefillArgs& A, const int items, ScanLds<DK>& S) {
    constexpr int C = kChunk;
    constexpr int BV = 32;
    constexpr int KR = DK + 16;
    constexpr int VR = BV + 16;
    const int H = A.H, HV = A.HV, dv = A.dv;
    const int hp = threadIdx.x - 256;              // 0..127
    const uint32_t qk_row = (uint32_t)H * DK * 2;  // bytes per token of q, k
    const uint32_t v_row = (uint32_t)HV * dv * 2;  // bytes per token of v
    // K and Q: piece p = hp + 128 q, row p / 16, 16-byte column chunk c = p % 16
    // holding columns 8 c .. 8 c + 7, stored as two 8-byte halves at their slots
    uint32_t kq_off[8];
    int kq_st[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int p = hp + 128 * q, row = p >> 4, c16 = p & 15;
        kq_off[q] = (uint32_t)row * qk_row + 16 * c16;
        // columns 8 c .. 8 c + 3 are slots 4 h + 0..3 of lane group 2 (c % 2)
        // in step c / 4 (h = (c / 2) % 2), stored at 32 kk + 8 lg + 4 h
        kq_st[q] = row * KR + 32 * (c16 >> 2) + 16 * (c16 & 1) + 4 * ((c16 >> 1) & 1);
    }
    // V: piece p = hp + 128 q (q < 2): token p / 4, rows 8 (p % 4) .. + 7 of the tile
    uint32_t v_off[2];
    int v_st[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int p = hp + 128 * q, tok = p >> 2, part = p & 3;
        v_off[q] = (uint32_t)tok * v_row + 16 * part;
        v_st[q] = tok * VR + 8 * part;
    }
    bf8_t kst[8], qst[8], vst[2], tst[6];
    float gst = 0.f, gnst = 0.f;
    auto load_chunk = [&](const ScanItem& it, const int jc) {
        const int t0 = it.sq + jc * C, L = min(C, it.eq - t0);
        const uint32_t kq_h = (uint32_t)it.hk * DK * 2;
        const uint32_t v_h = ((uint32_t)it.h * dv + (uint32_t)it.tile * BV) * 2;
        const uint32_t v_on = it.trans ? 0u : 1u;  // a transition item reads V as zero
        const __amdgpu_buffer_rsrc_t rk =
            in_rsrc(static_cast<const bf16_t*>(A.k) + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
        const __amdgpu_buffer_rsrc_t rq =
            in_rsrc(static_cast<const bf16_t*>(A.q) + (size_t)t0 * H * DK, (uint32_t)L * qk_row);
        const __amdgpu_buffer_rsrc_t rv =
            in_rsrc(static_cast<const bf16_t*>(A.v) + (size_t)t0 * HV * dv, v_on * L * v_row);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            kst[q] = bload8(rk, kq_off[q] + kq_h);
            qst[q] = bload8(rq, kq_off[q] + kq_h);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) vst[q] = bload8(rv, v_off[q] + v_h);
        const uint16_t* tp = A.ws_Tp + ((size_t)(it.c_first + jc) * HV + it.h) * kTpElems;
#pragma unroll
        for (int q = 0; q < 6; ++q) tst[q] = gld8(tp + 8 * (hp + 128 * q));
        const float* gp = A.ws_G + ((size_t)(it.c_first + jc) * HV + it.h) * C;
        // every lane loads (lanes hp >= C a copy): a value defined on some
        // lanes only would be copied between registers, which waits for it
        gst = gp[hp & (C - 1)];
        gnst = gp[L - 1];
    };
    auto stage_chunk = [&](int jc) {
        const int pb = jc & 1;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint4 k4 = __builtin_bit_cast(uint4, kst[q]);
            const uint4 q4 = __builtin_bit_cast(uint4, qst[q]);
            *reinterpret_cast<uint2*>(&S.Ks[pb][kq_st[q]]) = make_uint2(k4.x, k4.y);
            *reinterpret_cast<uint2*>(&S.Ks[pb][kq_st[q] + 8]) = make_uint2(k4.z, k4.w);
            *reinterpret_cast<uint2*>(&S.Qs[pb][kq_st[q]]) = make_uint2(q4.x, q4.y);
            *reinterpret_cast<uint2*>(&S.Qs[pb][kq_st[q] + 8]) = make_uint2(q4.z, q4.w);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) *reinterpret_cast<bf8_t*>(&S.Vs[pb][v_st[q]]) = vst[q];
#pragma unroll
        for (int q = 0; q < 6; ++q) *reinterpret_cast<bf8_t*>(&S.Tp[pb][8 * (hp + 128 * q)]) = tst[q];
        if (hp < C) {
            S.Gs[pb][0][hp] = gst;
            S.Gs[pb][1][hp] = exp2f_(gst);
            S.Gs[pb][2][hp] = exp2f_(gnst - gst);
        }
    };
    bool have = false;  // the registers hold item b's first chunk (loaded during the previous item)
    for (int b = blockIdx.x; b < items; b += gridDim.x) {
        __syncthreads();  // the previous item has finished with the LDS
        const ScanItem it = scan_item<DK>(A, b);
        if (!it.live) continue;
        const int nch = it.nch;
        ScanItem nx{};
        if (b + (int)gridDim.x < items) nx = scan_item<DK>(A, b + gridDim.x);
        if (!have) load_chunk(it, 0);
        stage_chunk(0);
        if (nch > 1)
            load_chunk(it, 1);
        else if (nx.live)
            load_chunk(nx, 0);
        __syncthreads();  // B0
        // the next chunk into the other buffers (their last reader finished
        // before the previous step's second barrier), the one after it in
        // flight; every step of this loop stages and loads, so the registers'
        // pending loads are the same on every path into it
        int jc = 0;
        for (; jc + 2 < nch; ++jc) {
            stage_chunk(jc + 1);
            load_chunk(it, jc + 2);
            __syncthreads();  // B1
            __syncthreads();  // B2
        }
        if (nch > 1) {
            // the last chunk staged, the next item's first in flight
            stage_chunk(nch - 1);
            if (nx.live) load_chunk(nx, 0);
            __syncthreads();  // B1
            __syncthreads();  // B2
        }
        __syncthreads();  // B1 of the last step
        __syncthreads();  // B2
        have = nx.live;
    }
}

// Persistent over work items, as the per-tile scan: workgroup blockIdx.x takes
// items blockIdx.x, blockIdx.x + gridDim.x, ... (the grid is a multiple of 8,
// so an item keeps its XCD).  The chain and output wavefronts run the item
// loop here, the staging wavefronts their own (the same items and barriers),
// which carries the next item's first chunk in registers.
template <int DK, typename Tout>
__global__ __launch_bounds__(384) void scan_tp_kernel(const PrefillArgs A, int items) {
    __shared__ ScanLds<DK> S;
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= 4) {
        scan_tp_stage<DK>(A, items, S);
        return;
    }
    for (int b = blockIdx.x; b < items; b += gridDim.x) {
        __syncthreads();  // the previous item has finished with the LDS
        scan_tp_item<DK, Tout>(A, b, S);
    }
}

hipError_t launch_prep_tp(const PrefillArgs& A) {
    const unsigned grid = (unsigned)((A.max_chunks + 7) / 8) * 8u * (unsigned)A.H;
    if ((A.HV / A.H) % 2 == 0)
        hipLaunchKernelGGL((prep_tp_kernel<128, 2>), dim3(grid), dim3(256), 0, A.stream, A);
    else
        hipLaunchKernelGGL((prep_tp_kernel<128, 1>), dim3(grid), dim3(256), 0, A.stream, A);
    return hipGetLastError();
}

hipError_t launch_scan_tp(const PrefillArgs& A, size_t grid, int items) {
    if (A.o_bf16)
        hipLaunchKernelGGL((scan_tp_kernel<128, bf16_t>), dim3((unsigned)grid), dim3(384), 0,
                           A.stream, A, items);
    else
        hipLaunchKernelGGL((scan_tp_kernel<128, float>), dim3((unsigned)grid), dim3(384), 0,
                           A.stream, A, items);
    return hipGetLastError();
}

}  // namespace gdn

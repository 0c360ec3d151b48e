// gdn_attn.hip -- one decode step of gated full attention (gfx950).
//
// The hybrid decoder's other token mixer (Qwen3.5-0.8B chat guide, section
// "Architektur": standard scaled dot-product attention; Core AI card for
// Qwen3.6-35B-A3B, introduction: head_dim 256, 16 query heads over 2
// key/value heads, partial mRoPE with theta = 1e7).  Per row n and query head
// h (key/value head h / G, G = Hq / Hkv):
//
//     qr = rope(q, p), kr = rope(k_new, p), p = pos[n]
//     s_t = scale qr . K_t (t < p: cached, rotated keys; t = p: kr)
//     o = sigmoid(gate) * sum_t softmax(s)_t V_t      (V_p = v_new)
//
// and the step appends kr and v_new to the cache at row p.  rope rotates the
// pairs (i, i + rd/2), i < rd/2, by p theta^(-2i/rd) (the same position on
// every mRoPE section, as for text).
//
// The step is bound by reading the cache: 2 D bytes of bf16 key and value per
// position and key/value head, against 4 G D flops.  Split over positions
// (flash decoding): a workgroup takes `split` positions of one (row, kv head)
// for all G query heads of the group, so each cache row is read once.  Scores
// on MFMA (v_mfma_f32_16x16x32_bf16, query heads as the 16 rows, q split into
// hi + lo bf16 against the exact bf16 keys), an online softmax per head, and
// P V on MFMA as well (v_mfma_f32_16x16x16_bf16 per 16 value dimensions, the
// block's value rows, read as whole cache lines, staged in the wavefront's
// LDS area and read back transposed; P split into hi + lo).  A second kernel
// merges the splits and applies the gate.
#include <math.h>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {

constexpr int kAttnWG = 256;       // threads of a split workgroup (4 wavefronts)
constexpr int kAttnTarget = 512;   // split workgroups a launch aims at (one round, 2 per CU)
constexpr int kAttnMinSplit = 256; // positions per split, at least
// The cache rows are read once per step: non-temporal loads (buffer cache
// policy nt) keep them from displacing other lines, measured ~2.5 % faster at
// the 35B-A3B shape
constexpr int kCacheNt = 2;

// Split size: about kAttnTarget workgroups over the batch (measured at 128
// rows x 8192 positions with two blocks in flight per wavefront: 512 beats
// 1024), each at least kAttnMinSplit positions.  Workspace: one partial result per split,
// [N, Hkv, nsplit, G, D + 2] fp32 (o relative to m, m, the sum).
void attn_plan(int N, int Hq, int Hkv, int D, int Lmax, int& split, int& nsplit, size_t& bytes) {
    const long pairs = (long)N * Hkv;
    long want = (kAttnTarget + pairs - 1) / (pairs > 0 ? pairs : 1);
    if (want < 1) want = 1;
    long sp = ((Lmax + want - 1) / want + 15) / 16 * 16;
    if (sp < kAttnMinSplit) sp = kAttnMinSplit;
    split = (int)sp;
    nsplit = (int)((Lmax + sp - 1) / sp);
    bytes = (size_t)pairs * nsplit * (Hq / Hkv) * (D + 2) * sizeof(float);
}

template <int D, int G>
// (at most 256 registers a lane: two workgroups on a CU, where the LDS of
// groups of up to 8 query heads allows two)
__global__ __launch_bounds__(kAttnWG, G <= 8 ? 2 : 1) void attn_split_kernel(const AttnArgs A) {
    constexpr int NKK = D / 32;   // MFMA k-steps over the head dimension
    constexpr int DPL = D / 64;   // value dimensions per lane in P V
    static_assert(G >= 1 && G <= 16 && D % 64 == 0, "shape");
    __shared__ __attribute__((aligned(16))) bf8_t qfr[NKK * 2 * 64];  // query fragments hi, lo
    __shared__ float cs[2][D / 2];     // cos, sin of the rotary pairs at the row's position
    // rotated queries of the group, then (after the positions) the exchange
    // area of the wavefront merge: one buffer, the uses do not overlap
    __shared__ __attribute__((aligned(16))) float qx[2 * G * D];
    float (*qf)[D] = reinterpret_cast<float (*)[D]>(qx);              // [G][D]
    float (*xo)[G][D] = reinterpret_cast<float (*)[G][D]>(qx);        // [2][G][D]
    __shared__ float krf[D];           // rotated new key
    __shared__ float snew[G];          // scores of the new position
    __shared__ float pb[4][16][16];    // per wavefront: P of a 16-position block [pos][head]
    __shared__ float al[4][16];        // per wavefront: rescale factors of a block [head]
    __shared__ float xm[2][G], xl[2][G];  // merging the wavefronts
    // per wavefront: a block's value rows [16][VR] bf16 (VR = D + 16: padded
    // rows keep the transposed reads off common banks), then, after the
    // positions, its o [G][D] fp32 on the way to the merge's layout
    constexpr int VR = D + 16;
    constexpr int VXF = (16 * VR / 2 > G * D) ? 16 * VR / 2 : G * D;  // floats per wavefront
    __shared__ __attribute__((aligned(16))) float vx[4][VXF];
    constexpr int NT = D / 16;  // 16-dimension tiles of P V

    const int Hkv = A.Hkv;
    const int n = blockIdx.y / Hkv, kvh = blockIdx.y - n * Hkv;
    const int pe = __builtin_amdgcn_readfirstlane(A.pos[n]);  // position of the new token
    if (pe < 0 || pe >= A.Lmax) return;  // caller error: no cache access (o reads NaN)
    const int L = pe + 1;
    const int sp = A.split;
    const int t0 = blockIdx.x * sp;
    if (t0 >= L) return;  // this split lies past the row's length
    const int t1 = min(t0 + sp, L);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, lg = l >> 4;
    const int rd = A.rd, half = rd / 2;

    const size_t kvrow = (size_t)n * Hkv + kvh;
    const uint16_t* qrow = A.q + ((size_t)n * A.Hq + (size_t)kvh * G) * D;
    const uint16_t* knew = A.k_new + kvrow * D;
    const uint16_t* vnew = A.v_new + kvrow * D;
    // rotary angles p theta^(-2j/rd) in double: positions reach tens of
    // thousands, where a float angle would be off by ~1e-3 rad
    for (int j = tid; j < half; j += kAttnWG) {
        const double a = (double)pe * exp2(-2.0 * j / rd * log2((double)A.theta));
        double sd, cd;
        sincos(a, &sd, &cd);
        cs[0][j] = (float)cd;
        cs[1][j] = (float)sd;
    }
    __syncthreads();
    auto rot = [&](const uint16_t* x, int i) {  // element i of rope(x)
        const float xi = bf16_to_f32(x[i]);
        if (i >= rd) return xi;
        return i < half ? xi * cs[0][i] - bf16_to_f32(x[i + half]) * cs[1][i]
                        : xi * cs[0][i - half] + bf16_to_f32(x[i - half]) * cs[1][i - half];
    };
    for (int e = tid; e < G * D; e += kAttnWG) qf[e / D][e % D] = rot(qrow + (size_t)(e / D) * D, e % D);
    const bool last = t1 == L;  // this workgroup holds the new position
    if (last)
        for (int e = tid; e < D; e += kAttnWG) krf[e] = rot(knew, e);
    __syncthreads();
    if (last) {
        // append the new key and value to the caches; their rows are read by no
        // workgroup of this step (the others stop before row pe)
        uint16_t* kc = A.k_cache + (kvrow * A.Lmax + pe) * D;
        uint16_t* vc = A.v_cache + (kvrow * A.Lmax + pe) * D;
        for (int e = tid; e < D; e += kAttnWG) {
            kc[e] = f32_to_bf16(krf[e]);
            vc[e] = vnew[e];
        }
        // the new position's scores in fp32 (its key is not yet bf16 in the cache)
        for (int g = w; g < G; g += 4) {
            float s = 0.f;
            for (int e = l; e < D; e += 64) s += qf[g][e] * krf[e];
            s = group_sum<64>(s);
            if (l == 0) snew[g] = s * A.scale;
        }
    }
    // query fragments (row = head, zero past G; k = head dimension), split
    // into hi and lo, in lane order in LDS: the wavefronts share them
    for (int kk = w; kk < NKK; kk += 4) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = lr < G ? qf[lr][32 * kk + 8 * lg + j] : 0.f;
        bf8_t h, o;
        split8(x, h, o);
        qfr[(kk * 2 + 0) * 64 + l] = h;
        qfr[(kk * 2 + 1) * 64 + l] = o;
    }
    __syncthreads();

    // cached rows t < pe of this (row, kv head); rows past them read as zero
    const uint16_t* kbase = A.k_cache + kvrow * A.Lmax * D;
    const uint16_t* vbase = A.v_cache + kvrow * A.Lmax * D;
    const __amdgpu_buffer_rsrc_t kr = in_rsrc(kbase, (uint32_t)pe * D * 2);
    const __amdgpu_buffer_rsrc_t vr = in_rsrc(vbase, (uint32_t)pe * D * 2);

    float m[4], ls[4];  // running max and sum for heads 4 lg + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m[r] = -INFINITY;
        ls[r] = 0.f;
    }
    // o^T on MFMA: oacc[t][r] = o[head lr][dim 16 t + 4 lg + r] (unnormalised,
    // relative to m; lanes lr >= G hold padding heads)
    f4_t oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) oacc[t] = f4_t{0.f, 0.f, 0.f, 0.f};
    // the new position's value row, as the cache words of this lane's dims
    uint32_t vnw[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < DPL; ++j) vnw[j / 2] |= (uint32_t)vnew[DPL * l + j] << (16 * (j & 1));
    uint16_t* const vw = reinterpret_cast<uint16_t*>(vx[w]);
    typedef short v4s_t __attribute__((ext_vector_type(4)));

    const int nblk = (t1 - t0 + 15) / 16;
    // Blocks b = w, w + 4, ... of this wavefront, two in flight: the loads of
    // the next block are issued before the current one is computed.  Loads of
    // a block past the split read positions >= pe, which the buffer resources
    // return as zero (no access), so they are issued unconditionally and the
    // wait counts stay static.
    typedef uint32_t vraw_t[16][(DPL + 1) / 2];
    auto load_block = [&](int b, bf8_t* kf, vraw_t& vraw) {
        const int P0 = t0 + 16 * b;
        // key fragments of 16 positions and the 16 value rows, all in flight
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            kf[kk] = __builtin_bit_cast(bf8_t, __builtin_amdgcn_raw_buffer_load_b128(
                kr, (int)(((P0 + lr) * D + 32 * kk + 8 * lg) * 2), 0, kCacheNt));
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            const uint32_t off = (uint32_t)((P0 + p) * D + DPL * l) * 2;
            if constexpr (DPL == 4) {
                typedef unsigned u2_t __attribute__((ext_vector_type(2)));
                const u2_t u = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(vr, (int)off, 0, kCacheNt));
                vraw[p][0] = u.x;
                vraw[p][1] = u.y;
            } else if constexpr (DPL == 2) {
                vraw[p][0] = __builtin_amdgcn_raw_buffer_load_b32(vr, (int)off, 0, kCacheNt);
            } else {
                vraw[p][0] = __builtin_amdgcn_raw_buffer_load_b16(vr, (int)off, 0, kCacheNt);
            }
        }
    };
    auto compute_block = [&](int b, const bf8_t* kf, const vraw_t& vraw) {
        const int P0 = t0 + 16 * b;
        f4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            sc = mfma(qfr[(kk * 2 + 0) * 64 + l], kf[kk], sc);
            sc = mfma(qfr[(kk * 2 + 1) * 64 + l], kf[kk], sc);
        }
        // sc[r] = score of head 4 lg + r at position P0 + lr
        const int t = P0 + lr;
        float pr[4], alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int g = 4 * lg + r;
            float s = sc[r] * A.scale;
            if (t == pe) s = (g < G) ? snew[g] : 0.f;
            if (t >= L) s = -INFINITY;
            float bm = s;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) bm = fmaxf(bm, __shfl_xor(bm, o, 64));
            const float mn = fmaxf(m[r], bm);
            alpha[r] = expf(m[r] - mn);  // 0 while m is -inf
            pr[r] = expf(s - mn);
            float ps = pr[r];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o, 64);
            ls[r] = ls[r] * alpha[r] + ps;
            m[r] = mn;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[w][lr][4 * lg + r] = pr[r];
        if (lr == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) al[w][4 * lg + r] = alpha[r];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // the block's value rows into this wavefront's area (the new
        // position's row from v_new; rows past pe read as zero)
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            uint32_t w0 = vraw[p][0], w1 = DPL == 4 ? vraw[p][DPL == 4 ? 1 : 0] : 0u;
            if (P0 + p == pe) {
                w0 = vnw[0];
                w1 = vnw[1];
            }
            if constexpr (DPL == 4)
                *reinterpret_cast<uint2*>(&vw[p * VR + 4 * l]) = make_uint2(w0, w1);
            else if constexpr (DPL == 2)
                *reinterpret_cast<uint32_t*>(&vw[p * VR + 2 * l]) = w0;
            else
                vw[p * VR + l] = (uint16_t)w0;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // rescale by the head's factor, then o^T += V^T P^T per tile: the B
        // operand is P^T (column head lr, positions 4 lg ..), split hi / lo;
        // the A operand V^T (row dim 16 t + lr, positions 4 lg ..) comes from
        // a transpose read, lane c of each 16-lane group pointing at row
        // 4 lg + c / 4, dims 16 t + 4 (c % 4) ..
        const float ah = al[w][lr];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[t][r] *= ah;
        float pf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pf[i] = pb[w][4 * lg + i][lr];
        uint2 phu, plu;
        split4(pf, phu, plu);
        const v4s_t ph = __builtin_bit_cast(v4s_t, phu), pl = __builtin_bit_cast(v4s_t, plu);
        const uint16_t* const vt = &vw[(4 * lg + (lr >> 2)) * VR + 4 * (lr & 3)];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const v4s_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t*)(vt + 16 * t));
            oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, oacc[t], 0, 0, 0);
            oacc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, oacc[t], 0, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();  // pb and al are rewritten by the next block
    };
    bf8_t kfa[NKK], kfb[NKK];
    vraw_t va, vb;
    load_block(w, kfa, va);
    for (int b = w; b < nblk; b += 8) {
        load_block(b + 4, kfb, vb);
        compute_block(b, kfa, va);
        load_block(b + 8, kfa, va);
        if (b + 4 < nblk) compute_block(b + 4, kfb, vb);
    }

    // o back to the merge's layout, acc[g][j] = o[head g][dim DPL l + j],
    // through this wavefront's area (its last block's reads are done: LDS
    // operations of one wavefront complete in order)
    float* const xw = vx[w];
    if (lr < G) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) xw[lr * D + 16 * t + 4 * lg + r] = oacc[t][r];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float acc[G][DPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[g][j] = xw[g * D + DPL * l + j];

    // merge the four wavefronts through LDS in two rounds (3 -> 1, 2 -> 0,
    // then 1 -> 0); a wavefront without positions holds m = -inf
    float mg[G], lsg[G];  // m and the sum of head g, for this lane's heads
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mg[g] = __shfl(m[g & 3], 16 * (g >> 2), 64);
        lsg[g] = __shfl(ls[g & 3], 16 * (g >> 2), 64);
    }
    auto put = [&](int slot) {
        if (l == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                xm[slot][g] = mg[g];
                xl[slot][g] = lsg[g];
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < DPL; ++j) xo[slot][g][DPL * l + j] = acc[g][j];
    };
    auto take = [&](int slot) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float m2 = xm[slot][g];
            const float mn = fmaxf(mg[g], m2);
            const float a1 = mg[g] == -INFINITY ? 0.f : expf(mg[g] - mn);
            const float a2 = m2 == -INFINITY ? 0.f : expf(m2 - mn);
            lsg[g] = lsg[g] * a1 + xl[slot][g] * a2;
#pragma unroll
            for (int j = 0; j < DPL; ++j) acc[g][j] = acc[g][j] * a1 + xo[slot][g][DPL * l + j] * a2;
            mg[g] = mn;
        }
    };
    if (w >= 2) put(w - 2);
    __syncthreads();
    if (w < 2) take(w);
    __syncthreads();
    if (w == 1) put(0);
    __syncthreads();
    if (w == 0) {
        take(0);
        float* part = A.part + ((kvrow * A.nsplit + blockIdx.x) * G) * (D + 2);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < DPL; ++j) part[g * (D + 2) + DPL * l + j] = acc[g][j];
        if (l < G) {
            float mm = mg[0], ll = lsg[0];
#pragma unroll
            for (int g = 1; g < G; ++g)
                if (l == g) {
                    mm = mg[g];
                    ll = lsg[g];
                }
            part[l * (D + 2) + D] = mm;
            part[l * (D + 2) + D + 1] = ll;
        }
    }
}

// Merge the partial results of one (row, query head), apply the gate, store
// o.  The maximum and the softmax denominator are block reductions over the
// partials; for the weighted sum, four groups of 64 threads take every fourth
// partial, each lane D/64 consecutive dimensions (one load per partial), and
// the groups are added through LDS.
template <int D, int G, typename Tout>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs A) {
    constexpr int DPT = D / 64;  // dimensions per lane
    __shared__ float red[256];
    __shared__ float sum4[4][D];
    const int n = blockIdx.x / A.Hq, h = blockIdx.x - n * A.Hq;
    const int kvh = h / G, g = h - kvh * G;
    const int tid = threadIdx.x, grp = tid >> 6, lane = tid & 63;
    const int pe = A.pos[n];
    Tout* o = static_cast<Tout*>(A.o) + ((size_t)n * A.Hq + h) * D;
    if (pe < 0 || pe >= A.Lmax) {  // caller error, reported as NaN outputs
        for (int d = tid; d < D; d += 256) io<Tout>::st(o + d, __builtin_nanf(""));
        return;
    }
    const int ns = (pe + A.split) / A.split;  // partials of the live splits
    const float* part = A.part + (((size_t)n * A.Hkv + kvh) * A.nsplit * G + g) * (D + 2);
    const size_t stride = (size_t)G * (D + 2);
    auto block_reduce = [&](float x, bool is_max) {
        red[tid] = x;
        __syncthreads();
        for (int off = 128; off > 0; off >>= 1) {
            if (tid < off) red[tid] = is_max ? fmaxf(red[tid], red[tid + off]) : red[tid] + red[tid + off];
            __syncthreads();
        }
        const float r = red[0];
        __syncthreads();
        return r;
    };
    float mx = -INFINITY;
    for (int s = tid; s < ns; s += 256) mx = fmaxf(mx, part[s * stride + D]);
    const float M = block_reduce(mx, true);
    float dn = 0.f;
    for (int s = tid; s < ns; s += 256) {
        const float ms = part[s * stride + D];
        if (ms != -INFINITY) dn += part[s * stride + D + 1] * expf(ms - M);
    }
    const float inv = 1.0f / block_reduce(dn, false);
    float acc[DPT] = {};
#pragma unroll 4
    for (int s = grp; s < ns; s += 4) {
        const float* ps = part + (size_t)s * stride;
        const float ms = ps[D];
        const float wgt = ms != -INFINITY ? expf(ms - M) : 0.f;
#pragma unroll
        for (int j = 0; j < DPT; ++j) acc[j] += wgt * ps[DPT * lane + j];
    }
#pragma unroll
    for (int j = 0; j < DPT; ++j) sum4[grp][DPT * lane + j] = acc[j];
    __syncthreads();
    for (int d = tid; d < D; d += 256) {
        float v = (sum4[0][d] + sum4[1][d] + sum4[2][d] + sum4[3][d]) * inv;
        if (A.gate) v *= 1.0f / (1.0f + expf(-bf16_to_f32(A.gate[((size_t)n * A.Hq + h) * D + d])));
        io<Tout>::st(o + d, v);
    }
}

template <int D, int G>
static hipError_t launch_attn_g(const AttnArgs& A) {
    hipLaunchKernelGGL((attn_split_kernel<D, G>), dim3(A.nsplit, A.N * A.Hkv), dim3(kAttnWG), 0,
                       A.stream, A);
    if (A.o_bf16)
        hipLaunchKernelGGL((attn_combine_kernel<D, G, bf16_t>), dim3(A.N * A.Hq), dim3(256), 0,
                           A.stream, A);
    else
        hipLaunchKernelGGL((attn_combine_kernel<D, G, float>), dim3(A.N * A.Hq), dim3(256), 0,
                           A.stream, A);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_attn_d(const AttnArgs& A) {
    switch (A.Hq / A.Hkv) {
        case 1: return launch_attn_g<D, 1>(A);
        case 2: return launch_attn_g<D, 2>(A);
        case 4: return launch_attn_g<D, 4>(A);
        case 8: return launch_attn_g<D, 8>(A);
        default: return launch_attn_g<D, 16>(A);
    }
}

hipError_t launch_attn_decode(const AttnArgs& A) {
    switch (A.D) {
        case 64: return launch_attn_d<64>(A);
        case 128: return launch_attn_d<128>(A);
        default: return launch_attn_d<256>(A);
    }
}

}  // namespace gdn

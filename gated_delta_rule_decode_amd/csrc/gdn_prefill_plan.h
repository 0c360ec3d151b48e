// gdn_prefill_plan.h -- the segment planner of the chunked prefill (gfx950):
// the chunk table of a packed batch, the choice of a segment length for the
// segment-parallel scan and the work lists of its combine and correction
// passes, run by one 256-thread workgroup.  Used by the planner kernel and by
// the d_k = 128 prep kernel, one of whose workgroups plans for small batches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"
#include "gdn_prefill_common.h"

namespace gdn {

// Exclusive prefix sum of count(i) over i < n; emit(i, position, count) is
// called once for every i.  Returns the total.  All 256 threads take part.
template <typename F, typename G>
__device__ inline int block_exclusive_scan(int n, F count, G emit, int* buf) {
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

// One workgroup of 256 threads: the chunk table (chunk_off, the first global
// chunk of every sequence), then the choice of the segment length, the
// segments of every sequence and the work lists of the combine and
// correction passes.  plan = {segments, correction items, segment length (0:
// none), sequences with more than one segment}.  Chunk counts of the first
// `cache` sequences stay in LDS.  The LDS comes from the caller: ibuf 256
// ints, cnt_sh and off_sh `cache` ints each, acc 3 x kNCand floats (items,
// chain steps, tokens of later segments), sc 2 ints.
__device__ inline void plan_segments(const PrefillArgs& A, int TV, int TK, int tp, int* ibuf, int* cnt_sh,
                              int* off_sh, int cache, float* acc_, int* sc) {
    const int kPlanCache = cache;
    float (*acc)[kNCand] = reinterpret_cast<float (*)[kNCand]>(acc_);
    int& s_cmax = sc[0];
    int& s_len = sc[1];
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

}  // namespace gdn

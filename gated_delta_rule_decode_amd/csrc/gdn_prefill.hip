// gdn_prefill.hip -- chunked (WY / UT-transform) prefill of the gated delta rule.
//
// Within a chunk of C = 64 tokens of one sequence and value head, with
// in-chunk cumulative log-decays G_t = g_1 + ... + g_t and gamma_t = e^{G_t},
// unrolling S_t = a_t S_{t-1} + u_t k_t^T, u_t = b_t (v_t - a_t S_{t-1} k_t),
// from the chunk's initial state S gives
//
//     (I + A) U = diag(b) V - diag(b gamma) K S^T,  A_ts = b_t e^{G_t-G_s} k_t.k_s (s < t)
//     O   = scale (diag(gamma) Q S^T + (tril(Q K^T) o e^{G_t-G_s}) U)
//     S'  = gamma_n S + U^T diag(e^{G_n - G}) K
//
// (the gated delta rule of Yang et al., ICLR 2025, in its chunkwise form).
// Decay factors are only ever formed as e^{G_t - G_s} with s <= t, never as a
// product e^{G_t} e^{-G_s}, so nothing overflows however fast the decay.
//
// Three kernels, all enqueued on the caller's stream:
//   chunk_table  cu_seqlens -> first chunk index of every sequence (chunks
//                restart at every sequence start; the last may be partial)
//   prep         one workgroup per (chunk, value head), chunk-parallel:
//                G, A, T = (I + A)^-1 by forward substitution, stores
//                T diag(b) and G in the workspace
//   scan         one workgroup per (sequence, value head, tile of BV state
//                rows), sequential over the sequence's chunks: keeps its
//                state tile on chip, forms U = T diag(b) (V - diag(gamma) K S^T),
//                writes O and advances S
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// Sequence bounds clamped into [0, T] so that a malformed cu_seqlens can
// produce wrong values but never an out-of-range access.
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int n, int T, int& s, int& e) {
    int a = cu[n], b = cu[n + 1];
    a = min(max(a, 0), T);
    b = min(max(b, a), T);
    s = a;
    e = b;
}

__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t* __restrict__ cu, int N,
                                                          int T, int32_t* __restrict__ chunk_off) {
    __shared__ int buf[256];
    int carry = 0;
    for (int base = 0; base < N; base += 256) {
        const int i = base + threadIdx.x;
        int cnt = 0;
        if (i < N) {
            int s, e;
            seq_bounds(cu, i, T, s, e);
            cnt = (e - s + kChunk - 1) / kChunk;
        }
        buf[threadIdx.x] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int add = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
            __syncthreads();
            buf[threadIdx.x] += add;
            __syncthreads();
        }
        if (i < N) chunk_off[i] = carry + buf[threadIdx.x] - cnt;
        carry += buf[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) chunk_off[N] = carry;
}

// Locate chunk c: sequence n with chunk_off[n] <= c < chunk_off[n+1].
__device__ __forceinline__ int find_seq(const int32_t* chunk_off, int N, int c) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= c) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <int DK, typename Tin>
__global__ __launch_bounds__(256) void prep_kernel(const Tin* __restrict__ k,
                                                   const float* __restrict__ g,
                                                   const float* __restrict__ beta,
                                                   const int32_t* __restrict__ cu,
                                                   const int32_t* __restrict__ chunk_off, int N,
                                                   int T, int H, int HV, int max_chunks,
                                                   float* __restrict__ wsT,
                                                   float* __restrict__ wsG) {
    constexpr int C = kChunk;
    __shared__ float Ks[C][DK + 1];
    __shared__ float Am[C][C + 1];
    __shared__ float Tm[C][C + 1];
    __shared__ float Gs[C], Bs[C];
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int total = min(chunk_off[N], max_chunks);
    if (c >= total) return;
    const int n = find_seq(chunk_off, N, c);
    int s, e;
    seq_bounds(cu, n, T, s, e);
    const int t0 = s + (c - chunk_off[n]) * C;
    const int L = min(C, e - t0);
    const int hk = h / (HV / H);

    for (int idx = tid; idx < C * (DK / 4); idx += 256) {
        const int t = idx / (DK / 4), c4 = 4 * (idx % (DK / 4));
        f4 val = {0.f, 0.f, 0.f, 0.f};
        if (t < L) val = io<Tin>::ld4(k + ((size_t)(t0 + t) * H + hk) * DK + c4);
        Ks[t][c4] = val.x;
        Ks[t][c4 + 1] = val.y;
        Ks[t][c4 + 2] = val.z;
        Ks[t][c4 + 3] = val.w;
    }
    if (tid < C) {
        Gs[tid] = tid < L ? g[(size_t)(t0 + tid) * HV + h] : 0.f;
        Bs[tid] = tid < L ? beta[(size_t)(t0 + tid) * HV + h] : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
        float acc = 0.f;
        for (int t = 0; t < C; ++t) {
            acc += Gs[t];
            Gs[t] = acc;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += 256) {
        const int t = idx / C, j = idx % C;
        float val = 0.f;
        if (j < t) {
            float d = 0.f;
#pragma unroll 8
            for (int x = 0; x < DK; ++x) d += Ks[t][x] * Ks[j][x];
            val = Bs[t] * expf(Gs[t] - Gs[j]) * d;
        }
        Am[t][j] = val;
    }
    __syncthreads();
    // T = (I + A)^-1: T[t][j] = [t == j] - sum_{j <= x < t} A[t][x] T[x][j]
    for (int t = 0; t < C; ++t) {
        if (tid < C) {
            const int j = tid;
            float val = (j == t) ? 1.f : 0.f;
            for (int x = j; x < t; ++x) val -= Am[t][x] * Tm[x][j];
            Tm[t][j] = val;
        }
        __syncthreads();
    }
    float* To = wsT + ((size_t)c * HV + h) * C * C;
    for (int idx = tid; idx < C * C; idx += 256) {
        const int t = idx / C, j = idx % C;
        To[idx] = (j <= t) ? Tm[t][j] * Bs[j] : 0.f;
    }
    if (tid < C) wsG[((size_t)c * HV + h) * C + tid] = Gs[tid];
}

template <int DK, int BV, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void scan_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, int N, int T, int H,
    int HV, int dv, int max_chunks, const float* __restrict__ wsT, const float* __restrict__ wsG,
    const float* s0, float* sfin, Tout* __restrict__ o, float scale) {
    constexpr int C = kChunk;
    constexpr int E = C * BV / 256;  // (t, i) entries per thread
    static_assert(E >= 1 && (BV * DK) % 256 == 0, "tile");
    __shared__ float Ss[BV][DK + 1];
    __shared__ float Ks[C][DK + 1];
    __shared__ float Qs[C][DK + 1];
    __shared__ float Tm[C][C + 1];
    __shared__ float Pm[C][C + 1];
    __shared__ float Xs[C][BV + 1];
    __shared__ float Us[C][BV + 1];
    __shared__ float Gs[C], Ws[C];

    const int tid = threadIdx.x;
    const int tiles = dv / BV;
    const int tile = blockIdx.x % tiles;
    const int nh = blockIdx.x / tiles;
    const int n = nh / HV, h = nh - n * HV;
    const int hk = h / (HV / H);
    const size_t sbase = ((size_t)nh * dv + (size_t)tile * BV) * DK;

    for (int idx = tid; idx < BV * DK; idx += 256) {
        const int i = idx / DK, j = idx % DK;
        Ss[i][j] = s0 ? s0[sbase + idx] : 0.f;
    }
    int s, e;
    seq_bounds(cu, n, T, s, e);
    const int nch = chunk_off[n + 1] - chunk_off[n];
    for (int jc = 0; jc < nch; ++jc) {
        const int c = chunk_off[n] + jc;
        if (c >= max_chunks) break;
        const int t0 = s + jc * C;
        const int L = min(C, e - t0);
        __syncthreads();
        for (int idx = tid; idx < C * (DK / 4); idx += 256) {
            const int t = idx / (DK / 4), c4 = 4 * (idx % (DK / 4));
            f4 kv = {0.f, 0.f, 0.f, 0.f}, qv = {0.f, 0.f, 0.f, 0.f};
            if (t < L) {
                const size_t off = ((size_t)(t0 + t) * H + hk) * DK + c4;
                kv = io<Tin>::ld4(k + off);
                qv = io<Tin>::ld4(q + off);
            }
            Ks[t][c4] = kv.x; Ks[t][c4 + 1] = kv.y; Ks[t][c4 + 2] = kv.z; Ks[t][c4 + 3] = kv.w;
            Qs[t][c4] = qv.x; Qs[t][c4 + 1] = qv.y; Qs[t][c4 + 2] = qv.z; Qs[t][c4 + 3] = qv.w;
        }
        for (int idx = tid; idx < C * BV; idx += 256) {
            const int t = idx / BV, i = idx % BV;
            Xs[t][i] = t < L ? io<Tin>::ld(v + ((size_t)(t0 + t) * HV + h) * dv + tile * BV + i) : 0.f;
        }
        const float* Tp = wsT + ((size_t)c * HV + h) * C * C;
        for (int idx = tid; idx < C * C; idx += 256) Tm[idx / C][idx % C] = Tp[idx];
        if (tid < C) Gs[tid] = wsG[((size_t)c * HV + h) * C + tid];
        __syncthreads();
        const float glast = Gs[L - 1];
        if (tid < C) Ws[tid] = tid < L ? expf(glast - Gs[tid]) : 0.f;
        // P = tril(Q K^T) o e^{G_t - G_j}
        for (int idx = tid; idx < C * C; idx += 256) {
            const int t = idx / C, j = idx % C;
            float val = 0.f;
            if (j <= t) {
                float d = 0.f;
#pragma unroll 8
                for (int x = 0; x < DK; ++x) d += Qs[t][x] * Ks[j][x];
                val = d * expf(Gs[t] - Gs[j]);
            }
            Pm[t][j] = val;
        }
        // K S^T and Q S^T; X = V - diag(gamma) K S^T
        float qs[E];
#pragma unroll
        for (int ee = 0; ee < E; ++ee) {
            const int idx = tid + 256 * ee;
            const int t = idx / BV, i = idx % BV;
            float ks = 0.f, qv = 0.f;
#pragma unroll 8
            for (int x = 0; x < DK; ++x) {
                ks += Ks[t][x] * Ss[i][x];
                qv += Qs[t][x] * Ss[i][x];
            }
            qs[ee] = qv;
            Xs[t][i] -= expf(Gs[t]) * ks;
        }
        __syncthreads();
        // U = T diag(b) X
#pragma unroll
        for (int ee = 0; ee < E; ++ee) {
            const int idx = tid + 256 * ee;
            const int t = idx / BV, i = idx % BV;
            float u = 0.f;
            for (int j = 0; j <= t; ++j) u += Tm[t][j] * Xs[j][i];
            Us[t][i] = u;
        }
        __syncthreads();
        // O = scale (diag(gamma) Q S^T + P U)
#pragma unroll
        for (int ee = 0; ee < E; ++ee) {
            const int idx = tid + 256 * ee;
            const int t = idx / BV, i = idx % BV;
            float acc = expf(Gs[t]) * qs[ee];
            for (int j = 0; j <= t; ++j) acc += Pm[t][j] * Us[j][i];
            if (t < L) io<Tout>::st(o + ((size_t)(t0 + t) * HV + h) * dv + tile * BV + i, scale * acc);
        }
        // S' = gamma_n S + U^T diag(e^{G_n - G}) K
        const float gn = expf(glast);
#pragma unroll 1
        for (int idx = tid; idx < BV * DK; idx += 256) {
            const int i = idx / DK, j = idx % DK;
            float acc = gn * Ss[i][j];
            for (int t = 0; t < L; ++t) acc += Ws[t] * Us[t][i] * Ks[t][j];
            Ss[i][j] = acc;
        }
    }
    __syncthreads();
    if (sfin) {
        for (int idx = tid; idx < BV * DK; idx += 256) sfin[sbase + idx] = Ss[idx / DK][idx % DK];
    }
}

__global__ void state_copy_kernel(const float* src, float* dst, size_t count) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_state_copy(const float* src, float* dst, size_t count, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    size_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst,
                       count);
    return hipGetLastError();
}

template <int DK, int BV, typename Tin, typename Tout>
static hipError_t launch_prefill_t(const PrefillArgs& A) {
    hipLaunchKernelGGL((prep_kernel<DK, Tin>), dim3(A.max_chunks, A.HV), dim3(256), 0, A.stream,
                       static_cast<const Tin*>(A.k), A.g, A.beta, A.cu_seqlens, A.chunk_off, A.N,
                       A.T, A.H, A.HV, A.max_chunks, A.ws_T, A.ws_G);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int tiles = A.dv / BV;
    hipLaunchKernelGGL((scan_kernel<DK, BV, Tin, Tout>), dim3((unsigned)(A.N * A.HV * tiles)),
                       dim3(256), 0, A.stream, static_cast<const Tin*>(A.q),
                       static_cast<const Tin*>(A.k), static_cast<const Tin*>(A.v), A.cu_seqlens,
                       A.chunk_off, A.N, A.T, A.H, A.HV, A.dv, A.max_chunks, A.ws_T, A.ws_G, A.s0,
                       A.s_final, static_cast<Tout*>(A.o), A.scale);
    return hipGetLastError();
}

template <int DK, typename Tin, typename Tout>
static hipError_t launch_prefill_dk(const PrefillArgs& A) {
    if (A.dv == 16) return launch_prefill_t<DK, 16, Tin, Tout>(A);
    return launch_prefill_t<DK, 32, Tin, Tout>(A);
}

template <typename Tin, typename Tout>
static hipError_t launch_prefill_io(const PrefillArgs& A) {
    switch (A.dk) {
        case 16: return launch_prefill_dk<16, Tin, Tout>(A);
        case 32: return launch_prefill_dk<32, Tin, Tout>(A);
        case 64: return launch_prefill_dk<64, Tin, Tout>(A);
        default: return launch_prefill_dk<128, Tin, Tout>(A);
    }
}

// The bf16-MFMA kernels where they apply (bf16 inputs, d_k in {64, 128}, d_v
// a multiple of 32); otherwise the chunk table and the fp32 vector-unit
// kernels above (every other supported shape, fp32 inputs).
hipError_t launch_prefill(const PrefillArgs& A) {
    if (prefill_mfma_eligible(A)) return launch_prefill_mfma(A);  // builds its own chunk table
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, A.stream, A.cu_seqlens, A.N,
                       A.T, A.chunk_off);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (A.in_bf16) {
        return A.o_bf16 ? launch_prefill_io<bf16_t, bf16_t>(A) : launch_prefill_io<bf16_t, float>(A);
    }
    return A.o_bf16 ? launch_prefill_io<float, bf16_t>(A) : launch_prefill_io<float, float>(A);
}

}  // namespace gdn

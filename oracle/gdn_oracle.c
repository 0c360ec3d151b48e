/*
 * gdn_oracle.c -- plain, slow fp64 CPU oracle for the Gated DeltaNet token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may call,
 * link or load this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code with the HIP kernels.
 *
 * What it computes.  The pages name the mixer without writing it out: the
 * Qwen3.5-0.8B chat guide (soniqo.audio, section "Architektur") describes the
 * DeltaNet layers as linear attention with a gated-delta-rule recurrence
 * followed by RMSNormGated; the Qwen3.6 card of the Core AI model zoo (intro)
 * gives the grouped value heads (each key/query head shared by two value
 * heads); the Swiftlet post (section "How It Works") stresses the fixed-size
 * recurrent state.  The recurrence used here is the published gated delta rule
 * (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025):
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T ,   o_t = S_t q_t
 *
 * with S_t a d_v x d_k matrix (row i <-> value dim, column j <-> key dim),
 * a_t = exp(g_t) the decay and b_t = beta_t the write strength, both per
 * (token, value head).  The readout uses the state AFTER the token's update
 * and is multiplied by `scale`.  Value head h reads key/query head h / (HV/H).
 *
 * RMSNormGated, per (token, value head) group of d_v values:
 *     y = x / sqrt(mean(x^2) + eps) * w * silu(z),   silu(z) = z / (1 + e^-z)
 *
 * The serving form of the decode step (gdn_oracle_decode_layer) adds the
 * layer's gate activations, an optional L2 normalisation of q and k and a slot
 * table into a pool of states; gdn_oracle_attn_decode is one decode step of
 * the decoder's other token mixer, gated full attention; see the comments at
 * those functions.
 *
 * Everything is computed in double from float32 inputs (bf16 inputs arrive as
 * exactly representable float32 values).  No chunking and no reordering beyond
 * the plain loops below; the (sequence, head) recurrences are independent and
 * run in parallel with OpenMP.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdn_oracle_version(void) { return 3; }

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One token of the rule for one (sequence, value head):
 *     S <- a S (I - b k k^T) + b v k^T,      o = scale * S q
 * with the readout taken from the state after the update.
 *   qt, kt : [dk] double      vt : [dv] float32
 *   S      : [dv, dk]         ot : [dv]        sk : [dv] scratch
 */
static void step_one(const double* qt, const double* kt, const float* vt, double a, double b,
                     int dk, int dv, double scale, double* S, double* ot, double* sk) {
    /* sk = S_{t-1} k_t */
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * kt[j];
        sk[i] = acc;
    }
    /* S_t = a S_{t-1} - a b (S_{t-1} k_t) k_t^T + b v_t k_t^T */
    for (int i = 0; i < dv; ++i) {
        for (int j = 0; j < dk; ++j) {
            double s = S[(size_t)i * dk + j];
            double upd = a * s;
            upd -= a * b * sk[i] * kt[j];
            upd += b * (double)vt[i] * kt[j];
            S[(size_t)i * dk + j] = upd;
        }
    }
    /* o_t = scale * S_t q_t */
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * qt[j];
        ot[i] = scale * acc;
    }
}

/*
 * One (sequence n, value head h) recurrence over tokens t0 .. t1-1.
 *   q, k  : [T, H, dk]     float32, token-major
 *   v     : [T, HV, dv]
 *   g, bt : [T, HV]        log-decay and beta
 *   S     : [dv, dk]       in: initial state, out: final state (double)
 *   o     : [T, HV, dv]    outputs for this head's rows (double)
 *   wk    : scratch of dv + 2 dk doubles
 */
static void recur_one(const float* q, const float* k, const float* v, const float* g,
                      const float* bt, long t0, long t1, int H, int HV, int dk, int dv,
                      int h, double scale, double* S, double* o, double* wk) {
    const int hk = h / (HV / H);          /* grouped value heads: key head of h */
    double* qd = wk + dv;
    double* kd = qd + dk;
    for (long t = t0; t < t1; ++t) {
        const float* kt = k + ((size_t)t * H + hk) * dk;
        const float* qt = q + ((size_t)t * H + hk) * dk;
        const float* vt = v + ((size_t)t * HV + h) * dv;
        for (int j = 0; j < dk; ++j) {
            qd[j] = (double)qt[j];
            kd[j] = (double)kt[j];
        }
        const double a = exp((double)g[(size_t)t * HV + h]);
        const double b = (double)bt[(size_t)t * HV + h];
        step_one(qd, kd, vt, a, b, dk, dv, scale, S, o + ((size_t)t * HV + h) * dv, wk);
    }
}

/*
 * The whole packed batch.
 *   cu_seqlens : [N+1] int32, sequence n holds tokens cu[n] .. cu[n+1]-1
 *   s0         : [N, HV, dv, dk] double, or NULL for zero initial states
 *   o          : [T, HV, dv] double (written for every token)
 *   s_final    : [N, HV, dv, dk] double, or NULL
 *   nthreads   : OpenMP threads (<= 0: the runtime's default)
 * Returns 0, or -1 on invalid sizes or a failed allocation.
 */
int gdn_oracle_recurrence(const float* q, const float* k, const float* v, const float* g,
                          const float* beta, const int32_t* cu_seqlens, int N, int H, int HV,
                          int dk, int dv, double scale, const double* s0, double* o,
                          double* s_final, int nthreads) {
    if (N < 0 || H <= 0 || HV <= 0 || HV % H != 0 || dk <= 0 || dv <= 0) return -1;
    const long pairs = (long)N * HV;
    const size_t ssz = (size_t)dv * dk;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
    for (long p = 0; p < pairs; ++p) {
        const int n = (int)(p / HV), h = (int)(p % HV);
        double* S = (double*)malloc(ssz * sizeof(double));
        double* sk = (double*)malloc((size_t)(dv + 2 * dk) * sizeof(double));
        if (!S || !sk) {
            failed = 1;
        } else {
            if (s0)
                memcpy(S, s0 + (size_t)p * ssz, ssz * sizeof(double));
            else
                memset(S, 0, ssz * sizeof(double));
            recur_one(q, k, v, g, beta, cu_seqlens[n], cu_seqlens[n + 1], H, HV, dk, dv, h,
                      scale, S, o, sk);
            if (s_final) memcpy(s_final + (size_t)p * ssz, S, ssz * sizeof(double));
        }
        free(S);
        free(sk);
    }
    return failed ? -1 : 0;
}

/*
 * RMSNormGated over groups of dv values.
 *   x : [groups, dv] double      z : [groups, dv] float32     w : [dv] float32
 *   y : [groups, dv] double
 * y = x / sqrt(mean(x^2) + eps) * w * z * sigmoid(z)
 */
int gdn_oracle_rmsnorm_gated(const double* x, const float* z, const float* w, long groups,
                             int dv, double eps, double* y) {
    if (groups < 0 || dv <= 0) return -1;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (long r = 0; r < groups; ++r) {
        const double* xr = x + (size_t)r * dv;
        const float* zr = z + (size_t)r * dv;
        double ss = 0.0;
        for (int i = 0; i < dv; ++i) ss += xr[i] * xr[i];
        const double inv = 1.0 / sqrt(ss / dv + eps);
        for (int i = 0; i < dv; ++i) {
            const double zi = (double)zr[i];
            const double gate = zi / (1.0 + exp(-zi));
            y[(size_t)r * dv + i] = xr[i] * inv * (double)w[i] * gate;
        }
    }
    return 0;
}

/*
 * Gate activations of the decode layer.  The pages name the gated delta rule
 * and its per-(token, value head) decay and write strength but not how the
 * layer produces them; this follows the published Gated DeltaNet layer
 * (Yang et al., ICLR 2025), as used by the Qwen3.5 DeltaNet layers:
 *     g    = -exp(A_log[h]) * softplus(a_raw[n, h] + dt_bias[h])    (log-decay)
 *     beta = sigmoid(b_raw[n, h])
 * softplus(x) = log(1 + e^x), written as max(x, 0) + log1p(e^-|x|), which is
 * the same number without overflow; sigmoid(x) = 1 / (1 + e^-x).
 *   a_raw, b_raw : [N, HV] float32    A_log : [HV]    dt_bias : [HV] or NULL (zeros)
 *   g, beta      : [N, HV] double
 */
static double softplus_d(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

int gdn_oracle_gates(const float* a_raw, const float* b_raw, const float* A_log,
                     const float* dt_bias, long N, int HV, double* g, double* beta) {
    if (N < 0 || HV <= 0) return -1;
    for (long n = 0; n < N; ++n) {
        for (int h = 0; h < HV; ++h) {
            const size_t i = (size_t)n * HV + h;
            const double x = (double)a_raw[i] + (dt_bias ? (double)dt_bias[h] : 0.0);
            g[i] = -exp((double)A_log[h]) * softplus_d(x);
            beta[i] = 1.0 / (1.0 + exp(-(double)b_raw[i]));
        }
    }
    return 0;
}

/* x <- x / sqrt(sum_j x_j^2 + eps) over d values. */
static void l2norm_row(double* x, int d, double eps) {
    double ss = 0.0;
    for (int j = 0; j < d; ++j) ss += x[j] * x[j];
    const double inv = 1.0 / sqrt(ss + eps);
    for (int j = 0; j < d; ++j) x[j] *= inv;
}

/*
 * Per-row L2 normalisation (the optional q/k normalisation of the decode layer):
 *   x : [rows, d] float32      y : [rows, d] double,  y = x / sqrt(sum x^2 + eps)
 */
int gdn_oracle_l2norm(const float* x, long rows, int d, double eps, double* y) {
    if (rows < 0 || d <= 0) return -1;
    for (long r = 0; r < rows; ++r) {
        for (int j = 0; j < d; ++j) y[(size_t)r * d + j] = (double)x[(size_t)r * d + j];
        l2norm_row(y + (size_t)r * d, d, eps);
    }
    return 0;
}

/*
 * Serving form of the decode step: one token per sequence against a pool of
 * states addressed through a slot table (the pages' decoder owns all recurrent
 * state and advances one token per call: Qwen3.5-0.8B Core ML card, "Model").
 *   q, k   : [N, H, dk] float32     v : [N, HV, dv] float32
 *   g, beta: [N, HV] double (log-decay and write strength, e.g. from gdn_oracle_gates)
 *   slots  : [N] int32 or NULL (sequence n uses slot n); a slot outside
 *            [0, num_slots) skips the sequence: its outputs are 0 and no state changes
 *   l2norm : nonzero -> q and k are divided by sqrt(sum of squares + l2_eps) first
 *   pool   : [num_slots, HV, dv, dk] double, advanced in place
 *   o      : [N, HV, dv] double
 * Returns 0, or -1 on invalid sizes, a slot used twice, or a failed allocation.
 */
int gdn_oracle_decode_layer(const float* q, const float* k, const float* v, const double* g,
                            const double* beta, const int32_t* slots, int num_slots, int N,
                            int H, int HV, int dk, int dv, double scale, int l2norm,
                            double l2_eps, double* pool, double* o, int nthreads) {
    if (N < 0 || num_slots < 0 || H <= 0 || HV <= 0 || HV % H != 0 || dk <= 0 || dv <= 0)
        return -1;
    if (!slots && num_slots < N) return -1;
    unsigned char* used = (unsigned char*)calloc((size_t)num_slots + 1, 1);
    if (!used) return -1;
    int failed = 0;
    for (int n = 0; n < N && !failed; ++n) {
        const int32_t s = slots ? slots[n] : n;
        if (s < 0 || s >= num_slots) continue;
        if (used[s]) failed = 1;
        used[s] = 1;
    }
    free(used);
    if (failed) return -1;
    const long pairs = (long)N * HV;
    const size_t ssz = (size_t)dv * dk;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
    for (long p = 0; p < pairs; ++p) {
        const int n = (int)(p / HV), h = (int)(p % HV);
        const int hk = h / (HV / H);
        const int32_t s = slots ? slots[n] : n;
        double* ot = o + (size_t)p * dv;
        if (s < 0 || s >= num_slots) {
            for (int i = 0; i < dv; ++i) ot[i] = 0.0;
            continue;
        }
        double* wk = (double*)malloc((size_t)(dv + 2 * dk) * sizeof(double));
        if (!wk) {
            failed = 1;
            continue;
        }
        double* qd = wk + dv;
        double* kd = qd + dk;
        for (int j = 0; j < dk; ++j) {
            qd[j] = (double)q[((size_t)n * H + hk) * dk + j];
            kd[j] = (double)k[((size_t)n * H + hk) * dk + j];
        }
        if (l2norm) {
            l2norm_row(qd, dk, l2_eps);
            l2norm_row(kd, dk, l2_eps);
        }
        step_one(qd, kd, v + (size_t)p * dv, exp(g[p]), beta[p], dk, dv, scale,
                 pool + ((size_t)s * HV + h) * ssz, ot, wk);
        free(wk);
    }
    return failed ? -1 : 0;
}

/*
 * Rotary position embedding on the first rd of d dimensions (the partial
 * rotary embedding of the gated attention layers: Core AI card for
 * Qwen3.6-35B-A3B, introduction, names partial mRoPE with theta = 1e7; for
 * text every mRoPE section carries the same position, which is plain RoPE).
 * Pairs (i, i + rd/2), i < rd/2, rotate by the angle p * theta^(-2i/rd):
 *     y_i        = x_i cos - x_{i+rd/2} sin
 *     y_{i+rd/2} = x_{i+rd/2} cos + x_i sin
 * Dimensions rd .. d-1 pass unchanged.
 *   x : [rows, d] float32    pos : [rows] int32    y : [rows, d] double
 */
static void rope_row(const double* x, int d, int rd, double theta, double p, double* y) {
    for (int j = 0; j < d; ++j) y[j] = x[j];
    const int half = rd / 2;
    for (int i = 0; i < half; ++i) {
        const double ang = p * pow(theta, -2.0 * i / rd);
        const double c = cos(ang), s = sin(ang);
        y[i] = x[i] * c - x[i + half] * s;
        y[i + half] = x[i + half] * c + x[i] * s;
    }
}

int gdn_oracle_rope(const float* x, const int32_t* pos, long rows, int d, int rd, double theta,
                    double* y) {
    if (rows < 0 || d <= 0 || rd < 0 || rd > d || rd % 2) return -1;
    double* xd = (double*)malloc((size_t)d * sizeof(double));
    if (!xd) return -1;
    for (long r = 0; r < rows; ++r) {
        for (int j = 0; j < d; ++j) xd[j] = (double)x[(size_t)r * d + j];
        rope_row(xd, d, rd, theta, (double)pos[r], y + (size_t)r * d);
    }
    free(xd);
    return 0;
}

/*
 * One decode step of gated full attention (standard scaled dot-product
 * attention: Qwen3.5-0.8B chat guide, section "Architektur"; GQA with query
 * head h reading key/value head h / (Hq / Hkv)), written out:
 *     qr = rope(q, pos), kr = rope(k_new, pos)
 *     s_t = scale * qr . K_t   for t < pos (cached keys, stored rotated), and
 *     s_pos = scale * qr . kr
 *     o = sum_t softmax(s)_t V_t   (V_pos = v_new),   o *= sigmoid(gate) if given
 *   q, gate : [N, Hq, d] float32 (gate may be NULL)
 *   knew, vnew : [N, Hkv, d] float32
 *   kc, vc  : [N, Hkv, Lmax, d] float32, rows t < pos[n] valid
 *   pos     : [N] int32, 0 <= pos < Lmax
 *   o       : [N, Hq, d] double
 *   kr_out  : [N, Hkv, d] double, the rotated new key (what the step appends)
 * Returns 0, or -1 on invalid sizes or a failed allocation.
 */
int gdn_oracle_attn_decode(const float* q, const float* gate, const float* knew,
                           const float* vnew, const float* kc, const float* vc,
                           const int32_t* pos, int N, int Hq, int Hkv, int d, int Lmax, int rd,
                           double theta, double scale, double* o, double* kr_out) {
    if (N < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || rd < 0 || rd > d || rd % 2 ||
        Lmax <= 0)
        return -1;
    for (int n = 0; n < N; ++n)
        if (pos[n] < 0 || pos[n] >= Lmax) return -1;
    int failed = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (long p = 0; p < (long)N * Hq; ++p) {
        const int n = (int)(p / Hq), h = (int)(p % Hq);
        const int hk = h / (Hq / Hkv);
        const int L = pos[n] + 1;
        double* buf = (double*)malloc((size_t)(4 * d + L) * sizeof(double));
        if (!buf) {
            failed = 1;
            continue;
        }
        double *xd = buf, *qr = buf + d, *kr = buf + 2 * d, *acc = buf + 3 * d, *sc = buf + 4 * d;
        for (int j = 0; j < d; ++j) xd[j] = (double)q[(size_t)p * d + j];
        rope_row(xd, d, rd, theta, (double)pos[n], qr);
        const size_t kvh = (size_t)n * Hkv + hk;
        for (int j = 0; j < d; ++j) xd[j] = (double)knew[kvh * d + j];
        rope_row(xd, d, rd, theta, (double)pos[n], kr);
        if (h % (Hq / Hkv) == 0)
            for (int j = 0; j < d; ++j) kr_out[kvh * d + j] = kr[j];
        double mx = -INFINITY;
        for (int t = 0; t < L; ++t) {
            const float* kt = kc + (kvh * Lmax + t) * d;
            double s = 0.0;
            for (int j = 0; j < d; ++j) s += qr[j] * (t < pos[n] ? (double)kt[j] : kr[j]);
            sc[t] = scale * s;
            if (sc[t] > mx) mx = sc[t];
        }
        double den = 0.0;
        for (int t = 0; t < L; ++t) {
            sc[t] = exp(sc[t] - mx);
            den += sc[t];
        }
        for (int j = 0; j < d; ++j) acc[j] = 0.0;
        for (int t = 0; t < L; ++t) {
            const float* vt = t < pos[n] ? vc + (kvh * Lmax + t) * d : vnew + kvh * d;
            for (int j = 0; j < d; ++j) acc[j] += sc[t] * (double)vt[j];
        }
        for (int j = 0; j < d; ++j) {
            double v = acc[j] / den;
            if (gate) v *= 1.0 / (1.0 + exp(-(double)gate[(size_t)p * d + j]));
            o[(size_t)p * d + j] = v;
        }
        free(buf);
    }
    return failed ? -1 : 0;
}

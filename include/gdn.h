/*
 * gdn.h -- libgdn: the Gated DeltaNet token mixer on AMD Instinct MI355X (gfx950).
 *
 * The mixer is the linear-attention layer of the Qwen3.5 / Qwen3.6 hybrid
 * decoders: the Qwen3.5-0.8B chat guide (soniqo.audio, section "Architektur")
 * describes 18 of its 24 layers as linear attention with a gated-delta-rule
 * recurrence followed by RMSNormGated; the Qwen3.6-35B-A3B card of the Core AI
 * model zoo (intro) runs 32 value heads over 16 key heads, each key/query head
 * shared by two value heads; the Swiftlet post ("How It Works") notes the
 * fixed-size recurrent state.  The recurrence is the gated delta rule (Yang,
 * Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025), per sequence and
 * value head:
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T        a_t = exp(g_t)
 *     o_t = scale * S_t q_t                                         b_t = beta_t
 *
 * S_t is d_v x d_k (row i <-> value dim, column j <-> key dim); the readout uses
 * the state after the token's update.  Value head h reads key/query head
 * h / (HV / H) (consecutive value heads share a key head).
 *
 * Conventions for every call
 *  - Pointers are device pointers unless stated.  Tensors are dense, row-major,
 *    with the layouts given per argument, and 16-byte aligned.
 *  - The caller owns all memory, including the prefill workspace.  The library
 *    allocates nothing, keeps no global state and is reentrant.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued and the call returns without synchronising.
 *  - Arguments are validated on the host before anything is enqueued.  On an
 *    error nothing is enqueued and no output is touched.  A kernel launch
 *    failure returns GDN_ERROR_HIP; device faults surface at the caller's next
 *    synchronisation.  No C++ exception crosses this interface.
 *  - Supported: d_k, d_v in {16, 32, 64, 128}; HV a multiple of H; chunk 64;
 *    q/k/v in GDN_F32 or GDN_BF16; outputs in GDN_F32 or GDN_BF16.  Other
 *    values return GDN_ERROR_NOT_SUPPORTED.  g and beta are fp32.
 *  - Preconditions not checked (documented): finite inputs; cu_seqlens
 *    non-decreasing with cu_seqlens[0] = 0 and cu_seqlens[N] = T_total.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_SUCCESS = 0,
    GDN_ERROR_INVALID_VALUE = 1, /* null pointer, bad size, misaligned pointer */
    GDN_ERROR_NOT_SUPPORTED = 2, /* a head size, chunk or dtype outside the list above */
    GDN_ERROR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    GDN_ERROR_HIP = 4            /* the HIP runtime reported an error at launch */
} gdn_status;

typedef enum gdn_dtype {
    GDN_F32 = 0,  /* IEEE binary32 */
    GDN_BF16 = 1  /* bfloat16 (upper 16 bits of binary32) */
} gdn_dtype;

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int gdn_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* gdn_status_string(int status);

/*
 * Name of the HIP error behind the most recent GDN_ERROR_HIP returned on the
 * calling thread ("hipSuccess" if there was none).  Static string, never NULL.
 * Before launching, each entry point clears a HIP error that earlier calls
 * left pending on this thread, so GDN_ERROR_HIP always refers to libgdn's
 * own launches.
 */
const char* gdn_last_hip_error(void);

/*
 * gdn_decode_step -- advance every sequence by one token against its resident
 * state, in place.  This is the single-step decoder that owns its recurrent
 * state and is advanced one token per call (Qwen3.5-0.8B Core ML card on
 * aimarketly.com, section "Model").
 *
 *   q, k     [N, H, dk]      in_dtype   query and key of the token
 *   v        [N, HV, dv]     in_dtype   value
 *   g        [N, HV]         fp32       log-decay, a = exp(g) (g <= 0 expected)
 *   beta     [N, HV]         fp32       write strength b
 *   state    [N, HV, dv, dk] fp32       S_{t-1} in, S_t out (read fully before
 *                                       any element is written; one lane owns
 *                                       each element)
 *   o        [N, HV, dv]     o_dtype    o_t = scale * S_t q_t
 *   N >= 0 sequences (N == 0 is a successful no-op).
 */
gdn_status gdn_decode_step(const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                           const float* g, const float* beta, float* state, void* o,
                           gdn_dtype o_dtype, int N, int H, int HV, int dk, int dv,
                           float scale, void* stream);

/*
 * gdn_decode_step_norm -- gdn_decode_step followed by RMSNormGated of each
 * head's outputs in the same kernel: the decode step and the norm that closes
 * the DeltaNet layer (Qwen3.5-0.8B chat guide, section "Architektur"), without
 * the round trip of o through memory and without a second launch.
 *
 *   q, k, v, g, beta, state   as gdn_decode_step
 *   z        [N, HV, dv]     z_dtype    gate input of the norm
 *   w        [dv]            w_dtype    norm weight shared by heads
 *   y        [N, HV, dv]     y_dtype    y = o / sqrt(mean_dv(o^2) + eps) * w * silu(z)
 *   o        [N, HV, dv]     o_dtype    the raw outputs too, or NULL to skip them
 *   eps >= 0.
 */
gdn_status gdn_decode_step_norm(const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                                const float* g, const float* beta, float* state, const void* z,
                                gdn_dtype z_dtype, const void* w, gdn_dtype w_dtype, void* y,
                                gdn_dtype y_dtype, void* o, gdn_dtype o_dtype, int N, int H,
                                int HV, int dk, int dv, float scale, float eps, void* stream);

/*
 * gdn_decode_layer -- the serving form of the decode step: the token mixer of
 * one DeltaNet layer for one token per sequence, in one launch, with the
 * steps on either side of the recurrence done in the kernel.
 *
 *  - State pool.  The decoder owns all recurrent state and is advanced one
 *    token per call (Qwen3.5-0.8B Core ML card, section "Model"); a server
 *    keeps the states of all live requests in one pool and names, per batch
 *    row, the slot to advance.  A slot outside [0, num_slots) skips that row:
 *    its o and y rows are written as 0 and no state is read or written.  Two
 *    rows naming the same slot race (caller error; every access stays inside
 *    the pool).
 *  - Gate activations.  The pages name the decay and the write strength but
 *    not how the layer produces them; given the raw per-(token, value head)
 *    projections, the kernel applies the Gated DeltaNet layer's
 *    parameterisation (Yang et al., ICLR 2025):
 *        g = -exp(A_log[h]) * softplus(a_raw + dt_bias[h]),  beta = sigmoid(b_raw)
 *  - q/k L2 norm.  Optionally q and k are divided by sqrt(sum of squares +
 *    l2_eps) per (row, key head) before the step.
 *  - RMSNormGated, as in gdn_decode_step_norm, when z, w and y are given.
 *
 * Zero-initialise the struct and fill in what is used; all pointers are
 * device pointers, 16-byte aligned except slots, a_raw, b_raw, g, beta,
 * A_log and dt_bias (element-aligned).
 */
typedef struct gdn_decode_layer_args {
    const void* q;          /* [N, H, dk]   in_dtype                                      */
    const void* k;          /* [N, H, dk]   in_dtype                                      */
    const void* v;          /* [N, HV, dv]  in_dtype                                      */
    gdn_dtype in_dtype;
    /* gates, activated: used when a_raw is NULL                                          */
    const float* g;         /* [N, HV] fp32 log-decay (a = exp(g))                        */
    const float* beta;      /* [N, HV] fp32                                               */
    /* gates, raw: used when a_raw is not NULL (then b_raw and A_log are required)        */
    const void* a_raw;      /* [N, HV] gate_dtype                                         */
    const void* b_raw;      /* [N, HV] gate_dtype                                         */
    gdn_dtype gate_dtype;
    const float* A_log;     /* [HV] fp32                                                  */
    const float* dt_bias;   /* [HV] fp32, or NULL for zeros                               */
    int qk_l2norm;          /* nonzero: L2-normalise q and k first                        */
    float l2_eps;           /* >= 0; > 0 keeps an all-zero q or k finite                  */
    float* state;           /* [num_slots, HV, dv, dk] fp32, advanced in place            */
    const int32_t* slots;   /* [N] int32, or NULL: row n uses slot n (num_slots >= N)     */
    int num_slots;          /* >= 0                                                       */
    void* o;                /* [N, HV, dv] o_dtype: scale * S_t q_t, or NULL if y is set  */
    gdn_dtype o_dtype;
    const void* z;          /* [N, HV, dv] z_dtype  RMSNormGated gate input, or NULL      */
    gdn_dtype z_dtype;
    const void* w;          /* [dv] w_dtype         RMSNormGated weight, or NULL          */
    gdn_dtype w_dtype;
    void* y;                /* [N, HV, dv] y_dtype  normed output, or NULL                */
    gdn_dtype y_dtype;
    float eps;              /* RMSNormGated epsilon, >= 0                                 */
    int N, H, HV, dk, dv;   /* N >= 0 rows (0 is a successful no-op)                      */
    float scale;
} gdn_decode_layer_args;

/* sizeof(gdn_decode_layer_args) as compiled into the library (binding check). */
size_t gdn_decode_layer_args_size(void);

/*
 * Returns GDN_ERROR_INVALID_VALUE for a NULL args, a missing or misaligned
 * pointer, a negative size or epsilon, neither o nor y given, y given without
 * z and w, or slots NULL with num_slots < N.
 */
gdn_status gdn_decode_layer(const gdn_decode_layer_args* args, void* stream);

/*
 * gdn_prefill_workspace_bytes -- device workspace that gdn_prefill_chunked
 * needs for this problem (a multiple of 256 bytes; 0 when T_total == 0).
 * Returns 0 for sizes that gdn_prefill_chunked would reject.  The size holds
 * the segment-parallel scan's buffers (per segment two d_v x d_k and one
 * d_k x d_k fp32 matrix per value head, and d_k fp32 per token and value
 * head) only when the call can segment: bf16 inputs with d_k in {64, 128},
 * sequences longer than 32 chunks, and (sequence, value head) chains that
 * leave the GPU's compute units idle.
 */
size_t gdn_prefill_workspace_bytes(int N, int T_total, int H, int HV, int dk, int dv,
                                   int chunk);

/*
 * gdn_prefill_workspace_bytes_seg -- the workspace of gdn_prefill_chunked_seg
 * with this segment_chunks (0: the same as gdn_prefill_workspace_bytes; -1:
 * no segment buffers; -2 or a forced length: the buffers whenever a sequence
 * may be longer than one segment).  Returns 0 for sizes or a segment_chunks
 * the call would reject.
 */
size_t gdn_prefill_workspace_bytes_seg(int N, int T_total, int H, int HV, int dk, int dv,
                                       int chunk, int segment_chunks);

/*
 * gdn_prefill_chunked -- a whole packed batch of prompts in the chunked
 * (WY / UT-transform) form, returning every output and the final states.
 * The result equals running the recurrence token by token (up to rounding);
 * chunks restart at every sequence start, so no token influences another
 * sequence.  Incremental use is exact: prefill(A) then prefill(B) from the
 * returned state equals prefill(A+B), as the Swiftlet post's correctness
 * section requires of incremental decoding.
 *
 *   q, k          [T_total, H, dk]    in_dtype  packed tokens of all sequences
 *   v             [T_total, HV, dv]   in_dtype
 *   g, beta       [T_total, HV]       fp32
 *   cu_seqlens    [N + 1]             int32     device; sequence n holds tokens
 *                                               cu_seqlens[n] .. cu_seqlens[n+1]-1
 *                                               (zero-length sequences allowed)
 *   initial_state [N, HV, dv, dk]     fp32      or NULL for zero states
 *   final_state   [N, HV, dv, dk]     fp32      or NULL; may equal initial_state
 *   o             [T_total, HV, dv]   o_dtype
 *   chunk         must be 64
 *   workspace     device memory of workspace_bytes >= gdn_prefill_workspace_bytes(...)
 *   N == 0 or T_total == 0 only copies initial_state to final_state (zeros if
 *   NULL) and is otherwise a no-op.
 */
gdn_status gdn_prefill_chunked(const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                               const float* g, const float* beta, const int32_t* cu_seqlens,
                               int N, int T_total, const float* initial_state,
                               float* final_state, void* o, gdn_dtype o_dtype, int H, int HV,
                               int dk, int dv, int chunk, float scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_chunked_seg -- gdn_prefill_chunked with control over its
 * segment-parallel scan.  The chunk map of the recurrence is affine in the
 * state it starts from, so a long sequence can be cut into segments of whole
 * chunks that run in parallel: each later segment runs once from a zero state
 * and once for its transition (the product of its token maps), a short pass
 * chains the segments' entry states, and a parallel pass adds each entry
 * state's contribution to the segment's outputs.  It pays when few, long
 * sequences leave most of the GPU idle (one long prompt), and costs extra
 * work otherwise; gdn_prefill_chunked decides on the device from the lengths.
 *
 *   segment_chunks   0: decide automatically (as gdn_prefill_chunked): only when
 *                      the (sequence, value head) chains leave CUs idle
 *                   -2: decide automatically from the lengths also when the
 *                      chains fill the GPU: for batches with one prompt far
 *                      longer than the rest (costs two near-empty launches
 *                      when it decides against segments)
 *                   -1: never segment
 *                  >= 32: segments of this many chunks (64 tokens each)
 *   workspace      at least gdn_prefill_workspace_bytes_seg(..., segment_chunks)
 *                  bytes, 256-byte aligned
 *   every other argument as gdn_prefill_chunked.
 * Applies to the bf16-MFMA path (bf16 inputs, d_k in {64, 128}, d_v a
 * multiple of 32); other shapes ignore it.  Other values of segment_chunks
 * return GDN_ERROR_INVALID_VALUE.
 */
gdn_status gdn_prefill_chunked_seg(const void* q, const void* k, const void* v,
                                   gdn_dtype in_dtype, const float* g, const float* beta,
                                   const int32_t* cu_seqlens, int N, int T_total,
                                   const float* initial_state, float* final_state, void* o,
                                   gdn_dtype o_dtype, int H, int HV, int dk, int dv, int chunk,
                                   float scale, int segment_chunks, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_chunked_noalloc -- gdn_prefill_chunked for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace is a static device array of
 * GDN_NOALLOC_SCRATCH_BYTES inside the library, one per GPU it runs on, held
 * until the process ends; its device address is looked up on the first call
 * on each device.  The call allocates nothing.  `stream` must belong to the
 * device current on the calling thread (the array of that device is used).
 *
 *   every argument as gdn_prefill_chunked (automatic segmentation), minus the
 *   workspace.
 * Returns GDN_ERROR_WORKSPACE, before any HIP call, when
 * gdn_prefill_workspace_bytes(N, T_total, H, HV, dk, dv, chunk) exceeds
 * GDN_NOALLOC_SCRATCH_BYTES; GDN_ERROR_HIP if the array's address cannot be
 * found.  Every call on one GPU uses that GPU's one array: calls that overlap
 * on one GPU (on different streams, or from different threads without an
 * order between their streams) race and give wrong results.  Nothing in the
 * array needs to start at zero, so the contents left by an earlier call do
 * not matter.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (256u * 1024u * 1024u)

gdn_status gdn_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       gdn_dtype in_dtype, const float* g, const float* beta,
                                       const int32_t* cu_seqlens, int N, int T_total,
                                       const float* initial_state, float* final_state, void* o,
                                       gdn_dtype o_dtype, int H, int HV, int dk, int dv,
                                       int chunk, float scale, void* stream);

/*
 * gdn_prefill_chunked_norm -- gdn_prefill_chunked followed by RMSNormGated of
 * each (token, value head)'s outputs: the prompt pass of the token mixer up to
 * the norm that closes the DeltaNet layer (Qwen3.5-0.8B chat guide, section
 * "Architektur").  Per (token, value head) group of dv outputs o:
 *
 *     y = o / sqrt(mean(o^2) + eps) * w * silu(z)
 *
 *   q .. final_state   as gdn_prefill_chunked
 *   z        [T_total, HV, dv]  z_dtype   gate input of the norm
 *   w        [dv]               w_dtype   norm weight shared by heads
 *   y        [T_total, HV, dv]  y_dtype   the normed outputs
 *   o        [T_total, HV, dv]  o_dtype   the raw outputs too, or NULL
 *   eps >= 0; chunk must be 64
 *   workspace device memory of workspace_bytes >=
 *             gdn_prefill_norm_workspace_bytes(...) (256-byte aligned)
 * The raw outputs go to o (or, when o is NULL, in fp32 to the workspace) and
 * a second launch applies the norm: a head's outputs come from four
 * workgroups, one per 32 state rows.  y may not be o.  Errors as
 * gdn_prefill_chunked, plus GDN_ERROR_INVALID_VALUE for a missing or
 * misaligned z, w or y, y == o or a negative eps.
 */
size_t gdn_prefill_norm_workspace_bytes(int N, int T_total, int H, int HV, int dk, int dv,
                                        int chunk);

gdn_status gdn_prefill_chunked_norm(const void* q, const void* k, const void* v,
                                    gdn_dtype in_dtype, const float* g, const float* beta,
                                    const int32_t* cu_seqlens, int N, int T_total,
                                    const float* initial_state, float* final_state,
                                    const void* z, gdn_dtype z_dtype, const void* w,
                                    gdn_dtype w_dtype, void* y, gdn_dtype y_dtype, void* o,
                                    gdn_dtype o_dtype, int H, int HV, int dk, int dv, int chunk,
                                    float scale, float eps, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * gdn_attn_decode -- one decode step of gated full attention, the hybrid
 * decoder's other token mixer (standard scaled dot-product attention: chat
 * guide (de), section "Architektur"; head_dim 256, 16 query heads over 2
 * key/value heads, partial mRoPE with theta = 1e7: Core AI card for
 * Qwen3.6-35B-A3B, introduction).  Per row n, query head h, key/value head
 * h / (Hq / Hkv), p = pos[n]:
 *
 *     qr = rope(q, p), kr = rope(k_new, p)
 *     o  = sigmoid(gate) * softmax_t(scale qr . K_t) V_t,   t = 0 .. p
 *
 * with K_t, V_t the cached rows for t < p and (kr, v_new) for t = p; the call
 * also writes kr (rounded to bf16) and v_new into the caches at row p.  rope
 * rotates the pairs (i, i + rotary_dim/2), i < rotary_dim/2, by the angle
 * p * rope_theta^(-2i/rotary_dim) and leaves the other dimensions as they
 * are (text tokens carry the same position on every mRoPE section).  The
 * pages give only the names of these parts; the rotate-half pairing, keys
 * cached after rotation and the sigmoid output gate are this library's
 * readings.
 */
typedef struct gdn_attn_decode_args {
    const void* q;          /* [N, Hq, D] bf16, before the rotary embedding           */
    const void* gate;       /* [N, Hq, D] bf16 output gate, or NULL for none          */
    const void* k_new;      /* [N, Hkv, D] bf16, before the rotary embedding          */
    const void* v_new;      /* [N, Hkv, D] bf16                                       */
    void* k_cache;          /* [N, Hkv, Lmax, D] bf16: rows t < pos[n] are read (keys  */
                            /* stored rotated), row pos[n] is written                  */
    void* v_cache;          /* [N, Hkv, Lmax, D] bf16, the same rows                   */
    const int32_t* pos;     /* [N] int32: 0 <= pos[n] < Lmax (not checked on the host) */
    void* o;                /* [N, Hq, D] o_dtype                                      */
    gdn_dtype o_dtype;
    int N, Hq, Hkv, D, Lmax;  /* D in {64, 128, 256}; Hq / Hkv in {1, 2, 4, 8, 16}     */
    int rotary_dim;         /* even, <= D (64 for head_dim 256 with a quarter rotated) */
    float rope_theta;       /* > 0 (1e7)                                               */
    float scale;            /* usually D^-1/2                                          */
    void* workspace;        /* device memory, 256-byte aligned, at least              */
    size_t workspace_bytes; /* gdn_attn_decode_workspace_bytes(N, Hq, Hkv, D, Lmax)    */
} gdn_attn_decode_args;

/* sizeof(gdn_attn_decode_args) as compiled into the library (binding check). */
size_t gdn_attn_decode_args_size(void);

/* Workspace gdn_attn_decode needs (partial results of its position splits). */
size_t gdn_attn_decode_workspace_bytes(int N, int Hq, int Hkv, int D, int Lmax);

/*
 * Returns GDN_ERROR_INVALID_VALUE for a NULL args, a missing or misaligned
 * pointer, non-positive sizes, an odd or too large rotary_dim, or
 * rope_theta <= 0; GDN_ERROR_NOT_SUPPORTED for other D, head ratios or
 * dtypes; GDN_ERROR_WORKSPACE for a missing or short workspace.  pos lives on
 * the device and is not checked on the host: a row with pos[n] outside
 * [0, Lmax) touches no cache and gets NaN outputs.
 */
gdn_status gdn_attn_decode(const gdn_attn_decode_args* args, void* stream);

/*
 * gdn_rmsnorm_gated -- RMSNormGated, the norm that closes each DeltaNet layer
 * (Qwen3.5-0.8B chat guide, section "Architektur").  Per (row, head) group of
 * dv values:
 *
 *     y = x / sqrt(mean(x^2) + eps) * w * silu(z),   silu(z) = z / (1 + e^-z)
 *
 *   x   [rows, HV, dv]  x_dtype      (usually the mixer output o)
 *   z   [rows, HV, dv]  z_dtype      gate input
 *   w   [dv]            w_dtype      weight shared by all heads
 *   y   [rows, HV, dv]  y_dtype      may alias x when y_dtype == x_dtype
 *   rows >= 0 (0 is a successful no-op), eps >= 0.
 */
gdn_status gdn_rmsnorm_gated(const void* x, gdn_dtype x_dtype, const void* z, gdn_dtype z_dtype,
                             const void* w, gdn_dtype w_dtype, void* y, gdn_dtype y_dtype,
                             int rows, int HV, int dv, float eps, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */

// gdn_internal.h -- host-side argument bundles and kernel launchers shared by
// the C-ABI layer (gdn_api.cpp) and the kernel translation units.  Arguments
// reaching a launcher have already been validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;
    void* o;          // may be null when fuse_norm
    bool in_bf16;
    bool o_bf16;
    int N, H, HV, dk, dv;
    float scale;
    // RMSNormGated fused after the update (gdn_decode_step_norm)
    bool fuse_norm;
    const void* z;
    const void* w;
    void* y;
    bool z_bf16, w_bf16, y_bf16;
    float eps;
    // serving form (gdn_decode_layer): slot table, raw gates, q/k L2 norm
    bool ext;
    const int32_t* slots;  // may be null: sequence n -> slot n
    int num_slots;         // state holds num_slots x HV heads
    const void* a_raw;     // null: g and beta are used as given
    const void* b_raw;
    bool gate_bf16;
    const float* A_log;
    const float* dt_bias;  // may be null
    bool l2norm;
    float l2_eps;
    hipStream_t stream;
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;
    const float* s0;   // may be null (zeros)
    float* s_final;    // may be null
    void* o;
    bool in_bf16;
    bool o_bf16;
    int N, T, H, HV, dk, dv;
    float scale;
    // workspace carve-up (device pointers into the caller's buffer)
    int32_t* chunk_off;  // [N + 1]
    float* ws_G;         // [max_chunks, HV, 64]      in-chunk cumulative log-decay
    // vector-unit path
    float* ws_T;         // [max_chunks, HV, 64, 64]  T' = (I + A)^-1 diag(beta), fp32
    // MFMA path (same memory as ws_T), each as hi + lo bf16 planes:
    //   R  = P T'                          [max_chunks, HV, 64, 64]   (row t, column c)
    //   Zt = K^T diag(e^{G_n - G}) T'      [max_chunks, HV, dk, 64]   (row j, column c)
    uint16_t* ws_Rh;
    uint16_t* ws_Rl;
    uint16_t* ws_Zh;
    uint16_t* ws_Zl;
    // T'-only path (same memory): T' = (I + A)^-1 diag(b) as ten 16 x 16
    // blocks per (chunk, value head), hi / lo bf16 in the scan's operand order
    uint16_t* ws_Tp;
    int max_chunks;
    // segment-parallel scan (MFMA path).  A sequence is cut into segments of
    // whole chunks; the plan is made on the device from cu_seqlens.
    int seg_req;         // 0: automatic; kSegAutoSkewed: automatic for skewed lengths;
                         // -1: never; >= kSegMinChunks: this segment length
    int seg_bound;       // capacity of the segment tables
    int corr_bound;      // capacity of the correction item table
    int32_t* plan;       // [kPlanInts]: nseg, ncorr, segment length (0: none), nmulti
    int32_t* seg_seq;    // [seg_bound] sequence of segment s
    int32_t* seg_c0;     // [seg_bound] global index of its first chunk
    int32_t* seg_nch;    // [seg_bound] its chunks
    int32_t* seg_idx;    // [seg_bound] its position in the sequence (0: first)
    int32_t* seq_seg0;   // [N] first segment of sequence n
    int32_t* seq_nseg;   // [N] segments of sequence n
    int32_t* multi_seq;  // [N] sequences with more than one segment
    int32_t* corr_seg;   // [corr_bound] correction item: its segment
    int32_t* corr_c0;    // [corr_bound] correction item: its first chunk (global index)
    float* ws_E;         // [seg_bound, HV, dv, dk] end state of a segment's own pass
    float* ws_Phi;       // [seg_bound, HV, dk, dk] transition of a segment
    float* ws_Sin;       // [seg_bound, HV, dv, dk] state entering a segment
    float* ws_W;         // [T, HV, dk] scale Phi_t q_t for tokens of later segments
    hipStream_t stream;
};

constexpr int kSegMinChunks = 32;  // shortest segment of the segment-parallel scan
constexpr int kSegAutoSkewed = -2; // segment_chunks: automatic, also when the chains fill the CUs
constexpr int kCorrChunks = 4;     // chunks per item of the correction pass
constexpr int kPlanInts = 8;

struct NormArgs {
    const void* x;
    const void* z;
    const void* w;
    void* y;
    bool x_bf16, z_bf16, w_bf16, y_bf16;
    long groups;
    int dv;
    float eps;
    hipStream_t stream;
};

// Workspace layout of gdn_prefill_chunked (byte offsets, 256-aligned).
struct PrefillLayout {
    size_t chunk_off, ws_G, ws_T, ws_Rh, ws_Rl, ws_Zh, ws_Zl;
    size_t plan, seg_seq, seg_c0, seg_nch, seg_idx, seq_seg0, seq_nseg, multi_seq, corr_seg,
        corr_c0, ws_E, ws_Phi, ws_Sin, ws_W;
    size_t total;
    int max_chunks, seg_bound, corr_bound;
};
// seg: reserve the segment-parallel scan's tables and buffers (only when
// prefill_may_segment says the call can segment)
PrefillLayout prefill_layout(int N, int T, int H, int HV, int dk, int dv, bool seg);
// Whether a prefill call of this shape can take the segment-parallel scan
// (the bf16 MFMA path with segments forced, or allowed and useful by the
// host's rule); the device plan then decides from the lengths.
bool prefill_may_segment(int N, int T, int HV, int dk, int dv, bool in_bf16, int seg_req);

// One decode step of gated full attention (gdn_attn_decode).
struct AttnArgs {
    const uint16_t* q;       // [N, Hq, D] bf16, before the rotary embedding
    const uint16_t* gate;    // [N, Hq, D] bf16 or null
    const uint16_t* k_new;   // [N, Hkv, D] bf16, before the rotary embedding
    const uint16_t* v_new;   // [N, Hkv, D] bf16
    uint16_t* k_cache;       // [N, Hkv, Lmax, D] bf16 (rotated keys)
    uint16_t* v_cache;       // [N, Hkv, Lmax, D] bf16
    const int32_t* pos;      // [N] position of the new token
    void* o;                 // [N, Hq, D]
    bool o_bf16;
    int N, Hq, Hkv, D, Lmax, rd;
    float theta, scale;
    int split;               // positions per split workgroup (multiple of 16)
    int nsplit;              // splits per (row, key/value head) in the grid
    float* part;             // [N, Hkv, nsplit, G, D + 2] fp32 partial results
    hipStream_t stream;
};
void attn_plan(int N, int Hq, int Hkv, int D, int Lmax, int& split, int& nsplit, size_t& bytes);
hipError_t launch_attn_decode(const AttnArgs& a);

// Device address (on the current device) and size of the static array that
// gdn_prefill_chunked_noalloc uses as its workspace; looked up once per device.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);
bool prefill_mfma_eligible(const PrefillArgs& a);
hipError_t launch_prefill_mfma(const PrefillArgs& a);
// T'-only prep and the chain / helper scan (d_k = 128)
hipError_t launch_prep_tp(const PrefillArgs& a);
hipError_t launch_scan_tp(const PrefillArgs& a, size_t grid, int items);
hipError_t launch_state_copy(const float* src, float* dst, size_t count, hipStream_t stream);
hipError_t launch_rmsnorm_gated(const NormArgs& a);

}  // namespace gdn

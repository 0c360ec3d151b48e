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
    int max_chunks;
    hipStream_t stream;
};

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
    size_t chunk_off, ws_G, ws_T, ws_Rh, ws_Rl, ws_Zh, ws_Zl, total;
    int max_chunks;
};
PrefillLayout prefill_layout(int N, int T, int H, int HV, int dk);

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);
bool prefill_mfma_eligible(const PrefillArgs& a);
hipError_t launch_prefill_mfma(const PrefillArgs& a);
hipError_t launch_state_copy(const float* src, float* dst, size_t count, hipStream_t stream);
hipError_t launch_rmsnorm_gated(const NormArgs& a);

}  // namespace gdn

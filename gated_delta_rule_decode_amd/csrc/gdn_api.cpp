// gdn_api.cpp -- the C ABI of libgdn: host-side validation and dispatch.
//
// Every check runs on the host before anything is enqueued; a failing check
// returns its status with no HIP call made and no output touched.  See
// include/gdn.h for the contract of each entry point.
#include "gdn.h"

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "gdn_internal.h"

namespace {

constexpr int kVersion = 200;  // 0.2.0

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool valid_dtype(gdn_dtype t) { return t == GDN_F32 || t == GDN_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool valid_seg_req(int r) {
    return r == 0 || r == -1 || r == gdn::kSegAutoSkewed || r >= gdn::kSegMinChunks;
}

gdn_status heads_status(int H, int HV, int dk, int dv) {
    if (H <= 0 || HV <= 0 || dk <= 0 || dv <= 0) return GDN_ERROR_INVALID_VALUE;
    if (HV % H != 0) return GDN_ERROR_INVALID_VALUE;
    if (!supported_d(dk) || !supported_d(dv)) return GDN_ERROR_NOT_SUPPORTED;
    return GDN_SUCCESS;
}

thread_local hipError_t t_last_hip_error = hipSuccess;

gdn_status from_hip(hipError_t e) {
    if (e == hipSuccess) return GDN_SUCCESS;
    t_last_hip_error = e;
    return GDN_ERROR_HIP;
}

// drop an error that earlier HIP calls left pending on this thread
void clear_pending() { (void)hipGetLastError(); }

}  // namespace

namespace gdn {

PrefillLayout prefill_layout(int N, int T, int H, int HV, int dk, int dv, bool seg) {
    (void)H;
    PrefillLayout L{};
    // upper bound on sum_n ceil(len_n / 64) given sum_n len_n = T
    const size_t maxc = ((size_t)T + (size_t)N * (kChunk - 1)) / kChunk;
    L.max_chunks = (int)maxc;
    const size_t tile = (size_t)kChunk * kChunk;  // elements of a 64 x 64 tile
    size_t off = 0;
    L.chunk_off = off;
    off = align256(off + ((size_t)N + 1) * sizeof(int32_t));
    L.ws_G = off;
    off = align256(off + maxc * HV * kChunk * sizeof(float));
    // one region, used by either path: T' in fp32 (vector-unit path), or R and
    // Z^T as hi and lo bf16 planes (MFMA path)
    const size_t region = off;
    L.ws_T = region;
    const size_t valu_end = align256(region + maxc * HV * tile * sizeof(float));
    const size_t rplane = align256(maxc * HV * tile * sizeof(uint16_t));
    const size_t zplane = align256(maxc * HV * (size_t)dk * kChunk * sizeof(uint16_t));
    L.ws_Rh = region;
    L.ws_Rl = region + rplane;
    L.ws_Zh = region + 2 * rplane;
    L.ws_Zl = region + 2 * rplane + zplane;
    const size_t mfma_end = region + 2 * rplane + 2 * zplane;
    off = valu_end > mfma_end ? valu_end : mfma_end;
    // segment-parallel scan: plan, tables and the per-segment states.  A call
    // that cannot segment has one segment per sequence and no correction
    // items, and never touches E, Phi, S_in or w: they take no space then.
    const size_t segb = seg ? (size_t)N + (maxc + kSegMinChunks - 1) / kSegMinChunks : (size_t)N;
    const size_t corrb = seg ? segb + maxc / kCorrChunks + 1 : 1;
    L.seg_bound = (int)segb;
    L.corr_bound = (int)corrb;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    L.plan = take(kPlanInts * sizeof(int32_t));
    L.seg_seq = take(segb * sizeof(int32_t));
    L.seg_c0 = take(segb * sizeof(int32_t));
    L.seg_nch = take(segb * sizeof(int32_t));
    L.seg_idx = take(segb * sizeof(int32_t));
    L.seq_seg0 = take((size_t)N * sizeof(int32_t));
    L.seq_nseg = take((size_t)N * sizeof(int32_t));
    L.multi_seq = take((size_t)N * sizeof(int32_t));
    L.corr_seg = take(corrb * sizeof(int32_t));
    L.corr_c0 = take(corrb * sizeof(int32_t));
    const size_t segs = seg ? segb : 0;
    L.ws_E = take(segs * HV * (size_t)dv * dk * sizeof(float));
    L.ws_Phi = take(segs * HV * (size_t)dk * dk * sizeof(float));
    L.ws_Sin = take(segs * HV * (size_t)dv * dk * sizeof(float));
    L.ws_W = take(seg ? (size_t)T * HV * dk * sizeof(float) : 0);
    L.total = off;
    return L;
}

}  // namespace gdn

extern "C" {

int gdn_version(void) { return kVersion; }

const char* gdn_last_hip_error(void) { return hipGetErrorName(t_last_hip_error); }

const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_SUCCESS: return "GDN_SUCCESS";
        case GDN_ERROR_INVALID_VALUE: return "GDN_ERROR_INVALID_VALUE";
        case GDN_ERROR_NOT_SUPPORTED: return "GDN_ERROR_NOT_SUPPORTED";
        case GDN_ERROR_WORKSPACE: return "GDN_ERROR_WORKSPACE";
        case GDN_ERROR_HIP: return "GDN_ERROR_HIP";
        default: return "GDN_UNKNOWN_STATUS";
    }
}

}  // extern "C"

namespace {

gdn_status decode_common(const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                         const float* g, const float* beta, float* state, int N, int H, int HV,
                         int dk, int dv) {
    if (N < 0) return GDN_ERROR_INVALID_VALUE;
    gdn_status st = heads_status(H, HV, dk, dv);
    if (st != GDN_SUCCESS) return st;
    if (!valid_dtype(in_dtype)) return GDN_ERROR_NOT_SUPPORTED;
    if (N == 0) return GDN_SUCCESS;
    if (!q || !k || !v || !g || !beta || !state) return GDN_ERROR_INVALID_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state))
        return GDN_ERROR_INVALID_VALUE;
    if ((size_t)N * HV > (size_t)(1u << 31) / (size_t)dv) return GDN_ERROR_NOT_SUPPORTED;
    return GDN_SUCCESS;
}

}  // namespace

extern "C" {

gdn_status gdn_decode_step(const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                           const float* g, const float* beta, float* state, void* o,
                           gdn_dtype o_dtype, int N, int H, int HV, int dk, int dv, float scale,
                           void* stream) {
    gdn_status st = decode_common(q, k, v, in_dtype, g, beta, state, N, H, HV, dk, dv);
    if (st != GDN_SUCCESS || N == 0) return st;
    if (!valid_dtype(o_dtype)) return GDN_ERROR_NOT_SUPPORTED;
    if (!o || !aligned16(o)) return GDN_ERROR_INVALID_VALUE;
    clear_pending();
    gdn::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
    a.in_bf16 = in_dtype == GDN_BF16; a.o_bf16 = o_dtype == GDN_BF16;
    a.N = N; a.H = H; a.HV = HV; a.dk = dk; a.dv = dv; a.scale = scale;
    a.fuse_norm = false;
    a.stream = static_cast<hipStream_t>(stream);
    return from_hip(gdn::launch_decode(a));
}

gdn_status gdn_decode_step_norm(const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                                const float* g, const float* beta, float* state, const void* z,
                                gdn_dtype z_dtype, const void* w, gdn_dtype w_dtype, void* y,
                                gdn_dtype y_dtype, void* o, gdn_dtype o_dtype, int N, int H,
                                int HV, int dk, int dv, float scale, float eps, void* stream) {
    gdn_status st = decode_common(q, k, v, in_dtype, g, beta, state, N, H, HV, dk, dv);
    if (st != GDN_SUCCESS) return st;
    if (!(eps >= 0.f)) return GDN_ERROR_INVALID_VALUE;
    if (!valid_dtype(z_dtype) || !valid_dtype(w_dtype) || !valid_dtype(y_dtype) ||
        !valid_dtype(o_dtype))
        return GDN_ERROR_NOT_SUPPORTED;
    if (N == 0) return GDN_SUCCESS;
    if (!z || !w || !y || !aligned16(z) || !aligned16(w) || !aligned16(y))
        return GDN_ERROR_INVALID_VALUE;
    if (o && !aligned16(o)) return GDN_ERROR_INVALID_VALUE;
    clear_pending();
    gdn::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
    a.in_bf16 = in_dtype == GDN_BF16; a.o_bf16 = o_dtype == GDN_BF16;
    a.N = N; a.H = H; a.HV = HV; a.dk = dk; a.dv = dv; a.scale = scale;
    a.fuse_norm = true;
    a.z = z; a.w = w; a.y = y;
    a.z_bf16 = z_dtype == GDN_BF16; a.w_bf16 = w_dtype == GDN_BF16; a.y_bf16 = y_dtype == GDN_BF16;
    a.eps = eps;
    a.stream = static_cast<hipStream_t>(stream);
    return from_hip(gdn::launch_decode(a));
}

size_t gdn_decode_layer_args_size(void) { return sizeof(gdn_decode_layer_args); }

gdn_status gdn_decode_layer(const gdn_decode_layer_args* p, void* stream) {
    if (!p) return GDN_ERROR_INVALID_VALUE;
    const gdn_decode_layer_args& x = *p;
    if (x.N < 0 || x.num_slots < 0) return GDN_ERROR_INVALID_VALUE;
    gdn_status st = heads_status(x.H, x.HV, x.dk, x.dv);
    if (st != GDN_SUCCESS) return st;
    const bool raw = x.a_raw != nullptr;
    const bool norm = x.y != nullptr;
    if (!valid_dtype(x.in_dtype) || (raw && !valid_dtype(x.gate_dtype)) ||
        (x.o && !valid_dtype(x.o_dtype)) ||
        (norm && (!valid_dtype(x.z_dtype) || !valid_dtype(x.w_dtype) || !valid_dtype(x.y_dtype))))
        return GDN_ERROR_NOT_SUPPORTED;
    if (!(x.l2_eps >= 0.f) || (norm && !(x.eps >= 0.f))) return GDN_ERROR_INVALID_VALUE;
    if (!x.slots && x.num_slots < x.N) return GDN_ERROR_INVALID_VALUE;
    if (x.N == 0) return GDN_SUCCESS;
    if (!x.q || !x.k || !x.v || !x.state || !aligned16(x.q) || !aligned16(x.k) ||
        !aligned16(x.v) || !aligned16(x.state))
        return GDN_ERROR_INVALID_VALUE;
    if (raw ? (!x.b_raw || !x.A_log) : (!x.g || !x.beta)) return GDN_ERROR_INVALID_VALUE;
    if (!x.o && !norm) return GDN_ERROR_INVALID_VALUE;
    if (x.o && !aligned16(x.o)) return GDN_ERROR_INVALID_VALUE;
    if (norm && (!x.z || !x.w || !aligned16(x.z) || !aligned16(x.w) || !aligned16(x.y)))
        return GDN_ERROR_INVALID_VALUE;
    if ((size_t)x.N * x.HV > (size_t)(1u << 31) / (size_t)x.dv) return GDN_ERROR_NOT_SUPPORTED;
    clear_pending();
    gdn::DecodeArgs a{};
    a.q = x.q; a.k = x.k; a.v = x.v; a.g = x.g; a.beta = x.beta; a.state = x.state; a.o = x.o;
    a.in_bf16 = x.in_dtype == GDN_BF16; a.o_bf16 = x.o && x.o_dtype == GDN_BF16;
    a.N = x.N; a.H = x.H; a.HV = x.HV; a.dk = x.dk; a.dv = x.dv; a.scale = x.scale;
    a.fuse_norm = norm;
    if (norm) {
        a.z = x.z; a.w = x.w; a.y = x.y;
        a.z_bf16 = x.z_dtype == GDN_BF16; a.w_bf16 = x.w_dtype == GDN_BF16;
        a.y_bf16 = x.y_dtype == GDN_BF16;
        a.eps = x.eps;
    }
    a.ext = true;
    a.slots = x.slots;
    a.num_slots = x.num_slots;
    if (raw) {
        a.a_raw = x.a_raw; a.b_raw = x.b_raw; a.gate_bf16 = x.gate_dtype == GDN_BF16;
        a.A_log = x.A_log; a.dt_bias = x.dt_bias;
    }
    a.l2norm = x.qk_l2norm != 0;
    a.l2_eps = x.l2_eps;
    a.stream = static_cast<hipStream_t>(stream);
    return from_hip(gdn::launch_decode(a));
}

size_t gdn_attn_decode_args_size(void) { return sizeof(gdn_attn_decode_args); }

}  // extern "C"

namespace {

gdn_status attn_shape_status(int N, int Hq, int Hkv, int D, int Lmax) {
    if (N < 0 || Hq <= 0 || Hkv <= 0 || Lmax <= 0 || Hq % Hkv) return GDN_ERROR_INVALID_VALUE;
    const int G = Hq / Hkv;
    if (D != 64 && D != 128 && D != 256) return GDN_ERROR_NOT_SUPPORTED;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return GDN_ERROR_NOT_SUPPORTED;
    if ((size_t)N * Hkv > 65535 || (size_t)Lmax * D * 2 > (size_t)INT32_MAX)
        return GDN_ERROR_NOT_SUPPORTED;
    return GDN_SUCCESS;
}

}  // namespace

extern "C" {

size_t gdn_attn_decode_workspace_bytes(int N, int Hq, int Hkv, int D, int Lmax) {
    if (attn_shape_status(N, Hq, Hkv, D, Lmax) != GDN_SUCCESS || N == 0) return 0;
    int split, nsplit;
    size_t bytes;
    gdn::attn_plan(N, Hq, Hkv, D, Lmax, split, nsplit, bytes);
    return align256(bytes);
}

gdn_status gdn_attn_decode(const gdn_attn_decode_args* p, void* stream) {
    if (!p) return GDN_ERROR_INVALID_VALUE;
    const gdn_attn_decode_args& x = *p;
    gdn_status st = attn_shape_status(x.N, x.Hq, x.Hkv, x.D, x.Lmax);
    if (st != GDN_SUCCESS) return st;
    if (!valid_dtype(x.o_dtype)) return GDN_ERROR_NOT_SUPPORTED;
    if (x.rotary_dim < 0 || x.rotary_dim > x.D || (x.rotary_dim & 1) || !(x.rope_theta > 0.f))
        return GDN_ERROR_INVALID_VALUE;
    if (x.N == 0) return GDN_SUCCESS;
    if (!x.q || !x.k_new || !x.v_new || !x.k_cache || !x.v_cache || !x.pos || !x.o)
        return GDN_ERROR_INVALID_VALUE;
    if (!aligned16(x.q) || !aligned16(x.k_new) || !aligned16(x.v_new) || !aligned16(x.k_cache) ||
        !aligned16(x.v_cache) || !aligned16(x.o) || (x.gate && !aligned16(x.gate)))
        return GDN_ERROR_INVALID_VALUE;
    gdn::AttnArgs a{};
    size_t need;
    gdn::attn_plan(x.N, x.Hq, x.Hkv, x.D, x.Lmax, a.split, a.nsplit, need);
    if (!x.workspace || x.workspace_bytes < need) return GDN_ERROR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(x.workspace) & 255u) != 0) return GDN_ERROR_WORKSPACE;
    a.q = static_cast<const uint16_t*>(x.q);
    a.gate = static_cast<const uint16_t*>(x.gate);
    a.k_new = static_cast<const uint16_t*>(x.k_new);
    a.v_new = static_cast<const uint16_t*>(x.v_new);
    a.k_cache = static_cast<uint16_t*>(x.k_cache);
    a.v_cache = static_cast<uint16_t*>(x.v_cache);
    a.pos = x.pos;
    a.o = x.o;
    a.o_bf16 = x.o_dtype == GDN_BF16;
    a.N = x.N; a.Hq = x.Hq; a.Hkv = x.Hkv; a.D = x.D; a.Lmax = x.Lmax; a.rd = x.rotary_dim;
    a.theta = x.rope_theta;
    a.scale = x.scale;
    a.part = static_cast<float*>(x.workspace);
    a.stream = static_cast<hipStream_t>(stream);
    clear_pending();
    return from_hip(gdn::launch_attn_decode(a));
}

size_t gdn_prefill_workspace_bytes_seg(int N, int T_total, int H, int HV, int dk, int dv,
                                       int chunk, int segment_chunks) {
    if (N < 0 || T_total < 0) return 0;
    if (heads_status(H, HV, dk, dv) != GDN_SUCCESS || chunk != gdn::kChunk) return 0;
    if (!valid_seg_req(segment_chunks)) return 0;
    if (N == 0 || T_total == 0) return 0;
    // the size covers bf16 inputs, the only ones that can segment
    const bool seg = gdn::prefill_may_segment(N, T_total, HV, dk, dv, true, segment_chunks);
    return gdn::prefill_layout(N, T_total, H, HV, dk, dv, seg).total;
}

size_t gdn_prefill_workspace_bytes(int N, int T_total, int H, int HV, int dk, int dv, int chunk) {
    return gdn_prefill_workspace_bytes_seg(N, T_total, H, HV, dk, dv, chunk, 0);
}

}  // extern "C"

namespace {

// Validates a prefill call and fills a.  Returns GDN_SUCCESS with *done set
// when nothing is left to launch (N == 0, or T_total == 0 after the state
// copy); workspace_need is the size the workspace must have.
gdn_status prefill_setup(const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                         const float* g, const float* beta, const int32_t* cu_seqlens, int N,
                         int T_total, const float* initial_state, float* final_state, void* o,
                         gdn_dtype o_dtype, int H, int HV, int dk, int dv, int chunk, float scale,
                         int segment_chunks, void* workspace, size_t workspace_bytes,
                         size_t workspace_need, void* stream, gdn::PrefillArgs& a, bool* done) {
    *done = true;
    if (N < 0 || T_total < 0) return GDN_ERROR_INVALID_VALUE;
    if (!valid_seg_req(segment_chunks)) return GDN_ERROR_INVALID_VALUE;
    gdn_status st = heads_status(H, HV, dk, dv);
    if (st != GDN_SUCCESS) return st;
    if (chunk != gdn::kChunk) return GDN_ERROR_NOT_SUPPORTED;
    if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype)) return GDN_ERROR_NOT_SUPPORTED;
    if (N == 0) return GDN_SUCCESS;
    if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
        return GDN_ERROR_INVALID_VALUE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t state_elems = (size_t)N * HV * dv * dk;
    if (T_total == 0) {
        if (!final_state || final_state == initial_state) return GDN_SUCCESS;
        clear_pending();
        return from_hip(gdn::launch_state_copy(initial_state, final_state, state_elems, s));
    }
    // the layout the query gives for this segment_chunks (the size covers
    // bf16 inputs; fp32 inputs never segment and use a prefix of it)
    const bool seg = gdn::prefill_may_segment(N, T_total, HV, dk, dv, true, segment_chunks);
    const gdn::PrefillLayout L = gdn::prefill_layout(N, T_total, H, HV, dk, dv, seg);
    if (workspace_need == 0) workspace_need = L.total;
    if (!q || !k || !v || !g || !beta || !cu_seqlens || !o) return GDN_ERROR_INVALID_VALUE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return GDN_ERROR_INVALID_VALUE;
    if ((size_t)L.max_chunks * HV > (size_t)(1u << 31) / (gdn::kChunk * gdn::kChunk))
        return GDN_ERROR_NOT_SUPPORTED;
    if (!workspace || workspace_bytes < workspace_need) return GDN_ERROR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN_ERROR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    a = gdn::PrefillArgs{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.cu_seqlens = cu_seqlens;
    a.s0 = initial_state; a.s_final = final_state; a.o = o;
    a.in_bf16 = in_dtype == GDN_BF16; a.o_bf16 = o_dtype == GDN_BF16;
    a.N = N; a.T = T_total; a.H = H; a.HV = HV; a.dk = dk; a.dv = dv; a.scale = scale;
    a.chunk_off = reinterpret_cast<int32_t*>(ws + L.chunk_off);
    a.ws_G = reinterpret_cast<float*>(ws + L.ws_G);
    a.ws_T = reinterpret_cast<float*>(ws + L.ws_T);
    a.ws_Rh = reinterpret_cast<uint16_t*>(ws + L.ws_Rh);
    a.ws_Rl = reinterpret_cast<uint16_t*>(ws + L.ws_Rl);
    a.ws_Zh = reinterpret_cast<uint16_t*>(ws + L.ws_Zh);
    a.ws_Zl = reinterpret_cast<uint16_t*>(ws + L.ws_Zl);
    a.ws_Tp = reinterpret_cast<uint16_t*>(ws + L.ws_Rh);
    a.max_chunks = L.max_chunks;
    a.seg_req = segment_chunks;
    a.seg_bound = L.seg_bound;
    a.corr_bound = L.corr_bound;
    a.plan = reinterpret_cast<int32_t*>(ws + L.plan);
    a.seg_seq = reinterpret_cast<int32_t*>(ws + L.seg_seq);
    a.seg_c0 = reinterpret_cast<int32_t*>(ws + L.seg_c0);
    a.seg_nch = reinterpret_cast<int32_t*>(ws + L.seg_nch);
    a.seg_idx = reinterpret_cast<int32_t*>(ws + L.seg_idx);
    a.seq_seg0 = reinterpret_cast<int32_t*>(ws + L.seq_seg0);
    a.seq_nseg = reinterpret_cast<int32_t*>(ws + L.seq_nseg);
    a.multi_seq = reinterpret_cast<int32_t*>(ws + L.multi_seq);
    a.corr_seg = reinterpret_cast<int32_t*>(ws + L.corr_seg);
    a.corr_c0 = reinterpret_cast<int32_t*>(ws + L.corr_c0);
    a.ws_E = reinterpret_cast<float*>(ws + L.ws_E);
    a.ws_Phi = reinterpret_cast<float*>(ws + L.ws_Phi);
    a.ws_Sin = reinterpret_cast<float*>(ws + L.ws_Sin);
    a.ws_W = reinterpret_cast<float*>(ws + L.ws_W);
    a.stream = s;
    *done = false;
    return GDN_SUCCESS;
}

gdn_status prefill_impl(const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                        const float* g, const float* beta, const int32_t* cu_seqlens, int N,
                        int T_total, const float* initial_state, float* final_state, void* o,
                        gdn_dtype o_dtype, int H, int HV, int dk, int dv, int chunk, float scale,
                        int segment_chunks, void* workspace, size_t workspace_bytes,
                        void* stream) {
    gdn::PrefillArgs a;
    bool done;
    const gdn_status st = prefill_setup(q, k, v, in_dtype, g, beta, cu_seqlens, N, T_total,
                                        initial_state, final_state, o, o_dtype, H, HV, dk, dv,
                                        chunk, scale, segment_chunks, workspace, workspace_bytes,
                                        0, stream, a, &done);
    if (st != GDN_SUCCESS || done) return st;
    clear_pending();
    return from_hip(gdn::launch_prefill(a));
}

// bytes of the fp32 outputs that gdn_prefill_chunked_norm keeps in its
// workspace, past the prefill's own part, when the norm is a launch of its own
size_t norm_o_bytes(int T_total, int HV, int dv) {
    return align256((size_t)T_total * HV * dv * sizeof(float));
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_chunked(const void* q, const void* k, const void* v, gdn_dtype in_dtype,
                               const float* g, const float* beta, const int32_t* cu_seqlens,
                               int N, int T_total, const float* initial_state,
                               float* final_state, void* o, gdn_dtype o_dtype, int H, int HV,
                               int dk, int dv, int chunk, float scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, in_dtype, g, beta, cu_seqlens, N, T_total, initial_state,
                        final_state, o, o_dtype, H, HV, dk, dv, chunk, scale, 0, workspace,
                        workspace_bytes, stream);
}

gdn_status gdn_prefill_chunked_seg(const void* q, const void* k, const void* v,
                                   gdn_dtype in_dtype, const float* g, const float* beta,
                                   const int32_t* cu_seqlens, int N, int T_total,
                                   const float* initial_state, float* final_state, void* o,
                                   gdn_dtype o_dtype, int H, int HV, int dk, int dv, int chunk,
                                   float scale, int segment_chunks, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, in_dtype, g, beta, cu_seqlens, N, T_total, initial_state,
                        final_state, o, o_dtype, H, HV, dk, dv, chunk, scale, segment_chunks,
                        workspace, workspace_bytes, stream);
}

gdn_status gdn_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       gdn_dtype in_dtype, const float* g, const float* beta,
                                       const int32_t* cu_seqlens, int N, int T_total,
                                       const float* initial_state, float* final_state, void* o,
                                       gdn_dtype o_dtype, int H, int HV, int dk, int dv,
                                       int chunk, float scale, void* stream) {
    // the size check is host-only and comes first: a call beyond the array
    // fails before any HIP call (sizes the prefill rejects give need == 0
    // and fail its own validation below)
    const size_t need = gdn_prefill_workspace_bytes(N, T_total, H, HV, dk, dv, chunk);
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERROR_WORKSPACE;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        clear_pending();
        const gdn_status st = from_hip(gdn::noalloc_scratch(&ws, &ws_bytes));
        if (st != GDN_SUCCESS) return st;
    }
    return prefill_impl(q, k, v, in_dtype, g, beta, cu_seqlens, N, T_total, initial_state,
                        final_state, o, o_dtype, H, HV, dk, dv, chunk, scale, 0, ws, ws_bytes,
                        stream);
}

size_t gdn_prefill_norm_workspace_bytes(int N, int T_total, int H, int HV, int dk, int dv,
                                        int chunk) {
    const size_t base = gdn_prefill_workspace_bytes(N, T_total, H, HV, dk, dv, chunk);
    return base == 0 ? 0 : base + norm_o_bytes(T_total, HV, dv);
}

gdn_status gdn_prefill_chunked_norm(const void* q, const void* k, const void* v,
                                    gdn_dtype in_dtype, const float* g, const float* beta,
                                    const int32_t* cu_seqlens, int N, int T_total,
                                    const float* initial_state, float* final_state,
                                    const void* z, gdn_dtype z_dtype, const void* w,
                                    gdn_dtype w_dtype, void* y, gdn_dtype y_dtype, void* o,
                                    gdn_dtype o_dtype, int H, int HV, int dk, int dv, int chunk,
                                    float scale, float eps, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    if (!valid_dtype(z_dtype) || !valid_dtype(w_dtype) || !valid_dtype(y_dtype))
        return GDN_ERROR_NOT_SUPPORTED;
    if (!(eps >= 0.f)) return GDN_ERROR_INVALID_VALUE;
    if (N > 0 && T_total > 0) {
        if (!z || !w || !y || !aligned16(z) || !aligned16(w) || !aligned16(y))
            return GDN_ERROR_INVALID_VALUE;
        if (o && o == y) return GDN_ERROR_INVALID_VALUE;
    }
    // the prefill writes o when it is given, else the workspace's fp32 outputs
    // (or, fused, y itself); the check of o is the prefill's own
    const size_t base = gdn_prefill_workspace_bytes(N, T_total, H, HV, dk, dv, chunk);
    const size_t need = base + (base ? norm_o_bytes(T_total, HV, dv) : 0);
    if (base && N > 0 && !o &&
        (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
        return GDN_ERROR_WORKSPACE;
    void* o_fp32 = (base && workspace) ? static_cast<char*>(workspace) + base : nullptr;
    gdn::PrefillArgs a;
    bool done;
    gdn_status st = prefill_setup(q, k, v, in_dtype, g, beta, cu_seqlens, N, T_total,
                                  initial_state, final_state, o ? o : o_fp32,
                                  o ? o_dtype : GDN_F32, H, HV, dk, dv, chunk, scale, 0, workspace,
                                  workspace_bytes, need, stream, a, &done);
    if (st != GDN_SUCCESS || done) return st;
    clear_pending();
    st = from_hip(gdn::launch_prefill(a));
    if (st != GDN_SUCCESS) return st;
    const long groups = (long)T_total * HV;
    gdn::NormArgs na{a.o, z, w, y, a.o_bf16, z_dtype == GDN_BF16, w_dtype == GDN_BF16,
                     y_dtype == GDN_BF16, groups, dv, eps, a.stream};
    return from_hip(gdn::launch_rmsnorm_gated(na));
}

gdn_status gdn_rmsnorm_gated(const void* x, gdn_dtype x_dtype, const void* z, gdn_dtype z_dtype,
                             const void* w, gdn_dtype w_dtype, void* y, gdn_dtype y_dtype,
                             int rows, int HV, int dv, float eps, void* stream) {
    if (rows < 0 || HV <= 0 || dv <= 0 || !(eps >= 0.f)) return GDN_ERROR_INVALID_VALUE;
    if (!supported_d(dv)) return GDN_ERROR_NOT_SUPPORTED;
    if (!valid_dtype(x_dtype) || !valid_dtype(z_dtype) || !valid_dtype(w_dtype) ||
        !valid_dtype(y_dtype))
        return GDN_ERROR_NOT_SUPPORTED;
    if (rows == 0) return GDN_SUCCESS;
    if (!x || !z || !w || !y) return GDN_ERROR_INVALID_VALUE;
    if (!aligned16(x) || !aligned16(z) || !aligned16(w) || !aligned16(y))
        return GDN_ERROR_INVALID_VALUE;
    if (x == y && x_dtype != y_dtype) return GDN_ERROR_INVALID_VALUE;
    const long groups = (long)rows * HV;
    if ((size_t)groups * dv >= ((size_t)1 << 40)) return GDN_ERROR_NOT_SUPPORTED;
    clear_pending();
    gdn::NormArgs a{x, z, w, y, x_dtype == GDN_BF16, z_dtype == GDN_BF16, w_dtype == GDN_BF16,
                    y_dtype == GDN_BF16, groups, dv, eps, static_cast<hipStream_t>(stream)};
    return from_hip(gdn::launch_rmsnorm_gated(a));
}

}  // extern "C"

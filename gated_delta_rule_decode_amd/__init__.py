"""libgdn -- the Gated DeltaNet token mixer on MI355X (gfx950): Python binding.

Thin ctypes marshalling over the C ABI declared in include/gdn.h.  Every step
of the computation runs in the HIP kernels of libgdn.so; torch supplies device
memory and the current stream only.  If libgdn.so is missing, every call
raises (there is no fallback path).

    decode_step(q, k, v, g, beta, state, ...)          -> o
    decode_step_norm(q, k, v, g, beta, state, z, w)    -> y (and o on request)
    decode_layer(q, k, v, state, ...)                  -> o and/or y (slot table,
                                                          raw gates, q/k L2 norm)
    prefill_chunked(q, k, v, g, beta, cu_seqlens, ...) -> (o, final_state)
    rmsnorm_gated(x, z, w, ...)                        -> y
    attn_decode(q, k_new, v_new, k_cache, v_cache, pos, ...) -> o (gated full attention)
    prefill_workspace_bytes(N, T_total, H, HV, dk, dv, chunk=64)

Layouts (row-major, contiguous): q, k [tokens, H, dk]; v [tokens, HV, dv];
g, beta [tokens, HV] fp32; state [N, HV, dv, dk] fp32; o [tokens, HV, dv].
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libgdn.so")

GDN_F32 = 0
GDN_BF16 = 1
STATUS = {0: "GDN_SUCCESS", 1: "GDN_ERROR_INVALID_VALUE", 2: "GDN_ERROR_NOT_SUPPORTED",
          3: "GDN_ERROR_WORKSPACE", 4: "GDN_ERROR_HIP"}

# every symbol include/gdn.h declares
EXPORTS = ("gdn_version", "gdn_status_string", "gdn_last_hip_error", "gdn_decode_step",
           "gdn_decode_step_norm", "gdn_decode_layer_args_size", "gdn_decode_layer",
           "gdn_prefill_workspace_bytes", "gdn_prefill_workspace_bytes_seg",
           "gdn_prefill_chunked", "gdn_prefill_chunked_seg", "gdn_prefill_chunked_noalloc",
           "gdn_prefill_norm_workspace_bytes", "gdn_prefill_chunked_norm",
           "gdn_attn_decode_args_size", "gdn_attn_decode_workspace_bytes", "gdn_attn_decode",
           "gdn_rmsnorm_gated")

__all__ = ["decode_step", "decode_step_norm", "decode_layer", "prefill_chunked",
           "prefill_chunked_norm", "rmsnorm_gated", "prefill_workspace_bytes",
           "prefill_norm_workspace_bytes", "attn_decode", "attn_decode_workspace_bytes",
           "DecodeLayerArgs", "AttnDecodeArgs", "GDNError", "lib", "LIBRARY", "EXPORTS", "version"]


class GDNError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        msg = f"{fn} returned {STATUS.get(status, status)}"
        super().__init__(msg + (f" ({detail})" if detail else ""))
        self.status = status


_LIB: Optional[ctypes.CDLL] = None
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class DecodeLayerArgs(ctypes.Structure):
    """Mirror of gdn_decode_layer_args (field order and types as in gdn.h)."""
    _fields_ = [
        ("q", _vp), ("k", _vp), ("v", _vp), ("in_dtype", _i),
        ("g", _vp), ("beta", _vp),
        ("a_raw", _vp), ("b_raw", _vp), ("gate_dtype", _i), ("A_log", _vp), ("dt_bias", _vp),
        ("qk_l2norm", _i), ("l2_eps", _f),
        ("state", _vp), ("slots", _vp), ("num_slots", _i),
        ("o", _vp), ("o_dtype", _i), ("z", _vp), ("z_dtype", _i), ("w", _vp), ("w_dtype", _i),
        ("y", _vp), ("y_dtype", _i), ("eps", _f),
        ("N", _i), ("H", _i), ("HV", _i), ("dk", _i), ("dv", _i), ("scale", _f),
    ]


class AttnDecodeArgs(ctypes.Structure):
    """Mirror of gdn_attn_decode_args (field order and types as in gdn.h)."""
    _fields_ = [
        ("q", _vp), ("gate", _vp), ("k_new", _vp), ("v_new", _vp), ("k_cache", _vp),
        ("v_cache", _vp), ("pos", _vp), ("o", _vp), ("o_dtype", _i),
        ("N", _i), ("Hq", _i), ("Hkv", _i), ("D", _i), ("Lmax", _i), ("rotary_dim", _i),
        ("rope_theta", _f), ("scale", _f), ("workspace", _vp), ("workspace_bytes", _sz),
    ]


def lib() -> ctypes.CDLL:
    """The loaded libgdn.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(f"libgdn.so is not built ({LIBRARY}); run "
                              "`python -m gated_delta_rule_decode_amd.build`")
        # torch ships its own HIP runtime (same soname, libamdhip64.so.7).
        # Loading torch first makes libgdn.so bind to that runtime; loaded the
        # other way round, the process would hold two HIP runtimes and the
        # second would find no device.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIBRARY)
        L.gdn_version.restype = _i
        L.gdn_version.argtypes = []
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_status_string.argtypes = [_i]
        L.gdn_last_hip_error.restype = ctypes.c_char_p
        L.gdn_last_hip_error.argtypes = []
        L.gdn_decode_step.restype = _i
        L.gdn_decode_step.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                      _i, _f, _vp]
        L.gdn_decode_step_norm.restype = _i
        L.gdn_decode_step_norm.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _i,
                                           _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _f, _f, _vp]
        L.gdn_decode_layer_args_size.restype = _sz
        L.gdn_decode_layer_args_size.argtypes = []
        L.gdn_decode_layer.restype = _i
        L.gdn_decode_layer.argtypes = [ctypes.POINTER(DecodeLayerArgs), _vp]
        if L.gdn_decode_layer_args_size() != ctypes.sizeof(DecodeLayerArgs):
            raise ImportError("gdn_decode_layer_args layout differs between gdn.h and the binding")
        L.gdn_attn_decode_args_size.restype = _sz
        L.gdn_attn_decode_args_size.argtypes = []
        L.gdn_attn_decode_workspace_bytes.restype = _sz
        L.gdn_attn_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
        L.gdn_attn_decode.restype = _i
        L.gdn_attn_decode.argtypes = [ctypes.POINTER(AttnDecodeArgs), _vp]
        if L.gdn_attn_decode_args_size() != ctypes.sizeof(AttnDecodeArgs):
            raise ImportError("gdn_attn_decode_args layout differs between gdn.h and the binding")
        L.gdn_prefill_workspace_bytes.restype = _sz
        L.gdn_prefill_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
        L.gdn_prefill_workspace_bytes_seg.restype = _sz
        L.gdn_prefill_workspace_bytes_seg.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
        L.gdn_prefill_chunked_seg.restype = _i
        L.gdn_prefill_chunked_seg.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _vp, _vp,
                                              _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]
        L.gdn_prefill_chunked.restype = _i
        L.gdn_prefill_chunked.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _vp, _vp,
                                          _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]
        L.gdn_prefill_chunked_noalloc.restype = _i
        L.gdn_prefill_chunked_noalloc.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _vp,
                                                  _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp]
        L.gdn_prefill_norm_workspace_bytes.restype = _sz
        L.gdn_prefill_norm_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
        L.gdn_prefill_chunked_norm.restype = _i
        L.gdn_prefill_chunked_norm.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _vp,
                                               _vp, _vp, _i, _vp, _i, _vp, _i, _vp, _i, _i, _i,
                                               _i, _i, _i, _f, _f, _vp, _sz, _vp]
        L.gdn_rmsnorm_gated.restype = _i
        L.gdn_rmsnorm_gated.argtypes = [_vp, _i, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _f, _vp]
        _LIB = L
    return _LIB


def version() -> int:
    return int(lib().gdn_version())


def _check(fn: str, status: int):
    if status != 0:
        detail = lib().gdn_last_hip_error().decode() if status == 4 else ""
        raise GDNError(fn, status, detail)


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name: str, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def decode_step(q, k, v, g, beta, state, *, o=None, scale: float = 1.0, out_dtype=None):
    """Advance N sequences by one token in place.

    q, k [N, H, dk], v [N, HV, dv] (same dtype, fp32 or bf16); g, beta [N, HV]
    fp32; state [N, HV, dv, dk] fp32 (updated in place).  Returns o [N, HV, dv]
    (fp32 unless ``out_dtype`` or a preallocated ``o`` says otherwise)."""
    torch = _torch()
    f32 = torch.float32
    N, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(g, "g", f32)
    _dev(beta, "beta", f32)
    _dev(state, "state", f32)
    if k.shape != q.shape or v.shape[0] != N or g.shape != (N, HV) or beta.shape != (N, HV) \
            or state.shape != (N, HV, dv, dk):
        raise ValueError("inconsistent decode shapes")
    if o is None:
        o = torch.empty((N, HV, dv), dtype=out_dtype or f32, device=q.device)
    _dev(o, "o")
    if o.shape != (N, HV, dv):
        raise ValueError("o shape")
    st = lib().gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta),
                               _ptr(state), _ptr(o), _dtype_code(o), N, H, HV, dk, dv,
                               float(scale), _stream(q.device))
    _check("gdn_decode_step", st)
    return o


def decode_step_norm(q, k, v, g, beta, state, z, w, *, y=None, o=None, scale: float = 1.0,
                     eps: float = 1e-6, out_dtype=None, return_o: bool = False):
    """decode_step followed by RMSNormGated of each head in one kernel.

    z [N, HV, dv] (fp32 or bf16), w [dv].  Returns y, or (y, o) with
    ``return_o`` (o is then written as well)."""
    torch = _torch()
    f32 = torch.float32
    N, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(g, "g", f32)
    _dev(beta, "beta", f32)
    _dev(state, "state", f32)
    _dev(z, "z")
    _dev(w, "w")
    if k.shape != q.shape or v.shape[0] != N or g.shape != (N, HV) or beta.shape != (N, HV) \
            or state.shape != (N, HV, dv, dk) or z.shape != (N, HV, dv) or w.shape != (dv,):
        raise ValueError("inconsistent decode shapes")
    if y is None:
        y = torch.empty((N, HV, dv), dtype=out_dtype or f32, device=q.device)
    _dev(y, "y")
    if return_o and o is None:
        o = torch.empty((N, HV, dv), dtype=f32, device=q.device)
    if o is not None:
        _dev(o, "o")
    st = lib().gdn_decode_step_norm(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta), _ptr(state), _ptr(z),
        _dtype_code(z), _ptr(w), _dtype_code(w), _ptr(y), _dtype_code(y), _ptr(o),
        _dtype_code(o) if o is not None else GDN_F32, N, H, HV, dk, dv, float(scale),
        float(eps), _stream(q.device))
    _check("gdn_decode_step_norm", st)
    return (y, o) if (return_o or o is not None) else y


def decode_layer(q, k, v, state, *, g=None, beta=None, a_raw=None, b_raw=None, A_log=None,
                 dt_bias=None, slots=None, qk_l2norm: bool = False, l2_eps: float = 1e-6,
                 z=None, w=None, y=None, o=None, scale: float = 1.0, eps: float = 1e-6,
                 out_dtype=None, return_o: bool = False):
    """The serving form of the decode step (one launch).

    state [S, HV, dv, dk] fp32 is a pool of S slots; ``slots`` [N] int32 names
    the slot of each row (None: row n uses slot n, S >= N).  Rows whose slot is
    outside [0, S) are skipped and read 0.  Gates: either ``g``/``beta`` [N, HV]
    fp32, or raw ``a_raw``/``b_raw`` [N, HV] (fp32 or bf16) with ``A_log``
    (and optionally ``dt_bias``) [HV] fp32, activated in the kernel as
    g = -exp(A_log) softplus(a_raw + dt_bias), beta = sigmoid(b_raw).
    ``qk_l2norm`` L2-normalises q and k first.  With ``z`` and ``w`` the
    result is y = RMSNormGated(o) (and o as well with ``return_o``);
    otherwise o."""
    torch = _torch()
    f32 = torch.float32
    N, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(state, "state", f32)
    if k.shape != q.shape or v.shape[0] != N or state.dim() != 4 \
            or tuple(state.shape[1:]) != (HV, dv, dk):
        raise ValueError("inconsistent decode shapes")
    a = DecodeLayerArgs()
    a.q, a.k, a.v, a.in_dtype = _ptr(q), _ptr(k), _ptr(v), _dtype_code(q)
    if a_raw is not None:
        if b_raw is None or A_log is None or g is not None or beta is not None:
            raise ValueError("raw gates need a_raw, b_raw and A_log (and no g / beta)")
        _dev(a_raw, "a_raw")
        _dev(b_raw, "b_raw", a_raw.dtype)
        _dev(A_log, "A_log", f32)
        if a_raw.shape != (N, HV) or b_raw.shape != (N, HV) or A_log.shape != (HV,):
            raise ValueError("gate shapes")
        if dt_bias is not None:
            _dev(dt_bias, "dt_bias", f32)
            if dt_bias.shape != (HV,):
                raise ValueError("dt_bias shape")
        a.a_raw, a.b_raw, a.gate_dtype = _ptr(a_raw), _ptr(b_raw), _dtype_code(a_raw)
        a.A_log, a.dt_bias = _ptr(A_log), _ptr(dt_bias)
    else:
        if g is None or beta is None:
            raise ValueError("give g and beta, or a_raw, b_raw and A_log")
        _dev(g, "g", f32)
        _dev(beta, "beta", f32)
        if g.shape != (N, HV) or beta.shape != (N, HV):
            raise ValueError("gate shapes")
        a.g, a.beta = _ptr(g), _ptr(beta)
    a.qk_l2norm, a.l2_eps = int(bool(qk_l2norm)), float(l2_eps)
    a.state, a.num_slots = _ptr(state), int(state.shape[0])
    if slots is not None:
        _dev(slots, "slots", torch.int32)
        if slots.shape != (N,):
            raise ValueError("slots shape")
        a.slots = _ptr(slots)
    norm = z is not None or w is not None
    if norm:
        if z is None or w is None:
            raise ValueError("RMSNormGated needs both z and w")
        _dev(z, "z")
        _dev(w, "w")
        if z.shape != (N, HV, dv) or w.shape != (dv,):
            raise ValueError("norm shapes")
        if y is None:
            y = torch.empty((N, HV, dv), dtype=out_dtype or f32, device=q.device)
        _dev(y, "y")
        a.z, a.z_dtype, a.w, a.w_dtype = _ptr(z), _dtype_code(z), _ptr(w), _dtype_code(w)
        a.y, a.y_dtype, a.eps = _ptr(y), _dtype_code(y), float(eps)
        if return_o and o is None:
            o = torch.empty((N, HV, dv), dtype=f32, device=q.device)
    elif o is None:
        o = torch.empty((N, HV, dv), dtype=out_dtype or f32, device=q.device)
    if o is not None:
        _dev(o, "o")
        if o.shape != (N, HV, dv):
            raise ValueError("o shape")
        a.o, a.o_dtype = _ptr(o), _dtype_code(o)
    a.N, a.H, a.HV, a.dk, a.dv, a.scale = N, H, HV, dk, dv, float(scale)
    st = lib().gdn_decode_layer(ctypes.byref(a), _stream(q.device))
    _check("gdn_decode_layer", st)
    if not norm:
        return o
    return (y, o) if (return_o or o is not None) else y


def prefill_workspace_bytes(N: int, T_total: int, H: int, HV: int, dk: int, dv: int,
                            chunk: int = 64, segment_chunks: int = 0) -> int:
    """Workspace bytes of prefill_chunked with this ``segment_chunks``."""
    return int(lib().gdn_prefill_workspace_bytes_seg(N, T_total, H, HV, dk, dv, chunk,
                                                     int(segment_chunks)))


def prefill_chunked(q, k, v, g, beta, cu_seqlens, *, initial_state=None, final_state=None,
                    o=None, scale: float = 1.0, chunk: int = 64, workspace=None,
                    out_dtype=None, return_final_state: bool = True,
                    segment_chunks: int = 0) -> Tuple:
    """Chunked prefill of a packed batch.

    q, k [T, H, dk], v [T, HV, dv]; g, beta [T, HV] fp32; cu_seqlens [N+1]
    int32 on the device; initial_state [N, HV, dv, dk] fp32 or None (zeros).
    ``segment_chunks``: 0 lets the library choose the segment-parallel scan
    (when the chains leave CUs idle), -2 also lets it segment one long prompt
    among short ones, -1 turns it off, >= 32 forces segments of that many
    chunks.
    Returns (o [T, HV, dv], final_state [N, HV, dv, dk] or None)."""
    torch = _torch()
    f32 = torch.float32
    T, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(g, "g", f32)
    _dev(beta, "beta", f32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, HV) or beta.shape != (T, HV):
        raise ValueError("inconsistent prefill shapes")
    if initial_state is not None:
        _dev(initial_state, "initial_state", f32)
        if initial_state.shape != (N, HV, dv, dk):
            raise ValueError("initial_state shape")
    if final_state is None and return_final_state:
        final_state = torch.empty((N, HV, dv, dk), dtype=f32, device=q.device)
    if final_state is not None:
        _dev(final_state, "final_state", f32)
    if o is None:
        o = torch.empty((T, HV, dv), dtype=out_dtype or f32, device=q.device)
    _dev(o, "o")
    need = prefill_workspace_bytes(N, T, H, HV, dk, dv, chunk, segment_chunks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    args = (_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
            T, _ptr(initial_state), _ptr(final_state), _ptr(o), _dtype_code(o), H, HV, dk, dv,
            chunk, float(scale))
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device))
    if segment_chunks == 0:
        st = lib().gdn_prefill_chunked(*args, *tail)
        _check("gdn_prefill_chunked", st)
    else:
        st = lib().gdn_prefill_chunked_seg(*args, int(segment_chunks), *tail)
        _check("gdn_prefill_chunked_seg", st)
    return o, final_state


def prefill_norm_workspace_bytes(N: int, T_total: int, H: int, HV: int, dk: int, dv: int,
                                 chunk: int = 64) -> int:
    return int(lib().gdn_prefill_norm_workspace_bytes(N, T_total, H, HV, dk, dv, chunk))


def prefill_chunked_norm(q, k, v, g, beta, cu_seqlens, z, w, *, initial_state=None,
                         final_state=None, y=None, o=None, scale: float = 1.0, eps: float = 1e-6,
                         chunk: int = 64, workspace=None, out_dtype=None,
                         return_final_state: bool = True, return_o: bool = False) -> Tuple:
    """prefill_chunked followed by RMSNormGated of every (token, value head).

    z [T, HV, dv] (fp32 or bf16), w [dv].  Returns (y, final_state), or
    (y, final_state, o) with ``return_o`` (o is then written as well)."""
    torch = _torch()
    f32 = torch.float32
    T, H, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name, q.dtype)
    _dev(g, "g", f32)
    _dev(beta, "beta", f32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(z, "z")
    _dev(w, "w")
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, HV) or beta.shape != (T, HV) \
            or z.shape != (T, HV, dv) or w.shape != (dv,):
        raise ValueError("inconsistent prefill shapes")
    if initial_state is not None:
        _dev(initial_state, "initial_state", f32)
        if initial_state.shape != (N, HV, dv, dk):
            raise ValueError("initial_state shape")
    if final_state is None and return_final_state:
        final_state = torch.empty((N, HV, dv, dk), dtype=f32, device=q.device)
    if final_state is not None:
        _dev(final_state, "final_state", f32)
    if y is None:
        y = torch.empty((T, HV, dv), dtype=out_dtype or f32, device=q.device)
    _dev(y, "y")
    if return_o and o is None:
        o = torch.empty((T, HV, dv), dtype=f32, device=q.device)
    if o is not None:
        _dev(o, "o")
    need = prefill_norm_workspace_bytes(N, T, H, HV, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    st = lib().gdn_prefill_chunked_norm(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, T,
        _ptr(initial_state), _ptr(final_state), _ptr(z), _dtype_code(z), _ptr(w), _dtype_code(w),
        _ptr(y), _dtype_code(y), _ptr(o), _dtype_code(o) if o is not None else GDN_F32, H, HV, dk,
        dv, chunk, float(scale), float(eps), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q.device))
    _check("gdn_prefill_chunked_norm", st)
    return (y, final_state, o) if (return_o or o is not None) else (y, final_state)


def attn_decode_workspace_bytes(N: int, Hq: int, Hkv: int, D: int, Lmax: int) -> int:
    return int(lib().gdn_attn_decode_workspace_bytes(N, Hq, Hkv, D, Lmax))


def attn_decode(q, k_new, v_new, k_cache, v_cache, pos, *, gate=None, o=None,
                rotary_dim: int = 64, rope_theta: float = 1e7, scale=None, out_dtype=None,
                workspace=None):
    """One decode step of gated full attention; appends the new key (rotated)
    and value to the caches at row pos[n].

    q (and gate) [N, Hq, D] bf16; k_new, v_new [N, Hkv, D] bf16; caches
    [N, Hkv, Lmax, D] bf16 (keys stored rotated); pos [N] int32 on the device.
    Returns o [N, Hq, D] (fp32 unless ``out_dtype`` or ``o`` says otherwise)."""
    torch = _torch()
    bf = torch.bfloat16
    N, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _dev(t, name, bf)
    _dev(pos, "pos", torch.int32)
    if k_new.shape != (N, Hkv, D) or v_new.shape != k_new.shape \
            or k_cache.shape != (N, Hkv, Lmax, D) or v_cache.shape != k_cache.shape \
            or pos.shape != (N,):
        raise ValueError("inconsistent attention shapes")
    if gate is not None:
        _dev(gate, "gate", bf)
        if gate.shape != q.shape:
            raise ValueError("gate shape")
    if o is None:
        o = torch.empty((N, Hq, D), dtype=out_dtype or torch.float32, device=q.device)
    _dev(o, "o")
    if workspace is None:
        need = attn_decode_workspace_bytes(N, Hq, Hkv, D, Lmax)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    a = AttnDecodeArgs()
    a.q, a.gate, a.k_new, a.v_new = _ptr(q), _ptr(gate), _ptr(k_new), _ptr(v_new)
    a.k_cache, a.v_cache, a.pos, a.o, a.o_dtype = (_ptr(k_cache), _ptr(v_cache), _ptr(pos),
                                                  _ptr(o), _dtype_code(o))
    a.N, a.Hq, a.Hkv, a.D, a.Lmax, a.rotary_dim = N, Hq, Hkv, D, Lmax, int(rotary_dim)
    a.rope_theta = float(rope_theta)
    a.scale = float(D ** -0.5 if scale is None else scale)
    a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = lib().gdn_attn_decode(ctypes.byref(a), _stream(q.device))
    _check("gdn_attn_decode", st)
    return o


def rmsnorm_gated(x, z, w, *, y=None, eps: float = 1e-6, out_dtype=None):
    """y = x / sqrt(mean(x^2) + eps) * w * silu(z) over the last axis (dv).

    x, z [..., HV, dv]; w [dv]; y may be x itself (in place) if dtypes match."""
    torch = _torch()
    _dev(x, "x")
    _dev(z, "z")
    _dev(w, "w")
    dv = x.shape[-1]
    HV = x.shape[-2] if x.dim() >= 2 else 1
    rows = x.numel() // (HV * dv) if x.numel() else 0
    if z.shape != x.shape or w.shape != (dv,):
        raise ValueError("inconsistent norm shapes")
    if y is None:
        y = torch.empty(x.shape, dtype=out_dtype or torch.float32, device=x.device)
    _dev(y, "y")
    if y.shape != x.shape:
        raise ValueError("y shape")
    st = lib().gdn_rmsnorm_gated(_ptr(x), _dtype_code(x), _ptr(z), _dtype_code(z), _ptr(w),
                                 _dtype_code(w), _ptr(y), _dtype_code(y), rows, HV, dv,
                                 float(eps), _stream(x.device))
    _check("gdn_rmsnorm_gated", st)
    return y

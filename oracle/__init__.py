"""fp64 CPU oracle for the Gated DeltaNet token mixer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The library's product path never does, and the
oracle imports nothing from the library: the two share no code.  The only
module both sides use is ``gdn_inputs``, which draws the seeded inputs.

The arithmetic lives in ``gdn_oracle.c`` (plain loops in double; see its
header for the definitions and the passages of the pages they follow).  This
wrapper builds it with gcc, loads it with ctypes and marshals numpy arrays.

Functions
  recurrence(...)   the plain step-by-step gated delta rule over a packed batch
  decode(...)       one token per sequence: the same loop with T = N
  rmsnorm_gated(...) y = x / sqrt(mean(x^2) + eps) * w * silu(z)
  gates(...)        g = -exp(A_log) softplus(a_raw + dt_bias), beta = sigmoid(b_raw)
  l2norm(...)       x / sqrt(sum x^2 + eps) per row
  decode_layer(...) one token per sequence against a slot-addressed state pool,
                    optionally with q/k L2-normalised first
  rope(...)         rotary embedding on the first rd dimensions (rotate-half pairs)
  attn_decode(...)  one decode step of gated full attention over a KV cache

Pinned by tests/test_oracle_pins.py (closed forms and invariants) and
tests/test_oracle_mutations.py (planted mistakes fail a pin).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_DIR, "gdn_oracle.c")
LIBRARY = os.path.join(_DIR, "libgdn_oracle.so")

__all__ = ["build", "load", "Oracle", "SOURCE", "LIBRARY"]


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", *extra_flags, source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)


def _ptr(a: Optional[np.ndarray], t):
    if a is None:
        return ctypes.cast(None, t)
    return a.ctypes.data_as(t)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


class Oracle:
    """A loaded oracle library (the default build, or e.g. a mutated copy)."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.gdn_oracle_recurrence.restype = ctypes.c_int
        lib.gdn_oracle_recurrence.argtypes = [
            _f32p, _f32p, _f32p, _f32p, _f32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, _f64p, _f64p, _f64p, ctypes.c_int]
        lib.gdn_oracle_rmsnorm_gated.restype = ctypes.c_int
        lib.gdn_oracle_rmsnorm_gated.argtypes = [
            _f64p, _f32p, _f32p, ctypes.c_long, ctypes.c_int, ctypes.c_double, _f64p]
        lib.gdn_oracle_max_threads.restype = ctypes.c_int
        lib.gdn_oracle_gates.restype = ctypes.c_int
        lib.gdn_oracle_gates.argtypes = [_f32p, _f32p, _f32p, _f32p, ctypes.c_long, ctypes.c_int,
                                         _f64p, _f64p]
        lib.gdn_oracle_l2norm.restype = ctypes.c_int
        lib.gdn_oracle_l2norm.argtypes = [_f32p, ctypes.c_long, ctypes.c_int, ctypes.c_double,
                                          _f64p]
        lib.gdn_oracle_decode_layer.restype = ctypes.c_int
        lib.gdn_oracle_decode_layer.argtypes = [
            _f32p, _f32p, _f32p, _f64p, _f64p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
            ctypes.c_double, _f64p, _f64p, ctypes.c_int]
        lib.gdn_oracle_rope.restype = ctypes.c_int
        lib.gdn_oracle_rope.argtypes = [_f32p, _i32p, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_double, _f64p]
        lib.gdn_oracle_attn_decode.restype = ctypes.c_int
        lib.gdn_oracle_attn_decode.argtypes = [
            _f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _i32p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
            ctypes.c_double, _f64p, _f64p]
        self._lib = lib

    def max_threads(self) -> int:
        return int(self._lib.gdn_oracle_max_threads())

    def recurrence(self, q, k, v, g, beta, cu_seqlens, *, scale: float = 1.0,
                   s0=None, threads: int = 0):
        """Packed-batch recurrence.

        q, k: [T, H, dk]; v: [T, HV, dv]; g, beta: [T, HV]; cu_seqlens: [N+1];
        s0: [N, HV, dv, dk] or None.  Returns (o [T, HV, dv], S [N, HV, dv, dk])
        in float64.
        """
        q, k, v, g, beta = _f32(q), _f32(k), _f32(v), _f32(g), _f32(beta)
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        T, H, dk = q.shape
        HV, dv = v.shape[1], v.shape[2]
        N = len(cu) - 1
        if k.shape != q.shape or v.shape[0] != T or g.shape != (T, HV) or beta.shape != (T, HV):
            raise ValueError("inconsistent shapes")
        if N < 0 or (N >= 0 and (cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0))):
            raise ValueError("cu_seqlens must run from 0 to T, non-decreasing")
        s0d = None
        if s0 is not None:
            s0d = np.ascontiguousarray(s0, dtype=np.float64)
            if s0d.shape != (N, HV, dv, dk):
                raise ValueError("s0 shape")
        o = np.zeros((T, HV, dv), dtype=np.float64)
        S = np.empty((N, HV, dv, dk), dtype=np.float64)
        rc = self._lib.gdn_oracle_recurrence(
            _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p), _ptr(g, _f32p), _ptr(beta, _f32p),
            _ptr(cu, _i32p), N, H, HV, dk, dv, float(scale), _ptr(s0d, _f64p), _ptr(o, _f64p),
            _ptr(S, _f64p), int(threads))
        if rc != 0:
            raise RuntimeError("oracle recurrence failed")
        return o, S

    def decode(self, q, k, v, g, beta, state, *, scale: float = 1.0, threads: int = 0):
        """One token per sequence.  q, k: [N, H, dk]; v: [N, HV, dv];
        g, beta: [N, HV]; state: [N, HV, dv, dk].  Returns (o, new_state)."""
        N = q.shape[0]
        cu = np.arange(N + 1, dtype=np.int32)
        return self.recurrence(q, k, v, g, beta, cu, scale=scale, s0=state, threads=threads)

    def rmsnorm_gated(self, x, z, w, *, eps: float = 1e-6):
        """Groups are the last axis of x and z ([..., dv]); w: [dv]."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        z = _f32(z)
        w = _f32(w)
        dv = x.shape[-1]
        if z.shape != x.shape or w.shape != (dv,):
            raise ValueError("shapes")
        y = np.empty_like(x)
        rc = self._lib.gdn_oracle_rmsnorm_gated(_ptr(x, _f64p), _ptr(z, _f32p), _ptr(w, _f32p),
                                                x.size // dv, dv, float(eps), _ptr(y, _f64p))
        if rc != 0:
            raise RuntimeError("oracle rmsnorm failed")
        return y

    def gates(self, a_raw, b_raw, A_log, dt_bias=None):
        """a_raw, b_raw: [..., HV]; A_log, dt_bias: [HV].  Returns (g, beta) in
        float64 with the shape of a_raw."""
        a_raw, b_raw, A_log = _f32(a_raw), _f32(b_raw), _f32(A_log)
        HV = A_log.shape[0]
        if a_raw.shape != b_raw.shape or a_raw.shape[-1:] != (HV,):
            raise ValueError("shapes")
        dt = None if dt_bias is None else _f32(dt_bias)
        if dt is not None and dt.shape != (HV,):
            raise ValueError("dt_bias shape")
        g = np.empty(a_raw.shape, dtype=np.float64)
        beta = np.empty(a_raw.shape, dtype=np.float64)
        rc = self._lib.gdn_oracle_gates(_ptr(a_raw, _f32p), _ptr(b_raw, _f32p),
                                        _ptr(A_log, _f32p), _ptr(dt, _f32p), a_raw.size // HV,
                                        HV, _ptr(g, _f64p), _ptr(beta, _f64p))
        if rc != 0:
            raise RuntimeError("oracle gates failed")
        return g, beta

    def l2norm(self, x, *, eps: float = 1e-6):
        """Rows are the last axis of x; returns float64."""
        x = _f32(x)
        d = x.shape[-1]
        y = np.empty(x.shape, dtype=np.float64)
        rc = self._lib.gdn_oracle_l2norm(_ptr(x, _f32p), x.size // d, d, float(eps),
                                         _ptr(y, _f64p))
        if rc != 0:
            raise RuntimeError("oracle l2norm failed")
        return y

    def decode_layer(self, q, k, v, g, beta, pool, *, slots=None, scale: float = 1.0,
                     l2norm: bool = False, l2_eps: float = 1e-6, threads: int = 0):
        """One token per sequence against a state pool.

        q, k: [N, H, dk]; v: [N, HV, dv]; g, beta: [N, HV] (any float type,
        used in float64); pool: [S, HV, dv, dk]; slots: [N] int32 or None
        (sequence n -> slot n).  Returns (o [N, HV, dv], new_pool) in float64;
        sequences whose slot lies outside [0, S) get o = 0 and touch no state."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        g = np.ascontiguousarray(g, dtype=np.float64)
        beta = np.ascontiguousarray(beta, dtype=np.float64)
        pool = np.array(pool, dtype=np.float64, copy=True, order="C")
        N, H, dk = q.shape
        HV, dv = v.shape[1], v.shape[2]
        if k.shape != q.shape or v.shape[0] != N or g.shape != (N, HV) or beta.shape != (N, HV):
            raise ValueError("inconsistent shapes")
        if pool.ndim != 4 or pool.shape[1:] != (HV, dv, dk):
            raise ValueError("pool shape")
        sl = None if slots is None else np.ascontiguousarray(slots, dtype=np.int32)
        if sl is not None and sl.shape != (N,):
            raise ValueError("slots shape")
        o = np.full((N, HV, dv), np.nan, dtype=np.float64)  # every element is written
        rc = self._lib.gdn_oracle_decode_layer(
            _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p), _ptr(g, _f64p), _ptr(beta, _f64p),
            _ptr(sl, _i32p), pool.shape[0], N, H, HV, dk, dv, float(scale), int(bool(l2norm)),
            float(l2_eps), _ptr(pool, _f64p), _ptr(o, _f64p), int(threads))
        if rc != 0:
            raise RuntimeError("oracle decode_layer failed (sizes, or a slot used twice)")
        return o, pool

    def rope(self, x, pos, *, rd: int, theta: float):
        """x: [..., d] float; pos: integer array with x's leading shape."""
        x = _f32(x)
        d = x.shape[-1]
        p = np.ascontiguousarray(np.broadcast_to(pos, x.shape[:-1]), dtype=np.int32)
        y = np.empty(x.shape, dtype=np.float64)
        rc = self._lib.gdn_oracle_rope(_ptr(x, _f32p), _ptr(p, _i32p), x.size // d, d, int(rd),
                                       float(theta), _ptr(y, _f64p))
        if rc != 0:
            raise RuntimeError("oracle rope failed")
        return y

    def attn_decode(self, q, knew, vnew, k_cache, v_cache, pos, *, gate=None, rd: int = 64,
                    theta: float = 1e7, scale: float = 1.0):
        """q (and gate): [N, Hq, d]; knew, vnew: [N, Hkv, d]; caches [N, Hkv, Lmax, d]
        (rows t < pos[n] valid, keys rotated); pos: [N].  Returns (o [N, Hq, d],
        rotated new key [N, Hkv, d]) in float64."""
        q, knew, vnew = _f32(q), _f32(knew), _f32(vnew)
        kc, vc = _f32(k_cache), _f32(v_cache)
        g = None if gate is None else _f32(gate)
        N, Hq, d = q.shape
        Hkv, Lmax = kc.shape[1], kc.shape[2]
        p = np.ascontiguousarray(pos, dtype=np.int32)
        if knew.shape != (N, Hkv, d) or vnew.shape != knew.shape or kc.shape != (N, Hkv, Lmax, d) \
                or vc.shape != kc.shape or p.shape != (N,) or (g is not None and g.shape != q.shape):
            raise ValueError("shapes")
        o = np.full((N, Hq, d), np.nan)
        kr = np.full((N, Hkv, d), np.nan)
        rc = self._lib.gdn_oracle_attn_decode(
            _ptr(q, _f32p), _ptr(g, _f32p), _ptr(knew, _f32p), _ptr(vnew, _f32p), _ptr(kc, _f32p),
            _ptr(vc, _f32p), _ptr(p, _i32p), N, Hq, Hkv, d, Lmax, int(rd), float(theta),
            float(scale), _ptr(o, _f64p), _ptr(kr, _f64p))
        if rc != 0:
            raise RuntimeError("oracle attn_decode failed")
        return o, kr


_DEFAULT: Optional[Oracle] = None


def load(path: Optional[str] = None) -> Oracle:
    """Load the oracle (building it first if no library exists or the source
    is newer than the library)."""
    global _DEFAULT
    if path is not None:
        return Oracle(path)
    if _DEFAULT is None:
        if (not os.path.exists(LIBRARY)
                or os.path.getmtime(SOURCE) > os.path.getmtime(LIBRARY)):
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT

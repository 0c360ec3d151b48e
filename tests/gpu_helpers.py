"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its binding, call the oracle on the same inputs, and measure
the difference.

Tolerances (bf16 inputs, fp32 state; fixed for this mixer): output rel-L2
<= 2e-3 over the whole output tensor and final-state max-abs <= 1e-3 over the
whole state tensor.  rel-L2 = |o_gpu - o_ref|_2 / |o_ref|_2.
"""
from __future__ import annotations

import sys

import numpy as np

O_REL_L2 = 2e-3
S_MAX_ABS = 1e-3
# fp32 inputs leave only fp32 rounding in the kernels: a much tighter bar
O_REL_L2_F32 = 2e-5
S_MAX_ABS_F32 = 2e-5


def say(msg: str):
    """Name the case before a GPU step, flushed, so a fault still says which."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(name: str):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def rel_l2(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(a - ref)
    return float(num / den) if den > 0 else float(num)


def max_abs(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(a - ref))) if a.size else 0.0


def gpu_prefill(x, *, scale=1.0, s0=None, out_dtype=None, final=True, segment_chunks=0):
    """Run gdn_prefill_chunked on PrefillInputs x; returns torch tensors."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    dt = torch_dtype(x.dtype)
    q, k, v = dev(x.q, dt), dev(x.k, dt), dev(x.v, dt)
    g, b = dev(x.g), dev(x.beta)
    cu = dev(x.cu_seqlens.astype(np.int32))
    init = None
    if s0 is not None:
        init = s0 if isinstance(s0, torch.Tensor) else dev(np.asarray(s0, np.float32))
    elif x.s0 is not None:
        init = dev(x.s0)
    o, S = gdn.prefill_chunked(q, k, v, g, b, cu, initial_state=init, scale=scale,
                               out_dtype=out_dtype, return_final_state=final,
                               segment_chunks=segment_chunks)
    return o, S


def oracle_prefill(orc, x, *, scale=1.0, s0=None):
    if s0 is None:
        s0 = x.s0
    return orc.recurrence(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, scale=scale, s0=s0)


def assert_parity(o_gpu, S_gpu, o_ref, S_ref, *, f32=False, what=""):
    ro = rel_l2(o_gpu, o_ref)
    ms = max_abs(S_gpu, S_ref) if S_ref is not None else 0.0
    tol_o = O_REL_L2_F32 if f32 else O_REL_L2
    tol_s = S_MAX_ABS_F32 if f32 else S_MAX_ABS
    print(f"[parity] {what}: o rel-L2 {ro:.3e} (<= {tol_o:.0e}), state max-abs {ms:.3e} "
          f"(<= {tol_s:.0e})", flush=True)
    assert ro <= tol_o, f"{what}: output rel-L2 {ro:.3e} > {tol_o:.0e}"
    assert ms <= tol_s, f"{what}: final-state max-abs {ms:.3e} > {tol_s:.0e}"
    return ro, ms

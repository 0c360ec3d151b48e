"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its binding, call the oracle on the same inputs, and measure
the difference.

Tolerances (bf16 inputs, fp32 state; fixed for this mixer): output rel-L2
<= 2e-3 over the whole output tensor and final-state max-abs <= 1e-3 over the
whole state tensor.  rel-L2 = |o_gpu - o_ref|_2 / |o_ref|_2.

The whole-tensor figure can hide one bad (sequence, head) or one bad row in a
large batch, so every comparison also takes, per (sequence, value head), the
rel-L2 of its outputs and the worst error of one output row (one token's d_v
values) against the RMS row norm of that (sequence, head), and bounds both:
a wrong head or a wrong row scores near 1, correct ones near the whole-tensor
figure.
"""
from __future__ import annotations

import sys

import numpy as np

O_REL_L2 = 2e-3
S_MAX_ABS = 1e-3
# fp32 inputs leave only fp32 rounding in the kernels: a much tighter bar
O_REL_L2_F32 = 2e-5
S_MAX_ABS_F32 = 2e-5
# worst (sequence, head) rel-L2 and worst row error over its head's RMS row norm
O_HEAD_REL = 1e-2
O_HEAD_REL_F32 = 1e-4


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


class HeadErrors:
    """Running worst per-(sequence, head) errors; feed it one sequence (or the
    whole batch) at a time, so large outputs are never held whole in fp64."""

    def __init__(self):
        self.head_rel = 0.0      # worst rel-L2 of one (sequence, head)'s outputs
        self.row_rel = 0.0       # worst row error / RMS row norm of its (sequence, head)
        self.state_abs = 0.0     # worst max-abs of one (sequence, head)'s final state
        self.where = {}

    def outputs(self, o, ref, seq_offset=0, layout="tokens"):
        """o, ref: [rows, HV, dv] (one sequence) or [steps, N, HV, dv] (a decode
        chain, grouped per sequence n over its steps)."""
        o = np.asarray(o, np.float64)
        ref = np.asarray(ref, np.float64)
        if o.size == 0:
            return
        if layout == "steps":  # [steps, N, HV, dv] -> groups (n, h) over steps
            err2 = np.sum((o - ref) ** 2, axis=-1)   # [steps, N, HV]
            ref2 = np.sum(ref ** 2, axis=-1)
            rows = o.shape[0]
            num = np.sqrt(err2.sum(axis=0))           # [N, HV]
            den = np.sqrt(ref2.sum(axis=0))
            rms = np.sqrt(ref2.sum(axis=0) / rows)
            row = np.sqrt(err2).max(axis=0)
        else:                  # [rows, HV, dv] of one sequence -> groups (h,)
            err2 = np.sum((o - ref) ** 2, axis=-1)   # [rows, HV]
            ref2 = np.sum(ref ** 2, axis=-1)
            rows = o.shape[0]
            num = np.sqrt(err2.sum(axis=0))[None]     # [1, HV]
            den = np.sqrt(ref2.sum(axis=0))[None]
            rms = np.sqrt(ref2.sum(axis=0) / rows)[None]
            row = np.sqrt(err2).max(axis=0)[None]
        with np.errstate(divide="ignore", invalid="ignore"):
            hr = np.where(den > 0, num / np.where(den > 0, den, 1), num)
            rr = np.where(rms > 0, row / np.where(rms > 0, rms, 1), row)
        i = np.unravel_index(int(np.argmax(hr)), hr.shape)
        if hr[i] > self.head_rel:
            self.head_rel = float(hr[i])
            self.where["head_rel"] = (int(i[0]) + seq_offset, int(i[1]))
        j = np.unravel_index(int(np.argmax(rr)), rr.shape)
        if rr[j] > self.row_rel:
            self.row_rel = float(rr[j])
            self.where["row_rel"] = (int(j[0]) + seq_offset, int(j[1]))

    def state(self, S, ref, seq_offset=0):
        """S, ref: [N, HV, dv, dk]."""
        S = np.asarray(S, np.float64)
        ref = np.asarray(ref, np.float64)
        if S.size == 0:
            return
        m = np.abs(S - ref).reshape(S.shape[0], S.shape[1], -1).max(axis=-1)
        i = np.unravel_index(int(np.argmax(m)), m.shape)
        if m[i] > self.state_abs:
            self.state_abs = float(m[i])
            self.where["state_abs"] = (int(i[0]) + seq_offset, int(i[1]))

    def check(self, *, f32=False, what=""):
        tol_h = O_HEAD_REL_F32 if f32 else O_HEAD_REL
        tol_s = S_MAX_ABS_F32 if f32 else S_MAX_ABS
        print(f"[parity] {what}: worst (seq, head) o rel-L2 {self.head_rel:.3e} at "
              f"{self.where.get('head_rel')}, worst row / head RMS {self.row_rel:.3e} at "
              f"{self.where.get('row_rel')}, worst (seq, head) state max-abs "
              f"{self.state_abs:.3e} at {self.where.get('state_abs')} "
              f"(<= {tol_h:.0e}, {tol_h:.0e}, {tol_s:.0e})", flush=True)
        assert self.head_rel <= tol_h, f"{what}: (seq, head) rel-L2 {self.head_rel:.3e} > {tol_h:.0e}"
        assert self.row_rel <= tol_h, f"{what}: row error {self.row_rel:.3e} > {tol_h:.0e}"
        assert self.state_abs <= tol_s, f"{what}: state max-abs {self.state_abs:.3e} > {tol_s:.0e}"


def head_errors(o_gpu, o_ref, S_gpu=None, S_ref=None, *, cu=None) -> HeadErrors:
    """Per-(sequence, head) errors of a whole result.  o: [T, HV, dv] packed
    tokens with cu_seqlens ``cu`` (None: one sequence), or [steps, N, HV, dv]
    (a decode chain)."""
    e = HeadErrors()
    o_gpu = np.asarray(o_gpu)
    if o_gpu.ndim == 4:
        e.outputs(o_gpu, o_ref, layout="steps")
    else:
        cu = [0, o_gpu.shape[0]] if cu is None else [int(c) for c in cu]
        for n in range(len(cu) - 1):
            e.outputs(o_gpu[cu[n]:cu[n + 1]], np.asarray(o_ref)[cu[n]:cu[n + 1]], seq_offset=n)
    if S_ref is not None:
        e.state(S_gpu, S_ref)
    return e


def assert_parity(o_gpu, S_gpu, o_ref, S_ref, *, f32=False, what="", cu=None):
    """Whole-tensor bars, then the per-(sequence, head) bars (o as for
    head_errors: [T, HV, dv] with ``cu``, or [steps, N, HV, dv])."""
    ro = rel_l2(o_gpu, o_ref)
    ms = max_abs(S_gpu, S_ref) if S_ref is not None else 0.0
    tol_o = O_REL_L2_F32 if f32 else O_REL_L2
    tol_s = S_MAX_ABS_F32 if f32 else S_MAX_ABS
    print(f"[parity] {what}: o rel-L2 {ro:.3e} (<= {tol_o:.0e}), state max-abs {ms:.3e} "
          f"(<= {tol_s:.0e})", flush=True)
    assert ro <= tol_o, f"{what}: output rel-L2 {ro:.3e} > {tol_o:.0e}"
    assert ms <= tol_s, f"{what}: final-state max-abs {ms:.3e} > {tol_s:.0e}"
    head_errors(o_gpu, o_ref, S_gpu, S_ref, cu=cu).check(f32=f32, what=what)
    return ro, ms

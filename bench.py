"""Benchmark of the Gated DeltaNet token mixer (libgdn) on one MI355X.

Default workload (one "step"): the Qwen3.6-35B-A3B DeltaNet job, 16 key/query
heads shared by 32 value heads (two value heads per key head: the Core AI
card for Qwen3.6-35B-A3B, introduction), d_k = d_v = 128, bf16 q/k/v, fp32
state, over 4 layer-states (4 x 256 MiB of decode state, beyond the 256 MB
Infinity Cache).  Per layer-state:

  * prefill: a packed batch of 2 x 8192-token prompts from zero states,
    followed by RMSNormGated of every output (gdn_prefill_chunked_norm);
  * seeding: decode row n starts from the prefill's final state n mod 2
    (a device gather of the two states into the 128-row decode batch);
  * decode: 128 steps at batch 128, decode + RMSNormGated in one kernel
    (gdn_decode_step_norm), each step advancing all 4 layer-states.

Every layer-state has its own inputs, all resident in HBM before timing
starts; each phase's launches are captured once in a HIP graph and replayed.
``value`` = tokens per second per DeltaNet layer over the whole job:
4 x (2 x 8192 + 128 x 128) tokens / job time.  The line also carries the
decode kernel's HBM roofline, the prefill call's HBM and MFMA fractions, the
long-context varlen prefill at its 131,072-token cap (8 packed sequences,
32 value heads, nonzero initial states) as a phase, and the fp64 oracle timed
on the host cores on a sample of the job.

    python bench.py [--steps K] [--warmup W]
                    [--workload job35b|job08b|prefill2|prefill3|prefill4|prefill4cap|prefill5|
                                decode3|serve|attn|norm|copy]

``job08b`` is the Qwen3.5-0.8B DeltaNet job over its 18 DeltaNet layers (18 of
24 layers; Qwen3.5-0.8B chat guide, section "Architektur"): 32 sequences,
16 key/query and 16 value heads, a 512-token prefill + RMSNormGated per
sequence, then 256 decode + RMSNormGated steps.

``prefill2|3|4|4cap|5`` time one prefill call per workload (4 x 4096 tokens at
the 0.8B shape; 2 x 8192 at the 35B-A3B shape; the long-context varlen draw;
the same at its 131,072-token cap; one 32768-token prompt) with the library's
own choice of scan and with segmentation off.

``decode3`` times the decode step alone at the 35B-A3B shape (batch 128, 4
layer-states).  ``serve`` times the serving form (gdn_decode_layer: 128 rows
from a pool of 256 slots, raw bf16 gates, q/k L2 norm, RMSNormGated; 30
DeltaNet layers).  ``attn`` times one decode step of the gated full-attention
layers of Qwen3.6-35B-A3B (16 query over 2 key/value heads, head_dim 256, a
quarter rotated, theta 1e7; 128 rows at position 8192).  ``norm`` times
RMSNormGated on its own.  ``copy`` is the calibration copy for the traffic
counters.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN tokens/s (prefill, decode) + % HBM/MFMA roofline, 1×MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector / matrix, TFLOP/s


# HBM traffic of the dominant kernel (fused decode + RMSNormGated, 0.8B decode
# job shape) from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by the same
# counters read for a copy of known size; recorded in
# profiles/decode_traffic_qwen35_08b.md together with the sha256 of the kernel
# source (and the local headers it includes) it was measured on.  Reported only
# while those sources are unchanged.
DECODE_TRAFFIC = {"kernel_source_sha256": "076fd1460782135513e283e43e4305599738b27696c883c62b2e249ee88187c7",
                  "bytes_per_launch": 68036973}


# The same for the serving decode step (gdn_decode.hip, 35B-A3B serving shape;
# profiles/serving_decode_traffic.md) and the attention decode step
# (gdn_attn.hip, split + combine kernels; profiles/attention_decode_traffic.md).
SERVE_TRAFFIC = {"kernel_source_sha256": "076fd1460782135513e283e43e4305599738b27696c883c62b2e249ee88187c7",
                 "bytes_per_launch": 543596916}
ATTN_TRAFFIC = {"kernel_source_sha256": "b4c7bd0b8563d7f0d784dc692deadbfa4d08b1b3b87439910dda3ff64a06dbdf",
                "bytes_per_launch": 2197192926}
# The fused decode at the 35B-A3B shape, batch 128 (gdn_decode.hip;
# profiles/decode_traffic_35b.md)
DECODE3_TRAFFIC = {"kernel_source_sha256": "076fd1460782135513e283e43e4305599738b27696c883c62b2e249ee88187c7",
                   "bytes_per_launch": 543826119}
# RMSNormGated on its own (gdn_rmsnorm.hip, 0.8B prefill output shape;
# profiles/rmsnorm_gated_traffic.md)
NORM_TRAFFIC = {"kernel_source_sha256": "8bba89fa6e221f323599e1e67999eda741660ccbc6dc39ab4157f42bfae53472",
                "bytes_per_launch": 335594827}


# Prefill counters from rocprofv3 runs of the bench lines (per call: issued
# bf16 MFMA flops from SQ_INSTS_VALU_MFMA_MOPS_BF16, and HBM bytes from
# FETCH_SIZE / WRITE_SIZE scaled by the copy calibration), keyed on the
# prefill kernel sources they were measured on (profiles/
# prefill_traffic_and_mfma.md).  The job's prefill call is workload 3's shape
# without an initial state, the cap phase is prefill4cap's.
PREFILL_SOURCES = ("gdn_prefill_mfma.hip", "gdn_prefill_tp.hip")
PREFILL_COUNTERS = {
    "kernel_source_sha256": "4ca8b49a8eaa23df991969aab3cdd2ae563bacb10cd19d39e94127e5e642e38c",
    "issued_mfma_flops": {"prefill2": 86704652288, "prefill3": 170724950016,
                          "prefill4cap": 1367133388800, "job35b": 170724950016,
                          "cap": 1367133388800},
    "traffic_bytes": {"prefill2": 512143287, "prefill3": 818358760, "prefill4cap": 6544831466,
                      "job35b": 818358760, "cap": 6544831466}}


def recorded(record, source):
    """A counter record when its kernel sources are unchanged, else None."""
    ok = record.get("kernel_source_sha256") == kernel_sources_sha256(source)
    return record if ok else None


def kernel_sources_sha256(source):
    """sha256 over a kernel source (or a tuple of them) and the local headers
    they include (and theirs), in include order."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "gated_delta_rule_decode_amd", "csrc")
    h, seen = hashlib.sha256(), []

    def visit(name):
        if name in seen or not os.path.exists(os.path.join(csrc, name)):
            return
        seen.append(name)
        with open(os.path.join(csrc, name), "rb") as f:
            data = f.read()
        h.update(data)
        for inc in re.findall(rb'#include "([^"]+)"', data):
            visit(inc.decode())

    for src in (source if isinstance(source, tuple) else (source,)):
        visit(src)
    return h.hexdigest()


def measured_traffic(record=None, source="gdn_decode.hip"):
    record = record or DECODE_TRAFFIC
    ok = kernel_sources_sha256(source) == record["kernel_source_sha256"]
    return record["bytes_per_launch"] if ok else None


def copy_same_bytes(nbytes, copies=18, reps=16):
    """A plain device copy (torch's copy_) moving the same bytes as one launch:
    nbytes read and nbytes written, over `copies` rotating buffer pairs, captured
    in a HIP graph and timed like the launches it is compared with."""
    import torch
    n = nbytes // 4
    src = [torch.randn(n, device="cuda") for _ in range(copies)]
    dst = [torch.empty(n, device="cuda") for _ in range(copies)]

    def run():
        for _ in range(reps):
            for a, b in zip(src, dst):
                b.copy_(a)

    g, s = graph_capture(run)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(3):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (3 * reps * copies)
    del g, src, dst
    torch.cuda.empty_cache()
    return {"kind": "torch copy_", "read_bytes": n * 4, "written_bytes": n * 4,
            "us": round(us, 3), "GBs": round(2 * n * 4 / (us * 1e-6) / 1e9, 1)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work (what the method must move / compute, not what a kernel does)
# ---------------------------------------------------------------------------

def decode_bytes_per_token(H, HV, dk, dv, in_bytes=2, y_bytes=4, z_bytes=2):
    """HBM bytes per token per layer of the fused decode + RMSNormGated step:
    read + write the fp32 state of every value head, read q, k (per key head),
    v, g, beta and the gate z, write y."""
    return (HV * dk * dv * 4 * 2 + H * dk * in_bytes * 2 + HV * dv * in_bytes
            + HV * 8 + HV * dv * z_bytes + HV * dv * y_bytes)


def prefill_bytes(T, N, H, HV, dk, dv, in_bytes=2, o_bytes=4, s0=False):
    """HBM bytes of one prefill call: q, k, v, g, beta in, o out, final state
    out (and initial state in when given)."""
    b = T * (H * dk * in_bytes * 2 + HV * dv * in_bytes + HV * 8 + HV * dv * o_bytes)
    b += N * HV * dk * dv * 4 * (2 if s0 else 1)
    return b


def prefill_flops(T, H, HV, dk, dv, C=64):
    """Flops of the chunked form per call, full C x C tiles: per key head and
    token K K^T and Q K^T (2 C dk each); per value head and token the
    triangular solve (C^2 / 3), U = T diag(b)(V - diag(gamma) K S^T)
    (2 dk dv + 2 C dv), O = diag(gamma) Q S^T + P U (2 dk dv + 2 C dv) and the
    state update U^T K (2 dk dv)."""
    per_k = 2 * C * dk * 2
    per_v = C * C / 3 + (2 * dk * dv + 2 * C * dv) * 2 + 2 * dk * dv
    return T * (H * per_k + HV * per_v)


def layer_bytes_per_row(H, HV, dk, dv, in_bytes=2, gate_bytes=2, z_bytes=2, y_bytes=4):
    """HBM bytes per row of the serving decode step (gdn_decode_layer with raw
    gates, q/k norm and RMSNormGated): the slot's fp32 state read and written,
    q, k, v, the two raw gates, z in, y out, the slot index."""
    return (HV * dk * dv * 4 * 2 + H * dk * in_bytes * 2 + HV * dv * in_bytes
            + HV * 2 * gate_bytes + HV * dv * z_bytes + HV * dv * y_bytes + 4)


def norm_bytes(rows, HV, dv, x_bytes=4, z_bytes=2, y_bytes=4):
    return rows * HV * dv * (x_bytes + z_bytes + y_bytes) + dv * 4


# ---------------------------------------------------------------------------

def graph_capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # one eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g, s


def cpu_baseline_decode_job(layers_sample: int, N, T, H, HV, d, steps, seed=0):
    """The fp64 oracle on a bounded sample of the decode job: ``layers_sample``
    layers, each a T-token prefill of N sequences, RMSNormGated, then ``steps``
    decode steps with RMSNormGated.  Returns (tokens/s per layer, seconds,
    threads)."""
    import gdn_inputs as gi
    import oracle
    orc = oracle.load()
    data = []
    for l in range(layers_sample):
        x = gi.make_prefill([T] * N, H, HV, d, d, seed=seed + l, stream=1001)
        dd = gi.make_decode(steps, N, H, HV, d, d, seed=seed + l, stream=2001, decay_stream=1001)
        data.append((x, dd))
    t0 = time.perf_counter()
    for x, dd in data:
        o, S = orc.recurrence(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
        orc.rmsnorm_gated(o, x.z, x.w)
        for t in range(steps):
            od, S = orc.decode(dd.q[t], dd.k[t], dd.v[t], dd.g[t], dd.beta[t], S)
            orc.rmsnorm_gated(od, dd.z[t], dd.w)
    dt = time.perf_counter() - t0
    return N * (T + steps) * layers_sample / dt, dt, orc.max_threads()


JOB35 = dict(name="qwen3.6-35b-a3b-deltanet-job", N=2, T=8192, H=16, HV=32, d=128,
             decode_N=128, decode_steps=128)


def cpu_baseline_job35b(samples: int, N, T, H, HV, d, dec_N, steps, seed=0):
    """The fp64 oracle on ``samples`` layer-states of the 35B-A3B job: the
    N x T-token prefill + RMSNormGated, then ``steps`` decode steps of dec_N
    rows (row n from the prefill's final state n mod N) + RMSNormGated.  Input
    generation is not timed.  Returns (tokens/s per layer, seconds, threads)."""
    import gdn_inputs as gi
    import oracle
    orc = oracle.load()
    secs = 0.0
    for l in range(samples):
        x = gi.make_prefill([T] * N, H, HV, d, d, seed=seed + l, stream=1003)
        dd = gi.make_decode(steps, dec_N, H, HV, d, d, seed=seed + l, stream=2003,
                            decay_stream=1003)
        t0 = time.perf_counter()
        o, S = orc.recurrence(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
        orc.rmsnorm_gated(o, x.z, x.w)
        del o
        S = S[np.arange(dec_N) % N]
        for t in range(steps):
            od, S = orc.decode(dd.q[t], dd.k[t], dd.v[t], dd.g[t], dd.beta[t], S)
            orc.rmsnorm_gated(od, dd.z[t], dd.w)
        secs += time.perf_counter() - t0
        del x, dd, S
    return (N * T + dec_N * steps) * samples / secs, secs, orc.max_threads()


def cpu_baseline_prefill(lengths, H, HV, d, s0_std=0.0, seed=0):
    """The fp64 oracle on a packed prefill of the given lengths + RMSNormGated
    (generation not timed).  Returns (tokens/s, seconds, threads)."""
    import gdn_inputs as gi
    import oracle
    orc = oracle.load()
    x = gi.make_prefill(list(lengths), H, HV, d, d, s0_std=s0_std, seed=seed, stream=1004)
    t0 = time.perf_counter()
    o, _ = orc.recurrence(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens, s0=x.s0)
    orc.rmsnorm_gated(o, x.z, x.w)
    secs = time.perf_counter() - t0
    return int(np.sum(lengths)) / secs, secs, orc.max_threads()


def timed_calls(fn, reps, stream, settle_s=0.25):
    """Average time of ``reps`` back-to-back calls of fn on ``stream``
    (HIP events on that stream), in microseconds, after at least ``settle_s``
    seconds of untimed calls so that the clocks have settled."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t_end = time.perf_counter() + settle_s
        while True:
            fn()
            stream.synchronize()
            if time.perf_counter() >= t_end:
                break
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def prefill_roofline(us, T, N, H, HV, d, *, s0=False, o_bytes=4, issued=None, traffic=None):
    """HBM and bf16-MFMA fractions of one prefill call of ``us`` microseconds
    (algorithmic bytes and flops; issued MFMA flops and counted HBM bytes per
    call from the recorded rocprofv3 counters when they match the sources)."""
    b = prefill_bytes(T, N, H, HV, d, d, o_bytes=o_bytes, s0=s0)
    f = prefill_flops(T, H, HV, d, d)
    sec = us * 1e-6
    out = {"call_us": round(us, 2), "tokens_per_s": round(T / sec, 1),
           "hbm_achieved_GBs": round(b / sec / 1e9, 1),
           "hbm_frac": round(b / sec / 1e9 / HBM_PEAK_GBS, 4),
           "tflops": round(f / sec / 1e12, 2),
           "mfma_bf16_frac": round(f / sec / 1e12 / BF16_PEAK_TFLOPS, 5),
           "algorithmic_bytes": b, "algorithmic_flops": f,
           "bound": "hbm" if b / (HBM_PEAK_GBS * 1e9) >= f / (BF16_PEAK_TFLOPS * 1e12) else "mfma"}
    if issued is not None:
        out["issued_mfma_flops"] = issued
        out["issued_mfma_bf16_frac"] = round(issued / sec / 1e12 / BF16_PEAK_TFLOPS, 5)
    out["traffic"] = traffic
    return out


def run_job35b(args):
    import torch
    import gated_delta_rule_decode_amd as gdn
    import gdn_inputs as gi

    J = JOB35
    N, T, H, HV, d, Nd = J["N"], J["T"], J["H"], J["HV"], J["d"], J["decode_N"]
    steps = args.decode_steps or J["decode_steps"]
    L = args.layer_states
    dev = torch.device("cuda", 0)
    log(f"35B-A3B job: prefill {N} x {T} H={H} HV={HV} d={d}, then decode batch {Nd} x "
        f"{steps} steps, {L} layer-states")
    head_scale = gi.decay_scale(0, 1003, HV, "qwen")
    cu = torch.tensor([0, T, 2 * T], dtype=torch.int32, device=dev)
    w = torch.ones(d, device=dev)
    seed_rows = torch.arange(Nd, device=dev) % N
    layers = []
    for l in range(L):
        q, k, v, g, b, z = gi.device_tokens((N * T,), H, HV, d, d, seed=3000 + l,
                                            head_scale=head_scale, device=dev)
        dq, dk_, dv_, dg, db, dz = gi.device_tokens((steps, Nd), H, HV, d, d, seed=6000 + l,
                                                    head_scale=head_scale, device=dev)
        layers.append(dict(q=q, k=k, v=v, g=g, b=b, z=z, dq=dq, dk=dk_, dv=dv_, dg=dg, db=db,
                           dz=dz, pf_state=torch.empty(N, HV, d, d, device=dev),
                           pool=torch.empty(Nd, HV, d, d, device=dev),
                           y=torch.empty(N * T, HV, d, device=dev),
                           yd=torch.empty(Nd, HV, d, device=dev)))
    ws = torch.empty(gdn.prefill_norm_workspace_bytes(N, N * T, H, HV, d, d),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prefill_phase():
        for Ly in layers:
            gdn.prefill_chunked_norm(Ly["q"], Ly["k"], Ly["v"], Ly["g"], Ly["b"], cu, Ly["z"], w,
                                     final_state=Ly["pf_state"], y=Ly["y"], workspace=ws)
            torch.index_select(Ly["pf_state"], 0, seed_rows, out=Ly["pool"])

    def decode_phase():
        for t in range(steps):
            for Ly in layers:
                gdn.decode_step_norm(Ly["dq"][t], Ly["dk"][t], Ly["dv"][t], Ly["dg"][t],
                                     Ly["db"][t], Ly["pool"], Ly["dz"][t], w, y=Ly["yd"])

    t0 = time.perf_counter()
    g_pf, s = graph_capture(prefill_phase)
    g_dec, _ = graph_capture(decode_phase)
    log(f"graphs captured in {time.perf_counter() - t0:.1f}s")
    for _ in range(args.warmup):
        g_pf.replay()
        g_dec.replay()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    with torch.cuda.stream(s):
        for i in range(args.steps):
            ev[i][0].record(s)
            g_pf.replay()
            ev[i][1].record(s)
            g_dec.replay()
            ev[i][2].record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    pf_ms = sum(a.elapsed_time(b_) for a, b_, _ in ev)
    dec_ms = sum(b_.elapsed_time(c) for _, b_, c in ev)
    job_ms = (pf_ms + dec_ms) / args.steps
    ms_per_step = max(job_ms, wall * 1e3 / args.steps)
    pf_tokens, dec_tokens = N * T * L, Nd * steps * L
    value = (pf_tokens + dec_tokens) / (ms_per_step * 1e-3)

    # dominant kernel: decode + RMSNormGated, steps x layer-states launches on s
    launches = steps * L
    dec_launch_us = dec_ms / args.steps * 1e3 / launches
    bytes_launch = decode_bytes_per_token(H, HV, d, d) * Nd
    achieved = bytes_launch / (dec_launch_us * 1e-6) / 1e9

    # one prefill call timed alone (layer-state 0): the job's call (prefill +
    # RMSNormGated), the bare prefill with fp32 o, and with bf16 o
    Ly = layers[0]
    o32 = torch.empty(N * T, HV, d, device=dev)
    o16 = torch.empty(N * T, HV, d, device=dev, dtype=torch.bfloat16)
    ws_p = torch.empty(gdn.prefill_workspace_bytes(N, N * T, H, HV, d, d), dtype=torch.uint8,
                       device=dev)
    us_norm = timed_calls(lambda: gdn.prefill_chunked_norm(
        Ly["q"], Ly["k"], Ly["v"], Ly["g"], Ly["b"], cu, Ly["z"], w, final_state=Ly["pf_state"],
        y=Ly["y"], workspace=ws), 5, s)
    us_f32 = timed_calls(lambda: gdn.prefill_chunked(
        Ly["q"], Ly["k"], Ly["v"], Ly["g"], Ly["b"], cu, final_state=Ly["pf_state"], o=o32,
        workspace=ws_p), 5, s)
    us_b16 = timed_calls(lambda: gdn.prefill_chunked(
        Ly["q"], Ly["k"], Ly["v"], Ly["g"], Ly["b"], cu, final_state=Ly["pf_state"], o=o16,
        workspace=ws_p), 5, s)
    del o32, o16, ws_p
    copy_ref = copy_same_bytes(Nd * HV * d * d * 4, copies=L, reps=8)
    rec = recorded(PREFILL_COUNTERS, PREFILL_SOURCES)
    pf_line = prefill_roofline(us_f32, N * T, N, H, HV, d,
                               issued=rec and rec["issued_mfma_flops"].get("job35b"),
                               traffic=rec and rec["traffic_bytes"].get("job35b"))
    pf_line["with_norm_call_us"] = round(us_norm, 2)
    pf_line["bf16_o"] = {k_: v_ for k_, v_ in prefill_roofline(us_b16, N * T, N, H, HV, d,
                                                               o_bytes=2).items()
                         if k_ in ("call_us", "tokens_per_s", "hbm_frac", "mfma_bf16_frac")}
    del layers, ws
    torch.cuda.empty_cache()

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s per DeltaNet layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": J["name"], "prefill_sequences": N, "prefill_tokens_per_seq": T,
                   "qk_heads": H, "v_heads": HV, "d_k": d, "d_v": d, "decode_batch": Nd,
                   "decode_steps": steps, "layer_states": L,
                   "decode_seeding": "row n from prefill final state n mod 2",
                   "inputs": "bf16", "state": "f32", "outputs": "f32 (RMSNormGated y)"},
        "phases": {"prefill_tokens_per_s_per_layer": round(pf_tokens / (pf_ms / args.steps * 1e-3), 1),
                   "decode_tokens_per_s_per_layer": round(dec_tokens / (dec_ms / args.steps * 1e-3), 1),
                   "prefill_ms_per_step": round(pf_ms / args.steps, 4),
                   "decode_ms_per_step": round(dec_ms / args.steps, 4),
                   "wall_ms_per_step": round(wall * 1e3 / args.steps, 4)},
        "roofline": {"kernel": "decode_kernel (decode + RMSNormGated)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(DECODE3_TRAFFIC),
                     "avg_launch_us": round(dec_launch_us, 3),
                     "algorithmic_bytes_per_launch": bytes_launch},
        "copy_same_bytes": copy_ref,
        "roofline_prefill": pf_line,
        "context": model_step_context(pf_tokens / (pf_ms / args.steps * 1e-3),
                                      dec_tokens / (dec_ms / args.steps * 1e-3), 30),
    }
    if not args.no_cap:
        out["phases"]["long_context_varlen_cap"] = prefill_cap_phase(args)
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a sample of the job")
        v_cpu, secs, thr = cpu_baseline_job35b(args.cpu_layers, N, T, H, HV, d, Nd, steps)
        out["cpu_baseline"] = {"value": round(v_cpu, 1), "unit": "tokens/s per DeltaNet layer",
                               "cores": thr, "kind": "oracle",
                               "sample": f"{args.cpu_layers} layer-state(s) of the job: "
                                         f"{N} x {T}-token prefill + RMSNormGated, then {Nd} "
                                         f"rows x {steps} decode steps + RMSNormGated, fp64, "
                                         f"{secs:.1f} s"}
    return out


def model_step_context(pf_tok_s, dec_tok_s, layers):
    """Context only: the per-layer rates over the DeltaNet layers of a whole
    model (18 of the 0.8B model's 24 layers; 30 of the 35B-A3B's 40: Core AI
    card, introduction), i.e. a model step with nothing but its DeltaNet
    mixers -- no attention, MoE, projections or sampling."""
    return {"deltanet_layers": layers,
            "gdn_only_prefill_tokens_per_s": round(pf_tok_s / layers, 1),
            "gdn_only_decode_tokens_per_s": round(dec_tok_s / layers, 1),
            "note": "per-layer rates divided by the model's DeltaNet layer count; "
                    "not a whole-model figure"}


def prefill_cap_phase(args):
    """The long-context varlen prefill at its 131,072-token cap (8 packed
    sequences, 16 key / 32 value heads, S0 ~ N(0, 0.02)): one call timed with
    the library's own choice of scan, fp32 and bf16 outputs, with its HBM and
    MFMA fractions and the oracle on a bounded sample of it."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    import gdn_inputs as gi
    w4 = gi.WORKLOADS[4]
    H, HV, d = w4["H"], w4["HV"], w4["dk"]
    lengths = np.array(gi.CAP_LENGTHS)
    N, T = len(lengths), int(lengths.sum())
    dev = torch.device("cuda", 0)
    log(f"varlen prefill at the cap: {T} tokens in {N} sequences")
    head_scale = gi.decay_scale(0, 1004, HV, "qwen")
    q, k, v, g, b, _ = gi.device_tokens((T,), H, HV, d, d, seed=4, head_scale=head_scale,
                                        device=dev, with_z=False)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).to(dev)
    s0 = torch.randn(N, HV, d, d, device=dev) * w4["s0_std"]
    sf = torch.empty(N, HV, d, d, device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(N, T, H, HV, d, d), dtype=torch.uint8,
                     device=dev)
    s = torch.cuda.Stream()
    res = {}
    for name, dt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        o = torch.empty(T, HV, d, device=dev, dtype=dt)
        us = timed_calls(lambda: gdn.prefill_chunked(q, k, v, g, b, cu, initial_state=s0,
                                                     final_state=sf, o=o, workspace=ws), 3, s)
        res[name] = us
        del o
    rec = recorded(PREFILL_COUNTERS, PREFILL_SOURCES)
    out = {"workload": "long-context-varlen-prefill at the 131,072-token cap",
           "lengths": [int(x) for x in lengths], "qk_heads": H, "v_heads": HV,
           "roofline": prefill_roofline(res["f32"], T, N, H, HV, d, s0=True,
                                        issued=rec and rec["issued_mfma_flops"].get("cap"),
                                        traffic=rec and rec["traffic_bytes"].get("cap")),
           "bf16_o": {k_: v_ for k_, v_ in prefill_roofline(res["bf16"], T, N, H, HV, d, s0=True,
                                                            o_bytes=2).items()
                      if k_ in ("call_us", "tokens_per_s", "hbm_frac", "mfma_bf16_frac")}}
    del q, k, v, g, b, s0, sf, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        sample = [5000, 1280]  # two of the cap's sequences
        v_cpu, secs, thr = cpu_baseline_prefill(sample, H, HV, d, s0_std=w4["s0_std"])
        out["cpu_baseline"] = {"value": round(v_cpu, 1), "unit": "tokens/s (one layer)",
                               "cores": thr, "kind": "oracle",
                               "sample": f"sequences of {sample} tokens of the cap batch, "
                                         f"32 value heads, prefill + RMSNormGated, fp64, "
                                         f"{secs:.1f} s"}
    return out


def run_decode_job(args):
    import torch
    import gated_delta_rule_decode_amd as gdn
    import gdn_inputs as gi

    N, H, HV, d, T, steps, L = 32, 16, 16, 128, 512, 256, args.layers
    if args.decode_steps:
        steps = args.decode_steps
    dev = torch.device("cuda", 0)
    bf = torch.bfloat16
    log(f"decode job: N={N} H={H} HV={HV} d={d} prefill T={T} steps={steps} layers={L}")
    head_scale = gi.decay_scale(0, 1001, HV, "qwen")
    layers = []
    for l in range(L):
        q, k, v, g, b, z = gi.device_tokens((N * T,), H, HV, d, d, seed=1000 + l,
                                            head_scale=head_scale, device=dev)
        dq, dk_, dv_, dg, db, dz = gi.device_tokens((steps, N), H, HV, d, d, seed=5000 + l,
                                                    head_scale=head_scale, device=dev)
        layers.append(dict(q=q, k=k, v=v, g=g, b=b, z=z, dq=dq, dk=dk_, dv=dv_, dg=dg, db=db,
                           dz=dz, state=torch.zeros(N, HV, d, d, device=dev),
                           o=torch.empty(N * T, HV, d, device=dev),
                           y=torch.empty(N * T, HV, d, device=dev),
                           od=torch.empty(N, HV, d, device=dev),
                           yd=torch.empty(N, HV, d, device=dev)))
    w = torch.ones(d, device=dev)
    cu = torch.arange(0, N * T + 1, T, dtype=torch.int32, device=dev)
    ws = torch.empty(gdn.prefill_norm_workspace_bytes(N, N * T, H, HV, d, d),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prefill_phase():
        for Ly in layers:
            gdn.prefill_chunked_norm(Ly["q"], Ly["k"], Ly["v"], Ly["g"], Ly["b"], cu, Ly["z"], w,
                                     final_state=Ly["state"], y=Ly["y"], workspace=ws)

    def decode_phase():
        for t in range(steps):
            for Ly in layers:
                gdn.decode_step_norm(Ly["dq"][t], Ly["dk"][t], Ly["dv"][t], Ly["dg"][t],
                                     Ly["db"][t], Ly["state"], Ly["dz"][t], w, y=Ly["yd"])

    t0 = time.perf_counter()
    g_pf, s = graph_capture(prefill_phase)
    g_dec, _ = graph_capture(decode_phase)
    log(f"graphs captured in {time.perf_counter() - t0:.1f}s")

    for _ in range(args.warmup):
        g_pf.replay()
        g_dec.replay()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    with torch.cuda.stream(s):
        for i in range(args.steps):
            ev[i][0].record(s)
            g_pf.replay()
            ev[i][1].record(s)
            g_dec.replay()
            ev[i][2].record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    pf_ms = sum(a.elapsed_time(b) for a, b, _ in ev)
    dec_ms = sum(b.elapsed_time(c) for _, b, c in ev)
    job_ms = (pf_ms + dec_ms) / args.steps
    ms_per_step = max(job_ms, wall * 1e3 / args.steps)

    tokens = N * (T + steps) * L
    value = tokens / (ms_per_step * 1e-3)
    pf_tok_s = N * T * L / (pf_ms / args.steps * 1e-3)
    dec_tok_s = N * steps * L / (dec_ms / args.steps * 1e-3)

    # dominant kernel: the fused decode + RMSNormGated step.  The decode phase
    # is exactly steps x layers launches of it on stream s, so its average
    # launch duration comes from the decode-phase HIP events of the timed region.
    launches = steps * L
    dec_launch_us = dec_ms / args.steps * 1e3 / launches
    bytes_launch = decode_bytes_per_token(H, HV, d, d) * N
    achieved = bytes_launch / (dec_launch_us * 1e-6) / 1e9

    # prefill kernels: one layer's call timed alone, the prefill by itself
    # (gdn_prefill_chunked) and with the norm (the job's call)
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    Ly = layers[0]
    with torch.cuda.stream(s):
        pe[0].record(s)
        for _ in range(5):
            gdn.prefill_chunked(Ly["q"], Ly["k"], Ly["v"], Ly["g"], Ly["b"], cu,
                                final_state=Ly["state"], o=Ly["o"], workspace=ws)
        pe[1].record(s)
        for _ in range(5):
            gdn.prefill_chunked_norm(Ly["q"], Ly["k"], Ly["v"], Ly["g"], Ly["b"], cu, Ly["z"], w,
                                     final_state=Ly["state"], y=Ly["y"], workspace=ws)
        pe[2].record(s)
    torch.cuda.synchronize()
    pf_call_us = pe[0].elapsed_time(pe[1]) * 1e3 / 5
    pf_norm_call_us = pe[1].elapsed_time(pe[2]) * 1e3 / 5
    pf_b = prefill_bytes(N * T, N, H, HV, d, d)
    pf_f = prefill_flops(N * T, H, HV, d, d)
    # a plain copy of the launch's state bytes, for the achievable bandwidth
    copy_ref = copy_same_bytes(N * HV * d * d * 4)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s per DeltaNet layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3.5-0.8b-deltanet-job", "sequences": N,
                   "qk_heads": H, "v_heads": HV, "d_k": d, "d_v": d,
                   "prefill_tokens_per_seq": T, "decode_steps": steps, "layers": L,
                   "inputs": "bf16", "state": "f32", "outputs": "f32"},
        "phases": {"prefill_tokens_per_s_per_layer": round(pf_tok_s, 1),
                   "decode_tokens_per_s_per_layer": round(dec_tok_s, 1),
                   "prefill_ms_per_step": round(pf_ms / args.steps, 4),
                   "decode_ms_per_step": round(dec_ms / args.steps, 4),
                   "wall_ms_per_step": round(wall * 1e3 / args.steps, 4)},
        "roofline": {"kernel": "decode_kernel (decode + RMSNormGated)", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "avg_launch_us": round(dec_launch_us, 3),
                     "algorithmic_bytes_per_launch": bytes_launch},
        "copy_same_bytes": copy_ref,
        "roofline_prefill": {"call_us": round(pf_call_us, 2),
                             "with_norm_call_us": round(pf_norm_call_us, 2),
                             "hbm_achieved_GBs": round(pf_b / (pf_call_us * 1e-6) / 1e9, 1),
                             "hbm_frac": round(pf_b / (pf_call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                             "tflops": round(pf_f / (pf_call_us * 1e-6) / 1e12, 2),
                             "mfma_bf16_frac": round(pf_f / (pf_call_us * 1e-6) / 1e12 /
                                                     BF16_PEAK_TFLOPS, 5),
                             "algorithmic_bytes": pf_b, "algorithmic_flops": pf_f},
        "context": model_step_context(pf_tok_s, dec_tok_s, 18),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a sample of the job")
        v_cpu, secs, thr = cpu_baseline_decode_job(args.cpu_layers, N, T, H, HV, d, steps)
        out["cpu_baseline"] = {"value": round(v_cpu, 1), "unit": "tokens/s per DeltaNet layer",
                               "cores": thr, "kind": "oracle",
                               "sample": f"{args.cpu_layers} layer(s) of the job: 32 x 512-token "
                                         f"prefill + {steps} decode steps + RMSNormGated, fp64, "
                                         f"{secs:.1f} s"}
    return out


LONG_PROMPT = {"name": "qwen3.5-0.8b-long-prompt-prefill", "N": 1, "T": 32768, "H": 16, "HV": 16,
               "dk": 128}


def run_prefill(args, cfg: str):
    import torch
    import gated_delta_rule_decode_amd as gdn
    import gdn_inputs as gi

    cap = cfg == "4cap"
    cfg_n = 4 if cap else int(cfg)
    w = LONG_PROMPT if cfg_n == 5 else gi.WORKLOADS[cfg_n]
    H, HV, d = w["H"], w["HV"], w["dk"]
    if cap:
        lengths = np.array(gi.CAP_LENGTHS)
    elif cfg_n == 4:
        lengths = gi.config_lengths(0)
    else:
        lengths = np.array([w["T"]] * w["N"])
    N, T = len(lengths), int(np.sum(lengths))
    dev = torch.device("cuda", 0)
    head_scale = gi.decay_scale(0, 1000 + cfg_n, HV, "qwen")
    q, k, v, g, b, _ = gi.device_tokens((T,), H, HV, d, d, seed=cfg_n, head_scale=head_scale,
                                        device=dev, with_z=False)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).to(dev)
    s0 = None
    if w.get("s0_std"):
        s0 = torch.randn(N, HV, d, d, device=dev) * w["s0_std"]
    o = torch.empty(T, HV, d, device=dev)
    o16 = torch.empty(T, HV, d, device=dev, dtype=torch.bfloat16)  # the bf16-o call
    sf = torch.empty(N, HV, d, d, device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(N, T, H, HV, d, d), dtype=torch.uint8, device=dev)
    def call(seg, out=None):
        gdn.prefill_chunked(q, k, v, g, b, cu, initial_state=s0, final_state=sf,
                            o=o if out is None else out, workspace=ws, segment_chunks=seg)

    def timed(seg, out=None):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            call(seg, out)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return max(e0.elapsed_time(e1), wall * 1e3) / args.steps

    # warm-up: the requested calls, and at least a quarter second of calls so
    # that the clocks have settled (each form in turn); then ten timed runs of
    # the library's own choice of the segment-parallel scan (0), interleaved
    # with ten of the same call writing bf16 o and three with segmentation off
    # (-1); the line reports medians and the spread of the ten
    t_end = time.perf_counter() + 0.25
    n_w = 0
    while n_w < args.warmup or time.perf_counter() < t_end:
        call(0)
        call(-1)
        call(0, o16)
        torch.cuda.synchronize()
        n_w += 1
    runs = {0: [], -1: [], "bf16": []}
    for i in range(10):
        runs[0].append(timed(0))
        runs["bf16"].append(timed(0, o16))
        if i % 3 == 0:
            runs[-1].append(timed(-1))
    ms = float(np.median(runs[0]))
    ms_whole = float(np.median(runs[-1]))
    ms16 = float(np.median(runs["bf16"]))
    one = np.array(runs[0]) * 1e3
    stats = {"runs": len(one), "calls_per_run": args.steps,
             "median_us": round(float(np.median(one)), 2), "min_us": round(float(one.min()), 2),
             "p90_us": round(float(np.percentile(one, 90)), 2)}
    del o16
    pb = prefill_bytes(T, N, H, HV, d, d, s0=s0 is not None)
    pfl = prefill_flops(T, H, HV, d, d)
    key = f"prefill{cfg}"
    rec = recorded(PREFILL_COUNTERS, PREFILL_SOURCES)
    issued = rec and rec["issued_mfma_flops"].get(key)
    out = {
        "metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s (one layer)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w["name"] + ("-at-the-cap" if cap else ""), "sequences": N,
                   "tokens": T,
                   "lengths": [int(x) for x in lengths], "qk_heads": H, "v_heads": HV,
                   "d_k": d, "d_v": d, "chunk": 64},
        "roofline": {"kernel": "prefill (all kernels of one call)", "bound": "hbm",
                     "achieved": round(pb / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(pb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": rec and rec["traffic_bytes"].get(key),
                     "algorithmic_bytes": pb, "algorithmic_flops": pfl,
                     "tflops": round(pfl / (ms * 1e-3) / 1e12, 2),
                     "mfma_bf16_frac": round(pfl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5),
                     "issued_mfma_flops": issued,
                     "issued_mfma_bf16_frac": issued and round(issued / (ms * 1e-3) / 1e12 /
                                                               BF16_PEAK_TFLOPS, 5)},
        "unsegmented_ms_per_step": round(ms_whole, 4),
        "call_us_stats": stats,
        "bf16_o": {k_: v_ for k_, v_ in prefill_roofline(ms16 * 1e3, T, N, H, HV, d,
                                                          s0=s0 is not None, o_bytes=2).items()
                   if k_ in ("call_us", "tokens_per_s", "hbm_frac", "mfma_bf16_frac")},
    }
    del q, k, v, g, b, o, sf, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        # a bounded sample of the same workload: its first 32768 tokens (of the
        # first sequences; all of workloads 2 and 3), all heads, prefill +
        # RMSNormGated
        sample, left = [], 32768
        for x in lengths:
            if left <= 0:
                break
            sample.append(int(min(x, left)))
            left -= sample[-1]
        v_cpu, secs, thr = cpu_baseline_prefill(sample, H, HV, d, s0_std=w.get("s0_std", 0.0))
        out["cpu_baseline"] = {"value": round(v_cpu, 1), "unit": "tokens/s (one layer)",
                               "cores": thr, "kind": "oracle",
                               "sample": f"sequences of {sample} tokens of the workload, "
                                         f"prefill + RMSNormGated, fp64, {secs:.1f} s"}
    return out


def run_copy(args):
    """Calibration for the HBM-traffic counters: a plain device copy of known
    size (256 MiB read + 256 MiB written per launch), timed like the rest."""
    import torch
    n = 64 * 1024 * 1024  # fp32 elements = 256 MiB
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = 2 * n * 4
    return {"metric": "device copy (counter calibration)", "value": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "bytes_per_launch": nbytes,
            "read_bytes_per_launch": n * 4, "write_bytes_per_launch": n * 4}


def attn_bytes(N, Hq, Hkv, D, ctx):
    """HBM bytes of one attention decode step: the cached keys and values of
    ctx positions read, q, gate, k_new, v_new in, o (fp32) out, the new key and
    value written to the caches."""
    return (N * Hkv * ctx * 2 * D * 2 + N * Hq * D * (2 + 2 + 4) + N * Hkv * D * 2 * 2
            + N * Hkv * D * 2 * 2)


def run_attn(args):
    import torch
    import gated_delta_rule_decode_amd as gdn

    N, Hq, Hkv, D, Lmax, P, L = 128, 16, 2, 256, 8320, 8192, 10
    dev = torch.device("cuda", 0)
    bf = torch.bfloat16
    log(f"attn: rows={N} Hq={Hq} Hkv={Hkv} D={D} position={P} cache rows={Lmax} layers={L}")
    gen = torch.Generator(device=dev).manual_seed(9)
    layers = []
    for _ in range(L):
        layers.append(dict(
            kc=torch.randn(N, Hkv, Lmax, D, device=dev, dtype=bf, generator=gen),
            vc=torch.randn(N, Hkv, Lmax, D, device=dev, dtype=bf, generator=gen),
            q=torch.randn(N, Hq, D, device=dev, dtype=bf, generator=gen),
            g=torch.randn(N, Hq, D, device=dev, dtype=bf, generator=gen),
            kn=torch.randn(N, Hkv, D, device=dev, dtype=bf, generator=gen),
            vn=torch.randn(N, Hkv, D, device=dev, dtype=bf, generator=gen),
            o=torch.empty(N, Hq, D, device=dev)))
    pos = torch.full((N,), P, dtype=torch.int32, device=dev)
    ws = torch.empty(gdn.attn_decode_workspace_bytes(N, Hq, Hkv, D, Lmax), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    def step():
        for Ly in layers:
            gdn.attn_decode(Ly["q"], Ly["kn"], Ly["vn"], Ly["kc"], Ly["vc"], pos, gate=Ly["g"],
                            o=Ly["o"], rotary_dim=64, rope_theta=1e7, workspace=ws)

    g_at, s = graph_capture(step)
    for _ in range(args.warmup):
        g_at.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(args.steps):
            g_at.replay()
        e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = max(e0.elapsed_time(e1), wall * 1e3) / args.steps
    launch_us = ms * 1e3 / L
    bytes_launch = attn_bytes(N, Hq, Hkv, D, P + 1)
    achieved = bytes_launch / (launch_us * 1e-6) / 1e9
    return {
        "metric": METRIC, "value": round(N * L / (ms * 1e-3), 1),
        "unit": "tokens/s per attention layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3.6-35b-a3b-gated-attention-decode", "rows": N,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "position": P,
                   "cache_rows": Lmax, "rotary_dim": 64, "rope_theta": 1e7, "layers": L,
                   "cache": "bf16", "outputs": "f32"},
        "roofline": {"kernel": "attn_split_kernel + attn_combine_kernel", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(ATTN_TRAFFIC, "gdn_attn.hip"),
                     "avg_launch_us": round(launch_us, 3),
                     "algorithmic_bytes_per_launch": bytes_launch},
    }


def run_decode3(args):
    """The 35B-A3B-shaped decode (16 key / 32 value heads, d = 128): batch 128,
    slot n starting from the final state n mod 2 of a 2 x 8192-token prefill,
    then ``steps`` decode steps (decode + RMSNormGated in one kernel) over 4
    layer-states (4 x 256 MiB, beyond the 256 MB Infinity Cache), each with
    its own inputs; the decode phase is captured in a HIP graph."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    import gdn_inputs as gi

    N, H, HV, d, T, L = 128, 16, 32, 128, 8192, 4
    steps = args.decode_steps or 128
    dev = torch.device("cuda", 0)
    log(f"decode3: N={N} H={H} HV={HV} d={d} prefill 2 x {T} steps={steps} layer-states={L}")
    head_scale = gi.decay_scale(0, 1003, HV, "qwen")
    cu = torch.tensor([0, T, 2 * T], dtype=torch.int32, device=dev)
    w = torch.ones(d, device=dev)
    layers = []
    for l in range(L):
        q, k, v, g, b, _ = gi.device_tokens((2 * T,), H, HV, d, d, seed=3000 + l,
                                            head_scale=head_scale, device=dev, with_z=False)
        _, S2 = gdn.prefill_chunked(q, k, v, g, b, cu)
        del q, k, v, g, b
        state = S2[torch.arange(N, device=dev) % 2].contiguous()
        dq, dk_, dv_, dg, db, dz = gi.device_tokens((steps, N), H, HV, d, d, seed=6000 + l,
                                                    head_scale=head_scale, device=dev)
        layers.append(dict(dq=dq, dk=dk_, dv=dv_, dg=dg, db=db, dz=dz, state=state,
                           yd=torch.empty(N, HV, d, device=dev)))
    torch.cuda.synchronize()

    def decode_phase():
        for t in range(steps):
            for Ly in layers:
                gdn.decode_step_norm(Ly["dq"][t], Ly["dk"][t], Ly["dv"][t], Ly["dg"][t],
                                     Ly["db"][t], Ly["state"], Ly["dz"][t], w, y=Ly["yd"])

    g_dec, s = graph_capture(decode_phase)
    for _ in range(args.warmup):
        g_dec.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(args.steps):
            g_dec.replay()
        e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = max(e0.elapsed_time(e1), wall * 1e3) / args.steps
    launch_us = ms * 1e3 / (steps * L)
    bytes_launch = decode_bytes_per_token(H, HV, d, d) * N
    achieved = bytes_launch / (launch_us * 1e-6) / 1e9
    return {
        "metric": METRIC, "value": round(N * steps * L / (ms * 1e-3), 1),
        "unit": "tokens/s per DeltaNet layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3.6-35b-a3b-deltanet-decode", "sequences": N,
                   "qk_heads": H, "v_heads": HV, "d_k": d, "d_v": d,
                   "seeded_from": "2 x 8192-token prefill (slot n from state n mod 2)",
                   "decode_steps": steps, "layer_states": L, "inputs": "bf16",
                   "state": "f32", "outputs": "f32"},
        "roofline": {"kernel": "decode_kernel (decode + RMSNormGated)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(DECODE3_TRAFFIC),
                     "avg_launch_us": round(launch_us, 3),
                     "algorithmic_bytes_per_launch": bytes_launch},
    }


def norm_bytes(rows, HV, dv, x_bytes=4, z_bytes=2, y_bytes=4, w_bytes=4):
    """HBM bytes of one RMSNormGated launch: x and z read, y written, the
    weight read once."""
    return rows * HV * dv * (x_bytes + z_bytes + y_bytes) + dv * w_bytes


def run_norm(args):
    """RMSNormGated on its own (gdn_rmsnorm_gated) at the 0.8B job's prefill
    output shape: 32 x 512 tokens, 16 value heads, d_v = 128, fp32 x, bf16 z,
    fp32 y; 18 layers, each with its own tensors, in a HIP graph."""
    import torch
    import gated_delta_rule_decode_amd as gdn

    rows, HV, dv, L = 32 * 512, 16, 128, args.layers
    dev = torch.device("cuda", 0)
    log(f"norm: rows={rows} HV={HV} dv={dv} layers={L}")
    gen = torch.Generator(device=dev).manual_seed(11)
    layers = [dict(x=torch.randn(rows, HV, dv, device=dev, generator=gen),
                   z=torch.randn(rows, HV, dv, device=dev, generator=gen).to(torch.bfloat16),
                   y=torch.empty(rows, HV, dv, device=dev)) for _ in range(L)]
    w = torch.ones(dv, device=dev)
    torch.cuda.synchronize()

    def step():
        for Ly in layers:
            gdn.rmsnorm_gated(Ly["x"], Ly["z"], w, y=Ly["y"])

    g_n, s = graph_capture(step)
    for _ in range(args.warmup):
        g_n.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(args.steps):
            g_n.replay()
        e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = max(e0.elapsed_time(e1), wall * 1e3) / args.steps
    launch_us = ms * 1e3 / L
    bytes_launch = norm_bytes(rows, HV, dv)
    achieved = bytes_launch / (launch_us * 1e-6) / 1e9
    return {
        "metric": METRIC, "value": round(rows * L / (ms * 1e-3), 1),
        "unit": "tokens/s per DeltaNet layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3.5-0.8b-rmsnormgated", "rows": rows, "v_heads": HV,
                   "d_v": dv, "layers": L, "x": "f32", "z": "bf16", "y": "f32"},
        "roofline": {"kernel": "rmsnorm_gated_kernel", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(NORM_TRAFFIC, "gdn_rmsnorm.hip"),
                     "avg_launch_us": round(launch_us, 3),
                     "algorithmic_bytes_per_launch": bytes_launch},
    }


def run_serve(args):
    import torch
    import gated_delta_rule_decode_amd as gdn
    import gdn_inputs as gi

    N, SLOTS, H, HV, d, L = 128, 256, 16, 32, 128, 30
    steps = args.decode_steps or 16
    dev = torch.device("cuda", 0)
    bf = torch.bfloat16
    log(f"serve: rows={N} slots={SLOTS} H={H} HV={HV} d={d} layers={L} steps={steps}")
    rng = np.random.default_rng(7)
    layers = []
    for l in range(L):
        r = gi.make_decode_raw(steps, N, H, HV, d, d, seed=7000 + l, gate_dtype="bf16")
        pool = torch.empty(SLOTS, HV, d, d, device=dev)
        pool.normal_(0.0, 0.02, generator=torch.Generator(device=dev).manual_seed(l))
        layers.append(dict(
            q=torch.from_numpy(r.q).to(dev, bf), k=torch.from_numpy(r.k).to(dev, bf),
            v=torch.from_numpy(r.v).to(dev, bf), z=torch.from_numpy(r.z).to(dev, bf),
            a=torch.from_numpy(r.a_raw).to(dev, bf), b=torch.from_numpy(r.b_raw).to(dev, bf),
            A_log=torch.from_numpy(r.A_log).to(dev), dt=torch.from_numpy(r.dt_bias).to(dev),
            w=torch.from_numpy(r.w).to(dev), pool=pool,
            slots=torch.from_numpy(np.stack([rng.permutation(SLOTS)[:N] for _ in range(steps)])
                                   .astype(np.int32)).to(dev),
            y=torch.empty(N, HV, d, device=dev)))
    scale = d ** -0.5
    torch.cuda.synchronize()

    def serve_phase():
        for t in range(steps):
            for Ly in layers:
                gdn.decode_layer(Ly["q"][t], Ly["k"][t], Ly["v"][t], Ly["pool"], a_raw=Ly["a"][t],
                                 b_raw=Ly["b"][t], A_log=Ly["A_log"], dt_bias=Ly["dt"],
                                 slots=Ly["slots"][t], qk_l2norm=True, z=Ly["z"][t], w=Ly["w"],
                                 y=Ly["y"], scale=scale)

    g_sv, s = graph_capture(serve_phase)
    for _ in range(args.warmup):
        g_sv.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(args.steps):
            g_sv.replay()
        e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms = max(e0.elapsed_time(e1), wall * 1e3) / args.steps
    launches = steps * L
    launch_us = ms * 1e3 / launches
    bytes_launch = layer_bytes_per_row(H, HV, d, d) * N
    achieved = bytes_launch / (launch_us * 1e-6) / 1e9

    # cost of the serving extras: the same launch on one contiguous state set
    # (rows 0..N-1 of layer 0's pool, no slot table) with and without them
    Ly = layers[0]
    st = Ly["pool"][:N]
    g32 = torch.full((N, HV), -0.1, device=dev)
    b32 = torch.full((N, HV), 0.5, device=dev)

    def timed(fn, reps=50):
        with torch.cuda.stream(s):
            for _ in range(3):
                fn()
            e0.record(s)
            for _ in range(reps):
                fn()
            e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    plain_us = timed(lambda: gdn.decode_step_norm(Ly["q"][0], Ly["k"][0], Ly["v"][0], g32, b32,
                                                  st, Ly["z"][0], Ly["w"], y=Ly["y"],
                                                  scale=scale))
    extras_us = timed(lambda: gdn.decode_layer(Ly["q"][0], Ly["k"][0], Ly["v"][0], st,
                                               a_raw=Ly["a"][0], b_raw=Ly["b"][0],
                                               A_log=Ly["A_log"], dt_bias=Ly["dt"],
                                               qk_l2norm=True, z=Ly["z"][0], w=Ly["w"],
                                               y=Ly["y"], scale=scale))
    copy_ref = copy_same_bytes(N * HV * d * d * 4, copies=4, reps=8)

    tokens = N * steps * L
    return {
        "metric": METRIC, "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s per DeltaNet layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3.6-35b-a3b-deltanet-serving-decode", "rows": N,
                   "state_slots": SLOTS, "qk_heads": H, "v_heads": HV, "d_k": d, "d_v": d,
                   "layers": L, "decode_steps": steps, "gates": "raw bf16",
                   "qk_l2norm": True, "norm": "RMSNormGated", "inputs": "bf16"},
        "roofline": {"kernel": "decode_kernel (serving: slots, gates, q/k norm, RMSNormGated)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(SERVE_TRAFFIC),
                     "avg_launch_us": round(launch_us, 3),
                     "algorithmic_bytes_per_launch": bytes_launch},
        "copy_same_bytes": copy_ref,
        "extras_cost": {"same_state_us_plain_decode_norm": round(plain_us, 3),
                        "same_state_us_layer_with_gates_l2_norm": round(extras_us, 3)},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="job35b",
                    choices=["job35b", "job08b", "decode", "prefill2", "prefill3", "prefill4",
                             "prefill4cap", "prefill5", "copy", "serve", "attn", "norm",
                             "decode3"])
    ap.add_argument("--layers", type=int, default=18,
                    help="DeltaNet layers of the 0.8B job (and the norm workload)")
    ap.add_argument("--layer-states", type=int, default=4,
                    help="layer-states of the 35B-A3B job")
    ap.add_argument("--decode-steps", type=int, default=0)
    ap.add_argument("--cpu-layers", type=int, default=0,
                    help="layer-states in the oracle's sample (default: 4 for the 35B-A3B "
                         "job, 12 for the 0.8B job)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cap", action="store_true",
                    help="35B-A3B job: skip the varlen-prefill-at-the-cap phase")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU only: libgdn has no multi-GPU path (every "
                  "(sequence, head) recurrence is independent; see the sharding notes). "
                  "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import gated_delta_rule_decode_amd as gdn
    gdn.lib()  # loud failure without the HIP library
    if args.workload == "job35b":
        args.cpu_layers = args.cpu_layers or 4
        out = run_job35b(args)
    elif args.workload in ("job08b", "decode"):
        args.cpu_layers = args.cpu_layers or 12
        out = run_decode_job(args)
    elif args.workload == "copy":
        out = run_copy(args)
    elif args.workload == "serve":
        out = run_serve(args)
    elif args.workload == "attn":
        out = run_attn(args)
    elif args.workload == "norm":
        out = run_norm(args)
    elif args.workload == "decode3":
        out = run_decode3(args)
    else:
        out = run_prefill(args, args.workload[len("prefill"):])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

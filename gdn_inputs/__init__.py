"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

This module is shared by the fp64 oracle's tests, the GPU parity tests, the
smoke check and the benchmark.  It draws random tensors with the shapes and
distributions of the five workloads and holds none of the mixer's own
arithmetic (no recurrence, no normalisation of outputs): only the recipe that
turns seeded normal draws into the inputs q, k, v, g, beta, z, w, the initial
state and the packed-batch offsets.

Workloads (Qwen3.5-0.8B and Qwen3.6-35B-A3B DeltaNet shapes; the 35B card on
the Core AI model zoo page, intro, gives the 32 value heads over 16 key heads):

  0  tiny step recurrence: N=1, H=HV=1, d=16, T=64, fp32, S0=0
  1  0.8B decode: N=32, H=HV=16, d=128, bf16; 512-token prefill then 256 steps
  2  0.8B chunked prefill: N=4 x T=4096, H=HV=16, d=128, bf16, S0=0
  3  35B-A3B GVA: prefill 2 x 8192 (H=16, HV=32), then decode 128 x 128 steps
  4  long-context varlen prefill: 8 sequences, log-uniform lengths in
     [256, 65536] with total <= 131072, H=16, HV=32, S0 ~ N(0, 0.02^2)

Recipe (the same for every workload unless stated):
  q, k ~ N(0, 1), L2-normalised per (token, head) in fp32, then rounded to
  bf16 with round-to-nearest-even (workload 0 keeps fp32).
  v ~ N(0, 1), rounded to bf16 (workload 0: fp32).
  g = -exp(A_h) * softplus(x), x ~ N(0, 1); A_h ~ U(0, ln 16) per value head
  (workload 0: A_h = 0, i.e. a = exp(-softplus(x))).  g is the log of the
  decay a and is stored in fp32.
  beta = sigmoid(x'), x' ~ N(0, 1), fp32.
  z ~ N(0, 1) rounded to bf16 (workload 0: fp32); the norm weight w = 1.

Raw decode-layer inputs (``make_decode_raw``), for the serving form of the
step that activates gates and normalises q, k itself: q, k ~ N(0, 1) NOT
normalised; a_raw, b_raw ~ N(0, 1) (the draws behind g and beta above);
A_log ~ U(0, ln 16) per value head (the same draw as A_h); dt_bias ~
N(0, dt_bias_std^2) per value head; w ~ 1 + N(0, 0.1^2).

Attention decode inputs (``make_attn``): q, gate, k_new, v_new and both
caches ~ N(0, 1) rounded to bf16; the cached keys are arbitrary values (they
stand for keys stored after their rotation); pos[n] ~ U[0, Lmax) unless given.

Every tensor comes from its own numpy Generator keyed by (seed, workload,
tensor tag), so a tensor does not depend on the order in which the others are
drawn.  Values that are bf16 are returned as float32 arrays holding exactly
representable bf16 numbers; ``bf16_bits`` gives their 16-bit patterns.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "round_bf16", "bf16_bits", "PrefillInputs", "DecodeInputs", "make_prefill",
    "make_decode", "config_lengths", "workload", "WORKLOADS", "decay_scale",
    "DecodeRawInputs", "make_decode_raw", "AttnInputs", "make_attn",
]

# tensor tags for the per-tensor generator streams
_TAG = {"q": 1, "k": 2, "v": 3, "g": 4, "beta": 5, "z": 6, "A": 7, "s0": 8, "len": 9,
        "dt": 10, "w": 11, "kc": 12, "vc": 13, "pos": 14}


def _rng(seed: int, stream: int, tag: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), _TAG[tag]])


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """16-bit patterns of float32 values that are exactly representable in bf16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-exact")
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    """L2-normalise the last axis in fp32 (input recipe, not mixer arithmetic)."""
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    n = np.maximum(n, np.float32(1e-12))
    return (x / n).astype(np.float32)


def decay_scale(seed: int, stream: int, HV: int, mode: str) -> np.ndarray:
    """Per-value-head decay scale exp(A_h) as float64 [HV]."""
    if mode == "unit":
        return np.ones(HV)
    if mode == "qwen":
        A = _rng(seed, stream, "A").uniform(0.0, math.log(16.0), size=HV)
        return np.exp(A)
    if mode == "mild":
        return np.full(HV, 0.02)
    raise ValueError(mode)


def _gates(seed, stream, shape_tokens, HV, mode):
    """g = -exp(A_h) softplus(x) and beta = sigmoid(x'), both fp32 [..., HV]."""
    scale = decay_scale(seed, stream, HV, mode)
    xg = _normal(_rng(seed, stream, "g"), shape_tokens + (HV,)).astype(np.float64)
    g = (-scale * np.logaddexp(0.0, xg)).astype(np.float32)
    xb = _normal(_rng(seed, stream, "beta"), shape_tokens + (HV,)).astype(np.float64)
    beta = (1.0 / (1.0 + np.exp(-xb))).astype(np.float32)
    return g, beta


@dataclass
class PrefillInputs:
    """A packed variable-length batch: token-major tensors [T_total, heads, d]."""
    q: np.ndarray          # [T, H, dk] float32 (bf16-exact when dtype == "bf16")
    k: np.ndarray          # [T, H, dk]
    v: np.ndarray          # [T, HV, dv]
    g: np.ndarray          # [T, HV] float32, log-decay (<= 0)
    beta: np.ndarray       # [T, HV] float32
    z: np.ndarray          # [T, HV, dv] norm gate input
    w: np.ndarray          # [dv] norm weight
    cu_seqlens: np.ndarray  # [N+1] int32
    s0: Optional[np.ndarray]  # [N, HV, dv, dk] float32 or None (zeros)
    dtype: str
    H: int
    HV: int
    dk: int
    dv: int
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens).astype(np.int64)


@dataclass
class DecodeInputs:
    """Per-step decode inputs, one token per sequence: [steps, N, heads, d]."""
    q: np.ndarray      # [steps, N, H, dk]
    k: np.ndarray      # [steps, N, H, dk]
    v: np.ndarray      # [steps, N, HV, dv]
    g: np.ndarray      # [steps, N, HV]
    beta: np.ndarray   # [steps, N, HV]
    z: np.ndarray      # [steps, N, HV, dv]
    w: np.ndarray      # [dv]
    dtype: str
    H: int
    HV: int
    dk: int
    dv: int

    @property
    def steps(self) -> int:
        return self.q.shape[0]

    @property
    def N(self) -> int:
        return self.q.shape[1]


def _qkvz(seed, stream, lead, H, HV, dk, dv, dtype):
    q = _unit_rows(_normal(_rng(seed, stream, "q"), lead + (H, dk)))
    k = _unit_rows(_normal(_rng(seed, stream, "k"), lead + (H, dk)))
    v = _normal(_rng(seed, stream, "v"), lead + (HV, dv))
    z = _normal(_rng(seed, stream, "z"), lead + (HV, dv))
    if dtype == "bf16":
        q, k, v, z = round_bf16(q), round_bf16(k), round_bf16(v), round_bf16(z)
    elif dtype != "f32":
        raise ValueError(dtype)
    return q, k, v, z


def make_prefill(lengths, H, HV, dk, dv, *, dtype="bf16", decay="qwen",
                 s0_std: float = 0.0, seed: int = 0, stream: int = 100) -> PrefillInputs:
    """A packed batch with the given sequence lengths (zero-length allowed)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if HV % H:
        raise ValueError("HV must be a multiple of H")
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q, k, v, z = _qkvz(seed, stream, (T,), H, HV, dk, dv, dtype)
    g, beta = _gates(seed, stream, (T,), HV, decay)
    s0 = None
    if s0_std > 0.0:
        s0 = (_normal(_rng(seed, stream, "s0"), (len(lengths), HV, dv, dk))
              * np.float32(s0_std)).astype(np.float32)
    w = np.ones(dv, dtype=np.float32)
    return PrefillInputs(q, k, v, g, beta, z, w, cu, s0, dtype, H, HV, dk, dv)


def make_decode(steps, N, H, HV, dk, dv, *, dtype="bf16", decay="qwen", seed: int = 0,
                stream: int = 200, decay_stream: Optional[int] = None) -> DecodeInputs:
    """Independent per-step decode inputs.  ``decay_stream`` selects which
    stream's per-head decay scale to use, so decode can share the prefill's
    heads (the decay scale is a per-head model parameter)."""
    q, k, v, z = _qkvz(seed, stream, (steps, N), H, HV, dk, dv, dtype)
    ds = stream if decay_stream is None else decay_stream
    scale = decay_scale(seed, ds, HV, decay)
    xg = _normal(_rng(seed, stream, "g"), (steps, N, HV)).astype(np.float64)
    g = (-scale * np.logaddexp(0.0, xg)).astype(np.float32)
    xb = _normal(_rng(seed, stream, "beta"), (steps, N, HV)).astype(np.float64)
    beta = (1.0 / (1.0 + np.exp(-xb))).astype(np.float32)
    w = np.ones(dv, dtype=np.float32)
    return DecodeInputs(q, k, v, g, beta, z, w, dtype, H, HV, dk, dv)


@dataclass
class DecodeRawInputs:
    """Per-step decode-layer inputs with raw gates: [steps, N, ...]."""
    q: np.ndarray        # [steps, N, H, dk]  not normalised
    k: np.ndarray        # [steps, N, H, dk]  not normalised
    v: np.ndarray        # [steps, N, HV, dv]
    a_raw: np.ndarray    # [steps, N, HV]
    b_raw: np.ndarray    # [steps, N, HV]
    A_log: np.ndarray    # [HV] float32
    dt_bias: np.ndarray  # [HV] float32
    z: np.ndarray        # [steps, N, HV, dv]
    w: np.ndarray        # [dv]
    dtype: str
    gate_dtype: str
    H: int
    HV: int
    dk: int
    dv: int

    @property
    def steps(self) -> int:
        return self.q.shape[0]

    @property
    def N(self) -> int:
        return self.q.shape[1]


def make_decode_raw(steps, N, H, HV, dk, dv, *, dtype="bf16", gate_dtype="f32", seed: int = 0,
                    stream: int = 300, dt_bias_std: float = 0.5) -> DecodeRawInputs:
    """Raw decode-layer inputs (q, k unnormalised; gates as projections)."""
    lead = (steps, N)
    q = _normal(_rng(seed, stream, "q"), lead + (H, dk))
    k = _normal(_rng(seed, stream, "k"), lead + (H, dk))
    v = _normal(_rng(seed, stream, "v"), lead + (HV, dv))
    z = _normal(_rng(seed, stream, "z"), lead + (HV, dv))
    a_raw = _normal(_rng(seed, stream, "g"), lead + (HV,))
    b_raw = _normal(_rng(seed, stream, "beta"), lead + (HV,))
    A_log = _rng(seed, stream, "A").uniform(0.0, math.log(16.0), size=HV).astype(np.float32)
    dt_bias = (_normal(_rng(seed, stream, "dt"), (HV,)) * np.float32(dt_bias_std)).astype(
        np.float32)
    w = (1.0 + 0.1 * _normal(_rng(seed, stream, "w"), (dv,))).astype(np.float32)
    if dtype == "bf16":
        q, k, v, z = round_bf16(q), round_bf16(k), round_bf16(v), round_bf16(z)
    elif dtype != "f32":
        raise ValueError(dtype)
    if gate_dtype == "bf16":
        a_raw, b_raw = round_bf16(a_raw), round_bf16(b_raw)
    elif gate_dtype != "f32":
        raise ValueError(gate_dtype)
    return DecodeRawInputs(q, k, v, a_raw, b_raw, A_log, dt_bias, z, w, dtype, gate_dtype, H,
                           HV, dk, dv)


@dataclass
class AttnInputs:
    """One attention decode step: [N, heads, D] tokens and [N, Hkv, Lmax, D] caches."""
    q: np.ndarray        # [N, Hq, D]
    gate: np.ndarray     # [N, Hq, D]
    k_new: np.ndarray    # [N, Hkv, D]
    v_new: np.ndarray    # [N, Hkv, D]
    k_cache: np.ndarray  # [N, Hkv, Lmax, D]
    v_cache: np.ndarray  # [N, Hkv, Lmax, D]
    pos: np.ndarray      # [N] int32


def make_attn(N, Hq, Hkv, D, Lmax, *, pos=None, seed: int = 0, stream: int = 500) -> AttnInputs:
    """bf16-exact attention decode inputs (float32 arrays)."""
    f = lambda tag, shape: round_bf16(_normal(_rng(seed, stream, tag), shape))
    q = f("q", (N, Hq, D))
    gate = f("z", (N, Hq, D))
    kn = f("k", (N, Hkv, D))
    vn = f("v", (N, Hkv, D))
    kc = f("kc", (N, Hkv, Lmax, D))
    vc = f("vc", (N, Hkv, Lmax, D))
    if pos is None:
        pos = _rng(seed, stream, "pos").integers(0, Lmax, size=N)
    pos = np.asarray(pos, dtype=np.int32)
    return AttnInputs(q, gate, kn, vn, kc, vc, pos)


def config_lengths(seed: int = 0, stream: int = 400, n: int = 8, lo: int = 256,
                   hi: int = 65536, cap: int = 131072) -> np.ndarray:
    """Workload 4 lengths: round(exp(U(ln lo, ln hi))), clamped to [lo, hi];
    the whole set of n is redrawn from the same stream until its sum <= cap."""
    rng = _rng(seed, stream, "len")
    while True:
        L = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))).astype(np.int64)
        L = np.clip(L, lo, hi)
        if int(L.sum()) <= cap:
            return L


# Workload 4 at its largest size: 131,072 tokens in 8 sequences, the longest at
# the 65,536-token maximum and the shortest at the 256-token minimum of the
# length draw (a packing the draw allows at its cap).
CAP_LENGTHS = (65536, 256, 30000, 12000, 9000, 8000, 5000, 1280)


# workload table: shapes only; the tests and the benchmark build the tensors
WORKLOADS = {
    0: dict(name="tiny-step-d16", N=1, T=64, H=1, HV=1, dk=16, dv=16, dtype="f32",
            decay="unit", decode_steps=64),
    1: dict(name="qwen3.5-0.8b-gdn-decode", N=32, T=512, H=16, HV=16, dk=128, dv=128,
            dtype="bf16", decay="qwen", decode_steps=256),
    2: dict(name="qwen3.5-0.8b-gdn-prefill", N=4, T=4096, H=16, HV=16, dk=128, dv=128,
            dtype="bf16", decay="qwen"),
    3: dict(name="qwen3.6-35b-a3b-gdn-gva", N=2, T=8192, H=16, HV=32, dk=128, dv=128,
            dtype="bf16", decay="qwen", decode_N=128, decode_steps=128),
    4: dict(name="long-context-varlen-prefill", N=8, H=16, HV=32, dk=128, dv=128,
            dtype="bf16", decay="qwen", s0_std=0.02),
}


def workload(cfg: int, seed: int = 0) -> PrefillInputs:
    """The prefill inputs of a workload at its full size (stream = 1000 + cfg)."""
    w = WORKLOADS[cfg]
    if cfg == 4:
        lengths = config_lengths(seed)
    else:
        lengths = [w["T"]] * w["N"]
    return make_prefill(lengths, w["H"], w["HV"], w["dk"], w["dv"], dtype=w["dtype"],
                        decay=w["decay"], s0_std=w.get("s0_std", 0.0), seed=seed,
                        stream=1000 + cfg)


# ---------------------------------------------------------------------------
# device-side draws (benchmark): the same recipe, drawn with torch on the GPU
# ---------------------------------------------------------------------------

def device_tokens(lead, H, HV, dk, dv, *, seed: int, head_scale, device, dtype=None,
                  with_z: bool = True):
    """q, k, v, g, beta (and z) for tokens with leading shape ``lead``, drawn
    on ``device`` with a seeded torch.Generator: q, k L2-normalised in fp32
    then rounded to ``dtype`` (bf16 by default); v, z ~ N(0,1) in ``dtype``;
    g = -head_scale * softplus(x), beta = sigmoid(x') in fp32.  head_scale is
    the per-value-head exp(A_h) ([HV] float64 numpy array)."""
    import torch
    dtype = dtype or torch.bfloat16
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    lead = tuple(lead)
    f32 = torch.float32

    def unit(shape):
        x = torch.randn(shape, generator=gen, device=device, dtype=f32)
        return (x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)).to(dtype)

    q = unit(lead + (H, dk))
    k = unit(lead + (H, dk))
    v = torch.randn(lead + (HV, dv), generator=gen, device=device, dtype=f32).to(dtype)
    sc = torch.as_tensor(np.asarray(head_scale, np.float32), device=device)
    xg = torch.randn(lead + (HV,), generator=gen, device=device, dtype=f32)
    g = (-sc * torch.nn.functional.softplus(xg)).contiguous()
    xb = torch.randn(lead + (HV,), generator=gen, device=device, dtype=f32)
    beta = torch.sigmoid(xb).contiguous()
    z = None
    if with_z:
        z = torch.randn(lead + (HV, dv), generator=gen, device=device, dtype=f32).to(dtype)
    return q, k, v, g, beta, z

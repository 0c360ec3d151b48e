"""gdn_decode_step on the GPU against the fp64 oracle.

A decode step is the recurrence advanced by one token per sequence; a chain of
steps must equal the oracle's token-by-token recurrence.  Full-size decode
workloads start from oracle prefill states, so no GPU prefill is involved
(except in the explicit chain test).
"""
import numpy as np
import pytest

import gdn_inputs as gi
from gpu_helpers import assert_parity, dev, gpu_prefill, host, rel_l2, say, torch_dtype

pytestmark = pytest.mark.gpu


def _gpu_decode_chain(d: gi.DecodeInputs, state0, *, scale=1.0, out_dtype=None):
    """Run d.steps decode calls in place on a device copy of state0."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    dt = torch_dtype(d.dtype)
    q, k, v = dev(d.q, dt), dev(d.k, dt), dev(d.v, dt)
    g, b = dev(d.g), dev(d.beta)
    state = state0.clone() if isinstance(state0, torch.Tensor) else dev(np.asarray(state0, np.float32))
    outs = []
    for t in range(d.steps):
        outs.append(gdn.decode_step(q[t], k[t], v[t], g[t], b[t], state, scale=scale,
                                    out_dtype=out_dtype))
    return torch.stack(outs), state


def _oracle_decode_chain(orc, d: gi.DecodeInputs, state0, *, scale=1.0):
    state = np.asarray(state0, np.float64)
    outs = []
    for t in range(d.steps):
        o, state = orc.decode(d.q[t], d.k[t], d.v[t], d.g[t], d.beta[t], state, scale=scale)
        outs.append(o)
    return np.stack(outs), state


def test_decode_tiny_d16_fp32_equals_recurrence(orc):
    """64 single-token steps of workload 0 equal the oracle's recurrence."""
    x = gi.workload(0)
    d = gi.DecodeInputs(x.q[:, None], x.k[:, None], x.v[:, None], x.g[:, None], x.beta[:, None],
                        x.z[:, None], x.w, "f32", 1, 1, 16, 16)
    say("decode tiny d=16 fp32, 64 steps")
    o, S = _gpu_decode_chain(d, np.zeros((1, 1, 16, 16), np.float32))
    o_ref, S_ref = orc.recurrence(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
    assert_parity(host(o)[:, 0], host(S), o_ref, S_ref, f32=True, what="decode workload 0")


_SEED_CACHE = {}


def _seed_states(orc, cfg, seed=0):
    """Oracle prefill states for a decode workload (fp64; computed once per
    process)."""
    if (cfg, seed) not in _SEED_CACHE:
        x = gi.workload(cfg, seed)
        _, S = orc.recurrence(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
        _SEED_CACHE[(cfg, seed)] = S
    return _SEED_CACHE[(cfg, seed)]


def _gpu_decode_norm_chain(d: gi.DecodeInputs, state0, *, with_o=True):
    """d.steps calls of gdn_decode_step_norm in place on a device copy of
    state0 (bf16 z, fp32 w and y); returns (y [steps, N, HV, dv], o or None,
    state)."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    dt = torch_dtype(d.dtype)
    q, k, v = dev(d.q, dt), dev(d.k, dt), dev(d.v, dt)
    g, b, z, w = dev(d.g), dev(d.beta), dev(d.z, torch.bfloat16), dev(d.w)
    state = dev(np.asarray(state0, np.float32))
    ys, os_ = [], []
    for t in range(d.steps):
        if with_o:
            y, o = gdn.decode_step_norm(q[t], k[t], v[t], g[t], b[t], state, z[t], w,
                                        return_o=True)
            os_.append(o)
        else:
            y = gdn.decode_step_norm(q[t], k[t], v[t], g[t], b[t], state, z[t], w)
        ys.append(y)
    torch.cuda.synchronize()
    return torch.stack(ys), (torch.stack(os_) if with_o else None), state


def test_decode_workload1_full(orc):
    """32 sequences x 16 heads, d=128, states from a 512-token prefill, then
    256 decode steps; also checks the per-step error does not grow (the
    state-write failure mode shows up as agreement that decays with time)."""
    w = gi.WORKLOADS[1]
    S0 = _seed_states(orc, 1).astype(np.float32)
    d = gi.make_decode(w["decode_steps"], w["N"], w["H"], w["HV"], 128, 128, seed=0,
                       stream=2001, decay_stream=1001)
    say("decode workload 1: 32 x 16 heads, 256 steps")
    o, S = _gpu_decode_chain(d, S0)
    o_ref, S_ref = _oracle_decode_chain(orc, d, S0)
    oh = host(o)
    assert_parity(oh, host(S), o_ref, S_ref, what="decode workload 1")
    _drift(oh, o_ref, "decode workload 1")


def test_decode_workload3_full(orc):
    """35B-A3B shape: batch 128, 16 key heads, 32 value heads, 128 steps;
    slot n starts from prefill state n mod 2 of the 2 x 8192 prefill."""
    w = gi.WORKLOADS[3]
    S2 = _seed_states(orc, 3)
    S0 = S2[np.arange(w["decode_N"]) % 2].astype(np.float32)
    d = gi.make_decode(w["decode_steps"], w["decode_N"], w["H"], w["HV"], 128, 128, seed=0,
                       stream=2003, decay_stream=1003)
    say("decode workload 3: 128 x 32 value heads, 128 steps")
    o, S = _gpu_decode_chain(d, S0)
    o_ref, S_ref = _oracle_decode_chain(orc, d, S0)
    assert_parity(host(o), host(S), o_ref, S_ref, what="decode workload 3")


def _drift(y, y_ref, what):
    """The per-step error must not grow along the chain (the state-write fault
    shows up as agreement that decays with time)."""
    per_step = np.array([rel_l2(y[t], y_ref[t]) for t in range(y.shape[0])])
    q = max(1, y.shape[0] // 4)
    print(f"[drift] {what}: first quarter max {per_step[:q].max():.3e}, last quarter max "
          f"{per_step[-q:].max():.3e}")
    assert per_step[-q:].max() <= 3 * per_step[:q].max() + 1e-7


def test_decode_step_norm_workload3_full(orc):
    """decode + RMSNormGated (the kernel the 35B-A3B decode figure is measured
    on) at workload 3's decode shape: 128 rows x 32 value heads over 16 key
    heads, one workgroup per head (4096 workgroups: the streamed schedule),
    16 chained steps from the prefill-seeded states (row n from state n mod
    2).  o, y and the state against the oracle; then the same chain without o
    (the benchmark's call) gives bit-identical y and state."""
    w = gi.WORKLOADS[3]
    N = w["decode_N"]
    S0 = _seed_states(orc, 3)[np.arange(N) % 2].astype(np.float32)
    d = gi.make_decode(16, N, w["H"], w["HV"], 128, 128, seed=0, stream=2003, decay_stream=1003)
    assert N * w["HV"] >= 1024  # the streamed schedule of the fused kernel
    say("decode+norm workload 3: 128 x 32 value heads, 16 steps (streamed fused kernel)")
    y, o, S = _gpu_decode_norm_chain(d, S0)
    o_ref, S_ref = _oracle_decode_chain(orc, d, S0)
    y_ref = orc.rmsnorm_gated(o_ref, d.z, d.w)
    assert_parity(host(o), host(S), o_ref, S_ref, what="decode+norm workload 3 o")
    assert_parity(host(y), host(S), y_ref, S_ref, what="decode+norm workload 3 y")
    _drift(host(y), y_ref, "decode+norm workload 3")
    say("decode+norm workload 3 without o")
    y2, _, S2 = _gpu_decode_norm_chain(d, S0, with_o=False)
    import torch
    assert torch.equal(y, y2) and torch.equal(S, S2)


def test_decode_step_norm_workload1_full(orc):
    """decode + RMSNormGated at workload 1's shape (32 sequences x 16 heads,
    512 workgroups: the two-phase schedule), all 256 steps from the 512-token
    prefill states: o, y and the state against the oracle, with the drift
    check on y."""
    w = gi.WORKLOADS[1]
    S0 = _seed_states(orc, 1).astype(np.float32)
    d = gi.make_decode(w["decode_steps"], w["N"], w["H"], w["HV"], 128, 128, seed=0,
                       stream=2001, decay_stream=1001)
    say("decode+norm workload 1: 32 x 16 heads, 256 steps (two-phase fused kernel)")
    y, o, S = _gpu_decode_norm_chain(d, S0)
    o_ref, S_ref = _oracle_decode_chain(orc, d, S0)
    y_ref = orc.rmsnorm_gated(o_ref, d.z, d.w)
    assert_parity(host(o), host(S), o_ref, S_ref, what="decode+norm workload 1 o")
    assert_parity(host(y), host(S), y_ref, S_ref, what="decode+norm workload 1 y")
    _drift(host(y), y_ref, "decode+norm workload 1")


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (32, 64), (64, 32), (128, 16),
                                   (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_head_sizes(orc, dk, dv, dtype):
    d = gi.make_decode(6, 3, 2, 4, dk, dv, dtype=dtype, seed=dk * dv)
    S0 = (np.random.default_rng(dk + dv).standard_normal((3, 4, dv, dk)) * 0.05).astype(np.float32)
    say(f"decode dk={dk} dv={dv} {dtype}")
    o, S = _gpu_decode_chain(d, S0, scale=dk ** -0.5)
    o_ref, S_ref = _oracle_decode_chain(orc, d, S0, scale=dk ** -0.5)
    assert_parity(host(o), host(S), o_ref, S_ref, f32=(dtype == "f32"),
                  what=f"decode dk={dk} dv={dv} {dtype}")


def test_decode_gva_equals_repeated_heads():
    d = gi.make_decode(3, 4, 2, 4, 128, 128, seed=21)
    S0 = (np.random.default_rng(1).standard_normal((4, 4, 128, 128)) * 0.02).astype(np.float32)
    say("decode GVA vs repeated heads")
    o1, S1 = _gpu_decode_chain(d, S0)
    e = gi.DecodeInputs(np.repeat(d.q, 2, axis=2), np.repeat(d.k, 2, axis=2), d.v, d.g, d.beta,
                        d.z, d.w, d.dtype, 4, 4, 128, 128)
    o2, S2 = _gpu_decode_chain(e, S0)
    assert np.array_equal(o1.cpu().numpy(), o2.cpu().numpy())
    assert np.array_equal(S1.cpu().numpy(), S2.cpu().numpy())


def test_decode_bf16_output(orc):
    import torch
    d = gi.make_decode(4, 8, 2, 4, 128, 128, seed=22)
    S0 = (np.random.default_rng(2).standard_normal((8, 4, 128, 128)) * 0.02).astype(np.float32)
    say("decode bf16 output")
    o, S = _gpu_decode_chain(d, S0, out_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    o_ref, S_ref = _oracle_decode_chain(orc, d, S0)
    assert rel_l2(host(o), o_ref) <= 4e-3
    assert np.max(np.abs(host(S) - S_ref)) <= 1e-3


def test_decode_deterministic():
    d = gi.make_decode(2, 16, 4, 8, 128, 128, seed=23)
    S0 = (np.random.default_rng(3).standard_normal((16, 8, 128, 128)) * 0.02).astype(np.float32)
    say("decode determinism")
    o1, S1 = _gpu_decode_chain(d, S0)
    o2, S2 = _gpu_decode_chain(d, S0)
    assert np.array_equal(o1.cpu().numpy(), o2.cpu().numpy())
    assert np.array_equal(S1.cpu().numpy(), S2.cpu().numpy())


def test_chain_prefill_then_decode_equals_oracle(orc):
    """GPU prefill (512 tokens) then GPU decode (64 steps) against the oracle
    running the same tokens; and decode steps equal a prefill of the same
    tokens (incremental equals whole-sequence)."""
    x = gi.make_prefill([512] * 4, 4, 8, 128, 128, seed=30)
    d = gi.make_decode(64, 4, 4, 8, 128, 128, seed=30, stream=31, decay_stream=100)
    say("chain: prefill 4 x 512 then 64 decode steps")
    _, S = gpu_prefill(x)
    o_dec, S_dec = _gpu_decode_chain(d, S)
    _, S_ref0 = orc.recurrence(x.q, x.k, x.v, x.g, x.beta, x.cu_seqlens)
    o_ref, S_ref = _oracle_decode_chain(orc, d, S_ref0)
    assert_parity(host(o_dec), host(S_dec), o_ref, S_ref, what="prefill -> decode chain")
    # the same 64 tokens as a prefill from the prefill state
    T = d.steps
    y = gi.PrefillInputs(d.q.transpose(1, 0, 2, 3).reshape(4 * T, 4, 128),
                         d.k.transpose(1, 0, 2, 3).reshape(4 * T, 4, 128),
                         d.v.transpose(1, 0, 2, 3).reshape(4 * T, 8, 128),
                         d.g.transpose(1, 0, 2).reshape(4 * T, 8),
                         d.beta.transpose(1, 0, 2).reshape(4 * T, 8), None, None,
                         np.arange(0, 4 * T + 1, T, dtype=np.int32), None, "bf16", 4, 8, 128, 128)
    o_pf, S_pf = gpu_prefill(y, s0=S)
    o_pf = host(o_pf).reshape(4, T, 8, 128).transpose(1, 0, 2, 3)
    assert_parity(o_pf, host(S_pf), o_ref, S_ref, what="decode tokens as prefill")


def test_graph_replay_matches_eager():
    """Decode + RMSNormGated captured in a HIP graph: every replay (with eager
    work and synchronisations between replays) equals the eager result."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    d = gi.make_decode(4, 8, 4, 8, 128, 128, seed=40)
    S0 = (np.random.default_rng(4).standard_normal((8, 8, 128, 128)) * 0.02).astype(np.float32)
    bf = torch.bfloat16
    q, k, v = dev(d.q, bf), dev(d.k, bf), dev(d.v, bf)
    g, b, z = dev(d.g), dev(d.beta), dev(d.z, bf)
    w = torch.ones(128, device="cuda")
    state = dev(S0)
    o = torch.empty(8, 8, 128, device="cuda")
    y = torch.empty(4, 8, 8, 128, device="cuda")

    def run():
        for t in range(4):
            gdn.decode_step(q[t], k[t], v[t], g[t], b[t], state, o=o)
            gdn.rmsnorm_gated(o, z[t], w, y=y[t])

    say("graph replay vs eager")
    run()
    torch.cuda.synchronize()
    y_eager, s_eager = y.clone(), state.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    state.copy_(dev(S0))
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        run()
    for rep in range(4):
        state.copy_(dev(S0))
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep}: outputs differ"
        assert torch.equal(state, s_eager), f"replay {rep}: state differs"
        _ = (y * 2).sum().item()  # eager work between replays


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (128, 128)])
@pytest.mark.parametrize("dtype,zdt,ydt", [("bf16", "bf16", "f32"), ("f32", "f32", "f32"),
                                           ("bf16", "bf16", "bf16")])
def test_decode_step_norm_parity(orc, dk, dv, dtype, zdt, ydt):
    """Fused decode + RMSNormGated against the oracle's decode then norm."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    T = {"f32": torch.float32, "bf16": torch.bfloat16}
    d = gi.make_decode(5, 6, 2, 4, dk, dv, dtype=dtype, seed=50 + dk + dv)
    r = np.random.default_rng(dk * dv)
    S0 = (r.standard_normal((6, 4, dv, dk)) * 0.05).astype(np.float32)
    w = r.standard_normal(dv).astype(np.float32)
    z = d.z if zdt == "bf16" or dtype == "f32" else gi.round_bf16(d.z)
    say(f"decode+norm dk={dk} dv={dv} {dtype} z={zdt} y={ydt}")
    dt = torch_dtype(dtype)
    q, k, v = dev(d.q, dt), dev(d.k, dt), dev(d.v, dt)
    g, b = dev(d.g), dev(d.beta)
    state = dev(S0)
    wt = dev(w)
    ys, os_ = [], []
    for t in range(d.steps):
        y, o = gdn.decode_step_norm(q[t], k[t], v[t], g[t], b[t], state, dev(z[t], T[zdt]), wt,
                                    scale=dk ** -0.5, out_dtype=T[ydt], return_o=True)
        ys.append(y)
        os_.append(o)
    o_ref, S_ref = _oracle_decode_chain(orc, d, S0, scale=dk ** -0.5)
    y_ref = orc.rmsnorm_gated(o_ref, z, w)
    f32 = dtype == "f32" and ydt == "f32"
    assert_parity(host(torch.stack(os_)), host(state), o_ref, S_ref, f32=(dtype == "f32"),
                  what=f"decode+norm o dk={dk} dv={dv}")
    err = rel_l2(host(torch.stack(ys)), y_ref)
    print(f"[parity] decode+norm y dk={dk} dv={dv} {dtype}/{zdt}/{ydt}: rel-L2 {err:.3e}")
    assert err <= (2e-5 if f32 else (4e-3 if ydt == "bf16" else 2e-3)), err


def test_decode_step_norm_without_o_matches_two_calls():
    """o = NULL skips the raw outputs; y and the state equal decode_step then
    rmsnorm_gated up to rounding of the norm's sum order."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    d = gi.make_decode(2, 8, 4, 8, 128, 128, seed=60)
    S0 = (np.random.default_rng(6).standard_normal((8, 8, 128, 128)) * 0.02).astype(np.float32)
    bf = torch.bfloat16
    q, k, v, g, b, z = (dev(d.q, bf), dev(d.k, bf), dev(d.v, bf), dev(d.g), dev(d.beta),
                        dev(d.z, bf))
    w = torch.ones(128, device="cuda")
    s1, s2 = dev(S0), dev(S0)
    say("decode+norm without o vs two calls")
    for t in range(d.steps):
        y1 = gdn.decode_step_norm(q[t], k[t], v[t], g[t], b[t], s1, z[t], w)
        o2 = gdn.decode_step(q[t], k[t], v[t], g[t], b[t], s2)
        y2 = gdn.rmsnorm_gated(o2, z[t], w)
        assert torch.equal(s1, s2)
        assert rel_l2(host(y1), host(y2)) < 1e-6

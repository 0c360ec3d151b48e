"""gdn_decode_layer (serving form of the decode step) on the GPU against the
fp64 oracle: raw gate activations, q/k L2 norm, the slot table into a state
pool, and RMSNormGated, alone and together.

Each side activates the raw gates and normalises q, k itself: the oracle's
gates()/decode_layer() in float64, the kernel in float32.
"""
import numpy as np
import pytest

import gdn_inputs as gi
from gpu_helpers import assert_parity, dev, head_errors, host, rel_l2, say, torch_dtype

pytestmark = pytest.mark.gpu


def _oracle_chain(orc, d, pool0, slots_per_step, *, scale, l2norm, raw=True, g=None, beta=None):
    """The oracle's layer step over all steps; returns (o [steps, N, HV, dv], pool)."""
    pool = np.asarray(pool0, np.float64)
    os_ = []
    for t in range(d.steps):
        if raw:
            gt, bt = orc.gates(d.a_raw[t], d.b_raw[t], d.A_log, d.dt_bias)
        else:
            gt, bt = g[t], beta[t]
        sl = None if slots_per_step is None else slots_per_step[t]
        o, pool = orc.decode_layer(d.q[t], d.k[t], d.v[t], gt, bt, pool, slots=sl, scale=scale,
                                   l2norm=l2norm, l2_eps=1e-6)
        os_.append(o)
    return np.stack(os_), pool


def _gpu_chain(d, pool0, slots_per_step, *, scale, l2norm, norm=False, out_dtype=None):
    import torch
    import gated_delta_rule_decode_amd as gdn
    dt = torch_dtype(d.dtype)
    gdt = torch_dtype(d.gate_dtype)
    q, k, v = dev(d.q, dt), dev(d.k, dt), dev(d.v, dt)
    a_raw, b_raw = dev(d.a_raw, gdt), dev(d.b_raw, gdt)
    A_log, dt_bias = dev(d.A_log), dev(d.dt_bias)
    z, w = dev(d.z, dt), dev(d.w)
    pool = dev(np.asarray(pool0, np.float32))
    os_, ys = [], []
    for t in range(d.steps):
        sl = None if slots_per_step is None else dev(slots_per_step[t].astype(np.int32))
        kw = dict(a_raw=a_raw[t], b_raw=b_raw[t], A_log=A_log, dt_bias=dt_bias, slots=sl,
                  qk_l2norm=l2norm, scale=scale, out_dtype=out_dtype)
        if norm:
            y, o = gdn.decode_layer(q[t], k[t], v[t], pool, z=z[t], w=w, return_o=True, **kw)
            ys.append(y)
        else:
            o = gdn.decode_layer(q[t], k[t], v[t], pool, **kw)
        os_.append(o)
    torch.cuda.synchronize()
    return torch.stack(os_), pool, (torch.stack(ys) if norm else None)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (128, 128)])
@pytest.mark.parametrize("dtype,gate_dtype", [("bf16", "f32"), ("bf16", "bf16"), ("f32", "f32")])
def test_layer_raw_gates_l2norm(orc, dk, dv, dtype, gate_dtype):
    """Raw gates + in-kernel q/k L2 norm over a chain of steps, no slot table."""
    d = gi.make_decode_raw(5, 3, 2, 4, dk, dv, dtype=dtype, gate_dtype=gate_dtype,
                           seed=dk + 3 * dv)
    S0 = (np.random.default_rng(dk * dv).standard_normal((3, 4, dv, dk)) * 0.05).astype(
        np.float32)
    say(f"layer raw gates + l2 dk={dk} dv={dv} {dtype}/{gate_dtype}")
    o, S, _ = _gpu_chain(d, S0, None, scale=dk ** -0.5, l2norm=True)
    o_ref, S_ref = _oracle_chain(orc, d, S0, None, scale=dk ** -0.5, l2norm=True)
    assert_parity(host(o), host(S), o_ref, S_ref, f32=(dtype == "f32"),
                  what=f"layer raw+l2 dk={dk} dv={dv} {dtype}/{gate_dtype}")


def test_layer_gates_without_l2norm(orc):
    """Raw gates alone on pre-normalised q, k (the recipe of the workloads)."""
    d = gi.make_decode_raw(4, 4, 2, 4, 128, 128, seed=71)
    q = gi.round_bf16(d.q / np.linalg.norm(d.q, axis=-1, keepdims=True))
    k = gi.round_bf16(d.k / np.linalg.norm(d.k, axis=-1, keepdims=True))
    d.q, d.k = q, k
    S0 = (np.random.default_rng(71).standard_normal((4, 4, 128, 128)) * 0.02).astype(np.float32)
    say("layer raw gates, no l2")
    o, S, _ = _gpu_chain(d, S0, None, scale=128 ** -0.5, l2norm=False)
    o_ref, S_ref = _oracle_chain(orc, d, S0, None, scale=128 ** -0.5, l2norm=False)
    assert_parity(host(o), host(S), o_ref, S_ref, what="layer raw gates")


def _slot_tables(rng, steps, N, S):
    """Per step: distinct slots for the live rows, -1 and S (out of range) for
    two skipped rows."""
    tabs = []
    for _ in range(steps):
        t = rng.permutation(S)[:N].astype(np.int32)
        t[rng.choice(N, 2, replace=False)] = np.array([-1, S], dtype=np.int32)
        tabs.append(t)
    return tabs


def test_layer_slot_table(orc):
    """A pool of 24 slots, 10 rows per step naming different slots (two rows
    skipped each step): the oracle's slot semantics, skipped rows read 0 and
    slots no row names keep their bits."""
    N, S = 10, 24
    d = gi.make_decode_raw(4, N, 2, 4, 128, 64, seed=72)
    rng = np.random.default_rng(72)
    pool0 = (rng.standard_normal((S, 4, 64, 128)) * 0.05).astype(np.float32)
    tabs = _slot_tables(rng, d.steps, N, S)
    say("layer slot table")
    o, pool, _ = _gpu_chain(d, pool0, tabs, scale=128 ** -0.5, l2norm=True)
    o_ref, pool_ref = _oracle_chain(orc, d, pool0, tabs, scale=128 ** -0.5, l2norm=True)
    assert_parity(host(o), host(pool), o_ref, pool_ref, what="layer slots")
    for t, tab in enumerate(tabs):
        skipped = (tab < 0) | (tab >= S)
        assert np.all(host(o)[t][skipped] == 0.0)
    named = np.unique(np.concatenate([t[(t >= 0) & (t < S)] for t in tabs]))
    untouched = np.setdiff1d(np.arange(S), named)
    assert untouched.size > 0
    assert np.array_equal(pool.cpu().numpy()[untouched], pool0[untouched])


@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_layer_fused_norm(orc, ydt):
    """Everything at once: slots, raw gates, q/k norm, RMSNormGated (y and o)."""
    import torch
    N, S = 8, 12
    d = gi.make_decode_raw(3, N, 2, 4, 128, 128, seed=73, gate_dtype="bf16")
    rng = np.random.default_rng(73)
    pool0 = (rng.standard_normal((S, 4, 128, 128)) * 0.05).astype(np.float32)
    tabs = _slot_tables(rng, d.steps, N, S)
    say(f"layer fused norm y={ydt}")
    o, pool, y = _gpu_chain(d, pool0, tabs, scale=128 ** -0.5, l2norm=True, norm=True,
                            out_dtype=torch_dtype(ydt))
    o_ref, pool_ref = _oracle_chain(orc, d, pool0, tabs, scale=128 ** -0.5, l2norm=True)
    y_ref = orc.rmsnorm_gated(o_ref, d.z, d.w)
    assert_parity(host(o), host(pool), o_ref, pool_ref, what="layer fused o")
    err = rel_l2(host(y), y_ref)
    print(f"[parity] layer fused y ({ydt}): rel-L2 {err:.3e}")
    assert err <= (4e-3 if ydt == "bf16" else 2e-3), err
    for t, tab in enumerate(tabs):
        skipped = (tab < 0) | (tab >= S)
        assert np.all(host(y)[t][skipped] == 0.0)


def test_layer_activated_gates_equal_decode_step():
    """With activated gates, no slot table and no norm the layer step advances
    the state exactly as gdn_decode_step does."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    d = gi.make_decode(3, 8, 4, 8, 128, 128, seed=74)
    S0 = (np.random.default_rng(74).standard_normal((8, 8, 128, 128)) * 0.02).astype(np.float32)
    bf = torch.bfloat16
    q, k, v, g, b = dev(d.q, bf), dev(d.k, bf), dev(d.v, bf), dev(d.g), dev(d.beta)
    s1, s2 = dev(S0), dev(S0)
    say("layer (activated gates) vs decode_step")
    for t in range(d.steps):
        o1 = gdn.decode_layer(q[t], k[t], v[t], s1, g=g[t], beta=b[t])
        o2 = gdn.decode_step(q[t], k[t], v[t], g[t], b[t], s2)
        torch.cuda.synchronize()
        assert rel_l2(host(o1), host(o2)) <= 1e-6
        assert float((s1 - s2).abs().max()) <= 1e-6
    print(f"[parity] layer vs decode_step bitwise: {bool(torch.equal(s1, s2))}")


def test_layer_full_size_gva(orc):
    """The 35B-A3B decode shape (128 rows, 16 key / 32 value heads, d = 128)
    served from a pool of 256 slots with raw gates, q/k norm and RMSNormGated,
    in the launch configuration of the benchmark; four steps against the
    oracle on every output and on every advanced slot."""
    N, S, H, HV = 128, 256, 16, 32
    d = gi.make_decode_raw(4, N, H, HV, 128, 128, seed=75, gate_dtype="bf16")
    rng = np.random.default_rng(75)
    pool0 = (rng.standard_normal((S, HV, 128, 128)) * 0.02).astype(np.float32)
    tabs = [rng.permutation(S)[:N].astype(np.int32) for _ in range(d.steps)]
    say("layer full size GVA 128 rows, 256 slots")
    o, pool, y = _gpu_chain(d, pool0, tabs, scale=128 ** -0.5, l2norm=True, norm=True)
    o_ref, pool_ref = _oracle_chain(orc, d, pool0, tabs, scale=128 ** -0.5, l2norm=True)
    y_ref = orc.rmsnorm_gated(o_ref, d.z, d.w)
    assert_parity(host(o), host(pool), o_ref, pool_ref, what="layer full size")
    err = rel_l2(host(y), y_ref)
    print(f"[parity] layer full size y: rel-L2 {err:.3e}")
    assert err <= 2e-3
    head_errors(host(y), y_ref).check(what="layer full size y")


def test_layer_bf16_gates_odd_count(orc):
    """bf16 raw gates whose count N HV is odd, on the streamed schedule (1025
    rows of one head: 1025 workgroups), over two steps.  The first step's
    gates start dword-aligned, and the dword holding the last one would reach
    past the array; the second step's are a slice that starts 2 bytes into a
    dword (2050 bytes into the buffer), so every row's gate sits in the other
    half of its dword and the first row's dword would start before the array.
    Every row of both steps against the oracle."""
    N = 1025
    d = gi.make_decode_raw(2, N, 1, 1, 128, 128, seed=78, gate_dtype="bf16")
    S0 = (np.random.default_rng(78).standard_normal((N, 1, 128, 128)) * 0.02).astype(np.float32)
    say("layer bf16 gates, odd count 1025 x 1 head (streamed)")
    o, S, y = _gpu_chain(d, S0, None, scale=128 ** -0.5, l2norm=True, norm=True)
    o_ref, S_ref = _oracle_chain(orc, d, S0, None, scale=128 ** -0.5, l2norm=True)
    y_ref = orc.rmsnorm_gated(o_ref, d.z, d.w)
    assert_parity(host(o), host(S), o_ref, S_ref, what="layer bf16 gates odd count")
    oh = host(o)
    for t in range(d.steps):  # the first and last rows on their own
        assert rel_l2(oh[t, 0], o_ref[t, 0]) <= 1e-3 and rel_l2(oh[t, N - 1], o_ref[t, N - 1]) <= 1e-3
    err = rel_l2(host(y), y_ref)
    print(f"[parity] layer bf16 gates odd count y: rel-L2 {err:.3e}")
    assert err <= 2e-3


def test_layer_graph_replay_matches_eager():
    """The layer step captured in a HIP graph, replayed several times with eager
    work in between, gives the eager results on every replay."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    N, S = 16, 32
    d = gi.make_decode_raw(1, N, 2, 4, 128, 128, seed=76)
    rng = np.random.default_rng(76)
    pool0 = (rng.standard_normal((S, 4, 128, 128)) * 0.02).astype(np.float32)
    slots = dev(rng.permutation(S)[:N].astype(np.int32))
    bf = torch.bfloat16
    q, k, v, z = dev(d.q[0], bf), dev(d.k[0], bf), dev(d.v[0], bf), dev(d.z[0], bf)
    a_raw, b_raw, A_log, dt_bias, w = (dev(d.a_raw[0]), dev(d.b_raw[0]), dev(d.A_log),
                                       dev(d.dt_bias), dev(d.w))
    pool_e, pool_g = dev(pool0), dev(pool0)
    y_g = torch.empty((N, 4, 128), device="cuda")

    def step(pool, y):
        return gdn.decode_layer(q, k, v, pool, a_raw=a_raw, b_raw=b_raw, A_log=A_log,
                                dt_bias=dt_bias, slots=slots, qk_l2norm=True, z=z, w=w, y=y,
                                scale=128 ** -0.5)

    say("layer graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(dev(pool0), torch.empty_like(y_g))  # warm-up outside the graph
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            step(pool_g, y_g)
    torch.cuda.synchronize()
    pool_g.copy_(dev(pool0))
    torch.cuda.synchronize()
    for rep in range(4):
        y_e = step(pool_e, None)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_e, y_g), rep
        assert torch.equal(pool_e, pool_g), rep
        _ = (y_e * 2).sum().item()  # eager work between replays

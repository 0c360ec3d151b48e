"""gdn_prefill_chunked on the GPU against the fp64 oracle, element by element.

Workloads at full size (the oracle finishes each in seconds), ragged and empty
sequences, every supported head size, grouped value heads, packed vs separate
sequences, chaining, aliasing and run-to-run determinism.
"""
import numpy as np
import pytest

import gdn_inputs as gi
from gpu_helpers import (assert_parity, dev, gpu_prefill, host, oracle_prefill, rel_l2, say,
                         torch_dtype)

pytestmark = pytest.mark.gpu


def test_prefill_varlen_at_the_token_cap(orc):
    """The long-context varlen prefill at its largest size: 8 packed sequences
    of 131,072 tokens in all, the longest at the 65,536-token maximum and the
    shortest at the 256-token minimum, 16 key / 32 value heads, S0 ~ N(0, 0.02);
    the library's own choice of scan.  Compared sequence by sequence, so the
    fp64 outputs are never held whole."""
    from gpu_helpers import O_REL_L2, S_MAX_ABS, HeadErrors
    lengths = list(gi.CAP_LENGTHS)
    assert sum(lengths) == 131072 and max(lengths) == 65536 and min(lengths) == 256
    x = gi.make_prefill(lengths, 16, 32, 128, 128, s0_std=0.02, seed=131)
    say(f"prefill varlen at the token cap: lengths={lengths}")
    o, S = gpu_prefill(x)
    Sh = host(S)
    num = den = 0.0
    worst = 0.0
    heads = HeadErrors()
    cu = x.cu_seqlens
    for n in range(x.N):
        a, e = int(cu[n]), int(cu[n + 1])
        o_ref, S_ref = orc.recurrence(x.q[a:e], x.k[a:e], x.v[a:e], x.g[a:e], x.beta[a:e],
                                      np.array([0, e - a], np.int32), s0=x.s0[n:n + 1])
        og = host(o[a:e])
        num += float(np.sum((og - o_ref) ** 2))
        den += float(np.sum(o_ref ** 2))
        worst = max(worst, float(np.max(np.abs(Sh[n] - S_ref[0]))))
        heads.outputs(og, o_ref, seq_offset=n)
        heads.state(Sh[n:n + 1], S_ref, seq_offset=n)
        del o_ref, og
    ro = (num / den) ** 0.5
    print(f"[parity] token cap: o rel-L2 {ro:.3e}, state max-abs {worst:.3e}", flush=True)
    assert ro <= O_REL_L2 and worst <= S_MAX_ABS
    heads.check(what="token cap")


def test_prefill_tiny_d16_fp32(orc):
    x = gi.workload(0)
    say("prefill tiny d=16 fp32")
    o, S = gpu_prefill(x)
    o_ref, S_ref = oracle_prefill(orc, x)
    assert_parity(host(o), host(S), o_ref, S_ref, f32=True, what="prefill workload 0",
                  cu=x.cu_seqlens)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_prefill_full_workload(orc, cfg):
    x = gi.workload(cfg)
    say(f"prefill workload {cfg}: N={x.N} T={x.T} H={x.H} HV={x.HV} lengths={list(x.lengths)}")
    o, S = gpu_prefill(x)
    o_ref, S_ref = oracle_prefill(orc, x)
    assert_parity(host(o), host(S), o_ref, S_ref, what=f"prefill workload {cfg}", cu=x.cu_seqlens)


@pytest.mark.parametrize("scale", [1.0, 128 ** -0.5])
def test_prefill_ragged_and_empty(orc, scale):
    lengths = [0, 1, 63, 64, 65, 130, 0, 200, 2]
    x = gi.make_prefill(lengths, 2, 4, 128, 128, s0_std=0.02, seed=3)
    say(f"prefill ragged lengths={lengths} scale={scale}")
    o, S = gpu_prefill(x, scale=scale)
    o_ref, S_ref = oracle_prefill(orc, x, scale=scale)
    assert_parity(host(o), host(S), o_ref, S_ref, what="ragged/empty", cu=x.cu_seqlens)
    # empty sequences return their initial state exactly
    Sh = S.cpu().numpy()
    assert np.array_equal(Sh[0], x.s0[0]) and np.array_equal(Sh[6], x.s0[6])


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (32, 64), (64, 32), (64, 64),
                                   (128, 16), (128, 32), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_head_sizes(orc, dk, dv, dtype):
    x = gi.make_prefill([70, 5, 129], 2, 4, dk, dv, dtype=dtype, s0_std=0.05, seed=dk + dv)
    say(f"prefill dk={dk} dv={dv} {dtype}")
    o, S = gpu_prefill(x, scale=dk ** -0.5)
    o_ref, S_ref = oracle_prefill(orc, x, scale=dk ** -0.5)
    assert_parity(host(o), host(S), o_ref, S_ref, f32=(dtype == "f32"),
                  what=f"dk={dk} dv={dv} {dtype}", cu=x.cu_seqlens)


def test_prefill_mild_decay_long_memory(orc):
    """Slow decay (g = -0.02 softplus(x)) keeps the state alive across many
    chunks, so the inter-chunk state path carries the result."""
    x = gi.make_prefill([1000, 333], 2, 4, 128, 128, decay="mild", s0_std=0.02, seed=11)
    say("prefill mild decay")
    o, S = gpu_prefill(x, scale=128 ** -0.5)
    o_ref, S_ref = oracle_prefill(orc, x, scale=128 ** -0.5)
    assert_parity(host(o), host(S), o_ref, S_ref, what="mild decay", cu=x.cu_seqlens)


def test_prefill_gva_equals_repeated_heads():
    """HV = 2H equals a call with H' = HV and q, k repeated per value head."""
    x = gi.make_prefill([100, 64], 2, 4, 128, 128, seed=5)
    say("prefill GVA vs repeated heads")
    o1, S1 = gpu_prefill(x)
    y = gi.PrefillInputs(np.repeat(x.q, 2, axis=1), np.repeat(x.k, 2, axis=1), x.v, x.g, x.beta,
                         x.z, x.w, x.cu_seqlens, x.s0, x.dtype, 4, 4, 128, 128)
    o2, S2 = gpu_prefill(y)
    assert np.array_equal(o1.cpu().numpy(), o2.cpu().numpy())
    assert np.array_equal(S1.cpu().numpy(), S2.cpu().numpy())


def test_prefill_packed_equals_separate():
    x = gi.make_prefill([77, 0, 128, 3], 1, 2, 64, 64, s0_std=0.1, seed=6)
    say("prefill packed vs separate")
    o, S = gpu_prefill(x)
    o, S = o.cpu().numpy(), S.cpu().numpy()
    cu = x.cu_seqlens
    for n in range(x.N):
        a, e = cu[n], cu[n + 1]
        y = gi.PrefillInputs(x.q[a:e], x.k[a:e], x.v[a:e], x.g[a:e], x.beta[a:e], x.z[a:e], x.w,
                             np.array([0, e - a], np.int32), x.s0[n:n + 1], x.dtype, 1, 2, 64, 64)
        on, Sn = gpu_prefill(y)
        assert np.array_equal(o[a:e], on.cpu().numpy())
        assert np.array_equal(S[n], Sn.cpu().numpy()[0])


def test_prefill_split_equals_whole(orc):
    """prefill(A) then prefill(B) from the returned state equals prefill(A+B)
    (incremental equals whole-sequence processing)."""
    x = gi.make_prefill([300], 2, 4, 128, 128, decay="mild", seed=8)
    cut = 131
    say("prefill split vs whole")
    o_all, S_all = gpu_prefill(x)
    part = lambda a, e, s0: gi.PrefillInputs(x.q[a:e], x.k[a:e], x.v[a:e], x.g[a:e],
                                             x.beta[a:e], x.z[a:e], x.w,
                                             np.array([0, e - a], np.int32), s0, x.dtype, 2, 4,
                                             128, 128)
    o1, S1 = gpu_prefill(part(0, cut, None))
    o2, S2 = gpu_prefill(part(cut, 300, None), s0=S1)
    o_ref, S_ref = oracle_prefill(orc, x)
    o_split = np.concatenate([host(o1), host(o2)])
    assert_parity(o_split, host(S2), o_ref, S_ref, what="split prefill", cu=x.cu_seqlens)
    assert_parity(host(o_all), host(S_all), o_ref, S_ref, what="whole prefill", cu=x.cu_seqlens)


def test_prefill_final_state_may_alias_initial():
    import gated_delta_rule_decode_amd as gdn
    x = gi.make_prefill([90, 40], 2, 2, 64, 128, s0_std=0.1, seed=9)
    say("prefill aliasing final == initial")
    o1, S1 = gpu_prefill(x)
    dt = torch_dtype(x.dtype)
    st = dev(x.s0)
    o2, S2 = gdn.prefill_chunked(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta),
                                 dev(x.cu_seqlens), initial_state=st, final_state=st)
    assert S2.data_ptr() == st.data_ptr()
    assert np.array_equal(o1.cpu().numpy(), o2.cpu().numpy())
    assert np.array_equal(S1.cpu().numpy(), st.cpu().numpy())


def test_prefill_deterministic():
    x = gi.make_prefill([500, 257], 2, 4, 128, 128, s0_std=0.02, seed=10)
    say("prefill determinism")
    o1, S1 = gpu_prefill(x)
    o2, S2 = gpu_prefill(x)
    assert np.array_equal(o1.cpu().numpy(), o2.cpu().numpy())
    assert np.array_equal(S1.cpu().numpy(), S2.cpu().numpy())


def test_prefill_bf16_output(orc):
    import torch
    x = gi.make_prefill([200, 64], 2, 4, 128, 128, seed=12)
    say("prefill bf16 output")
    o, S = gpu_prefill(x, out_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    o_ref, S_ref = oracle_prefill(orc, x)
    # rounding o alone to bf16 costs about 1.6e-3 rel-L2
    r = rel_l2(host(o), o_ref)
    assert r <= 4e-3, r


def test_prefill_nan_stays_in_its_sequence():
    """A NaN in one sequence's values leaves every other sequence bit-identical."""
    x = gi.make_prefill([70, 70, 70], 1, 2, 64, 64, seed=13)
    say("prefill NaN isolation")
    o1, S1 = gpu_prefill(x)
    v = x.v.copy()
    v[70 + 5, 1, 3] = np.nan
    y = gi.PrefillInputs(x.q, x.k, v, x.g, x.beta, x.z, x.w, x.cu_seqlens, x.s0, x.dtype, 1, 2,
                         64, 64)
    o2, S2 = gpu_prefill(y)
    o1, o2, S1, S2 = (t.cpu().numpy() for t in (o1, o2, S1, S2))
    for n in (0, 2):
        sl = slice(70 * n, 70 * n + 70)
        assert np.array_equal(o1[sl], o2[sl])
        assert np.array_equal(S1[n], S2[n])
    assert np.array_equal(o1[70:140, 0], o2[70:140, 0])  # the other head too
    assert np.isnan(o2[70 + 5:140, 1]).any()


def test_prefill_zero_tokens_copies_state():
    import torch
    import gated_delta_rule_decode_amd as gdn
    N, H, HV, d = 3, 1, 2, 32
    s0 = torch.randn(N, HV, d, d, device="cuda")
    e = torch.empty(0, H, d, device="cuda")
    ev = torch.empty(0, HV, d, device="cuda")
    eg = torch.empty(0, HV, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    say("prefill with zero tokens")
    o, S = gdn.prefill_chunked(e, e, ev, eg, eg, cu, initial_state=s0)
    assert torch.equal(S, s0)
    o, S = gdn.prefill_chunked(e, e, ev, eg, eg, cu)
    assert torch.count_nonzero(S).item() == 0


@pytest.mark.parametrize("ratio", [1, 3, 4, 6, 8])
def test_prefill_value_heads_per_key_head(orc, ratio):
    """1, 3, 4, 6 and 8 value heads per key head on the MFMA kernels, which
    take any ratio: the prep forms K K^T once per key head and takes its value
    heads one at a time for an odd count, two at a time for an even one (3:
    three single passes; 6: three paired passes)."""
    x = gi.make_prefill([130, 70, 1], 1, ratio, 128, 128, dtype="bf16", s0_std=0.05,
                        seed=40 + ratio)
    say(f"prefill value heads per key head = {ratio}")
    o, S = gpu_prefill(x)
    o_ref, S_ref = oracle_prefill(orc, x)
    assert_parity(host(o), host(S), o_ref, S_ref, what=f"value heads per key head {ratio}",
                  cu=x.cu_seqlens)


def _lengths_many(seed, n, hi):
    rng = np.random.default_rng(seed)
    out = [int(x) for x in rng.integers(0, hi, size=n)]
    out[0], out[1], out[2], out[3] = 0, 1, 64, 65  # empty, one token, whole and ragged chunks
    return out


@pytest.mark.parametrize("H,HV,N", [(16, 16, 32), (8, 16, 32), (16, 32, 16)])
def test_prefill_many_chains_matches_oracle(orc, H, HV, N):
    """At least 512 (sequence, value head) chains at d = 128: 2048 or more
    (chain, 32-row tile) items, taken by the CUs in turn."""
    lengths = _lengths_many(100 + HV + N, N, 300)
    x = gi.make_prefill(lengths, H, HV, 128, 128, s0_std=0.02, seed=101 + H)
    say(f"prefill many chains: N={N} H={H} HV={HV} T={sum(lengths)}")
    o, S = gpu_prefill(x, scale=128 ** -0.5)
    o_ref, S_ref = oracle_prefill(orc, x, scale=128 ** -0.5)
    assert_parity(host(o), host(S), o_ref, S_ref, what=f"many chains H={H} HV={HV}",
                  cu=x.cu_seqlens)


@pytest.mark.parametrize("N", [255, 256, 257, 300])
def test_prefill_batches_of_hundreds_of_sequences(orc, N):
    """Batches of a few hundred short prompts at d = 128 (the planner's block
    scans take 256 sequences per round, so both sides of that size), with
    empty, one-token, whole-chunk and ragged prompts."""
    lengths = _lengths_many(200 + N, N, 140)
    x = gi.make_prefill(lengths, 2, 4, 128, 128, s0_std=0.02, seed=300 + N)
    say(f"prefill batch of {N} sequences: T={sum(lengths)}")
    o, S = gpu_prefill(x, scale=128 ** -0.5)
    o_ref, S_ref = oracle_prefill(orc, x, scale=128 ** -0.5)
    assert_parity(host(o), host(S), o_ref, S_ref, what=f"batch of {N} sequences",
                  cu=x.cu_seqlens)


def test_prefill_result_does_not_depend_on_the_batch():
    """Every (chain, 32-row tile) item runs the same code on its own data, so
    the same sequences give the same outputs and final states bit for bit in
    one call of 512 chains and in two calls of 256."""
    lengths = _lengths_many(7, 32, 400)
    x = gi.make_prefill(lengths, 16, 16, 128, 128, s0_std=0.02, decay="mild", seed=102)
    say("prefill: one call of 512 chains vs two of 256")
    o, S = gpu_prefill(x, scale=128 ** -0.5)
    o, S = host(o), host(S)
    cu = x.cu_seqlens
    for half in (slice(0, 16), slice(16, 32)):
        a, e = cu[half.start], cu[half.stop]
        y = gi.PrefillInputs(x.q[a:e], x.k[a:e], x.v[a:e], x.g[a:e], x.beta[a:e], x.z[a:e], x.w,
                             (cu[half.start:half.stop + 1] - a).astype(np.int32), x.s0[half],
                             x.dtype, 16, 16, 128, 128)
        oh, Sh = gpu_prefill(y, scale=128 ** -0.5)
        assert np.array_equal(host(oh), o[a:e]) and np.array_equal(host(Sh), S[half])


def test_prefill_many_chains_forced_segments(orc):
    """Forced segments with 512 chains: transition items (from the identity,
    V = 0), the combine and the correction passes."""
    lengths = [2100] * 8 + [0, 70] + [1500] * 22
    x = gi.make_prefill(lengths, 16, 16, 128, 128, s0_std=0.02, decay="mild", seed=103)
    say(f"prefill many chains, segments of 32 chunks: T={sum(lengths)}")
    o, S = gpu_prefill(x, scale=128 ** -0.5, segment_chunks=32)
    o_ref, S_ref = oracle_prefill(orc, x, scale=128 ** -0.5)
    assert_parity(host(o), host(S), o_ref, S_ref, what="many chains, segmented", cu=x.cu_seqlens)

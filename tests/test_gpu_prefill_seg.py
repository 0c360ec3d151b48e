"""The segment-parallel scan of gdn_prefill_chunked on the GPU against the
fp64 oracle.

A segment is a run of whole chunks of one sequence; every segment after the
first runs from a zero state and from the identity (its transition), and the
segments are then chained and their outputs corrected.  The tests force
segment lengths (32 chunks, the shortest) on sequences a few segments long,
mix segmented and unsegmented sequences in one packed batch, and run the
automatic choice on one long prompt at full size.
"""
import numpy as np
import pytest

import gdn_inputs as gi
from gpu_helpers import (O_REL_L2, S_MAX_ABS, HeadErrors, assert_parity, gpu_prefill, host,
                         oracle_prefill, rel_l2, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lengths,H,HV,dk,dv", [
    ([6000], 1, 1, 128, 128),          # 94 chunks: segments of 32, 32, 30
    ([4097], 1, 2, 128, 64),           # a one-token last chunk; two value heads per key head
    ([8192], 2, 2, 64, 128),           # d_k = 64
    ([2048, 5000, 100, 0, 4100], 2, 4, 128, 128),  # segmented and whole sequences, an empty one
])
@pytest.mark.parametrize("with_s0", [False, True])
def test_forced_segments_match_oracle(orc, lengths, H, HV, dk, dv, with_s0):
    x = gi.make_prefill(lengths, H, HV, dk, dv, s0_std=0.02 if with_s0 else 0.0,
                        seed=sum(lengths) + dk)
    say(f"prefill segments of 32 chunks: lengths={lengths} H={H} HV={HV} dk={dk} dv={dv} s0={with_s0}")
    o, S = gpu_prefill(x, scale=dk ** -0.5, segment_chunks=32)
    o_ref, S_ref = oracle_prefill(orc, x, scale=dk ** -0.5)
    assert_parity(host(o), host(S), o_ref, S_ref, what=f"segmented {lengths}", cu=x.cu_seqlens)


def test_segmented_equals_whole_scan(orc):
    """Forced segments, segmentation off and the automatic choice give the
    same outputs and states to well inside the parity bar."""
    x = gi.make_prefill([7000, 3000], 2, 4, 128, 128, s0_std=0.02, seed=91)
    say("prefill segmented vs whole")
    o1, S1 = gpu_prefill(x, scale=128 ** -0.5, segment_chunks=32)
    o2, S2 = gpu_prefill(x, scale=128 ** -0.5, segment_chunks=-1)
    o3, S3 = gpu_prefill(x, scale=128 ** -0.5, segment_chunks=0)
    r12 = rel_l2(host(o1), host(o2))
    s12 = float(np.max(np.abs(host(S1) - host(S2))))
    print(f"[parity] segmented vs whole: o rel-L2 {r12:.3e}, state max-abs {s12:.3e}")
    assert r12 <= 2e-5 and s12 <= 2e-5
    assert rel_l2(host(o3), host(o2)) <= 2e-5


def test_segmented_bf16_output(orc):
    import torch
    x = gi.make_prefill([5000], 2, 2, 128, 128, seed=92)
    say("prefill segmented, bf16 output")
    o, S = gpu_prefill(x, scale=128 ** -0.5, segment_chunks=32, out_dtype=torch.bfloat16)
    o_ref, S_ref = oracle_prefill(orc, x, scale=128 ** -0.5)
    err = rel_l2(host(o), o_ref)
    print(f"[parity] segmented bf16 o: rel-L2 {err:.3e}")
    assert err <= 4e-3
    assert float(np.max(np.abs(host(S) - S_ref))) <= 1e-3


def test_segmented_final_state_may_alias_initial(orc):
    import torch
    import gated_delta_rule_decode_amd as gdn
    from gpu_helpers import dev
    x = gi.make_prefill([4500, 300], 1, 2, 128, 128, s0_std=0.02, seed=93)
    bf = torch.bfloat16
    q, k, v = dev(x.q, bf), dev(x.k, bf), dev(x.v, bf)
    g, b, cu = dev(x.g), dev(x.beta), dev(x.cu_seqlens.astype(np.int32))
    S = dev(x.s0)
    say("prefill segmented, final state in place")
    o, _ = gdn.prefill_chunked(q, k, v, g, b, cu, initial_state=S, final_state=S,
                               segment_chunks=32)
    o_ref, S_ref = oracle_prefill(orc, x)
    assert_parity(host(o), host(S), o_ref, S_ref, what="segmented in place", cu=x.cu_seqlens)


def test_long_prompt_automatic(orc):
    """One 32768-token prompt at the 0.8B shape (16 heads, d = 128): the
    automatic choice, against the oracle on every output and state."""
    x = gi.make_prefill([32768], 16, 16, 128, 128, seed=94)
    say("prefill one 32768-token prompt, automatic segmentation")
    o, S = gpu_prefill(x, scale=128 ** -0.5)
    o_ref, S_ref = oracle_prefill(orc, x, scale=128 ** -0.5)
    assert_parity(host(o), host(S), o_ref, S_ref, what="long prompt automatic", cu=x.cu_seqlens)


def _long_memory(x):
    """The same inputs with a decay near 1 (g scaled by 1e-5) and a weak
    write strength (beta scaled by 0.02): the state carries across thousands
    of tokens, so a segment's entry state shapes its outputs and end state."""
    x.g = (x.g * np.float32(1e-5)).astype(np.float32)
    x.beta = (x.beta * np.float32(0.02)).astype(np.float32)
    return x


@pytest.mark.parametrize("lengths,H,HV,dk,dv", [
    ([6000], 1, 2, 128, 128),
    ([2048, 5000, 4100], 2, 4, 128, 64),
    ([7000], 1, 1, 64, 128),
])
def test_long_memory_segments_match_oracle(orc, lengths, H, HV, dk, dv):
    x = _long_memory(gi.make_prefill(lengths, H, HV, dk, dv, s0_std=0.5, seed=7 + sum(lengths)))
    # the carried state matters: the oracle's final state moves with S0
    _, S_a = oracle_prefill(orc, x)
    _, S_b = oracle_prefill(orc, x, s0=np.zeros_like(x.s0))
    assert float(np.max(np.abs(S_a - S_b))) > 0.1
    say(f"prefill long memory, segments of 32 chunks: lengths={lengths} dk={dk} dv={dv}")
    o, S = gpu_prefill(x, scale=dk ** -0.5, segment_chunks=32)
    o_ref, S_ref = oracle_prefill(orc, x, scale=dk ** -0.5)
    assert_parity(host(o), host(S), o_ref, S_ref, what=f"long memory segmented {lengths}",
                  cu=x.cu_seqlens)
    o2, S2 = gpu_prefill(x, scale=dk ** -0.5, segment_chunks=-1)
    r = rel_l2(host(o), host(o2))
    d = float(np.max(np.abs(host(S) - host(S2))))
    print(f"[parity] long memory segmented vs whole: o rel-L2 {r:.3e}, state max-abs {d:.3e}")
    assert r <= 2e-5 and d <= 2e-5


@pytest.mark.parametrize("segment_chunks", [0, 32, -1])
def test_prefill_graph_replay_matches_eager(segment_chunks):
    """The prefill (planner, prep, scan and, when segmented, the combine and
    correction passes) captured in a HIP graph: every replay, with eager work
    and synchronisations between the replays, equals the eager call bit for
    bit."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    x = gi.make_prefill([4500, 300, 2100], 2, 4, 128, 128, s0_std=0.02, seed=93)
    say(f"prefill graph replay vs eager, segment_chunks={segment_chunks}")
    bf = torch.bfloat16
    q, k, v = (torch.from_numpy(a).to("cuda", bf) for a in (x.q, x.k, x.v))
    g, b = torch.from_numpy(x.g).cuda(), torch.from_numpy(x.beta).cuda()
    cu = torch.from_numpy(x.cu_seqlens.astype(np.int32)).cuda()
    s0 = torch.from_numpy(x.s0).cuda()
    T, N = int(x.cu_seqlens[-1]), len(x.cu_seqlens) - 1
    o = torch.empty(T, 4, 128, device="cuda")
    sf = torch.empty(N, 4, 128, 128, device="cuda")
    ws = torch.empty(gdn.prefill_workspace_bytes(N, T, 2, 4, 128, 128,
                                                 segment_chunks=segment_chunks),
                     dtype=torch.uint8, device="cuda")

    def run():
        gdn.prefill_chunked(q, k, v, g, b, cu, initial_state=s0, final_state=sf, o=o,
                            workspace=ws, scale=128 ** -0.5, segment_chunks=segment_chunks)

    run()
    torch.cuda.synchronize()
    o_eager, s_eager = o.clone(), sf.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=s):
        run()
    for rep in range(4):
        o.zero_()
        sf.zero_()
        ws.fill_(0xAB)  # the workspace holds nothing across calls
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), f"replay {rep}: outputs differ"
        assert torch.equal(sf, s_eager), f"replay {rep}: final states differ"
        _ = (o * 2).sum().item()  # eager work between replays


@pytest.mark.parametrize("mode", [-2, 0])
def test_skewed_batch_automatic(orc, mode):
    """A batch whose chains already fill the CUs (16 x 32 = 512) but whose
    longest sequence is 32 times the rest: with segment_chunks = -2 the
    planner cuts that sequence into segments, which run beside the short ones;
    with 0 it runs unsegmented.  Compared with the oracle sequence by
    sequence."""
    lengths, H, HV = [32768] + [1024] * 15, 16, 32
    x = gi.make_prefill(lengths, H, HV, 128, 128, s0_std=0.02, seed=95 + len(lengths))
    say(f"prefill skewed batch, mode {mode}: lengths={lengths[:4]}.. N={len(lengths)} HV={HV}")
    o, S = gpu_prefill(x, segment_chunks=mode)
    Sh = host(S)
    num = den = worst = 0.0
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
    ro = (num / den) ** 0.5
    print(f"[parity] skewed batch: o rel-L2 {ro:.3e}, state max-abs {worst:.3e}", flush=True)
    heads.check(what=f"skewed batch mode {mode}")
    assert ro <= O_REL_L2 and worst <= S_MAX_ABS

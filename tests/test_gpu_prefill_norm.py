"""gdn_prefill_chunked_norm on the GPU: the chunked prefill followed by
RMSNormGated of every (token, value head).  The library runs the norm as a
second launch on fp32 outputs kept in the workspace (a head's outputs come
from four workgroups, one per 32 state rows).  Checked against the fp64
oracle (the norm of the oracle's outputs) and, bit for bit, against the two
separate calls.
"""
import dataclasses

import numpy as np
import pytest

import gdn_inputs as gi
from gpu_helpers import (O_REL_L2, S_MAX_ABS, dev, gpu_prefill, head_errors, host, max_abs,
                         oracle_prefill, rel_l2, say, torch_dtype)

pytestmark = pytest.mark.gpu


def _lengths_many(seed, n, hi):
    rng = np.random.default_rng(seed)
    out = [int(x) for x in rng.integers(0, hi, size=n)]
    out[0], out[1], out[2], out[3] = 0, 1, 64, 65  # empty, one token, whole and ragged chunks
    return out


def _norm_call(x, *, scale, zd="bf16", wd="f32", yd="f32", return_o=False, final=True):
    import torch
    import gated_delta_rule_decode_amd as gdn
    dt = torch_dtype(x.dtype)
    cu = dev(x.cu_seqlens.astype(np.int32))
    init = dev(x.s0) if x.s0 is not None else None
    return gdn.prefill_chunked_norm(dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g),
                                    dev(x.beta), cu, dev(x.z, torch_dtype(zd)),
                                    dev(x.w, torch_dtype(wd)), initial_state=init, scale=scale,
                                    eps=1e-6, out_dtype=torch_dtype(yd), return_o=return_o,
                                    return_final_state=final)


def _two_calls(x, *, scale, zd="bf16", wd="f32", yd="f32"):
    """gdn_prefill_chunked (fp32 outputs) then gdn_rmsnorm_gated."""
    import gated_delta_rule_decode_amd as gdn
    o, S = gpu_prefill(x, scale=scale)
    y = gdn.rmsnorm_gated(o, dev(x.z, torch_dtype(zd)), dev(x.w, torch_dtype(wd)), eps=1e-6,
                          out_dtype=torch_dtype(yd))
    return y, S, o


def _norm_lengths(kind, HV, N):
    if kind == "many":      # >= 512 chains, short sequences: one segment each
        return _lengths_many(300 + HV + N, N, 300)
    if kind == "long":      # one long prompt on few chains: segmented
        return [20000]
    return [32768] + [1024] * 15  # "skewed": 512 chains, unsegmented


@pytest.mark.parametrize("kind,H,HV,N,zd,wd,yd", [("many", 16, 16, 32, "bf16", "f32", "f32"),
                                                  ("many", 8, 16, 32, "f32", "bf16", "f32"),
                                                  ("many", 16, 32, 16, "bf16", "bf16", "bf16"),
                                                  ("long", 4, 4, 1, "bf16", "f32", "f32"),
                                                  ("long", 2, 4, 1, "f32", "f32", "bf16"),
                                                  ("skewed", 16, 32, 16, "bf16", "f32", "f32")])
def test_prefill_norm_matches_oracle(orc, kind, H, HV, N, zd, wd, yd):
    lengths = _norm_lengths(kind, HV, N)
    x = gi.make_prefill(lengths, H, HV, 128, 128, s0_std=0.02,
                        decay="mild" if kind != "many" else "qwen", seed=301 + H)
    # a weight that is not all ones (bf16-exact when passed as bf16)
    wv = (1.0 + 0.5 * np.random.default_rng(HV + N).standard_normal(128)).astype(np.float32)
    x = dataclasses.replace(x, w=gi.round_bf16(wv) if wd == "bf16" else wv)
    say(f"prefill+norm ({kind}): N={len(lengths)} H={H} HV={HV} z={zd} w={wd} y={yd} "
        f"T={sum(lengths)}")
    y, S = _norm_call(x, scale=128 ** -0.5, zd=zd, wd=wd, yd=yd)
    o_ref, S_ref = oracle_prefill(orc, x, scale=128 ** -0.5)
    y_ref = orc.rmsnorm_gated(o_ref, x.z, x.w, eps=1e-6)
    ry, ms = rel_l2(host(y), y_ref), max_abs(host(S), S_ref)
    tol_y = 4e-3 if yd == "bf16" else O_REL_L2
    print(f"[parity] prefill+norm: y rel-L2 {ry:.3e} (<= {tol_y:.0e}), state max-abs {ms:.3e}",
          flush=True)
    assert ry <= tol_y and ms <= S_MAX_ABS
    head_errors(host(y), y_ref, host(S), S_ref, cu=x.cu_seqlens).check(what="prefill+norm y")


@pytest.mark.parametrize("case", ["many", "long-segmented", "few", "dv64-segmented", "with-o"])
def test_prefill_norm_equals_two_calls(case):
    """The call is exactly the two calls, bit for bit: 512 chains, a long
    prompt taken in segments, few chains, d_v = 64 with segments, and a call
    that also asks for the raw outputs."""
    if case == "many":
        x = gi.make_prefill(_lengths_many(7, 32, 400), 16, 16, 128, 128, s0_std=0.02,
                            decay="mild", seed=302)
    elif case == "long-segmented":
        x = gi.make_prefill([30000, 3000], 4, 4, 128, 128, s0_std=0.02, decay="mild", seed=307)
    elif case == "few":
        x = gi.make_prefill([200, 0, 129, 64], 2, 4, 128, 128, s0_std=0.02, seed=303)
    elif case == "dv64-segmented":
        x = gi.make_prefill([20000], 4, 4, 128, 64, s0_std=0.02, decay="mild", seed=304)
    else:
        x = gi.make_prefill(_lengths_many(9, 32, 200), 16, 16, 128, 128, s0_std=0.02, seed=305)
    say(f"prefill+norm {case} vs two calls: lengths={list(x.lengths)[:6]} HV={x.HV}")
    if case == "with-o":
        y, S, o = _norm_call(x, scale=128 ** -0.5, return_o=True)
    else:
        y, S = _norm_call(x, scale=128 ** -0.5)
    y2, S2, o2 = _two_calls(x, scale=128 ** -0.5)
    assert np.array_equal(host(y), host(y2))
    assert np.array_equal(host(S), host(S2))
    if case == "with-o":
        assert np.array_equal(host(o), host(o2))


def test_prefill_norm_graph_replay_matches_eager():
    """The call captured in a HIP graph: every replay, with eager work
    and synchronisations between them, reproduces the eager result."""
    import torch
    import gated_delta_rule_decode_amd as gdn
    x = gi.make_prefill(_lengths_many(11, 32, 150), 16, 16, 128, 128, s0_std=0.02, seed=306)
    say("prefill+norm graph replay")
    dt = torch_dtype(x.dtype)
    args = (dev(x.q, dt), dev(x.k, dt), dev(x.v, dt), dev(x.g), dev(x.beta),
            dev(x.cu_seqlens.astype(np.int32)), dev(x.z, torch.bfloat16), dev(x.w))
    s0 = dev(x.s0)
    y_e, S_e = gdn.prefill_chunked_norm(*args, initial_state=s0, scale=128 ** -0.5)
    torch.cuda.synchronize()
    y = torch.empty_like(y_e)
    S = torch.empty_like(S_e)
    ws = torch.empty(gdn.prefill_norm_workspace_bytes(x.N, x.T, 16, 16, 128, 128),
                     dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gdn.prefill_chunked_norm(*args, initial_state=s0, final_state=S, y=y, workspace=ws,
                                 scale=128 ** -0.5)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        gdn.prefill_chunked_norm(*args, initial_state=s0, final_state=S, y=y, workspace=ws,
                                 scale=128 ** -0.5)
    torch.cuda.synchronize()
    for _ in range(3):
        y.fill_(float("nan"))
        S.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e) and torch.equal(S, S_e)

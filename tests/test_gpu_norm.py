"""gdn_rmsnorm_gated on the GPU against the fp64 oracle."""
import numpy as np
import pytest

import gdn_inputs as gi
from gpu_helpers import dev, gpu_prefill, host, oracle_prefill, rel_l2, say

pytestmark = pytest.mark.gpu


def _cases():
    for dv in (16, 32, 64, 128):
        for xd, zd, wd, yd in (("f32", "f32", "f32", "f32"), ("f32", "bf16", "f32", "f32"),
                               ("bf16", "bf16", "bf16", "bf16"), ("f32", "bf16", "bf16", "bf16")):
            yield dv, xd, zd, wd, yd


@pytest.mark.parametrize("dv,xd,zd,wd,yd", list(_cases()))
def test_norm_parity(orc, dv, xd, zd, wd, yd):
    import torch
    r = np.random.default_rng(dv)
    rows, HV = 37, 3
    x = (r.standard_normal((rows, HV, dv)) * 2).astype(np.float32)
    z = r.standard_normal((rows, HV, dv)).astype(np.float32)
    w = r.standard_normal(dv).astype(np.float32)
    if xd == "bf16":
        x = gi.round_bf16(x)
    if zd == "bf16":
        z = gi.round_bf16(z)
    if wd == "bf16":
        w = gi.round_bf16(w)
    T = {"f32": torch.float32, "bf16": torch.bfloat16}
    import gated_delta_rule_decode_amd as gdn
    say(f"norm dv={dv} x={xd} z={zd} w={wd} y={yd}")
    y = gdn.rmsnorm_gated(dev(x, T[xd]), dev(z, T[zd]), dev(w, T[wd]), eps=1e-6,
                          out_dtype=T[yd])
    y_ref = orc.rmsnorm_gated(x, z, w, eps=1e-6)
    err = rel_l2(host(y), y_ref)
    assert err <= (4e-3 if yd == "bf16" else 2e-6), err


def test_norm_in_place():
    import torch
    import gated_delta_rule_decode_amd as gdn
    r = np.random.default_rng(5)
    x = r.standard_normal((9, 4, 128)).astype(np.float32)
    z = r.standard_normal((9, 4, 128)).astype(np.float32)
    w = np.ones(128, np.float32)
    say("norm in place")
    xt = dev(x)
    y1 = gdn.rmsnorm_gated(xt, dev(z), dev(w))
    y2 = gdn.rmsnorm_gated(xt, dev(z), dev(w), y=xt)
    assert y2.data_ptr() == xt.data_ptr()
    assert torch.equal(y1, xt)


def test_norm_on_mixer_output(orc):
    """End to end: RMSNormGated of the GPU prefill output against the oracle's
    norm of the oracle's output (workload 0 shape and a 128-dim batch)."""
    import gated_delta_rule_decode_amd as gdn
    for x, f32 in ((gi.workload(0), True), (gi.make_prefill([300, 77], 2, 4, 128, 128, seed=4), False)):
        say(f"norm of mixer output dv={x.dv}")
        o, _ = gpu_prefill(x)
        zt = dev(x.z, o.dtype if x.dtype == "f32" else None)
        import torch
        zt = dev(x.z, torch.bfloat16 if x.dtype == "bf16" else torch.float32)
        y = gdn.rmsnorm_gated(o, zt, dev(x.w))
        o_ref, _ = oracle_prefill(orc, x)
        y_ref = orc.rmsnorm_gated(o_ref, x.z, x.w)
        err = rel_l2(host(y), y_ref)
        assert err <= (2e-5 if f32 else 2e-3), err

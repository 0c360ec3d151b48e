"""The C-ABI library loads, exports every declared symbol and validates its
arguments on the host.  No call here reaches a kernel launch: every call either
fails validation (which happens before any HIP call) or is an N == 0 no-op."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_decode_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

FAKE = 0x10000  # an aligned non-null address; validation fails before any use
MISALIGNED = 0x10004


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gdn.LIBRARY):
        import gated_delta_rule_decode_amd.build as b
        b.build()
    return gdn.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(gdn.EXPORTS)
    for name in names:
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_version_and_status_strings(L):
    assert gdn.version() == 200
    for code, name in gdn.STATUS.items():
        assert L.gdn_status_string(code).decode() == name
    assert L.gdn_status_string(99).decode() == "GDN_UNKNOWN_STATUS"


def _decode(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=1, g=FAKE, beta=FAKE, state=FAKE, o=FAKE, o_dt=0,
             N=2, H=2, HV=4, dk=128, dv=128, scale=1.0)
    a.update(kw)
    return L.gdn_decode_step(a["q"], a["k"], a["v"], a["in_dt"], a["g"], a["beta"], a["state"],
                             a["o"], a["o_dt"], a["N"], a["H"], a["HV"], a["dk"], a["dv"],
                             a["scale"], None)


def test_decode_validation(L):
    assert _decode(L, N=0) == 0                      # no-op
    assert _decode(L, N=0, q=None) == 0              # no-op ignores pointers
    assert _decode(L, N=-1) == 1
    assert _decode(L, q=None) == 1
    assert _decode(L, state=None) == 1
    assert _decode(L, o=MISALIGNED) == 1
    assert _decode(L, HV=3) == 1                     # HV % H != 0
    assert _decode(L, H=0) == 1
    assert _decode(L, dk=96) == 2
    assert _decode(L, dv=256) == 2
    assert _decode(L, in_dt=7) == 2
    assert _decode(L, o_dt=-1) == 2


def _prefill(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=1, g=FAKE, beta=FAKE, cu=FAKE, N=2, T=100, s0=None,
             sf=FAKE, o=FAKE, o_dt=0, H=2, HV=4, dk=128, dv=128, chunk=64, scale=1.0,
             ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return L.gdn_prefill_chunked(a["q"], a["k"], a["v"], a["in_dt"], a["g"], a["beta"], a["cu"],
                                 a["N"], a["T"], a["s0"], a["sf"], a["o"], a["o_dt"], a["H"],
                                 a["HV"], a["dk"], a["dv"], a["chunk"], a["scale"], a["ws"],
                                 a["wsb"], None)


def test_prefill_validation(L):
    assert _prefill(L, N=0) == 0
    assert _prefill(L, N=-1) == 1
    assert _prefill(L, T=-5) == 1
    assert _prefill(L, chunk=32) == 2
    assert _prefill(L, dk=48) == 2
    assert _prefill(L, HV=5) == 1
    assert _prefill(L, cu=None) == 1
    assert _prefill(L, o=None) == 1
    assert _prefill(L, k=MISALIGNED) == 1
    assert _prefill(L, s0=MISALIGNED) == 1
    assert _prefill(L, ws=None) == 3
    need = gdn.prefill_workspace_bytes(2, 100, 2, 4, 128, 128)
    assert _prefill(L, wsb=need - 1) == 3
    assert _prefill(L, ws=FAKE + 16) == 3            # workspace must be 256-aligned
    assert _prefill(L, o_dt=3) == 2
    seg = lambda n: L.gdn_prefill_chunked_seg(FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 2, 100, None,
                                              FAKE, FAKE, 0, 2, 4, 128, 128, 64, 1.0, n, None,
                                              0, None)
    for bad in (1, 31, -3):
        assert seg(bad) == 1                          # segment length below 32 chunks
    for ok in (0, -1, -2, 32, 1000):
        assert seg(ok) == 3                           # passes that check, fails on the workspace


def _may_segment(N, T, HV, dk, dv, seg_req):
    """The host's rule for whether a bf16 call can take the segment-parallel
    scan: segments when forced, always possible under the skewed automatic
    mode, or automatically when the (chain, 32-row tile) items leave CUs idle
    (fewer than 128 items at d_k = 128, 256 at d_k = 64)."""
    if dk not in (64, 128) or dv % 32:
        return False
    TV = dv // 32
    idle = 128 if dk == 128 else 256
    longer = (T + 63) // 64 > 32
    return seg_req > 0 or (seg_req == -2 and longer) or (seg_req == 0 and longer
                                                          and N * HV * TV < idle)


def _want_bytes(N, T, HV, dk, dv, seg):
    al = lambda x: (x + 255) // 256 * 256
    maxc = (T + N * 63) // 64
    head = al(4 * (N + 1)) + al(maxc * HV * 64 * 4)
    valu = al(maxc * HV * 64 * 64 * 4)
    mfma = 2 * al(maxc * HV * 64 * 64 * 2) + 2 * al(maxc * HV * dk * 64 * 2)
    segb = N + (maxc + 31) // 32 if seg else N
    corrb = segb + maxc // 4 + 1 if seg else 1
    segs = segb if seg else 0
    tail = (al(8 * 4) + 4 * al(segb * 4) + 3 * al(N * 4) + 2 * al(corrb * 4)
            + 2 * al(segs * HV * dv * dk * 4) + al(segs * HV * dk * dk * 4)
            + al((T if seg else 0) * HV * dk * 4))
    return head + max(valu, mfma) + tail


def test_prefill_workspace_bytes(L):
    f = gdn.prefill_workspace_bytes
    assert f(0, 100, 2, 4, 128, 128) == 0
    assert f(2, 0, 2, 4, 128, 128) == 0
    assert f(2, 100, 2, 4, 128, 128, 32) == 0
    assert f(2, 100, 2, 4, 96, 128) == 0
    assert f(2, 100, 2, 4, 128, 128, segment_chunks=5) == 0   # a length the call rejects
    for N, T, H, HV, dk, dv in ((1, 1, 1, 1, 16, 16), (4, 16384, 16, 16, 128, 128),
                                (8, 131072, 16, 32, 128, 128), (3, 65, 2, 2, 64, 128),
                                (1, 32768, 16, 16, 128, 128), (2, 8192, 16, 32, 128, 128),
                                (1, 6000, 1, 2, 128, 64)):
        for req in (0, -1, -2, 32):
            seg = _may_segment(N, T, HV, dk, dv, req)
            got = f(N, T, H, HV, dk, dv, segment_chunks=req)
            assert got == _want_bytes(N, T, HV, dk, dv, seg), (N, T, HV, dk, dv, req)
            assert got % 256 == 0
        assert f(N, T, H, HV, dk, dv) == L.gdn_prefill_workspace_bytes(N, T, H, HV, dk, dv, 64)
    # one long prompt on few chains segments by default; a batch that fills the GPU does not
    assert _may_segment(1, 32768, 16, 128, 128, 0)
    assert not _may_segment(8, 131072, 32, 128, 128, 0)


def test_prefill_workspace_without_segments_at_the_token_cap():
    """At the long-context varlen cap (8 sequences, 131,072 tokens, 32 value
    heads) the default call cannot segment (its 1024 per-tile chains fill the
    GPU): its workspace holds no segment buffers and is over 2 GB smaller than
    a call with forced segments."""
    args = (8, 131072, 16, 32, 128, 128)
    auto = gdn.prefill_workspace_bytes(*args)
    forced = gdn.prefill_workspace_bytes(*args, segment_chunks=32)
    off = gdn.prefill_workspace_bytes(*args, segment_chunks=-1)
    print(f"workspace at the cap: default {auto / 2**30:.2f} GiB, forced segments "
          f"{forced / 2**30:.2f} GiB")
    assert auto == off
    assert forced - auto >= 2 * 10 ** 9


def _prefill_norm(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=1, g=FAKE, beta=FAKE, cu=FAKE, N=2, T=100, s0=None,
             sf=FAKE, z=FAKE, zd=1, w=FAKE, wd=0, y=FAKE, yd=0, o=None, o_dt=0, H=2, HV=4,
             dk=128, dv=128, chunk=64, scale=1.0, eps=1e-6, ws=None, wsb=0)
    a.update(kw)
    return L.gdn_prefill_chunked_norm(
        a["q"], a["k"], a["v"], a["in_dt"], a["g"], a["beta"], a["cu"], a["N"], a["T"], a["s0"],
        a["sf"], a["z"], a["zd"], a["w"], a["wd"], a["y"], a["yd"], a["o"], a["o_dt"], a["H"],
        a["HV"], a["dk"], a["dv"], a["chunk"], a["scale"], a["eps"], a["ws"], a["wsb"], None)


def test_prefill_norm_validation(L):
    need = gdn.prefill_norm_workspace_bytes(2, 100, 2, 4, 128, 128)
    # the prefill's workspace plus fp32 outputs for the norm's own launch
    assert need == gdn.prefill_workspace_bytes(2, 100, 2, 4, 128, 128) + (100 * 4 * 128 * 4 + 255) // 256 * 256
    assert gdn.prefill_norm_workspace_bytes(0, 100, 2, 4, 128, 128) == 0
    assert gdn.prefill_norm_workspace_bytes(2, 100, 2, 4, 96, 128) == 0
    assert _prefill_norm(L, N=0) == 0
    assert _prefill_norm(L, N=-1) == 1
    assert _prefill_norm(L, eps=-1.0) == 1
    assert _prefill_norm(L, zd=3) == 2
    assert _prefill_norm(L, yd=3) == 2
    for arg in ("z", "w", "y"):
        assert _prefill_norm(L, **{arg: None}) == 1
        assert _prefill_norm(L, **{arg: MISALIGNED}) == 1
    assert _prefill_norm(L, o=FAKE + 256, y=FAKE + 256, ws=FAKE, wsb=need) == 1  # y == o
    assert _prefill_norm(L, chunk=32) == 2
    assert _prefill_norm(L, dk=48) == 2
    assert _prefill_norm(L, HV=5) == 1
    assert _prefill_norm(L) == 3                     # no workspace
    assert _prefill_norm(L, ws=FAKE, wsb=need - 1) == 3
    assert _prefill_norm(L, ws=FAKE + 16, wsb=need) == 3
    # the documented size holds whether or not o is given
    ws_prefill = gdn.prefill_workspace_bytes(2, 100, 2, 4, 128, 128)
    assert _prefill_norm(L, o=FAKE + 256, ws=FAKE, wsb=ws_prefill) == 3


def _norm(L, **kw):
    a = dict(x=FAKE, xd=0, z=FAKE, zd=1, w=FAKE, wd=0, y=FAKE, yd=0, rows=4, HV=2, dv=128,
             eps=1e-6)
    a.update(kw)
    return L.gdn_rmsnorm_gated(a["x"], a["xd"], a["z"], a["zd"], a["w"], a["wd"], a["y"], a["yd"],
                               a["rows"], a["HV"], a["dv"], a["eps"], None)


def test_norm_validation(L):
    assert _norm(L, rows=0) == 0
    assert _norm(L, rows=-1) == 1
    assert _norm(L, eps=-1.0) == 1
    assert _norm(L, eps=float("nan")) == 1
    assert _norm(L, z=None) == 1
    assert _norm(L, y=MISALIGNED) == 1
    assert _norm(L, dv=80) == 2
    assert _norm(L, zd=5) == 2
    assert _norm(L, yd=1) == 1                       # y aliases x with another dtype


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(2, 2, 16)
    with pytest.raises(ValueError):
        gdn.rmsnorm_gated(x, x, torch.ones(16))


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gdn, "LIBRARY", str(tmp_path / "missing.so"))
    monkeypatch.setattr(gdn, "_LIB", None)
    with pytest.raises(ImportError):
        gdn.lib()


def test_library_binds_to_torch_hip_runtime():
    """libgdn.so must share torch's HIP runtime (one runtime per process)."""
    gdn.lib()
    maps = open("/proc/self/maps").read()
    runtimes = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(runtimes) == 1, runtimes


def _decode_norm(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=1, g=FAKE, beta=FAKE, state=FAKE, z=FAKE, z_dt=1,
             w=FAKE, w_dt=0, y=FAKE, y_dt=0, o=None, o_dt=0, N=2, H=2, HV=4, dk=128, dv=128,
             scale=1.0, eps=1e-6)
    a.update(kw)
    return L.gdn_decode_step_norm(a["q"], a["k"], a["v"], a["in_dt"], a["g"], a["beta"],
                                  a["state"], a["z"], a["z_dt"], a["w"], a["w_dt"], a["y"],
                                  a["y_dt"], a["o"], a["o_dt"], a["N"], a["H"], a["HV"],
                                  a["dk"], a["dv"], a["scale"], a["eps"], None)


def test_decode_norm_validation(L):
    assert _decode_norm(L, N=0) == 0
    assert _decode_norm(L, N=-1) == 1
    assert _decode_norm(L, z=None) == 1
    assert _decode_norm(L, y=None) == 1
    assert _decode_norm(L, w=MISALIGNED) == 1
    assert _decode_norm(L, o=MISALIGNED) == 1
    assert _decode_norm(L, eps=-1.0) == 1
    assert _decode_norm(L, state=None) == 1
    assert _decode_norm(L, dv=48) == 2
    assert _decode_norm(L, z_dt=9) == 2
    assert _decode_norm(L, HV=6, H=4) == 1


def _layer(L, **kw):
    a = gdn.DecodeLayerArgs()
    base = dict(q=FAKE, k=FAKE, v=FAKE, in_dtype=1, g=FAKE, beta=FAKE, state=FAKE, num_slots=0,
                o=FAKE, o_dtype=0, N=0, H=2, HV=4, dk=64, dv=64, scale=1.0, l2_eps=1e-6,
                eps=1e-6)
    base.update(kw)
    for name, val in base.items():
        setattr(a, name, val)
    return L.gdn_decode_layer(ctypes.byref(a), None)


def test_decode_layer_struct_layout(L):
    """The binding's mirror of gdn_decode_layer_args has the library's size and
    the header's field order."""
    assert L.gdn_decode_layer_args_size() == ctypes.sizeof(gdn.DecodeLayerArgs)
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct gdn_decode_layer_args \{(.*?)\}", text, re.S).group(1)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        names = decl.split(None, 1)[1] if not decl.startswith("const") else decl.split(None, 2)[2]
        fields += [n.strip().lstrip("*").strip() for n in names.split(",")]
    assert fields == [f for f, _ in gdn.DecodeLayerArgs._fields_]


def test_decode_layer_validation(L):
    OK, INVALID, UNSUP = 0, 1, 2
    assert L.gdn_decode_layer(None, None) == INVALID
    assert _layer(L) == OK                                   # N == 0, num_slots 0 with slots
    assert _layer(L, N=3, num_slots=2) == INVALID            # no slot table: num_slots < N
    assert _layer(L, N=-1) == INVALID
    assert _layer(L, num_slots=-1, slots=FAKE) == INVALID
    assert _layer(L, dk=48) == UNSUP
    assert _layer(L, HV=3) == INVALID
    assert _layer(L, in_dtype=7) == UNSUP
    assert _layer(L, l2_eps=-1.0) == INVALID
    assert _layer(L, l2_eps=float("nan")) == INVALID
    n1 = dict(N=1, num_slots=1)
    assert _layer(L, q=0, **n1) == INVALID
    assert _layer(L, state=MISALIGNED, **n1) == INVALID
    assert _layer(L, g=0, **n1) == INVALID                   # activated gates missing
    assert _layer(L, a_raw=FAKE, gate_dtype=1, **n1) == INVALID        # raw: b_raw, A_log missing
    assert _layer(L, a_raw=FAKE, b_raw=FAKE, gate_dtype=5, A_log=FAKE, **n1) == UNSUP
    assert _layer(L, o=0, **n1) == INVALID                   # neither o nor y
    assert _layer(L, o=0, y=FAKE, y_dtype=0, z=FAKE, z_dtype=0, **n1) == INVALID  # no w
    assert _layer(L, y=FAKE, y_dtype=0, z=FAKE, z_dtype=0, w=FAKE, w_dtype=0, eps=-1.0,
                  **n1) == INVALID
    assert _layer(L, o=MISALIGNED, **n1) == INVALID


def _attn(L, **kw):
    a = gdn.AttnDecodeArgs()
    base = dict(q=FAKE, k_new=FAKE, v_new=FAKE, k_cache=FAKE, v_cache=FAKE, pos=FAKE, o=FAKE,
                o_dtype=0, N=2, Hq=16, Hkv=2, D=256, Lmax=100, rotary_dim=64, rope_theta=1e7,
                scale=0.0625, workspace=FAKE, workspace_bytes=1 << 30)
    base.update(kw)
    for name, val in base.items():
        setattr(a, name, val)
    return L.gdn_attn_decode(ctypes.byref(a), None)


def test_attn_decode_validation(L):
    OK, INVALID, UNSUP, WS = 0, 1, 2, 3
    assert L.gdn_attn_decode_args_size() == ctypes.sizeof(gdn.AttnDecodeArgs)
    assert L.gdn_attn_decode(None, None) == INVALID
    assert _attn(L, N=0) == OK
    assert _attn(L, N=-1) == INVALID
    assert _attn(L, Hq=15) == INVALID
    assert _attn(L, Hq=12, Hkv=2) == UNSUP          # group of 6
    assert _attn(L, D=96) == UNSUP
    assert _attn(L, o_dtype=4) == UNSUP
    assert _attn(L, rotary_dim=63) == INVALID
    assert _attn(L, rotary_dim=512) == INVALID
    assert _attn(L, rope_theta=0.0) == INVALID
    assert _attn(L, q=0) == INVALID
    assert _attn(L, k_cache=MISALIGNED) == INVALID
    assert _attn(L, workspace=0) == WS
    need = L.gdn_attn_decode_workspace_bytes(2, 16, 2, 256, 100)
    assert need > 0 and need % 256 == 0
    assert _attn(L, workspace_bytes=need - 1) == WS
    assert _attn(L, workspace=FAKE + 16) == WS
    assert L.gdn_attn_decode_workspace_bytes(2, 16, 2, 96, 100) == 0

"""Host-side logic of bench.py, checked without a GPU: the one-GPU guard, the
algorithmic byte counts the roofline divides by, and the keying of the
recorded HBM-traffic figures on the kernel sources."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_exits_too():
    env = dict(os.environ, WORLD_SIZE="2", RANK="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2
    assert r.stderr == ""  # only rank 0 prints


def test_decode_bytes_per_token_qwen35_shape():
    # state read + written per value head, q and k per key head (bf16), v, z
    # (bf16), g and beta (fp32), y (fp32): 16 heads at d = 128
    per_head_state = 128 * 128 * 4 * 2
    expect = 16 * per_head_state + 16 * 128 * 2 * 2 + 16 * 128 * 2 + 16 * 8 + 16 * 128 * 2 + 16 * 128 * 4
    assert bench.decode_bytes_per_token(16, 16, 128, 128) == expect == 2_121_856
    assert bench.decode_bytes_per_token(16, 16, 128, 128) * 32 == 67_899_392


def test_decode_bytes_scale_with_value_heads_not_key_heads():
    a = bench.decode_bytes_per_token(16, 32, 128, 128)
    b = bench.decode_bytes_per_token(16, 16, 128, 128)
    # the second 16 value heads add their state, v, z, y and gates; q, k stay
    assert a - b == 16 * (128 * 128 * 8 + 128 * 2 + 8 + 128 * 2 + 128 * 4)


def test_prefill_bytes_workload2():
    T, N = 4 * 4096, 4
    b = bench.prefill_bytes(T, N, 16, 16, 128, 128)
    per_token = 16 * 128 * 2 * 2 + 16 * 128 * 2 + 16 * 8 + 16 * 128 * 4
    assert b == T * per_token + N * 16 * 128 * 128 * 4 == 341_835_776
    # an initial state adds one more state read
    assert bench.prefill_bytes(T, N, 16, 16, 128, 128, s0=True) - b == N * 16 * 128 * 128 * 4


def test_traffic_record_is_keyed_on_the_sources():
    rec = dict(bench.DECODE_TRAFFIC)
    sha = bench.kernel_sources_sha256("gdn_decode.hip")
    assert len(sha) == 64 and sha == bench.kernel_sources_sha256("gdn_decode.hip")
    assert bench.measured_traffic(dict(rec, kernel_source_sha256=sha)) == rec["bytes_per_launch"]
    assert bench.measured_traffic(dict(rec, kernel_source_sha256="0" * 64)) is None


def test_kernel_hash_covers_included_headers(tmp_path, monkeypatch):
    csrc = tmp_path / "gated_delta_rule_decode_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text('#include "h.h"\nint main() { return 0; }\n')
    (csrc / "h.h").write_text("// header one\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    first = bench.kernel_sources_sha256("k.hip")
    (csrc / "h.h").write_text("// header two\n")
    assert bench.kernel_sources_sha256("k.hip") != first


def test_norm_bytes_job_prefill_shape():
    # fp32 x read, bf16 z read, fp32 y written per element; the weight once
    rows, HV, dv = 32 * 512, 16, 128
    assert bench.norm_bytes(rows, HV, dv) == rows * HV * dv * 10 + dv * 4 == 335_544_832

"""bench.py contract checks that need no GPU: one-GPU refusal and the
algorithmic work/byte counts the roofline divides by."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_algorithmic_counts():
    # chunk 64, head dim 128, 16 q/k and 32 v heads
    assert bench.prefill_alg_flops_per_token(16, 32, 128) == 5_242_880
    assert bench.prefill_alg_bytes(1, 1, 16, 32, 128, init=False) - 32 * 128 * 128 * 4 == 33_024
    assert bench.prefill_alg_bytes(65536, 1, 16, 32, 128, init=True) == 65536 * 33_024 + 2 * 32 * 128 * 128 * 4
    assert bench.decode_alg_bytes(256, 16, 32, 128) == 1_107_361_792
    assert bench.decode_alg_bytes(256, 16, 32, 128, state_bytes=2) == 1_107_361_792 - 256 * 32 * 128 * 128 * 4
    # the n-token step: one state read + write per call, n tokens per sequence
    assert bench.decode_tokens_alg_bytes(256, 1, 16, 32, 128) == 1_107_361_792
    assert bench.decode_tokens_alg_bytes(256, 4, 16, 32, 128) == 1_107_361_792 + 3 * 256 * 33_024
    assert bench.decode_tokens_alg_bytes(256, 4, 16, 32, 128, commit=False) == \
        256 * 32 * 128 * 128 * 4 + 4 * 256 * 33_024 + 256 * 3 * 8192 * 2


def test_stored_traffic_follows_the_sources():
    # each committed PMC figure is reported only for the sources of its own kernel
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return
    for line in open(path).read().splitlines():
        if "=" not in line or line.startswith("#"):
            continue
        key, val = (x.strip() for x in line.split("=", 1))
        if key not in bench.TRAFFIC_SOURCES:
            continue
        nbytes, h = val.split()
        t = bench.stored_traffic(key)
        if h == bench.source_hash(key):
            assert t == int(float(nbytes))
        else:
            assert t is None


def test_stored_traffic_is_dropped_when_its_kernel_changes(tmp_path, monkeypatch):
    # a figure whose hash does not match its kernel's sources reads as None; another
    # kernel's figure is unaffected
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = bench.source_hash("decode_bytes_per_launch")
    (prof / "traffic.txt").write_text(
        f"decode_bytes_per_launch = 123 {good}\n"
        "prefill_full_bytes_per_launch = 456 0000000000000000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "linear_attention_sequence_causal_amd" / "csrc"
    csrc.mkdir(parents=True)
    import shutil
    for name in os.listdir(os.path.join(ROOT, "linear_attention_sequence_causal_amd", "csrc")):
        shutil.copy(os.path.join(ROOT, "linear_attention_sequence_causal_amd", "csrc", name), csrc)
    assert bench.stored_traffic("decode_bytes_per_launch") == 123
    assert bench.stored_traffic("prefill_full_bytes_per_launch") is None
    assert bench.stored_traffic("attention_bytes_per_launch") is None
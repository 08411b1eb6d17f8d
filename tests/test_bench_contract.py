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
    # the committed PMC figures are reported only for the kernel sources they were taken on
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return
    vals = dict(l.split("=", 1) for l in open(path).read().splitlines()
                if "=" in l and not l.startswith("#"))
    vals = {k.strip(): v.strip() for k, v in vals.items()}
    t = bench.stored_traffic("decode_bytes_per_launch")
    if vals.get("source_hash") == bench.source_hash():
        assert t == int(vals["decode_bytes_per_launch"])
    else:
        assert t is None

#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet mixer (prefill and decode) on one MI355X.

Prints ONE JSON line.  The headline is prefill tokens/s of one sequence of
65,536 tokens with 16 q/k heads, 32 v heads, head dim 128 (bf16 activations,
fp32 state, initial state ~ N(0, 0.01^2)); the same line carries decode
steps/s of 256 sequences x 1000 consecutive steps (fp32 states 32x128x128,
conv cache of 3 tokens) under "decode".  Inputs are seeded synthetic tensors
(gdn_synth) resident in HBM before the timed region.

Roofline accounting (algorithmic work only, never the extra work the kernels
choose to do):
  prefill FLOP/token = Hk*4*C*D + Hv*(6*C*D + 6*D^2)        (C = 64, D = 128)
  prefill bytes/token = 2*(2*Hk*D + 3*Hv*D) + 2*4*Hv   (+ initial and final state)
  decode bytes/step  = B*Hv*D*D*4*2 (state read + write) + B*33,024 (tokens)
                       + B*3*Cc*2*2 (conv cache read + write)
  bf16-state decode  = the same with 2-byte state elements
  n-token step bytes = the same with n*B*33,024 token bytes (commit pass); a
                       verify pass (commit 0) reads the state and cache only
Peaks: MI355X dense bf16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# The unit of prefill work is the chunk-64 WY/UT form's FLOP count per token
# (5,242,880 at 16/32 heads, d = 128), fixed whatever chunk the kernel runs: the
# kernel's 32-token chunks execute fewer intra-chunk products (the same formula at
# C = 32 gives 4,194,304), so the MFMA fraction below is the token rate expressed
# in that fixed unit, not a count of the products issued.
ALG_CHUNK = 64
KERNEL_CHUNK = 32


def prefill_alg_flops_per_token(Hk, Hv, D, C=ALG_CHUNK):
    return Hk * 4 * C * D + Hv * (6 * C * D + 6 * D * D)


def prefill_alg_bytes(T, N, Hk, Hv, D, act_bytes=2, init=True):
    per_tok = act_bytes * (2 * Hk * D + 3 * Hv * D) + 2 * 4 * Hv
    states = N * Hv * D * D * 4 * (2 if init else 1)
    return T * per_tok + states


def decode_alg_bytes(B, Hk, Hv, D, act_bytes=2, state_bytes=4):
    Cc = 2 * Hk * D + Hv * D
    state = B * Hv * D * D * state_bytes * 2
    tokens = B * (act_bytes * (2 * Hk * D + 3 * Hv * D) + 2 * 4 * Hv)
    cache = B * 3 * Cc * act_bytes * 2
    return state + tokens + cache


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_sequence_causal_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash():
        return None
    try:
        return int(float(vals[kernel_key]))
    except (KeyError, ValueError):
        return None


def rel_l2(x, ref):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def bench_prefill(args, torch, gdn, S):
    w = S.PREFILL_64K
    d = S.prefill_inputs(w, "cuda")
    T = d["q"].shape[0]
    Hk, Hv, D = w.num_qk_heads, w.num_v_heads, w.head_dim

    def step():
        return gdn.prefill(d["q"], d["k"], d["v"], d["a"], d["b"], d["z"], d["conv_w"],
                           d["A_log"], d["dt_bias"], d["norm_w"], init_state=d["init_state"],
                           out=out, final_state=fs)

    out = torch.empty_like(d["v"])
    fs = torch.empty((1, Hv, D, D), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    call_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = wall * 1e3 / args.steps

    # per-kernel attribution: HIP events between the library's kernels, same stream
    os.environ["GDN_KERNEL_TIMING"] = "1"
    per = {}
    n_attr = max(3, min(10, args.steps))
    for _ in range(n_attr):
        step()
        t = gdn.last_kernel_times()
        for k_, v_ in (t or {}).items():
            per[k_] = per.get(k_, 0.0) + v_ / n_attr
    os.environ.pop("GDN_KERNEL_TIMING", None)
    torch.cuda.synchronize()

    flops = prefill_alg_flops_per_token(Hk, Hv, D) * T
    nbytes = prefill_alg_bytes(T, 1, Hk, Hv, D, init=True)
    call_avg = sum(call_ms) / len(call_ms)
    dom = max(per, key=per.get) if per else None
    dom_ms = per.get(dom, call_avg) if dom else call_avg
    res = dict(T=T, out=out, fs=fs, d=d, ms_per_step=ms_per_step, call_ms=call_avg,
               call_ms_min=min(call_ms), flops=flops, bytes=nbytes, per_kernel_ms=per,
               dominant=dom, dominant_ms=dom_ms)
    return res


def bench_decode(args, torch, gdn, S, state_bf16=False, toks=None):
    w = S.DECODE_B256
    steps = args.decode_steps
    setup = S.decode_setup(w, "cuda")
    if toks is None:
        toks = S.decode_tokens(w, setup, steps, "cuda")
    state, cache = setup["state"], setup["conv_cache"]
    if state_bf16:  # reduced-precision storage of the same start state
        state = state.to(torch.bfloat16)
    o = torch.empty((w.decode_batch, w.num_v_heads, w.head_dim), dtype=torch.bfloat16,
                    device="cuda")

    def one(s):
        gdn.decode_step(toks["q"][s], toks["k"][s], toks["v"][s], toks["a"][s], toks["b"][s],
                        toks["z"][s], setup["conv_w"], setup["A_log"], setup["dt_bias"],
                        setup["norm_w"], state, cache, out=o)

    for s in range(min(args.warmup, steps)):  # warm-up steps advance the state; fine
        one(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        one(s)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1)
    nbytes = decode_alg_bytes(w.decode_batch, w.num_qk_heads, w.num_v_heads, w.head_dim,
                              state_bytes=2 if state_bf16 else 4)
    return dict(steps=steps, wall_s=wall, ms_per_step=ev_ms / steps, bytes=nbytes,
                w=w, setup=setup, toks=toks)


def bench_prefill_config(args, torch, gdn, S, w):
    """Whole-call time of one of the other prefill workloads (T=4096; varlen N=64)."""
    d = S.prefill_inputs(w, "cuda")
    T = d["q"].shape[0]
    N = d["cu_seqlens"].numel() - 1
    Hk, Hv, D = w.num_qk_heads, w.num_v_heads, w.head_dim
    out = torch.empty_like(d["v"])
    fs = torch.empty((N, Hv, D, D), dtype=torch.float32, device="cuda")

    def step():
        gdn.prefill(d["q"], d["k"], d["v"], d["a"], d["b"], d["z"], d["conv_w"], d["A_log"],
                    d["dt_bias"], d["norm_w"], init_state=d["init_state"],
                    cu_seqlens=d["cu_seqlens"], out=out, final_state=fs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    reps = max(3, args.steps // 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = prefill_alg_flops_per_token(Hk, Hv, D) * T
    nbytes = prefill_alg_bytes(T, N, Hk, Hv, D, init=d["init_state"] is not None)
    del d, out, fs
    return {"value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms, "calls": reps,
            "config": {"workload": w.name, "num_seqs": N, "total_tokens": T},
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def decode_tokens_alg_bytes(B, n, Hk, Hv, D, act_bytes=2, commit=True):
    Cc = 2 * Hk * D + Hv * D
    rw = 2 if commit else 1
    state = B * Hv * D * D * 4 * rw
    tokens = n * B * (act_bytes * (2 * Hk * D + 3 * Hv * D) + 2 * 4 * Hv)
    cache = B * 3 * Cc * act_bytes * rw
    return state + tokens + cache


def bench_decode_tokens(args, torch, gdn, S, dec=None):
    """n new tokens per sequence per call (B=256, 16/32 heads): commit passes that
    advance the state, and verify passes (commit 0) that only read it."""
    w, n, calls = S.DECODE_B256, args.tokens_n, args.tokens_calls
    B, Hk, Hv, D = w.decode_batch, w.num_qk_heads, w.num_v_heads, w.head_dim
    setup = S.decode_setup(w, "cuda")
    toks = S.decode_tokens(w, setup, calls * n, "cuda")
    bn = {k_: v_.reshape((calls, n) + tuple(v_.shape[1:])).transpose(1, 2).contiguous()
          for k_, v_ in toks.items()}
    del toks
    state, cache = setup["state"], setup["conv_cache"]
    o = torch.empty((B, n, Hv, D), dtype=torch.bfloat16, device="cuda")
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")

    def one(c, commit):
        gdn.decode_tokens(bn["q"][c], bn["k"][c], bn["v"][c], bn["a"][c], bn["b"][c],
                          bn["z"][c], setup["conv_w"], setup["A_log"], setup["dt_bias"],
                          setup["norm_w"], state, cache, num_commit=commit, out=o)

    res = {}
    for name, commit in (("verify", zeros), ("commit", None)):
        for c in range(min(args.warmup, calls)):
            one(c, commit)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for c in range(calls):
            one(c, commit)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / calls
    nb_c = decode_tokens_alg_bytes(B, n, Hk, Hv, D, commit=True)
    nb_v = decode_tokens_alg_bytes(B, n, Hk, Hv, D, commit=False)
    t = res["commit"] * 1e-3
    gbs = nb_c / t / 1e9
    return {"value": B * n / t, "unit": "tokens/s", "ms_per_step": res["commit"],
            "calls": calls,
            "config": {"workload": f"decode_tokens_B{B}_n{n}_hk{Hk}_hv{Hv}_d{D}_bf16",
                       "batch": B, "n_tokens": n, "calls": calls},
            "roofline": {"bound": "hbm", "kernel": "decode_tokens (commit all)",
                         "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": stored_traffic("decode_tokens_bytes_per_launch"),
                         "alg_bytes_per_launch": nb_c, "launch_ms": res["commit"]},
            "verify": {"ms_per_step": res["verify"], "tokens_per_s": B * n / (res["verify"] * 1e-3),
                       "alg_bytes_per_launch": nb_v,
                       "hbm_frac": nb_v / (res["verify"] * 1e-3) / 1e9 / PEAK_HBM_GBS}}


def cpu_baseline_prefill(res, S, oracle):
    """fp64 oracle on the first `n` tokens of the same workload, all heads."""
    import numpy as np
    d = res["d"]
    n = int(os.environ.get("GDN_BENCH_ORACLE_TOKENS", "65536"))
    f = lambda t: S.to_f64(t[:n]) if t is not None else None
    threads = min(oracle.default_threads(), d["v"].shape[1])
    t0 = time.perf_counter()
    o_ref, _, _ = oracle.prefill(f(d["q"]), f(d["k"]), f(d["v"]), f(d["a"]), f(d["b"]),
                                 f(d["z"]), S.to_f64(d["conv_w"]), S.to_f64(d["A_log"]),
                                 S.to_f64(d["dt_bias"]), S.to_f64(d["norm_w"]),
                                 init_state=S.to_f64(d["init_state"]), nthreads=threads)
    dt = time.perf_counter() - t0
    err = rel_l2(S.to_f64(res["out"][:n]), o_ref)
    return dict(value=n / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"first {n} of the 65536 tokens of the workload, all 32 v heads, fp64, "
                       f"{dt:.1f} s"), err


def cpu_baseline_decode(dec, S, oracle):
    import numpy as np
    n = int(os.environ.get("GDN_BENCH_ORACLE_DECODE_STEPS", "32"))
    w, setup, toks = dec["w"], dec["setup"], dec["toks"]
    f = S.to_f64
    # fresh copies of the decode start state (the GPU run advanced its own)
    s2 = S.decode_setup(w, "cuda")
    st, cc = f(s2["state"]), f(s2["conv_cache"])
    threads = min(oracle.default_threads(), w.decode_batch * w.num_v_heads)
    t0 = time.perf_counter()
    for s in range(n):
        _, st, cc = oracle.decode_step(f(toks["q"][s]), f(toks["k"][s]), f(toks["v"][s]),
                                       f(toks["a"][s]), f(toks["b"][s]), f(toks["z"][s]),
                                       f(setup["conv_w"]), f(setup["A_log"]),
                                       f(setup["dt_bias"]), f(setup["norm_w"]), st, cc,
                                       nthreads=threads)
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="steps/s", cores=threads, kind="oracle",
                sample=f"{n} decode steps of the B=256 workload (all sequences and heads), "
                       f"fp64, {dt:.1f} s")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed prefill calls")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--only", choices=("all", "prefill", "decode", "tokens"), default="all")
    ap.add_argument("--tokens-n", type=int, default=4,
                    help="new tokens per sequence of the n-token step leg (1..8)")
    ap.add_argument("--tokens-calls", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="also run a device copy of this many GiB (PMC scale factor)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the mixer is built and measured on a single "
              "MI355X; multi-GPU runs are not part of this benchmark.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gdn_synth as S
    import linear_attention_sequence_causal_amd as gdn
    gdn.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    line = {"metric": "GDN prefill tokens/s at T=64K (16qk/32v heads,d=128); "
                      "decode steps/s at B=256",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic"}

    if args.only in ("all", "prefill"):
        pre = bench_prefill(args, torch, gdn, S)
        t_dom = pre["dominant_ms"] * 1e-3
        t_call = pre["call_ms"] * 1e-3
        ach = pre["flops"] / t_dom / 1e12
        line.update({
            "value": pre["T"] / (pre["ms_per_step"] * 1e-3),
            "unit": "tokens/s",
            "ms_per_step": pre["ms_per_step"],
            "config": {"workload": "prefill_T65536_hk16_hv32_d128_bf16", "num_seqs": 1,
                       "seq_len": pre["T"], "num_qk_heads": 16, "num_v_heads": 32,
                       "head_dim": 128, "chunk": KERNEL_CHUNK, "state": "fp32"},
            "roofline": {
                "bound": "mfma", "kernel": f"prefill {pre['dominant']} pass",
                "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS,
                "traffic": stored_traffic("prefill_full_bytes_per_launch"),
                "alg_flops_per_launch": pre["flops"],
                # the same formula at the kernel's own chunk size (what its products amount to)
                "chunk32_form_flops_per_launch":
                    prefill_alg_flops_per_token(16, 32, 128, C=KERNEL_CHUNK) * pre["T"],
                "launch_ms": pre["dominant_ms"],
            },
            "prefill_path": {
                "call_ms": pre["call_ms"], "call_ms_min": pre["call_ms_min"],
                "mfma_frac": pre["flops"] / t_call / 1e12 / PEAK_BF16_TFLOPS,
                "hbm_frac": pre["bytes"] / t_call / 1e9 / PEAK_HBM_GBS,
                "alg_bytes": pre["bytes"], "per_kernel_ms": pre["per_kernel_ms"],
            },
        })
        # the other prefill workloads (parity configs), tokens/s of the whole call
        line["prefill_configs"] = {w.name: bench_prefill_config(args, torch, gdn, S, w)
                                   for w in (S.PREFILL_4K, S.VARLEN_64)}
    if args.only in ("all", "decode"):
        dec = bench_decode(args, torch, gdn, S)
        t = dec["ms_per_step"] * 1e-3
        gbs = dec["bytes"] / t / 1e9
        dline = {"value": 1.0 / t, "unit": "steps/s", "ms_per_step": dec["ms_per_step"],
                 "steps": dec["steps"],
                 "config": {"workload": "decode_B256_hk16_hv32_d128_bf16", "batch": 256,
                            "steps": dec["steps"]},
                 "roofline": {"bound": "hbm", "kernel": "decode_step", "achieved": gbs,
                              "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                              "traffic": stored_traffic("decode_bytes_per_launch"),
                              "alg_bytes_per_launch": dec["bytes"],
                              "launch_ms": dec["ms_per_step"]}}
        # the same steps with the state stored in bf16 (fp32 arithmetic; its own tolerance)
        d16 = bench_decode(args, torch, gdn, S, state_bf16=True, toks=dec["toks"])
        t16 = d16["ms_per_step"] * 1e-3
        g16 = d16["bytes"] / t16 / 1e9
        dline["bf16_state"] = {
            "value": 1.0 / t16, "unit": "steps/s", "ms_per_step": d16["ms_per_step"],
            "roofline": {"bound": "hbm", "kernel": "decode_step (bf16 state)", "achieved": g16,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": g16 / PEAK_HBM_GBS,
                         "alg_bytes_per_launch": d16["bytes"], "launch_ms": d16["ms_per_step"]}}
        if args.only == "decode":
            line.update({"value": dline["value"], "unit": "steps/s",
                         "ms_per_step": dline["ms_per_step"], "config": dline["config"],
                         "roofline": dline["roofline"], "bf16_state": dline["bf16_state"]})
        else:
            line["decode"] = dline
    if args.only in ("all", "tokens"):
        tl = bench_decode_tokens(args, torch, gdn, S)
        if args.only == "tokens":
            line.update({"value": tl["value"], "unit": "tokens/s",
                         "ms_per_step": tl["ms_per_step"], "config": tl["config"],
                         "roofline": tl["roofline"], "verify": tl["verify"]})
        else:
            line["decode_tokens"] = tl
    if not args.no_cpu_baseline and args.only != "tokens":
        import oracle
        if args.only in ("all", "prefill"):
            cb, err = cpu_baseline_prefill(pre, S, oracle)
            line["cpu_baseline"] = cb
            line["parity_sample_o_rel_l2"] = err
        if args.only in ("all", "decode"):
            cbd = cpu_baseline_decode(dec, S, oracle)
            if args.only == "decode":
                line["cpu_baseline"] = cbd
            else:
                line["decode"]["cpu_baseline"] = cbd
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

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
  fp8-state decode   = the same with 1-byte state elements + B*Hv*D*4*2 (row scales)
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


# The kernel sources each stored traffic figure depends on (gdn_device.h is shared).
TRAFFIC_SOURCES = {
    "prefill_full_bytes_per_launch": ("gdn_prefill.hip", "gdn_prefill_plan.h", "gdn_device.h"),
    "decode_bytes_per_launch": ("gdn_decode.hip", "gdn_device.h"),
    "decode_tokens_bytes_per_launch": ("gdn_decode.hip", "gdn_device.h"),
    "attention_bytes_per_launch": ("gdn_attention.hip", "gdn_attention.h", "gdn_device.h"),
}


def source_hash(kernel_key):
    """Hash of the sources of one kernel (the files its stored traffic depends on)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_sequence_causal_amd", "csrc")
    for name in TRAFFIC_SOURCES[kernel_key]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was taken on
    the current sources of that kernel (else None).  profiles/traffic.txt holds one line
    per kernel: `<key> = <bytes> <source hash>`."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#") or "=" not in line:
            continue
        k, v = (x.strip() for x in line.split("=", 1))
        if k != kernel_key:
            continue
        parts = v.split()
        if len(parts) != 2 or parts[1] != source_hash(kernel_key):
            return None
        try:
            return int(float(parts[0]))
        except ValueError:
            return None
    return None


def progress(msg):
    """One line on stderr as each leg finishes (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def rel_l2(x, ref):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def bench_prefill(args, torch, gdn, S, slow_decay=None, d=None):
    """The 65,536-token prefill; slow_decay = exp(A_log) for every head (alpha ~
    exp(-slow_decay * softplus(a + dt_bias)) per token), which makes the segment maps
    non-negligible so that the map and combine passes walk every chunk."""
    import math
    w = S.PREFILL_64K
    if d is None:
        d = S.prefill_inputs(w, "cuda")
    if slow_decay is not None:
        d = dict(d)
        d["A_log"] = torch.full_like(d["A_log"], math.log(slow_decay))
    T = d["q"].shape[0]
    Hk, Hv, D = w.num_qk_heads, w.num_v_heads, w.head_dim

    def step():
        return gdn.prefill(d["q"], d["k"], d["v"], d["a"], d["b"], d["z"], d["conv_w"],
                           d["A_log"], d["dt_bias"], d["norm_w"], init_state=d["init_state"],
                           out=out, final_state=fs)

    out = torch.empty_like(d["v"])
    fs = torch.empty((1, Hv, D, D), dtype=torch.float32, device="cuda")
    # Untimed settle calls first: on a fresh box the full pass shortens over its first
    # ~25 back-to-back calls (1.1-1.35 ms down to ~0.95 ms) while the clocks ramp up;
    # then the warm-up, the timed calls and the per-kernel attribution all see the
    # steady state (the warm-only trace selection skips settle + warm-up dispatches).
    for _ in range(args.settle):
        step()
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
    n_attr = max(3, args.steps)
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
               dominant=dom, dominant_ms=dom_ms, n_attr=n_attr)
    return res


def fp8_rows(torch, x):
    """E4M3 values and per-row power-of-two scales of a state (the smallest 2^e with
    max|row| <= 448 * 2^e), for the fp8-storage decode leg's start state."""
    m = x.abs().amax(dim=-1)
    e = torch.ceil(torch.log2(torch.where(m > 0, m / 448.0, torch.ones_like(m))))
    sc = torch.exp2(e)
    return (x / sc[..., None]).to(torch.float8_e4m3fn), sc.float().contiguous()


def bench_decode(args, torch, gdn, S, state_bf16=False, toks=None, state_fp8=False):
    w = S.DECODE_B256
    steps = args.decode_steps
    setup = S.decode_setup(w, "cuda")
    if toks is None:
        toks = S.decode_tokens(w, setup, steps, "cuda")
    state, cache = setup["state"], setup["conv_cache"]
    scale = None
    if state_bf16:  # reduced-precision storage of the same start state
        state = state.to(torch.bfloat16)
    if state_fp8:
        state, scale = fp8_rows(torch, state)
    o = torch.empty((w.decode_batch, w.num_v_heads, w.head_dim), dtype=torch.bfloat16,
                    device="cuda")

    def one(s):
        gdn.decode_step(toks["q"][s], toks["k"][s], toks["v"][s], toks["a"][s], toks["b"][s],
                        toks["z"][s], setup["conv_w"], setup["A_log"], setup["dt_bias"],
                        setup["norm_w"], state, cache, out=o, state_scale=scale)

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
                              state_bytes=2 if state_bf16 else 1 if state_fp8 else 4)
    if state_fp8:  # the per-row scales, read and written
        nbytes += w.decode_batch * w.num_v_heads * w.head_dim * 4 * 2
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


def bench_projections(args, torch, gdn, S):
    """The projections around the mixer at the layer's size (T = 65536 tokens, d_model =
    2048, 16/32 heads): the in-projection (N = 12,352 outputs into q, k, v, z, a, b), the
    output projection (K = 4096, N = 2048), each against the 16-bit dense MFMA peak; and
    torch.matmul (hipBLASLt) on the same shapes for comparison."""
    w = S.LAYER_64K
    d_model = 2048
    d = S.layer_inputs(w, d_model, "cuda")
    T, Hk, Hv, D = int(sum(w.lengths)), w.num_qk_heads, w.num_v_heads, w.head_dim
    n_in = 2 * Hk * D + 2 * Hv * D + 2 * Hv
    outs = gdn.in_projection(d["x"], d["w_in"], Hk, Hv, D)
    o = torch.randn((T, Hv, D), device="cuda").to(torch.bfloat16)
    y = torch.empty((T, d_model), dtype=torch.bfloat16, device="cuda")
    p = gdn.GdnParams(Hk, Hv, D, gdn.GDN_BF16, 1.0, 1e-6, 1e-6, None, None, None, None, 0)
    L = gdn.lib()
    import ctypes
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def in_proj():
        L.gdn_in_projection(ptr(d["x"]), ptr(d["w_in"]), ctypes.byref(p), T, d_model,
                            *[ptr(t) for t in outs], gdn._stream())

    def out_proj():
        L.gdn_out_projection(ptr(o), ptr(d["w_out"]), ctypes.byref(p), T, d_model, ptr(y),
                             gdn._stream())

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {}
    for name, fn, n, k in (("in_projection", in_proj, n_in, d_model),
                           ("out_projection", out_proj, d_model, Hv * D)):
        ms = timed(fn)
        fl = 2.0 * T * n * k
        a_ = torch.empty((T, k), dtype=torch.bfloat16, device="cuda")
        b_ = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
        ms_t = timed(lambda: torch.matmul(a_, b_.t()))
        del a_, b_
        res[name] = {"ms": ms, "shape": {"M": T, "N": n, "K": k},
                     "alg_flops_per_launch": fl,
                     "roofline": {"bound": "mfma", "achieved": fl / (ms * 1e-3) / 1e12,
                                  "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                  "frac": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
                     "torch_matmul_ms": ms_t,
                     "torch_matmul_frac": fl / (ms_t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del d, outs, o, y
    torch.cuda.empty_cache()
    return res


def attention_alg_flops(lengths, Hq, D):
    """Causal attention: query t of a sequence meets t + 1 keys (positions from 0), each
    costing D multiply-adds for q.k and D for p.v, per query head."""
    return sum(4.0 * D * Hq * L * (L + 1) / 2 for L in lengths)


def bench_attention(args, torch, gdn, S, w, reps=None):
    """The hybrid's gated full-attention layer on one workload (QK-Norm + RoPE prologue and
    the causal GQA kernel, the whole call timed with HIP events)."""
    d = S.attention_inputs(w, "cuda")
    T = int(sum(d["lengths"]))
    cu = d["cu_seqlens"] if len(d["lengths"]) > 1 else None
    o = torch.empty_like(d["q"])

    def call():
        gdn.gated_attention(d["q"], d["k"], d["v"], d["gate"], d["q_norm_w"], d["k_norm_w"],
                            cu, rotary_dim=d["rotary_dim"], out=o)

    reps = reps or max(3, min(args.steps, 10))
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    fl = attention_alg_flops(d["lengths"], w.num_q_heads, w.head_dim)
    ach = fl / (ms * 1e-3) / 1e12
    res = {"value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms, "calls": reps,
           "config": {"workload": w.name, "num_seqs": len(d["lengths"]), "tokens": T,
                      "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                      "head_dim": w.head_dim, "rotary_dim": w.rotary_dim},
           "roofline": {"bound": "mfma", "kernel": "gated attention call (prologue + "
                                                   "attention kernel)",
                        "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": ach / PEAK_BF16_TFLOPS, "alg_flops_per_launch": fl,
                        "launch_ms": ms,
                        "traffic": stored_traffic("attention_bytes_per_launch")
                        if w.name == S.ATTN_64K.name else None}}
    del d, o
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_prefill(res, S, oracle):
    """The fp64 oracle on the same 65,536-token workload, all heads, on the host's
    cores (one thread per (sequence, v head) unit, at most 32); then one thread on the
    first 2048 tokens.  Also returns the oracle's o and final state for parity."""
    d = res["d"]
    f = S.to_f64
    threads = min(oracle.default_threads(), d["v"].shape[1])
    args = lambda n: (f(d["q"][:n]), f(d["k"][:n]), f(d["v"][:n]), f(d["a"][:n]), f(d["b"][:n]),
                      f(d["z"][:n]), f(d["conv_w"]), f(d["A_log"]), f(d["dt_bias"]),
                      f(d["norm_w"]))
    T = d["q"].shape[0]
    a_full = args(T)
    t0 = time.perf_counter()
    o_ref, fs_ref, _ = oracle.prefill(*a_full, init_state=f(d["init_state"]), nthreads=threads)
    dt = time.perf_counter() - t0
    del a_full
    n1 = 2048
    a_one = args(n1)
    t1 = time.perf_counter()
    oracle.prefill(*a_one, init_state=f(d["init_state"]), nthreads=1)
    dt1 = time.perf_counter() - t1
    cb = dict(value=T / dt, unit="tokens/s", cores=threads, kind="oracle",
              sample=f"all {T} tokens of the workload, all 32 v heads, fp64, {dt:.1f} s",
              cpu_model=cpu_model(),
              single_thread={"value": n1 / dt1, "unit": "tokens/s", "cores": 1,
                             "sample": f"first {n1} tokens, all 32 v heads, {dt1:.1f} s"})
    return cb, o_ref, fs_ref


def decode_parity_and_cpu(args, torch, gdn, S, oracle):
    """n decode steps of the B=256 workload from its start, on the GPU (untimed) and
    with the fp64 oracle (timed on the host cores: the CPU baseline); o of every step
    and the state and cache after step n compared."""
    import numpy as np
    w = S.DECODE_B256
    n = args.oracle_decode_steps
    setup = S.decode_setup(w, "cuda")
    toks = S.decode_tokens(w, setup, n, "cuda")
    f = S.to_f64
    st, cc = f(setup["state"]), f(setup["conv_cache"])
    outs = []
    for s_ in range(n):
        outs.append(gdn.decode_step(toks["q"][s_], toks["k"][s_], toks["v"][s_], toks["a"][s_],
                                    toks["b"][s_], toks["z"][s_], setup["conv_w"],
                                    setup["A_log"], setup["dt_bias"], setup["norm_w"],
                                    setup["state"], setup["conv_cache"]))
    torch.cuda.synchronize()
    threads = min(oracle.default_threads(), w.decode_batch * w.num_v_heads)
    num = den = 0.0
    t0 = time.perf_counter()
    for s_ in range(n):
        o_r, st, cc = oracle.decode_step(f(toks["q"][s_]), f(toks["k"][s_]), f(toks["v"][s_]),
                                         f(toks["a"][s_]), f(toks["b"][s_]), f(toks["z"][s_]),
                                         f(setup["conv_w"]), f(setup["A_log"]),
                                         f(setup["dt_bias"]), f(setup["norm_w"]), st, cc,
                                         nthreads=threads)
        og = f(outs[s_])
        num += float(np.sum((og - o_r) ** 2))
        den += float(np.sum(o_r ** 2))
    dt = time.perf_counter() - t0
    parity = {"o": (num / den) ** 0.5, "state": rel_l2(f(setup["state"]), st),
              "conv_cache_bitwise": bool(np.array_equal(f(setup["conv_cache"]), cc)),
              "checked": f"{n} consecutive steps, all 256 sequences and heads"}
    cb = dict(value=n / dt, unit="steps/s", cores=threads, kind="oracle",
              sample=f"{n} decode steps of the B=256 workload (all sequences and heads), "
                     f"fp64, {dt:.1f} s (includes the host copies of each step's inputs)",
              cpu_model=cpu_model())
    return cb, parity


def prefill_parity(torch, gdn, S, oracle, w, group):
    """GPU prefill of workload w against the oracle over every head, `group` q/k heads
    per oracle call: relative L2 of o and of the final states (whole tensors)."""
    import numpy as np
    d = S.prefill_inputs(w, "cuda")
    o, fs = gdn.prefill(d["q"], d["k"], d["v"], d["a"], d["b"], d["z"], d["conv_w"],
                        d["A_log"], d["dt_bias"], d["norm_w"], init_state=d["init_state"],
                        cu_seqlens=d["cu_seqlens"], conv_state=d["conv_in"])
    torch.cuda.synchronize()
    Hk, Hv, D = w.num_qk_heads, w.num_v_heads, w.head_dim
    f = S.to_f64
    cu = d["cu_seqlens"].cpu().numpy()
    num = {"o": 0.0, "s": 0.0}
    den = {"o": 0.0, "s": 0.0}
    for g0 in range(0, Hk, group):
        qi, vi, ch = oracle.select_heads(range(g0, min(Hk, g0 + group)), Hk, Hv, D)
        ti = lambda x: torch.as_tensor(x, device="cuda")
        sel = lambda t, idx, dim=1: f(t.index_select(dim, ti(idx)))
        o_r, fs_r, _ = oracle.prefill(
            sel(d["q"], qi), sel(d["k"], qi), sel(d["v"], vi), sel(d["a"], vi), sel(d["b"], vi),
            sel(d["z"], vi), sel(d["conv_w"], ch, 0), sel(d["A_log"], vi, 0),
            sel(d["dt_bias"], vi, 0), f(d["norm_w"]), cu_seqlens=cu,
            init_state=None if d["init_state"] is None else sel(d["init_state"], vi),
            conv_in=None if d["conv_in"] is None else sel(d["conv_in"], ch, 2))
        og, fg = sel(o, vi), sel(fs, vi)
        num["o"] += float(np.sum((og - o_r) ** 2))
        den["o"] += float(np.sum(o_r ** 2))
        num["s"] += float(np.sum((fg - fs_r) ** 2))
        den["s"] += float(np.sum(fs_r ** 2))
        del o_r, fs_r, og, fg
    del d, o, fs
    return {"o": (num["o"] / den["o"]) ** 0.5, "state": (num["s"] / den["s"]) ** 0.5,
            "checked": "all tokens, heads and sequences"}


def summarize_trace(db_path, skip, count=None):
    """Per-kernel durations from a rocprofv3 kernel-trace database (its `kernels`
    view), grouped by kernel name and grid size, in dispatch order: dispatches
    skip .. skip + count - 1 of each group (skip = the warm-up calls; count = None for
    all the rest).  Returns a list of dicts."""
    import sqlite3
    import statistics
    con = sqlite3.connect(db_path)
    cols = [r[1] for r in con.execute("PRAGMA table_info(kernels)")]
    pick = lambda *names: next(c for c in names if c in cols)
    name_c = pick("name", "kernel_name", "kernel")
    grid_c = pick("grid_size", "grid_size_x", "grid_x", "grid")
    rows = con.execute(f'SELECT "{name_c}", "{grid_c}", start, "end" FROM kernels '
                       f'ORDER BY start').fetchall()
    groups = {}
    for name, grid, t0, t1 in rows:
        groups.setdefault((name, grid), []).append((t1 - t0) / 1e3)  # ns -> us
    out = []
    for (name, grid), durs in groups.items():
        warm = durs[skip:] if len(durs) > skip else durs
        if count is not None:
            warm = warm[:count]
        out.append({"kernel": name, "grid": grid, "dispatches": len(durs), "used": len(warm),
                    "min_us": min(warm), "median_us": statistics.median(warm),
                    "mean_us": statistics.fmean(warm), "max_us": max(warm)})
    return sorted(out, key=lambda r: -r["mean_us"] * r["used"])


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        # python bench.py --summarize-trace <results.db> [skip [count]]
        skip = int(sys.argv[3]) if len(sys.argv) > 3 else 0
        count = int(sys.argv[4]) if len(sys.argv) > 4 else None
        for r in summarize_trace(sys.argv[2], skip, count):
            if r["kernel"].startswith(("gdn::", "void gdn::")):
                print(json.dumps(r))
        return
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed prefill calls")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=int, default=30,
                    help="untimed prefill calls before the warm-up (clock ramp)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--only", choices=("all", "prefill", "decode", "tokens", "attention"),
                    default="all")
    ap.add_argument("--tokens-n", type=int, default=4,
                    help="new tokens per sequence of the n-token step leg (1..8)")
    ap.add_argument("--tokens-calls", type=int, default=100)
    ap.add_argument("--oracle-decode-steps", type=int, default=100,
                    help="decode steps the oracle recomputes (CPU baseline and parity)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle legs (CPU baseline and parity)")
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
    oracle_on = not args.no_cpu_baseline
    if oracle_on:
        import oracle
    parity = {}

    if args.only in ("all", "prefill"):
        pre = bench_prefill(args, torch, gdn, S)
        progress(f"prefill T=65536: {pre['call_ms']:.3f} ms per call")
        t_dom = pre["dominant_ms"] * 1e-3
        t_call = pre["call_ms"] * 1e-3
        ach = pre["flops"] / t_dom / 1e12
        c32 = prefill_alg_flops_per_token(16, 32, 128, C=KERNEL_CHUNK) * pre["T"]
        line.update({
            "value": pre["T"] / (pre["ms_per_step"] * 1e-3),
            "unit": "tokens/s",
            "ms_per_step": pre["ms_per_step"],
            "config": {"workload": "prefill_T65536_hk16_hv32_d128_bf16", "num_seqs": 1,
                       "seq_len": pre["T"], "num_qk_heads": 16, "num_v_heads": 32,
                       "head_dim": 128, "chunk": KERNEL_CHUNK, "state": "fp32",
                       "mfma_operands": "fp16, fp32 accumulation"},
            "roofline": {
                "bound": "mfma", "kernel": f"prefill {pre['dominant']} pass",
                "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS,
                "traffic": stored_traffic("prefill_full_bytes_per_launch"),
                "alg_flops_per_launch": pre["flops"],
                "launch_ms": pre["dominant_ms"],
                "launch_ms_source": f"HIP events on the library's stream around the full "
                                    f"pass, mean of {pre['n_attr']} warm calls",
                # the same formula at the kernel's own chunk size (the products it issues)
                "chunk32_form_flops_per_launch": c32,
                "chunk32_form_frac": c32 / t_dom / 1e12 / PEAK_BF16_TFLOPS,
            },
            "prefill_path": {
                "call_ms": pre["call_ms"], "call_ms_min": pre["call_ms_min"],
                "mfma_frac": pre["flops"] / t_call / 1e12 / PEAK_BF16_TFLOPS,
                "hbm_frac": pre["bytes"] / t_call / 1e9 / PEAK_HBM_GBS,
                "alg_bytes": pre["bytes"], "per_kernel_ms": pre["per_kernel_ms"],
            },
        })
        # the same workload with slow decay (exp(A_log) = 0.03): every segment map is
        # non-negligible, so the map and combine passes walk every chunk
        slow = bench_prefill(args, torch, gdn, S, slow_decay=0.03, d=pre["d"])
        progress(f"prefill slow decay: {slow['call_ms']:.3f} ms per call")
        line["prefill_slow_decay"] = {
            "value": slow["T"] / (slow["call_ms"] * 1e-3), "unit": "tokens/s",
            "ms_per_step": slow["call_ms"], "per_kernel_ms": slow["per_kernel_ms"],
            "config": {"workload": "prefill_T65536_hk16_hv32_bf16, exp(A_log) = 0.03"}}
        del slow
        # the other prefill workloads, tokens/s of the whole call
        line["prefill_configs"] = {w.name: bench_prefill_config(args, torch, gdn, S, w)
                                   for w in (S.PREFILL_4K, S.VARLEN_64)}
        # the projections on either side of the mixer at the same T
        progress("prefill T=4096 and varlen done")
        pj = bench_projections(args, torch, gdn, S)
        progress("projections done")
        line["projections"] = pj
        line["layer_ms"] = (pj["in_projection"]["ms"] + pre["call_ms"] +
                            pj["out_projection"]["ms"])
        if oracle_on:
            cb, o_ref, fs_ref = cpu_baseline_prefill(pre, S, oracle)
            progress("oracle prefill (CPU baseline) done")
            line["cpu_baseline"] = cb
            parity[S.PREFILL_64K.name] = {"o": rel_l2(S.to_f64(pre["out"]), o_ref),
                                          "state": rel_l2(S.to_f64(pre["fs"]), fs_ref),
                                          "checked": "all tokens and heads"}
            del o_ref, fs_ref
            for w, grp in ((S.TINY, 1), (S.PREFILL_4K, 16), (S.VARLEN_64, 4)):
                parity[w.name] = prefill_parity(torch, gdn, S, oracle, w, grp)
        del pre
        torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        dec = bench_decode(args, torch, gdn, S)
        progress(f"decode: {dec['ms_per_step']:.4f} ms per step")
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
        # ... and in fp8 (E4M3 values, one power-of-two scale per state row)
        d8 = bench_decode(args, torch, gdn, S, state_fp8=True, toks=dec["toks"])
        t8 = d8["ms_per_step"] * 1e-3
        g8 = d8["bytes"] / t8 / 1e9
        dline["fp8_state"] = {
            "value": 1.0 / t8, "unit": "steps/s", "ms_per_step": d8["ms_per_step"],
            "roofline": {"bound": "hbm", "kernel": "decode_step (fp8 state)", "achieved": g8,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": g8 / PEAK_HBM_GBS,
                         "alg_bytes_per_launch": d8["bytes"], "launch_ms": d8["ms_per_step"]}}
        del dec, d16, d8
        torch.cuda.empty_cache()
        if oracle_on:
            cbd, par = decode_parity_and_cpu(args, torch, gdn, S, oracle)
            progress("oracle decode done")
            dline["cpu_baseline"] = cbd
            parity[S.DECODE_B256.name] = par
        if args.only == "decode":
            line.update({"value": dline["value"], "unit": "steps/s",
                         "ms_per_step": dline["ms_per_step"], "config": dline["config"],
                         "roofline": dline["roofline"], "bf16_state": dline["bf16_state"],
                         "fp8_state": dline["fp8_state"]})
            if "cpu_baseline" in dline:
                line["cpu_baseline"] = dline.pop("cpu_baseline")
        else:
            line["decode"] = dline
    if args.only in ("all", "tokens"):
        tl = bench_decode_tokens(args, torch, gdn, S)
        progress("n-token step done")
        if args.only == "tokens":
            line.update({"value": tl["value"], "unit": "tokens/s",
                         "ms_per_step": tl["ms_per_step"], "config": tl["config"],
                         "roofline": tl["roofline"], "verify": tl["verify"]})
        else:
            line["decode_tokens"] = tl
    if args.only in ("all", "attention"):
        al = {}
        for w in (S.ATTN_64K, S.ATTN_4K, S.ATTN_VARLEN):
            al[w.name] = bench_attention(args, torch, gdn, S, w)
            progress(f"attention {w.name}: {al[w.name]['ms_per_call']:.3f} ms per call")
        if args.only == "attention":
            a0 = al[S.ATTN_64K.name]
            line.update({"value": a0["value"], "unit": "tokens/s",
                         "ms_per_step": a0["ms_per_call"], "config": a0["config"],
                         "roofline": a0["roofline"], "attention": al})
        else:
            line["gated_attention"] = al
    if parity:
        line["parity"] = parity
    line.setdefault("cpu_baseline", None)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""GPU parity of the chunked prefill against the fp64 oracle.

Bars (relative L2 over the whole tensor): o <= 3e-3, final state <= 1e-3.
Indexing is bit-exact: a packed sequence's rows and final state equal its
standalone run bit for bit.  Full-size workloads run in the launch
configuration the benchmark uses and are checked over every head, token and
sequence: the oracle runs one group of q/k heads (and their v heads) at a time
to bound host memory, and the squared errors are summed over the groups, so the
relative L2 is that of the whole tensor.
"""
import numpy as np
import pytest
import torch

import gdn_synth as S
import oracle

gpu = pytest.mark.gpu
O_TOL, STATE_TOL = 3e-3, 1e-3


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def _gdn():
    import linear_attention_sequence_causal_amd as gdn
    return gdn


def run_gpu(d, cu=True, **kw):
    gdn = _gdn()
    args = dict(init_state=d["init_state"], conv_state=d["conv_in"])
    args.update(kw)
    out = gdn.prefill(d["q"], d["k"], d["v"], d["a"], d["b"], d["z"], d["conv_w"], d["A_log"],
                      d["dt_bias"], d["norm_w"], cu_seqlens=d["cu_seqlens"] if cu else None,
                      return_conv_state=True, **args)
    torch.cuda.synchronize()
    return out


def run_oracle(d, qk_heads=None, q_scale=1.0):
    """Oracle on the given q/k heads (and their v heads); returns (o, fs, v_idx)."""
    f = S.to_f64
    Hk = d["q"].shape[1]
    Hv = d["v"].shape[1]
    D = d["q"].shape[2]
    if qk_heads is None:
        qk_heads = range(Hk)
    qi, vi, ch = oracle.select_heads(qk_heads, Hk, Hv, D)
    qi_t = torch.as_tensor(qi, device=d["q"].device)
    vi_t = torch.as_tensor(vi, device=d["q"].device)
    ch_t = torch.as_tensor(ch, device=d["q"].device)
    sel = lambda t, idx, dim=1: f(t.index_select(dim, idx))
    init = d["init_state"]
    conv_in = d["conv_in"]
    o, fs, co = oracle.prefill(
        sel(d["q"], qi_t), sel(d["k"], qi_t), sel(d["v"], vi_t), sel(d["a"], vi_t),
        sel(d["b"], vi_t), sel(d["z"], vi_t), sel(d["conv_w"], ch_t, 0), sel(d["A_log"], vi_t, 0),
        sel(d["dt_bias"], vi_t, 0), f(d["norm_w"]), cu_seqlens=d["cu_seqlens"].cpu().numpy(),
        init_state=None if init is None else sel(init, vi_t),
        conv_in=None if conv_in is None else sel(conv_in, ch_t, 2), q_scale=q_scale)
    return o, fs, co, vi


def check_parity(d, qk_heads=None, tag="", group=None):
    """GPU run against the oracle on the given q/k heads (all by default), `group`
    q/k heads per oracle call; returns the GPU outputs."""
    o, fs, co = run_gpu(d)
    Hk = d["q"].shape[1]
    heads = list(range(Hk)) if qk_heads is None else list(qk_heads)
    group = group or len(heads)
    num = {"o": 0.0, "s": 0.0}
    den = {"o": 0.0, "s": 0.0}
    for i in range(0, len(heads), group):
        o_ref, fs_ref, _, vi = run_oracle(d, heads[i:i + group])
        vi_t = torch.as_tensor(vi, device=o.device)
        o_g = S.to_f64(o.index_select(1, vi_t))
        fs_g = S.to_f64(fs.index_select(1, vi_t))
        assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(fs_g))
        num["o"] += float(np.sum((o_g - o_ref) ** 2))
        den["o"] += float(np.sum(o_ref ** 2))
        num["s"] += float(np.sum((fs_g - fs_ref) ** 2))
        den["s"] += float(np.sum(fs_ref ** 2))
        del o_ref, fs_ref, o_g, fs_g
    eo = (num["o"] / max(den["o"], 1e-300)) ** 0.5
    es = (num["s"] / max(den["s"], 1e-300)) ** 0.5
    print(f"{tag}: o rel-L2 {eo:.3e}  final-state rel-L2 {es:.3e}", flush=True)
    assert eo <= O_TOL, eo
    assert es <= STATE_TOL, es
    return o, fs, co


@gpu
def test_tiny_fp32_full_parity():
    d = S.prefill_inputs(S.TINY, "cuda")
    _, _, co = check_parity(d, tag="T=512 Hk=1 Hv=2 fp32")


@gpu
def test_prefill_4k_full_parity():
    d = S.prefill_inputs(S.PREFILL_4K, "cuda")
    check_parity(d, tag="T=4096 Hk=16 Hv=32 bf16")


@gpu
@pytest.mark.parametrize("hk,hv", [(4, 4), (2, 8), (3, 3), (2, 6)])
def test_head_layouts(hk, hv):
    """One v head per q/k head (r = 1), four (r = 4: two workgroups of two v heads per
    q/k head), three (r = 3: one v head per workgroup), and a head count that is not a
    multiple of the workgroup id groups of 8; multi-segment (T = 2000)."""
    w = S.scaled(S.PREFILL_4K, lengths=(2000, 300), num_qk_heads=hk, num_v_heads=hv,
                 seed=30 + hv, init_state_std=0.01, conv_history=True)
    d = S.prefill_inputs(w, "cuda")
    check_parity(d, tag=f"Hk={hk} Hv={hv} T=2300")


@gpu
def test_q_scale_and_norm_weight():
    """q_scale = 1/sqrt(128) and a non-uniform RMSNorm weight (the workloads use 1 and
    ones): q_scale reaches M, its fp32 diagonal and Q H; the weight the epilogue."""
    import math
    w = S.scaled(S.PREFILL_4K, lengths=(700, 333), num_qk_heads=2, num_v_heads=4, seed=40,
                 init_state_std=0.01)
    d = S.prefill_inputs(w, "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(41)
    d["norm_w"] = torch.rand(128, generator=g, device="cuda") + 0.5
    qs = 1.0 / math.sqrt(128)
    o, fs, _ = run_gpu(d, q_scale=qs)
    o_ref, fs_ref, _, vi = run_oracle(d, q_scale=qs)
    eo, es = rel_l2(S.to_f64(o)[:, vi], o_ref), rel_l2(S.to_f64(fs)[:, vi], fs_ref)
    print(f"q_scale 1/sqrt(128), random norm weight: o rel-L2 {eo:.3e} state rel-L2 {es:.3e}")
    assert eo <= O_TOL and es <= STATE_TOL


@gpu
def test_prefill_64k_all_heads():
    """T = 65536, 16/32 heads, initial state ~ N(0, 0.01^2): o and the final state of
    all 32 v heads."""
    d = S.prefill_inputs(S.PREFILL_64K, "cuda")
    check_parity(d, tag="T=65536 bf16, all 32 v heads", group=4)


@gpu
def test_varlen_64_all_heads():
    """64 packed sequences of 128-32768 tokens: o and the 64 final states of all 32 v
    heads."""
    d = S.prefill_inputs(S.VARLEN_64, "cuda")
    check_parity(d, tag=f"varlen N=64 T={d['q'].shape[0]}, all 32 v heads", group=2)


@gpu
@pytest.mark.parametrize("T", [1, 2, 3, 63, 64, 65, 130, 700])
def test_ragged_lengths_small_heads(T):
    w = S.scaled(S.PREFILL_4K, lengths=(T,), num_qk_heads=2, num_v_heads=4, seed=100 + T,
                 init_state_std=0.01, conv_history=True)
    d = S.prefill_inputs(w, "cuda")
    o, fs, co = check_parity(d, tag=f"T={T}")
    _, _, co_ref, _ = run_oracle(d)
    assert np.array_equal(S.to_f64(co), co_ref)  # conv state: raw rows, bit-exact


@gpu
@pytest.mark.parametrize("alog", [0.15, 0.03])
def test_slow_decay_multi_segment(alog):
    """Slow decay (alpha ~ 0.9 .. 0.98 per token): the segment maps are not
    negligible, so the map pass computes A and B over every chunk and the
    combine pass must carry the state across segment boundaries."""
    import math
    w = S.scaled(S.PREFILL_4K, lengths=(2600, 900), num_qk_heads=2, num_v_heads=4, seed=21,
                 init_state_std=0.01)
    d = S.prefill_inputs(w, "cuda")
    d["A_log"] = torch.full_like(d["A_log"], math.log(alog))
    o, fs, _ = run_gpu(d)
    o_ref, fs_ref, _, _ = run_oracle(d)
    eo, es = rel_l2(S.to_f64(o), o_ref), rel_l2(S.to_f64(fs), fs_ref)
    print(f"slow decay exp(A_log)={alog}: o rel-L2 {eo:.3e} final-state rel-L2 {es:.3e}")
    assert eo <= O_TOL and es <= STATE_TOL


@gpu
def test_segment_maps_alternate_zero_and_nonzero():
    """Along one sequence the decay switches between almost none and strong from one
    segment to the next, so the segments' A maps alternate between negligible (flagged
    zero: the next segment starts from the B map itself) and not (the combine pass
    chains them, reloading the state from a B map after a zero one).  Two of the four
    heads take the pattern in opposite phase.

    The weak segments are the no-decay regime (nothing damps the rounding of the MFMA
    operands); both outputs are held to the main bars (a wrong start state gives errors
    of order 0.1-1)."""
    T = 3000
    w = S.scaled(S.PREFILL_4K, lengths=(T,), num_qk_heads=2, num_v_heads=4, seed=22,
                 init_state_std=0.01)
    d = S.prefill_inputs(w, "cuda")
    d["A_log"] = torch.zeros_like(d["A_log"])      # g = -softplus(a + dt_bias)
    d["dt_bias"] = torch.zeros_like(d["dt_bias"])
    # segments of 256 tokens for T = 3000 and 4 v heads (the last two are 224 tokens)
    blk = (torch.arange(T, device="cuda") // 256) % 2
    weak = torch.full((T,), -12.0, device="cuda")   # g ~ -6e-6 per token
    strong = torch.full((T,), 3.0, device="cuda")   # g ~ -3 per token
    for h in range(4):
        phase = blk if h % 2 == 0 else 1 - blk
        d["a"][:, h] = torch.where(phase == 1, strong, weak)
    o, fs, _ = run_gpu(d)
    o_ref, fs_ref, _, vi = run_oracle(d)
    eo, es = rel_l2(S.to_f64(o)[:, vi], o_ref), rel_l2(S.to_f64(fs)[:, vi], fs_ref)
    print(f"alternating zero/non-zero segment maps: o rel-L2 {eo:.3e} final-state rel-L2 "
          f"{es:.3e}")
    assert eo <= O_TOL and es <= STATE_TOL


@gpu
def test_varlen_with_empty_and_short_sequences():
    w = S.scaled(S.PREFILL_4K, lengths=(5, 0, 1, 64, 2, 0, 129, 3, 600), num_qk_heads=2,
                 num_v_heads=4, seed=7, init_state_std=0.01, conv_history=True)
    d = S.prefill_inputs(w, "cuda")
    o, fs, co = check_parity(d, tag="varlen with empty/short sequences")
    # empty sequences return their initial state bit for bit
    for n in (1, 5):
        assert torch.equal(fs[n], d["init_state"][n])
        assert torch.equal(co[n], d["conv_in"][n])


@gpu
def test_many_packed_sequences():
    """More sequences than the segment table's 1024 threads take in one pass (1,502: short
    ones of 0..80 tokens around two long ones that split into several segments of at most
    2048 tokens), so the table's scan runs in several passes and the full pass's
    longest-first order sorts segments of many different lengths."""
    lengths = [int(x) for x in np.random.default_rng(11).integers(0, 81, 1500)]
    lengths.insert(700, 5000)
    lengths.insert(1200, 9001)
    w = S.scaled(S.PREFILL_4K, lengths=tuple(lengths), num_qk_heads=1, num_v_heads=2, seed=12,
                 init_state_std=0.01, conv_history=True)
    d = S.prefill_inputs(w, "cuda")
    check_parity(d, tag=f"{len(lengths)} packed sequences")


@gpu
def test_packing_is_bit_exact():
    """Each packed sequence's o rows and final state equal its standalone run."""
    w = S.scaled(S.PREFILL_4K, lengths=(300, 77, 1024, 5, 2000), seed=9, init_state_std=0.01,
                 conv_history=True)
    d = S.prefill_inputs(w, "cuda")
    o, fs, co = run_gpu(d)
    cu = d["cu_seqlens"].cpu().tolist()
    gdn = _gdn()
    for n in range(len(cu) - 1):
        sl = slice(cu[n], cu[n + 1])
        on, fn, cn = gdn.prefill(d["q"][sl].contiguous(), d["k"][sl].contiguous(),
                                 d["v"][sl].contiguous(), d["a"][sl].contiguous(),
                                 d["b"][sl].contiguous(), d["z"][sl].contiguous(), d["conv_w"],
                                 d["A_log"], d["dt_bias"], d["norm_w"],
                                 init_state=d["init_state"][n:n + 1].contiguous(),
                                 conv_state=d["conv_in"][n:n + 1].contiguous(),
                                 return_conv_state=True)
        torch.cuda.synchronize()
        # segments start at each sequence's first token and the segment length
        # is the same for the packed (T = 3406) and standalone runs (256 tokens)
        assert torch.equal(on, o[sl])
        assert torch.equal(fn, fs[n:n + 1])
        assert torch.equal(cn, co[n:n + 1])


@gpu
def test_packing_bit_exact_single_segment():
    """With every sequence inside one segment the packed and standalone runs
    execute the same chunk sequence: bitwise equal."""
    w = S.scaled(S.PREFILL_4K, lengths=(200, 64, 1, 255, 90), num_qk_heads=2, num_v_heads=4,
                 seed=11, init_state_std=0.01, conv_history=True)
    d = S.prefill_inputs(w, "cuda")
    o, fs, co = run_gpu(d)
    cu = d["cu_seqlens"].cpu().tolist()
    gdn = _gdn()
    for n in range(len(cu) - 1):
        sl = slice(cu[n], cu[n + 1])
        on, fn = gdn.prefill(d["q"][sl].contiguous(), d["k"][sl].contiguous(),
                             d["v"][sl].contiguous(), d["a"][sl].contiguous(),
                             d["b"][sl].contiguous(), d["z"][sl].contiguous(), d["conv_w"],
                             d["A_log"], d["dt_bias"], d["norm_w"],
                             init_state=d["init_state"][n:n + 1].contiguous(),
                             conv_state=d["conv_in"][n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(on, o[sl])
        assert torch.equal(fn, fs[n:n + 1])


@gpu
def test_identity_gates_keep_state_and_zero_gate_zeroes_output():
    w = S.scaled(S.PREFILL_4K, lengths=(1000,), num_qk_heads=2, num_v_heads=4, seed=12,
                 init_state_std=0.01)
    d = S.prefill_inputs(w, "cuda")
    d["b"] = torch.full_like(d["b"], -float("inf"))       # beta = 0
    d["A_log"] = torch.full_like(d["A_log"], -float("inf"))  # alpha = 1
    d["z"] = torch.zeros_like(d["z"])
    o, fs, _ = run_gpu(d)
    assert torch.equal(fs, d["init_state"])
    assert torch.count_nonzero(o) == 0


@gpu
def test_final_state_may_alias_init_state():
    w = S.scaled(S.PREFILL_4K, lengths=(3000, 700), num_qk_heads=2, num_v_heads=4, seed=13,
                 init_state_std=0.01)
    d = S.prefill_inputs(w, "cuda")
    o_ref, fs_ref, _ = run_gpu(d)
    st = d["init_state"].clone()
    gdn = _gdn()
    o, fs = gdn.prefill(d["q"], d["k"], d["v"], d["a"], d["b"], d["z"], d["conv_w"], d["A_log"],
                        d["dt_bias"], d["norm_w"], cu_seqlens=d["cu_seqlens"], init_state=st,
                        final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(st, fs_ref)


@gpu
def test_deterministic():
    d = S.prefill_inputs(S.scaled(S.PREFILL_4K, seed=14), "cuda")
    o1, f1, _ = run_gpu(d)
    o2, f2, _ = run_gpu(d)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@gpu
def test_one_sequence_with_or_without_cu_seqlens_is_bitwise():
    """One sequence builds no segment table: its records come from (segment length, T).
    Given as cu_seqlens = [0, T] or as NULL, the call runs the same segments (several
    here, with a ragged tail) and is bitwise equal."""
    w = S.scaled(S.PREFILL_4K, lengths=(1517,), num_qk_heads=2, num_v_heads=4, seed=19,
                 init_state_std=0.01, conv_history=True)
    d = S.prefill_inputs(w, "cuda")
    o1, f1, c1 = run_gpu(d, cu=True)
    o2, f2, c2 = run_gpu(d, cu=False)
    assert torch.equal(o1, o2) and torch.equal(f1, f2) and torch.equal(c1, c2)
    o_ref, fs_ref, _, _ = run_oracle(d)
    assert rel_l2(S.to_f64(o1), o_ref) <= O_TOL and rel_l2(S.to_f64(f1), fs_ref) <= STATE_TOL


def _split_run(d, t0):
    gdn = _gdn()
    ca = lambda t, a, b: t[a:b].contiguous()
    T = d["q"].shape[0]
    oa, fa, cva = gdn.prefill(ca(d["q"], 0, t0), ca(d["k"], 0, t0), ca(d["v"], 0, t0),
                              ca(d["a"], 0, t0), ca(d["b"], 0, t0), ca(d["z"], 0, t0),
                              d["conv_w"], d["A_log"], d["dt_bias"], d["norm_w"],
                              init_state=d["init_state"], return_conv_state=True)
    ob, fb = gdn.prefill(ca(d["q"], t0, T), ca(d["k"], t0, T), ca(d["v"], t0, T),
                         ca(d["a"], t0, T), ca(d["b"], t0, T), ca(d["z"], t0, T),
                         d["conv_w"], d["A_log"], d["dt_bias"], d["norm_w"],
                         init_state=fa, conv_state=cva)
    torch.cuda.synchronize()
    return torch.cat([oa, ob]), fb


@gpu
def test_split_sequence_carries_state():
    """prefill(x) equals prefill(x[t0:], init = final(x[:t0]), conv = conv(x[:t0]))
    within the bars (the split changes chunk boundaries, segments and which
    chunks take the split-precision state update)."""
    w = S.scaled(S.PREFILL_4K, lengths=(1280,), num_qk_heads=2, num_v_heads=4, seed=15,
                 init_state_std=0.01)
    d = S.prefill_inputs(w, "cuda")
    o, fs, _ = run_gpu(d)
    for t0 in (256, 100, 1):
        o2, fb = _split_run(d, t0)
        assert rel_l2(S.to_f64(o2), S.to_f64(o)) < O_TOL
        assert rel_l2(S.to_f64(fb), S.to_f64(fs)) < STATE_TOL


@gpu
def test_split_at_chunk_boundary_is_bitwise():
    """With one segment (up to 256 tokens here), a split at a multiple of the 32-token
    chunk runs exactly the same chunk sequence with the same arithmetic per chunk (no
    chunk's precision depends on where the sequence ends): bitwise equal."""
    w = S.scaled(S.PREFILL_4K, lengths=(256,), num_qk_heads=2, num_v_heads=4, seed=17,
                 init_state_std=0.01)
    d = S.prefill_inputs(w, "cuda")
    o, fs, _ = run_gpu(d)
    for t0 in (64, 160):
        o2, fb = _split_run(d, t0)
        assert torch.equal(o2, o) and torch.equal(fb, fs)


@gpu
def test_decode_after_prefill_matches_longer_prefill():
    gdn = _gdn()
    w = S.scaled(S.PREFILL_4K, lengths=(777,), num_qk_heads=16, num_v_heads=32, seed=16,
                 init_state_std=0.01)
    d = S.prefill_inputs(w, "cuda")
    T, n = 770, 7
    o_all, fs_all, _ = run_gpu(d)
    c = lambda t, a, b: t[a:b].contiguous()
    o_p, st, cs = gdn.prefill(c(d["q"], 0, T), c(d["k"], 0, T), c(d["v"], 0, T),
                              c(d["a"], 0, T), c(d["b"], 0, T), c(d["z"], 0, T), d["conv_w"],
                              d["A_log"], d["dt_bias"], d["norm_w"], init_state=d["init_state"],
                              return_conv_state=True)
    outs = [o_p]
    for t in range(T, T + n):
        outs.append(gdn.decode_step(c(d["q"], t, t + 1), c(d["k"], t, t + 1), c(d["v"], t, t + 1),
                                    c(d["a"], t, t + 1), c(d["b"], t, t + 1), c(d["z"], t, t + 1),
                                    d["conv_w"], d["A_log"], d["dt_bias"], d["norm_w"], st, cs))
    torch.cuda.synchronize()
    o2 = torch.cat(outs)
    assert rel_l2(S.to_f64(o2), S.to_f64(o_all)) < O_TOL
    assert rel_l2(S.to_f64(st), S.to_f64(fs_all)) < STATE_TOL


@gpu
def test_delta_rule_write_reproduces_the_last_value():
    """beta = 1 (b = +inf), alpha = 1 (A_log = -inf): the last write makes the state map the
    last key to the last value, S_T k_T = v_T with the post-prologue k and v ("Qwen3-Next
    80B-A3B" field guide, cutaway 02: with beta = 1 the write replaces the value read
    under k).  No decay damps the rounding of the MFMA operands here; o and the final
    state are held to the main bars, and the delta-rule write to 1e-3 (a wrong write
    gives errors of order 1)."""
    w = S.scaled(S.PREFILL_4K, lengths=(200,), num_qk_heads=1, num_v_heads=2, seed=13,
                 init_state_std=0.0)
    d = S.prefill_inputs(w, "cuda")
    d["b"] = torch.full_like(d["b"], float("inf"))
    d["A_log"] = torch.full_like(d["A_log"], -float("inf"))
    o, fs, _ = run_gpu(d)
    o_ref, fs_ref, _, _ = run_oracle(d)
    eo, es = rel_l2(S.to_f64(o), o_ref), rel_l2(S.to_f64(fs), fs_ref)
    f = S.to_f64
    wr = []
    for h in range(2):
        _, kk, vv = oracle.prologue(f(d["q"]), f(d["k"]), f(d["v"]), f(d["conv_w"]), h)
        Sk = f(fs[0, h]).T @ kk[-1]  # stored H = S^T
        wr.append(np.linalg.norm(Sk - vv[-1]) / np.linalg.norm(vv[-1]))
        # the oracle's own state meets it to rounding (pinned on the CPU as P2)
        assert np.linalg.norm(fs_ref[0, h].T @ kk[-1] - vv[-1]) <= 1e-6 * np.linalg.norm(vv[-1])
    print(f"beta=1 alpha=1: o rel-L2 {eo:.3e} final-state rel-L2 {es:.3e}; "
          f"|S k - v|/|v| {max(wr):.3e}")
    assert eo <= O_TOL and es <= STATE_TOL and max(wr) <= 1e-3


@gpu
def test_extreme_gates_stay_finite_and_match():
    """alpha -> 0 on some heads (A_log = 100: e^g underflows), beta in {0, 1} on others
    (b = -inf, +inf): no NaN, and o and the final state match the oracle."""
    w = S.scaled(S.PREFILL_4K, lengths=(300,), num_qk_heads=2, num_v_heads=4, seed=14)
    d = S.prefill_inputs(w, "cuda")
    d["A_log"][0] = 100.0
    d["b"][:, 1] = float("inf")
    d["b"][:, 2] = -float("inf")
    d["A_log"][3] = 100.0
    d["b"][::7, 3] = -float("inf")
    check_parity(d, tag="extreme gates")


@gpu
def test_invalid_cu_seqlens_is_reported_and_runs_nothing():
    """cu_seqlens that does not end at T, or that decreases: the device-side check
    leaves o and the final states unwritten and sets the error flag, which
    check_device_errors() reports once; a valid call afterwards runs normally."""
    gdn = _gdn()
    w = S.scaled(S.PREFILL_4K, lengths=(300, 200), num_qk_heads=2, num_v_heads=4, seed=18,
                 init_state_std=0.01)
    d = S.prefill_inputs(w, "cuda")
    gdn.check_device_errors()  # nothing pending
    # (one-sequence tables are checked by the kernels themselves: no table is built)
    for bad in ([0, 300, 499], [0, 350, 300, 500], [5, 300, 500], [0, 499], [3, 500]):
        cu = torch.tensor(bad, dtype=torch.int32, device="cuda")
        N = cu.numel() - 1
        o = torch.full_like(d["v"], 7.0)
        fs = torch.full((N, 4, 128, 128), 7.0, device="cuda")
        gdn.prefill(d["q"], d["k"], d["v"], d["a"], d["b"], d["z"], d["conv_w"], d["A_log"],
                    d["dt_bias"], d["norm_w"], cu_seqlens=cu, out=o, final_state=fs)
        with pytest.raises(gdn.GdnError, match="cu_seqlens"):
            gdn.check_device_errors()
        assert bool(torch.all(o == 7.0)) and bool(torch.all(fs == 7.0))
        gdn.check_device_errors()  # cleared
    o, fs, _ = run_gpu(d)
    o_ref, fs_ref, _, _ = run_oracle(d)
    assert rel_l2(S.to_f64(o), o_ref) <= O_TOL and rel_l2(S.to_f64(fs), fs_ref) <= STATE_TOL
    gdn.check_device_errors()


@gpu
def test_sigmoid_output_gate_variant():
    """The epilogue with the sigmoid output gate (gdn_params.output_gate =
    GDN_GATE_SIGMOID) against the oracle's sigmoid-gated mixer, with a multi-segment
    sequence and a short one; the final states equal the SiLU-gated run's bit for bit
    (the gate touches o only)."""
    w = S.scaled(S.PREFILL_4K, lengths=(2300, 70), num_qk_heads=2, num_v_heads=4, seed=23,
                 init_state_std=0.01, conv_history=True)
    d = S.prefill_inputs(w, "cuda")
    o, fs, _ = run_gpu(d, output_gate="sigmoid")
    _, fs_silu, _ = run_gpu(d)
    f = S.to_f64
    o_ref, fs_ref, _ = oracle.prefill(
        f(d["q"]), f(d["k"]), f(d["v"]), f(d["a"]), f(d["b"]), f(d["z"]), f(d["conv_w"]),
        f(d["A_log"]), f(d["dt_bias"]), f(d["norm_w"]), cu_seqlens=d["cu_seqlens"].cpu().numpy(),
        init_state=f(d["init_state"]), conv_in=f(d["conv_in"]), output_gate="sigmoid")
    eo, es = rel_l2(f(o), o_ref), rel_l2(f(fs), fs_ref)
    print(f"sigmoid output gate: o rel-L2 {eo:.3e} final-state rel-L2 {es:.3e}")
    assert eo <= O_TOL and es <= STATE_TOL
    assert torch.equal(fs, fs_silu)

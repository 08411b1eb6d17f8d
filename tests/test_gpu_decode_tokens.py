"""GPU parity of the multi-token step (n new tokens per sequence on a cached state)
against the fp64 oracle.

Bars as for decode: relative L2 <= 3e-3 on o (dominated by its bf16 rounding) and
<= 1e-3 on the state; the arithmetic is fp32, so the state lands far below.  The
conv cache holds raw inputs and must match bit for bit, and a verify pass
(num_commit = 0) must leave state and cache bit for bit.
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


def _case(w, n, dev="cuda"):
    """Setup and n tokens per sequence in the [B, n, ...] layout."""
    setup = S.decode_setup(w, dev)
    toks = S.decode_tokens(w, setup, n, dev)
    bn = {key: val.transpose(0, 1).contiguous() for key, val in toks.items()}
    return setup, bn


def _gpu(setup, t, state, cache, num_commit=None, q_scale=1.0):
    import linear_attention_sequence_causal_amd as gdn
    o = gdn.decode_tokens(t["q"], t["k"], t["v"], t["a"], t["b"], t["z"], setup["conv_w"],
                          setup["A_log"], setup["dt_bias"], setup["norm_w"], state, cache,
                          num_commit=num_commit, q_scale=q_scale)
    torch.cuda.synchronize()
    return o


def _oracle(setup, t, state, cache, sel=slice(None), num_commit=None, q_scale=1.0):
    f = S.to_f64
    return oracle.decode_tokens(f(t["q"][sel]), f(t["k"][sel]), f(t["v"][sel]), f(t["a"][sel]),
                                f(t["b"][sel]), f(t["z"][sel]), f(setup["conv_w"]),
                                f(setup["A_log"]), f(setup["dt_bias"]), f(setup["norm_w"]),
                                f(state[sel]), f(cache[sel]), num_commit=num_commit,
                                q_scale=q_scale)


def _check(setup, t, n, sel=slice(None), num_commit=None, label=""):
    st0, cc0 = setup["state"].clone(), setup["conv_cache"].clone()
    commit_dev = None
    if num_commit is not None:
        commit_dev = torch.tensor(num_commit, dtype=torch.int32, device="cuda")
    o = _gpu(setup, t, setup["state"], setup["conv_cache"], commit_dev)
    o_ref, st_ref, cc_ref = _oracle(setup, t, st0, cc0, sel, num_commit)
    f = S.to_f64
    eo, es = rel_l2(f(o[sel]), o_ref), rel_l2(f(setup["state"][sel]), st_ref)
    print(f"{label}: o rel-L2 {eo:.3e} state rel-L2 {es:.3e}")
    assert eo < O_TOL
    assert es < 1e-5
    assert np.array_equal(f(setup["conv_cache"][sel]), cc_ref)
    return o, st0, cc0


@gpu
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
def test_tokens_match_oracle_bf16(n):
    w = S.scaled(S.DECODE_B256, decode_batch=4, seed=60 + n)
    setup, t = _case(w, n)
    _check(setup, t, n, label=f"decode_tokens n={n} Hk=16 Hv=32")


@gpu
def test_tokens_fp32_small_heads():
    w = S.scaled(S.DECODE_B256, decode_batch=3, num_qk_heads=1, num_v_heads=2,
                 act_dtype=torch.float32, seed=70)
    setup, t = _case(w, 4)
    st0, cc0 = setup["state"].clone(), setup["conv_cache"].clone()
    o = _gpu(setup, t, setup["state"], setup["conv_cache"])
    o_ref, st_ref, cc_ref = _oracle(setup, t, st0, cc0)
    assert rel_l2(S.to_f64(o), o_ref) < 1e-5
    assert rel_l2(S.to_f64(setup["state"]), st_ref) < 1e-5
    assert np.array_equal(S.to_f64(setup["conv_cache"]), cc_ref)


@gpu
@pytest.mark.parametrize("hk,hv,n", [(4, 4, 3), (2, 8, 3), (3, 9, 3), (1, 1, 3), (4, 4, 6),
                                     (3, 9, 7), (2, 10, 4), (1, 7, 2), (1, 8, 5)])
def test_tokens_head_layouts(hk, hv, n):
    """One to eight v heads per q/k head, with four and with eight token slots: every v
    head's workgroup convolves the q/k rows from the cache, which a second kernel
    advances afterwards."""
    w = S.scaled(S.DECODE_B256, decode_batch=5, num_qk_heads=hk, num_v_heads=hv,
                 seed=71 + hv + 16 * n)
    setup, t = _case(w, n)
    _check(setup, t, n, label=f"decode_tokens n={n} Hk={hk} Hv={hv}")


@gpu
def test_tokens_commit_counts():
    """Per-sequence commit counts (0, partial, all, clamped): o of all n tokens; state
    and cache advanced by the count; count 0 leaves both bit for bit."""
    n = 5
    w = S.scaled(S.DECODE_B256, decode_batch=6, seed=80)
    setup, t = _case(w, n)
    commit = [0, 1, 5, 3, 2, 7]
    o, st0, cc0 = _check(setup, t, n, num_commit=commit, label="decode_tokens commit")
    assert torch.equal(setup["state"][0], st0[0])
    assert torch.equal(setup["conv_cache"][0], cc0[0])


@gpu
def test_verify_then_commit():
    """Speculative flow: a verify pass (commit 0) changes nothing; the commit pass with
    the accepted counts gives the same outputs bit for bit and the oracle's state."""
    n = 4
    w = S.scaled(S.DECODE_B256, decode_batch=4, seed=81)
    setup, t = _case(w, n)
    st0, cc0 = setup["state"].clone(), setup["conv_cache"].clone()
    zeros = torch.zeros(4, dtype=torch.int32, device="cuda")
    o1 = _gpu(setup, t, setup["state"], setup["conv_cache"], zeros)
    assert torch.equal(setup["state"], st0) and torch.equal(setup["conv_cache"], cc0)
    accepted = [4, 0, 2, 1]
    o2 = _gpu(setup, t, setup["state"], setup["conv_cache"],
              torch.tensor(accepted, dtype=torch.int32, device="cuda"))
    assert torch.equal(o1, o2)
    _, st_ref, cc_ref = _oracle(setup, t, st0, cc0, num_commit=accepted)
    assert rel_l2(S.to_f64(setup["state"]), st_ref) < 1e-5
    assert np.array_equal(S.to_f64(setup["conv_cache"]), cc_ref)


@gpu
def test_tokens_equal_successive_single_steps():
    """n tokens at once against n single decode steps on the GPU."""
    import linear_attention_sequence_causal_amd as gdn
    n = 6
    w = S.scaled(S.DECODE_B256, decode_batch=3, seed=82)
    setup, t = _case(w, n)
    st1, cc1 = setup["state"].clone(), setup["conv_cache"].clone()
    o = _gpu(setup, t, setup["state"], setup["conv_cache"])
    outs = []
    for i in range(n):
        outs.append(gdn.decode_step(t["q"][:, i].contiguous(), t["k"][:, i].contiguous(),
                                    t["v"][:, i].contiguous(), t["a"][:, i].contiguous(),
                                    t["b"][:, i].contiguous(), t["z"][:, i].contiguous(),
                                    setup["conv_w"], setup["A_log"], setup["dt_bias"],
                                    setup["norm_w"], st1, cc1))
    torch.cuda.synchronize()
    f = S.to_f64
    assert rel_l2(f(o), np.stack([f(x) for x in outs], 1)) < 1e-4
    assert rel_l2(f(setup["state"]), f(st1)) < 1e-6
    assert torch.equal(setup["conv_cache"], cc1)


@gpu
@pytest.mark.parametrize("commit", [None, "mixed"])
def test_tokens_full_batch_all_sequences(commit):
    """B=256, 16/32 heads, n=4 in the launch configuration the benchmark times, every
    sequence, head and token against the oracle; with all tokens committed and with
    per-sequence commit counts 0..4 (the cache channels of a q/k head are read and
    advanced by one workgroup only, so no sequence sees another's advance)."""
    n = 4
    w = S.DECODE_B256
    setup, t = _case(w, n)
    nc = None if commit is None else [i % (n + 1) for i in range(w.decode_batch)]
    _check(setup, t, n, num_commit=nc, label=f"decode_tokens B=256 n=4 commit={commit}")


@gpu
def test_tokens_extreme_gates():
    """alpha = 0 (A_log = 100: e^g underflows), alpha = 1 (A_log = -inf), beta in {0, 1}
    (b = -inf, +inf), and a decay of about e^-80 per token, whose product over the call
    underflows: the state carried divided by the running decay product (and rescaled
    when that product gets small) still matches the oracle."""
    import math
    n = 8
    w = S.scaled(S.DECODE_B256, decode_batch=4, num_qk_heads=2, num_v_heads=8, seed=83)
    setup, t = _case(w, n)
    setup["A_log"][0] = 100.0
    setup["A_log"][1] = -float("inf")
    setup["A_log"][2] = math.log(16.0)
    t["a"][:, :, 2] = 5.0
    t["b"][:, :, 3] = float("inf")
    t["b"][:, :, 4] = -float("inf")
    _check(setup, t, n, label="decode_tokens extreme gates")


@gpu
def test_tokens_q_scale_and_norm_weight():
    """q_scale = 1/sqrt(128) and a non-uniform RMSNorm weight (the workloads use 1 and
    ones)."""
    import math
    n = 4
    w = S.scaled(S.DECODE_B256, decode_batch=4, num_qk_heads=2, num_v_heads=8, seed=84)
    setup, t = _case(w, n)
    g = torch.Generator(device="cuda")
    g.manual_seed(85)
    setup["norm_w"] = torch.rand(128, generator=g, device="cuda") + 0.5
    qs = 1.0 / math.sqrt(128)
    st0, cc0 = setup["state"].clone(), setup["conv_cache"].clone()
    o = _gpu(setup, t, setup["state"], setup["conv_cache"], q_scale=qs)
    o_ref, st_ref, cc_ref = _oracle(setup, t, st0, cc0, q_scale=qs)
    f = S.to_f64
    eo, es = rel_l2(f(o), o_ref), rel_l2(f(setup["state"]), st_ref)
    print(f"decode_tokens q_scale 1/sqrt(128), random norm weight: o {eo:.3e} state {es:.3e}")
    assert eo < O_TOL and es < 1e-5
    assert np.array_equal(f(setup["conv_cache"]), cc_ref)


@gpu
def test_tokens_zero_batch_is_a_no_op():
    w = S.scaled(S.DECODE_B256, decode_batch=1, seed=83)
    setup, t = _case(w, 2)
    empty = {key: val[:0] for key, val in t.items()}
    o = _gpu(setup, empty, setup["state"][:0], setup["conv_cache"][:0])
    assert o.numel() == 0


@gpu
def test_tokens_sigmoid_output_gate_variant():
    import linear_attention_sequence_causal_amd as gdn
    n = 4
    w = S.scaled(S.DECODE_B256, decode_batch=4, num_qk_heads=2, num_v_heads=4, seed=86)
    setup, t = _case(w, n)
    st0, cc0 = setup["state"].clone(), setup["conv_cache"].clone()
    o = gdn.decode_tokens(t["q"], t["k"], t["v"], t["a"], t["b"], t["z"], setup["conv_w"],
                          setup["A_log"], setup["dt_bias"], setup["norm_w"], setup["state"],
                          setup["conv_cache"], output_gate="sigmoid")
    torch.cuda.synchronize()
    f = S.to_f64
    o_ref, st_ref, _ = oracle.decode_tokens(f(t["q"]), f(t["k"]), f(t["v"]), f(t["a"]),
                                            f(t["b"]), f(t["z"]), f(setup["conv_w"]),
                                            f(setup["A_log"]), f(setup["dt_bias"]),
                                            f(setup["norm_w"]), f(st0), f(cc0),
                                            output_gate="sigmoid")
    eo = rel_l2(f(o), o_ref)
    print(f"decode_tokens sigmoid output gate: o rel-L2 {eo:.3e}")
    assert eo < O_TOL and rel_l2(f(setup["state"]), st_ref) < 1e-5

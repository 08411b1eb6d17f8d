"""gdn_prefill_noalloc (the prefill for callers that cannot allocate) against
gdn_prefill, called through the C ABI on the same inputs: two calls in a row on the
library's static workspace, the second with a smaller problem (the array keeps the
first call's contents), each bitwise equal to gdn_prefill with a fresh workspace
(same kernels, same launch plan), and a problem larger than the static workspace
rejected before anything runs."""
import ctypes

import pytest
import torch

import gdn_synth as S

gpu = pytest.mark.gpu


def _abi_noalloc(gdn, d, o, fs, cso, q_scale=1.0):
    T, Hk, D = d["q"].shape
    Hv = d["v"].shape[1]
    N = d["cu_seqlens"].numel() - 1
    p = gdn.make_params(Hk, Hv, D, d["q"].dtype, d["conv_w"], d["A_log"], d["dt_bias"],
                        d["norm_w"], q_scale)
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = gdn.lib().gdn_prefill_noalloc(
        ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["a"]), ptr(d["b"]), ptr(d["z"]),
        ctypes.byref(p), ptr(d["init_state"]), ptr(d["cu_seqlens"]), N, T, ptr(d["conv_in"]),
        ptr(o), ptr(fs), ptr(cso), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@gpu
def test_noalloc_prefill_matches_prefill_twice():
    import linear_attention_sequence_causal_amd as gdn
    cases = [
        # first: one long sequence in several segments (maps, combine, start copies)
        S.scaled(S.PREFILL_4K, lengths=(3000, 700, 1), num_qk_heads=2, num_v_heads=4, seed=201,
                 init_state_std=0.01, conv_history=True),
        # second, smaller: fewer, shorter sequences on the same (dirty) array
        S.scaled(S.PREFILL_4K, lengths=(500, 33), num_qk_heads=2, num_v_heads=4, seed=202,
                 init_state_std=0.01, conv_history=True),
    ]
    for w in cases:
        d = S.prefill_inputs(w, "cuda")
        o_ref, fs_ref, cs_ref = gdn.prefill(
            d["q"], d["k"], d["v"], d["a"], d["b"], d["z"], d["conv_w"], d["A_log"],
            d["dt_bias"], d["norm_w"], init_state=d["init_state"], cu_seqlens=d["cu_seqlens"],
            conv_state=d["conv_in"], return_conv_state=True)
        o = torch.full_like(o_ref, 3.0)
        fs = torch.full_like(fs_ref, 3.0)
        cs = torch.full_like(cs_ref, 3.0)
        st = _abi_noalloc(gdn, d, o, fs, cs)
        torch.cuda.synchronize()
        assert st == 0, gdn.lib().gdn_last_error().decode()
        assert torch.equal(o, o_ref)
        assert torch.equal(fs, fs_ref)
        assert torch.equal(cs, cs_ref)


@gpu
def test_noalloc_prefill_rejects_problems_above_its_workspace():
    import linear_attention_sequence_causal_amd as gdn
    w = S.scaled(S.PREFILL_4K, lengths=(16,), num_qk_heads=1, num_v_heads=2, seed=203)
    d = S.prefill_inputs(w, "cuda")
    # the same tiny tensors, declared as 2^20 tokens in 64 sequences of 32 v heads: the
    # host rejects the call from its sizes alone, before any launch
    p = gdn.make_params(16, 32, 128, torch.bfloat16, d["conv_w"], d["A_log"], d["dt_bias"])
    need = gdn.lib().gdn_prefill_workspace_bytes(ctypes.byref(p), 64, 1 << 20)
    assert need > gdn.NOALLOC_WORKSPACE_BYTES
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    o = torch.full_like(d["v"], 3.0)
    st = gdn.lib().gdn_prefill_noalloc(
        ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["a"]), ptr(d["b"]), ptr(d["z"]),
        ctypes.byref(p), None, ptr(d["cu_seqlens"]), 64, 1 << 20, None, ptr(o), ptr(o), None,
        None)
    assert st == 3  # GDN_ERR_WORKSPACE
    assert "gdn_prefill_noalloc" in gdn.lib().gdn_last_error().decode()
    torch.cuda.synchronize()
    assert bool(torch.all(o == 3.0))

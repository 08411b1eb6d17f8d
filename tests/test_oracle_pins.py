"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the worked
two-token example (tests/golden), closed forms, invariants, special cases that
reduce to textbook formulas, and brute force on tiny inputs.  The passages:
field guide "Qwen3-Next 80B-A3B", cutaway 02 (six update steps, counts, RMSNorm
and SiLU(z) gate); Qwen3.8-Flash-Next model card (decay gate g, chunk state
update); tech report Fig. 2 caption (short causal convs, L2-normalised q/k,
decay and write gates).
"""
import json
import math
import os

import numpy as np
import torch
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "two_token_example.json")


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _l2(x, eps=1e-6):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


# --------------------------------------------------------------- scalars

def test_scalar_closed_forms():
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), abs=1e-15)
    assert oracle.softplus(math.log(math.e - 1.0)) == pytest.approx(1.0, abs=1e-15)
    assert oracle.softplus(40.0) == pytest.approx(40.0, rel=1e-15)
    assert oracle.softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-12)
    assert oracle.softplus(float("inf")) == float("inf")
    assert oracle.softplus(float("-inf")) == 0.0
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(math.log(3.0)) == pytest.approx(0.75, abs=1e-15)
    assert oracle.sigmoid(float("inf")) == 1.0
    assert oracle.sigmoid(float("-inf")) == 0.0
    assert oracle.silu(2.0) == pytest.approx(2.0 / (1.0 + math.exp(-2.0)), abs=1e-15)
    assert oracle.silu(0.0) == 0.0


def test_gate_closed_forms():
    # A_log = 0, a + dt_bias = 0  ->  g = -ln 2  ->  alpha = 1/2;  b = 0 -> beta = 1/2
    al, be = oracle.gates([0.0], [0.0], 0.0, 0.0)
    assert al[0] == pytest.approx(0.5, abs=1e-15) and be[0] == 0.5
    # A_log = ln 3, a + dt_bias = ln(e - 1)  ->  g = -3
    al, _ = oracle.gates([math.log(math.e - 1.0) - 0.25], [0.0], math.log(3.0), 0.25)
    assert al[0] == pytest.approx(math.exp(-3.0), rel=1e-14)
    # the bias enters inside softplus, not outside
    al1, _ = oracle.gates([1.0], [0.0], 0.0, -1.0)
    assert al1[0] == pytest.approx(0.5, abs=1e-15)
    # extremes: A_log = -inf -> alpha = 1; A_log = 100 -> alpha underflows to 0
    al, be = oracle.gates([0.3, -2.0], [float("inf"), float("-inf")], float("-inf"), 0.0)
    assert np.all(al == 1.0) and be[0] == 1.0 and be[1] == 0.0
    al, _ = oracle.gates([0.3, -2.0], [0.0, 0.0], 100.0, 0.0)
    assert np.all(al == 0.0) and not np.any(np.isnan(al))


# ------------------------------------------------------- worked example (P4)

def test_two_token_worked_example():
    ex = json.load(open(GOLDEN))
    y, S = oracle.recurrence(ex["alpha"], ex["beta"], ex["q"], ex["k"], ex["v"])
    np.testing.assert_allclose(y, ex["y"], atol=1e-15)
    np.testing.assert_allclose(S, ex["S2"], atol=1e-15)
    y1, S1 = oracle.recurrence(ex["alpha"][:1], ex["beta"][:1], ex["q"][:1], ex["k"][:1],
                               ex["v"][:1])
    np.testing.assert_allclose(S1, ex["S1"], atol=1e-15)
    # beta_2 = 1: the write makes S2 k2 = v2 exactly
    _, Sb = oracle.recurrence(ex["alpha"], [0.5, 1.0], ex["q"], ex["k"], ex["v"])
    np.testing.assert_allclose(Sb, ex["S2_beta2_one"], atol=1e-15)
    np.testing.assert_allclose(Sb @ np.array(ex["k"][1]), ex["v"][1], atol=1e-15)
    # epilogue of y2 (w = 1, eps = 0, z large so SiLU(z) = z; divide it out)
    z = np.full((1, 2), 60.0)
    o = oracle.epilogue(np.array([ex["y"][1]]), z, None, rms_eps=0.0)
    np.testing.assert_allclose(o[0] / 60.0, ex["y2_rmsnorm_eps0"], atol=1e-15)
    # the carried state is read with S0 q (beta = 0, alpha = 1)
    yc, Sc = oracle.recurrence([1.0, 1.0], [0.0, 0.0], ex["q"], ex["k"], ex["v"],
                               S0=ex["carry_S0"])
    np.testing.assert_allclose(yc, ex["carry_y"], atol=1e-15)
    assert np.array_equal(Sc, np.array(ex["carry_S0"]))


def test_two_token_example_through_the_mixer():
    """The worked example's gates and keys through the whole mixer; the stored
    state must be H = S^T.

    One-hot conv taps on the current token and raw q, k = 40 * (golden unit
    vectors) make the post-prologue q, k equal the golden ones to 1e-15
    (SiLU(40) = 40 (1 - 4e-18), SiLU(0) = 0, then L2 normalisation).  v passes
    through SiLU, so the expected state is rebuilt from SiLU(v) with the
    cutaway's six steps.
    """
    ex = json.load(open(GOLDEN))
    D, Hk, Hv = 2, 1, 1
    kk = np.array(ex["k"]) * 40.0
    qq = np.array(ex["q"]) * 40.0
    vv = np.array(ex["v"])
    conv_w = np.zeros((2 * Hk * D + Hv * D, 4))
    conv_w[:, 3] = 1.0
    z = np.full((2, Hv, D), 60.0)
    o, fs, _ = oracle.prefill(qq.reshape(2, Hk, D), kk.reshape(2, Hk, D), vv.reshape(2, Hv, D),
                              np.zeros((2, Hv)), np.zeros((2, Hv)), z, conv_w, [0.0], [0.0],
                              None, l2_eps=0.0, rms_eps=0.0)
    qpost = _silu(qq) / np.linalg.norm(_silu(qq), axis=1, keepdims=True)
    kpost = _silu(kk) / np.linalg.norm(_silu(kk), axis=1, keepdims=True)
    np.testing.assert_allclose(kpost, ex["k"], atol=1e-15)
    np.testing.assert_allclose(qpost, ex["q"], atol=1e-15)
    vpost = _silu(vv)
    S = np.zeros((2, 2))
    ys = []
    for t in range(2):  # alpha = beta = 1/2 from A_log = a = dt_bias = b = 0
        S = 0.5 * S
        e = vpost[t] - S @ kpost[t]
        S = S + 0.5 * np.outer(e, kpost[t])
        ys.append(S @ qpost[t])
    np.testing.assert_allclose(fs[0, 0], S.T, atol=1e-14)
    assert abs(fs[0, 0][0, 1] - fs[0, 0][1, 0]) > 1e-3  # not symmetric: orientation matters
    yt = np.array(ys)
    oref = yt / np.sqrt((yt ** 2).mean(1, keepdims=True)) * _silu(60.0)
    np.testing.assert_allclose(o[:, 0, :], oref, atol=1e-13)


# ------------------------------------------------------ recurrence invariants

def _rand_unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def test_p1_identity_gates_keep_state():
    rng = np.random.default_rng(1)
    D, T = 8, 13
    S0 = rng.standard_normal((D, D))
    q, k, v = rng.standard_normal((T, D)), _rand_unit(rng, T, D), rng.standard_normal((T, D))
    y, S = oracle.recurrence(np.ones(T), np.zeros(T), q, k, v, S0=S0)
    assert np.array_equal(S, S0)
    np.testing.assert_allclose(y, q @ S0.T, atol=1e-13)


def test_p2_full_write_reproduces_value():
    rng = np.random.default_rng(2)
    D, T = 16, 20
    k = _rand_unit(rng, T, D)
    v = rng.standard_normal((T, D))
    q = rng.standard_normal((T, D))
    S = rng.standard_normal((D, D))
    for t in range(T):
        _, S = oracle.recurrence([1.0], [1.0], q[t:t + 1], k[t:t + 1], v[t:t + 1], S0=S)
        np.testing.assert_allclose(S @ k[t], v[t], atol=1e-13)


def test_p3_state_size_fixed():
    rng = np.random.default_rng(3)
    D = 4
    for T in (1, 17, 512):
        _, S = oracle.recurrence(rng.uniform(0.5, 1, T), rng.uniform(0, 1, T),
                                 rng.standard_normal((T, D)), _rand_unit(rng, T, D),
                                 rng.standard_normal((T, D)))
        assert S.shape == (D, D)


def test_p5_orthogonal_keys_is_decayed_linear_attention():
    """With orthonormal keys the read-back is zero, so the recurrence reduces to
    decay-masked causal linear attention: y = ((Q K^T) * Dmask) diag(beta) V."""
    rng = np.random.default_rng(5)
    D = T = 12
    K = np.linalg.qr(rng.standard_normal((D, D)))[0].T  # rows orthonormal
    Q = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    alpha = rng.uniform(0.3, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    y, _ = oracle.recurrence(alpha, beta, Q, K, V)
    Dm = np.zeros((T, T))
    for t in range(T):
        for s in range(t + 1):
            Dm[t, s] = np.prod(alpha[s + 1:t + 1])  # decay applied after the write at s
    yref = ((Q @ K.T) * Dm) @ (beta[:, None] * V)
    np.testing.assert_allclose(y, yref, atol=1e-13)


def test_p6_projection_property():
    rng = np.random.default_rng(6)
    D, T = 10, 15
    k = _rand_unit(rng, T, D)
    q, v = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    S = rng.standard_normal((D, D))
    for t in range(T):
        P = np.eye(D) - np.outer(k[t], k[t])
        _, Sn = oracle.recurrence([1.0], [1.0], q[t:t + 1], k[t:t + 1], v[t:t + 1], S0=S)
        np.testing.assert_allclose(Sn @ P, S @ P, atol=1e-13)
        S = Sn


def test_p12_forgetting_limit():
    rng = np.random.default_rng(12)
    D, T = 8, 9
    q, k, v = rng.standard_normal((T, D)), _rand_unit(rng, T, D), rng.standard_normal((T, D))
    beta = rng.uniform(0, 1, T)
    al, _ = oracle.gates(rng.standard_normal(T), np.zeros(T), 100.0, 0.0)
    assert np.all(al == 0.0)
    y, S = oracle.recurrence(al, beta, q, k, v, S0=rng.standard_normal((D, D)))
    np.testing.assert_allclose(S, beta[-1] * np.outer(v[-1], k[-1]), atol=1e-15)
    np.testing.assert_allclose(y, (beta * (k * q).sum(1))[:, None] * v, atol=1e-14)
    assert not np.any(np.isnan(y))


def test_decay_precedes_read_and_write():
    """Order of the cutaway: decay, then read S'k, then write.  A single token
    with S0 = I, k = e0, v = 0: S1 = alpha I - beta alpha e0 e0^T."""
    D = 3
    alpha, beta = 0.25, 0.5
    k = np.array([[1.0, 0, 0]])
    y, S = oracle.recurrence([alpha], [beta], np.array([[0, 1.0, 0]]), k, np.zeros((1, D)),
                             S0=np.eye(D))
    ref = alpha * np.eye(D) - beta * alpha * np.outer(k[0], k[0])
    np.testing.assert_allclose(S, ref, atol=1e-16)
    np.testing.assert_allclose(y[0], ref @ np.array([0, 1.0, 0]), atol=1e-16)


def test_p11_scale_invariance_in_v():
    rng = np.random.default_rng(11)
    D, T = 8, 10
    q, k, v = rng.standard_normal((T, D)), _rand_unit(rng, T, D), rng.standard_normal((T, D))
    al, be = rng.uniform(0.2, 1, T), rng.uniform(0, 1, T)
    y1, _ = oracle.recurrence(al, be, q, k, v)
    y3, _ = oracle.recurrence(al, be, q, k, 3.0 * v)
    np.testing.assert_allclose(y3, 3.0 * y1, rtol=1e-12, atol=1e-14)
    z = rng.standard_normal((T, D))
    np.testing.assert_allclose(oracle.epilogue(y3, z, rms_eps=0.0),
                               oracle.epilogue(y1, z, rms_eps=0.0), rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------ prologue pins

def _mixer_inputs(rng, T, Hk, Hv, D, scale=1.0):
    q = rng.standard_normal((T, Hk, D)) * scale
    k = rng.standard_normal((T, Hk, D)) * scale
    v = rng.standard_normal((T, Hv, D)) * scale
    return q, k, v


def test_p10_conv_taps_and_channel_sections():
    rng = np.random.default_rng(10)
    T, Hk, Hv, D = 9, 2, 4, 8
    Cc = 2 * Hk * D + Hv * D
    q, k, v = _mixer_inputs(rng, T, Hk, Hv, D)
    hist = rng.standard_normal((3, Cc))
    w = np.zeros((Cc, 4))
    w[: Hk * D, 3] = 1.0            # q: current token
    w[Hk * D: 2 * Hk * D, 2] = 1.0  # k: one step back
    w[2 * Hk * D:, 0] = 1.0         # v: three steps back
    for h in range(Hv):
        g = h // (Hv // Hk)
        qo, ko, vo = oracle.prologue(q, k, v, w, h, hist=hist, l2_eps=1e-6)
        np.testing.assert_allclose(qo, _l2(_silu(q[:, g])), atol=1e-15)
        kprev = np.concatenate([hist[2:3, Hk * D + g * D: Hk * D + (g + 1) * D], k[:-1, g]])
        np.testing.assert_allclose(ko, _l2(_silu(kprev)), atol=1e-15)
        c0 = 2 * Hk * D + h * D
        vprev = np.concatenate([hist[:, c0:c0 + D], v[:-3, h]])
        np.testing.assert_allclose(vo, _silu(vprev), atol=1e-15)
    # zero history by default: v three steps back is SiLU(0) = 0 for t < 3
    _, _, vo = oracle.prologue(q, k, v, w, 1)
    assert np.all(vo[:3] == 0.0)


def test_conv_is_a_weighted_sum_of_four_taps():
    rng = np.random.default_rng(13)
    T, Hk, Hv, D = 7, 1, 2, 4
    Cc = 2 * Hk * D + Hv * D
    q, k, v = _mixer_inputs(rng, T, Hk, Hv, D)
    w = rng.standard_normal((Cc, 4))
    _, _, vo = oracle.prologue(q, k, v, w, 1, l2_eps=0.0)
    c0 = 2 * Hk * D + 1 * D
    xpad = np.concatenate([np.zeros((3, D)), v[:, 1]])
    pre = sum(w[c0:c0 + D, j][None, :] * xpad[j:j + T] for j in range(4))
    np.testing.assert_allclose(vo, _silu(pre), atol=1e-14)


def test_l2_normalisation_and_query_scale():
    rng = np.random.default_rng(14)
    T, Hk, Hv, D = 5, 1, 1, 16
    q, k, v = _mixer_inputs(rng, T, Hk, Hv, D, scale=3.0)
    w = np.zeros((2 * D + D, 4))
    w[:, 3] = 1.0
    qo, ko, _ = oracle.prologue(q, k, v, w, 0, q_scale=0.5, l2_eps=0.0)
    np.testing.assert_allclose(np.linalg.norm(ko, axis=1), 1.0, atol=1e-15)
    np.testing.assert_allclose(np.linalg.norm(qo, axis=1), 0.5, atol=1e-15)
    # eps keeps an all-zero vector at zero instead of NaN
    qz = np.zeros_like(q)
    w0 = np.zeros_like(w)
    qo, ko, _ = oracle.prologue(qz, qz, v, w0, 0, l2_eps=1e-6)
    assert np.all(qo == 0.0) and np.all(ko == 0.0)


# ------------------------------------------------------------ epilogue pins

def test_epilogue_closed_forms():
    D = 8
    c = -0.3
    y = np.full((1, D), c)
    wn = np.linspace(0.5, 2.0, D)
    z = np.full((1, D), 2.0)
    o = oracle.epilogue(y, z, wn, rms_eps=1e-6)
    np.testing.assert_allclose(o[0], c / math.sqrt(c * c + 1e-6) * wn * _silu(2.0), atol=1e-15)
    o0 = oracle.epilogue(np.random.default_rng(0).standard_normal((3, D)), np.zeros((3, D)))
    assert np.all(o0 == 0.0)


# --------------------------------------------------------------- mixer pins

def _mixer_case(rng, lengths, Hk=2, Hv=4, D=16, init=True, hist=True):
    T = int(sum(lengths))
    N = len(lengths)
    Cc = 2 * Hk * D + Hv * D
    q, k, v = _mixer_inputs(rng, T, Hk, Hv, D)
    return dict(
        q=q, k=k, v=v, a=rng.standard_normal((T, Hv)), b=rng.standard_normal((T, Hv)),
        z=rng.standard_normal((T, Hv, D)), conv_w=rng.standard_normal((Cc, 4)) * 0.5,
        A_log=rng.uniform(0, math.log(16), Hv), dt_bias=rng.uniform(-1, 1, Hv),
        norm_w=rng.uniform(0.5, 1.5, D),
        cu=np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64),
        init=rng.standard_normal((N, Hv, D, D)) * 0.1 if init else None,
        hist=rng.standard_normal((N, 3, Cc)) if hist else None)


def _run(c, sl=None, cu=None, init="keep", hist="keep"):
    sl = slice(None) if sl is None else sl
    return oracle.prefill(c["q"][sl], c["k"][sl], c["v"][sl], c["a"][sl], c["b"][sl],
                          c["z"][sl], c["conv_w"], c["A_log"], c["dt_bias"], c["norm_w"],
                          cu_seqlens=c["cu"] if cu is None else cu,
                          init_state=c["init"] if isinstance(init, str) else init,
                          conv_in=c["hist"] if isinstance(hist, str) else hist)


def test_p1_mixer_level_state_unchanged():
    rng = np.random.default_rng(21)
    c = _mixer_case(rng, [11])
    c["b"][:] = -np.inf
    c["A_log"][:] = -np.inf
    o, fs, _ = _run(c)
    assert np.array_equal(fs, c["init"])
    # y = S0 q = H0^T q  with q from the prologue
    for h in range(4):
        qo, _, _ = oracle.prologue(c["q"], c["k"], c["v"], c["conv_w"], h, hist=c["hist"][0])
        y = qo @ c["init"][0, h]
        yn = y / np.sqrt((y * y).mean(1, keepdims=True) + 1e-6)
        np.testing.assert_allclose(o[:, h], yn * c["norm_w"] * _silu(c["z"][:, h]), atol=1e-13)


def test_p2_mixer_level_full_write():
    rng = np.random.default_rng(22)
    c = _mixer_case(rng, [6])
    c["b"][:] = np.inf
    c["A_log"][:] = -np.inf
    _, fs, _ = _run(c)
    for h in range(4):
        _, ko, vo = oracle.prologue(c["q"], c["k"], c["v"], c["conv_w"], h, hist=c["hist"][0])
        S = fs[0, h].T
        np.testing.assert_allclose(S @ ko[-1], vo[-1], atol=1e-5 * np.abs(vo[-1]).max())


def test_gqa_head_mapping():
    """v heads 2g and 2g+1 read q/k head g: make q.k positive on q/k head 0 and
    negative on head 1; in the forgetting limit o flips sign exactly there."""
    T, Hk, Hv, D = 3, 2, 4, 4
    Cc = 2 * Hk * D + Hv * D
    q = np.zeros((T, Hk, D))
    k = np.zeros((T, Hk, D))
    k[:, :, 0] = 30.0
    q[:, 0, 0] = 30.0
    q[:, 1, 0], q[:, 1, 1] = -30.0, 30.0  # SiLU -> (-~0, 30): q.k slightly negative
    rng = np.random.default_rng(23)
    v = np.abs(rng.standard_normal((T, Hv, D))) + 5.0
    w = np.zeros((Cc, 4))
    w[:, 3] = 1.0
    z = np.full((T, Hv, D), 40.0)
    o, _, _ = oracle.prefill(q, k, v, np.zeros((T, Hv)), np.zeros((T, Hv)), z, w,
                             np.full(Hv, 100.0), np.zeros(Hv), None)
    assert np.all(o[:, 0:2] > 0) and np.all(o[:, 2:4] < 0)


def test_p7_split_sequence_bitwise():
    rng = np.random.default_rng(7)
    T = 23
    c = _mixer_case(rng, [T])
    o_full, fs_full, co_full = _run(c)
    for t0 in (1, 2, 3, 10, 22):
        oa, fa, ca = _run(c, sl=slice(0, t0), cu=[0, t0])
        ob, fb, cb = _run(c, sl=slice(t0, T), cu=[0, T - t0], init=fa, hist=ca)
        assert np.array_equal(np.concatenate([oa, ob]), o_full)
        assert np.array_equal(fb, fs_full)
        assert np.array_equal(cb, co_full)


def test_p8_decode_after_prefill_bitwise():
    rng = np.random.default_rng(8)
    T, n = 9, 4
    c = _mixer_case(rng, [T + n])
    o_full, fs_full, co_full = _run(c)
    o_pre, st, cache = _run(c, sl=slice(0, T), cu=[0, T])
    for i in range(n):
        t = T + i
        sl = slice(t, t + 1)
        o_t, st, cache = oracle.decode_step(c["q"][sl], c["k"][sl], c["v"][sl], c["a"][sl],
                                            c["b"][sl], c["z"][sl], c["conv_w"], c["A_log"],
                                            c["dt_bias"], c["norm_w"], st, cache)
        assert np.array_equal(o_t, o_full[sl])
    assert np.array_equal(st, fs_full)
    assert np.array_equal(cache, co_full)


def test_varlen_packing_equals_separate_runs():
    rng = np.random.default_rng(30)
    lengths = [5, 0, 1, 2, 17, 3]
    c = _mixer_case(rng, lengths)
    o, fs, co = _run(c)
    cu = c["cu"]
    for n, L in enumerate(lengths):
        sl = slice(cu[n], cu[n + 1])
        on, fn, cn = _run(c, sl=sl, cu=[0, L], init=c["init"][n:n + 1], hist=c["hist"][n:n + 1])
        assert np.array_equal(on, o[sl])
        assert np.array_equal(fn[0], fs[n])
        assert np.array_equal(cn[0], co[n])
    # an empty sequence returns its initial state and its history unchanged
    assert np.array_equal(fs[1], c["init"][1])
    assert np.array_equal(co[1], c["hist"][1])


def test_conv_out_holds_last_three_raw_rows():
    rng = np.random.default_rng(31)
    Hk, Hv, D = 1, 2, 4
    c = _mixer_case(rng, [5, 2], Hk=Hk, Hv=Hv, D=D)
    _, _, co = _run(c)
    raw = np.concatenate([c["q"].reshape(-1, Hk * D), c["k"].reshape(-1, Hk * D),
                          c["v"].reshape(-1, Hv * D)], axis=1)
    assert np.array_equal(co[0], raw[2:5])
    # length 2: one row of inherited history, then the two tokens
    assert np.array_equal(co[1], np.concatenate([c["hist"][1][2:3], raw[5:7]]))


def test_no_nan_at_extreme_gates():
    rng = np.random.default_rng(32)
    c = _mixer_case(rng, [12])
    c["a"][::2] = 30.0
    c["b"][1::3] = np.inf
    c["b"][2::3] = -np.inf
    c["A_log"][0] = 100.0
    c["A_log"][1] = -np.inf
    o, fs, _ = _run(c)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(fs))


# ----------------------------------------------- multi-token step (decode n tokens)

def _token_batch(rng, B, n, Hk=2, Hv=4, D=16):
    """B sequences with a cached state and conv cache, n new tokens each ([B, n, ...])."""
    c = _mixer_case(rng, [n] * B, Hk, Hv, D)
    sh = lambda x: x.reshape((B, n) + x.shape[1:])
    return dict(q=sh(c["q"]), k=sh(c["k"]), v=sh(c["v"]), a=sh(c["a"]), b=sh(c["b"]),
                z=sh(c["z"]), conv_w=c["conv_w"], A_log=c["A_log"], dt_bias=c["dt_bias"],
                norm_w=c["norm_w"], state=c["init"], cache=c["hist"])


def _tokens(t, num_commit=None):
    return oracle.decode_tokens(t["q"], t["k"], t["v"], t["a"], t["b"], t["z"], t["conv_w"],
                                t["A_log"], t["dt_bias"], t["norm_w"], t["state"], t["cache"],
                                num_commit=num_commit)


def _steps(t, count):
    """`count` single decode steps of every sequence: outputs per step, state, cache."""
    st, cache, outs = t["state"], t["cache"], []
    for i in range(count):
        o_i, st, cache = oracle.decode_step(
            t["q"][:, i], t["k"][:, i], t["v"][:, i], t["a"][:, i], t["b"][:, i], t["z"][:, i],
            t["conv_w"], t["A_log"], t["dt_bias"], t["norm_w"], st, cache)
        outs.append(o_i)
    return outs, st, cache


def test_decode_tokens_equals_successive_single_steps():
    """n tokens at once = n single steps in order (outputs, state and cache), bitwise."""
    rng = np.random.default_rng(41)
    for n in (1, 2, 5):
        t = _token_batch(rng, 3, n)
        o, st, cache = _tokens(t)
        outs, st1, cache1 = _steps(t, n)
        for i in range(n):
            assert np.array_equal(o[:, i], outs[i])
        assert np.array_equal(st, st1)
        assert np.array_equal(cache, cache1)


def test_decode_tokens_commit_prefix():
    """num_commit[b] = c: outputs of all n tokens, state and cache after the first c
    (c = 0 leaves both bit for bit; out-of-range counts clamp to 0..n)."""
    rng = np.random.default_rng(42)
    n = 5
    t = _token_batch(rng, 5, n)
    commit = [0, 2, 5, 3, 9]
    o, st, cache = _tokens(t, commit)
    o_all, _, _ = _tokens(t)
    assert np.array_equal(o, o_all)
    for bb, c in enumerate(commit):
        c = min(max(c, 0), n)
        one = {key: (val[bb:bb + 1] if key in ("q", "k", "v", "a", "b", "z", "state", "cache")
                     else val) for key, val in t.items()}
        _, st1, cache1 = _steps(one, c)
        assert np.array_equal(st[bb], st1[0])
        assert np.array_equal(cache[bb], cache1[0])
    assert np.array_equal(st[0], t["state"][0]) and np.array_equal(cache[0], t["cache"][0])


def test_decode_tokens_after_prefill_is_the_longer_prefill():
    """prefill(T) then n tokens on its state and cache = prefill(T + n), bitwise."""
    rng = np.random.default_rng(43)
    T, n = 11, 4
    c = _mixer_case(rng, [T + n])
    o_full, fs_full, co_full = _run(c)
    _, st, cache = _run(c, sl=slice(0, T), cu=[0, T])
    sl = slice(T, T + n)
    o, st2, cache2 = oracle.decode_tokens(
        c["q"][None, sl], c["k"][None, sl], c["v"][None, sl], c["a"][None, sl],
        c["b"][None, sl], c["z"][None, sl], c["conv_w"], c["A_log"], c["dt_bias"],
        c["norm_w"], st, cache)
    assert np.array_equal(o[0], o_full[sl])
    assert np.array_equal(st2, fs_full)
    assert np.array_equal(cache2, co_full)


# ------------------------------------------------ bf16 storage of the decode state

def test_round_bf16_hand_values_and_ties():
    one = 1.0
    assert oracle.round_bf16(one + 2.0 ** -8) == 1.0                  # tie -> even (1.0)
    assert oracle.round_bf16(one + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie -> even mantissa
    assert oracle.round_bf16(one + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(-3.0) == -3.0 and oracle.round_bf16(0.0) == 0.0
    assert oracle.round_bf16(0.1) == 0.10009765625                   # 0x3DCD
    assert np.isinf(oracle.round_bf16(np.inf))


def test_round_bf16_matches_the_fp32_to_bf16_conversion():
    """For fp32 inputs (a single rounding either way) it is torch's RNE cast."""
    import torch
    rng = np.random.default_rng(44)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_bf16_state_step_keeps_a_frozen_state_bit_for_bit():
    """beta = 0, alpha = 1: the stored (bf16-valued) state comes back unchanged."""
    rng = np.random.default_rng(45)
    t = _token_batch(rng, 2, 1)
    st0 = oracle.round_bf16(t["state"])
    _, st, _ = oracle.decode_step_bf16_state(
        t["q"][:, 0], t["k"][:, 0], t["v"][:, 0], t["a"][:, 0], np.full_like(t["b"][:, 0], -np.inf),
        t["z"][:, 0], t["conv_w"], np.full_like(t["A_log"], -np.inf), t["dt_bias"], t["norm_w"],
        st0, t["cache"])
    assert np.array_equal(st, st0)


def test_bf16_state_step_is_the_exact_step_rounded():
    """Same outputs and cache as the fp32-storage step; the state is its rounding, so
    it lies within half a bf16 unit (2^-9 relative) of the exact one."""
    rng = np.random.default_rng(46)
    t = _token_batch(rng, 3, 1)
    st0 = oracle.round_bf16(t["state"])
    args = (t["q"][:, 0], t["k"][:, 0], t["v"][:, 0], t["a"][:, 0], t["b"][:, 0], t["z"][:, 0],
            t["conv_w"], t["A_log"], t["dt_bias"], t["norm_w"], st0, t["cache"])
    o1, s1, c1 = oracle.decode_step(*args)
    o2, s2, c2 = oracle.decode_step_bf16_state(*args)
    assert np.array_equal(o1, o2) and np.array_equal(c1, c2)
    nz = s1 != 0
    assert np.all(np.abs(s2[nz] - s1[nz]) <= np.abs(s1[nz]) * 2.0 ** -8)
    assert not np.array_equal(s1, s2)  # the rounding is real


# ------------------------------------------------- fp8 (E4M3) state storage


def test_round_fp8_hand_values_and_ties():
    r = oracle.round_fp8_e4m3
    assert r(448.0) == 448.0 and r(-448.0) == -448.0          # largest finite value
    assert r(1.0 + 2.0 ** -4) == 1.0                            # tie -> even mantissa 000
    assert r(1.0 + 3 * 2.0 ** -4) == 1.25                       # tie -> even mantissa 010
    assert r(1.0 + 2.0 ** -4 + 2.0 ** -20) == 1.125
    assert r(0.1) == 0.1015625                                  # 1.625 * 2^-4
    assert r(2.0 ** -6) == 2.0 ** -6                            # smallest normal
    assert r(3 * 2.0 ** -10) == 2.0 ** -8                       # subnormal tie -> even (2/512)
    assert r(2.0 ** -10) == 0.0                                 # half the smallest subnormal
    assert r(0.0) == 0.0


def test_round_fp8_matches_torchs_e4m3fn_cast():
    """An independent implementation of the same format: torch's float8_e4m3fn."""
    g = torch.Generator().manual_seed(5)
    x = torch.randn(200000, generator=g, dtype=torch.float64) * torch.exp(
        torch.randn(200000, generator=g, dtype=torch.float64) * 3.0)
    x = x.clamp(-448.0, 448.0).to(torch.float32)
    ref = x.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_fp8_e4m3(x.to(torch.float64).numpy()), ref)
    # every code decodes to a value the rounding maps to itself
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    vals = codes[torch.isfinite(codes)].numpy()
    assert np.array_equal(oracle.round_fp8_e4m3(vals), vals)


def test_fp8_row_scales_are_the_smallest_power_of_two_that_fits():
    x = np.array([[448.0, -1.0], [448.5, 0.0], [0.0, 0.0], [-3.5, 1.0], [1e-30, 0.0]])
    s = oracle.fp8_row_scales(x)
    assert list(s[:4]) == [1.0, 2.0, 1.0, 2.0 ** -7]
    for row, sc in zip(x, s):
        m = np.max(np.abs(row))
        if m > 0:
            assert m <= 448.0 * sc and m > 448.0 * sc / 2
    q, sc = oracle.quantize_fp8_rows(x)
    assert np.all(np.abs(q) <= 448.0)
    assert np.allclose(q * sc[:, None], x, rtol=2.0 ** -4, atol=0.0)


def test_fp8_state_step_keeps_a_frozen_state_bit_for_bit():
    """beta = 0, alpha = 1: the state is unchanged, so re-quantising a stored state gives
    back the same values (a row whose largest stored code rounded down to 224 moves to
    half the scale and doubled codes, the same values)."""
    rng = np.random.default_rng(3)
    B, Hk, Hv, D = 2, 1, 2, 128
    Cc = 2 * Hk * D + Hv * D
    st = rng.normal(0, 0.01, (B, Hv, D, D))
    sq, ss = oracle.quantize_fp8_rows(st)
    q = rng.normal(size=(B, Hk, D)); k = rng.normal(size=(B, Hk, D))
    v = rng.normal(size=(B, Hv, D)); z = rng.normal(size=(B, Hv, D))
    a = rng.normal(size=(B, Hv)); b = np.full((B, Hv), -np.inf)
    cw = rng.normal(0, 0.5, (Cc, 4)); cache = rng.normal(size=(B, 3, Cc))
    _, q2, s2, _ = oracle.decode_step_fp8_state(q, k, v, a, b, z, cw, np.full(Hv, -np.inf),
                                                np.zeros(Hv), np.ones(D), sq, ss, cache)
    assert np.array_equal(q2 * s2[..., None], sq * ss[..., None])
    assert np.all(np.abs(q2) <= 448.0)


# ------------------------------------------------- sigmoid output-gate variant


def test_sigmoid_gate_epilogue_closed_forms():
    """o = RMSNorm(y) * w * sigmoid(z): z = 0 halves the normalised y; a constant y
    normalises to its sign; and since SiLU(z) = z sigmoid(z), the SiLU-gated output
    is the sigmoid-gated one times z."""
    rng = np.random.default_rng(8)
    y = rng.normal(size=(5, 16))
    nw = rng.uniform(0.5, 1.5, 16)
    o0 = oracle.epilogue(y, np.zeros_like(y), nw, rms_eps=0.0, output_gate="sigmoid")
    rms = np.sqrt(np.mean(y * y, axis=1, keepdims=True))
    assert np.allclose(o0, 0.5 * y / rms * nw, rtol=1e-14, atol=0)
    c = np.full((1, 16), -2.5)
    zc = np.linspace(-3, 3, 16)[None]
    oc = oracle.epilogue(c, zc, None, rms_eps=0.0, output_gate="sigmoid")
    assert np.allclose(oc, -1.0 / (1.0 + np.exp(-zc)), rtol=1e-14, atol=0)
    z = rng.normal(size=y.shape) * 3
    o_sig = oracle.epilogue(y, z, nw, output_gate="sigmoid")
    o_silu = oracle.epilogue(y, z, nw)
    assert np.allclose(o_silu, o_sig * z, rtol=1e-13, atol=1e-15)


def test_sigmoid_gate_reaches_the_mixer_outputs_only():
    """Through the whole mixer the gate changes o exactly as in the epilogue (o_silu =
    o_sigmoid * z) and leaves the final state and conv state alone; decode agrees."""
    rng = np.random.default_rng(9)
    T, Hk, Hv, D = 40, 1, 2, 128
    Cc = 2 * Hk * D + Hv * D
    q = rng.normal(size=(T, Hk, D)); k = rng.normal(size=(T, Hk, D))
    v = rng.normal(size=(T, Hv, D)); z = rng.normal(size=(T, Hv, D))
    a = rng.normal(size=(T, Hv)); b = rng.normal(size=(T, Hv))
    cw = rng.normal(0, 0.5, (Cc, 4)); A_log = rng.uniform(0, np.log(16), Hv)
    dt = rng.uniform(-1, 1, Hv)
    o1, f1, c1 = oracle.prefill(q, k, v, a, b, z, cw, A_log, dt)
    o2, f2, c2 = oracle.prefill(q, k, v, a, b, z, cw, A_log, dt, output_gate="sigmoid")
    assert np.array_equal(f1, f2) and np.array_equal(c1, c2)
    assert np.allclose(o1, o2 * z, rtol=1e-12, atol=1e-15)
    st = rng.normal(0, 0.01, (1, Hv, D, D)); cache = rng.normal(size=(1, 3, Cc))
    od, _, _ = oracle.decode_step(q[:1], k[:1], v[:1], a[:1], b[:1], z[:1], cw, A_log, dt,
                                  None, st, cache, output_gate="sigmoid")
    od1, _, _ = oracle.decode_step(q[:1], k[:1], v[:1], a[:1], b[:1], z[:1], cw, A_log, dt,
                                   None, st, cache)
    assert np.allclose(od1, od * z[:1], rtol=1e-12, atol=1e-15)


# ------------------------------------------------- projections around the mixer


def test_linear_is_the_matrix_product_by_brute_force():
    rng = np.random.default_rng(11)
    x = rng.normal(size=(5, 7))
    w = rng.normal(size=(3, 7))
    y = oracle.linear(x, w)
    for m in range(5):
        for n in range(3):
            acc = 0.0
            for kk in range(7):
                acc += x[m, kk] * w[n, kk]
            assert abs(y[m, n] - acc) <= 1e-13 * (1 + abs(acc))


def test_one_hot_projections_reduce_the_layer_to_the_mixer():
    """w_in with one-hot rows picks hidden features as q, k, v, z, a, b, and w_out = I
    returns o: the layer equals the mixer on the picked features, bit for bit."""
    rng = np.random.default_rng(12)
    T, Hk, Hv, D = 37, 1, 2, 128
    n_in = 2 * Hk * D + 2 * Hv * D + 2 * Hv
    d_model = n_in + 5
    x = rng.normal(size=(T, d_model))
    perm = rng.permutation(d_model)[:n_in]
    w_in = np.zeros((n_in, d_model))
    w_in[np.arange(n_in), perm] = 1.0
    w_out = np.eye(Hv * D)
    Cc = 2 * Hk * D + Hv * D
    cw = rng.normal(0, 0.5, (Cc, 4))
    A_log = rng.uniform(0, np.log(16), Hv)
    dt = rng.uniform(-1, 1, Hv)
    y, fs, co = oracle.gdn_layer(x, w_in, w_out, cw, A_log, dt, None, Hk, Hv, D)
    sel = x[:, perm]
    c = np.cumsum([0, Hk * D, Hk * D, Hv * D, Hv * D, Hv, Hv])
    q, k = sel[:, c[0]:c[1]].reshape(T, Hk, D), sel[:, c[1]:c[2]].reshape(T, Hk, D)
    v, z = sel[:, c[2]:c[3]].reshape(T, Hv, D), sel[:, c[3]:c[4]].reshape(T, Hv, D)
    a, b = sel[:, c[4]:c[5]], sel[:, c[5]:c[6]]
    o, fs2, co2 = oracle.prefill(q, k, v, a, b, z, cw, A_log, dt, None)
    assert np.array_equal(y, o.reshape(T, Hv * D))
    assert np.array_equal(fs, fs2) and np.array_equal(co, co2)


# ------------------------------------------------- gated full attention


def _attn_case(T, Hq=4, Hkv=2, D=16, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(T, Hq, D)), rng.normal(size=(T, Hkv, D)),
            rng.normal(size=(T, Hkv, D)), rng.normal(size=(T, Hq, D)),
            rng.uniform(0.5, 1.5, D), rng.uniform(0.5, 1.5, D))


def test_attention_first_token_returns_its_gated_value():
    """Softmax over a single (causal) key is 1: o_0 = v_0 * sigmoid(gate_0)."""
    q, k, v, g, wq, wk = _attn_case(5)
    o = oracle.gated_attention(q, k, v, g, wq, wk, rotary_dim=8)
    for h in range(4):
        assert np.allclose(o[0, h], v[0, h // 2] / (1 + np.exp(-g[0, h])), rtol=1e-14)


def test_attention_equal_keys_average_the_values():
    """All keys equal (same raw k at every position and no rotation): every causal
    score of a query is the same, so o_t = mean(v_0..t) * sigmoid(gate_t)."""
    q, k, v, g, wq, wk = _attn_case(9, seed=1)
    k[:] = k[0]
    o = oracle.gated_attention(q, k, v, g, wq, wk, rotary_dim=0)
    for t in range(9):
        for h in range(4):
            ref = v[:t + 1, h // 2].mean(axis=0) / (1 + np.exp(-g[t, h]))
            assert np.allclose(o[t, h], ref, rtol=1e-13, atol=1e-15)


def test_attention_grouped_query_mapping():
    """Negating the values of kv head 1 negates exactly the outputs of q heads 2, 3
    (Hq = 4, Hkv = 2: q head h reads kv head h // 2)."""
    q, k, v, g, wq, wk = _attn_case(7, seed=2)
    o1 = oracle.gated_attention(q, k, v, g, wq, wk, rotary_dim=8)
    v2 = v.copy()
    v2[:, 1] *= -1
    o2 = oracle.gated_attention(q, k, v2, g, wq, wk, rotary_dim=8)
    assert np.array_equal(o2[:, :2], o1[:, :2]) and np.allclose(o2[:, 2:], -o1[:, 2:], rtol=0)


def test_partial_rope_rotates_pairs_and_keeps_the_rest():
    """Dims i and i + r/2 (i < r/2) rotate by pos * theta^(-2i/r); dims >= r are
    untouched; a rotation keeps each pair's norm and q.k depends on the position
    difference only."""
    rng = np.random.default_rng(3)
    x = rng.normal(size=(3, 1, 16))
    pos = np.array([0.0, 1.0, 5.0])
    y = oracle.partial_rope(x, pos, 8, 100.0)
    assert np.array_equal(y[0], x[0])                  # position 0: no rotation
    assert np.array_equal(y[:, :, 8:], x[:, :, 8:])
    i, p = 2, 5.0
    a = p * 100.0 ** (-2 * i / 8)
    x1, x2 = x[2, 0, i], x[2, 0, i + 4]
    assert np.isclose(y[2, 0, i], x1 * np.cos(a) - x2 * np.sin(a), rtol=1e-14)
    assert np.isclose(y[2, 0, i + 4], x2 * np.cos(a) + x1 * np.sin(a), rtol=1e-14)
    qv, kv = rng.normal(size=(1, 1, 16)), rng.normal(size=(1, 1, 16))
    d1 = np.sum(oracle.partial_rope(qv, [7.0], 8, 100.0) * oracle.partial_rope(kv, [3.0], 8, 100.0))
    d2 = np.sum(oracle.partial_rope(qv, [14.0], 8, 100.0) * oracle.partial_rope(kv, [10.0], 8, 100.0))
    assert np.isclose(d1, d2, rtol=1e-12)


def test_qk_norm_is_rms_normalisation_with_weight():
    x = np.array([[[3.0, 4.0]]])
    y = oracle.attn_rms_norm(x, np.array([2.0, 1.0]), 0.0)
    r = np.sqrt((9 + 16) / 2)
    assert np.allclose(y, [[[6.0 / r, 4.0 / r]]], rtol=1e-15)


def test_attention_sequences_do_not_see_each_other():
    """Packed sequences equal separate runs (positions restart at each sequence)."""
    q, k, v, g, wq, wk = _attn_case(12, seed=4)
    cu = [0, 5, 5, 12]
    o = oracle.gated_attention(q, k, v, g, wq, wk, cu, rotary_dim=8)
    for b, e in ((0, 5), (5, 12)):
        oe = oracle.gated_attention(q[b:e], k[b:e], v[b:e], g[b:e], wq, wk, rotary_dim=8)
        assert np.array_equal(o[b:e], oe)


def test_attention_without_rotation_and_gate_is_causal_sdpa():
    """With unit-RMS q and k (QK-Norm then the identity: weights None, eps 0), no rotated
    dims and a gate of 40 (sigmoid = 1 to 4e-18), the mixer is plain causal softmax
    attention: it must equal torch's scaled_dot_product_attention (CPU, fp64) with the
    kv heads repeated for the grouped queries."""
    rng = np.random.default_rng(5)
    T, Hq, Hkv, D = 23, 4, 2, 16
    q, k, v = (rng.normal(size=(T, H, D)) for H in (Hq, Hkv, Hkv))
    q /= np.sqrt(np.mean(q * q, axis=-1, keepdims=True))
    k /= np.sqrt(np.mean(k * k, axis=-1, keepdims=True))
    g = np.full((T, Hq, D), 40.0)
    o = oracle.gated_attention(q, k, v, g, None, None, rotary_dim=0, norm_eps=0.0, scale=0.3)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           scale=0.3)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_attention_rows_match_the_whole_output():
    """The sampled form gives the rows of the whole output (first, middle and last
    tokens of packed sequences, a sequence of length 1 included)."""
    q, k, v, g, wq, wk = _attn_case(20, seed=6)
    cu = [0, 7, 8, 20]
    o = oracle.gated_attention(q, k, v, g, wq, wk, cu, rotary_dim=8)
    rows = [0, 3, 6, 7, 8, 13, 19]
    orows = oracle.gated_attention_rows(q[rows], k, v, g[rows], wq, wk, rows, cu, rotary_dim=8)
    assert np.allclose(orows, o[rows], rtol=1e-12, atol=1e-14)

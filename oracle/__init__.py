"""fp64 CPU oracle of the Gated DeltaNet token mixer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  It shares no code with the GPU library
(``linear_attention_sequence_causal_amd``) and neither imports the other.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, token by token); this
module builds it with gcc when needed and marshals numpy arrays to it.  See the
header of ``gdn_oracle.c`` for the passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_gdn.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c into liboracle_gdn.so with gcc (plain -O2)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            d = ctypes.c_double
            pd = ctypes.POINTER(ctypes.c_double)
            p64 = ctypes.POINTER(ctypes.c_int64)
            i32 = ctypes.c_int
            i64 = ctypes.c_int64
            lib.oracle_sigmoid.restype = d
            lib.oracle_sigmoid.argtypes = [d]
            lib.oracle_silu.restype = d
            lib.oracle_silu.argtypes = [d]
            lib.oracle_softplus.restype = d
            lib.oracle_softplus.argtypes = [d]
            lib.oracle_gates.restype = None
            lib.oracle_gates.argtypes = [i64, pd, pd, d, d, pd, pd]
            lib.oracle_prologue.restype = None
            lib.oracle_prologue.argtypes = [i64, i32, i32, i32, i32, pd, pd, pd, pd, pd,
                                            d, d, pd, pd, pd]
            lib.oracle_recurrence.restype = None
            lib.oracle_recurrence.argtypes = [i64, i32, pd, pd, pd, pd, pd, pd, pd]
            lib.oracle_epilogue.restype = None
            lib.oracle_epilogue.argtypes = [i64, i32, pd, pd, i64, pd, d, pd, i64]
            lib.oracle_prefill.restype = i32
            lib.oracle_prefill.argtypes = [i32, p64, i32, i32, i32, pd, pd, pd, pd, pd, pd,
                                           pd, pd, pd, pd, d, d, d, pd, pd, pd, pd, pd, i32]
            lib.oracle_decode_step.restype = i32
            lib.oracle_decode_step.argtypes = [i32, i32, i32, i32, pd, pd, pd, pd, pd, pd,
                                               pd, pd, pd, pd, d, d, d, pd, pd, pd, i32]
            lib.oracle_epilogue_gated.restype = None
            lib.oracle_epilogue_gated.argtypes = [i64, i32, pd, pd, i64, pd, d, pd, i64, i32]
            lib.oracle_prefill_gated.restype = i32
            lib.oracle_prefill_gated.argtypes = lib.oracle_prefill.argtypes + [i32]
            lib.oracle_decode_step_gated.restype = i32
            lib.oracle_decode_step_gated.argtypes = lib.oracle_decode_step.argtypes + [i32]
            _lib = lib
    return _lib


GATES = {"silu": 0, "sigmoid": 1}  # output gate of the epilogue


def _f64(x):
    """C-contiguous float64 copy (or view) of x; None stays None."""
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# ----------------------------------------------------------------- scalars

def sigmoid(u: float) -> float:
    return _load().oracle_sigmoid(float(u))


def silu(u: float) -> float:
    return _load().oracle_silu(float(u))


def softplus(u: float) -> float:
    return _load().oracle_softplus(float(u))


def gates(a, b, A_log: float, dt_bias: float):
    """alpha, beta of one head for token arrays a, b (model-card decay gate)."""
    a = _f64(a).ravel()
    b = _f64(b).ravel()
    al = np.empty_like(a)
    be = np.empty_like(a)
    _load().oracle_gates(a.size, _ptr(a), _ptr(b), float(A_log), float(dt_bias),
                         _ptr(al), _ptr(be))
    return al, be


# ------------------------------------------------------------------ stages

def prologue(q, k, v, conv_w, h: int, hist=None, q_scale=1.0, l2_eps=1e-6):
    """Post-conv/SiLU/L2 q, k (q/k head h // r) and v (v head h) of one sequence.

    q, k: [T, Hk, D]; v: [T, Hv, D]; conv_w: [Cc, 4]; hist: [3, Cc] or None.
    Returns three [T, D] float64 arrays.
    """
    q, k, v, conv_w, hist = map(_f64, (q, k, v, conv_w, hist))
    T, Hk, D = q.shape
    Hv = v.shape[1]
    qo = np.empty((T, D))
    ko = np.empty((T, D))
    vo = np.empty((T, D))
    _load().oracle_prologue(T, Hk, Hv, D, h, _ptr(q), _ptr(k), _ptr(v), _ptr(conv_w),
                            _ptr(hist), float(q_scale), float(l2_eps),
                            _ptr(qo), _ptr(ko), _ptr(vo))
    return qo, ko, vo


def recurrence(alpha, beta, q, k, v, S0=None):
    """Bare gated delta recurrence of one head (column convention, S: key->value).

    q, k, v: [T, D]; alpha, beta: [T]; S0: [D, D] (S[value][key]) or None.
    Returns (y [T, D], S_T [D, D]).
    """
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    T, D = q.shape
    S = np.zeros((D, D)) if S0 is None else _f64(S0).copy()
    y = np.empty((T, D))
    _load().oracle_recurrence(T, D, _ptr(alpha), _ptr(beta), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(S), _ptr(y))
    return y, S


def epilogue(y, z, norm_w=None, rms_eps=1e-6, output_gate="silu"):
    """RMS-normalise y per token over D, scale by norm_w, gate with SiLU(z) (or
    sigmoid(z) with output_gate="sigmoid")."""
    y, z, norm_w = map(_f64, (y, z, norm_w))
    T, D = y.shape
    o = np.empty((T, D))
    _load().oracle_epilogue_gated(T, D, _ptr(y), _ptr(z), D, _ptr(norm_w), float(rms_eps),
                                  _ptr(o), D, GATES[output_gate])
    return o


# ------------------------------------------------------------------- mixer

def prefill(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w=None, *,
            cu_seqlens=None, init_state=None, conv_in=None,
            q_scale=1.0, l2_eps=1e-6, rms_eps=1e-6, nthreads=None, output_gate="silu"):
    """Whole mixer over packed sequences, fp64.

    Returns (o [T, Hv, D], final_state [N, Hv, D, D] as H = S^T, conv_out [N, 3, Cc]).
    """
    q, k, v, a, b, z = map(_f64, (q, k, v, a, b, z))
    conv_w, A_log, dt_bias, norm_w = map(_f64, (conv_w, A_log, dt_bias, norm_w))
    init_state, conv_in = _f64(init_state), _f64(conv_in)
    T, Hk, D = q.shape
    Hv = v.shape[1]
    if cu_seqlens is None:
        cu_seqlens = [0, T]
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.size - 1
    Cc = 2 * Hk * D + Hv * D
    o = np.empty((T, Hv, D))
    fs = np.empty((N, Hv, D, D))
    co = np.empty((N, 3, Cc))
    rc = _load().oracle_prefill_gated(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), Hk, Hv, D,
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(z), _ptr(conv_w), _ptr(A_log),
        _ptr(dt_bias), _ptr(norm_w), float(q_scale), float(l2_eps), float(rms_eps),
        _ptr(init_state), _ptr(conv_in), _ptr(o), _ptr(fs), _ptr(co),
        int(nthreads or default_threads()), GATES[output_gate])
    if rc != 0:
        raise ValueError("oracle_prefill: invalid arguments")
    return o, fs, co


def decode_step(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, state, conv_cache, *,
                q_scale=1.0, l2_eps=1e-6, rms_eps=1e-6, nthreads=None, output_gate="silu"):
    """One decode step for B sequences.  Returns (o, new_state, new_conv_cache)."""
    q, k, v, a, b, z = map(_f64, (q, k, v, a, b, z))
    conv_w, A_log, dt_bias, norm_w = map(_f64, (conv_w, A_log, dt_bias, norm_w))
    state = _f64(state).copy()
    cache = _f64(conv_cache).copy()
    B, Hk, D = q.shape
    Hv = v.shape[1]
    o = np.empty((B, Hv, D))
    rc = _load().oracle_decode_step_gated(
        B, Hk, Hv, D, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(z), _ptr(conv_w),
        _ptr(A_log), _ptr(dt_bias), _ptr(norm_w), float(q_scale), float(l2_eps),
        float(rms_eps), _ptr(state), _ptr(cache), _ptr(o), int(nthreads or default_threads()),
        GATES[output_gate])
    if rc != 0:
        raise ValueError("oracle_decode_step: invalid arguments")
    return o, state, cache


def round_bf16(x):
    """Nearest bf16 value of each fp64 element (8 significant bits, ties to even),
    returned as fp64.  Normal range only: x = m 2^e with 0.5 <= |m| < 1, and m is
    rounded to a multiple of 2^-8."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def decode_step_bf16_state(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, state, conv_cache,
                           **kw):
    """One decode step with the state stored in bf16: the step in fp64 on the stored
    (bf16-valued) state, then the new state rounded to the nearest bf16 value.
    Returns (o, new_state, new_conv_cache)."""
    o, st, cache = decode_step(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, state,
                               conv_cache, **kw)
    return o, round_bf16(st), cache


FP8_MAX = 448.0  # largest finite OCP E4M3 value, 1.75 * 2^8


def round_fp8_e4m3(x):
    """Nearest OCP E4M3 value of each fp64 element (ties to even), as fp64, for
    |x| <= 448.  E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; normal values
    from 2^-6 carry 4 significant bits, smaller ones are multiples of 2^-9."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                              # x = m 2^e, 0.5 <= |m| < 1
    normal = np.ldexp(np.rint(np.ldexp(m, 4)), e - 4)
    sub = np.rint(np.ldexp(x, 9)) / 512.0
    return np.where(np.abs(x) >= 2.0 ** -6, normal, sub)


def fp8_row_scales(x):
    """Per-row power-of-two scales of the fp8 state storage: for each row (last axis)
    the smallest 2^e with max|row| <= 448 * 2^e (1 for an all-zero row)."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(np.abs(x), axis=-1)
    f, E = np.frexp(np.where(m > 0, m, 1.0))       # m = f 2^E, 0.5 <= f < 1
    e = (E - 1) - 8 + (2.0 * f > 1.75)              # 448 = 1.75 * 2^8
    return np.where(m > 0, np.ldexp(1.0, e), 1.0)


def quantize_fp8_rows(x):
    """(stored values, scales): each row divided by its scale and rounded to E4M3;
    the stored state is values * scales[..., None]."""
    s = fp8_row_scales(x)
    return round_fp8_e4m3(np.asarray(x, dtype=np.float64) / s[..., None]), s


def decode_step_fp8_state(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, state_q,
                          state_scale, conv_cache, **kw):
    """One decode step with the state stored in fp8 (E4M3 values state_q [B, Hv, D, D]
    times one power-of-two scale per state row, state_scale [B, Hv, D]): the step in
    fp64 on the stored state, then the new state re-quantised row by row.
    Returns (o, new_state_q, new_state_scale, new_conv_cache)."""
    st = np.asarray(state_q, dtype=np.float64) * np.asarray(state_scale, np.float64)[..., None]
    o, st, cache = decode_step(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, st,
                               conv_cache, **kw)
    qv, sc = quantize_fp8_rows(st)
    return o, qv, sc, cache


def decode_tokens(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, state, conv_cache, *,
                  num_commit=None, q_scale=1.0, l2_eps=1e-6, rms_eps=1e-6, nthreads=None,
                  output_gate="silu"):
    """n new tokens per sequence on a cached state (multi-token decode / verify / commit).

    q, k [B, n, Hk, D]; v, z [B, n, Hv, D]; a, b [B, n, Hv].  Returns
    (o [B, n, Hv, D], new_state, new_conv_cache): o holds the outputs of all n tokens
    (token t after tokens 0..t, as n decode steps give them); the state and the cache
    are those after the first num_commit[b] tokens (clamped to 0..n; None = n).

    The token-by-token recurrence of the prefill oracle does both: the outputs are
    one prefill of the n tokens of every sequence (packed, history = the cache,
    initial state = the cached state), the committed state and cache one prefill of
    each sequence's first num_commit[b] tokens.
    """
    q, k, v, a, b, z = map(_f64, (q, k, v, a, b, z))
    B, n, Hk, D = q.shape
    Hv = v.shape[2]
    state, cache = _f64(state), _f64(conv_cache)
    flat = lambda x: x.reshape((B * n,) + x.shape[2:])
    kw = dict(q_scale=q_scale, l2_eps=l2_eps, rms_eps=rms_eps, nthreads=nthreads,
              output_gate=output_gate)
    cu = np.arange(B + 1, dtype=np.int64) * n
    o, _, _ = prefill(flat(q), flat(k), flat(v), flat(a), flat(b), flat(z), conv_w, A_log,
                      dt_bias, norm_w, cu_seqlens=cu, init_state=state, conv_in=cache, **kw)
    commit = np.full(B, n, dtype=np.int64) if num_commit is None else \
        np.clip(np.asarray(num_commit, dtype=np.int64).reshape(B), 0, n)
    sel = np.concatenate([np.arange(bb * n, bb * n + commit[bb]) for bb in range(B)]).astype(np.int64)
    cuc = np.concatenate([[0], np.cumsum(commit)]).astype(np.int64)
    _, fs, co = prefill(flat(q)[sel], flat(k)[sel], flat(v)[sel], flat(a)[sel], flat(b)[sel],
                        flat(z)[sel], conv_w, A_log, dt_bias, norm_w, cu_seqlens=cuc,
                        init_state=state, conv_in=cache, **kw)
    return o.reshape(B, n, Hv, D), fs, co


# --------------------------------------------------------- projections

def linear(x, w):
    """y = x w^T in fp64: x [M, K] (one token per row), w [N, K] (one row of weights per
    output feature).  A plain matrix product (the projections on either side of the
    mixer: tech report Fig. 2 caption, the projected q/k/v streams; field guide
    cutaway 02, the gated output is projected)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def in_projection(x, w_in, Hk: int, Hv: int, D: int):
    """The mixer's inputs from hidden states x [T, d_model]: y = x w_in^T, split by
    columns into q, k [T, Hk, D], v, z [T, Hv, D], a, b [T, Hv] (rows of w_in in the
    order q | k | v | z | a | b)."""
    y = linear(x, w_in)
    T = y.shape[0]
    cuts = np.cumsum([0, Hk * D, Hk * D, Hv * D, Hv * D, Hv, Hv])
    if cuts[-1] != y.shape[1]:
        raise ValueError("w_in must have 2*Hk*D + 2*Hv*D + 2*Hv rows")
    part = [y[:, cuts[i]:cuts[i + 1]] for i in range(6)]
    return (part[0].reshape(T, Hk, D), part[1].reshape(T, Hk, D), part[2].reshape(T, Hv, D),
            part[3].reshape(T, Hv, D), part[4], part[5])


def gdn_layer(x, w_in, w_out, conv_w, A_log, dt_bias, norm_w, Hk: int, Hv: int, D: int,
              **kw):
    """The whole layer: in-projection, mixer (prefill), output projection of o read as
    [T, Hv*D].  Returns (y [T, d_model], final_state, conv_out)."""
    q, k, v, z, a, b = in_projection(x, w_in, Hk, Hv, D)
    o, fs, co = prefill(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, **kw)
    return linear(o.reshape(o.shape[0], Hv * D), w_out), fs, co


# ------------------------------------------------- gated full attention

def attn_rms_norm(x, w, eps):
    """QK-Norm: RMSNorm over the head dimension (last axis) times the weight w
    ("Qwen3.8-Flash-Next" model card, attention entry: per-head RMSNorm of queries and
    keys before RoPE; "Qwen3-Next 80B-A3B" field guide, cutaway 03)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * (1.0 if w is None else np.asarray(w, np.float64))


def partial_rope(x, pos, rotary_dim, theta):
    """RoPE on the first rotary_dim dims of each head (model card: partial_rotary_factor
    0.25, each head split into a rotated part and a position-free part; field guide
    cutaway 03: 64 of 256 dims).  Rotate-half pairing: dim i and i + rotary_dim/2
    rotate by the angle pos * theta^(-2i/rotary_dim), i < rotary_dim/2.
    x [T, H, D], pos [T]."""
    x = np.asarray(x, dtype=np.float64)
    half = rotary_dim // 2
    inv = theta ** (-2.0 * np.arange(half) / rotary_dim)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]       # [T, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:rotary_dim]
    out = x.copy()
    out[..., :half] = x1 * c - x2 * s
    out[..., half:rotary_dim] = x2 * c + x1 * s
    return out


def gated_attention(q, k, v, gate, q_norm_w, k_norm_w, cu_seqlens=None, *, rotary_dim=64,
                    theta=10000.0, norm_eps=1e-6, scale=None):
    """The hybrid's gated full-attention mixer (field guide cutaway 03; model card
    attention entries), fp64:
        q^ = RoPE(RMSNorm(q) w_q),  k^ = RoPE(RMSNorm(k) w_k)      (positions from 0 in
                                                                    each sequence)
        o  = softmax_causal(q^ k^T * scale) v  *  sigmoid(gate)
    with grouped queries: q head h reads kv head h / (Hq / Hkv).
    q, gate [T, Hq, D]; k, v [T, Hkv, D]; returns o [T, Hq, D]."""
    q, k, v, gate = (np.asarray(x, dtype=np.float64) for x in (q, k, v, gate))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = D ** -0.5 if scale is None else scale
    cu = np.asarray([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    o = np.zeros_like(q)
    for n in range(cu.size - 1):
        b, e = int(cu[n]), int(cu[n + 1])
        if e == b:
            continue
        pos = np.arange(e - b)
        qh = partial_rope(attn_rms_norm(q[b:e], q_norm_w, norm_eps), pos, rotary_dim, theta)
        kh = partial_rope(attn_rms_norm(k[b:e], k_norm_w, norm_eps), pos, rotary_dim, theta)
        mask = np.tril(np.ones((e - b, e - b), dtype=bool))
        for h in range(Hq):
            g = h // (Hq // Hkv)
            sc = qh[:, h, :] @ kh[:, g, :].T * scale
            sc = np.where(mask, sc, -np.inf)
            sc -= sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p /= p.sum(axis=1, keepdims=True)
            o[b:e, h, :] = (p @ v[b:e, g, :]) / (1.0 + np.exp(-gate[b:e, h, :]))
    return o


def gated_attention_rows(q_rows, k, v, gate_rows, q_norm_w, k_norm_w, rows, cu_seqlens=None,
                         *, rotary_dim=64, theta=10000.0, norm_eps=1e-6, scale=None):
    """gated_attention at the query tokens `rows` only (for sizes where the whole output
    is too costly): q_rows, gate_rows [len(rows), Hq, D] are q and gate at those tokens;
    each row attends to the keys of its sequence up to itself, exactly as in
    gated_attention.  Returns o [len(rows), Hq, D]."""
    q, k, v, gate = (np.asarray(x, dtype=np.float64) for x in (q_rows, k, v, gate_rows))
    T, Hkv, D = k.shape
    Hq = q.shape[1]
    scale = D ** -0.5 if scale is None else scale
    cu = np.asarray([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    out = np.zeros((len(rows), Hq, D))
    for j, t in enumerate(rows):
        n = int(np.searchsorted(cu, t, side="right")) - 1
        b = int(cu[n])
        pos = np.arange(t + 1 - b)
        kh = partial_rope(attn_rms_norm(k[b:t + 1], k_norm_w, norm_eps), pos, rotary_dim, theta)
        qh = partial_rope(attn_rms_norm(q[j:j + 1], q_norm_w, norm_eps), pos[-1:], rotary_dim,
                          theta)[0]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            sc = kh[:, g, :] @ qh[h] * scale
            p = np.exp(sc - sc.max())
            p /= p.sum()
            out[j, h] = (p @ v[b:t + 1, g, :]) / (1.0 + np.exp(-gate[j, h]))
    return out


def select_heads(qk_heads, Hk: int, Hv: int, D: int):
    """Index helpers to run the oracle on a subset of q/k heads (and their v heads).

    Returns (qk_idx, v_idx, conv_channel_idx) for slicing q/k [.., Hk, D],
    v/z/a/b [.., Hv(, D)] and conv weights / history [.., Cc].
    """
    r = Hv // Hk
    qk_idx = np.asarray(sorted(qk_heads), dtype=np.int64)
    v_idx = np.asarray([g * r + j for g in qk_idx for j in range(r)], dtype=np.int64)
    ch = [g * D + i for g in qk_idx for i in range(D)]
    ch += [Hk * D + g * D + i for g in qk_idx for i in range(D)]
    ch += [2 * Hk * D + h * D + i for h in v_idx for i in range(D)]
    return qk_idx, v_idx, np.asarray(ch, dtype=np.int64)

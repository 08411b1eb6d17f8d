"""Gated DeltaNet token mixer on MI355X (gfx950): thin Python binding.

Every step of the mixer runs in the HIP kernels of ``libgdn.so`` (built from
``csrc/`` by ``build.py``); this module only marshals torch tensors (device
memory and the current stream) into the C ABI declared in ``include/gdn.h``.
There is no CPU fallback: if the library is missing, loading fails loudly.

Mixer definition: "Qwen3-Next 80B-A3B" field guide, cutaway 02 (gated delta
update, counts, RMSNorm + SiLU(z) gate); "Qwen3.8-Flash-Next" model card
(decay gate, chunk state update); tech report Fig. 2 caption (short convs,
L2-normalised q/k).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_BF16, GDN_F32 = 0, 1
GATES = {"silu": 0, "sigmoid": 1}  # gdn_gate
STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARGUMENT", 2: "GDN_ERR_UNSUPPORTED",
          3: "GDN_ERR_WORKSPACE", 4: "GDN_ERR_NO_DEVICE", 5: "GDN_ERR_HIP"}
EXPORTED = ("gdn_prefill_workspace_bytes", "gdn_prefill", "gdn_prefill_noalloc",
            "gdn_decode_step", "gdn_decode_step_fp8_state",
            "gdn_decode_step_bf16_state", "gdn_decode_tokens", "gdn_prefill_last_kernel_times",
            "gdn_linear", "gdn_in_projection", "gdn_out_projection",
            "gdn_gated_attention_workspace_bytes", "gdn_gated_attention",
            "gdn_check_device_errors", "gdn_status_string", "gdn_last_error", "gdn_version")
PREFILL_KERNELS = ("segment_table", "maps", "combine", "full", "conv_state_out")


class GdnParams(ctypes.Structure):
    _fields_ = [("num_qk_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("q_scale", ctypes.c_float), ("l2_eps", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("conv_weight", ctypes.c_void_p),
                ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("norm_weight", ctypes.c_void_p), ("output_gate", ctypes.c_int32)]


class GdnAttnParams(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rotary_dim", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("scale", ctypes.c_float), ("q_norm_weight", ctypes.c_void_p),
                ("k_norm_weight", ctypes.c_void_p)]


class GdnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m linear_attention_sequence_causal_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            pp = ctypes.POINTER(GdnParams)
            L.gdn_prefill_workspace_bytes.restype = sz
            L.gdn_prefill_workspace_bytes.argtypes = [pp, i32, i64]
            L.gdn_prefill.restype = ctypes.c_int
            L.gdn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, pp, vp, vp, i32, i64, vp, vp, vp,
                                      vp, vp, sz, vp]
            L.gdn_prefill_noalloc.restype = ctypes.c_int
            L.gdn_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, pp, vp, vp, i32, i64, vp, vp,
                                              vp, vp, vp]
            L.gdn_decode_step.restype = ctypes.c_int
            L.gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, pp, vp, vp, vp, i32, vp]
            L.gdn_decode_step_bf16_state.restype = ctypes.c_int
            L.gdn_decode_step_bf16_state.argtypes = [vp, vp, vp, vp, vp, vp, pp, vp, vp, vp, i32,
                                                     vp]
            L.gdn_decode_step_fp8_state.restype = ctypes.c_int
            L.gdn_decode_step_fp8_state.argtypes = [vp, vp, vp, vp, vp, vp, pp, vp, vp, vp, vp,
                                                    i32, vp]
            L.gdn_decode_tokens.restype = ctypes.c_int
            L.gdn_decode_tokens.argtypes = [vp, vp, vp, vp, vp, vp, pp, vp, vp, vp, vp, i32, i32,
                                            vp]
            L.gdn_status_string.restype = ctypes.c_char_p
            L.gdn_status_string.argtypes = [ctypes.c_int]
            L.gdn_last_error.restype = ctypes.c_char_p
            L.gdn_last_error.argtypes = []
            L.gdn_version.restype = ctypes.c_char_p
            L.gdn_version.argtypes = []
            L.gdn_linear.restype = ctypes.c_int
            L.gdn_linear.argtypes = [vp, vp, i64, i32, i32, vp, vp]
            L.gdn_in_projection.restype = ctypes.c_int
            L.gdn_in_projection.argtypes = [vp, vp, pp, i64, i32, vp, vp, vp, vp, vp, vp, vp]
            L.gdn_out_projection.restype = ctypes.c_int
            L.gdn_out_projection.argtypes = [vp, vp, pp, i64, i32, vp, vp]
            ap = ctypes.POINTER(GdnAttnParams)
            L.gdn_gated_attention_workspace_bytes.restype = sz
            L.gdn_gated_attention_workspace_bytes.argtypes = [ap, i64]
            L.gdn_gated_attention.restype = ctypes.c_int
            L.gdn_gated_attention.argtypes = [vp, vp, vp, vp, ap, vp, i32, i64, vp, vp, sz, vp]
            L.gdn_check_device_errors.restype = ctypes.c_int
            L.gdn_check_device_errors.argtypes = [vp]
            L.gdn_prefill_last_kernel_times.restype = ctypes.c_int
            L.gdn_prefill_last_kernel_times.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                        ctypes.c_int]
            _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise GdnError(status, lib().gdn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_params(num_qk_heads, num_v_heads, head_dim, act_dtype, conv_w, A_log, dt_bias,
                norm_w=None, q_scale=1.0, l2_eps=1e-6, rms_eps=1e-6,
                output_gate="silu") -> GdnParams:
    dt = GDN_BF16 if act_dtype == torch.bfloat16 else GDN_F32 if act_dtype == torch.float32 else -1
    return GdnParams(int(num_qk_heads), int(num_v_heads), int(head_dim), dt, float(q_scale),
                     float(l2_eps), float(rms_eps), _ptr(conv_w), _ptr(A_log), _ptr(dt_bias),
                     _ptr(norm_w), GATES[output_gate])


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to the mixer must be contiguous")


def workspace_bytes(params: GdnParams, num_seqs: int, total_tokens: int) -> int:
    n = lib().gdn_prefill_workspace_bytes(ctypes.byref(params), int(num_seqs), int(total_tokens))
    if n == ctypes.c_size_t(-1).value:
        raise GdnError(1, lib().gdn_last_error().decode())
    return n


_ws_cache = {}


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def prefill(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w=None, *, init_state=None,
            cu_seqlens=None, conv_state=None, return_conv_state=False, q_scale=1.0,
            l2_eps=1e-6, rms_eps=1e-6, out=None, final_state=None, output_gate="silu"):
    """Chunked prefill over packed sequences -> (o, final_state[, conv_state_out]).

    q, k [T, Hk, D]; v, z [T, Hv, D] (bf16 or fp32); a, b [T, Hv] fp32;
    conv_w [Cc, 4]; A_log, dt_bias [Hv]; norm_w [D] or None; init_state
    [N, Hv, D, D] fp32 or None; cu_seqlens [N+1] int32 or None (one sequence);
    conv_state [N, 3, Cc] or None.  Outputs are allocated on q's device unless
    given; the work is enqueued on torch's current stream.
    """
    T, Hk, D = q.shape
    Hv = v.shape[1]
    N = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    _contig(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, init_state, cu_seqlens, conv_state)
    p = make_params(Hk, Hv, D, q.dtype, conv_w, A_log, dt_bias, norm_w, q_scale, l2_eps, rms_eps,
                    output_gate)
    o = torch.empty_like(v) if out is None else out
    fs = (torch.empty((N, Hv, D, D), dtype=torch.float32, device=q.device)
          if final_state is None else final_state)
    Cc = 2 * Hk * D + Hv * D
    cso = torch.empty((N, 3, Cc), dtype=q.dtype, device=q.device) if return_conv_state else None
    nbytes = workspace_bytes(p, N, T)
    ws = _workspace(nbytes, q.device)
    _check(lib().gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(z),
                             ctypes.byref(p), _ptr(init_state), _ptr(cu_seqlens), N, T,
                             _ptr(conv_state), _ptr(o), _ptr(fs), _ptr(cso), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream()))
    if return_conv_state:
        return o, fs, cso
    return o, fs


NOALLOC_WORKSPACE_BYTES = 128 << 20


def prefill_noalloc(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, *, init_state=None,
                    cu_seqlens=None, conv_state=None, q_scale=1.0, l2_eps=1e-6, rms_eps=1e-6,
                    out, final_state, conv_state_out=None, output_gate="silu"):
    """gdn_prefill_noalloc: the prefill with the library's static workspace, into
    caller-provided outputs (nothing is allocated)."""
    T, Hk, D = q.shape
    Hv = v.shape[1]
    N = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    _contig(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, init_state, cu_seqlens, conv_state,
            out, final_state, conv_state_out)
    p = make_params(Hk, Hv, D, q.dtype, conv_w, A_log, dt_bias, norm_w, q_scale, l2_eps, rms_eps,
                    output_gate)
    _check(lib().gdn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(z),
                                     ctypes.byref(p), _ptr(init_state), _ptr(cu_seqlens), N, T,
                                     _ptr(conv_state), _ptr(out), _ptr(final_state),
                                     _ptr(conv_state_out), _stream()))
    return out, final_state


def decode_step(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, state, conv_state, *,
                q_scale=1.0, l2_eps=1e-6, rms_eps=1e-6, out=None, state_scale=None,
                output_gate="silu"):
    """One decode step; updates `state` and `conv_state` in place, returns o.

    q, k [B, Hk, D]; v, z [B, Hv, D]; a, b [B, Hv]; state [B, Hv, D, D] fp32, or bf16 or
    float8_e4m3fn for the reduced-precision storage modes (fp32 arithmetic, state rounded
    on store; fp8 also needs state_scale [B, Hv, D] fp32, one power of two per row,
    updated in place); conv_state [B, 3, Cc] in the activation dtype.
    """
    B, Hk, D = q.shape
    Hv = v.shape[1]
    _contig(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, state, conv_state)
    p = make_params(Hk, Hv, D, q.dtype, conv_w, A_log, dt_bias, norm_w, q_scale, l2_eps, rms_eps,
                    output_gate)
    o = torch.empty_like(v) if out is None else out
    if state.dtype == torch.float8_e4m3fn:
        if state_scale is None or state_scale.dtype != torch.float32:
            raise ValueError("fp8 state storage needs a float32 state_scale [B, Hv, D]")
        _contig(state_scale)
        _check(lib().gdn_decode_step_fp8_state(
            _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(z), ctypes.byref(p), _ptr(state),
            _ptr(state_scale), _ptr(conv_state), _ptr(o), B, _stream()))
        return o
    if state.dtype == torch.bfloat16:  # reduced-precision storage of the state
        fn = lib().gdn_decode_step_bf16_state
    elif state.dtype == torch.float32:
        fn = lib().gdn_decode_step
    else:
        raise ValueError("state must be float32, bfloat16 or float8_e4m3fn")
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(z), ctypes.byref(p), _ptr(state),
              _ptr(conv_state), _ptr(o), B, _stream()))
    return o


def decode_tokens(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, state, conv_state, *,
                  num_commit=None, q_scale=1.0, l2_eps=1e-6, rms_eps=1e-6, out=None,
                  output_gate="silu"):
    """n new tokens per sequence on a cached state; returns o [B, n, Hv, D].

    q, k [B, n, Hk, D]; v, z [B, n, Hv, D]; a, b [B, n, Hv]; state [B, Hv, D, D] fp32 and
    conv_state [B, 3, Cc] advance in place by num_commit[b] tokens (int32 [B] on the
    device, clamped to 0..n; None = n).
    """
    B, n, Hk, D = q.shape
    Hv = v.shape[2]
    _contig(q, k, v, a, b, z, conv_w, A_log, dt_bias, norm_w, state, conv_state, num_commit)
    if num_commit is not None and (num_commit.dtype != torch.int32 or num_commit.numel() != B):
        raise ValueError("num_commit must be an int32 tensor of B elements")
    p = make_params(Hk, Hv, D, q.dtype, conv_w, A_log, dt_bias, norm_w, q_scale, l2_eps, rms_eps,
                    output_gate)
    o = torch.empty_like(v) if out is None else out
    _check(lib().gdn_decode_tokens(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(z),
                                   ctypes.byref(p), _ptr(state), _ptr(conv_state),
                                   _ptr(num_commit), _ptr(o), B, n, _stream()))
    return o


def linear(x, w, out=None):
    """y = x w^T on bf16 MFMA (fp32 accumulation, bf16 out): x [M, K], w [N, K]."""
    M, K = x.shape
    N = w.shape[0]
    _contig(x, w)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _check(lib().gdn_linear(_ptr(x), _ptr(w), M, N, K, _ptr(y), _stream()))
    return y


def in_projection(x, w_in, num_qk_heads, num_v_heads, head_dim=128, act_dtype=torch.bfloat16):
    """(q, k, v, z, a, b) of the mixer from hidden states x [T, d_model] bf16 and
    w_in [2*Hk*D + 2*Hv*D + 2*Hv, d_model] bf16 (rows q | k | v | z | a | b)."""
    T, d_model = x.shape
    Hk, Hv, D = num_qk_heads, num_v_heads, head_dim
    _contig(x, w_in)
    dev = x.device
    q = torch.empty((T, Hk, D), dtype=act_dtype, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((T, Hv, D), dtype=act_dtype, device=dev)
    z = torch.empty_like(v)
    a = torch.empty((T, Hv), dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    p = GdnParams(Hk, Hv, D, GDN_BF16 if act_dtype == torch.bfloat16 else GDN_F32, 1.0, 1e-6,
                  1e-6, None, None, None, None, 0)
    _check(lib().gdn_in_projection(_ptr(x), _ptr(w_in), ctypes.byref(p), T, d_model, _ptr(q),
                                   _ptr(k), _ptr(v), _ptr(z), _ptr(a), _ptr(b), _stream()))
    return q, k, v, z, a, b


def out_projection(o, w_out, out=None):
    """y [T, d_model] bf16 = o w_out^T for o [T, Hv, D] bf16, w_out [d_model, Hv*D]."""
    T, Hv, D = o.shape
    d_model = w_out.shape[0]
    _contig(o, w_out)
    y = torch.empty((T, d_model), dtype=torch.bfloat16, device=o.device) if out is None else out
    p = GdnParams(1, Hv, D, GDN_BF16, 1.0, 1e-6, 1e-6, None, None, None, None, 0)
    _check(lib().gdn_out_projection(_ptr(o), _ptr(w_out), ctypes.byref(p), T, d_model, _ptr(y),
                                    _stream()))
    return y


def gated_attention(q, k, v, gate, q_norm_w=None, k_norm_w=None, cu_seqlens=None, *,
                    rotary_dim=64, theta=10000.0, norm_eps=1e-6, scale=None, out=None):
    """The hybrid's gated full-attention mixer (QK-Norm, partial RoPE, causal GQA softmax,
    sigmoid output gate) -> o [T, Hq, D] bf16.  q, gate [T, Hq, D] and k, v [T, Hkv, D]
    bf16, D = 256; norm weights [D] fp32 or None; cu_seqlens [N+1] int32 or None."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    _contig(q, k, v, gate, q_norm_w, k_norm_w, cu_seqlens)
    N = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    p = GdnAttnParams(Hq, Hkv, D, int(rotary_dim), float(theta), float(norm_eps),
                      0.0 if scale is None else float(scale), _ptr(q_norm_w), _ptr(k_norm_w))
    nbytes = lib().gdn_gated_attention_workspace_bytes(ctypes.byref(p), T)
    if nbytes == ctypes.c_size_t(-1).value:
        raise GdnError(1, lib().gdn_last_error().decode())
    ws = _workspace(nbytes, q.device)
    o = torch.empty_like(q) if out is None else out
    _check(lib().gdn_gated_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), ctypes.byref(p),
                                     _ptr(cu_seqlens), N, T, _ptr(o), _ptr(ws),
                                     0 if ws is None else ws.numel(),
                                     _stream()))
    return o


def check_device_errors():
    """Raise GdnError if a kernel of an earlier call on the current device found invalid
    device-resident arguments (an invalid cu_seqlens table); clears the flag.
    Synchronises torch's current stream."""
    _check(lib().gdn_check_device_errors(_stream()))


def last_kernel_times():
    """{kernel name: ms} of the last prefill call made with GDN_KERNEL_TIMING=1."""
    buf = (ctypes.c_float * len(PREFILL_KERNELS))()
    n = lib().gdn_prefill_last_kernel_times(buf, len(PREFILL_KERNELS))
    if n < 0:
        return None
    return {PREFILL_KERNELS[i]: float(buf[i]) for i in range(n)}


def version() -> str:
    return lib().gdn_version().decode()

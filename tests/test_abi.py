"""C-ABI checks that need no GPU: exports, status strings, argument validation.

All validation happens on the host before any HIP call, so invalid arguments
are reported here without a device, and valid calls report GDN_ERR_NO_DEVICE
in a container without a GPU.  Output buffers are host memory in these tests
(the library never dereferences them on the host); they must be untouched
after an error.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import linear_attention_sequence_causal_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = gdn.lib()
    declared = _declared_functions()
    assert set(declared) == set(gdn.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings_and_version():
    L = gdn.lib()
    for code, name in gdn.STATUS.items():
        assert L.gdn_status_string(code).decode() == name
    assert gdn.version().startswith("gdn-gfx950")


def _host(n, dtype=np.float32, fill=7.0):
    return np.full(n, fill, dtype=dtype)


def _params(Hk=2, Hv=4, D=128, dtype=gdn.GDN_BF16, host=None):
    host = host or {}
    Cc = 2 * Hk * D + Hv * D
    host.setdefault("conv", _host(max(Cc, 1) * 4))
    host.setdefault("alog", _host(max(Hv, 1)))
    host.setdefault("dt", _host(max(Hv, 1)))
    p = gdn.GdnParams(Hk, Hv, D, dtype, 1.0, 1e-6, 1e-6, host["conv"].ctypes.data,
                      host["alog"].ctypes.data, host["dt"].ctypes.data, None)
    return p, host


def _decode(p, B=2, out=None, **over):
    bufs = {n: _host(1 << 16) for n in ("q", "k", "v", "a", "b", "z", "state", "cache")}
    o = out if out is not None else _host(1 << 16)
    ptr = {n: ctypes.c_void_p(x.ctypes.data) for n, x in bufs.items()}
    ptr.update(over)
    return gdn.lib().gdn_decode_step(ptr["q"], ptr["k"], ptr["v"], ptr["a"], ptr["b"], ptr["z"],
                                     ctypes.byref(p) if p is not None else None, ptr["state"],
                                     ptr["cache"], ctypes.c_void_p(o.ctypes.data), B, None)


def _tokens(p, B=2, n=4, out=None, **over):
    bufs = {n_: _host(1 << 16) for n_ in ("q", "k", "v", "a", "b", "z", "state", "cache")}
    o = out if out is not None else _host(1 << 16)
    ptr = {n_: ctypes.c_void_p(x.ctypes.data) for n_, x in bufs.items()}
    ptr.update(over)
    return gdn.lib().gdn_decode_tokens(ptr["q"], ptr["k"], ptr["v"], ptr["a"], ptr["b"],
                                       ptr["z"], ctypes.byref(p) if p is not None else None,
                                       ptr["state"], ptr["cache"], None,
                                       ctypes.c_void_p(o.ctypes.data), B, n, None)


def _prefill(p, N=1, T=64, out=None, ws=None, ws_bytes=0, cu=True, **over):
    bufs = {n: _host(1 << 16) for n in ("q", "k", "v", "a", "b", "z", "fs")}
    o = out if out is not None else _host(1 << 16)
    cu_arr = np.zeros(N + 1, dtype=np.int32)
    ptr = {n: ctypes.c_void_p(x.ctypes.data) for n, x in bufs.items()}
    ptr.update(over)
    return gdn.lib().gdn_prefill(ptr["q"], ptr["k"], ptr["v"], ptr["a"], ptr["b"], ptr["z"],
                                 ctypes.byref(p) if p is not None else None, None,
                                 ctypes.c_void_p(cu_arr.ctypes.data) if cu else None, N, T, None,
                                 ctypes.c_void_p(o.ctypes.data), ptr["fs"], None,
                                 ws, ws_bytes, None)


INVALID, UNSUPPORTED, WORKSPACE, NO_DEVICE = 1, 2, 3, 4


def test_decode_argument_errors_leave_outputs_untouched():
    o = _host(1 << 16, fill=3.0)
    p, h = _params()
    assert _decode(None, out=o) == INVALID
    p, h = _params(Hk=3, Hv=4)
    assert _decode(p, out=o) == INVALID
    assert "multiple" in gdn.lib().gdn_last_error().decode()
    p, h = _params(D=64)
    assert _decode(p, out=o) == UNSUPPORTED
    p, h = _params(dtype=7)
    assert _decode(p, out=o) == INVALID
    p, h = _params()
    assert _decode(p, B=-1, out=o) == INVALID
    assert _decode(p, out=o, q=None) == INVALID
    p, h = _params(Hk=1, Hv=16)
    assert _decode(p, out=o) == UNSUPPORTED  # ratio above the decode kernel's limit
    p, h = _params()
    p.conv_weight = None
    assert _decode(p, out=o) == INVALID
    assert np.all(o == 3.0)


def test_decode_tokens_argument_errors_leave_outputs_untouched():
    o = _host(1 << 16, fill=4.0)
    p, h = _params()
    assert _tokens(None, out=o) == INVALID
    assert _tokens(p, n=0, out=o) == INVALID
    assert _tokens(p, n=9, out=o) == INVALID
    assert "n_tokens" in gdn.lib().gdn_last_error().decode()
    assert _tokens(p, B=-1, out=o) == INVALID
    assert _tokens(p, out=o, state=None) == INVALID
    p, h = _params(Hk=1, Hv=16)
    assert _tokens(p, out=o) == UNSUPPORTED
    p, h = _params(D=64)
    assert _tokens(p, out=o) == UNSUPPORTED
    assert np.all(o == 4.0)


def test_prefill_argument_errors():
    o = _host(1 << 16, fill=5.0)
    p, h = _params()
    assert _prefill(None, out=o) == INVALID
    assert _prefill(p, N=-1, out=o) == INVALID
    assert _prefill(p, T=-3, out=o) == INVALID
    assert _prefill(p, N=2, cu=False, out=o) == INVALID
    assert _prefill(p, out=o, z=None) == INVALID
    assert _prefill(p, out=o, fs=None) == INVALID
    p64, _ = _params(D=64)
    assert _prefill(p64, out=o) == UNSUPPORTED
    assert np.all(o == 5.0)


def test_prefill_workspace_rules():
    p, h = _params(Hk=16, Hv=32)
    L = gdn.lib()
    n_short = L.gdn_prefill_workspace_bytes(ctypes.byref(p), 1, 0)
    assert 0 < n_short < 4096  # the device-built segment table only
    n_long = L.gdn_prefill_workspace_bytes(ctypes.byref(p), 1, 65536)
    assert n_long > 1 << 20  # long sequences are split into segments that need maps
    assert L.gdn_prefill_workspace_bytes(ctypes.byref(p), 0, 0) == 0
    assert L.gdn_prefill_workspace_bytes(ctypes.byref(p), -1, 10) == ctypes.c_size_t(-1).value
    o = _host(1 << 16, fill=1.0)
    assert _prefill(p, T=65536, out=o, ws=None, ws_bytes=0) == WORKSPACE
    ws = _host(16)
    assert _prefill(p, T=65536, out=o, ws=ctypes.c_void_p(ws.ctypes.data),
                    ws_bytes=n_long - 1) == WORKSPACE
    assert np.all(o == 1.0)


def test_valid_calls_report_missing_device(monkeypatch):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    p, h = _params()
    assert _decode(p) == NO_DEVICE
    assert _tokens(p) == NO_DEVICE
    bufs = {n: _host(1 << 16) for n in ("q", "k", "v", "a", "b", "z", "state", "cache", "o")}
    ptr = {n: ctypes.c_void_p(x.ctypes.data) for n, x in bufs.items()}
    assert gdn.lib().gdn_decode_step_bf16_state(
        ptr["q"], ptr["k"], ptr["v"], ptr["a"], ptr["b"], ptr["z"], ctypes.byref(p),
        ptr["state"], ptr["cache"], ptr["o"], 2, None) == NO_DEVICE
    n = gdn.lib().gdn_prefill_workspace_bytes(ctypes.byref(p), 1, 64)
    raw = np.zeros(n + 512, dtype=np.uint8)
    addr = (raw.ctypes.data + 255) // 256 * 256
    assert _prefill(p, ws=ctypes.c_void_p(addr), ws_bytes=n) == NO_DEVICE
    assert np.all(raw == 0)


def test_noalloc_prefill_rejects_problems_above_its_workspace_without_a_device():
    """gdn_prefill_noalloc checks the problem's workspace against its static array on
    the host, before the device check: no output is touched."""
    p, host = _params(Hk=16, Hv=32)
    need = gdn.lib().gdn_prefill_workspace_bytes(ctypes.byref(p), 64, 1 << 20)
    assert need > gdn.NOALLOC_WORKSPACE_BYTES
    bufs = {n: _host(1 << 10) for n in ("q", "k", "v", "a", "b", "z", "cu")}
    o, fs = _host(1 << 10), _host(1 << 10)
    ptr = lambda x: ctypes.c_void_p(x.ctypes.data)
    st = gdn.lib().gdn_prefill_noalloc(ptr(bufs["q"]), ptr(bufs["k"]), ptr(bufs["v"]),
                                       ptr(bufs["a"]), ptr(bufs["b"]), ptr(bufs["z"]),
                                       ctypes.byref(p), None, ptr(bufs["cu"]), 64, 1 << 20, None,
                                       ptr(o), ptr(fs), None, None)
    assert st == 3  # GDN_ERR_WORKSPACE
    assert "gdn_prefill_noalloc" in gdn.lib().gdn_last_error().decode()
    assert np.all(o == 7.0) and np.all(fs == 7.0)
    # the 65536-token single-sequence workload fits
    assert gdn.lib().gdn_prefill_workspace_bytes(ctypes.byref(p), 1, 65536) <= \
        gdn.NOALLOC_WORKSPACE_BYTES


def test_output_gate_must_be_silu_or_sigmoid():
    p, host = _params()
    p.output_gate = 2
    o = _host(1 << 16)
    assert _decode(p, out=o) == 1  # GDN_ERR_INVALID_ARGUMENT
    assert "output_gate" in gdn.lib().gdn_last_error().decode()
    assert np.all(o == 7.0)
    p.output_gate = 1
    assert _decode(p, out=o) == 4  # valid: reaches the (missing) device


def _attn_params(Hq=16, Hkv=2, D=256, rot=64, theta=1e4, eps=1e-6):
    return gdn.GdnAttnParams(Hq, Hkv, D, rot, theta, eps, 0.0, None, None)


def test_gated_attention_argument_errors_leave_outputs_untouched():
    L = gdn.lib()
    T = 8
    q = _host(T * 16 * 256)
    kv = _host(T * 2 * 256)
    o = _host(T * 16 * 256)
    ptr = lambda x: ctypes.c_void_p(x.ctypes.data)

    def call(p, N=1, cu=None, out=o, ws=None, ws_bytes=0):
        return L.gdn_gated_attention(ptr(q), ptr(kv), ptr(kv), ptr(q), ctypes.byref(p), cu, N,
                                     T, ptr(out), ws, ws_bytes, None)

    cases = [(_attn_params(Hq=3, Hkv=2), 1, "multiple"),
             (_attn_params(D=128), 2, "256"),
             (_attn_params(rot=24), 1, "rotary_dim"),
             (_attn_params(rot=272), 1, "rotary_dim"),
             (_attn_params(theta=0.0), 1, "rope_theta"),
             (_attn_params(eps=-1.0), 1, "norm_eps")]
    for p, code, word in cases:
        assert call(p) == code, word
        assert word in L.gdn_last_error().decode()
    assert call(_attn_params(), N=2) == 1             # cu_seqlens required for N > 1
    assert call(_attn_params(), out=q) == 1           # o aliases q
    assert call(_attn_params()) == 3                  # workspace missing
    assert np.all(o == 7.0)


def test_gated_attention_workspace_and_missing_device():
    import torch
    L = gdn.lib()
    p = _attn_params()
    assert L.gdn_gated_attention_workspace_bytes(ctypes.byref(p), 0) == 0
    n = L.gdn_gated_attention_workspace_bytes(ctypes.byref(p), 100)
    assert 2 * 100 * 18 * 256 <= n <= 2 * 100 * 18 * 256 + 512
    assert L.gdn_gated_attention_workspace_bytes(ctypes.byref(_attn_params(D=64)), 1) == \
        ctypes.c_size_t(-1).value
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    T = 100
    q, kv, o = _host(T * 16 * 256), _host(T * 2 * 256), _host(T * 16 * 256)
    raw = np.zeros(n + 512, dtype=np.uint8)
    addr = (raw.ctypes.data + 255) // 256 * 256
    ptr = lambda x: ctypes.c_void_p(x.ctypes.data)
    st = L.gdn_gated_attention(ptr(q), ptr(kv), ptr(kv), ptr(q), ctypes.byref(p), None, 1, T,
                               ptr(o), ctypes.c_void_p(addr), n, None)
    assert st == NO_DEVICE
    assert np.all(o == 7.0) and np.all(raw == 0)


def test_gated_attention_size_limit_is_reported_before_anything_else():
    """T * (Hq + Hkv) >= 2^27 is refused on the host (GDN_ERR_UNSUPPORTED), by the call and
    by the workspace query, before any pointer or device is looked at."""
    L = gdn.lib()
    p = _attn_params()
    T = (1 << 27) // 18 + 1
    assert L.gdn_gated_attention_workspace_bytes(ctypes.byref(p), T) == ctypes.c_size_t(-1).value
    assert L.gdn_gated_attention(None, None, None, None, ctypes.byref(p), None, 1, T, None, None,
                                 0, None) == 2
    assert "2^27" in L.gdn_last_error().decode()
    assert L.gdn_gated_attention_workspace_bytes(ctypes.byref(p), T - 1) != ctypes.c_size_t(-1).value

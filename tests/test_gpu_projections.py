"""GPU parity of the projections around the mixer (bf16 MFMA GEMMs) against the fp64
oracle's plain matrix products, and of the whole layer (in-projection, mixer, output
projection).

Bars: one GEMM output is rounded to bf16 once (2^-9 relative at most, ~1.6e-3 rms over
a tensor), with fp32 accumulation well below that: relative L2 <= 3e-3.  With small
integer inputs every product and partial sum is exact in fp32 and the result an
integer of at most 256, exact in bf16: then the GPU must match bit for bit, which pins
the operand layouts, the tiling and the column scatter exactly.  The layer rounds the
projected q, k, v, z (bf16) before the mixer, o after it and y at the end: three
roundings in sequence, each ~1.6e-3 rms, passed through the mixer's sensitivity to its
inputs; its bar is 1e-2 on y and on the final state (measured values are printed).
"""
import numpy as np
import pytest
import torch

import gdn_synth as S
import oracle

gpu = pytest.mark.gpu


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def _gdn():
    import linear_attention_sequence_causal_amd as gdn
    return gdn


def _rand(shape, seed, std=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * std).to(torch.bfloat16)


def _ints(shape, seed, lo=-2, hi=2):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(lo, hi + 1, shape, generator=g, device="cuda").to(torch.bfloat16)


@gpu
@pytest.mark.parametrize("M,N,K", [(1, 96, 64), (300, 200, 128), (1000, 2048, 2048),
                                   (513, 12352, 256), (257, 2048, 4096)])
def test_linear_matches_oracle(M, N, K):
    gdn = _gdn()
    x, w = _rand((M, K), 1000 + M), _rand((N, K), 2000 + N, K ** -0.5)
    y = gdn.linear(x, w)
    torch.cuda.synchronize()
    ref = oracle.linear(S.to_f64(x), S.to_f64(w))
    e = rel_l2(S.to_f64(y), ref)
    print(f"linear M={M} N={N} K={K}: rel-L2 {e:.3e}")
    assert e <= 3e-3


@gpu
@pytest.mark.parametrize("M,N,K", [(300, 200, 64), (1000, 4100, 128)])
def test_linear_integer_inputs_are_bitwise(M, N, K):
    """Inputs in {-2..2}: every product and sum is an integer below 2^8 in magnitude,
    exact in fp32 accumulation and in the bf16 output."""
    gdn = _gdn()
    x, w = _ints((M, K), 3000 + M, -1, 1), _ints((N, K), 4000 + N, -2, 2)
    y = gdn.linear(x, w)
    torch.cuda.synchronize()
    ref = oracle.linear(S.to_f64(x), S.to_f64(w))
    assert np.abs(ref).max() <= 256
    assert np.array_equal(S.to_f64(y), ref)


@gpu
@pytest.mark.parametrize("Hk,Hv", [(2, 4), (2, 32)])
def test_in_projection_scatters_into_the_mixer_inputs(Hk, Hv):
    """All six outputs against the oracle's split (bitwise with integer inputs), then
    random inputs.  With Hv = 4 the a and b column ranges are not multiples of the
    32-column tile (the per-lane epilogue); with Hv = 32 every range is, and the epilogue
    stores each tile through one buffer (bf16 q, k, v, z and fp32 a, b)."""
    gdn = _gdn()
    T, d_model, D = 333, 192, 128
    n_in = 2 * Hk * D + 2 * Hv * D + 2 * Hv
    x, w = _ints((T, d_model), 5000, -1, 1), _ints((n_in, d_model), 5001, -1, 1)
    outs = gdn.in_projection(x, w, Hk, Hv, D)
    torch.cuda.synchronize()
    refs = oracle.in_projection(S.to_f64(x), S.to_f64(w), Hk, Hv, D)
    for name, o, r in zip("qkvzab", outs, refs):
        assert np.array_equal(S.to_f64(o), r), name
    x, w = _rand((T, d_model), 5002), _rand((n_in, d_model), 5003, d_model ** -0.5)
    outs = gdn.in_projection(x, w, Hk, Hv, D)
    torch.cuda.synchronize()
    refs = oracle.in_projection(S.to_f64(x), S.to_f64(w), Hk, Hv, D)
    for name, o, r in zip("qkvzab", outs, refs):
        e = rel_l2(S.to_f64(o), r)
        assert e <= (3e-3 if o.dtype == torch.bfloat16 else 1e-5), (name, e)


@gpu
def test_layer_matches_oracle():
    """x -> in-projection -> mixer (prefill) -> output projection on the GPU against the
    oracle's fp64 layer."""
    gdn = _gdn()
    w = S.scaled(S.LAYER_64K, lengths=(1000,), num_qk_heads=2, num_v_heads=4, seed=55)
    d = S.layer_inputs(w, 256, "cuda")
    Hk, Hv, D = 2, 4, 128
    q, k, v, z, a, b = gdn.in_projection(d["x"], d["w_in"], Hk, Hv, D)
    o, fs = gdn.prefill(q, k, v, a, b, z, d["conv_w"], d["A_log"], d["dt_bias"], d["norm_w"],
                        init_state=d["init_state"])
    y = gdn.out_projection(o, d["w_out"])
    torch.cuda.synchronize()
    f = S.to_f64
    y_ref, fs_ref, _ = oracle.gdn_layer(f(d["x"]), f(d["w_in"]), f(d["w_out"]), f(d["conv_w"]),
                                        f(d["A_log"]), f(d["dt_bias"]), f(d["norm_w"]), Hk, Hv,
                                        D, init_state=f(d["init_state"]))
    ey, es = rel_l2(f(y), y_ref), rel_l2(f(fs), fs_ref)
    print(f"layer T=1000 d_model=256: y rel-L2 {ey:.3e} final-state rel-L2 {es:.3e}")
    assert ey <= 1e-2 and es <= 1e-2


@gpu
def test_projections_full_size_sampled_rows():
    """The benchmark's projections (T = 65536, d_model = 2048, 16/32 heads) in their
    launch configuration; the oracle recomputes 96 sampled tokens' rows (each row of a
    product depends on that token's row of x only)."""
    gdn = _gdn()
    d = S.layer_inputs(S.LAYER_64K, 2048, "cuda")
    Hk, Hv, D = 16, 32, 128
    outs = gdn.in_projection(d["x"], d["w_in"], Hk, Hv, D)
    o = _rand((65536, Hv, D), 6000)
    y = gdn.out_projection(o, d["w_out"])
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(6001)
    rows = torch.randperm(65536, generator=g)[:96].sort().values.cuda()
    f = S.to_f64
    refs = oracle.in_projection(f(d["x"].index_select(0, rows)), f(d["w_in"]), Hk, Hv, D)
    for name, out, r in zip("qkvzab", outs, refs):
        e = rel_l2(f(out.index_select(0, rows)), r)
        assert e <= 3e-3, (name, e)
    y_ref = oracle.linear(f(o.index_select(0, rows).reshape(96, Hv * D)), f(d["w_out"]))
    e = rel_l2(f(y.index_select(0, rows)), y_ref)
    print(f"out projection T=65536 sampled rows: rel-L2 {e:.3e}")
    assert e <= 3e-3

"""Seeded synthetic inputs for the Gated DeltaNet mixer workloads.

This module only draws random numbers; it holds none of the mixer's arithmetic.
Both the GPU path's tests/benchmark and the fp64 oracle take their inputs from
here (the oracle receives exact float64 copies of the same tensors).

Recipe (one generator per workload, seeded with the workload's seed; draws in
this fixed order, each as a whole row-major tensor):
  1. sequence lengths (varlen workload only): L_i = floor(exp(U(ln 128, ln 32768)))
  2. conv weights [Cc, 4] ~ N(0, 1/4)        (standard deviation 0.5)
  3. A_log [Hv] ~ U(0, ln 16)
  4. dt_bias [Hv] ~ U(-1, 1)
  5. initial state [N, Hv, D, D] ~ N(0, 0.01^2), or zeros
  6. conv history [N, 3, Cc] ~ N(0, 1) (decode cache), or none
  7. q, k, v, z ~ N(0, 1), a, b ~ N(0, 1), each [T, ...] token-major
Activations are drawn in fp32 and rounded to bf16 with round-to-nearest-even
(torch's conversion) when the workload is bf16; gates, parameters and states
stay fp32.  The norm weight is all ones.  Draws use torch.Generator on the
device the tensors live on, so large workloads are generated in HBM directly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_qk_heads: int = 16
    num_v_heads: int = 32
    head_dim: int = 128
    act_dtype: torch.dtype = torch.bfloat16
    lengths: tuple = ()           # prefill: per-sequence lengths (filled for varlen on draw)
    varlen: int = 0               # >0: number of log-uniform sequences to draw
    init_state_std: float = 0.0   # 0 => zero initial state
    decode_batch: int = 0         # >0: decode workload with this batch
    decode_steps: int = 0
    conv_history: bool = False

    @property
    def conv_channels(self) -> int:
        return 2 * self.num_qk_heads * self.head_dim + self.num_v_heads * self.head_dim


TINY = Workload("tiny_T512_hk1_hv2_fp32", seed=0, num_qk_heads=1, num_v_heads=2,
                act_dtype=torch.float32, lengths=(512,))
PREFILL_4K = Workload("prefill_T4096_hk16_hv32_bf16", seed=1, lengths=(4096,))
PREFILL_64K = Workload("prefill_T65536_hk16_hv32_bf16", seed=2, lengths=(65536,),
                       init_state_std=0.01)
DECODE_B256 = Workload("decode_B256_hk16_hv32_bf16_1000steps", seed=3, decode_batch=256,
                       decode_steps=1000, init_state_std=0.01, conv_history=True)
VARLEN_64 = Workload("varlen_N64_len128to32768_hk16_hv32_bf16", seed=4, varlen=64,
                     init_state_std=0.01)

ALL = (TINY, PREFILL_4K, PREFILL_64K, DECODE_B256, VARLEN_64)


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller test cases)."""
    return replace(w, **kw)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device, std=1.0):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _uniform(shape, lo, hi, g, device):
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def draw_lengths(n: int, g, device) -> list:
    u = _uniform((n,), math.log(128.0), math.log(32768.0), g, device).double().cpu()
    return [int(math.floor(math.exp(x))) for x in u.tolist()]


def prefill_inputs(w: Workload, device="cpu") -> dict:
    """All inputs of one prefill workload as torch tensors on `device`."""
    g = _gen(w.seed, device)
    lengths = list(w.lengths)
    if w.varlen:
        lengths = draw_lengths(w.varlen, g, device)
    N = len(lengths)
    T = int(sum(lengths))
    Hk, Hv, D = w.num_qk_heads, w.num_v_heads, w.head_dim
    Cc = w.conv_channels
    conv_w = _normal((Cc, 4), g, device, std=0.5)
    A_log = _uniform((Hv,), 0.0, math.log(16.0), g, device)
    dt_bias = _uniform((Hv,), -1.0, 1.0, g, device)
    if w.init_state_std > 0:
        init_state = _normal((N, Hv, D, D), g, device, std=w.init_state_std)
    else:
        init_state = None
    conv_in = _normal((N, 3, Cc), g, device).to(w.act_dtype) if w.conv_history else None
    q = _normal((T, Hk, D), g, device).to(w.act_dtype)
    k = _normal((T, Hk, D), g, device).to(w.act_dtype)
    v = _normal((T, Hv, D), g, device).to(w.act_dtype)
    z = _normal((T, Hv, D), g, device).to(w.act_dtype)
    a = _normal((T, Hv), g, device)
    b = _normal((T, Hv), g, device)
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    return dict(q=q, k=k, v=v, a=a, b=b, z=z, conv_w=conv_w, A_log=A_log, dt_bias=dt_bias,
                norm_w=torch.ones(D, device=device, dtype=torch.float32),
                init_state=init_state, conv_in=conv_in,
                cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device),
                lengths=lengths)


LAYER_64K = Workload("layer_T65536_d2048_hk16_hv32_bf16", seed=5, lengths=(65536,),
                     init_state_std=0.01)


def layer_inputs(w: Workload, d_model: int, device="cpu") -> dict:
    """Inputs of a whole layer (in-projection, mixer, output projection): the mixer's
    parameters and initial state as prefill_inputs draws them (steps 1-5), then hidden
    states x [T, d_model] ~ N(0, 1), w_in [2HkD + 2HvD + 2Hv, d_model] ~ N(0, 1/d_model)
    (so the projected q, k, v, z, a, b are ~ N(0, 1) as in the other workloads) and
    w_out [d_model, Hv*D] ~ N(0, 1/(Hv*D)), all rounded to bf16."""
    g = _gen(w.seed, device)
    T = int(sum(w.lengths))
    Hk, Hv, D = w.num_qk_heads, w.num_v_heads, w.head_dim
    Cc = w.conv_channels
    conv_w = _normal((Cc, 4), g, device, std=0.5)
    A_log = _uniform((Hv,), 0.0, math.log(16.0), g, device)
    dt_bias = _uniform((Hv,), -1.0, 1.0, g, device)
    init_state = (_normal((1, Hv, D, D), g, device, std=w.init_state_std)
                  if w.init_state_std > 0 else None)
    n_in = 2 * Hk * D + 2 * Hv * D + 2 * Hv
    x = _normal((T, d_model), g, device).to(torch.bfloat16)
    w_in = _normal((n_in, d_model), g, device, std=d_model ** -0.5).to(torch.bfloat16)
    w_out = _normal((d_model, Hv * D), g, device, std=(Hv * D) ** -0.5).to(torch.bfloat16)
    return dict(x=x, w_in=w_in, w_out=w_out, conv_w=conv_w, A_log=A_log, dt_bias=dt_bias,
                norm_w=torch.ones(D, device=device, dtype=torch.float32),
                init_state=init_state, d_model=d_model)


@dataclass(frozen=True)
class AttnWorkload:
    """Inputs of the hybrid's gated full-attention layer: 16 query heads over 2 key/value
    heads of dim 256, RoPE on 64 dims."""
    name: str
    seed: int
    lengths: tuple = ()
    varlen: int = 0               # >0: number of log-uniform sequences to draw
    num_q_heads: int = 16
    num_kv_heads: int = 2
    head_dim: int = 256
    rotary_dim: int = 64


ATTN_64K = AttnWorkload("attn_T65536_hq16_hkv2_d256_bf16", seed=6, lengths=(65536,))
ATTN_4K = AttnWorkload("attn_T4096_hq16_hkv2_d256_bf16", seed=7, lengths=(4096,))
ATTN_VARLEN = AttnWorkload("attn_varlen_N64_len128to32768_hq16_hkv2_d256_bf16", seed=8,
                           varlen=64)


def attention_inputs(w: AttnWorkload, device="cpu") -> dict:
    """Inputs of one attention workload.  Draws, in this order: sequence lengths (varlen
    only, as draw_lengths), the QK-Norm weights [D] ~ 1 + N(0, 0.1^2) (q, then k), then
    q [T, Hq, D], k [T, Hkv, D], v [T, Hkv, D], gate [T, Hq, D] ~ N(0, 1) rounded to bf16."""
    g = _gen(w.seed, device)
    lengths = draw_lengths(w.varlen, g, device) if w.varlen else list(w.lengths)
    T = int(sum(lengths))
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    q_norm_w = 1.0 + _normal((D,), g, device, std=0.1)
    k_norm_w = 1.0 + _normal((D,), g, device, std=0.1)
    q = _normal((T, Hq, D), g, device).to(torch.bfloat16)
    k = _normal((T, Hkv, D), g, device).to(torch.bfloat16)
    v = _normal((T, Hkv, D), g, device).to(torch.bfloat16)
    gate = _normal((T, Hq, D), g, device).to(torch.bfloat16)
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    return dict(q=q, k=k, v=v, gate=gate, q_norm_w=q_norm_w, k_norm_w=k_norm_w,
                cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device),
                lengths=lengths, rotary_dim=w.rotary_dim)


def decode_setup(w: Workload, device="cpu") -> dict:
    """Parameters, initial per-sequence state and conv cache of a decode workload."""
    g = _gen(w.seed, device)
    B, Hk, Hv, D = w.decode_batch, w.num_qk_heads, w.num_v_heads, w.head_dim
    Cc = w.conv_channels
    conv_w = _normal((Cc, 4), g, device, std=0.5)
    A_log = _uniform((Hv,), 0.0, math.log(16.0), g, device)
    dt_bias = _uniform((Hv,), -1.0, 1.0, g, device)
    state = _normal((B, Hv, D, D), g, device, std=w.init_state_std)
    conv_cache = _normal((B, 3, Cc), g, device).to(w.act_dtype)
    return dict(conv_w=conv_w, A_log=A_log, dt_bias=dt_bias,
                norm_w=torch.ones(D, device=device, dtype=torch.float32),
                state=state, conv_cache=conv_cache, gen=g)


def decode_tokens(w: Workload, setup: dict, steps: int, device="cpu") -> dict:
    """Token inputs of `steps` consecutive decode steps, stacked on a leading
    step axis: q, k [S, B, Hk, D], v, z [S, B, Hv, D], a, b [S, B, Hv].
    Continues the workload's generator after decode_setup."""
    g = setup["gen"]
    B, Hk, Hv, D = w.decode_batch, w.num_qk_heads, w.num_v_heads, w.head_dim
    q = _normal((steps, B, Hk, D), g, device).to(w.act_dtype)
    k = _normal((steps, B, Hk, D), g, device).to(w.act_dtype)
    v = _normal((steps, B, Hv, D), g, device).to(w.act_dtype)
    z = _normal((steps, B, Hv, D), g, device).to(w.act_dtype)
    a = _normal((steps, B, Hv), g, device)
    b = _normal((steps, B, Hv), g, device)
    return dict(q=q, k=k, v=v, z=z, a=a, b=b)


def to_f64(t):
    """Exact float64 numpy copy of a tensor (None passes through)."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()

"""The chunk-form (WY/UT) identities equal the token-by-token recurrence.

The chunk form is what the GPU prefill computes; here it is an independent
fp64 NumPy model (oracle/chunk_form.py) checked against the C oracle to 1e-12
for several chunk sizes, partial tail chunks, initial states and extreme gates.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.chunk_form import chunk_recurrence


def _case(rng, T, D, gate="typical"):
    k = rng.standard_normal((T, D))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((T, D))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    v = rng.standard_normal((T, D))
    if gate == "typical":
        a = rng.standard_normal(T)
        A_log = rng.uniform(0, math.log(16))
        dt = rng.uniform(-1, 1)
    elif gate == "slow":
        a = rng.standard_normal(T) - 4.0
        A_log = math.log(0.01)
        dt = 0.0
    else:  # "mixed": saturating gates
        a = rng.standard_normal(T) * 8.0
        A_log = rng.uniform(-3, 3)
        dt = 0.0
    b = rng.standard_normal(T) * (1.0 if gate != "mixed" else 10.0)
    alpha, beta = oracle.gates(a, b, A_log, dt)
    return q, k, v, alpha, beta


@pytest.mark.parametrize("chunk", [1, 16, 32, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("gate", ["typical", "slow", "mixed"])
def test_chunk_form_matches_recurrence(chunk, T, gate):
    rng = np.random.default_rng(1000 * chunk + T + len(gate))
    D = 32
    q, k, v, alpha, beta = _case(rng, T, D, gate)
    H0 = rng.standard_normal((D, D)) * 0.1
    y_ref, S_ref = oracle.recurrence(alpha, beta, q, k, v, S0=H0.T)
    with np.errstate(divide="ignore"):
        g = np.log(alpha)
    y, H = chunk_recurrence(g, beta, q, k, v, H0=H0, chunk=chunk)
    scale_y = max(1.0, np.abs(y_ref).max())
    np.testing.assert_allclose(y, y_ref, atol=1e-12 * scale_y)
    np.testing.assert_allclose(H, S_ref.T, atol=1e-12 * max(1.0, np.abs(S_ref).max()))

"""The chunkwise form (oracle/chunked_ref.py) equals the token-by-token oracle.

This pins the reading of the chunk equations that the GPU kernels implement
(direction of the decays, beta in W and U, strict mask for A, inclusive mask for
the output) before any GPU code is involved.  C = 1 collapses to the recurrence.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import chunked_ref


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(B, T, H, dk, dv, gate, seed, la_const=None):
    r = np.random.default_rng(seed)
    q = unit(r.standard_normal((B, T, H, dk)))
    k = unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    if gate == "head":
        la = -np.log1p(np.exp(r.standard_normal((B, T, H)))) * np.exp(r.uniform(-3, 0, (B, T, H)))
    elif gate == "key":
        la = -np.log1p(np.exp(r.standard_normal((B, T, H, dk))))
    else:
        la = None
    if la_const is not None:
        la = np.full_like(la, la_const)
    s0 = r.standard_normal((B, H, dk, dv)) * 0.3
    return q, k, v, beta, la, s0


@pytest.mark.parametrize("gate", ["none", "head", "key"])
@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
@pytest.mark.parametrize("dk,dv,T", [(16, 8, 200), (8, 16, 77), (12, 12, 64)])
def test_chunked_equals_recurrence(gate, chunk, dk, dv, T):
    q, k, v, beta, la, s0 = case(2, T, 2, dk, dv, gate, seed=chunk * 1000 + dk + T)
    o_ref, f_ref = oracle.fwd(q, k, v, beta, la, s0, gate=gate)
    o_c, f_c = chunked_ref.fwd(q, k, v, beta, la, s0, chunk=chunk)
    scale = max(np.abs(o_ref).max(), 1.0)
    np.testing.assert_allclose(o_c, o_ref, atol=1e-12 * scale, rtol=0)
    np.testing.assert_allclose(f_c, f_ref, atol=1e-12 * max(np.abs(f_ref).max(), 1.0), rtol=0)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_chunked_adversarial_gate(gate):
    """log alpha = -5 on every step: the whole-chunk log decay reaches -320; the
    chunk form must not overflow (every exponent it takes is <= 0)."""
    q, k, v, beta, la, s0 = case(1, 130, 1, 16, 8, gate, seed=9, la_const=-5.0)
    o_ref, f_ref = oracle.fwd(q, k, v, beta, la, s0, gate=gate)
    o_c, f_c = chunked_ref.fwd(q, k, v, beta, la, s0, chunk=64)
    assert np.isfinite(o_c).all() and np.isfinite(f_c).all()
    np.testing.assert_allclose(o_c, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(f_c, f_ref, atol=1e-12, rtol=0)


def test_ut_inverse_is_a_triangular_solve():
    r = np.random.default_rng(0)
    A = np.tril(r.standard_normal((64, 64)) * 0.2, -1)
    T = chunked_ref.forward_substitution_inverse(A)
    np.testing.assert_allclose((np.eye(64) + A) @ T, np.eye(64), atol=1e-12)
    np.testing.assert_allclose(T, scipy.linalg.solve_triangular(np.eye(64) + A, np.eye(64), lower=True),
                               atol=1e-12)


def test_chunk_cumsum_matches_numpy():
    x = np.random.default_rng(1).standard_normal((64, 5))
    np.testing.assert_allclose(chunked_ref.chunk_cumsum(x), np.cumsum(x, axis=0), atol=1e-14)


def test_dropping_beta_from_U_is_detected():
    """Reading W = T K, U = T V literally (without beta) breaks equality with the recurrence."""
    q, k, v, beta, la, s0 = case(1, 64, 1, 8, 8, "head", seed=4)
    o_ref, _ = oracle.fwd(q, k, v, beta, la, s0)
    G = np.repeat(np.cumsum(la[0, :, 0])[:, None], 8, axis=1)
    res = chunked_ref.chunk_step(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], G, s0[0, 0])
    np.testing.assert_allclose(res["O"], o_ref[0, :, 0], atol=1e-12)
    U_wrong = res["T"] @ v[0, :, 0]
    W_wrong = res["T"] @ (k[0, :, 0] * np.exp(G))
    D_wrong = U_wrong - W_wrong @ s0[0, 0]
    O_wrong = (q[0, :, 0] * np.exp(G)) @ s0[0, 0] + res["P"] @ D_wrong
    assert np.abs(O_wrong - o_ref[0, :, 0]).max() > 1e-3

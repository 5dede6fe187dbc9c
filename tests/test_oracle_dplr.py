"""Pins for the oracle's diagonal-plus-low-rank transition (oracle.fwd_dplr):
  - with b = k and a = -alpha beta k, and v scaled by beta, it is the (gated) delta
    rule of oracle.fwd (the delta rule's transition alpha (I - beta k k^T) is
    Diag(alpha) plus that rank-one term);
  - with a = 0 (no low-rank term) it is the additive write of oracle.fwd;
  - it equals the product of the dense transition matrices Diag(alpha_t) + b_t a_t^T
    applied to the initial state, plus the dense sum of the writes, for every
    output and the final state (per-channel decays included).
"""
import numpy as np
import pytest

import oracle


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(B, T, H, dk, dv, gate, seed):
    r = np.random.default_rng(seed)
    q, k = unit(r.standard_normal((B, T, H, dk))), unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    la = None if gate == "none" else (-np.log1p(np.exp(r.standard_normal((B, T, H)))) if gate == "head"
                                      else -np.log1p(np.exp(r.standard_normal((B, T, H, dk)))))
    s0 = r.standard_normal((B, H, dk, dv)) * 0.5
    return q, k, v, beta, la, s0


@pytest.mark.parametrize("gate", ["none", "head"])
def test_reduces_to_delta_rule(gate):
    q, k, v, beta, la, s0 = case(2, 37, 3, 6, 4, gate, seed=1)
    alpha = np.ones_like(beta) if la is None else np.exp(la)
    a = -(alpha * beta)[..., None] * k
    o1, f1 = oracle.fwd_dplr(q, k, beta[..., None] * v, a, k, la, s0)
    o2, f2 = oracle.fwd(q, k, v, beta, la, s0)
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(f1, f2, atol=1e-12, rtol=0)


@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_no_low_rank_term_is_additive_write(gate):
    q, k, v, beta, la, s0 = case(2, 29, 2, 5, 3, gate, seed=2)
    b = np.random.default_rng(3).standard_normal(q.shape)
    o1, f1 = oracle.fwd_dplr(q, k, v, np.zeros_like(q), b, la, s0)
    o2, f2 = oracle.fwd(q, k, v, None, la, s0, write="add")
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(f1, f2, atol=1e-12, rtol=0)


@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_equals_dense_transition_products(gate):
    T, dk, dv = 9, 4, 3
    q, k, v, beta, la, s0 = case(1, T, 1, dk, dv, gate, seed=4)
    r = np.random.default_rng(5)
    a, b = r.standard_normal(q.shape) * 0.5, r.standard_normal(q.shape) * 0.5
    o, fs = oracle.fwd_dplr(q, k, v, a, b, la, s0)
    if la is None:
        alpha = np.ones((T, dk))
    elif la.ndim == 3:
        alpha = np.repeat(np.exp(la[0, :, 0])[:, None], dk, axis=1)
    else:
        alpha = np.exp(la[0, :, 0])
    # S_t = S_{t-1} Q_t + v_t k_t^T with Q_t = Diag(alpha_t) + a_t b_t^T, S = M^T
    S = s0[0, 0].T.copy()
    for t in range(T):
        Qt = np.diag(alpha[t]) + np.outer(a[0, t, 0], b[0, t, 0])
        S = S @ Qt + np.outer(v[0, t, 0], k[0, t, 0])
        np.testing.assert_allclose(o[0, t, 0], S @ q[0, t, 0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(fs[0, 0], S.T, atol=1e-12, rtol=0)


def test_constant_gate_is_per_token_broadcast():
    """One constant decay per head ([H]) equals the same value given at every token."""
    q, k, v, beta, la, s0 = case(2, 21, 3, 5, 4, "none", seed=11)
    r = np.random.default_rng(12)
    a, b = r.standard_normal(q.shape) * 0.4, r.standard_normal(q.shape) * 0.4
    g = np.log(np.array([0.9, 0.75, 0.99]))
    o1, f1 = oracle.fwd_dplr(q, k, v, a, b, g, s0)
    o2, f2 = oracle.fwd_dplr(q, k, v, a, b, np.broadcast_to(g, (2, 21, 3)).copy(), s0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(f1, f2)


@pytest.mark.parametrize("C", [1, 5, 16, 64])
@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_chunked_form_equals_recurrence(C, gate):
    """The chunk equations (oracle/chunked_ref.py: chunk_step_dplr) that the GPU kernel
    implements, against the token recurrence."""
    from oracle import chunked_ref
    T, dk, dv = 150, 8, 5
    q, k, v, beta, la, s0 = case(1, T, 1, dk, dv, gate, seed=C + 7)
    r = np.random.default_rng(C)
    a, b = unit(r.standard_normal(q.shape)) * -0.6, unit(r.standard_normal(q.shape))
    o, fs = oracle.fwd_dplr(q, k, v, a, b, la, s0)
    oc, mc = chunked_ref.chunked_dplr(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0],
                                      None if la is None else la[0, :, 0], s0[0, 0], C=C)
    np.testing.assert_allclose(oc, o[0, :, 0], atol=1e-10, rtol=1e-10)
    np.testing.assert_allclose(mc, fs[0, 0], atol=1e-10, rtol=1e-10)

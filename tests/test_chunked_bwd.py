"""The chunkwise gradients (oracle/chunked_ref.py: chunk_step_bwd, chunked_bwd) equal
the token-level gradients of the pinned oracle (oracle.bwd) for several chunk
lengths, ragged lengths and strong decays: this fixes the chunk equations of the
backward that the GPU kernels implement."""
import numpy as np
import pytest

import oracle
from oracle import chunked_ref


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


@pytest.mark.parametrize("C", [1, 3, 16, 64])
@pytest.mark.parametrize("gate", ["none", "head"])
@pytest.mark.parametrize("T", [1, 40, 130])
def test_chunked_gradients_equal_token_gradients(C, gate, T):
    r = np.random.default_rng(T * 7 + C)
    dk, dv = 8, 5
    q, k = unit(r.standard_normal((T, dk))), unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal(T)))
    la = None if gate == "none" else -np.log1p(np.exp(r.standard_normal(T))) * 2.0
    M0 = r.standard_normal((dk, dv)) * 0.5
    dO, dMT = r.standard_normal((T, dv)), r.standard_normal((dk, dv))
    got = chunked_ref.chunked_bwd(q, k, v, beta, la, M0, dO, dMT, C=C)
    ref = oracle.bwd(q[None, :, None], k[None, :, None], v[None, :, None], beta[None, :, None],
                     None if la is None else la[None, :, None], M0[None, None], dO[None, :, None], dMT[None, None])
    names = ["dq", "dk", "dv", "dbeta", "dlog_alpha", "dM0"]
    refs = [ref[0][0, :, 0], ref[1][0, :, 0], ref[2][0, :, 0], ref[3][0, :, 0],
            None if la is None else ref[4][0, :, 0], ref[5][0, 0]]
    for name, g, rr in zip(names, got, refs):
        if rr is None:
            continue
        np.testing.assert_allclose(g, rr, atol=1e-10, rtol=1e-10, err_msg=name)


@pytest.mark.parametrize("C", [1, 3, 16, 64])
@pytest.mark.parametrize("gate", ["none", "head"])
@pytest.mark.parametrize("T", [1, 40, 130])
def test_chunked_additive_gradients_equal_token_gradients(C, gate, T):
    """The additive write's chunk adjoint (Delta = V, no A or T) against oracle.bwd."""
    r = np.random.default_rng(T * 11 + C)
    dk, dv = 7, 5
    q, k = unit(r.standard_normal((T, dk))), unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    la = None if gate == "none" else -np.log1p(np.exp(r.standard_normal(T))) * 2.0
    M0 = r.standard_normal((dk, dv)) * 0.5
    dO, dMT = r.standard_normal((T, dv)), r.standard_normal((dk, dv))
    got = chunked_ref.chunked_bwd(q, k, v, None, la, M0, dO, dMT, C=C, write="add")
    ref = oracle.bwd(q[None, :, None], k[None, :, None], v[None, :, None], None,
                     None if la is None else la[None, :, None], M0[None, None], dO[None, :, None], dMT[None, None],
                     write="add")
    names = ["dq", "dk", "dv", "dlog_alpha", "dM0"]
    refs = [ref[0][0, :, 0], ref[1][0, :, 0], ref[2][0, :, 0], None if la is None else ref[4][0, :, 0], ref[5][0, 0]]
    gots = [got[0], got[1], got[2], got[4], got[5]]
    for name, g, rr in zip(names, gots, refs):
        if rr is None:
            continue
        np.testing.assert_allclose(g, rr, atol=1e-10, rtol=1e-10, err_msg=name)

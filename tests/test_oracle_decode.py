"""Pins for the pooled multi-token decode of the oracle (oracle.decode_pool).

decode_pool composes the per-token recurrence (oracle_step).  These tests tie it to
the whole-sequence recurrence (oracle_fwd), a separate code path that the pins in
test_oracle_pins.py fix against the pages: L tokens from a pool slot give the same
outputs and final state as a forward pass over those L tokens, each stored
intermediate state equals the forward pass over that prefix, calls chain, and a
speculative continuation from an accepted prefix equals the forward pass over the
accepted tokens followed by the new ones.  Padding streams read and write nothing.
"""
import numpy as np
import pytest

import oracle


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def tokens(N, L, H, dk, dv, gate, seed):
    r = np.random.default_rng(seed)
    q = unit(r.standard_normal((N, L, H, dk)))
    k = unit(r.standard_normal((N, L, H, dk)))
    v = r.standard_normal((N, L, H, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((N, L, H))))
    if gate == "head":
        la = -np.log1p(np.exp(r.standard_normal((N, L, H))))
    elif gate == "key":
        la = -np.log1p(np.exp(r.standard_normal((N, L, H, dk))))
    else:
        la = None
    return q, k, v, beta, la


def sl(x, n, t0, t1):
    return None if x is None else x[n:n + 1, t0:t1]


def fwd_stream(q, k, v, beta, la, n, t0, t1, s0, gate):
    """oracle_fwd over tokens [t0, t1) of stream n (as a batch of one)."""
    return oracle.fwd(sl(q, n, t0, t1), sl(k, n, t0, t1), sl(v, n, t0, t1), sl(beta, n, t0, t1),
                      sl(la, n, t0, t1), s0[None], gate=gate)


@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_pool_decode_matches_forward_and_prefixes(gate):
    N, L, H, dk, dv, P = 5, 4, 2, 6, 3, 40
    q, k, v, beta, la = tokens(N, L, H, dk, dv, gate, seed=7)
    pool = np.random.default_rng(1).standard_normal((P, H, dk, dv))
    src = np.array([3, 17, -1, 0, 39])           # stream 2 is padding
    dst = 20 + np.arange(N * L).reshape(N, L)    # every intermediate state stored
    dst[1, 2] = -1                               # ... except this one
    dst[4, 3] = P                                # out of range: not stored
    o, out = oracle.decode_pool(q, k, v, beta, la, pool, src, dst, gate=gate)
    written = set()
    for n in range(N):
        if src[n] < 0:
            assert np.isnan(o[n]).all()
            continue
        of, ff = fwd_stream(q, k, v, beta, la, n, 0, L, pool[src[n]], gate)
        np.testing.assert_allclose(o[n], of[0], atol=1e-13, rtol=0)
        for t in range(L):
            if 0 <= dst[n, t] < P:
                _, fp = fwd_stream(q, k, v, beta, la, n, 0, t + 1, pool[src[n]], gate)
                np.testing.assert_allclose(out[dst[n, t]], fp[0], atol=1e-13, rtol=0)
                written.add(int(dst[n, t]))
        if 0 <= dst[n, L - 1] < P:
            np.testing.assert_allclose(out[dst[n, L - 1]], ff[0], atol=1e-13, rtol=0)
    for s in range(P):
        if s not in written:
            np.testing.assert_array_equal(out[s], pool[s])


def test_pool_decode_in_place_and_no_store():
    N, L, H, dk, dv, P = 3, 2, 1, 4, 4, 3
    q, k, v, beta, la = tokens(N, L, H, dk, dv, "head", seed=9)
    pool = np.random.default_rng(2).standard_normal((P, H, dk, dv))
    src = np.array([2, 0, 1])
    none = np.full((N, L), -1)
    o1, out1 = oracle.decode_pool(q, k, v, beta, la, pool, src, none)
    np.testing.assert_array_equal(out1, pool)          # nothing stored
    dst = none.copy()
    dst[:, -1] = src                                   # in place: last state back to its slot
    o2, out2 = oracle.decode_pool(q, k, v, beta, la, pool, src, dst)
    np.testing.assert_array_equal(o1, o2)              # outputs do not depend on the stores
    for n in range(N):
        _, ff = fwd_stream(q, k, v, beta, la, n, 0, L, pool[src[n]], "head")
        np.testing.assert_allclose(out2[src[n]], ff[0], atol=1e-13, rtol=0)
    # the slots are read before they are written: a rotation of the slots
    dst_rot = none.copy()
    dst_rot[:, -1] = np.roll(src, 1)
    _, out3 = oracle.decode_pool(q, k, v, beta, la, pool, src, dst_rot)
    for n in range(N):
        _, ff = fwd_stream(q, k, v, beta, la, n, 0, L, pool[src[n]], "head")
        np.testing.assert_allclose(out3[dst_rot[n, -1]], ff[0], atol=1e-13, rtol=0)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_speculative_accept_and_continue(gate):
    """Draft L tokens with every state stored; accept j of them; continue from the
    accepted state's slot: equals the forward pass over the accepted tokens followed
    by the next ones."""
    N, L, H, dk, dv = 4, 4, 2, 5, 3
    P = N + N * L
    q, k, v, beta, la = tokens(N, 2 * L, H, dk, dv, gate, seed=11)
    pool = np.random.default_rng(3).standard_normal((P, H, dk, dv)) * 0.5
    src = np.arange(N)
    dst = N + np.arange(N * L).reshape(N, L)
    first = (slice(None), slice(0, L))
    _, pool1 = oracle.decode_pool(q[first], k[first], v[first], beta[first], None if la is None else la[first],
                                  pool, src, dst, gate=gate)
    accepted = np.array([0, 1, 3, 2])  # index of the last accepted draft token per stream
    src2 = dst[np.arange(N), accepted]
    nxt = (slice(None), slice(L, 2 * L))
    o2, pool2 = oracle.decode_pool(q[nxt], k[nxt], v[nxt], beta[nxt], None if la is None else la[nxt],
                                   pool1, src2, np.full((N, L), -1), gate=gate)
    for n in range(N):
        j = accepted[n] + 1
        # accepted tokens 0..j-1, then the L new tokens
        idx = list(range(j)) + list(range(L, 2 * L))
        pick = lambda x: None if x is None else x[n:n + 1, idx]
        of, _ = oracle.fwd(pick(q), pick(k), pick(v), pick(beta), pick(la), pool[n][None], gate=gate)
        np.testing.assert_allclose(o2[n], of[0, j:], atol=1e-13, rtol=0)


def test_chained_calls_equal_one_forward():
    N, H, dk, dv = 2, 2, 4, 6
    q, k, v, beta, la = tokens(N, 7, H, dk, dv, "key", seed=13)
    pool = np.random.default_rng(5).standard_normal((N, H, dk, dv))
    src = np.arange(N)
    cur = pool
    outs = []
    for t0, t1 in [(0, 3), (3, 4), (4, 7)]:
        part = (slice(None), slice(t0, t1))
        dst = np.full((N, t1 - t0), -1)
        dst[:, -1] = src
        o, cur = oracle.decode_pool(q[part], k[part], v[part], beta[part], la[part], cur, src, dst)
        outs.append(o)
    o = np.concatenate(outs, axis=1)
    for n in range(N):
        of, ff = fwd_stream(q, k, v, beta, la, n, 0, 7, pool[n], "key")
        np.testing.assert_allclose(o[n], of[0], atol=1e-13, rtol=0)
        np.testing.assert_allclose(cur[n], ff[0], atol=1e-13, rtol=0)

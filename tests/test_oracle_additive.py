"""Pins for the oracle's additive write (write="add"): M_t = Diag(a_t) M_{t-1} + k_t v_t^T.

The pages state the additive family in closed form; each test compares the
token-by-token oracle with that closed form written out as a brute-force sum:
  - RetNet ("Linear Attention Variants", RetNet section): a fixed per-head decay
    gamma, parallel form (Q K^T * D) V with the decay mask D[t, i] = gamma^(t - i);
  - gated linear attention ("Decoding Hybrid Linear Attention Architectures",
    sec. 3 item 4; "Linear Attention Variants", GLA section): per-channel decays,
    so the (t, i) weight is sum_c q_t[c] k_i[c] prod_{i < j <= t} alpha_j[c];
  - the plain linear-transformer sum ("Linear Attention Variants", "The Shared
    Machinery"), no gate: O = Q M0 + tril(Q K^T) V.
Further: with orthonormal keys the delta rule at beta = 1 writes exactly what the
additive rule writes; the additive state is linear in (V, M0); and a mutant of the C
source that scales the additive write by beta is caught.
"""
import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle

rng = np.random.default_rng(2024)


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def tokens(T, H, dk, dv, seed):
    r = np.random.default_rng(seed)
    return (unit(r.standard_normal((1, T, H, dk))), unit(r.standard_normal((1, T, H, dk))),
            r.standard_normal((1, T, H, dv)), r.standard_normal((1, H, dk, dv)) * 0.5)


def test_retnet_decay_mask_parallel_form():
    T, H, dk, dv = 23, 3, 5, 4
    q, k, v, s0 = tokens(T, H, dk, dv, seed=1)
    gamma = 1.0 - 2.0 ** (-5.0 - np.arange(H))   # the per-head decays the RetNet passage gives
    o, fs = oracle.fwd(q, k, v, None, np.log(gamma), s0, write="add")
    for h in range(H):
        Q, K, V, g = q[0, :, h], k[0, :, h], v[0, :, h], gamma[h]
        t = np.arange(T)
        D = np.where(t[:, None] >= t[None, :], g ** (t[:, None] - t[None, :]).astype(float), 0.0)
        ref = (Q @ K.T * D) @ V + (g ** (t + 1))[:, None] * (Q @ s0[0, h])
        np.testing.assert_allclose(o[0, :, h], ref, atol=1e-12, rtol=0)
        MT = g ** T * s0[0, h] + sum(g ** (T - 1 - i) * np.outer(K[i], V[i]) for i in range(T))
        np.testing.assert_allclose(fs[0, h], MT, atol=1e-12, rtol=0)


def test_gla_per_channel_decay_brute_force():
    T, H, dk, dv = 17, 2, 6, 3
    q, k, v, s0 = tokens(T, H, dk, dv, seed=2)
    la = -np.log1p(np.exp(rng.standard_normal((1, T, H, dk))))
    o, fs = oracle.fwd(q, k, v, None, la, s0, write="add")
    for h in range(H):
        A = np.exp(la[0, :, h])  # [T, dk]
        for t in range(T):
            acc = (np.prod(A[:t + 1], axis=0) * q[0, t, h]) @ s0[0, h]
            for i in range(t + 1):
                w = q[0, t, h] * k[0, i, h] * np.prod(A[i + 1:t + 1], axis=0)
                acc = acc + w.sum() * v[0, i, h]
            np.testing.assert_allclose(o[0, t, h], acc, atol=1e-12, rtol=0)


def test_linear_transformer_sum():
    T, H, dk, dv = 12, 2, 4, 5
    q, k, v, s0 = tokens(T, H, dk, dv, seed=3)
    o, fs = oracle.fwd(q, k, v, None, None, s0, write="add")
    for h in range(H):
        Q, K, V = q[0, :, h], k[0, :, h], v[0, :, h]
        np.testing.assert_allclose(o[0, :, h], np.tril(Q @ K.T) @ V + Q @ s0[0, h], atol=1e-12, rtol=0)
        np.testing.assert_allclose(fs[0, h], s0[0, h] + K.T @ V, atol=1e-12, rtol=0)


@pytest.mark.parametrize("gate", ["none", "head"])
def test_orthonormal_keys_delta_at_beta_one_equals_add(gate):
    T, dk, dv = 6, 8, 3
    k = np.linalg.qr(rng.standard_normal((dk, dk)))[0][:T].reshape(1, T, 1, dk)
    q = unit(rng.standard_normal((1, T, 1, dk)))
    v = rng.standard_normal((1, T, 1, dv))
    la = None if gate == "none" else -np.abs(rng.standard_normal((1, T, 1))) * 0.3
    od, fd = oracle.fwd(q, k, v, np.ones((1, T, 1)), la, None, gate=gate)  # zero start: nothing to erase
    oa, fa = oracle.fwd(q, k, v, None, la, None, gate=gate, write="add")
    np.testing.assert_allclose(od, oa, atol=1e-12, rtol=0)
    np.testing.assert_allclose(fd, fa, atol=1e-12, rtol=0)


def test_additive_state_is_linear():
    T, H, dk, dv = 9, 2, 4, 4
    q, k, v, s0 = tokens(T, H, dk, dv, seed=5)
    v2, s2 = rng.standard_normal(v.shape), rng.standard_normal(s0.shape)
    la = -np.log1p(np.exp(rng.standard_normal((1, T, H, dk))))
    o1, f1 = oracle.fwd(q, k, v, None, la, s0, write="add")
    o2, f2 = oracle.fwd(q, k, v2, None, la, s2, write="add")
    o3, f3 = oracle.fwd(q, k, 2 * v - 3 * v2, None, la, 2 * s0 - 3 * s2, write="add")
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, atol=1e-12)
    np.testing.assert_allclose(f3, 2 * f1 - 3 * f2, atol=1e-12)


def test_const_gate_equals_broadcast_head_gate():
    T, H, dk, dv = 7, 3, 4, 4
    q, k, v, s0 = tokens(T, H, dk, dv, seed=6)
    beta = rng.uniform(0.1, 0.9, (1, T, H))
    lg = np.log(np.array([0.5, 0.9, 0.99]))
    for write in ("delta", "add"):
        b = beta if write == "delta" else None
        oc, fc = oracle.fwd(q, k, v, b, lg, s0, write=write)
        oh, fh = oracle.fwd(q, k, v, b, np.broadcast_to(lg, (1, T, H)).copy(), s0, write=write)
        np.testing.assert_array_equal(oc, oh)
        np.testing.assert_array_equal(fc, fh)


def test_step_and_pool_decode_additive():
    N, L, H, dk, dv = 3, 4, 2, 5, 3
    r = np.random.default_rng(7)
    q, k = unit(r.standard_normal((N, L, H, dk))), unit(r.standard_normal((N, L, H, dk)))
    v = r.standard_normal((N, L, H, dv))
    la = -np.log1p(np.exp(r.standard_normal((N, L, H, dk))))
    pool = r.standard_normal((N, H, dk, dv))
    src = np.arange(N)
    dst = np.full((N, L), -1)
    dst[:, -1] = src
    o, out = oracle.decode_pool(q, k, v, None, la, pool, src, dst, write="add")
    for n in range(N):
        of, ff = oracle.fwd(q[n:n + 1], k[n:n + 1], v[n:n + 1], None, la[n:n + 1], pool[n][None], write="add")
        np.testing.assert_allclose(o[n], of[0], atol=1e-13, rtol=0)
        np.testing.assert_allclose(out[n], ff[0], atol=1e-13, rtol=0)


def _additive_pin_passes(lib):
    T, H, dk, dv = 9, 1, 4, 3
    q, k, v, s0 = tokens(T, H, dk, dv, seed=8)
    o, _ = oracle.fwd(q, k, v, np.full((1, T, H), 0.5), None, s0, write="add", lib=lib)
    Q, K, V = q[0, :, 0], k[0, :, 0], v[0, :, 0]
    return bool(np.allclose(o[0, :, 0], np.tril(Q @ K.T) @ V + Q @ s0[0, 0], atol=1e-12))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_beta_in_additive_write_is_caught():
    path = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")
    src = open(path).read()
    old = "M[i * dv + j] += k[i] * v[j];"
    assert src.count(old) == 1
    with tempfile.TemporaryDirectory() as d:
        good = os.path.join(d, "good.so")
        oracle.build(force=True, src=path, out=good)
        assert _additive_pin_passes(oracle.load(good))
        mpath = os.path.join(d, "mut.c")
        open(mpath, "w").write(src.replace(old, "M[i * dv + j] += beta * k[i] * v[j];"))
        bad = os.path.join(d, "mut.so")
        oracle.build(force=True, src=mpath, out=bad)
        assert not _additive_pin_passes(oracle.load(bad))

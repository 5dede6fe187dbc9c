"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test states what fixes the expected value: an exact rational fixture, a
second independent statement of the update from the pages, an autograd gradient
step, a closed form, an invariant, or a brute-force formula.  The last test plants
mistakes in a copy of the oracle's C source and checks that the pins catch them.
"""
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.golden.derive_recurrence_small import read_cases

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "recurrence_small.txt")
rng = np.random.default_rng(12345)


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_case(B, T, H, dk, dv, gate, seed=0, state=True, gate_scale=1.0):
    r = np.random.default_rng(seed)
    q = unit(r.standard_normal((B, T, H, dk)))
    k = unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    if gate == "head":
        la = -gate_scale * np.log1p(np.exp(r.standard_normal((B, T, H))))
    elif gate == "key":
        la = -gate_scale * np.log1p(np.exp(r.standard_normal((B, T, H, dk))))
    else:
        la = None
    s0 = r.standard_normal((B, H, dk, dv)) * 0.5 if state else None
    return q, k, v, beta, la, s0


def gate_vec(la, b, t, h, dk):
    if la is None:
        return np.ones(dk)
    if la.ndim == 3:
        return np.full(dk, np.exp(la[b, t, h]))
    return np.exp(la[b, t, h])


# --------------------------------------------------------------------------
# 1. exact rational fixtures (hand-derived; tests/golden/recurrence_small.txt)
@pytest.mark.parametrize("name", sorted(read_cases(GOLDEN).keys()))
def test_golden_exact_fixture(name):
    case = read_cases(GOLDEN)[name]
    f = lambda m: np.array([[float(x) for x in row] for row in m])
    k, v, q = f(case["k"]), f(case["v"]), f(case["q"])
    T, dk = k.shape
    dv = v.shape[1]
    beta = f(case["beta"])[:, 0]
    alpha = f(case["alpha"])
    if case["gate"] == "none":
        la = None
    elif case["gate"] == "head":
        la = np.log(alpha[:, 0]).reshape(1, T, 1)
    else:
        la = np.log(alpha).reshape(1, T, 1, dk)
    o, fs = oracle.fwd(q.reshape(1, T, 1, dk), k.reshape(1, T, 1, dk), v.reshape(1, T, 1, dv),
                       beta.reshape(1, T, 1), la, f(case["M0"]).reshape(1, 1, dk, dv),
                       gate=case["gate"])
    np.testing.assert_allclose(o[0, :, 0], f(case["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(fs[0, 0], f(case["MT"]), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# 2. second statement of the update: matrix-product forms
#    M-orientation (Decoding Hybrid..., sec. 3 item 6):  M <- (I - b k k^T) Diag(a) M + b k v^T
#    S-orientation (scalar gate, spec form):       S <- a S (I - b k k^T) + b v k^T, o = S q
@pytest.mark.parametrize("gate", ["none", "head", "key"])
@pytest.mark.parametrize("dk,dv", [(6, 4), (4, 6), (8, 8)])
def test_matrix_product_form(gate, dk, dv):
    B, T, H = 2, 23, 2
    q, k, v, beta, la, s0 = rand_case(B, T, H, dk, dv, gate, seed=dk * 10 + dv)
    o, fs = oracle.fwd(q, k, v, beta, la, s0, gate=gate)
    for b in range(B):
        for h in range(H):
            M = s0[b, h].copy()
            S = s0[b, h].T.copy()
            for t in range(T):
                kt, vt, qt, bt = k[b, t, h], v[b, t, h], q[b, t, h], beta[b, t, h]
                a = gate_vec(la, b, t, h, dk)
                M = (np.eye(dk) - bt * np.outer(kt, kt)) @ np.diag(a) @ M + bt * np.outer(kt, vt)
                np.testing.assert_allclose(o[b, t, h], M.T @ qt, atol=1e-12, rtol=0)
                if gate != "key":
                    S = a[0] * S @ (np.eye(dk) - bt * np.outer(kt, kt)) + bt * np.outer(vt, kt)
                    np.testing.assert_allclose(o[b, t, h], S @ qt, atol=1e-12, rtol=0)
            np.testing.assert_allclose(fs[b, h], M, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# 3. one gradient step per token ("Linear Attention Variants", DeltaNet section):
#    M <- M' - beta * grad_{M'} 1/2 |M'^T k - v|^2  with M' = Diag(a) M, gradient by autograd
@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_lms_gradient_step_autograd(gate):
    N, H, dk, dv, T = 3, 2, 5, 7, 9
    q, k, v, beta, la, s0 = rand_case(1, T * N, H, dk, dv, gate, seed=7)
    state = np.random.default_rng(3).standard_normal((N, H, dk, dv))
    for t in range(T):
        sl = slice(t * N, (t + 1) * N)
        qt, kt, vt, bt = q[0, sl], k[0, sl], v[0, sl], beta[0, sl]
        lat = None if la is None else la[0, sl]
        o, new_state = oracle.step(qt, kt, vt, bt, lat, state, gate=gate)
        for n in range(N):
            for h in range(H):
                a = gate_vec(None if la is None else la[:, sl], 0, n, h, dk)
                Mp = torch.tensor(np.diag(a) @ state[n, h], requires_grad=True)
                loss = 0.5 * ((Mp.T @ torch.tensor(kt[n, h]) - torch.tensor(vt[n, h])) ** 2).sum()
                loss.backward()
                M_ref = (Mp - bt[n, h] * Mp.grad).detach().numpy()
                np.testing.assert_allclose(new_state[n, h], M_ref, atol=1e-12, rtol=0)
                np.testing.assert_allclose(o[n, h], M_ref.T @ qt[n, h], atol=1e-12, rtol=0)
        state = new_state


# --------------------------------------------------------------------------
# 4. invariants and closed forms
@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_I1_beta_zero_only_decays(gate):
    """beta = 0: nothing is written; M_t = Diag(exp(sum log alpha)) M0 (alpha = 1 keeps S)."""
    B, T, H, dk, dv = 2, 40, 3, 8, 5
    q, k, v, beta, la, s0 = rand_case(B, T, H, dk, dv, gate, seed=11, gate_scale=0.05)
    beta = np.zeros_like(beta)
    o, fs = oracle.fwd(q, k, v, beta, la, s0, gate=gate)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                if la is None:
                    d = np.ones(dk)
                elif la.ndim == 3:
                    d = np.full(dk, np.exp(la[b, :t + 1, h].sum()))
                else:
                    d = np.exp(la[b, :t + 1, h].sum(axis=0))
                Mt = d[:, None] * s0[b, h]
                np.testing.assert_allclose(o[b, t, h], Mt.T @ q[b, t, h], atol=1e-12, rtol=0)
            np.testing.assert_allclose(fs[b, h], Mt, atol=1e-12, rtol=0)


@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_I2_replace_reads_back_value(gate):
    """beta = 1, |k| = 1, q = k: the read returns the value just written, exactly."""
    B, T, H, dk, dv = 2, 50, 2, 8, 6
    q, k, v, beta, la, s0 = rand_case(B, T, H, dk, dv, gate, seed=12)
    o, _ = oracle.fwd(k, k, v, np.ones_like(beta), la, s0, gate=gate)
    np.testing.assert_allclose(o, v, atol=1e-12, rtol=0)


def test_I3_orthonormal_keys_retrieve_every_value():
    """beta = 1, alpha = 1, orthonormal keys: M_T^T k_i = v_i for every i, any M0."""
    dk, dv, T = 16, 5, 12
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :T].T.reshape(1, T, 1, dk)
    v = rng.standard_normal((1, T, 1, dv))
    s0 = rng.standard_normal((1, 1, dk, dv))
    _, fs = oracle.fwd(k, k, v, np.ones((1, T, 1)), None, s0)
    np.testing.assert_allclose(k[0, :, 0] @ fs[0, 0], v[0, :, 0], atol=1e-12, rtol=0)


def test_I4_orthogonal_keys_additive_limit():
    """Orthogonal keys, M0 = 0, alpha = 1: the erase term vanishes and
    M_T = sum_i beta_i k_i v_i^T (beta = 1 is the plain sum S_t = S_{t-1} + v_t k_t^T)."""
    dk, dv, T = 12, 7, 10
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = (Qm[:, :T].T * rng.uniform(0.3, 2.0, size=(T, 1))).reshape(1, T, 1, dk)
    v = rng.standard_normal((1, T, 1, dv))
    for beta in (np.ones((1, T, 1)), rng.uniform(0.1, 1.0, size=(1, T, 1))):
        _, fs = oracle.fwd(k, k, v, beta, None, None)
        expect = sum(beta[0, i, 0] * np.outer(k[0, i, 0], v[0, i, 0]) for i in range(T))
        np.testing.assert_allclose(fs[0, 0], expect, atol=1e-12, rtol=0)


def test_I5_scalar_gate_decay_mask_parallel_form():
    """Orthonormal keys, M0 = 0, beta = 1, scalar gates: O = (Q K^T * D) V with
    D[t,i] = exp(G_t - G_i) for t >= i (the retention parallel form Q K^T (.) D)."""
    dk, dv, T = 16, 6, 16
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm.T[:T]
    q = unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    la = -np.log1p(np.exp(rng.standard_normal(T)))
    o, _ = oracle.fwd(q.reshape(1, T, 1, dk), k.reshape(1, T, 1, dk), v.reshape(1, T, 1, dv),
                      np.ones((1, T, 1)), la.reshape(1, T, 1), None)
    G = np.cumsum(la)
    D = np.zeros((T, T))
    for t in range(T):
        for i in range(t + 1):
            D[t, i] = np.exp(G[t] - G[i])
    np.testing.assert_allclose(o[0, :, 0], ((q @ k.T) * D) @ v, atol=1e-12, rtol=0)


def test_I6_per_key_decays_with_basis_keys():
    """Keys e_{pi(t)} (distinct basis vectors), M0 = 0, beta = 1, per-channel gates:
    o_t = sum_{i<=t} v_i q_t[pi(i)] exp(G_t[pi(i)] - G_i[pi(i)])."""
    dk, dv, T = 10, 4, 10
    perm = rng.permutation(dk)[:T]
    k = np.eye(dk)[perm]
    q = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    la = -np.log1p(np.exp(rng.standard_normal((T, dk))))
    o, _ = oracle.fwd(q.reshape(1, T, 1, dk), k.reshape(1, T, 1, dk), v.reshape(1, T, 1, dv),
                      np.ones((1, T, 1)), la.reshape(1, T, 1, dk), None)
    G = np.cumsum(la, axis=0)
    for t in range(T):
        expect = sum(v[i] * q[t, perm[i]] * np.exp(G[t, perm[i]] - G[i, perm[i]]) for i in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], expect, atol=1e-12, rtol=0)


@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_I7_linear_in_values_and_state_and_column_permutation(gate):
    B, T, H, dk, dv = 1, 30, 2, 6, 5
    q, k, v1, beta, la, s1 = rand_case(B, T, H, dk, dv, gate, seed=21)
    _, _, v2, _, _, s2 = rand_case(B, T, H, dk, dv, gate, seed=22)
    o1, f1 = oracle.fwd(q, k, v1, beta, la, s1, gate=gate)
    o2, f2 = oracle.fwd(q, k, v2, beta, la, s2, gate=gate)
    o3, f3 = oracle.fwd(q, k, 2 * v1 - 3 * v2, beta, la, 2 * s1 - 3 * s2, gate=gate)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, atol=1e-11, rtol=0)
    np.testing.assert_allclose(f3, 2 * f1 - 3 * f2, atol=1e-11, rtol=0)
    p = np.random.default_rng(5).permutation(dv)
    o4, f4 = oracle.fwd(q, k, v1[..., p], beta, la, s1[..., p], gate=gate)
    np.testing.assert_allclose(o4, o1[..., p], atol=1e-13, rtol=0)
    np.testing.assert_allclose(f4, f1[..., p], atol=1e-13, rtol=0)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_I8_varlen_split_resume_and_step(gate):
    H, dk, dv = 2, 6, 4
    lengths = [5, 1, 17, 9]
    T = sum(lengths)
    q, k, v, beta, la, _ = rand_case(1, T, H, dk, dv, gate, seed=31)
    s0 = np.random.default_rng(2).standard_normal((len(lengths), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, fs = oracle.fwd(q, k, v, beta, la, s0, cu_seqlens=cu, gate=gate)
    # packed == separate runs
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        sl = (slice(None), slice(a, b))
        on, fn = oracle.fwd(q[sl], k[sl], v[sl], beta[sl], None if la is None else la[sl],
                            s0[n:n + 1], gate=gate)
        np.testing.assert_allclose(o[sl], on, atol=1e-13, rtol=0)
        np.testing.assert_allclose(fs[n], fn[0], atol=1e-13, rtol=0)
    # split / resume at every cut of the longest sequence
    a, b = cu[2], cu[3]
    for cut in (1, 8, 16):
        s1 = (slice(None), slice(a, a + cut))
        s2 = (slice(None), slice(a + cut, b))
        o1, f1 = oracle.fwd(q[s1], k[s1], v[s1], beta[s1], la[s1], s0[2:3], gate=gate)
        o2, f2 = oracle.fwd(q[s2], k[s2], v[s2], beta[s2], la[s2], f1, gate=gate)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o[:, a:b], atol=1e-13, rtol=0)
        np.testing.assert_allclose(f2[0], fs[2], atol=1e-13, rtol=0)
    # forward(T-1) then one step == forward(T)
    sl = (slice(None), slice(a, b - 1))
    _, fprev = oracle.fwd(q[sl], k[sl], v[sl], beta[sl], la[sl], s0[2:3], gate=gate)
    ost, fst = oracle.step(q[:, b - 1], k[:, b - 1], v[:, b - 1], beta[:, b - 1], la[:, b - 1], fprev,
                           gate=gate)
    np.testing.assert_allclose(ost, o[:, b - 1], atol=1e-13, rtol=0)
    np.testing.assert_allclose(fst[0], fs[2], atol=1e-13, rtol=0)


def test_empty_sequences_keep_state():
    H, dk, dv = 2, 4, 3
    lengths = [0, 3, 0]
    q, k, v, beta, la, _ = rand_case(1, 3, H, dk, dv, "head", seed=41)
    s0 = np.random.default_rng(4).standard_normal((3, H, dk, dv))
    _, fs = oracle.fwd(q, k, v, beta, la, s0, cu_seqlens=np.array([0, 0, 3, 3]))
    np.testing.assert_array_equal(fs[0], s0[0])
    np.testing.assert_array_equal(fs[2], s0[2])


# --------------------------------------------------------------------------
# 5. planted mistakes: each mutant of the C source must fail at least one pin
MUTANTS = {
    "no_scalar_decay": ("for (i = 0; i < dk * dv; ++i) M[i] *= a;", "for (i = 0; i < dk * dv; ++i) M[i] *= 1.0;"),
    "key_gate_wrong_index": ("double a = exp(log_alpha[i]);", "double a = exp(log_alpha[0]);"),
    "erase_sign": ("(v[j] - r[j])", "(v[j] + r[j])"),
    "no_beta": ("double bk = beta * k[i];", "double bk = k[i];"),
    "read_with_key": ("o[j] += M[i * dv + j] * q[i];", "o[j] += M[i * dv + j] * k[i];"),
    "retrieve_transposed": ("r[j] += M[i * dv + j] * k[i];", "r[j] += M[j * dv + i] * k[i];"),
    "read_before_write": ("  /* 2. retrieve r = M^T k */",
                          "  for (j = 0; j < dv; ++j) o[j] = 0.0;\n  for (i = 0; i < dk; ++i)\n"
                          "    for (j = 0; j < dv; ++j) o[j] += M[i * dv + j] * q[i];\n"
                          "  if (0)\n  /* 2. retrieve r = M^T k */"),
}


def _pins_pass(lib):
    """A compact subset of the pins, run against a given oracle library."""
    ok = True
    for name, case in read_cases(GOLDEN).items():
        f = lambda m: np.array([[float(x) for x in row] for row in m])
        k, v, q = f(case["k"]), f(case["v"]), f(case["q"])
        T, dk = k.shape
        dv = v.shape[1]
        alpha = f(case["alpha"])
        la = None if case["gate"] == "none" else (
            np.log(alpha[:, 0]).reshape(1, T, 1) if case["gate"] == "head" else np.log(alpha).reshape(1, T, 1, dk))
        o, fs = oracle.fwd(q.reshape(1, T, 1, dk), k.reshape(1, T, 1, dk), v.reshape(1, T, 1, dv),
                           f(case["beta"]).reshape(1, T, 1), la, f(case["M0"]).reshape(1, 1, dk, dv),
                           gate=case["gate"], lib=lib)
        ok &= np.allclose(o[0, :, 0], f(case["o"]), atol=1e-12) and np.allclose(fs[0, 0], f(case["MT"]), atol=1e-12)
    q, k, v, beta, la, s0 = rand_case(1, 20, 1, 6, 4, "key", seed=3)
    o, fs = oracle.fwd(q, k, v, beta, la, s0, gate="key", lib=lib)
    M = s0[0, 0].copy()
    for t in range(20):
        a = np.exp(la[0, t, 0])
        M = (np.eye(6) - beta[0, t, 0] * np.outer(k[0, t, 0], k[0, t, 0])) @ np.diag(a) @ M \
            + beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0])
        ok &= np.allclose(o[0, t, 0], M.T @ q[0, t, 0], atol=1e-12)
    return bool(ok)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_mistakes_are_caught():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")).read()
    with tempfile.TemporaryDirectory() as d:
        good = os.path.join(d, "good.so")
        oracle.build(force=True, src=os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c"), out=good)
        assert _pins_pass(oracle.load(good)), "pins must pass on the unmodified oracle"
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) == 1, name
            path = os.path.join(d, name + ".c")
            open(path, "w").write(src.replace(old, new))
            so = os.path.join(d, name + ".so")
            oracle.build(force=True, src=path, out=so)
            assert not _pins_pass(oracle.load(so)), "mutant %s was not caught" % name

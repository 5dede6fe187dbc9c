"""Pins for the gradients with one decay per key channel (the channel-wise gate of
"Decoding Hybrid Linear Attention Architectures", sec. 3 item 6; gated linear
attention's gate with the additive write, item 4): oracle.bwd's reverse sweep, and the
chunk adjoint (oracle/chunked_ref.py: chunk_step_bwd_key) that the GPU kernels follow.

  - central finite differences of the pinned forward oracle for a random linear loss,
    on every input entry of a small case, both write rules;
  - torch autograd (float64) of the recurrence written with torch operations, on
    packed sequences of several lengths, both write rules;
  - a planted mistake in the per-row decay of the carried gradient must fail the first
    check;
  - the chunk adjoint equals the token adjoint to 1e-10 for chunk lengths 1, 3, 16, 64,
    ragged lengths and strong decays.
"""
import os
import shutil
import tempfile

import numpy as np
import pytest
import torch

import oracle
from oracle import chunked_ref


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(B, T, H, dk, dv, seed, write="delta"):
    r = np.random.default_rng(seed)
    q, k = unit(r.standard_normal((B, T, H, dk))), unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = None if write == "add" else 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    la = -np.log1p(np.exp(r.standard_normal((B, T, H, dk))))
    s0 = r.standard_normal((B, H, dk, dv)) * 0.5
    wo, ws = r.standard_normal((B, T, H, dv)), r.standard_normal((B, H, dk, dv))
    return q, k, v, beta, la, s0, wo, ws


def loss(inputs, wo, ws, write, lib=None):
    o, fs = oracle.fwd(*inputs, write=write, lib=lib) if lib else oracle.fwd(*inputs, write=write)
    return float((o * wo).sum() + (fs * ws).sum())


def fd_check(grads, base, wo, ws, write, tol=1e-7, lib=None):
    h = 1e-6
    for name, x in base.items():
        if x is None:
            continue
        for idx in np.ndindex(x.shape):
            plus, minus = dict(base), dict(base)
            plus[name] = x.copy(); plus[name][idx] += h
            minus[name] = x.copy(); minus[name][idx] -= h
            args = lambda d: (d["q"], d["k"], d["v"], d["beta"], d["la"], d["s0"])
            fd = (loss(args(plus), wo, ws, write) - loss(args(minus), wo, ws, write)) / (2 * h)
            assert abs(fd - grads[name][idx]) <= tol * max(1.0, abs(fd)), (name, idx, fd, grads[name][idx])


@pytest.mark.parametrize("write", ["delta", "add"])
def test_key_gradients_match_finite_differences(write):
    q, k, v, beta, la, s0, wo, ws = case(1, 6, 2, 3, 2, seed=13, write=write)
    dq, dk, dv, db, dla, dinit = oracle.bwd(q, k, v, beta, la, s0, wo, ws, write=write)
    assert dla.shape == la.shape
    fd_check(dict(q=dq, k=dk, v=dv, beta=db, la=dla, s0=dinit),
             dict(q=q, k=k, v=v, beta=beta, la=la, s0=s0), wo, ws, write)


def torch_recurrence(q, k, v, beta, la, s0, cu, write):
    outs, finals = [], []
    for n in range(len(cu) - 1):
        M = s0[n]
        for t in range(int(cu[n]), int(cu[n + 1])):
            M = M * torch.exp(la[0, t])[:, :, None]  # row i of each head's state decays by alpha_i
            if write == "add":
                M = M + torch.einsum("hi,hj->hij", k[0, t], v[0, t])
            else:
                r = torch.einsum("hij,hi->hj", M, k[0, t])
                M = M + beta[0, t][:, None, None] * torch.einsum("hi,hj->hij", k[0, t], v[0, t] - r)
            outs.append(torch.einsum("hij,hi->hj", M, q[0, t]))
        finals.append(M)
    return torch.stack(outs)[None], torch.stack(finals)


@pytest.mark.parametrize("write", ["delta", "add"])
def test_key_gradients_match_torch_autograd(write):
    lengths = [5, 0, 13, 64, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, dk, dv = int(cu[-1]), 2, 6, 4
    q, k, v, beta, la, _, _, _ = case(1, T, H, dk, dv, seed=15, write=write)
    r = np.random.default_rng(18)
    s0 = r.standard_normal((len(lengths), H, dk, dv)) * 0.5
    wo, ws = r.standard_normal((1, T, H, dv)), r.standard_normal((len(lengths), H, dk, dv))
    xs = (q, k, v, np.zeros((1, T, H)) if beta is None else beta, la, s0)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in xs]
    o, fs = torch_recurrence(*ts, cu, write)
    ((o * torch.tensor(wo)).sum() + (fs * torch.tensor(ws)).sum()).backward()
    got = oracle.bwd(q, k, v, beta, la, s0, wo, ws, cu_seqlens=cu, write=write)
    for name, g, t in zip(["dq", "dk", "dv", "dbeta", "dla", "dinit"], got, ts):
        if g is None:
            continue
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-11, rtol=1e-11, err_msg=name)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_mistake_in_channel_decay_is_caught():
    """Carrying the gradient back with the first row's decay for every key row (right
    for a scalar gate, wrong for a per-channel one) must fail the finite differences."""
    path = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")
    src = open(path).read()
    old = """          G[i * dv + j] -= kt[i] * de[j];
          dli += G[i * dv + j] * Mp[i * dv + j];
          G[i * dv + j] *= arow[i];"""
    assert src.count(old) == 1
    q, k, v, beta, la, s0, wo, ws = case(1, 5, 1, 3, 2, seed=14)
    with tempfile.TemporaryDirectory() as d:
        mpath = os.path.join(d, "mut.c")
        open(mpath, "w").write(src.replace(old, old.replace("*= arow[i];", "*= arow[0];")))
        lib = oracle.load(oracle.build(force=True, src=mpath, out=os.path.join(d, "mut.so")))
        got = oracle.bwd(q, k, v, beta, la, s0, wo, ws, lib=lib)
    with pytest.raises(AssertionError):
        fd_check(dict(q=got[0], k=got[1], v=got[2], beta=got[3], la=got[4], s0=got[5]),
                 dict(q=q, k=k, v=v, beta=beta, la=la, s0=s0), wo, ws, "delta")


@pytest.mark.parametrize("C", [1, 3, 16, 64])
@pytest.mark.parametrize("write", ["delta", "add"])
@pytest.mark.parametrize("T", [1, 40, 130])
def test_chunked_key_gradients_equal_token_gradients(C, write, T):
    r = np.random.default_rng(T * 13 + C)
    dk, dv = 8, 5
    q, k = unit(r.standard_normal((T, dk))), unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    beta = None if write == "add" else 1 / (1 + np.exp(-r.standard_normal(T)))
    la = -np.log1p(np.exp(r.standard_normal((T, dk)))) * 2.0  # strong per-channel decays
    M0 = r.standard_normal((dk, dv)) * 0.5
    dO, dMT = r.standard_normal((T, dv)), r.standard_normal((dk, dv))
    got = chunked_ref.chunked_bwd(q, k, v, beta, la, M0, dO, dMT, C=C, write=write)
    ref = oracle.bwd(q[None, :, None], k[None, :, None], v[None, :, None],
                     None if beta is None else beta[None, :, None], la[None, :, None], M0[None, None],
                     dO[None, :, None], dMT[None, None], write=write)
    refs = [ref[0][0, :, 0], ref[1][0, :, 0], ref[2][0, :, 0], None if beta is None else ref[3][0, :, 0],
            ref[4][0, :, 0], ref[5][0, 0]]
    for name, g, rr in zip(["dq", "dk", "dv", "dbeta", "dlog_alpha", "dM0"], got, refs):
        if rr is None:
            continue
        np.testing.assert_allclose(g, rr, atol=1e-10, rtol=1e-10, err_msg=name)

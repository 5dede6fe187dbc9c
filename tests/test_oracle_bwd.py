"""Pins for the oracle's gradients (oracle.bwd, the reverse sweep in gdn_oracle.c).

Two independent checks of the hand-derived token adjoint:
  - central finite differences of the pinned forward oracle (oracle.fwd) for a
    random linear loss L = <W_o, o> + <W_s, final_state>, on every input entry of a
    small case (q, k, v, beta, log alpha, the initial state);
  - torch autograd (float64) of the recurrence written with torch operations, on a
    larger case with several sequences, packed lengths and a partial decay.
A mutant of the adjoint (the erase term of dk dropped) must fail the first check.
"""
import os
import shutil
import tempfile

import numpy as np
import pytest
import torch

import oracle


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(B, T, H, dk, dv, gate, seed):
    r = np.random.default_rng(seed)
    q, k = unit(r.standard_normal((B, T, H, dk))), unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    la = None if gate == "none" else (-np.log1p(np.exp(r.standard_normal((B, T, H)))) if gate == "head"
                                      else np.log(np.array([0.9, 0.6, 0.97][:H])))
    s0 = r.standard_normal((B, H, dk, dv)) * 0.5
    wo, ws = r.standard_normal((B, T, H, dv)), r.standard_normal((B, H, dk, dv))
    return q, k, v, beta, la, s0, wo, ws


def loss(inputs, wo, ws, lib=None):
    o, fs = oracle.fwd(*inputs, lib=lib) if lib else oracle.fwd(*inputs)
    return float((o * wo).sum() + (fs * ws).sum())


@pytest.mark.parametrize("gate", ["none", "head", "const"])
def test_gradients_match_finite_differences(gate):
    q, k, v, beta, la, s0, wo, ws = case(1, 7, 2, 3, 2, gate, seed=3)
    dq, dk, dv, db, dla, dinit = oracle.bwd(q, k, v, beta, la, s0, wo, ws)
    names = ["q", "k", "v", "beta", "la", "s0"]
    grads = dict(q=dq, k=dk, v=dv, beta=db, la=dla, s0=dinit)
    base = dict(q=q, k=k, v=v, beta=beta, la=la, s0=s0)
    h = 1e-6
    for name in names:
        x = base[name]
        if x is None:
            continue
        for idx in np.ndindex(x.shape):
            plus, minus = dict(base), dict(base)
            plus[name] = x.copy(); plus[name][idx] += h
            minus[name] = x.copy(); minus[name][idx] -= h
            args = lambda d: (d["q"], d["k"], d["v"], d["beta"], d["la"], d["s0"])
            fd = (loss(args(plus), wo, ws) - loss(args(minus), wo, ws)) / (2 * h)
            assert abs(fd - grads[name][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grads[name][idx])


def torch_recurrence(q, k, v, beta, la, s0, cu):
    """The recurrence with torch operations (decay, retrieve, write, read)."""
    outs, finals = [], []
    for n in range(len(cu) - 1):
        M = s0[n]
        for t in range(int(cu[n]), int(cu[n + 1])):
            if la is not None:
                M = M * torch.exp(la[0, t])[:, None, None]
            r = torch.einsum("hij,hi->hj", M, k[0, t])
            M = M + beta[0, t][:, None, None] * torch.einsum("hi,hj->hij", k[0, t], v[0, t] - r)
            outs.append(torch.einsum("hij,hi->hj", M, q[0, t]))
        finals.append(M)
    return torch.stack(outs)[None], torch.stack(finals)


def test_gradients_match_torch_autograd():
    lengths = [5, 0, 13, 64, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, dk, dv = int(cu[-1]), 3, 6, 4
    q, k, v, beta, la, _, _, _ = case(1, T, H, dk, dv, "head", seed=5)
    r = np.random.default_rng(8)
    s0 = r.standard_normal((len(lengths), H, dk, dv)) * 0.5
    wo, ws = r.standard_normal((1, T, H, dv)), r.standard_normal((len(lengths), H, dk, dv))
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, beta, la, s0)]
    o, fs = torch_recurrence(*ts, cu)
    ((o * torch.tensor(wo)).sum() + (fs * torch.tensor(ws)).sum()).backward()
    got = oracle.bwd(q, k, v, beta, la, s0, wo, ws, cu_seqlens=cu)
    for g, t in zip(got, ts):
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-11, rtol=1e-11)


def test_no_final_gradient_and_no_initial_state():
    q, k, v, beta, la, _, wo, _ = case(2, 11, 2, 4, 3, "head", seed=9)
    dq, dk, dv, db, dla, dinit = oracle.bwd(q, k, v, beta, la, None, wo, None)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, beta, la)]
    flat = lambda x: x.reshape(1, 22, *x.shape[2:])
    o, _ = torch_recurrence(*[flat(t) for t in ts], torch.zeros(2, 2, 4, 3, dtype=torch.float64), [0, 11, 22])
    (o * torch.tensor(wo.reshape(1, 22, 2, 3))).sum().backward()
    for g, t in zip((dq, dk, dv, db, dla), ts):
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-11, rtol=1e-11)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_mistake_in_adjoint_is_caught():
    path = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")
    src = open(path).read()
    old = "dk_out[th * dk + i] = bt * acc - acc2;"
    assert src.count(old) == 1
    q, k, v, beta, la, s0, wo, ws = case(1, 5, 1, 3, 2, "head", seed=4)
    with tempfile.TemporaryDirectory() as d:
        mpath = os.path.join(d, "mut.c")
        open(mpath, "w").write(src.replace(old, "dk_out[th * dk + i] = bt * acc;"))
        lib = oracle.load(oracle.build(force=True, src=mpath, out=os.path.join(d, "mut.so")))
        _, dk, _, _, _, _ = oracle.bwd(q, k, v, beta, la, s0, wo, ws, lib=lib)
    h, base = 1e-6, (q, k, v, beta, la, s0)
    kp, km = k.copy(), k.copy()
    kp[0, 2, 0, 1] += h
    km[0, 2, 0, 1] -= h
    fd = (loss((q, kp, v, beta, la, s0), wo, ws) - loss((q, km, v, beta, la, s0), wo, ws)) / (2 * h)
    assert abs(fd - dk[0, 2, 0, 1]) > 1e-6

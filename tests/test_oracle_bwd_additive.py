"""Pins for the oracle's gradients of the additive write (oracle.bwd with write="add",
the reverse sweep in gdn_oracle.c), the rule M_t = a_t M_{t-1} + k_t v_t^T, o_t = M_t^T q_t
of gated linear attention and RetNet:
  - central finite differences of the pinned forward oracle (oracle.fwd, write="add")
    for a random linear loss on every input entry of a small case, for no gate, one
    decay per (token, head) and one constant decay per head;
  - torch autograd (float64) of the additive recurrence written with torch
    operations, on packed sequences of several lengths (one empty);
  - a mutant of the additive adjoint (the decay dropped from the carried gradient)
    must fail the finite differences.
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
    la = None if gate == "none" else (-np.log1p(np.exp(r.standard_normal((B, T, H)))) if gate == "head"
                                      else np.log(np.array([0.9, 0.6, 0.97][:H])))
    s0 = r.standard_normal((B, H, dk, dv)) * 0.5
    wo, ws = r.standard_normal((B, T, H, dv)), r.standard_normal((B, H, dk, dv))
    return q, k, v, la, s0, wo, ws


def loss(q, k, v, la, s0, wo, ws):
    o, fs = oracle.fwd(q, k, v, None, la, s0, write="add")
    return float((o * wo).sum() + (fs * ws).sum())


def finite_difference_errors(grads, base, wo, ws, h=1e-6):
    """Largest |finite difference - gradient| (relative to max(1, |fd|)) per input."""
    worst = {}
    for name, x in base.items():
        if x is None:
            continue
        for idx in np.ndindex(x.shape):
            plus, minus = dict(base), dict(base)
            plus[name] = x.copy(); plus[name][idx] += h
            minus[name] = x.copy(); minus[name][idx] -= h
            fd = (loss(**plus, wo=wo, ws=ws) - loss(**minus, wo=wo, ws=ws)) / (2 * h)
            err = abs(fd - grads[name][idx]) / max(1.0, abs(fd))
            worst[name] = max(worst.get(name, 0.0), err)
    return worst


@pytest.mark.parametrize("gate", ["none", "head", "const"])
def test_additive_gradients_match_finite_differences(gate):
    q, k, v, la, s0, wo, ws = case(1, 7, 2, 3, 2, gate, seed=13)
    dq, dk, dv, db, dla, dinit = oracle.bwd(q, k, v, None, la, s0, wo, ws, write="add")
    assert db is None
    grads = dict(q=dq, k=dk, v=dv, la=dla, s0=dinit)
    worst = finite_difference_errors(grads, dict(q=q, k=k, v=v, la=la, s0=s0), wo, ws)
    assert max(worst.values()) <= 1e-7, worst


def torch_additive(q, k, v, la, s0, cu):
    outs, finals = [], []
    for n in range(len(cu) - 1):
        M = s0[n]
        for t in range(int(cu[n]), int(cu[n + 1])):
            if la is not None:
                M = M * torch.exp(la[0, t])[:, None, None]
            M = M + torch.einsum("hi,hj->hij", k[0, t], v[0, t])
            outs.append(torch.einsum("hij,hi->hj", M, q[0, t]))
        finals.append(M)
    return torch.stack(outs)[None], torch.stack(finals)


def test_additive_gradients_match_torch_autograd():
    lengths = [6, 0, 21, 64, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, dk, dv = int(cu[-1]), 3, 5, 4
    q, k, v, la, _, _, _ = case(1, T, H, dk, dv, "head", seed=15)
    r = np.random.default_rng(16)
    s0 = r.standard_normal((len(lengths), H, dk, dv)) * 0.5
    wo, ws = r.standard_normal((1, T, H, dv)), r.standard_normal((len(lengths), H, dk, dv))
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, la, s0)]
    o, fs = torch_additive(*ts, cu)
    ((o * torch.tensor(wo)).sum() + (fs * torch.tensor(ws)).sum()).backward()
    dq, dk_, dv_, db, dla, dinit = oracle.bwd(q, k, v, None, la, s0, wo, ws, cu_seqlens=cu, write="add")
    for g, t in zip((dq, dk_, dv_, dla, dinit), ts):
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-11, rtol=1e-11)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_planted_mistake_in_additive_adjoint_is_caught():
    path = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")
    src = open(path).read()
    old = """            dli += G[i * dv + j] * Mp[i * dv + j];
            G[i * dv + j] *= arow[i];"""
    assert src.count(old) == 1
    q, k, v, la, s0, wo, ws = case(1, 6, 1, 3, 2, "head", seed=17)
    with tempfile.TemporaryDirectory() as d:
        mpath = os.path.join(d, "mut.c")
        open(mpath, "w").write(src.replace(old, "            dli += G[i * dv + j] * Mp[i * dv + j];"))
        lib = oracle.load(oracle.build(force=True, src=mpath, out=os.path.join(d, "mut.so")))
        got = oracle.bwd(q, k, v, None, la, s0, wo, ws, lib=lib, write="add")
    grads = dict(q=got[0], k=got[1], v=got[2], la=got[4], s0=got[5])
    worst = finite_difference_errors(grads, dict(q=q, k=k, v=v, la=la, s0=s0), wo, ws)
    assert max(worst.values()) > 1e-3, worst

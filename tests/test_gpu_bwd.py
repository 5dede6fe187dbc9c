"""GPU parity of the backward pass (gdn_bwd_chunked, through the C ABI) against the
fp64 oracle's gradients (oracle.bwd).

Metric: max |x - x_ref| / max |x_ref| per gradient tensor.  Tolerance: 2e-2 with
bf16 inputs (the forward states are recomputed with bf16 matrix-core operands, as in
the forward pass), 1e-4 in the fp32 mode; the backward arithmetic itself is fp32.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
NAMES = ["dq", "dk", "dv", "dbeta", "dlog_alpha", "dinitial_state"]


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as g
    return g


def relerr(x, ref):
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (den if den > 0 else 1.0))


def grads_inputs(inp, seed, dfinal=True):
    g = torch.Generator().manual_seed(seed)
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    dout = torch.randn(B, T, H, dv, generator=g).to(inp["q"].dtype)
    dfs = torch.randn(inp["N"], H, dk, dv, generator=g) * 0.1 if dfinal else None
    return dout, dfs


def check(gdn, inp, seed=0, dfinal=True, tol=None):
    dout, dfs = grads_inputs(inp, seed, dfinal)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    got = gdn.bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"], dout.cuda(),
                          None if dfs is None else dfs.cuda(), d["cu_seqlens"])
    torch.cuda.synchronize()
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["initial_state"], dout, dfs,
                     cu_seqlens=inp["cu_seqlens"])
    tol = tol or TOL[inp["dtype"]]
    errs = {}
    for name, g_, r in zip(NAMES, got, ref):
        if r is None:
            assert g_ is None
            continue
        assert torch.isfinite(g_.float()).all(), name
        errs[name] = relerr(g_, r)
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, "errors %s (tol %.1e)" % ({k: "%.2e" % v for k, v in errs.items()}, tol)
    return errs


@pytest.mark.parametrize("T", [1, 63, 64, 130])
@pytest.mark.parametrize("gate", ["none", "head"])
def test_bwd_bf16_ragged(gdn, T, gate):
    check(gdn, synth.random_inputs(2, T, 3, 128, 128, gate, "bf16", seed=T, state_std=0.05), seed=T)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("gate", ["none", "head"])
def test_bwd_head_dims(gdn, dk, dv, gate):
    check(gdn, synth.random_inputs(2, 150, 2, dk, dv, gate, "bf16", seed=dk + dv, state_std=0.05), seed=1)


@pytest.mark.parametrize("B,H,dv,width", [(2, 2, 128, 16), (16, 8, 64, 32), (32, 8, 128, 64)])
@pytest.mark.parametrize("gate", ["head", "key"])
def test_bwd_reverse_pass_widths(gdn, B, H, dv, width, gate):
    """The reverse pass takes the widest value block of 64, 32 or 16 columns that still
    gives N H d_v / width >= 256 workgroups (else 16); these shapes select each width."""
    pairs = B * H
    assert (pairs * dv // 64 >= 256) == (width == 64)
    assert (pairs * dv // 64 < 256 <= pairs * dv // 32) == (width == 32)
    check(gdn, synth.random_inputs(B, 130, H, 128, dv, gate, "bf16", seed=width, state_std=0.05), seed=width)


@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("gate", ["none", "head"])
def test_bwd_fp32(gdn, dv, gate):
    check(gdn, synth.random_inputs(2, 190, 2, 64, dv, gate, "f32", seed=dv, state_std=0.1), seed=2)


def test_bwd_without_state_or_final_gradient(gdn):
    check(gdn, synth.random_inputs(3, 100, 2, 128, 128, "head", "bf16", seed=5), seed=3, dfinal=False)


@pytest.mark.parametrize("gate", ["none", "head"])
def test_bwd_varlen(gdn, gate):
    inp = synth.random_inputs(1, None, 3, 128, 128, gate, "bf16", seed=6, lengths=[1, 0, 200, 64, 65, 17])
    inp["initial_state"] = torch.randn(inp["N"], 3, 128, 128, generator=torch.Generator().manual_seed(9)) * 0.05
    check(gdn, inp, seed=4)


def test_bwd_strong_decay(gdn):
    inp = synth.random_inputs(2, 256, 2, 128, 128, "head", "bf16", seed=7, state_std=0.05)
    inp["log_alpha"] = inp["log_alpha"] * 0 - 5.0
    check(gdn, inp, seed=5)


def test_bwd_deterministic(gdn):
    inp = synth.random_inputs(2, 200, 2, 128, 128, "head", "bf16", seed=8, state_std=0.05)
    dout, dfs = grads_inputs(inp, 6)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    run = lambda: gdn.bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"],
                                  dout.cuda(), dfs.cuda())
    a, b = run(), run()
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_350m_shape_full(gdn):
    """The 350M-class layer shape (B=16, T=2048, H=8, d=128, scalar gate), checked in full."""
    check(gdn, synth.workload_inputs("gdn-350m-bf16-B16-T2048-H8-d128"), seed=11)

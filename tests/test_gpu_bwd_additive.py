"""GPU parity of the backward pass for the additive write (gated linear attention /
RetNet training) and for the constant per-head decay, through the C ABI
(gdn_bwd_chunked), against the fp64 oracle's gradients (oracle.bwd).

Metric: max |x - x_ref| / max |x_ref| per gradient tensor; 2e-2 with bf16 inputs,
1e-4 in the fp32 mode.  The constant decay's gradient is one value per head (the sum
over every token of every sequence), summed on the GPU in a fixed order.
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
    x = x.detach().double().cpu().numpy()
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (den if den > 0 else 1.0))


def inputs(B, T, H, dk, dv, gate, dtype, seed, write, lengths=None, state_std=0.05):
    """gate: none | head | const (RetNet's fixed per-head decays)."""
    inp = synth.random_inputs(B, T, H, dk, dv, "head" if gate == "const" else gate, dtype, seed=seed,
                              state_std=state_std, lengths=lengths)
    if gate == "const":
        inp["log_alpha"] = synth.retnet_log_gamma(H)
    if write == "add":
        inp["beta"] = None
    inp["write"] = write
    return inp


def check(gdn, inp, seed=0, dfinal=True):
    g = torch.Generator().manual_seed(seed)
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    dout = torch.randn(B, T, H, dv, generator=g).to(inp["q"].dtype)
    dfs = torch.randn(inp["N"], H, dk, dv, generator=g) * 0.1 if dfinal else None
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    got = gdn.bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"], dout.cuda(),
                          None if dfs is None else dfs.cuda(), d["cu_seqlens"], write=inp["write"])
    torch.cuda.synchronize()
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["initial_state"], dout, dfs,
                     cu_seqlens=inp["cu_seqlens"], write=inp["write"])
    tol = TOL[inp["dtype"]]
    errs = {}
    for name, g_, r in zip(NAMES, got, ref):
        if r is None:
            assert g_ is None, name
            continue
        assert tuple(g_.shape) == tuple(r.shape), name
        assert torch.isfinite(g_.float()).all(), name
        errs[name] = relerr(g_, r)
    print(inp["write"], {k: "%.2e" % v for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, "errors %s (tol %.1e)" % ({k: "%.2e" % v for k, v in errs.items()}, tol)


@pytest.mark.parametrize("T", [1, 64, 130])
@pytest.mark.parametrize("gate", ["none", "head", "const"])
def test_additive_bwd_bf16(gdn, T, gate):
    check(gdn, inputs(2, T, 3, 128, 128, gate, "bf16", seed=T + 5, write="add"), seed=T)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64)])
def test_additive_bwd_head_dims(gdn, dk, dv):
    check(gdn, inputs(2, 150, 2, dk, dv, "head", "bf16", seed=dk + dv, write="add"), seed=1)


@pytest.mark.parametrize("gate", ["none", "head", "const"])
def test_additive_bwd_fp32(gdn, gate):
    check(gdn, inputs(2, 190, 2, 64, 64, gate, "f32", seed=9, write="add", state_std=0.1), seed=2)


@pytest.mark.parametrize("write", ["add", "delta"])
def test_bwd_varlen_constant_decay(gdn, write):
    """Packed sequences (one empty) with RetNet's decays: the [H] gradient sums over all."""
    check(gdn, inputs(1, None, 4, 128, 128, "const", "bf16", seed=11, write=write,
                      lengths=[1, 200, 0, 64, 77], state_std=None), seed=3, dfinal=False)


@pytest.mark.parametrize("T", [64, 130])
def test_delta_bwd_constant_decay(gdn, T):
    check(gdn, inputs(2, T, 3, 128, 128, "const", "bf16", seed=T + 1, write="delta"), seed=4)


def test_constant_decay_gradient_without_tokens(gdn):
    """T = 0: the [H] decay gradient is zero and the initial-state gradient is dfinal."""
    inp = inputs(2, 0, 3, 128, 128, "const", "bf16", seed=12, write="add")
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    dfs = torch.randn(2, 3, 128, 128).cuda()
    got = gdn.bwd_chunked(d["q"], d["k"], d["v"], None, d["log_alpha"], d["initial_state"],
                          torch.empty(2, 0, 3, 128, dtype=torch.bfloat16, device="cuda"), dfs, write="add")
    torch.cuda.synchronize()
    assert torch.equal(got[4], torch.zeros(3, device="cuda"))
    assert torch.equal(got[5], dfs)


@pytest.mark.parametrize("B,H,dv,width", [(2, 2, 128, 16), (16, 8, 64, 32), (32, 8, 128, 64)])
@pytest.mark.parametrize("gate", ["head", "key"])
def test_additive_bwd_reverse_pass_widths(gdn, B, H, dv, width, gate):
    """The additive write at each value-block width of the reverse pass (the widest of
    64, 32 or 16 columns that gives N H d_v / width >= 256 workgroups, else 16); with one
    decay per key channel the 16-column block reads its operands through LDS staging."""
    pairs = B * H
    assert (pairs * dv // 64 >= 256) == (width == 64)
    assert (pairs * dv // 64 < 256 <= pairs * dv // 32) == (width == 32)
    check(gdn, inputs(B, 130, H, 128, dv, gate, "bf16", seed=width + 1, write="add"), seed=width)


def test_retnet_backward_full_size(gdn):
    """The RetNet workload (B16, T2048, H8, d128, fixed decays, additive write)."""
    check(gdn, synth.workload_inputs("retnet-bf16-B16-T2048-H8-d128"), seed=13)

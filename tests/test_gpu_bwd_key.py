"""GPU parity of the gradients with one decay per key channel (gdn_bwd_chunked with
GDN_GATE_KEY, through the C ABI) against the fp64 oracle's gradients (oracle.bwd).

Metric: max |x - x_ref| / max |x_ref| per gradient tensor.  Tolerance: 2e-2 with bf16
inputs, 1e-4 in the fp32 mode (the arithmetic is fp32 or split bf16 pairs, about 2^-17
relative per product).  Both write rules: the delta rule with the channel-wise gate and
gated linear attention's additive write.
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


def key_window_plan(N, H, dv, T):
    """Window lengths of the windowed per-key-channel path on this GPU: the shortest
    window of at least 16 chunks whose N H preparation items per chunk fill whole rounds
    of the CUs the state pass leaves free (batch mode, at least two windows)."""
    import math
    free = torch.cuda.get_device_properties(0).multi_processor_count - N * H * (dv // 64)
    nchunks = (T + 63) // 64
    if free <= 0:
        return []
    per_round = free / (N * H)
    wlen = max(16, int(math.floor(math.ceil(16 / per_round) * per_round)))
    if nchunks < 2 * wlen:
        return []
    return [min(wlen, nchunks - w * wlen) for w in range((nchunks + wlen - 1) // wlen)]


def inputs(B, T, H, dk, dv, dtype, seed, write="delta", state=True, lengths=None):
    inp = synth.random_inputs(B, T, H, dk, dv, "key", dtype, seed=seed, state_std=0.05 if state else None,
                              lengths=lengths)
    if write == "add":
        inp["beta"] = None
    inp["write"] = write
    return inp


def grads_inputs(inp, seed, dfinal=True):
    g = torch.Generator().manual_seed(seed)
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    dout = torch.randn(B, T, H, dv, generator=g).to(inp["q"].dtype)
    dfs = torch.randn(inp["N"], H, dk, dv, generator=g) * 0.1 if dfinal else None
    return dout, dfs


def run_gpu(gdn, inp, dout, dfs):
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    got = gdn.bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"], dout.cuda(),
                          None if dfs is None else dfs.cuda(), d["cu_seqlens"], write=inp["write"])
    torch.cuda.synchronize()
    return got


def compare(got, ref, tol):
    errs = {}
    for name, g_, r in zip(NAMES, got, ref):
        if r is None:
            assert g_ is None, name
            continue
        assert torch.isfinite(g_.float()).all(), name
        errs[name] = relerr(g_, r)
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, "errors %s (tol %.1e)" % ({k: "%.2e" % v for k, v in errs.items()}, tol)
    return errs


def check(gdn, inp, seed=0, dfinal=True, tol=None):
    dout, dfs = grads_inputs(inp, seed, dfinal)
    got = run_gpu(gdn, inp, dout, dfs)
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["initial_state"], dout, dfs,
                     cu_seqlens=inp["cu_seqlens"], write=inp["write"])
    return compare(got, ref, tol or TOL[inp["dtype"]])


@pytest.mark.parametrize("write", ["delta", "add"])
@pytest.mark.parametrize("T", [1, 63, 64, 130])
def test_bwd_key_ragged(gdn, T, write):
    check(gdn, inputs(2, T, 3, 128, 128, "bf16", seed=T, write=write), seed=T)


@pytest.mark.parametrize("write", ["delta", "add"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_bwd_key_head_dims(gdn, dk, dv, write):
    check(gdn, inputs(2, 150, 2, dk, dv, "bf16", seed=dk + dv, write=write), seed=1)


@pytest.mark.parametrize("write", ["delta", "add"])
@pytest.mark.parametrize("dk", [64, 128])
def test_bwd_key_fp32(gdn, dk, write):
    check(gdn, inputs(2, 190, 2, dk, 64, "f32", seed=dk, write=write), seed=2)


@pytest.mark.parametrize("write", ["delta", "add"])
def test_bwd_key_varlen(gdn, write):
    check(gdn, inputs(1, None, 3, 128, 128, "bf16", seed=6, write=write, lengths=[1, 0, 200, 64, 65, 17]), seed=4)


def test_bwd_key_without_state_or_final_gradient(gdn):
    check(gdn, inputs(3, 100, 2, 128, 128, "bf16", seed=5, state=False), seed=3, dfinal=False)


@pytest.mark.parametrize("write", ["delta", "add"])
def test_bwd_key_strong_decay(gdn, write):
    """About -5 per token and channel (-320 over a chunk): every pairwise factor must stay
    finite through the split at row 7 of each 16-row block."""
    inp = inputs(2, 200, 2, 128, 128, "bf16", seed=7, write=write)
    la = inp["log_alpha"]
    inp["log_alpha"] = torch.full_like(la, -5.0) + 0.5 * torch.rand(la.shape, generator=torch.Generator().manual_seed(3))
    check(gdn, inp, seed=5)


def test_bwd_key_deterministic(gdn):
    inp = inputs(2, 200, 2, 128, 128, "bf16", seed=8)
    dout, dfs = grads_inputs(inp, 6)
    a, b = run_gpu(gdn, inp, dout, dfs), run_gpu(gdn, inp, dout, dfs)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("write", ["delta", "add"])
def test_bwd_key_windowed_states_ragged(gdn, write):
    """Batch sequences of 45 chunks with a ragged last chunk (T = 64 * 44 + 29) at N = 2,
    H = 16: the chunk states are recomputed in windows (18, 18 and 9 chunks on 256 CUs),
    the state carried between them; two (sequence, head) pairs against the oracle in full."""
    T = 64 * 44 + 29
    plan = key_window_plan(2, 16, 128, T)
    assert len(plan) >= 3 and plan[-1] < plan[0], plan
    inp = synth.random_inputs(2, T, 16, 128, 128, "key", "bf16", seed=77, state_std=0.05)
    inp["write"] = write
    if write == "add":
        inp["beta"] = None
    dout, dfs = grads_inputs(inp, 23)
    got = run_gpu(gdn, inp, dout, dfs)
    for n, h in [(0, 1), (1, 14)]:
        sl = lambda x: None if x is None else x[n:n + 1, :, h:h + 1].contiguous()
        ref = oracle.bwd(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl(inp["log_alpha"]),
                         inp["initial_state"][n:n + 1, h:h + 1], sl(dout), dfs[n:n + 1, h:h + 1], write=write,
                         nthreads=1)
        part = [None if g_ is None else (g_[n:n + 1, h:h + 1] if i == 5 else g_[n:n + 1, :, h:h + 1])
                for i, g_ in enumerate(got)]
        compare(part, ref, TOL["bf16"])


@pytest.mark.parametrize("name,pairs", [("kda-bf16-B2-T16384-H16-d128", [(0, 0), (1, 15)]),
                                        ("gla-bf16-B2-T16384-H16-d128", [(1, 3)])])
def test_bwd_key_long_workload(gdn, name, pairs):
    """The per-key-channel workload (B=2, T=16384, H=16, d=128) and its additive-write
    twin: the GPU computes every gradient of the whole batch; the oracle (whose reverse
    sweep keeps every token's state, 2 GB per sequence and head at this length) recomputes
    the listed (sequence, head) pairs in full."""
    inp = synth.workload_inputs(name)
    inp["write"] = inp.get("write", "delta")
    dout, dfs = grads_inputs(inp, 21)
    got = run_gpu(gdn, inp, dout, dfs)
    for n, h in pairs:
        sl = lambda x: None if x is None else x[n:n + 1, :, h:h + 1].contiguous()
        ref = oracle.bwd(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl(inp["log_alpha"]),
                         None if inp["initial_state"] is None else inp["initial_state"][n:n + 1, h:h + 1],
                         sl(dout), dfs[n:n + 1, h:h + 1], write=inp["write"], nthreads=1)
        part = [None if g_ is None else (g_[n:n + 1, h:h + 1] if i == 5 else g_[n:n + 1, :, h:h + 1])
                for i, g_ in enumerate(got)]
        compare(part, ref, TOL["bf16"])

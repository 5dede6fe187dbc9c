"""GPU parity of the additive write (gated linear attention, RetNet, the plain
linear transformer) and of the constant per-head decay, through the C ABI, against
the fp64 oracle.

Metric: max |x - x_ref| / max |x_ref| per output tensor; 2e-2 for bf16 inputs, 1e-4
for the fp32 mode (states: 1e-5 in the decode kernels, whose arithmetic is fp32
throughout).  The RetNet decays are the pages' example schedule 1 - 2^(-5-h).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


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


def inputs(B, T, H, dk, dv, gate, dtype, seed, state=True, lengths=None):
    """gate: none | head | key | const (RetNet's fixed per-head decays)."""
    inp = synth.random_inputs(B, T, H, dk, dv, "head" if gate == "const" else gate, dtype, seed=seed,
                              state_std=0.05 if state else None, lengths=lengths)
    if gate == "const":
        inp["log_alpha"] = synth.retnet_log_gamma(H)
    inp["gate"] = gate
    return inp


def check(gdn, inp, write="add", tol=None):
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    beta = None if write == "add" else d["beta"]
    o, fs = gdn.fwd_chunked(d["q"], d["k"], d["v"], beta, d["log_alpha"], d["initial_state"], d["cu_seqlens"],
                            write=write)
    torch.cuda.synchronize()
    o_ref, fs_ref = oracle.fwd(inp["q"], inp["k"], inp["v"], None if write == "add" else inp["beta"],
                               inp["log_alpha"], inp["initial_state"], inp["cu_seqlens"], write=write)
    tol = tol or TOL[inp["dtype"]]
    eo, ef = relerr(o, o_ref), relerr(fs, fs_ref)
    assert np.isfinite(o.float().cpu().numpy()).all()
    assert eo <= tol and ef <= tol, "o err %.3e, state err %.3e (tol %.1e)" % (eo, ef, tol)


@pytest.mark.parametrize("T", [1, 64, 130])
@pytest.mark.parametrize("gate", ["none", "head", "key", "const"])
@pytest.mark.parametrize("dk", [64, 128])
def test_additive_bf16(gdn, gate, T, dk):
    check(gdn, inputs(2, T, 3, dk, 128, gate, "bf16", seed=T + dk))


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("gate", ["none", "head", "key", "const"])
def test_additive_fp32(gdn, gate, dk):
    check(gdn, inputs(2, 150, 2, dk, 64, gate, "f32", seed=7))


@pytest.mark.parametrize("write", ["delta", "add"])
@pytest.mark.parametrize("gate", ["none", "head", "key", "const"])
@pytest.mark.parametrize("dtype,dv,B", [("f32", 64, 16), ("f32", 128, 8), ("bf16", 64, 16)])
def test_fused_64_column_blocks(gdn, dtype, dv, B, gate, write):
    """d_k = 64 with N H d_v / 64 = 256 (sequence, head, 64 columns) blocks: the fused
    kernel then gives each workgroup 64 value columns instead of 32."""
    check(gdn, inputs(B, 150, 16, 64, dv, gate, dtype, seed=41 + dv), write=write)


@pytest.mark.parametrize("gate", ["key", "const"])
def test_additive_varlen(gdn, gate):
    check(gdn, inputs(1, None, 4, 128, 64, gate, "bf16", seed=8, state=False, lengths=[1, 200, 64, 0, 77]))


@pytest.mark.parametrize("dk", [64, 128])
def test_constant_decay_delta_rule(gdn, dk):
    """The delta rule with a fixed per-head decay."""
    check(gdn, inputs(2, 190, 3, dk, 128, "const", "bf16", seed=9), write="delta")


def test_retnet_decay_schedule_long_sequence(gdn):
    """RetNet at the 350M-class layer shape with the slowest decays of the schedule
    (gamma up to 1 - 2^-12): states grow to ~1e3 times a single write."""
    check(gdn, inputs(16, 2048, 8, 128, 128, "const", "bf16", seed=10, state=False))


def test_gla_per_key_decay_long_sequence(gdn):
    check(gdn, inputs(2, 4096, 4, 128, 128, "key", "bf16", seed=11))


@pytest.mark.parametrize("gate", ["none", "head", "key", "const"])
@pytest.mark.parametrize("L", [1, 5])
def test_additive_decode_and_step(gdn, gate, L):
    N, H, dk, dv = 6, 3, 128, 128
    inp = synth.pool_decode_inputs(N, L, H, dk, dv, N + N * L, "head" if gate == "const" else gate, "bf16",
                                   seed=L + 3, store="all", padding=1)
    if gate == "const":
        inp["log_alpha"] = synth.retnet_log_gamma(H)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    pool = d["state_pool"].clone()
    o = gdn.decode(d["q"], d["k"], d["v"], None, d["log_alpha"], pool, d["src_slots"], d["dst_slots"], write="add")
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle.decode_pool(inp["q"], inp["k"], inp["v"], None, inp["log_alpha"], inp["state_pool"],
                                         inp["src_slots"], inp["dst_slots"], write="add")
    act = inp["src_slots"].numpy() >= 0
    assert relerr(o.cpu()[act], o_ref[act]) <= TOL["bf16"]
    written = np.unique(inp["dst_slots"].numpy()[act].ravel())
    written = written[written >= 0]
    assert relerr(pool.cpu()[written], pool_ref[written]) <= 1e-5
    # the in-place single step on the same streams' first token
    src = inp["src_slots"][act].long()
    st = inp["state_pool"][src].cuda()
    sel = lambda x: x[act][:, 0].contiguous().cuda()
    la = d["log_alpha"] if gate == "const" else (None if inp["log_alpha"] is None else sel(inp["log_alpha"]))
    o1 = gdn.recurrent_step(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), None, la, st, write="add")
    torch.cuda.synchronize()
    la_ref = inp["log_alpha"] if gate == "const" else (None if inp["log_alpha"] is None else inp["log_alpha"][act][:, 0])
    o1_ref, st_ref = oracle.step(inp["q"][act][:, 0], inp["k"][act][:, 0], inp["v"][act][:, 0], None, la_ref,
                                 inp["state_pool"][src], write="add")
    assert relerr(o1.cpu(), o1_ref) <= TOL["bf16"]
    assert relerr(st.cpu(), st_ref) <= 1e-5


@pytest.mark.parametrize("name", ["retnet-bf16-B16-T2048-H8-d128", "gla-bf16-B2-T16384-H16-d128"])
def test_additive_workloads_full_size(gdn, name):
    """The benchmark's additive-write workloads, at their full sizes, checked in full."""
    inp = synth.workload_inputs(name)
    check(gdn, inp, write=inp["write"])

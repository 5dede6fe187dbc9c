"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Metric: max |x - x_ref| / max |x_ref| per output tensor.  Tolerances: 2e-2 for
bf16 inputs with fp32 accumulation, 1e-4 for the fp32 mode.
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


def to_dev(inp):
    return {k: (v.cuda() if hasattr(v, "cuda") else v) for k, v in inp.items()}


def run_gpu(gdn, inp, output_final_state=True):
    d = to_dev(inp)
    o, fs = gdn.fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"],
                            d["cu_seqlens"], output_final_state=output_final_state)
    torch.cuda.synchronize()
    return o.cpu(), (fs.cpu() if fs is not None else None)


def run_oracle(inp):
    return oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"],
                      inp["initial_state"], inp["cu_seqlens"], gate=inp["gate"])


def check(gdn, inp, tol=None):
    tol = tol or TOL[inp["dtype"]]
    o, fs = run_gpu(gdn, inp)
    o_ref, fs_ref = run_oracle(inp)
    eo, ef = relerr(o, o_ref), relerr(fs, fs_ref)
    assert np.isfinite(o.float().numpy()).all() and np.isfinite(fs.numpy()).all()
    assert eo <= tol and ef <= tol, "o err %.3e, state err %.3e (tol %.1e)" % (eo, ef, tol)
    return eo, ef


# ---------------------------------------------------------------- small shapes
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_bf16_ragged_lengths(gdn, T, gate):
    inp = synth.random_inputs(2, T, 3, 128, 128, gate, "bf16", seed=T, state_std=0.05)
    check(gdn, inp)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("gate", ["head", "key"])
def test_bf16_head_dims(gdn, dk, dv, with_state, gate):
    inp = synth.random_inputs(2, 130, 2, dk, dv, gate, "bf16", seed=dk + dv,
                              state_std=0.05 if with_state else None)
    check(gdn, inp)


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("gate", ["none", "head", "key"])
def test_fp32_mode(gdn, dk, dv, gate):
    inp = synth.random_inputs(2, 190, 2, dk, dv, gate, "f32", seed=dv + dk, state_std=0.1)
    check(gdn, inp)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_fp32_dk128_varlen(gdn, gate):
    """fp32 I/O with d_k = 128 on packed sequences with partial chunks and an empty one."""
    inp = synth.random_inputs(1, None, 3, 128, 128, gate, "f32", seed=19, state_std=0.1,
                              lengths=[1, 64, 130, 0, 77])
    check(gdn, inp)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_varlen_small(gdn, gate):
    lengths = [1, 64, 65, 130, 7, 0, 300]
    inp = synth.random_inputs(1, None, 2, 128, 128, gate, "bf16", seed=3, state_std=0.05,
                              lengths=lengths)
    check(gdn, inp)


def test_varlen_key_many_short(gdn):
    """Per-key-channel gate on packed sequences whose lengths straddle chunk
    boundaries (1..130 tokens, including empty ones): every chunk slot of the
    preparation pass is owned by exactly one (sequence, chunk)."""
    lengths = [1, 63, 64, 65, 0, 127, 128, 129, 2, 70, 0, 130, 5, 64, 33, 97]
    inp = synth.random_inputs(1, None, 3, 128, 128, "key", "bf16", seed=17, state_std=0.05,
                              lengths=lengths)
    check(gdn, inp)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_varlen_many_sequences(gdn, gate):
    """More than 8192 packed sequences: no processing-order table, and for the
    per-key-channel gate the chunk slots are searched over all of them."""
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(0, 4, size=8200)]
    lengths[100] = 70  # one sequence longer than a chunk
    inp = synth.random_inputs(1, None, 1, 128, 64, gate, "bf16", seed=33, state_std=0.05,
                              lengths=lengths)
    check(gdn, inp)


def test_key_prepared_call_repeats(gdn):
    """The per-key-channel gate through PreparedFwd: the workspace holding the
    prepared chunk operands is reused across launches with identical results."""
    inp = synth.random_inputs(2, 300, 2, 128, 64, "key", "bf16", seed=23, state_std=0.05)
    d = to_dev(inp)
    call = gdn.PreparedFwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"])
    o1, f1 = call.launch()
    o1, f1 = o1.clone(), f1.clone()
    o2, f2 = call.launch()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    o_ref, fs_ref = run_oracle(inp)
    assert relerr(o2.cpu(), o_ref) <= TOL["bf16"] and relerr(f2.cpu(), fs_ref) <= TOL["bf16"]


@pytest.mark.parametrize("gate", ["head", "key"])
@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_strong_decay(gdn, gate, dtype, dk):
    """Log decay of -5 per token (-320 per chunk): the per-position factors of every
    decay product must stay finite and the result match the recurrence."""
    inp = synth.random_inputs(2, 200, 2, dk, 128, gate, dtype, seed=21, state_std=0.05)
    la = inp["log_alpha"]
    inp["log_alpha"] = torch.full_like(la, -5.0) + 0.5 * torch.rand(la.shape, generator=torch.Generator().manual_seed(2))
    check(gdn, inp)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_varlen_equals_separate_runs(gdn, gate):
    lengths = [70, 5, 129]
    inp = synth.random_inputs(1, None, 2, 128, 128, gate, "bf16", seed=8, state_std=0.05,
                              lengths=lengths)
    o, fs = run_gpu(gdn, inp)
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lengths)):
        sl = slice(cu[n], cu[n + 1])
        sub = dict(inp, q=inp["q"][:, sl].contiguous(), k=inp["k"][:, sl].contiguous(),
                   v=inp["v"][:, sl].contiguous(), beta=inp["beta"][:, sl].contiguous(),
                   log_alpha=inp["log_alpha"][:, sl].contiguous(),
                   initial_state=inp["initial_state"][n:n + 1].contiguous(), cu_seqlens=None)
        o1, f1 = run_gpu(gdn, sub)
        assert torch.equal(o1, o[:, sl]), n
        assert torch.equal(f1[0], fs[n]), n


def test_replace_invariant_gpu(gdn):
    """beta = 1, q = k (unit norm): the read returns the value just written."""
    inp = synth.random_inputs(1, 256, 2, 128, 128, "head", "bf16", seed=5)
    inp["beta"] = torch.ones_like(inp["beta"])
    inp["q"] = inp["k"].clone()
    o, _ = run_gpu(gdn, inp)
    v = inp["v"].double().numpy()
    assert relerr(o, v) <= 2e-2


@pytest.mark.parametrize("gate", ["head", "key"])
def test_beta_zero_keeps_decayed_state(gdn, gate):
    inp = synth.random_inputs(2, 100, 2, 128, 128, gate, "bf16", seed=6, state_std=0.1)
    inp["beta"] = torch.zeros_like(inp["beta"])
    o, fs = run_gpu(gdn, inp)
    d = torch.exp(inp["log_alpha"].double().sum(dim=1))  # [B, H] or [B, H, d_k]
    d = d[:, :, None, None] if gate == "head" else d[:, :, :, None]
    expect = d * inp["initial_state"].double()
    assert relerr(fs, expect.numpy()) <= 1e-5


@pytest.mark.parametrize("gate", ["head", "key"])
def test_deterministic_and_aliased_state(gdn, gate):
    inp = synth.random_inputs(2, 300, 4, 128, 128, gate, "bf16", seed=9, state_std=0.05)
    o1, f1 = run_gpu(gdn, inp)
    o2, f2 = run_gpu(gdn, inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    d = to_dev(inp)
    st = d["initial_state"].clone()
    o3, f3 = gdn.fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], st, None,
                             final_state=st)
    torch.cuda.synchronize()
    assert f3.data_ptr() == st.data_ptr()
    assert torch.equal(o3.cpu(), o1) and torch.equal(st.cpu(), f1)


def test_no_final_state_output(gdn):
    inp = synth.random_inputs(1, 100, 2, 128, 128, "head", "bf16", seed=10)
    o, fs = run_gpu(gdn, inp, output_final_state=False)
    assert fs is None
    o_ref, _ = run_oracle(inp)
    assert relerr(o, o_ref) <= 2e-2


# ---------------------------------------------------------------- workloads
def test_workload_deltanet_fp32(gdn):
    check(gdn, synth.workload_inputs("deltanet-fp32-B1-T256-H2-d64"))


def test_workload_gdn_bf16_B4(gdn):
    check(gdn, synth.workload_inputs("gdn-bf16-B4-T2048-H8-d128"))


def test_workload_gdn_350m(gdn):
    check(gdn, synth.workload_inputs("gdn-350m-bf16-B16-T2048-H8-d128"))


def test_workload_kda_long(gdn):
    check(gdn, synth.workload_inputs("kda-bf16-B2-T16384-H16-d128"))


@pytest.mark.parametrize("write", ["delta", "add"])
@pytest.mark.parametrize("dv", [64, 128])
def test_key_gate_windows(gdn, write, dv):
    """Long batch sequences with one decay per key channel run as windows of chunks (the
    state carried between launches).  45 chunks with a ragged tail at N = 2, H = 16 give
    three windows on 256 CUs (18, 18 and 9 chunks at d_v = 128; 21, 21 and 3 at 64).
    Against the oracle, and bit for bit against the same sequences packed (a packed call
    runs without windows)."""
    T = 64 * 44 + 37
    plan = key_window_plan(2, 16, dv, T)
    assert len(plan) >= 3 and plan[-1] < plan[0], plan
    inp = synth.random_inputs(2, T, 16, 128, dv, "key", "bf16", seed=61 + dv, state_std=0.05)
    if write == "add":
        inp["beta"] = None
    d = to_dev(inp)
    o, fs = gdn.fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"], write=write)
    cu = torch.tensor([0, T, 2 * T], dtype=torch.int32, device="cuda")
    flat = lambda x: None if x is None else x.reshape(1, 2 * T, *x.shape[2:]).contiguous()
    o2, fs2 = gdn.fwd_chunked(flat(d["q"]), flat(d["k"]), flat(d["v"]), flat(d["beta"]), flat(d["log_alpha"]),
                              d["initial_state"], cu, write=write)
    torch.cuda.synchronize()
    assert torch.equal(o.reshape(1, 2 * T, 16, dv), o2) and torch.equal(fs, fs2)
    o_ref, fs_ref = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["initial_state"],
                               gate="key", write=write)
    assert relerr(o.cpu(), o_ref) <= TOL["bf16"] and relerr(fs.cpu(), fs_ref) <= TOL["bf16"]


@pytest.fixture(scope="module")
def varlen_run(gdn):
    """The packed workload (32 sequences, 283,220 tokens, 16 heads) on the GPU and in
    the oracle, computed once for the tests below."""
    inp = synth.workload_inputs("gdn-varlen-bf16-N32-H16-d128")
    o, fs = run_gpu(gdn, inp)
    o_ref, fs_ref = run_oracle(inp)
    return inp, o, fs, o_ref, fs_ref


def test_workload_varlen_full(varlen_run):
    """Every sequence and every head of the packed workload against the oracle: the
    whole tensors, and each sequence's rows and final state on their own (so that a
    short sequence cannot hide behind a long one's larger values)."""
    inp, o, fs, o_ref, fs_ref = varlen_run
    assert np.isfinite(o.float().numpy()).all() and np.isfinite(fs.numpy()).all()
    assert relerr(o, o_ref) <= 2e-2 and relerr(fs, fs_ref) <= 2e-2
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(cu) - 1):
        sl = slice(cu[n], cu[n + 1])
        assert relerr(o[:, sl], o_ref[:, sl]) <= 2e-2, n
        assert relerr(fs[n], fs_ref[n]) <= 2e-2, n


def test_workload_varlen_decode(gdn, varlen_run):
    """The packed workload's decode leg: 64 single-token recurrent steps at batch 256 x
    16 heads, from the 32 final states tiled 8 times (stream s starts from sequence
    s mod 32), fresh seeded tokens per step.  The oracle steps from the same GPU
    states, so each step's o is held to the bf16 bound and the fp32 pool to 1e-5;
    the whole chain (prefill then decode) is also held end to end against the oracle
    run from its own final states."""
    inp, _, fs, _, fs_ref = varlen_run
    spec = synth.WORKLOADS["gdn-varlen-bf16-N32-H16-d128"]
    batch, steps = spec["decode_batch"], spec["decode_steps"]
    dec = synth.decode_inputs(batch, spec["H"], spec["dk"], spec["dv"], steps, spec["gate"], spec["dtype"],
                              seed=spec["seed"] + 1)
    st = synth.decode_initial_states(fs, batch).cuda()
    ref = synth.decode_initial_states(fs, batch).double().numpy()
    chain = fs_ref[np.arange(batch) % fs_ref.shape[0]]
    for s in range(steps):
        o = gdn.recurrent_step(dec["q"][s].cuda(), dec["k"][s].cuda(), dec["v"][s].cuda(),
                               dec["beta"][s].cuda(), dec["log_alpha"][s].cuda(), st)
        torch.cuda.synchronize()
        o_ref, ref = oracle.step(dec["q"][s], dec["k"][s], dec["v"][s], dec["beta"][s], dec["log_alpha"][s], ref)
        o_chain, chain = oracle.step(dec["q"][s], dec["k"][s], dec["v"][s], dec["beta"][s], dec["log_alpha"][s],
                                     chain)
        assert relerr(o.cpu(), o_ref) <= 2e-2, s
        assert relerr(o.cpu(), o_chain) <= 2e-2, s
    assert relerr(st.cpu(), ref) <= 1e-5
    assert relerr(st.cpu(), chain) <= 2e-2


# ---------------------------------------------------------------- decode step
@pytest.mark.parametrize("gate", ["none", "head", "key"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_recurrent_step_matches_oracle(gdn, gate, dtype):
    N, H, dk, dv, steps = 5, 3, 128, 64, 6
    dec = synth.decode_inputs(N, H, dk, dv, steps, gate, dtype, seed=11)
    state0 = torch.randn(N, H, dk, dv, generator=torch.Generator().manual_seed(1)) * 0.1
    st = state0.cuda()
    ref = state0.double().numpy()
    for s in range(steps):
        la = None if dec["log_alpha"] is None else dec["log_alpha"][s]
        o = gdn.recurrent_step(dec["q"][s].cuda(), dec["k"][s].cuda(), dec["v"][s].cuda(),
                               dec["beta"][s].cuda(), None if la is None else la.cuda(), st)
        torch.cuda.synchronize()
        o_ref, ref = oracle.step(dec["q"][s], dec["k"][s], dec["v"][s], dec["beta"][s], la, ref, gate=gate)
        tol = TOL[dtype] if dtype == "bf16" else 1e-5
        assert relerr(o.cpu(), o_ref) <= tol, s
        assert relerr(st.cpu(), ref) <= 1e-5, s


def test_forward_then_step_equals_longer_forward(gdn):
    inp = synth.random_inputs(2, 129, 2, 128, 128, "head", "bf16", seed=12, state_std=0.05)
    head = {k: (v[:, :128].contiguous() if k in ("q", "k", "v", "beta", "log_alpha") else v)
            for k, v in inp.items()}
    _, fs = run_gpu(gdn, head)
    st = fs.cuda()
    o = gdn.recurrent_step(inp["q"][:, 128].contiguous().cuda(), inp["k"][:, 128].contiguous().cuda(),
                           inp["v"][:, 128].contiguous().cuda(), inp["beta"][:, 128].contiguous().cuda(),
                           inp["log_alpha"][:, 128].contiguous().cuda(), st)
    torch.cuda.synchronize()
    o_ref, f_ref = run_oracle(inp)
    assert relerr(o.cpu(), o_ref[:, 128]) <= 2e-2
    assert relerr(st.cpu(), f_ref) <= 2e-2


def test_prepared_call_matches_direct_call(gdn):
    inp = synth.random_inputs(2, 150, 2, 128, 128, "head", "bf16", seed=13, state_std=0.05)
    o_ref, f_ref = run_gpu(gdn, inp)
    d = to_dev(inp)
    call = gdn.PreparedFwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"], None)
    for _ in range(2):
        o, fs = call.launch()
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), o_ref) and torch.equal(fs.cpu(), f_ref)


@pytest.mark.parametrize("gate", ["head", "key"])
def test_side_stream(gdn, gate):
    """A call queued on a stream other than torch's current one: the workspace the
    binding allocates (the per-key-channel gate's prepared operands) stays reserved for
    that stream's work, and the results equal those of a call on the current stream."""
    inp = synth.random_inputs(2, 200, 2, 128, 128, gate, "bf16", seed=29, state_std=0.05)
    o_ref, f_ref = run_gpu(gdn, inp)
    d = to_dev(inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, fs = gdn.fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"], None,
                            stream=side)
    junk = [torch.full((1 << 20,), 3.0, device="cuda") for _ in range(8)]  # reuses freed blocks, if any
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o.cpu(), o_ref) and torch.equal(fs.cpu(), f_ref)

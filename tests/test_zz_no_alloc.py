"""The allocation-free forward (gdn_fwd_chunked_static) against the forward with a
caller workspace (gdn_fwd_chunked), through the C ABI on the GPU.

Both run the same kernels on the same inputs, so the outputs must be identical.  Two
calls in a row, the second smaller, exercise the reuse of the per-GPU scratch array
(its contents from the first call must not leak into the second); the per-key-channel
gate on packed sequences uses both parts of the scratch (the processing-order table and
the prepared chunk operands).  A call whose scratch need exceeds the array is refused
before anything is launched.
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as g
    return g


def dev(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def both(gdn, inp, write="delta"):
    d = dev(inp)
    beta = None if write == "add" else d["beta"]
    o_ref, f_ref = gdn.fwd_chunked(d["q"], d["k"], d["v"], beta, d["log_alpha"], d["initial_state"],
                                   d["cu_seqlens"], write=write)
    o = torch.full_like(o_ref, 7.0)
    fs = torch.full_like(f_ref, 7.0)
    gdn.fwd_chunked_static(d["q"], d["k"], d["v"], beta, d["log_alpha"], d["initial_state"], d["cu_seqlens"],
                           out=o, final_state=fs, write=write)
    torch.cuda.synchronize()
    return o, fs, o_ref, f_ref


@pytest.mark.parametrize("gate,dk,write", [("key", 128, "delta"), ("key", 128, "add"), ("head", 128, "delta"),
                                           ("key", 64, "delta")])
def test_static_scratch_matches_workspace_call(gdn, gate, dk, write):
    big = synth.random_inputs(1, None, 4, dk, 128, gate, "bf16", seed=51, state_std=0.05,
                              lengths=[700, 1, 0, 2000, 130, 64])
    small = synth.random_inputs(1, None, 3, dk, 64, gate, "bf16", seed=52, state_std=0.05,
                                lengths=[65, 200, 3])
    for inp in (big, small):  # the second call is smaller: stale scratch must not matter
        o, fs, o_ref, f_ref = both(gdn, inp, write)
        assert torch.equal(o, o_ref) and torch.equal(fs, f_ref)


def test_static_scratch_batch_mode_needs_none(gdn):
    inp = synth.random_inputs(2, 300, 2, 128, 128, "head", "bf16", seed=53, state_std=0.05)
    o, fs, o_ref, f_ref = both(gdn, inp)
    assert torch.equal(o, o_ref) and torch.equal(fs, f_ref)


def test_static_scratch_refuses_larger_needs(gdn):
    """The per-key-channel gate at 65,536 tokens x 4 heads needs about 270 MB of
    scratch: refused with GDN_ERR_WORKSPACE, outputs untouched."""
    B, T, H = 1, 65536, 4
    q = torch.zeros(B, T, H, 128, dtype=torch.bfloat16, device="cuda")
    la = torch.zeros(B, T, H, 128, device="cuda")
    beta = torch.zeros(B, T, H, device="cuda")
    args = gdn.make_fwd_args(q, q, q, beta, la, None, None, q, None)
    assert gdn.fwd_workspace_size(args) > gdn.STATIC_SCRATCH_BYTES
    out = torch.full_like(q, 7.0)
    with pytest.raises(RuntimeError, match="workspace"):
        gdn.fwd_chunked_static(q, q, q, beta, la, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)

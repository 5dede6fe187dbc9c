"""Packed-sequence offsets that break the contract (cu_seqlens must be non-decreasing and
end at T): the kernels validate each sequence's offsets on the device and leave the
outputs of a malformed sequence unwritten, as include/gdn.h documents.  Offsets here:
[0, 100, 400, 300] over 300 packed tokens; sequence 0 is valid, sequence 1 ends past T
and sequence 2 ends before it starts.  Tokens 100 .. 299 belong to no valid sequence,
so their output rows keep the caller's sentinel, and so do the final states of
sequences 1 and 2.  The backward's kernels skip the malformed sequences the same way;
its test checks the valid sequence's gradients.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_20_amd as g
    return g


def relerr(x, ref):
    x = x.detach().double().cpu().numpy()
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def malformed(inp):
    cu = torch.tensor([0, 100, 400, 300], dtype=torch.int32)
    return dict(inp, cu_seqlens=cu, N=3)


def check_untouched(o, fs):
    assert torch.all(o[0, 100:].float() == SENTINEL)
    assert torch.all(fs[1:] == SENTINEL)


@pytest.mark.parametrize("dk", [64, 128])
def test_forward_leaves_malformed_sequences_untouched(gdn, dk):
    inp = malformed(synth.random_inputs(1, 300, 2, dk, 128, "head", "bf16", seed=41))
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o = torch.full((1, 300, 2, 128), SENTINEL, dtype=torch.bfloat16, device="cuda")
    fs = torch.full((3, 2, dk, 128), SENTINEL, device="cuda")
    gdn.fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], None, d["cu_seqlens"], out=o, final_state=fs)
    torch.cuda.synchronize()
    check_untouched(o, fs)
    o_ref, fs_ref = oracle.fwd(inp["q"][:, :100], inp["k"][:, :100], inp["v"][:, :100], inp["beta"][:, :100],
                               inp["log_alpha"][:, :100])
    assert relerr(o[:, :100], o_ref) <= 2e-2 and relerr(fs[:1], fs_ref) <= 2e-2


def test_dplr_leaves_malformed_sequences_untouched(gdn):
    inp = malformed(synth.dplr_inputs(1, 300, 2, 128, 128, "head", "bf16", seed=42))
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o = torch.full((1, 300, 2, 128), SENTINEL, dtype=torch.bfloat16, device="cuda")
    fs = torch.full((3, 2, 128, 128), SENTINEL, device="cuda")
    gdn.fwd_dplr(d["q"], d["k"], d["v"], d["a"], d["b"], d["log_alpha"], None, d["cu_seqlens"], out=o,
                 final_state=fs)
    torch.cuda.synchronize()
    check_untouched(o, fs)
    sl = lambda x: x[:, :100]
    o_ref, fs_ref = oracle.fwd_dplr(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["a"]), sl(inp["b"]),
                                    sl(inp["log_alpha"]))
    assert relerr(o[:, :100], o_ref) <= 2e-2 and relerr(fs[:1], fs_ref) <= 2e-2


@pytest.mark.parametrize("write,gate", [("delta", "head"), ("add", "head"), ("delta", "const"),
                                        ("add", "const")])
def test_backward_with_malformed_sequences(gdn, write, gate):
    """The valid sequence's gradients are exact; the malformed ones are skipped.  With
    the constant per-head decay the [H] gradient sums the valid sequence's tokens only
    (tokens 100 .. 299 belong to no valid sequence and contribute nothing)."""
    inp = malformed(synth.random_inputs(1, 300, 2, 128, 128, "head", "bf16", seed=43))
    if gate == "const":
        inp["log_alpha"] = synth.retnet_log_gamma(2)
    if write == "add":
        inp["beta"] = None
    g = torch.Generator().manual_seed(44)
    dout = torch.randn(1, 300, 2, 128, generator=g).to(torch.bfloat16)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    got = gdn.bwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], None, dout.cuda(), None,
                          d["cu_seqlens"], write=write)
    torch.cuda.synchronize()
    sl = lambda x: None if x is None or x.dim() == 1 else x[:, :100]
    if gate == "const":
        sl_la = inp["log_alpha"]
    else:
        sl_la = sl(inp["log_alpha"])
    ref = oracle.bwd(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl_la, None,
                     sl(dout), None, write=write)
    for name, g_, r in zip(["dq", "dk", "dv", "dbeta", "dlog_alpha"], got[:5], ref[:5]):
        if r is None:
            continue
        assert relerr(g_ if g_.dim() == 1 else g_[:, :100], r) <= 2e-2, name
    assert relerr(got[5][:1], ref[5]) <= 2e-2

"""Seeded synthetic inputs for the (gated) delta-rule forward.

Shared by the tests and the benchmark.  This module holds none of the method's
arithmetic: it only draws random tensors on the CPU torch generator, in a fixed
order, with the shapes and value distributions of the workloads below.

Distributions (the same for every workload unless stated):
  q, k   ~ N(0,1), L2-normalised per (token, head) in fp32, then cast to the I/O dtype
  v      ~ N(0,1), cast to the I/O dtype
  beta   = sigmoid(N(0,1)), fp32
  gate   "head": log alpha = -softplus(N(0,1)) * exp(U(-3,0)), one value per (token, head)
         "key":  log alpha = -softplus(N(0,1)), one value per (token, head, key channel)
         "none": absent
         "const": one fixed log decay per head, log(1 - 2^(-5-h)) (RetNet's schedule)
  write  "delta" (default) or "add" (beta absent)
  state  optional initial state ~ N(0, std^2), fp32, layout [N,H,d_k,d_v] (M = S^T)
  dplr   the diagonal-plus-low-rank transition's a = -kappa, b = kappa * w, with kappa
         ~ N(0,1) L2-normalised and w = sigmoid(N(0,1)) per key channel (so the
         low-rank correction shrinks the state along kappa by a factor in (0, 1)),
         drawn from a second generator seeded seed + 7919; beta is dropped
Draw order: sequence lengths (varlen), q, k, v, beta logits, gate factors, initial
state, then decode tokens.
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

# The workloads.  Sizes follow the pages' model scale (350M-class layer: hidden
# 1024 = 8 heads x 128) and chunk length 64; the names say what they are.
WORKLOADS = {
    "deltanet-fp32-B1-T256-H2-d64": dict(
        B=1, T=256, H=2, dk=64, dv=64, gate="none", dtype="f32", state_std=None, seed=1000),
    "gdn-bf16-B4-T2048-H8-d128": dict(
        B=4, T=2048, H=8, dk=128, dv=128, gate="head", dtype="bf16", state_std=None, seed=1001),
    "gdn-350m-bf16-B16-T2048-H8-d128": dict(
        B=16, T=2048, H=8, dk=128, dv=128, gate="head", dtype="bf16", state_std=0.02, seed=1002),
    "kda-bf16-B2-T16384-H16-d128": dict(
        B=2, T=16384, H=16, dk=128, dv=128, gate="key", dtype="bf16", state_std=None, seed=1003),
    "gdn-varlen-bf16-N32-H16-d128": dict(
        N=32, len_lo=512, len_hi=16384, H=16, dk=128, dv=128, gate="head", dtype="bf16",
        state_std=None, seed=1004, decode_steps=64, decode_batch=256),
    # the additive write at the same shapes: RetNet (fixed per-head decays, the
    # pages' schedule 1 - 2^(-5-h)) and gated linear attention (per-key decays)
    "retnet-bf16-B16-T2048-H8-d128": dict(
        B=16, T=2048, H=8, dk=128, dv=128, gate="const", write="add", dtype="bf16", state_std=0.02,
        seed=1005),
    "gla-bf16-B2-T16384-H16-d128": dict(
        B=2, T=16384, H=16, dk=128, dv=128, gate="key", write="add", dtype="bf16", state_std=None,
        seed=1006),
    # the diagonal-plus-low-rank transition with the scalar gate, at the 350M-class shape
    "dplr-bf16-B16-T2048-H8-d128": dict(
        B=16, T=2048, H=8, dk=128, dv=128, gate="head", write="dplr", dtype="bf16", state_std=0.02,
        seed=1007),
    # ... and with one decay per key channel (the page's Diag(alpha_t) + a b^T)
    "dplr-key-bf16-B16-T2048-H8-d128": dict(
        B=16, T=2048, H=8, dk=128, dv=128, gate="key", write="dplr", dtype="bf16", state_std=0.02,
        seed=1008),
}

CHUNK = 64

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def _draw_tokens(g, lead, H, dk, dv, gate, dtype):
    """q, k, v, beta, log_alpha for token positions of shape ``lead``."""
    q = _unit(torch.randn(*lead, H, dk, generator=g)).to(dtype)
    k = _unit(torch.randn(*lead, H, dk, generator=g)).to(dtype)
    v = torch.randn(*lead, H, dv, generator=g).to(dtype)
    beta = torch.sigmoid(torch.randn(*lead, H, generator=g))
    if gate == "head":
        a = F.softplus(torch.randn(*lead, H, generator=g))
        s = torch.exp(torch.rand(*lead, H, generator=g) * 3.0 - 3.0)
        log_alpha = -(a * s)
    elif gate == "key":
        log_alpha = -F.softplus(torch.randn(*lead, H, dk, generator=g))
    else:
        log_alpha = None
    return q, k, v, beta, log_alpha


def random_inputs(B, T, H, dk, dv, gate="head", dtype="bf16", seed=0, state_std=None,
                  lengths=None):
    """Inputs for one call.  With ``lengths`` the tokens are packed (B must be 1)
    and ``cu_seqlens`` (int32, N+1 offsets) is returned; T is then sum(lengths)."""
    g = torch.Generator().manual_seed(int(seed))
    dt = _DTYPES[dtype]
    cu = None
    N = B
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        B, T, N = 1, int(cu[-1]), len(lengths)
    q, k, v, beta, la = _draw_tokens(g, (B, T), H, dk, dv, gate, dt)
    s0 = None
    if state_std is not None:
        s0 = torch.randn(N, H, dk, dv, generator=g) * float(state_std)
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=la, initial_state=s0, cu_seqlens=cu,
                gate=gate, dtype=dtype, N=N)


def dplr_inputs(B, T, H, dk, dv, gate="head", dtype="bf16", seed=0, state_std=None, lengths=None):
    """Inputs of the diagonal-plus-low-rank transition: those of ``random_inputs``
    without beta, plus a = -kappa and b = kappa * w (kappa a unit vector, w in (0, 1)
    per key channel) in the I/O dtype."""
    out = random_inputs(B, T, H, dk, dv, gate, dtype, seed=seed, state_std=state_std, lengths=lengths)
    g = torch.Generator().manual_seed(int(seed) + 7919)
    lead = tuple(out["q"].shape[:2])
    kappa = _unit(torch.randn(*lead, H, dk, generator=g))
    w = torch.sigmoid(torch.randn(*lead, H, dk, generator=g))
    dt = _DTYPES[dtype]
    out["a"], out["b"] = (-kappa).to(dt), (kappa * w).to(dt)
    out["beta"], out["write"] = None, "dplr"
    return out


def retnet_log_gamma(H: int) -> torch.Tensor:
    """Fixed per-head log decays log(1 - 2^(-5 - h)), h = 0..H-1: the head-wise decay
    schedule that the RetNet passage gives as its example (float32 [H])."""
    h = torch.arange(H, dtype=torch.float64)
    return torch.log1p(-torch.pow(2.0, -5.0 - h)).to(torch.float32)


def varlen_lengths(spec):
    g = torch.Generator().manual_seed(int(spec["seed"]))
    return torch.randint(spec["len_lo"], spec["len_hi"] + 1, (spec["N"],), generator=g).tolist()


def workload_inputs(name: str):
    """Inputs of a named workload (CPU tensors).  For the varlen workload the
    sequence lengths are drawn first from the same seed."""
    spec = WORKLOADS[name]
    if "N" in spec:
        lengths = varlen_lengths(spec)
        out = random_inputs(1, None, spec["H"], spec["dk"], spec["dv"], spec["gate"],
                            spec["dtype"], seed=spec["seed"] + 7919, lengths=lengths)
        out["lengths"] = lengths
        return out
    if spec.get("write") == "dplr":
        return dplr_inputs(spec["B"], spec["T"], spec["H"], spec["dk"], spec["dv"], spec["gate"],
                           spec["dtype"], seed=spec["seed"], state_std=spec["state_std"])
    const = spec["gate"] == "const"
    out = random_inputs(spec["B"], spec["T"], spec["H"], spec["dk"], spec["dv"],
                        "none" if const else spec["gate"], spec["dtype"], seed=spec["seed"],
                        state_std=spec["state_std"])
    if const:
        out["log_alpha"], out["gate"] = retnet_log_gamma(spec["H"]), "const"
    out["write"] = spec.get("write", "delta")
    if out["write"] == "add":
        out["beta"] = None
    return out


def decode_inputs(N, H, dk, dv, steps, gate="head", dtype="bf16", seed=0):
    """Per-step single-token inputs for ``steps`` decode steps of N streams:
    q,k [steps,N,H,dk], v [steps,N,H,dv], beta [steps,N,H], log_alpha
    [steps,N,H](,dk)."""
    g = torch.Generator().manual_seed(int(seed))
    q, k, v, beta, la = _draw_tokens(g, (steps, N), H, dk, dv, gate, _DTYPES[dtype])
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=la, gate=gate, dtype=dtype)


def pool_decode_inputs(N, L, H, dk, dv, pool_size, gate="head", dtype="bf16", seed=0,
                       store="last", padding=0, state_std=0.05):
    """Inputs of one pooled decode call: tokens q,k [N,L,H,dk], v [N,L,H,dv], beta
    [N,L,H], log_alpha; a pool [P,H,dk,dv] of N(0, state_std^2) states; src_slots
    int32 [N] drawn without replacement from a random permutation of the slots, the
    first ``padding`` streams set to -1 (padding); dst_slots int32 [N,L]:
    ``store="last"`` writes the last state back to the stream's own slot (plain
    decoding), ``"all"`` gives every token a spare slot of its own (speculative
    drafts), ``"none"`` stores nothing."""
    g = torch.Generator().manual_seed(int(seed))
    q, k, v, beta, la = _draw_tokens(g, (N, L), H, dk, dv, gate, _DTYPES[dtype])
    pool = torch.randn(pool_size, H, dk, dv, generator=g) * float(state_std)
    need = N + (N * L if store == "all" else 0)
    assert pool_size >= need, "pool too small for the requested slots"
    perm = torch.randperm(pool_size, generator=g).to(torch.int32)
    src = perm[:N].clone()
    src[:padding] = -1
    dst = torch.full((N, L), -1, dtype=torch.int32)
    if store == "last":
        dst[:, -1] = src
    elif store == "all":
        dst = perm[N:N + N * L].reshape(N, L).clone()
        dst[:padding] = -1
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=la, state_pool=pool, src_slots=src,
                dst_slots=dst, gate=gate, dtype=dtype)


def decode_initial_states(final_states: torch.Tensor, batch: int) -> torch.Tensor:
    """Decode streams start from the prefill's final states, tiled: stream s takes
    sequence s mod N_prefill."""
    n = final_states.shape[0]
    idx = torch.arange(batch) % n
    return final_states[idx].clone()

"""Benchmark of the chunked gated delta-rule forward on one MI355X.

One step = one gdn_fwd_chunked call over one batch of the 350M-class layer shape
(B=16, T=2048, H=8, d_k=d_v=128, bf16 q/k/v/o, fp32 beta/log alpha/state, chunk 64,
random fp32 initial state): every step of the chunked method runs in that call.
Inputs are synthetic (seeded), resident in HBM before timing, and rotated over
four copies so that no step finds its inputs in the 256 MB last-level cache.

Settle and warm-up: from idle, the GPU's power controller needs about 25-30 ms of
continuous load to settle (launch durations first dip below and then rise above the
sustained rate, with socket power at its 1400 W limit).  Before the W warm-up steps,
the benchmark therefore runs untimed headline launches for --settle-ms (default 50 ms)
of wall time, so that the timed steps measure the sustained rate a continuously
running layer sees whatever W is; the line reports the settle phase ("settle").

Prints ONE JSON line.  `value`, `ms_per_step`, `tflops` and `mfma_peak_frac` all use
the whole-job wall time of the K timed steps.  `roofline` relates the kernel's
algorithmic bytes (q, k, v read and o written in bf16, beta and log alpha in fp32,
initial and final fp32 state) to its average launch duration measured with HIP events
on the stream the kernel runs on (`launch_ms`); `frac_at_ms_per_step` is the same
fraction on the wall-clock step time.  `cpu_baseline` times the fp64 oracle on the
host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--all]
                       [--no-cpu] [--calibrate-copy MIB] [--only WORKLOAD[:bwd]]

--only runs just one named workload's forward (or, with ":bwd", its backward) for the
given steps and prints its measurement line instead of the headline: the form the
per-kernel counter profiles use.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gated-delta-rule fwd tokens/sec and % MFMA peak, 1×MI355X"
HEADLINE = "gdn-350m-bf16-B16-T2048-H8-d128"
PEAK_HBM_GBS = 8000.0
PEAK_MFMA = {"bf16": 2516.6, "f32": 157.3}  # dense TFLOP/s
# sources of the kernel that runs the headline workload (bf16, d_k = 128, scalar gate)
KERNEL_SOURCES = ["gated_delta_rule_20_amd/csrc/gdn_fwd_pipe.hip", "gated_delta_rule_20_amd/csrc/gdn_common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_pipe_gdn-350m.txt")
ROTATE = 4
CHUNK = 64
SETTLE_MS = 50.0  # continuous load before timing the workloads other than the headline


def alg_counts(tokens, H, dk, dv, nseq, gate, esize, has_init, has_final=True, write="delta"):
    """Algorithmic flops and bytes of the chunked method (chunk 64).

    flops per token-head: 2C(3 d_k + 2 d_v) + 6 d_k d_v + C^2/3 (Gram tiles, UT inverse,
    W and U, W M, K^T Delta, Q M, Q K^T, P Delta; multiply-add = 2).  The additive
    write has no erase: 2C(d_k + d_v) + 4 d_k d_v (Q K^T, P V, Q M, K^T V).  The
    diagonal-plus-low-rank transition ("dplr"): 4C(d_k + d_v) + 8 d_k d_v + C^2/3 (four
    lower-triangular Gram products, P_qk V, A_ak V, T R, P_qb U, Q M, A M and the two
    state products; T's inverse).
    bytes: q, k, v (and a, b for "dplr") read and o written in the I/O dtype, beta
    (delta write only) and
    log alpha in fp32 (per token for "head", per channel for "key", one value per
    head for "const"), the fp32 initial state read (if given) and final state written.
    """
    C = CHUNK
    if write == "add":
        f_th = 2 * C * (dk + dv) + 4 * dk * dv
    elif write == "dplr":
        f_th = 4 * C * (dk + dv) + 8 * dk * dv + C * C / 3.0
    else:
        f_th = 2 * C * (3 * dk + 2 * dv) + 6 * dk * dv + C * C / 3.0
    b_th = (esize * ((4 if write == "dplr" else 2) * dk + 2 * dv) + (4 if write == "delta" else 0)
            + (4 if gate == "head" else 4 * dk if gate == "key" else 0))
    state = 4 * dk * dv * nseq * H * ((1 if has_init else 0) + (1 if has_final else 0))
    return f_th * tokens * H, b_th * tokens * H + state


def kernel_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if
    the summary is missing or was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sha") != kernel_sha():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_device_inputs(inp, copies):
    import torch
    sets = []
    for _ in range(copies):
        d = {}
        for k, v in inp.items():
            d[k] = v.cuda().clone() if isinstance(v, torch.Tensor) else v
        sets.append(d)
    return sets


def time_chunked(gdn, sets, steps, warmup, settle_ms=0.0):
    """Whole-job time of `steps` calls (barrier + synchronize on both sides) after
    `warmup` untimed calls (None: as many as fill SETTLE_MS), and the average
    per-launch duration from HIP events on the launch stream.  With settle_ms > 0,
    untimed calls run first until that much wall time has passed (reported as the
    third value: the number of settle launches)."""
    import torch
    # one validated call per input copy: each timed step is a single library call
    stream = torch.cuda.current_stream()
    calls = [gdn.PreparedDplr(d["q"], d["k"], d["v"], d["a"], d["b"], d["log_alpha"], d["initial_state"],
                              d["cu_seqlens"]) if d.get("write") == "dplr" else
             gdn.PreparedFwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"],
                             d["cu_seqlens"], write=d.get("write", "delta")) for d in sets]

    def call(i):
        calls[i % len(calls)].launch(stream)

    settled = 0
    if settle_ms > 0:
        torch.cuda.synchronize()
        t_end = time.perf_counter() + settle_ms / 1e3
        while time.perf_counter() < t_end:
            for _ in range(16):
                call(settled)
                settled += 1
            torch.cuda.synchronize()
    if warmup is None:
        # enough launches for SETTLE_MS of continuous load, from one timed call
        call(0)
        torch.cuda.synchronize()
        t = time.perf_counter()
        call(1)
        torch.cuda.synchronize()
        warmup = max(2, int(SETTLE_MS / 1e3 / (time.perf_counter() - t)) + 1)
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    # HIP events on the launch stream around the whole timed region: the launches
    # run back to back, so (end - start) / steps is the average launch duration
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / steps, settled


def time_decode(gdn, spec, final_states, steps=64, cpu=False):
    import torch
    import synth
    batch = spec["decode_batch"]
    dec = synth.decode_inputs(batch, spec["H"], spec["dk"], spec["dv"], steps, spec["gate"],
                              spec["dtype"], seed=spec["seed"] + 1)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in dec.items()}
    st = synth.decode_initial_states(final_states.cpu(), batch).cuda()
    out = torch.empty((batch, spec["H"], spec["dv"]), dtype=d["q"].dtype, device="cuda")
    torch.cuda.synchronize()
    t = time.perf_counter()
    gdn.recurrent_step(d["q"][0], d["k"][0], d["v"][0], d["beta"][0], d["log_alpha"][0], st, out=out)
    torch.cuda.synchronize()
    warm = max(4, int(SETTLE_MS / 1e3 / (time.perf_counter() - t)) + 1)
    for i in range(warm):
        s = i % steps
        gdn.recurrent_step(d["q"][s], d["k"][s], d["v"][s], d["beta"][s], d["log_alpha"][s], st, out=out)
    st = synth.decode_initial_states(final_states.cpu(), batch).cuda()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        gdn.recurrent_step(d["q"][s], d["k"][s], d["v"][s], d["beta"][s], d["log_alpha"][s], st, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    bytes_step = batch * spec["H"] * (2 * 4 * spec["dk"] * spec["dv"] + 2 * (2 * spec["dk"] + 2 * spec["dv"]) + 8)
    res = {"workload": "gdn-decode-bf16-N%d-H%d-d%d" % (batch, spec["H"], spec["dk"]),
           "ms_per_step": ms, "tokens_per_s": batch / (ms / 1e3),
           "hbm_gbs": bytes_step / (ms / 1e3) / 1e9, "hbm_frac": bytes_step / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}
    if cpu:
        import oracle
        st_h = synth.decode_initial_states(final_states.cpu(), batch)
        t0 = time.perf_counter()
        oracle.step(dec["q"][0], dec["k"][0], dec["v"][0], dec["beta"][0], dec["log_alpha"][0], st_h)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": batch / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": "one decode step of all %d streams x %d heads (%.2f s)" % (batch, spec["H"], dt)}
    return res


def time_dplr_step(gdn, N=256, H=16, dk=128, dv=128, steps=64, cpu=False):
    """gdn_fwd_dplr_step, one token per stream, scalar gate, state in place (N x H states
    of d_k x d_v fp32, 268 MB at the default shape).  Algorithmic bytes per stream and
    head: the state read and written in fp32, q, k, a, b, v read and o written in bf16,
    log alpha read."""
    import torch
    import synth
    inp = synth.dplr_inputs(N, steps, H, dk, dv, "head", "bf16", seed=1107, state_std=0.02)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    tok = {k: [d[k][:, s].contiguous() for s in range(steps)] for k in ("q", "k", "v", "a", "b", "log_alpha")}
    st = d["initial_state"].clone()
    out = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda")
    call = lambda s: gdn.dplr_step(tok["q"][s], tok["k"][s], tok["v"][s], tok["a"][s], tok["b"][s],
                                   tok["log_alpha"][s], st, out=out)
    torch.cuda.synchronize()
    t = time.perf_counter()
    call(0)
    torch.cuda.synchronize()
    warm = max(4, int(SETTLE_MS / 1e3 / (time.perf_counter() - t)) + 1)
    for i in range(warm):
        call(i % steps)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        call(s)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    bytes_step = N * H * (2 * 4 * dk * dv + 2 * (4 * dk + 2 * dv) + 4)
    res = {"workload": "dplr-decode-bf16-N%d-H%d-d%d" % (N, H, dk), "ms_per_step": ms,
            "tokens_per_s": N / (ms / 1e3), "hbm_gbs": bytes_step / (ms / 1e3) / 1e9,
            "hbm_frac": bytes_step / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}
    if cpu:
        import oracle
        one = {k: (v[:, :1] if isinstance(v, torch.Tensor) and v.dim() > 1 and k != "initial_state" else v)
               for k, v in inp.items()}
        t0 = time.perf_counter()
        oracle.fwd_dplr(one["q"], one["k"], one["v"], one["a"], one["b"], one["log_alpha"], one["initial_state"],
                        nthreads=oracle.max_threads())
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": N / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
                               "sample": "one decode step of all %d streams x %d heads (%.2f s)" % (N, H, dt)}
    return res


def time_pool_decode(gdn, N, L, H, dk, dv, store, steps=64):
    """gdn_fwd_decode: L tokens for each of N streams per call, states in a pool.
    ``store="last"`` writes each stream's state back in place; ``"all"`` stores the
    state after every token into slots of its own (speculative drafts)."""
    import torch
    import synth
    P = N + (N * L if store == "all" else 0)
    inp = synth.pool_decode_inputs(N, L, H, dk, dv, P, "head", "bf16", seed=97, store=store)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    out = torch.empty((N, L, H, dv), dtype=d["q"].dtype, device="cuda")
    args = (d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["state_pool"], d["src_slots"], d["dst_slots"])
    torch.cuda.synchronize()
    t = time.perf_counter()
    gdn.decode(*args, out=out)
    torch.cuda.synchronize()
    warm = max(4, int(SETTLE_MS / 1e3 / (time.perf_counter() - t)) + 1)
    for _ in range(warm):
        gdn.decode(*args, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        gdn.decode(*args, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    state = 4 * dk * dv
    writes = 1 if store == "last" else L
    tok = 2 * (2 * dk + 2 * dv) + 8  # q, k, v, o in bf16; beta and log alpha in fp32
    nbytes = N * H * (state * (1 + writes) + L * tok)
    return {"workload": "gdn-decode-pool-bf16-N%d-L%d-H%d-d%d-store-%s" % (N, L, H, dk, store),
            "ms_per_step": ms, "tokens_per_s": N * L / (ms / 1e3), "alg_bytes": nbytes,
            "hbm_gbs": nbytes / (ms / 1e3) / 1e9, "hbm_frac": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}


def time_dplr_pool_decode(gdn, N=256, L=4, H=16, dk=128, dv=128, steps=64):
    """gdn_fwd_dplr_decode: L tokens for each of N streams per call, scalar gate, each
    stream's state read from and written back to its own pool slot.  Algorithmic bytes:
    the state read and written once per call in fp32, and per token q, k, a, b, v read
    and o written in bf16 and log alpha read."""
    import torch
    import synth
    inp = synth.dplr_inputs(N, L, H, dk, dv, "head", "bf16", seed=1207, state_std=0.02)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    pool = d["initial_state"].clone()
    src = torch.arange(N, dtype=torch.int32, device="cuda")
    dst = torch.full((N, L), -1, dtype=torch.int32, device="cuda")
    dst[:, L - 1] = src
    out = torch.empty((N, L, H, dv), dtype=torch.bfloat16, device="cuda")
    args = (d["q"], d["k"], d["v"], d["a"], d["b"], d["log_alpha"], pool, src, dst)
    torch.cuda.synchronize()
    t = time.perf_counter()
    gdn.dplr_decode(*args, out=out)
    torch.cuda.synchronize()
    warm = max(4, int(SETTLE_MS / 1e3 / (time.perf_counter() - t)) + 1)
    for _ in range(warm):
        gdn.dplr_decode(*args, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        gdn.dplr_decode(*args, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = N * H * (2 * 4 * dk * dv + L * (2 * (4 * dk + 2 * dv) + 4))
    return {"workload": "dplr-decode-pool-bf16-N%d-L%d-H%d-d%d-in-place" % (N, L, H, dk), "ms_per_step": ms,
            "tokens_per_s": N * L / (ms / 1e3), "alg_bytes": nbytes, "hbm_gbs": nbytes / (ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}


def time_bwd(gdn, name, steps=20, cpu=False):
    """gdn_bwd_chunked on a workload: the gradients of o and of the final state are
    seeded N(0,1) and N(0, 0.1^2).  Algorithmic bytes: q, k, v, dout read and dq, dk,
    dv written in the I/O dtype, beta (delta write) and a per-token log alpha read and
    their gradients written in fp32, the initial state and the final-state gradient
    read and the initial-state gradient written in fp32.  Algorithmic flops: the
    forward recomputation (as for the forward) plus, per token and head, 14 C d_k +
    10 C d_v + 14 d_k d_v + 4 C^2 for the delta write's backward products, or 6 C d_k
    + 4 C d_v + 8 d_k d_v for the additive write's (each product counted once)."""
    import torch
    import synth
    spec = synth.WORKLOADS[name]
    inp = synth.workload_inputs(name)
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    g = torch.Generator().manual_seed(spec["seed"] + 77)
    dout_h = torch.randn(B, T, H, dv, generator=g).to(inp["q"].dtype)
    dfs_h = torch.randn(inp["N"], H, dk, dv, generator=g) * 0.1
    dout, dfs = dout_h.cuda(), dfs_h.cuda()
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    write = inp.get("write", "delta")
    call = gdn.PreparedBwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["initial_state"], dout, dfs,
                           d["cu_seqlens"], write=write)
    torch.cuda.synchronize()
    t = time.perf_counter()
    call.launch()
    torch.cuda.synchronize()
    warm = max(2, int(SETTLE_MS / 1e3 / (time.perf_counter() - t)) + 1)
    for _ in range(warm):
        call.launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call.launch()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tokens = B * T
    esize = 2 if spec["dtype"] == "bf16" else 4
    th = tokens * H
    per_tok = (8 if write == "delta" else 0) + (8 if spec["gate"] == "head" else 8 * dk if spec["gate"] == "key" else 0)
    # dfinal read, dinit written, and the initial state read when there is one
    nstate = (2 + (1 if inp["initial_state"] is not None else 0)) * 4 * dk * dv * inp["N"] * H
    nbytes = th * (esize * (4 * dk + 3 * dv) + per_tok) + nstate
    fwd_flops, _ = alg_counts(tokens, H, dk, dv, inp["N"], spec["gate"], esize, True, write=write)
    if write == "add":
        flops = fwd_flops + th * (6 * CHUNK * dk + 4 * CHUNK * dv + 8 * dk * dv)
    else:
        flops = fwd_flops + th * (14 * CHUNK * dk + 10 * CHUNK * dv + 14 * dk * dv + 4 * CHUNK * CHUNK)
    res = {"workload": name + " backward", "ms_per_step": ms, "tokens_per_s": tokens / (ms / 1e3),
            "alg_bytes": nbytes, "hbm_gbs": nbytes / (ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, "alg_flops": flops,
            "tflops": flops / (ms / 1e3) / 1e12}
    if cpu:
        res["cpu_baseline"] = cpu_baseline_sample(dict(inp, dout=dout_h, dfinal=dfs_h), "bwd", max_tokens=8192)
    return res


def cpu_baseline(inp, H):
    """The fp64 oracle on the host cores, on the whole workload (bounded: a few
    seconds), best of two runs."""
    import oracle
    threads = oracle.max_threads()
    best = None
    for _ in range(2):
        t0 = time.perf_counter()
        oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["initial_state"],
                   inp["cu_seqlens"], nthreads=threads)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    tokens = inp["q"].shape[0] * inp["q"].shape[1]
    return {"value": tokens / best, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "whole workload (%d tokens x %d heads), fp64 token-by-token recurrence, "
                      "OpenMP over (sequence, head), best of 2 runs (%.2f s)" % (tokens, H, best)}


def _leading(inp, max_tokens):
    """The leading batch rows (or packed sequences) of a workload, up to max_tokens
    tokens (at least one row or sequence), all heads: (sliced inputs, tokens, text)."""
    import torch
    out = dict(inp)
    s0 = inp.get("initial_state")
    if inp.get("cu_seqlens") is None:
        B, T = inp["q"].shape[:2]
        nb = max(1, min(B, max_tokens // max(T, 1)))
        for k in ("q", "k", "v", "a", "b", "beta", "log_alpha", "dout"):
            if out.get(k) is not None and out[k].dim() > 1:
                out[k] = out[k][:nb]
        out["initial_state"] = None if s0 is None else s0[:nb]
        return out, nb * T, "the first %d of %d batch rows" % (nb, B)
    cu = [int(x) for x in inp["cu_seqlens"]]
    n = 1
    while n < len(cu) - 1 and cu[n + 1] <= max_tokens:
        n += 1
    for k in ("q", "k", "v", "a", "b", "beta", "log_alpha", "dout"):
        if out.get(k) is not None and out[k].dim() > 1:
            out[k] = out[k][:, :cu[n]]
    out["cu_seqlens"] = torch.tensor(cu[:n + 1], dtype=torch.int32)
    out["initial_state"] = None if s0 is None else s0[:n]
    return out, cu[n], "the first %d of %d packed sequences" % (n, len(cu) - 1)


def cpu_baseline_sample(inp, kind="fwd", max_tokens=32768):
    """The fp64 oracle timed beside a GPU line, on a bounded sample of the same workload
    (leading rows or sequences, all heads; one run of a few seconds on the host cores):
    kind "fwd" (oracle.fwd, either write rule), "dplr" (oracle.fwd_dplr) or "bwd"
    (oracle.bwd, with inp["dout"] and inp["dfinal"])."""
    import oracle
    threads = oracle.max_threads()
    smp, tokens, text = _leading(inp, max_tokens)
    H = inp["q"].shape[2]
    t0 = time.perf_counter()
    if kind == "dplr":
        oracle.fwd_dplr(smp["q"], smp["k"], smp["v"], smp["a"], smp["b"], smp["log_alpha"], smp["initial_state"],
                        smp["cu_seqlens"], nthreads=threads)
    elif kind == "bwd":
        dfinal = smp.get("dfinal")
        if dfinal is not None and smp["initial_state"] is not None:
            dfinal = dfinal[:smp["initial_state"].shape[0]]
        oracle.bwd(smp["q"], smp["k"], smp["v"], smp["beta"], smp["log_alpha"], smp["initial_state"], smp["dout"],
                   dfinal, cu_seqlens=smp["cu_seqlens"], nthreads=threads, write=smp.get("write", "delta"))
    else:
        oracle.fwd(smp["q"], smp["k"], smp["v"], smp["beta"], smp["log_alpha"], smp["initial_state"],
                   smp["cu_seqlens"], nthreads=threads, write=smp.get("write", "delta"))
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%s (%d tokens x %d heads), one run (%.2f s)" % (text, tokens, H, dt)}


def bench_workload(gdn, name, steps, warmup, settle_ms=0.0):
    import synth
    spec = synth.WORKLOADS[name]
    inp = synth.workload_inputs(name)
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    sets = make_device_inputs(inp, ROTATE)
    wall, launch_ms, settled = time_chunked(gdn, sets, steps, warmup, settle_ms)
    tokens = B * T
    esize = 2 if spec["dtype"] == "bf16" else 4
    flops, nbytes = alg_counts(tokens, H, dk, dv, inp["N"], spec["gate"], esize,
                               inp["initial_state"] is not None, write=spec.get("write", "delta"))
    res = {"workload": name, "ms_per_step": wall / steps * 1e3, "launch_ms": launch_ms,
           "tokens_per_s": tokens / (wall / steps), "alg_flops": flops, "alg_bytes": nbytes,
           "tflops": flops / (launch_ms / 1e3) / 1e12,
           "mfma_frac": flops / (launch_ms / 1e3) / 1e12 / PEAK_MFMA["f32" if spec.get("write") == "dplr"
                                                                     else spec["dtype"]],
           "hbm_gbs": nbytes / (launch_ms / 1e3) / 1e9,
           "hbm_frac": nbytes / (launch_ms / 1e3) / 1e9 / PEAK_HBM_GBS, "settle_launches": settled}
    return res, inp, sets


def calibrate_copy(mib):
    """Two launches of a plain elementwise kernel reading `mib` MiB once and writing them
    once: the known-size reference for the HBM byte counters of a profile run."""
    if not mib:
        return
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=600,
                    help="untimed launches before the timed ones (after the settle phase)")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed launches for this much wall time first, so that the power "
                         "controller has settled before the warm-up and timed steps (0: none)")
    ap.add_argument("--all", action="store_true", help="also report every workload (extra lines on stderr)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only", default=None, metavar="WORKLOAD[:bwd]",
                    help="run only this workload (forward, or backward with ':bwd') and print its line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after timing, run twice a plain elementwise kernel that reads MIB MiB once "
                         "and writes them once: the known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_20_amd as gdn
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.only:
        name, _, part = args.only.partition(":")
        if name not in synth.WORKLOADS:
            sys.exit("unknown workload %r; known: %s" % (name, ", ".join(sorted(synth.WORKLOADS))))
        if part == "bwd":
            r = time_bwd(gdn, name, steps=args.steps)
        else:
            r, _, _ = bench_workload(gdn, name, args.steps, args.warmup, args.settle_ms)
        calibrate_copy(args.calibrate_copy)
        print(json.dumps(r))
        return

    res, inp, sets = bench_workload(gdn, HEADLINE, args.steps, args.warmup, args.settle_ms)
    spec = synth.WORKLOADS[HEADLINE]
    B, T, H, dk = inp["q"].shape
    achieved = res["alg_bytes"] / (res["launch_ms"] / 1e3) / 1e9
    step_s = res["ms_per_step"] / 1e3
    traffic = read_traffic()
    line = {
        "metric": METRIC,
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k L2-normalised, v; sigmoid beta; -softplus*exp(U) "
                "log decay; N(0,0.02^2) initial state)",
        "config": {"workload": HEADLINE, "B": B, "T": T, "H": H, "d_k": dk, "d_v": inp["v"].shape[-1],
                   "chunk": CHUNK, "gate": spec["gate"], "initial_state": True,
                   "rotated_input_copies": ROTATE},
        "settle": {"wall_ms": args.settle_ms, "launches": res["settle_launches"],
                   "note": "untimed headline launches before the warm-up, so that the GPU's power "
                           "controller has settled"},
        "tflops": res["alg_flops"] / step_s / 1e12,
        "mfma_peak_frac": res["alg_flops"] / step_s / 1e12 / PEAK_MFMA["bf16"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "launch_ms": res["launch_ms"],
                     "frac_at_ms_per_step": res["alg_bytes"] / step_s / 1e9 / PEAK_HBM_GBS,
                     "alg_bytes": res["alg_bytes"], "traffic": traffic},
    }
    calibrate_copy(args.calibrate_copy)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(inp, H)
    if args.all:
        extra = []
        del sets
        torch.cuda.empty_cache()
        for name in ["gdn-bf16-B4-T2048-H8-d128", "kda-bf16-B2-T16384-H16-d128",
                     "gdn-varlen-bf16-N32-H16-d128", "deltanet-fp32-B1-T256-H2-d64",
                     "retnet-bf16-B16-T2048-H8-d128", "gla-bf16-B2-T16384-H16-d128",
                     "dplr-bf16-B16-T2048-H8-d128", "dplr-key-bf16-B16-T2048-H8-d128"]:
            try:
                r, winp, wsets = bench_workload(gdn, name, max(5, args.steps // 5), None)
                if not args.no_cpu:
                    r["cpu_baseline"] = cpu_baseline_sample(winp, "dplr" if winp.get("write") == "dplr" else "fwd")
            except RuntimeError as e:
                extra.append({"workload": name, "error": str(e)})
                continue
            if name.startswith("gdn-varlen"):
                d = wsets[0]
                _, fs = gdn.fwd_chunked(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], None,
                                        d["cu_seqlens"])
                torch.cuda.synchronize()
                extra.append(time_decode(gdn, synth.WORKLOADS[name], fs, cpu=not args.no_cpu))
                del fs
                for store in ("last", "all"):
                    extra.append(time_pool_decode(gdn, 256, 4, 16, 128, 128, store))
            del wsets
            torch.cuda.empty_cache()
            extra.append(r)
        extra.append(time_dplr_step(gdn, cpu=not args.no_cpu))
        extra.append(time_dplr_pool_decode(gdn))
        torch.cuda.empty_cache()
        extra.append(time_bwd(gdn, HEADLINE, cpu=not args.no_cpu))
        torch.cuda.empty_cache()
        extra.append(time_bwd(gdn, "retnet-bf16-B16-T2048-H8-d128", cpu=not args.no_cpu))
        torch.cuda.empty_cache()
        # (no CPU line: the oracle's reverse sweep keeps 2 GB of states per sequence and head here)
        extra.append(time_bwd(gdn, "kda-bf16-B2-T16384-H16-d128", steps=5))
        torch.cuda.empty_cache()
        extra.append(time_bwd(gdn, "gla-bf16-B2-T16384-H16-d128", steps=5))
        torch.cuda.empty_cache()
        for e in extra:
            print(json.dumps(e), file=sys.stderr)
    print(json.dumps(line))


if __name__ == "__main__":
    main()

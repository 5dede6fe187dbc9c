"""fp64 CPU oracle for the (gated) delta-rule forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and it
shares no code with that library: the arithmetic lives in ``gdn_oracle.c``
(token-by-token recurrence, see that file's header for the passages it follows)
and ``chunked_ref.py`` (the chunkwise form, used only to pin the chunk
equations).  This module only converts arrays to fp64 and calls the C code.

Parity status: every function here is pinned.  ``fwd`` and ``step`` by
``tests/test_oracle_pins.py`` (closed forms, invariants, an autograd-derived
gradient step, exact rational fixtures under ``tests/golden/`` and planted-mistake
checks); ``decode_pool`` by ``tests/test_oracle_decode.py`` (against ``fwd`` over
the same tokens and over every stored prefix, chained and speculative calls); ``bwd``
by ``tests/test_oracle_bwd.py`` and, for the additive write,
``tests/test_oracle_bwd_additive.py`` (central finite differences of ``fwd`` and torch
autograd of the recurrence in fp64, planted mutants); ``fwd_dplr`` by ``tests/test_oracle_dplr.py``
(reduces exactly to the delta rule and to the additive write, and equals the
product of the dense transition matrices); the
additive write (``write="add"``) and the constant per-head gate by
``tests/test_oracle_additive.py`` (RetNet's decay-mask parallel form, the
gated-linear-attention brute-force sum, the plain linear-transformer sum, agreement
with the delta rule on orthonormal keys, linearity and a planted mutant).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

GATES = {"none": 0, "head": 1, "key": 2}
WRITES = {"delta": 0, "add": 1}


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the C oracle with gcc (OpenMP, -O2) into a shared library."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load (building first if needed) the oracle library; returns the ctypes handle."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        _lib = _declare(ctypes.CDLL(build()))
    return _lib


def _declare(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_fwd.restype = ctypes.c_int
    lib.oracle_fwd.argtypes = [ctypes.c_int, ip, ip, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.oracle_step.restype = ctypes.c_int
    lib.oracle_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_bwd.restype = ctypes.c_int
    lib.oracle_bwd.argtypes = [ctypes.c_int, ip, ip, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.oracle_fwd_dplr.restype = ctypes.c_int
    lib.oracle_fwd_dplr.argtypes = [ctypes.c_int, ip, ip, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (CPU); upcast exactly, as the GPU sees the same bits
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def infer_gate(log_alpha, token_ndim: int) -> str:
    if log_alpha is None:
        return "none"
    if np.ndim(log_alpha) == 1:
        return "const"
    return "head" if np.ndim(log_alpha) == token_ndim else "key"


def _per_token(log_alpha, lead):
    """A constant per-head log decay [H] as the same value at every token position
    [*lead, H] (a layout change only)."""
    return np.ascontiguousarray(np.broadcast_to(log_alpha, tuple(lead) + log_alpha.shape))


def fwd(q, k, v, beta, log_alpha=None, initial_state=None, cu_seqlens=None, gate=None,
        nthreads: int = 0, lib=None, write: str = "delta"):
    """Run the recurrence over whole sequences.

    Batch mode: q,k [B,T,H,d_k], v [B,T,H,d_v], beta [B,T,H] (None with the additive
    write), log_alpha None | [H] (one constant decay per head) | [B,T,H] | [B,T,H,d_k];
    varlen mode: B == 1 and ``cu_seqlens`` (N+1 offsets).  ``initial_state`` None
    (zeros) or [N,H,d_k,d_v] with M = S^T.  ``write``: "delta" (erase, then write) or
    "add" (M += k v^T).
    Returns (o [B,T,H,d_v], final_state [N,H,d_k,d_v]) as fp64 numpy arrays.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    log_alpha, initial_state = _f64(log_alpha), _f64(initial_state)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if gate is None:
        gate = infer_gate(log_alpha, 3)
    if gate == "const":
        log_alpha, gate = _per_token(log_alpha, (B, T)), "head"
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64)
        assert B == 1 and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
        start, lens = cu[:-1].copy(), np.diff(cu)
    else:
        start = np.arange(B, dtype=np.int64) * T
        lens = np.full(B, T, dtype=np.int64)
    N = len(start)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    fs = np.zeros((N, H, dk, dv), dtype=np.float64)
    lib = lib or load()
    rc = lib.oracle_fwd(N, start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                        lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
                        GATES[gate], WRITES[write], _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
                        _ptr(initial_state), _ptr(o), _ptr(fs), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_fwd failed (%d)" % rc)
    return o, fs


def bwd(q, k, v, beta, log_alpha, initial_state, dout, dfinal=None, cu_seqlens=None, gate=None,
        nthreads: int = 0, lib=None, write: str = "delta"):
    """Gradients of the recurrence (the delta write, or the additive write with beta
    None; no gate, one decay per (token, head), one per (token, head, key channel), or one
    constant decay per head [H]) with
    respect to q, k, v, beta, log_alpha and the initial state, given dout [B,T,H,d_v]
    (the gradient of o) and dfinal None | [N,H,d_k,d_v] (the gradient of the final
    state).  Shapes as for ``fwd``.  Returns (dq, dk, dv, dbeta or None, dlog_alpha or
    None, dinit [N,H,d_k,d_v]) in fp64; for the constant gate dlog_alpha is [H] (the
    per-token gradients summed)."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    log_alpha, initial_state, dout, dfinal = _f64(log_alpha), _f64(initial_state), _f64(dout), _f64(dfinal)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if gate is None:
        gate = infer_gate(log_alpha, 3)
    const = gate == "const"
    if const:
        log_alpha, gate = _per_token(log_alpha, (B, T)), "head"
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64)
        start, lens = cu[:-1].copy(), np.diff(cu)
    else:
        start = np.arange(B, dtype=np.int64) * T
        lens = np.full(B, T, dtype=np.int64)
    N = len(start)
    dq, dk_ = np.zeros_like(q), np.zeros_like(k)
    dv_ = np.zeros_like(v)
    db = None if write == "add" else np.zeros_like(beta)
    dla = np.zeros((B, T, H)) if gate == "head" else np.zeros((B, T, H, dk)) if gate == "key" else None
    dinit = np.zeros((N, H, dk, dv))
    lib = lib or load()
    rc = lib.oracle_bwd(N, start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                        lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv, GATES[gate],
                        WRITES[write], _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(initial_state),
                        _ptr(dout), _ptr(dfinal), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(db), _ptr(dla),
                        _ptr(dinit), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_bwd failed (%d)" % rc)
    if const:
        dla = dla.sum(axis=(0, 1))
    return dq, dk_, dv_, db, dla, dinit


def fwd_dplr(q, k, v, a, b, log_alpha=None, initial_state=None, cu_seqlens=None, gate=None,
             nthreads: int = 0, lib=None):
    """The diagonal-plus-low-rank transition M_t = Diag(alpha_t) M_{t-1} + b_t (a_t^T
    M_{t-1}) + k_t v_t^T, o_t = M_t^T q_t, over whole sequences.  q, k, a, b
    [B,T,H,d_k], v [B,T,H,d_v], log_alpha None | [H] (one constant decay per head) |
    [B,T,H] | [B,T,H,d_k]; other arguments as for ``fwd``.  Returns (o, final_state) in
    fp64."""
    q, k, v, a, b = _f64(q), _f64(k), _f64(v), _f64(a), _f64(b)
    log_alpha, initial_state = _f64(log_alpha), _f64(initial_state)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if gate is None:
        gate = infer_gate(log_alpha, 3)
    if gate == "const":
        log_alpha, gate = _per_token(log_alpha, (B, T)), "head"
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64)
        start, lens = cu[:-1].copy(), np.diff(cu)
    else:
        start = np.arange(B, dtype=np.int64) * T
        lens = np.full(B, T, dtype=np.int64)
    N = len(start)
    o = np.zeros((B, T, H, dv))
    fs = np.zeros((N, H, dk, dv))
    lib = lib or load()
    rc = lib.oracle_fwd_dplr(N, start.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                             lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv, GATES[gate],
                             _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha), _ptr(initial_state),
                             _ptr(o), _ptr(fs), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_fwd_dplr failed (%d)" % rc)
    return o, fs


def step(q, k, v, beta, log_alpha, state, gate=None, lib=None, write: str = "delta"):
    """One token per stream: q,k [N,H,d_k], v [N,H,d_v], beta [N,H] (None with the
    additive write), log_alpha None | [H] | [N,H] | [N,H,d_k], state [N,H,d_k,d_v].
    Returns (o [N,H,d_v], new_state)."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    log_alpha = _f64(log_alpha)
    st = _f64(state).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    if gate is None:
        gate = infer_gate(log_alpha, 2)
    if gate == "const":
        log_alpha, gate = _per_token(log_alpha, (N,)), "head"
    o = np.zeros((N, H, dv), dtype=np.float64)
    lib = lib or load()
    rc = lib.oracle_step(N, H, dk, dv, GATES[gate], WRITES[write], _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                         _ptr(log_alpha), _ptr(st), _ptr(o))
    if rc != 0:
        raise RuntimeError("oracle_step failed (%d)" % rc)
    return o, st


def decode_pool(q, k, v, beta, log_alpha, pool, src_slots, dst_slots, gate=None, lib=None,
                write: str = "delta"):
    """L decode tokens per stream against a pool of states, by repeated ``step``.

    q,k [N,L,H,d_k], v [N,L,H,d_v], beta [N,L,H] (None with the additive write),
    log_alpha None | [H] | [N,L,H] | [N,L,H,d_k]; pool [P,H,d_k,d_v] (M = S^T);
    src_slots [N] and dst_slots [N,L]
    integers.  Stream n is active when 0 <= src_slots[n] < P: its state is read from
    that slot (all reads happen before any write), its L tokens run through the
    recurrence in order, and the state after token t is stored into slot
    dst_slots[n, t] when that is in [0, P).  Inactive streams read and write nothing.
    Returns (o [N,L,H,d_v] with NaN rows for inactive streams, the pool afterwards),
    both fp64.  Writes land in (stream, token) order.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    log_alpha, pool = _f64(log_alpha), _f64(pool)
    src = np.asarray(src_slots.cpu() if hasattr(src_slots, "cpu") else src_slots, dtype=np.int64)
    dst = np.asarray(dst_slots.cpu() if hasattr(dst_slots, "cpu") else dst_slots, dtype=np.int64)
    N, L, H, dk = q.shape
    dv = v.shape[-1]
    P = pool.shape[0]
    if gate is None:
        gate = infer_gate(log_alpha, 3)
    if gate == "const":
        log_alpha, gate = _per_token(log_alpha, (N, L)), "head"
    o = np.full((N, L, H, dv), np.nan)
    out = pool.copy()
    act = np.nonzero((src >= 0) & (src < P))[0]
    if len(act) == 0:
        return o, out
    states = pool[src[act]].copy()  # every read before any write
    for t in range(L):
        la = None if log_alpha is None else log_alpha[act, t]
        bt = None if beta is None else beta[act, t]
        o_t, states = step(q[act, t], k[act, t], v[act, t], bt, la, states, gate=gate, lib=lib, write=write)
        o[act, t] = o_t
        for j, n in enumerate(act):
            if 0 <= dst[n, t] < P:
                out[dst[n, t]] = states[j]
    return o, out


def max_threads() -> int:
    return load().oracle_max_threads()

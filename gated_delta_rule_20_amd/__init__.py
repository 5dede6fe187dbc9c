"""MI355X (gfx950) chunked gated delta-rule forward -- Python binding.

Thin ctypes marshalling over the C ABI of ``include/gdn.h`` (``libgdn.so``, built
in-tree by ``gated_delta_rule_20_amd/build.py``).  Every step of the computation
runs in the library's HIP kernels; PyTorch only supplies device memory and the
current stream.  There is no fallback: if the library is missing this module
raises on import.

The names follow the C ABI: ``fwd_chunked`` wraps ``gdn_fwd_chunked``,
``fwd_chunked_static`` wraps ``gdn_fwd_chunked_static`` (the same forward with the
library's own per-GPU scratch array instead of a workspace), ``recurrent_step`` wraps
``gdn_fwd_recurrent_step``, ``decode`` wraps
``gdn_fwd_decode``, ``bwd_chunked`` wraps ``gdn_bwd_chunked``, ``fwd_dplr`` wraps
``gdn_fwd_dplr``, ``dplr_step`` wraps ``gdn_fwd_dplr_step`` and ``dplr_decode`` wraps
``gdn_fwd_dplr_decode``.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "gdn.h")

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = 0, -1, -2, -3, -4
GDN_F32, GDN_BF16 = 0, 1
GDN_GATE_NONE, GDN_GATE_HEAD, GDN_GATE_KEY, GDN_GATE_HEAD_CONST = 0, 1, 2, 3
GDN_WRITE_DELTA, GDN_WRITE_ADD = 0, 1
WRITES = {"delta": GDN_WRITE_DELTA, "add": GDN_WRITE_ADD}
CHUNK = 64


class FwdArgs(ctypes.Structure):
    """Mirror of ``gdn_fwd_args``."""
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("d_k", ctypes.c_int), ("d_v", ctypes.c_int), ("chunk", ctypes.c_int),
                ("N", ctypes.c_int), ("dtype", ctypes.c_int), ("gate", ctypes.c_int),
                ("write", ctypes.c_int),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p),
                ("initial_state", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class StepArgs(ctypes.Structure):
    """Mirror of ``gdn_step_args``."""
    _fields_ = [("N", ctypes.c_int), ("H", ctypes.c_int), ("d_k", ctypes.c_int),
                ("d_v", ctypes.c_int), ("dtype", ctypes.c_int), ("gate", ctypes.c_int),
                ("write", ctypes.c_int),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p),
                ("state", ctypes.c_void_p), ("o", ctypes.c_void_p)]


class DecodeArgs(ctypes.Structure):
    """Mirror of ``gdn_decode_args``."""
    _fields_ = [("N", ctypes.c_int), ("L", ctypes.c_int), ("H", ctypes.c_int),
                ("d_k", ctypes.c_int), ("d_v", ctypes.c_int), ("dtype", ctypes.c_int),
                ("gate", ctypes.c_int), ("write", ctypes.c_int), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p),
                ("state_pool", ctypes.c_void_p), ("pool_size", ctypes.c_int),
                ("src_slots", ctypes.c_void_p), ("dst_slots", ctypes.c_void_p), ("o", ctypes.c_void_p)]


class BwdArgs(ctypes.Structure):
    """Mirror of ``gdn_bwd_args``."""
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("d_k", ctypes.c_int), ("d_v", ctypes.c_int), ("chunk", ctypes.c_int),
                ("N", ctypes.c_int), ("dtype", ctypes.c_int), ("gate", ctypes.c_int),
                ("write", ctypes.c_int),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p),
                ("initial_state", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("dout", ctypes.c_void_p), ("dfinal_state", ctypes.c_void_p),
                ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("dbeta", ctypes.c_void_p), ("dlog_alpha", ctypes.c_void_p),
                ("dinitial_state", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class DplrArgs(ctypes.Structure):
    """Mirror of ``gdn_dplr_args``."""
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("d_k", ctypes.c_int), ("d_v", ctypes.c_int), ("chunk", ctypes.c_int),
                ("N", ctypes.c_int), ("dtype", ctypes.c_int), ("gate", ctypes.c_int),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("a", ctypes.c_void_p),
                ("b", ctypes.c_void_p), ("v", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p),
                ("initial_state", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class DplrStepArgs(ctypes.Structure):
    """Mirror of ``gdn_dplr_step_args``."""
    _fields_ = [("N", ctypes.c_int), ("H", ctypes.c_int), ("d_k", ctypes.c_int), ("d_v", ctypes.c_int),
                ("dtype", ctypes.c_int), ("gate", ctypes.c_int),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p), ("state", ctypes.c_void_p),
                ("o", ctypes.c_void_p)]


class DplrDecodeArgs(ctypes.Structure):
    """Mirror of ``gdn_dplr_decode_args``."""
    _fields_ = [("N", ctypes.c_int), ("L", ctypes.c_int), ("H", ctypes.c_int), ("d_k", ctypes.c_int),
                ("d_v", ctypes.c_int), ("dtype", ctypes.c_int), ("gate", ctypes.c_int),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p), ("state_pool", ctypes.c_void_p),
                ("pool_size", ctypes.c_int), ("src_slots", ctypes.c_void_p), ("dst_slots", ctypes.c_void_p),
                ("o", ctypes.c_void_p)]


def load_library(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError("libgdn.so is not built (%s); run `python __graft_entry__.py build` "
                          "or gated_delta_rule_20_amd/build.py" % path)
    lib = ctypes.CDLL(path)
    lib.gdn_fwd_workspace_size.restype = ctypes.c_size_t
    lib.gdn_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdArgs)]
    lib.gdn_fwd_chunked.restype = ctypes.c_int
    lib.gdn_fwd_chunked.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
    lib.gdn_fwd_chunked_static.restype = ctypes.c_int
    lib.gdn_fwd_chunked_static.argtypes = [ctypes.POINTER(FwdArgs), ctypes.c_void_p]
    lib.gdn_fwd_recurrent_step.restype = ctypes.c_int
    lib.gdn_fwd_recurrent_step.argtypes = [ctypes.POINTER(StepArgs), ctypes.c_void_p]
    lib.gdn_fwd_decode.restype = ctypes.c_int
    lib.gdn_fwd_decode.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
    lib.gdn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.gdn_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdArgs)]
    lib.gdn_bwd_chunked.restype = ctypes.c_int
    lib.gdn_bwd_chunked.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p]
    lib.gdn_fwd_dplr_decode.restype = ctypes.c_int
    lib.gdn_fwd_dplr_decode.argtypes = [ctypes.POINTER(DplrDecodeArgs), ctypes.c_void_p]
    lib.gdn_fwd_dplr_step.restype = ctypes.c_int
    lib.gdn_fwd_dplr_step.argtypes = [ctypes.POINTER(DplrStepArgs), ctypes.c_void_p]
    lib.gdn_dplr_workspace_size.restype = ctypes.c_size_t
    lib.gdn_dplr_workspace_size.argtypes = [ctypes.POINTER(DplrArgs)]
    lib.gdn_fwd_dplr.restype = ctypes.c_int
    lib.gdn_fwd_dplr.argtypes = [ctypes.POINTER(DplrArgs), ctypes.c_void_p]
    lib.gdn_status_str.restype = ctypes.c_char_p
    lib.gdn_status_str.argtypes = [ctypes.c_int]
    lib.gdn_version.restype = ctypes.c_int
    return lib


# torch ships its own HIP runtime (soname libamdhip64.so.7).  Loading torch first makes
# libgdn.so bind to that same runtime; loaded the other way round, the process ends up
# with two runtimes and the second one finds no device.
import torch  # noqa: E402,F401

_lib = load_library()


def header_functions(path: str = HEADER_PATH):
    """Names of the functions declared in include/gdn.h."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, re.M)))


def status_str(status: int) -> str:
    return _lib.gdn_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != GDN_OK:
        raise RuntimeError("%s failed: %s (%d)" % (what, status_str(status), status))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require(cond, msg: str):
    if not cond:
        raise ValueError(msg)


def _same_device(tensors, ref):
    for name, t in tensors:
        if t is not None:
            _require(t.is_cuda and t.device == ref.device,
                      "%s must be on the GPU device of q (%s), got %s" % (name, ref.device, t.device))


def _check_write(write):
    _require(write in WRITES, "write must be 'delta' or 'add'")
    return WRITES[write]


def check_fwd_tensors(q, k, v, beta, log_alpha=None, initial_state=None, cu_seqlens=None,
                      out=None, final_state=None, write="delta"):
    """Host-side shape, dtype and layout checks for fwd_chunked.

    The C ABI receives bare pointers and sizes, so the shapes it is told must be
    the shapes of the buffers; this raises ValueError on any mismatch before a
    pointer is handed over.  Device placement is checked last."""
    import torch
    named = [("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
             ("initial_state", initial_state), ("cu_seqlens", cu_seqlens), ("out", out),
             ("final_state", final_state)]
    _require(q.dim() == 4, "q must be [B, T, H, d_k], got shape %s" % (tuple(q.shape),))
    B, T, H, dk = q.shape
    _require(q.dtype in (torch.bfloat16, torch.float32), "q must be bfloat16 or float32")
    _require(tuple(k.shape) == (B, T, H, dk), "k must have the shape of q")
    _require(v.dim() == 4 and tuple(v.shape[:3]) == (B, T, H), "v must be [B, T, H, d_v]")
    dv = v.shape[3]
    _require(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share one dtype")
    _check_write(write)
    if write == "add":
        _require(beta is None, "beta must be None with the additive write")
    else:
        _require(beta is not None and tuple(beta.shape) == (B, T, H) and beta.dtype == torch.float32,
                 "beta must be float32 [B, T, H]")
    if log_alpha is not None:
        _require(log_alpha.dtype == torch.float32, "log_alpha must be float32")
        _require(tuple(log_alpha.shape) in ((H,), (B, T, H), (B, T, H, dk)),
                 "log_alpha must be [H] (one constant decay per head), [B, T, H] (one decay per "
                 "token and head) or [B, T, H, d_k]")
    if cu_seqlens is not None:
        _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2,
                 "cu_seqlens must be int32 [N + 1] with N >= 1")
        _require(B == 1, "packed sequences (cu_seqlens) need B == 1")
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _require(tuple(t.shape) == (N, H, dk, dv) and t.dtype == torch.float32,
                     "%s must be float32 [N, H, d_k, d_v] = %s" % (name, (N, H, dk, dv)))
    if out is not None:
        _require(tuple(out.shape) == (B, T, H, dv) and out.dtype == q.dtype,
                 "out must be [B, T, H, d_v] in the dtype of q")
    for name, t in named:
        if t is not None:
            _require(t.is_contiguous(), "%s must be contiguous" % name)
    _same_device(named, q)
    return N


def check_step_tensors(q, k, v, beta, log_alpha, state, out=None, write="delta"):
    """Host-side checks for recurrent_step (see check_fwd_tensors)."""
    import torch
    named = [("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
             ("state", state), ("out", out)]
    _require(q.dim() == 3, "q must be [N, H, d_k]")
    N, H, dk = q.shape
    _require(q.dtype in (torch.bfloat16, torch.float32), "q must be bfloat16 or float32")
    _require(tuple(k.shape) == (N, H, dk), "k must have the shape of q")
    _require(v.dim() == 3 and tuple(v.shape[:2]) == (N, H), "v must be [N, H, d_v]")
    dv = v.shape[2]
    _require(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share one dtype")
    _check_write(write)
    if write == "add":
        _require(beta is None, "beta must be None with the additive write")
    else:
        _require(beta is not None and tuple(beta.shape) == (N, H) and beta.dtype == torch.float32,
                 "beta must be float32 [N, H]")
    if log_alpha is not None:
        _require(log_alpha.dtype == torch.float32 and tuple(log_alpha.shape) in ((H,), (N, H), (N, H, dk)),
                 "log_alpha must be float32 [H], [N, H] or [N, H, d_k]")
    _require(tuple(state.shape) == (N, H, dk, dv) and state.dtype == torch.float32,
             "state must be float32 [N, H, d_k, d_v]")
    if out is not None:
        _require(tuple(out.shape) == (N, H, dv) and out.dtype == q.dtype, "out must be [N, H, d_v]")
    for name, t in named:
        if t is not None:
            _require(t.is_contiguous(), "%s must be contiguous" % name)
    _same_device(named, q)


def check_decode_tensors(q, k, v, beta, log_alpha, state_pool, src_slots, dst_slots, out=None, write="delta"):
    """Host-side checks for decode (see check_fwd_tensors).  Slot values live on the
    device and are not inspected here."""
    import torch
    named = [("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
             ("state_pool", state_pool), ("src_slots", src_slots), ("dst_slots", dst_slots), ("out", out)]
    _require(q.dim() == 4, "q must be [N, L, H, d_k]")
    N, L, H, dk = q.shape
    _require(L >= 1, "q must hold at least one token per stream")
    _require(q.dtype in (torch.bfloat16, torch.float32), "q must be bfloat16 or float32")
    _require(tuple(k.shape) == (N, L, H, dk), "k must have the shape of q")
    _require(v.dim() == 4 and tuple(v.shape[:3]) == (N, L, H), "v must be [N, L, H, d_v]")
    dv = v.shape[3]
    _require(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share one dtype")
    _check_write(write)
    if write == "add":
        _require(beta is None, "beta must be None with the additive write")
    else:
        _require(beta is not None and tuple(beta.shape) == (N, L, H) and beta.dtype == torch.float32,
                 "beta must be float32 [N, L, H]")
    if log_alpha is not None:
        _require(log_alpha.dtype == torch.float32 and tuple(log_alpha.shape) in ((H,), (N, L, H), (N, L, H, dk)),
                 "log_alpha must be float32 [H], [N, L, H] or [N, L, H, d_k]")
    _require(state_pool.dim() == 4 and tuple(state_pool.shape[1:]) == (H, dk, dv) and
             state_pool.shape[0] >= 1 and state_pool.dtype == torch.float32,
             "state_pool must be float32 [P, H, d_k, d_v] with P >= 1")
    _require(tuple(src_slots.shape) == (N,) and src_slots.dtype == torch.int32, "src_slots must be int32 [N]")
    _require(tuple(dst_slots.shape) == (N, L) and dst_slots.dtype == torch.int32,
             "dst_slots must be int32 [N, L]")
    if out is not None:
        _require(tuple(out.shape) == (N, L, H, dv) and out.dtype == q.dtype, "out must be [N, L, H, d_v]")
    for name, t in named:
        if t is not None:
            _require(t.is_contiguous(), "%s must be contiguous" % name)
    _same_device(named, q)


def gate_code(log_alpha, token_ndim: int) -> int:
    """Gate of a log_alpha tensor: None, [H] (constant per head), token_ndim dims
    (one value per token and head) or one more (per key channel)."""
    if log_alpha is None:
        return GDN_GATE_NONE
    if log_alpha.dim() == 1:
        return GDN_GATE_HEAD_CONST
    return GDN_GATE_HEAD if log_alpha.dim() == token_ndim else GDN_GATE_KEY


def make_fwd_args(q, k, v, beta, log_alpha=None, initial_state=None, cu_seqlens=None, o=None,
                  final_state=None, chunk: int = CHUNK, write: str = "delta") -> FwdArgs:
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    return FwdArgs(B=B, T=T, H=H, d_k=dk, d_v=dv, chunk=chunk, N=N, dtype=_dtype_code(q),
                   gate=gate_code(log_alpha, 3), write=WRITES[write], q=_ptr(q), k=_ptr(k), v=_ptr(v),
                   beta=_ptr(beta),
                   log_alpha=_ptr(log_alpha), initial_state=_ptr(initial_state),
                   cu_seqlens=_ptr(cu_seqlens), o=_ptr(o), final_state=_ptr(final_state),
                   workspace=None, workspace_bytes=0)


def fwd_workspace_size(args: FwdArgs) -> int:
    return int(_lib.gdn_fwd_workspace_size(ctypes.byref(args)))


def fwd_chunked(q, k, v, beta, log_alpha=None, initial_state=None, cu_seqlens=None,
                output_final_state: bool = True, chunk: int = CHUNK, out=None, final_state=None,
                workspace=None, stream=None, write: str = "delta"):
    """Chunked forward (gdn_fwd_chunked).

    q, k [B,T,H,d_k] and v [B,T,H,d_v] (bf16 or fp32, CUDA, contiguous); beta [B,T,H]
    fp32 (None with write="add"); log_alpha None | [H] (constant per head) | [B,T,H] |
    [B,T,H,d_k] fp32; initial_state None | [N,H,d_k,d_v] fp32 (M = S^T); cu_seqlens
    None | int32 [N+1] (then B == 1).  write: "delta" (the delta rule) or "add" (the
    additive write of gated linear attention / RetNet).
    Returns (o [B,T,H,d_v], final_state [N,H,d_k,d_v] or None).  Asynchronous on the
    current (or given) stream.
    """
    import torch
    N = check_fwd_tensors(q, k, v, beta, log_alpha, initial_state, cu_seqlens, out,
                          final_state if output_final_state else None, write)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    args = make_fwd_args(q, k, v, beta, log_alpha, initial_state, cu_seqlens, out,
                         final_state if output_final_state else None, chunk, write)
    need = fwd_workspace_size(args)
    own = None
    if need:
        if workspace is None or workspace.numel() < need:
            workspace = own = torch.empty(need, dtype=torch.uint8, device=q.device)
        args.workspace, args.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _check(_lib.gdn_fwd_chunked(ctypes.byref(args), _stream(stream)), "gdn_fwd_chunked")
    _keep_for_stream(own, stream)
    return out, (final_state if output_final_state else None)


STATIC_SCRATCH_BYTES = 128 << 20  # GDN_STATIC_SCRATCH_BYTES of include/gdn.h


def fwd_chunked_static(q, k, v, beta, log_alpha=None, initial_state=None, cu_seqlens=None,
                       out=None, final_state=None, stream=None, write: str = "delta"):
    """Chunked forward without a workspace (gdn_fwd_chunked_static): the library uses
    its own scratch array on this GPU (at most STATIC_SCRATCH_BYTES; larger needs
    raise) and allocates nothing.  The caller passes every output: ``out``
    [B,T,H,d_v] and ``final_state`` None | [N,H,d_k,d_v] fp32.  Calls that may overlap
    on one GPU race on the shared scratch.  Other arguments as for fwd_chunked."""
    _require(out is not None, "out must be given (this entry point allocates nothing)")
    check_fwd_tensors(q, k, v, beta, log_alpha, initial_state, cu_seqlens, out, final_state, write)
    args = make_fwd_args(q, k, v, beta, log_alpha, initial_state, cu_seqlens, out, final_state, CHUNK, write)
    _check(_lib.gdn_fwd_chunked_static(ctypes.byref(args), _stream(stream)), "gdn_fwd_chunked_static")
    return out, final_state


class PreparedFwd:
    """A validated gdn_fwd_chunked call on fixed buffers, for repeated launches.

    Checks the tensors once and keeps the marshalled argument struct, so that each
    ``launch`` is a single call into the library (no per-call Python checks).  The
    tensors are held by reference and must keep their storage; ``o`` and
    ``final_state`` are overwritten by every launch."""

    def __init__(self, q, k, v, beta, log_alpha=None, initial_state=None, cu_seqlens=None,
                 out=None, final_state=None, output_final_state: bool = True, workspace=None,
                 chunk: int = CHUNK, write: str = "delta"):
        import torch
        if output_final_state and final_state is None:
            B, T, H, dk = q.shape
            N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
            final_state = torch.empty((N, H, dk, v.shape[-1]), dtype=torch.float32, device=q.device)
        if out is None:
            out = torch.empty(tuple(v.shape), dtype=q.dtype, device=q.device)
        check_fwd_tensors(q, k, v, beta, log_alpha, initial_state, cu_seqlens, out,
                          final_state if output_final_state else None, write)
        self.args = make_fwd_args(q, k, v, beta, log_alpha, initial_state, cu_seqlens, out,
                                  final_state if output_final_state else None, chunk, write)
        need = fwd_workspace_size(self.args)
        if need and (workspace is None or workspace.numel() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if need:
            self.args.workspace, self.args.workspace_bytes = workspace.data_ptr(), workspace.numel()
        self._keep = (q, k, v, beta, log_alpha, initial_state, cu_seqlens, workspace)
        self.out, self.final_state = out, (final_state if output_final_state else None)
        self._ref = ctypes.byref(self.args)

    def launch(self, stream=None):
        """Enqueue the forward on `stream` (default: torch's current stream)."""
        _check(_lib.gdn_fwd_chunked(self._ref, _stream(stream)), "gdn_fwd_chunked")
        return self.out, self.final_state


def check_dplr_tensors(q, k, v, a, b, log_alpha=None, initial_state=None, cu_seqlens=None, out=None,
                       final_state=None):
    """Host-side checks for fwd_dplr: those of fwd_chunked with the additive write,
    plus a and b shaped and typed like q.  Returns N."""
    for name, t in (("a", a), ("b", b)):
        _require(t is not None and tuple(t.shape) == tuple(q.shape) and t.dtype == q.dtype,
                 "%s must have the shape and dtype of q" % name)
        _require(t.is_contiguous(), "%s must be contiguous" % name)
    N = check_fwd_tensors(q, k, v, None, log_alpha, initial_state, cu_seqlens, out, final_state, "add")
    _same_device([("a", a), ("b", b)], q)
    return N


def make_dplr_args(q, k, v, a, b, log_alpha, initial_state, cu_seqlens, o, final_state,
                   chunk: int = CHUNK) -> DplrArgs:
    B, T, H, dk = q.shape
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    return DplrArgs(B=B, T=T, H=H, d_k=dk, d_v=v.shape[-1], chunk=chunk, N=N, dtype=_dtype_code(q),
                    gate=gate_code(log_alpha, 3), q=_ptr(q), k=_ptr(k), a=_ptr(a), b=_ptr(b), v=_ptr(v),
                    log_alpha=_ptr(log_alpha), initial_state=_ptr(initial_state),
                    cu_seqlens=_ptr(cu_seqlens), o=_ptr(o), final_state=_ptr(final_state),
                    workspace=None, workspace_bytes=0)


def dplr_workspace_size(args: DplrArgs) -> int:
    return int(_lib.gdn_dplr_workspace_size(ctypes.byref(args)))


class PreparedDplr:
    """A validated gdn_fwd_dplr call on fixed buffers (see PreparedFwd)."""

    def __init__(self, q, k, v, a, b, log_alpha=None, initial_state=None, cu_seqlens=None, out=None,
                 final_state=None, output_final_state: bool = True, chunk: int = CHUNK, workspace=None):
        import torch
        B, T, H, dk = q.shape
        N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
        if output_final_state and final_state is None:
            final_state = torch.empty((N, H, dk, v.shape[-1]), dtype=torch.float32, device=q.device)
        if out is None:
            out = torch.empty(tuple(v.shape), dtype=q.dtype, device=q.device)
        fs = final_state if output_final_state else None
        check_dplr_tensors(q, k, v, a, b, log_alpha, initial_state, cu_seqlens, out, fs)
        self.args = make_dplr_args(q, k, v, a, b, log_alpha, initial_state, cu_seqlens, out, fs, chunk)
        need = dplr_workspace_size(self.args)
        self.own_workspace = None
        if need:
            if workspace is None or workspace.numel() < need:
                workspace = self.own_workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            self.args.workspace, self.args.workspace_bytes = workspace.data_ptr(), workspace.numel()
        self._keep = (q, k, v, a, b, log_alpha, initial_state, cu_seqlens, workspace)
        self.out, self.final_state = out, fs
        self._ref = ctypes.byref(self.args)

    def launch(self, stream=None):
        _check(_lib.gdn_fwd_dplr(self._ref, _stream(stream)), "gdn_fwd_dplr")
        return self.out, self.final_state


def fwd_dplr(q, k, v, a, b, log_alpha=None, initial_state=None, cu_seqlens=None,
             output_final_state: bool = True, chunk: int = CHUNK, out=None, final_state=None, stream=None,
             workspace=None):
    """Chunked forward of the diagonal-plus-low-rank transition (gdn_fwd_dplr):
    M_t = Diag(alpha_t) M_{t-1} + b_t (a_t^T M_{t-1}) + k_t v_t^T, o_t = M_t^T q_t.

    q, k, a, b [B,T,H,d_k] and v [B,T,H,d_v] (one dtype, bf16 or fp32); log_alpha None
    | [H] (constant per head) | [B,T,H] | [B,T,H,d_k] (one decay per key channel) fp32;
    initial_state, cu_seqlens as for fwd_chunked; workspace (uint8, per-channel gate
    only) allocated here when not given.  Returns (o, final_state or None),
    asynchronous on the current (or given) stream."""
    p = PreparedDplr(q, k, v, a, b, log_alpha, initial_state, cu_seqlens, out, final_state,
                     output_final_state, chunk, workspace)
    res = p.launch(stream)
    _keep_for_stream(p.own_workspace, stream)
    return res


def dplr_step(q, k, v, a, b, log_alpha, state, out=None, stream=None):
    """One decode token per stream of the diagonal-plus-low-rank transition
    (gdn_fwd_dplr_step): q, k, a, b [N,H,d_k], v [N,H,d_v] (one dtype), log_alpha None |
    [H] | [N,H] | [N,H,d_k] fp32, state [N,H,d_k,d_v] fp32 updated in place.  Returns o
    [N,H,d_v]."""
    import torch
    for name, t in (("a", a), ("b", b)):
        _require(t is not None and tuple(t.shape) == tuple(q.shape) and t.dtype == q.dtype,
                 "%s must have the shape and dtype of q" % name)
        _require(t.is_contiguous(), "%s must be contiguous" % name)
    check_step_tensors(q, k, v, None, log_alpha, state, out, write="add")
    _same_device([("a", a), ("b", b)], q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    args = DplrStepArgs(N=N, H=H, d_k=dk, d_v=dv, dtype=_dtype_code(q), gate=gate_code(log_alpha, 2),
                        q=_ptr(q), k=_ptr(k), a=_ptr(a), b=_ptr(b), v=_ptr(v), log_alpha=_ptr(log_alpha),
                        state=_ptr(state), o=_ptr(out))
    _check(_lib.gdn_fwd_dplr_step(ctypes.byref(args), _stream(stream)), "gdn_fwd_dplr_step")
    return out


def dplr_decode(q, k, v, a, b, log_alpha, state_pool, src_slots, dst_slots, out=None, stream=None):
    """Serving decode of the diagonal-plus-low-rank transition (gdn_fwd_dplr_decode): q, k,
    a, b [N,L,H,d_k], v [N,L,H,d_v] (one dtype), log_alpha None | [H] | [N,L,H] |
    [N,L,H,d_k] fp32, state_pool [P,H,d_k,d_v] fp32, src_slots int32 [N], dst_slots int32
    [N,L] (see gdn_fwd_decode for the slot convention).  Returns o [N,L,H,d_v]."""
    import torch
    for name, t in (("a", a), ("b", b)):
        _require(t is not None and tuple(t.shape) == tuple(q.shape) and t.dtype == q.dtype,
                 "%s must have the shape and dtype of q" % name)
        _require(t.is_contiguous(), "%s must be contiguous" % name)
    check_decode_tensors(q, k, v, None, log_alpha, state_pool, src_slots, dst_slots, out, write="add")
    _same_device([("a", a), ("b", b)], q)
    N, L, H, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((N, L, H, dv), dtype=q.dtype, device=q.device)
    args = DplrDecodeArgs(N=N, L=L, H=H, d_k=dk, d_v=dv, dtype=_dtype_code(q), gate=gate_code(log_alpha, 3),
                          q=_ptr(q), k=_ptr(k), a=_ptr(a), b=_ptr(b), v=_ptr(v), log_alpha=_ptr(log_alpha),
                          state_pool=_ptr(state_pool), pool_size=state_pool.shape[0], src_slots=_ptr(src_slots),
                          dst_slots=_ptr(dst_slots), o=_ptr(out))
    _check(_lib.gdn_fwd_dplr_decode(ctypes.byref(args), _stream(stream)), "gdn_fwd_dplr_decode")
    return out


def recurrent_step(q, k, v, beta, log_alpha, state, out=None, stream=None, write: str = "delta"):
    """One decode token per stream (gdn_fwd_recurrent_step).

    q, k [N,H,d_k], v [N,H,d_v] (bf16 or fp32); beta [N,H] (None with write="add");
    log_alpha None | [H] | [N,H] | [N,H,d_k]; state [N,H,d_k,d_v] fp32, updated in
    place.  Returns o [N,H,d_v].
    """
    import torch
    check_step_tensors(q, k, v, beta, log_alpha, state, out, write)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    args = StepArgs(N=N, H=H, d_k=dk, d_v=dv, dtype=_dtype_code(q), gate=gate_code(log_alpha, 2),
                    write=WRITES[write], q=_ptr(q), k=_ptr(k), v=_ptr(v), beta=_ptr(beta), log_alpha=_ptr(log_alpha),
                    state=_ptr(state), o=_ptr(out))
    _check(_lib.gdn_fwd_recurrent_step(ctypes.byref(args), _stream(stream)), "gdn_fwd_recurrent_step")
    return out


def decode(q, k, v, beta, log_alpha, state_pool, src_slots, dst_slots, out=None, stream=None,
           write: str = "delta"):
    """Serving decode (gdn_fwd_decode): L tokens per stream against a pool of states.

    q, k [N,L,H,d_k], v [N,L,H,d_v] (bf16 or fp32); beta [N,L,H] (None with
    write="add"); log_alpha None | [H] | [N,L,H] | [N,L,H,d_k]; state_pool
    [P,H,d_k,d_v] fp32; src_slots int32 [N] (slot
    each stream starts from; outside [0, P): padding stream, skipped); dst_slots int32
    [N,L] (slot receiving the state after each token; outside [0, P): not stored).
    Returns o [N,L,H,d_v]; rows of padding streams are left as they were in ``out``
    (uninitialised if ``out`` is None).
    """
    import torch
    check_decode_tensors(q, k, v, beta, log_alpha, state_pool, src_slots, dst_slots, out, write)
    N, L, H, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((N, L, H, dv), dtype=q.dtype, device=q.device)
    args = DecodeArgs(N=N, L=L, H=H, d_k=dk, d_v=dv, dtype=_dtype_code(q), gate=gate_code(log_alpha, 3),
                      write=WRITES[write],
                      q=_ptr(q), k=_ptr(k), v=_ptr(v), beta=_ptr(beta), log_alpha=_ptr(log_alpha),
                      state_pool=_ptr(state_pool), pool_size=state_pool.shape[0],
                      src_slots=_ptr(src_slots), dst_slots=_ptr(dst_slots), o=_ptr(out))
    _check(_lib.gdn_fwd_decode(ctypes.byref(args), _stream(stream)), "gdn_fwd_decode")
    return out


class PreparedBwd:
    """A validated gdn_bwd_chunked call on fixed buffers (see PreparedFwd); the
    gradients are overwritten by every launch."""

    def __init__(self, q, k, v, beta, log_alpha, initial_state, dout, dfinal_state=None, cu_seqlens=None,
                 output_dinitial: bool = True, write: str = "delta"):
        self.args, self.outs, self._keep = _bwd_args(q, k, v, beta, log_alpha, initial_state, dout,
                                                     dfinal_state, cu_seqlens, output_dinitial, None, write)
        self._ref = ctypes.byref(self.args)

    def launch(self, stream=None):
        _check(_lib.gdn_bwd_chunked(self._ref, _stream(stream)), "gdn_bwd_chunked")
        return self.outs


def _keep_for_stream(buf, stream):
    """A scratch buffer allocated here on torch's current stream but used by work queued
    on another stream: tell the caching allocator, so that the block is not handed out
    again before that stream's work is done."""
    if buf is not None and stream is not None:
        buf.record_stream(stream)


def _bwd_args(q, k, v, beta, log_alpha, initial_state, dout, dfinal_state, cu_seqlens, output_dinitial,
              workspace, write="delta"):
    import torch
    N = check_fwd_tensors(q, k, v, beta, log_alpha, initial_state, cu_seqlens, dout, dfinal_state, write)
    _require(log_alpha is None or log_alpha.dim() in (1, 3, 4),
             "log_alpha must be None, [H] (one constant decay per head), [B, T, H] (one decay per token "
             "and head) or [B, T, H, d_k] (one decay per key channel)")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbeta = torch.empty_like(beta) if write == "delta" else None
    dla = torch.empty_like(log_alpha) if log_alpha is not None else None
    dinit = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device) if output_dinitial else None
    args = BwdArgs(B=B, T=T, H=H, d_k=dk, d_v=dv, chunk=CHUNK, N=N, dtype=_dtype_code(q),
                   gate=gate_code(log_alpha, 3), write=WRITES[write], q=_ptr(q), k=_ptr(k), v=_ptr(v),
                   beta=_ptr(beta), log_alpha=_ptr(log_alpha), initial_state=_ptr(initial_state),
                   cu_seqlens=_ptr(cu_seqlens), dout=_ptr(dout), dfinal_state=_ptr(dfinal_state),
                   dq=_ptr(dq), dk=_ptr(dk_), dv=_ptr(dv_), dbeta=_ptr(dbeta), dlog_alpha=_ptr(dla),
                   dinitial_state=_ptr(dinit), workspace=None, workspace_bytes=0)
    need = int(_lib.gdn_bwd_workspace_size(ctypes.byref(args)))
    if need:
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        args.workspace, args.workspace_bytes = workspace.data_ptr(), workspace.numel()
    keep = (q, k, v, beta, log_alpha, initial_state, dout, dfinal_state, cu_seqlens, workspace)
    return args, (dq, dk_, dv_, dbeta, dla, dinit), keep


def bwd_chunked(q, k, v, beta, log_alpha, initial_state, dout, dfinal_state=None, cu_seqlens=None,
                output_dinitial: bool = True, workspace=None, stream=None, write: str = "delta"):
    """Gradients of fwd_chunked (gdn_bwd_chunked) for the delta write (beta [B,T,H]) or
    the additive write (write="add", beta None), with no gate, one decay per (token,
    head) ([B,T,H]), one per key channel ([B,T,H,d_k]) or one constant decay per head
    ([H]).  Inputs as for fwd_chunked,
    plus dout [B,T,H,d_v] (dtype of q) and dfinal_state None | [N,H,d_k,d_v] fp32.
    Returns (dq, dk, dv, dbeta or None, dlog_alpha or None (shaped like log_alpha),
    dinitial_state or None)."""
    args, outs, keep = _bwd_args(q, k, v, beta, log_alpha, initial_state, dout, dfinal_state, cu_seqlens,
                                 output_dinitial, workspace, write)
    _check(_lib.gdn_bwd_chunked(ctypes.byref(args), _stream(stream)), "gdn_bwd_chunked")
    _keep_for_stream(keep[-1] if keep[-1] is not workspace else None, stream)
    return outs


def version() -> int:
    return int(_lib.gdn_version())

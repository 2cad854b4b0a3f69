"""MiniMax Sparse Attention (MSA) forward pass for AMD Instinct MI355X (gfx950).

A thin ctypes binding of ``libmsa.so`` (C ABI in ``include/msa.h``).  It only
marshals arguments: torch supplies device memory and the current stream, and
every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing or a call fails, an exception is raised.

Entry points (same names as the C ABI):
    msa_index_topk, msa_invert_workspace_size, msa_invert_blocks,
    msa_invert_status, msa_sparse_attn_fwd, msa_combine, msa_workspace_size,
    msa_forward
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_DTYPE_BF16 = 0
MSA_DTYPE_FP8_E4M3 = 1

EXPORTS = (
    "msa_abi_version", "msa_status_string", "msa_last_hip_error", "msa_index_topk",
    "msa_invert_workspace_size", "msa_invert_blocks", "msa_invert_status",
    "msa_sparse_attn_fwd", "msa_combine", "msa_workspace_size", "msa_forward",
    "msa_dense_attn_fwd", "msa_decode_workspace_size", "msa_decode", "msa_index_topk_forced",
    "msa_window_select", "msa_backward_workspace_size", "msa_backward", "msa_decode_static",
)

# Size of the device scratch msa_decode_static works in (MSA_STATIC_SCRATCH_BYTES).
STATIC_SCRATCH_BYTES = 64 * 1024 * 1024


class MSAError(RuntimeError):
    """A nonzero status from the library (or the library is missing)."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(what)


class msa_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("G", ctypes.c_int32), ("d_h", ctypes.c_int32), ("d_idx", ctypes.c_int32),
                ("B_k", ctypes.c_int32), ("k", ctypes.c_int32), ("N", ctypes.c_int64),
                ("H_idx", ctypes.c_int32)]

    @property
    def B(self) -> int:
        return -(-self.N // self.B_k)

    @property
    def H_sel(self) -> int:
        """Selection groups (index heads)."""
        return self.H_idx or self.H_kv

    @property
    def G_sel(self) -> int:
        """Query heads per selection group."""
        return self.H_q // self.H_sel


# MSA_DEFAULT_Q_CHUNK: msa_forward's query rows per pass when opts.q_chunk is 0
DEFAULT_Q_CHUNK = 16384


class msa_opts(ctypes.Structure):
    _fields_ = [("qkv_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("q_scale", ctypes.c_float), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("q_chunk", ctypes.c_int64)]


def make_dims(batch, N, H_q, H_kv, d_h, d_idx, B_k, k, H_idx=0) -> msa_dims:
    return msa_dims(batch=batch, H_q=H_q, H_kv=H_kv, G=H_q // H_kv if H_kv else 0, d_h=d_h,
                    d_idx=d_idx, B_k=B_k, k=k, N=N, H_idx=H_idx)


def make_opts(dtype: str = "bf16", softmax_scale: float = 0.0, q_scale: float = 1.0,
              k_scale: float = 1.0, v_scale: float = 1.0, q_chunk: int = 0) -> msa_opts:
    code = {"bf16": MSA_DTYPE_BF16, "fp8": MSA_DTYPE_FP8_E4M3}[dtype]
    return msa_opts(qkv_dtype=code, softmax_scale=softmax_scale, q_scale=q_scale,
                    k_scale=k_scale, v_scale=v_scale, reserved=0, q_chunk=q_chunk)


_lib = None


def lib():
    """Load libmsa.so (raises MSAError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MSAError(-1, f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        D, O = ctypes.POINTER(msa_dims), ctypes.POINTER(msa_opts)
        sig = {
            "msa_abi_version": ([], ctypes.c_int),
            "msa_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "msa_last_hip_error": ([], ctypes.c_int),
            "msa_index_topk": ([D, P, P, I64, I64, P, P], ctypes.c_int),
            "msa_invert_workspace_size": ([D, I64, I64, ctypes.POINTER(SZ)], ctypes.c_int),
            "msa_invert_blocks": ([D, P, I64, I64, P, P, P, SZ, P], ctypes.c_int),
            "msa_invert_status": ([P, ctypes.POINTER(ctypes.c_int32), P], ctypes.c_int),
            "msa_sparse_attn_fwd": ([D, O, P, P, P, P, P, P, I64, I64, P, P, P], ctypes.c_int),
            "msa_combine": ([D, P, P, P, I64, I64, P, P, P], ctypes.c_int),
            "msa_workspace_size": ([D, O, ctypes.POINTER(SZ)], ctypes.c_int),
            "msa_forward": ([D, O, P, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
            "msa_dense_attn_fwd": ([D, O, P, P, P, I64, I64, P, P, P], ctypes.c_int),
            "msa_decode_workspace_size": ([D, O, ctypes.POINTER(SZ)], ctypes.c_int),
            "msa_decode": ([D, O, P, P, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
            "msa_index_topk_forced": ([D, P, P, I64, I64, ctypes.c_int, ctypes.c_int, P, P], ctypes.c_int),
            "msa_window_select": ([D, I64, I64, P, P], ctypes.c_int),
            "msa_backward_workspace_size": ([D, O, ctypes.POINTER(SZ)], ctypes.c_int),
            "msa_backward": ([D, O, ctypes.c_float] + [P] * 16 + [SZ, P], ctypes.c_int),
            "msa_decode_static": ([D, O, P, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        msg = L.msa_status_string(status).decode()
        if status == 6:
            msg += f" (hipError {L.msa_last_hip_error()})"
        raise MSAError(status, f"{what}: {msg}")


def _p(t) -> Optional[ctypes.c_void_p]:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t) -> ctypes.c_void_p:
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t):
    import torch
    if not t.is_cuda:
        raise MSAError(1, "tensor arguments must be device tensors")
    if not t.is_contiguous():
        raise MSAError(2, "tensor arguments must be contiguous")
    return torch.cuda.device(t.device)


def _empty(shape, dtype, like):
    import torch
    return torch.empty(shape, dtype=dtype, device=like.device)


# ----------------------------------------------------------------------------- entry points

def msa_index_topk(dims: msa_dims, q_idx, k_idx, q_begin: int = 0, q_count: Optional[int] = None,
                   block_idx=None):
    """Index branch.  Returns block_idx int32 [batch, H_sel, q_count, k]."""
    import torch
    q_count = dims.N - q_begin if q_count is None else q_count
    if block_idx is None:
        block_idx = _empty((dims.batch, dims.H_sel, q_count, dims.k), torch.int32, q_idx)
    with _dev(q_idx):
        _check(lib().msa_index_topk(ctypes.byref(dims), _p(q_idx), _p(k_idx), q_begin, q_count,
                                    _p(block_idx), _stream(q_idx)), "msa_index_topk")
    return block_idx


def msa_index_topk_forced(dims: msa_dims, q_idx, k_idx, force_first: bool = True, local_window: int = 1,
                          q_begin: int = 0, q_count: Optional[int] = None, block_idx=None):
    """Index branch with forced block 0 and/or a forced local window of blocks."""
    import torch
    q_count = dims.N - q_begin if q_count is None else q_count
    if block_idx is None:
        block_idx = _empty((dims.batch, dims.H_sel, q_count, dims.k), torch.int32, q_idx)
    with _dev(q_idx):
        _check(lib().msa_index_topk_forced(ctypes.byref(dims), _p(q_idx), _p(k_idx), q_begin, q_count,
                                           int(force_first), int(local_window), _p(block_idx),
                                           _stream(q_idx)), "msa_index_topk_forced")
    return block_idx


def msa_window_select(dims: msa_dims, q_begin: int = 0, q_count: Optional[int] = None, block_idx=None,
                      device=None):
    """FLOP-matched sliding-window selection int32 [batch, H_sel, q_count, k]."""
    import torch
    q_count = dims.N - q_begin if q_count is None else q_count
    if block_idx is None:
        block_idx = torch.empty((dims.batch, dims.H_sel, q_count, dims.k), dtype=torch.int32,
                                device=device or "cuda")
    with _dev(block_idx):
        _check(lib().msa_window_select(ctypes.byref(dims), q_begin, q_count, _p(block_idx),
                                       _stream(block_idx)), "msa_window_select")
    return block_idx


def msa_invert_workspace_size(dims: msa_dims, q_begin: int, q_count: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_invert_workspace_size(ctypes.byref(dims), q_begin, q_count, ctypes.byref(n)),
           "msa_invert_workspace_size")
    return n.value


def msa_invert_blocks(dims: msa_dims, block_idx, q_begin: int = 0, q_count: Optional[int] = None,
                      blk_offsets=None, blk_entries=None, sched=None):
    """Inversion + work list.  Returns (blk_offsets, blk_entries, sched)."""
    import torch
    q_count = dims.N - q_begin if q_count is None else q_count
    B_c = -(-(q_begin + q_count) // dims.B_k)
    if blk_offsets is None:
        blk_offsets = _empty((dims.batch, dims.H_sel, B_c + 1), torch.int32, block_idx)
    if blk_entries is None:
        blk_entries = _empty((dims.batch * dims.H_sel * q_count * dims.k,), torch.int32, block_idx)
    nbytes = msa_invert_workspace_size(dims, q_begin, q_count)
    if sched is None:
        sched = _empty(((nbytes + 3) // 4,), torch.int32, block_idx)
    with _dev(block_idx):
        _check(lib().msa_invert_blocks(ctypes.byref(dims), _p(block_idx), q_begin, q_count,
                                       _p(blk_offsets), _p(blk_entries), _p(sched),
                                       sched.numel() * sched.element_size(), _stream(block_idx)),
               "msa_invert_blocks")
    return blk_offsets, blk_entries, sched


def msa_invert_status(sched) -> int:
    """Synchronises the current stream; returns the skipped out-of-range ids."""
    out = ctypes.c_int32(0)
    with _dev(sched):
        _check(lib().msa_invert_status(_p(sched), ctypes.byref(out), _stream(sched)),
               "msa_invert_status")
    return out.value


def msa_sparse_attn_fwd(dims: msa_dims, opts: msa_opts, q, k, v, blk_offsets, blk_entries, sched,
                        q_begin: int = 0, q_count: Optional[int] = None, o_part=None,
                        lse_part=None):
    """KV-outer sparse attention.  Returns (o_part bf16 [batch, H_sel, q_count, k, G_sel, d_h],
    lse_part fp32 [batch, H_sel, q_count, k, G_sel])."""
    import torch
    q_count = dims.N - q_begin if q_count is None else q_count
    shp = (dims.batch, dims.H_sel, q_count, dims.k, dims.G_sel)
    if o_part is None:
        o_part = _empty(shp + (dims.d_h,), torch.bfloat16, q)
    if lse_part is None:
        lse_part = _empty(shp, torch.float32, q)
    with _dev(q):
        _check(lib().msa_sparse_attn_fwd(ctypes.byref(dims), ctypes.byref(opts), _p(q), _p(k), _p(v),
                                         _p(blk_offsets), _p(blk_entries), _p(sched), q_begin,
                                         q_count, _p(o_part), _p(lse_part), _stream(q)),
               "msa_sparse_attn_fwd")
    return o_part, lse_part


def msa_combine(dims: msa_dims, block_idx, o_part, lse_part, q_begin: int = 0,
                q_count: Optional[int] = None, o=None, lse=None, want_lse: bool = False):
    """LSE merge.  Returns (o bf16 [batch, N, H_q, d_h], lse fp32 [batch, N, H_q] or None)."""
    import torch
    q_count = dims.N - q_begin if q_count is None else q_count
    if o is None:
        o = _empty((dims.batch, dims.N, dims.H_q, dims.d_h), torch.bfloat16, o_part)
    if lse is None and want_lse:
        lse = _empty((dims.batch, dims.N, dims.H_q), torch.float32, o_part)
    with _dev(o_part):
        _check(lib().msa_combine(ctypes.byref(dims), _p(block_idx), _p(o_part), _p(lse_part),
                                 q_begin, q_count, _p(o), _p(lse), _stream(o_part)), "msa_combine")
    return o, lse


def msa_workspace_size(dims: msa_dims, opts: msa_opts) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_workspace_size(ctypes.byref(dims), ctypes.byref(opts), ctypes.byref(n)),
           "msa_workspace_size")
    return n.value


def msa_forward(dims: msa_dims, opts: msa_opts, q, k, v, q_idx, k_idx, o=None, lse=None,
                block_idx_out=None, workspace=None, want_lse: bool = False):
    """The whole forward pass.  Returns (o, lse or None, block_idx_out or None)."""
    import torch
    if o is None:
        o = _empty((dims.batch, dims.N, dims.H_q, dims.d_h), torch.bfloat16, q)
    if lse is None and want_lse:
        lse = _empty((dims.batch, dims.N, dims.H_q), torch.float32, q)
    nbytes = msa_workspace_size(dims, opts)
    if workspace is None:
        workspace = _empty((nbytes,), torch.uint8, q)
    with _dev(q):
        _check(lib().msa_forward(ctypes.byref(dims), ctypes.byref(opts), _p(q), _p(k), _p(v),
                                 _p(q_idx), _p(k_idx), _p(o), _p(lse), _p(block_idx_out),
                                 _p(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(q)), "msa_forward")
    return o, lse, block_idx_out


def msa_dense_attn_fwd(dims: msa_dims, opts: msa_opts, q, k, v, q_begin: int = 0,
                       q_count: Optional[int] = None, o=None, lse=None, want_lse: bool = False):
    """Dense causal GQA attention (the baseline).  Returns (o bf16 [batch, N, H_q, d_h],
    lse fp32 [batch, N, H_q] or None); rows outside [q_begin, q_begin + q_count) of a
    freshly allocated o are uninitialised."""
    import torch
    q_count = dims.N - q_begin if q_count is None else q_count
    if o is None:
        o = _empty((dims.batch, dims.N, dims.H_q, dims.d_h), torch.bfloat16, q)
    if lse is None and want_lse:
        lse = _empty((dims.batch, dims.N, dims.H_q), torch.float32, q)
    with _dev(q):
        _check(lib().msa_dense_attn_fwd(ctypes.byref(dims), ctypes.byref(opts), _p(q), _p(k), _p(v),
                                        q_begin, q_count, _p(o), _p(lse), _stream(q)),
               "msa_dense_attn_fwd")
    return o, lse


def msa_decode_workspace_size(dims: msa_dims, opts: msa_opts) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_decode_workspace_size(ctypes.byref(dims), ctypes.byref(opts), ctypes.byref(n)),
           "msa_decode_workspace_size")
    return n.value


def msa_decode(dims: msa_dims, opts: msa_opts, q, q_idx, k, v, k_idx, o=None, lse=None,
               block_idx_out=None, workspace=None, want_lse: bool = False, seq_lens=None):
    """One decode step: the last token of each sequence (position seq_lens[b] - 1,
    or N - 1 when seq_lens is None; seq_lens an int32 device tensor [batch]).
    q [batch, H_q, d_h], q_idx [batch, H_sel, d_idx]; caches as for msa_forward.
    Returns (o bf16 [batch, H_q, d_h], lse fp32 [batch, H_q] or None, block_idx_out)."""
    import torch
    if o is None:
        o = _empty((dims.batch, dims.H_q, dims.d_h), torch.bfloat16, q)
    if lse is None and want_lse:
        lse = _empty((dims.batch, dims.H_q), torch.float32, q)
    nbytes = msa_decode_workspace_size(dims, opts)
    if workspace is None:
        workspace = _empty((nbytes,), torch.uint8, q)
    with _dev(q):
        _check(lib().msa_decode(ctypes.byref(dims), ctypes.byref(opts), _p(q), _p(q_idx), _p(k), _p(v),
                                _p(k_idx), _p(seq_lens), _p(o), _p(lse), _p(block_idx_out), _p(workspace),
                                workspace.numel() * workspace.element_size(), _stream(q)),
               "msa_decode")
    return o, lse, block_idx_out


def msa_decode_static(dims: msa_dims, opts: msa_opts, q, q_idx, k, v, k_idx, o=None, lse=None,
                      block_idx_out=None, want_lse: bool = False, seq_lens=None):
    """msa_decode without a workspace: the library's static device scratch is
    used instead (for callers that cannot allocate).  Arguments and result as
    for msa_decode; steps needing more than STATIC_SCRATCH_BYTES raise."""
    import torch
    if o is None:
        o = _empty((dims.batch, dims.H_q, dims.d_h), torch.bfloat16, q)
    if lse is None and want_lse:
        lse = _empty((dims.batch, dims.H_q), torch.float32, q)
    with _dev(q):
        _check(lib().msa_decode_static(ctypes.byref(dims), ctypes.byref(opts), _p(q), _p(q_idx), _p(k),
                                       _p(v), _p(k_idx), _p(seq_lens), _p(o), _p(lse), _p(block_idx_out),
                                       _stream(q)),
               "msa_decode_static")
    return o, lse, block_idx_out


def msa_backward_workspace_size(dims: msa_dims, opts: msa_opts) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().msa_backward_workspace_size(ctypes.byref(dims), ctypes.byref(opts), ctypes.byref(n)),
           "msa_backward_workspace_size")
    return n.value


def msa_backward(dims: msa_dims, opts: msa_opts, q, k, v, q_idx, k_idx, o, lse, d_o, block_idx,
                 kl_weight: float = 1.0, index: bool = True, want_kl: bool = True, workspace=None):
    """Backward pass: gradients of the sparse main attention (dq, dk, dv) and,
    when ``index``, the KL alignment gradient of the index branch (dq_idx,
    dk_idx) and the per-row KL [batch, H_sel, N] (when ``want_kl``).
    Inputs as msa_forward's, plus its output o, lse and block_idx and the
    output gradient d_o.  Returns a dict of the outputs (None when skipped)."""
    import torch
    B, N = dims.batch, dims.N
    out = {
        "dq": _empty((B, N, dims.H_q, dims.d_h), torch.bfloat16, q),
        "dk": _empty((B, N, dims.H_kv, dims.d_h), torch.bfloat16, q),
        "dv": _empty((B, N, dims.H_kv, dims.d_h), torch.bfloat16, q),
        "dq_idx": _empty((B, N, dims.H_sel, dims.d_idx), torch.bfloat16, q) if index else None,
        "dk_idx": _empty((B, N, dims.d_idx), torch.bfloat16, q) if index else None,
        "kl": _empty((B, dims.H_sel, N), torch.float32, q) if index and want_kl else None,
    }
    nbytes = msa_backward_workspace_size(dims, opts)
    if workspace is None:
        workspace = _empty((nbytes,), torch.uint8, q)
    with _dev(q):
        _check(lib().msa_backward(ctypes.byref(dims), ctypes.byref(opts), float(kl_weight), _p(q), _p(k), _p(v),
                                  _p(q_idx), _p(k_idx), _p(o), _p(lse), _p(d_o), _p(block_idx),
                                  _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dq_idx"]),
                                  _p(out["dk_idx"]), _p(out["kl"]), _p(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(q)),
               "msa_backward")
    return out


def default_softmax_scale(d_h: int) -> float:
    return 1.0 / math.sqrt(d_h)

"""Exact IO-aware attention for MI355X (gfx950): Python binding of libfa.so.

Thin ctypes marshalling over the C ABI declared in include/fa.h: it checks
the inputs the way the first page's reference implementation does (rank,
floating dtype, matching dtypes, widths, lengths, devices), allocates the
outputs with torch on the inputs' device and passes raw device pointers and
the current HIP stream.  Every arithmetic step runs in the library's
kernels; there is no fallback.  If libfa.so has not been built this raises.

    o, lse = forward(q, k, v, causal=False)     # q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,dv]
    o, lse = forward_splitkv(q, k, v)            # same result, keys split over workgroups
    dq, dk, dv = backward(q, k, v, o, lse, do, causal=False)   # [B,H,N,d] each
"""

import ctypes
import math
import os

import torch

__all__ = ["forward", "forward_splitkv", "backward", "backward_prep", "backward_dkdv", "backward_dq",
           "forward_dropout", "backward_dropout", "dropout_applied_p", "forward_varlen", "backward_varlen", "workspace_for",
           "library", "FAError", "LIB_PATH", "status_string"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
_lib = None


class FAError(RuntimeError):
    """A non-zero fa_status returned by the library."""

    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


def library():
    """The loaded libfa.so (ctypes.CDLL).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_16_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_fwd.restype = i
        lib.fa_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_fwd_f32.restype = i
        lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
        lib.fa_fwd_ex.restype = i
        lib.fa_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        lib.fa_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
        lib.fa_fwd_splitkv.restype = i
        lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
        lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_bwd.restype = i
        lib.fa_bwd_prep.argtypes = [vp, vp, vp, vp, i, i, i, i, f, vp]
        lib.fa_bwd_prep.restype = i
        lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_bwd_dkdv.restype = i
        lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_bwd_dq.restype = i
        u64, u32 = ctypes.c_uint64, ctypes.c_uint32
        lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, f, u64, u32, vp]
        lib.fa_fwd_dropout.restype = i
        lib.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, f, u64, u32, vp]
        lib.fa_bwd_dropout.restype = i
        lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        lib.fa_fwd_varlen.restype = i
        lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        lib.fa_bwd_varlen.restype = i
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i64p, i64p, i64p, f, i, vp]
        lib.fa_fwd_strided.restype = i
        lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
        lib.fa_bwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i64p, i64p, i64p, f, i,
                                       vp]
        lib.fa_bwd_strided.restype = i
        lib.fa_bwd_ex.restype = i
        lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_bwd_noalloc.restype = i
        lib.fa_dropout_applied_p.argtypes = [f]
        lib.fa_dropout_applied_p.restype = f
        lib.fa_status_string.argtypes = [i]
        lib.fa_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status):
    return library().fa_status_string(int(status)).decode()


_KERNEL_DTYPES = (torch.bfloat16, torch.float32)


def _check(q, k, v, square=True, strided=False):
    """Host-side check of the inputs against the C ABI (include/fa.h).

    The rules are listed once, in the order they are tested; the first one
    broken raises.  square=False admits the general shapes of fa_fwd_ex
    (Q [B,H,Nq,d], K [B,H,Nk,d], V [B,H,Nk,dv]); strided=True admits views
    with a unit head-dim stride (fa_fwd_strided).  Head widths outside the
    kernels' set come back from the library as FA_ERR_HEADDIM.
    """
    shapes = lambda: f"q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}"
    rules = (
        (lambda: q.dim() == k.dim() == v.dim() == 4, ValueError,
         lambda: f"q, k, v: expected 4-D [batch, heads, rows, width] tensors, got {shapes()}"),
        (lambda: q.dtype == k.dtype == v.dtype and q.dtype in _KERNEL_DTYPES, TypeError,
         lambda: f"q, k, v: one dtype, bfloat16 (or float32 for the float32 kernel), got "
                 f"{q.dtype}, {k.dtype}, {v.dtype}"),
        (lambda: q.shape[:2] == k.shape[:2] == v.shape[:2], ValueError,
         lambda: f"q, k, v: batch and head counts must agree, got {shapes()}"),
        (lambda: q.shape[3] == k.shape[3] and q.shape[3] > 0 and v.shape[3] > 0, ValueError,
         lambda: f"score width: q and k need one positive width d (and v a positive width), got {shapes()}"),
        (lambda: k.shape[2] == v.shape[2], ValueError,
         lambda: f"key count: k and v need the same number of rows, got {shapes()}"),
        (lambda: not square or q.shape == k.shape == v.shape, ValueError,
         lambda: f"this entry point takes one shared [B, H, N, d] shape, got {shapes()}"),
        (lambda: (all(t.stride(-1) == 1 for t in (q, k, v)) if strided
                  else all(t.is_contiguous() for t in (q, k, v))), ValueError,
         lambda: ("q, k, v: views need unit stride along the head dimension" if strided
                  else "q, k, v: this entry point takes contiguous tensors")),
        (lambda: q.device == k.device == v.device and q.device.type == "cuda", ValueError,
         lambda: f"q, k, v: all on one GPU (the kernels have no CPU path), got {q.device}, {k.device}, {v.device}"),
    )
    for ok, exc, message in rules:
        if not ok():
            raise exc(message())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _outputs(q, v, out, lse):
    B, H, Nq = q.shape[:3]
    dv = v.shape[-1]
    o = out if out is not None else torch.empty((B, H, Nq, dv), dtype=torch.float32, device=q.device)
    l = lse if lse is not None else torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if o.shape != (B, H, Nq, dv) or l.shape != (B, H, Nq) or o.dtype != torch.float32 or l.dtype != torch.float32:
        raise ValueError("out must be float32 [B, H, Nq, dv] and lse float32 [B, H, Nq]")
    if not (o.is_contiguous() and l.is_contiguous()) or o.device != q.device or l.device != q.device:
        raise ValueError("out and lse must be contiguous and on Q's device")
    return o, l


def forward(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Exact attention: returns (O float32 [B,H,Nq,dv], L float32 [B,H,Nq]).

    L is the natural-log logsumexp of the scaled, masked scores of each row.
    bf16 inputs run the matrix-core kernel (fa_fwd for one shared [B,H,N,d]
    shape, fa_fwd_ex for Nq != Nk or dv != d, fa_fwd_strided for views such as
    slices of a packed QKV tensor); float32 inputs run the float32 kernel
    (fa_fwd_f32, one shared contiguous shape).  Causal masking is upper-left.
    ``out``/``lse`` may be preallocated.
    """
    bf16 = q.dtype == torch.bfloat16
    _check(q, k, v, square=not bf16, strided=bf16)
    B, H, Nq, d = q.shape
    Nk, dv = k.shape[2], v.shape[3]
    o, l = _outputs(q, v, out, lse)
    lib = library()
    sc, cz, stream = _scale(scale, d), int(bool(causal)), _stream(q.device)
    if bf16 and not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        arr = lambda t: (ctypes.c_int64 * 3)(*t.stride()[:3])
        name, st = "fa_fwd_strided", lib.fa_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, Nq, Nk,
                                                        d, dv, arr(q), arr(k), arr(v), sc, cz, stream)
    elif q.dtype == torch.float32:
        name, st = "fa_fwd_f32", lib.fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, Nq, d, sc, cz,
                                                stream)
    elif Nq == Nk and dv == d:
        name, st = "fa_fwd", lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, Nq, d, sc, cz, stream)
    else:
        name, st = "fa_fwd_ex", lib.fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, Nq, Nk, d, dv, sc,
                                              cz, stream)
    if st != FA_OK:
        raise FAError(name, st)
    return o, l


def forward_splitkv(q, k, v, causal=False, scale=None, n_splits=0, workspace=None, out=None, lse=None):
    """Split-KV forward (fa_fwd_splitkv): the same result as forward() for
    bf16 inputs, with the key tiles cut into ``n_splits`` ranges handled by
    separate workgroups and merged by logsumexp (0: chosen for the grid).
    Meant for few query rows against long key sequences (decoding)."""
    _check(q, k, v, square=False)
    if q.dtype != torch.bfloat16:
        raise TypeError("the split-KV forward takes bfloat16 Q, K, V")
    B, H, Nq, d = q.shape
    Nk, dv = k.shape[2], v.shape[3]
    o, l = _outputs(q, v, out, lse)
    lib = library()
    need = lib.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, dv, int(n_splits))
    if workspace is None:
        workspace = torch.empty((max(need, 4),), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need or workspace.device != q.device:
        raise ValueError(f"workspace must hold {need} bytes on Q's device")
    st = lib.fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), _ptr(workspace), B, H, Nq, Nk, d, dv,
                            _scale(scale, d), int(bool(causal)), int(n_splits), _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_fwd_splitkv", st)
    return o, l


def _check_bwd(q, k, v, o, lse, do, square=True, strided=False):
    _check(q, k, v, square=square, strided=strided)
    if v.shape[3] != q.shape[3]:
        raise ValueError(f"backward: v needs the width of q and k (dv = d), got {tuple(v.shape)} for d = {q.shape[3]}")
    if q.dtype != torch.bfloat16 or do.dtype != torch.bfloat16:
        raise TypeError("backward takes bfloat16 Q, K, V and dO")
    if do.shape != q.shape or o.shape != q.shape or lse.shape != q.shape[:3]:
        raise ValueError("dO and O must match Q's shape and L must be [B, H, N]")
    if o.dtype != torch.float32 or lse.dtype != torch.float32:
        raise TypeError("O and L must be float32 (as returned by forward)")
    if not (do.is_contiguous() and o.is_contiguous() and lse.is_contiguous()):
        raise ValueError("dO, O and L must be contiguous")
    if not (do.device == o.device == lse.device == q.device):
        raise ValueError("all tensors must be on the same device")


def _out(t, like):
    """A float32 output of Q's shape: a new tensor, or the given one after checks."""
    if t is None:
        return torch.empty(like.shape, dtype=torch.float32, device=like.device)
    if t.dtype != torch.float32 or t.shape != like.shape or t.device != like.device or not t.is_contiguous():
        raise ValueError("outputs must be contiguous float32 tensors of Q's shape on Q's device")
    return t


def workspace_for(q, workspace=None):
    """The backward workspace for Q's shape: the given one (checked) or a new one."""
    B, H, N, d = q.shape
    ws_bytes = library().fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        return torch.empty((max(ws_bytes, 4),), dtype=torch.uint8, device=q.device)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on Q's device")
    if workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace too small: need {ws_bytes} bytes")
    return workspace


def backward(q, k, v, o, lse, do, causal=False, scale=None, workspace=None):
    """Gradients (dQ [B,H,Nq,d], dK and dV [B,H,Nk,d], float32) of sum(dO * O).

    ``o`` and ``lse`` must be the forward's outputs for the same inputs; the
    probability tiles are recomputed from them.  bf16 inputs only.  Q may
    have a different number of rows than K and V (fa_bwd_ex, upper-left
    causal mask), V the width of Q and K.  With one row count, Q, K and V
    may be views with a unit head-dim stride, such as slices of a packed QKV
    tensor (fa_bwd_strided; K and V sharing a row stride).
    """
    strided = not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous())
    _check_bwd(q, k, v, o, lse, do, square=False, strided=strided)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if strided and Nq != Nk:
        raise ValueError("strided views take one row count for Q, K and V")
    workspace = workspace_for(q, workspace)
    dq = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, H, Nk, d), dtype=torch.float32, device=q.device)
    dv = torch.empty_like(dk)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace))
    tail = (_scale(scale, d), int(bool(causal)), _stream(q.device))
    if strided:
        arr = lambda t: (ctypes.c_int64 * 3)(*t.stride()[:3])
        name, st = "fa_bwd_strided", library().fa_bwd_strided(*args, B, H, Nq, d, arr(q), arr(k), arr(v), *tail)
    elif Nq == Nk:
        name, st = "fa_bwd", library().fa_bwd(*args, B, H, Nq, d, *tail)
    else:
        name, st = "fa_bwd_ex", library().fa_bwd_ex(*args, B, H, Nq, Nk, d, *tail)
    if st != FA_OK:
        raise FAError(name, st)
    return dq, dk, dv


def _dropout_args(p, seed, offset):
    p = float(p)
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    seed, offset = int(seed), int(offset)
    if not (0 <= seed < 2 ** 64) or not (0 <= offset < 2 ** 32):
        raise ValueError("seed must fit 64 bits and offset 32 bits (unsigned)")
    return p, seed, offset


def dropout_applied_p(p):
    """The dropout probability the kernels apply for a requested ``p``
    (fa_dropout_applied_p): p is quantised to t / 256 with
    t = min(255, round(256 p)), e.g. 0.1 -> 26/256 = 0.1015625."""
    p, _, _ = _dropout_args(p, 0, 0)
    return float(library().fa_dropout_applied_p(p))


def forward_dropout(q, k, v, p, seed, offset=0, causal=False, scale=None, out=None, lse=None):
    """forward() with dropout on the normalised weights (fa_fwd_dropout).

    The mask is a function of (seed, offset, head, row, key) only, so
    backward_dropout with the same arguments regenerates it.  bf16 inputs of
    one shared [B,H,N,d] shape; L is the logsumexp without dropout.
    Returns (O, L, p_applied): the probability actually applied, p quantised
    to a multiple of 1/256 (see dropout_applied_p).
    """
    if q.dtype != torch.bfloat16:
        raise TypeError("dropout takes bfloat16 Q, K, V")
    p, seed, offset = _dropout_args(p, seed, offset)
    _check(q, k, v)
    B, H, N, d = q.shape
    o, l = _outputs(q, v, out, lse)
    st = library().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, N, d, _scale(scale, d),
                                  int(bool(causal)), p, seed, offset, _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_fwd_dropout", st)
    return o, l, dropout_applied_p(p)


def backward_dropout(q, k, v, o, lse, do, p, seed, offset=0, causal=False, scale=None, workspace=None):
    """Gradients of sum(dO * O) for O = forward_dropout(q, k, v, p, seed,
    offset, causal, scale) (fa_bwd_dropout); the mask is regenerated."""
    _check_bwd(q, k, v, o, lse, do)
    p, seed, offset = _dropout_args(p, seed, offset)
    B, H, N, d = q.shape
    workspace = workspace_for(q, workspace)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    st = library().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(workspace), B, H, N, d, _scale(scale, d), int(bool(causal)), p, seed,
                                  offset, _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_bwd_dropout", st)
    return dq, dk, dv


def _check_varlen(q, k, v, cu_seqlens, max_seqlen):
    for t in (q, k, v):
        if t.dtype != torch.bfloat16:
            raise TypeError("packed sequences take bfloat16 Q, K, V")
        if t.dim() != 3:
            raise ValueError("packed Q, K, V must be rank 3 [H, total, d]")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("packed Q, K and V must have one shape [H, total, d]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise TypeError("cu_seqlens must be a 1-D int32 tensor of B + 1 offsets")
    if not all(t.is_contiguous() for t in (q, k, v, cu_seqlens)):
        raise ValueError("packed tensors and cu_seqlens must be contiguous")
    if not (q.device == k.device == v.device == cu_seqlens.device) or q.device.type != "cuda":
        raise ValueError("packed tensors and cu_seqlens must be on one GPU")
    max_seqlen = int(max_seqlen)
    if max_seqlen < 0 or max_seqlen > q.shape[1]:
        raise ValueError("max_seqlen must be in [0, total]")
    return max_seqlen


def _dense_on(device, **tensors):
    """The kernels address these buffers as dense arrays from their data
    pointer: each must be contiguous and on the inputs' device."""
    for name, t in tensors.items():
        if not t.is_contiguous() or t.device != device:
            raise ValueError(f"{name} must be a contiguous tensor on {device}")


def forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None, out=None, lse=None):
    """Attention over packed variable-length sequences (fa_fwd_varlen).

    q, k, v: bf16 [H, total, d]; sequence b holds rows cu_seqlens[b] ..
    cu_seqlens[b+1]-1 of every head (cu_seqlens: int32 [B+1] on the GPU);
    max_seqlen bounds the longest sequence.  Returns O float32 [H, total, d]
    and L float32 [H, total]; rows attend within their own sequence.
    """
    max_seqlen = _check_varlen(q, k, v, cu_seqlens, max_seqlen)
    H, total, d = q.shape
    B = cu_seqlens.numel() - 1
    o = out if out is not None else torch.empty((H, total, d), dtype=torch.float32, device=q.device)
    l = lse if lse is not None else torch.empty((H, total), dtype=torch.float32, device=q.device)
    if o.shape != (H, total, d) or l.shape != (H, total) or o.dtype != torch.float32 or l.dtype != torch.float32:
        raise ValueError("out must be float32 [H, total, d] and lse float32 [H, total]")
    _dense_on(q.device, out=o, lse=l)
    st = library().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), _ptr(cu_seqlens), B, H, total,
                                 max_seqlen, d, _scale(scale, d), int(bool(causal)), _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_fwd_varlen", st)
    return o, l


def backward_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen, causal=False, scale=None, workspace=None):
    """Gradients (dQ, dK, dV), float32 [H, total, d], of sum(dO * O) for
    O = forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal, scale)
    (fa_bwd_varlen)."""
    max_seqlen = _check_varlen(q, k, v, cu_seqlens, max_seqlen)
    H, total, d = q.shape
    B = cu_seqlens.numel() - 1
    if do.dtype != torch.bfloat16 or do.shape != q.shape:
        raise ValueError("dO must be a bfloat16 tensor of Q's shape")
    if o.dtype != torch.float32 or o.shape != q.shape or lse.dtype != torch.float32 or lse.shape != (H, total):
        raise ValueError("O and L must be the float32 outputs of forward_varlen")
    ws_bytes = library().fa_bwd_workspace_bytes(1, H, total, d)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 4),), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace too small: need {ws_bytes} bytes")
    _dense_on(q.device, dO=do, O=o, L=lse, workspace=workspace)
    dq = torch.empty((H, total, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    st = library().fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(workspace), _ptr(cu_seqlens), B, H, total, max_seqlen, d,
                                 _scale(scale, d), int(bool(causal)), _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_bwd_varlen", st)
    return dq, dk, dv


def backward_prep(o, lse, do, workspace, scale=None):
    """First backward phase: per-row scale * (dO . O) and L log2(e) into ``workspace``."""
    if do.dtype != torch.bfloat16 or o.dtype != torch.float32 or lse.dtype != torch.float32:
        raise TypeError("dO bfloat16, O and L float32")
    if do.ndim != 4 or o.shape != do.shape or lse.shape != do.shape[:3]:
        raise ValueError("dO and O must be [B, H, N, d] and L [B, H, N]")
    if not (do.is_contiguous() and o.is_contiguous() and lse.is_contiguous()):
        raise ValueError("dO, O and L must be contiguous")
    B, H, N, d = do.shape
    workspace = workspace_for(do, workspace)
    st = library().fa_bwd_prep(_ptr(do), _ptr(o), _ptr(lse), _ptr(workspace), B, H, N, d, _scale(scale, d),
                               _stream(do.device))
    if st != FA_OK:
        raise FAError("fa_bwd_prep", st)
    return workspace


def backward_dkdv(q, k, v, do, workspace, causal=False, scale=None, dk=None, dv=None):
    """Second backward phase: (dK, dV) from a workspace filled by backward_prep."""
    _check(q, k, v)
    if q.dtype != torch.bfloat16 or do.dtype != torch.bfloat16 or do.shape != q.shape:
        raise TypeError("bfloat16 Q, K, V and dO of one shape")
    B, H, N, d = q.shape
    workspace = workspace_for(q, workspace)
    dk, dv = _out(dk, q), _out(dv, q)
    st = library().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(workspace), _ptr(dk), _ptr(dv), B, H, N, d,
                               _scale(scale, d), int(bool(causal)), _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_bwd_dkdv", st)
    return dk, dv


def backward_dq(q, k, v, do, workspace, causal=False, scale=None, dq=None):
    """Third backward phase: dQ from a workspace filled by backward_prep."""
    _check(q, k, v)
    if q.dtype != torch.bfloat16 or do.dtype != torch.bfloat16 or do.shape != q.shape:
        raise TypeError("bfloat16 Q, K, V and dO of one shape")
    B, H, N, d = q.shape
    workspace = workspace_for(q, workspace)
    dq = _out(dq, q)
    st = library().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(workspace), _ptr(dq), B, H, N, d,
                             _scale(scale, d), int(bool(causal)), _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_bwd_dq", st)
    return dq

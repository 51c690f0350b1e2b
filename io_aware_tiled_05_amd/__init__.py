"""MI355X-native exact tiled attention (FlashAttention) — Python binding.

Thin wrappers over the C ABI of ``libfa.so`` (include/fa.h) with the same
names.  They only marshal arguments: check shapes, dtypes and devices of
torch tensors, allocate outputs with torch, and pass raw device pointers plus
the HIP stream.  Every step of the computation runs in the HIP kernels; there
is no CPU or PyTorch fallback.

Every buffer a caller passes (outputs, lse, workspace, key lengths, block
masks) is checked for shape, dtype, device and layout before its pointer
reaches the library, since the kernels write through it without bounds.
When ``stream`` is not the current stream, tensors that the binding
allocates are marked as used on ``stream`` (``record_stream``), so torch's
caching allocator does not hand their memory to other work while the
kernels still run.
"""

from __future__ import annotations

import math

from ._lib import FaLayout, FaStrides
from ._lib import (FA_BF16, FA_BWD_STAGE_D, FA_BWD_STAGE_DKDV, FA_BWD_STAGE_DQ,  # noqa: F401
                   FA_BWD_STAGE_GRADS,  # noqa: F401
                   FA_ERR_HIP, FA_ERR_INVALID, FA_ERR_TOO_LARGE, FA_ERR_UNSUPPORTED,  # noqa: F401
                   FA_F16, FA_F32, FA_NOALLOC_SCRATCH_BYTES, FA_OK, FaError, check,  # noqa: F401
                   load)

__all__ = ["fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_fwd_blocksparse", "fa_bwd_blocksparse",
           "fa_bwd_stage", "fa_bwd_workspace_size", "fa_decode", "fa_decode_workspace_size",
           "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_strided", "fa_bwd_strided", "FaError",
           "load"]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_qkv(*ts):
    """Tensors of q's shape, dtype and device, contiguous [B, H, N, d]."""
    q = ts[0]
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in ts:
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, dO and the gradients must share shape and dtype")
        if not t.is_cuda or t.device != q.device:
            raise ValueError("tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")


def _check_lse(lse, q, rows=None):
    """lse: contiguous float32 [B, H, rows] (rows = N) on q's device."""
    torch = _torch()
    B, H, N = q.shape[0], q.shape[1], q.shape[2] if rows is None else rows
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_cuda
            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 tensor [{B}, {H}, {N}] on q's GPU")


def _check_workspace(ws, q, need):
    if not ws.is_cuda or ws.device != q.device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's GPU")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes; {need} needed")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, q):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return stream.cuda_stream


def _keep(stream, q, *ts):
    """Mark tensors the binding allocated (or copied) as in use on
    ``stream`` when it is not q's current stream."""
    torch = _torch()
    if stream is None or stream == torch.cuda.current_stream(q.device):
        return
    for t in ts:
        if t is not None:
            t.record_stream(stream)


def _call(q, name, *args):
    """The C entry point `name` with q's device current (the library launches
    on the current device, which must be the one that owns the stream)."""
    torch = _torch()
    with torch.cuda.device(q.device):
        return getattr(load(), name)(*args)


def _key_len(key_len, q):
    torch = _torch()
    if key_len is None:
        return None
    if (key_len.dtype != torch.int32 or not key_len.is_cuda or key_len.device != q.device
            or key_len.numel() != q.shape[0]):
        raise ValueError("key_len must be an int32 tensor [B] on the same GPU")
    return key_len.contiguous()


def _block_mask(block_mask, q, block_size):
    torch = _torch()
    if (block_mask.dtype != torch.uint8 or not block_mask.is_cuda
            or block_mask.device != q.device or block_mask.dim() != 2):
        raise ValueError("block_mask must be a uint8 [nb, nb] tensor on the same GPU")
    nb = (q.shape[2] + block_size - 1) // block_size
    if tuple(block_mask.shape) != (nb, nb):
        raise ValueError(f"block_mask must be [{nb}, {nb}]")
    return block_mask.contiguous()


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _fwd_outputs(q, out, lse):
    """(o, lse, allocated): the caller's buffers checked, or new ones."""
    torch = _torch()
    B, H, N, _ = q.shape
    made = []
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
        made.append(out)
    _check_qkv(q, out)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        made.append(lse)
    _check_lse(lse, q)
    return out, lse, made


def fa_fwd(q, k, v, scale=None, causal=False, key_len=None, out=None, lse=None,
           stream=None):
    """O, lse = softmax(q k^T * scale + mask) v; see include/fa.h (fa_fwd)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    kl = _key_len(key_len, q)
    o, lse, made = _fwd_outputs(q, out, lse)
    st = _call(q, "fa_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
               _scale(scale, d), int(bool(causal)), _ptr(kl), _dtype_code(q), _stream(stream, q))
    check("fa_fwd", st)
    _keep(stream, q, kl, *made)
    return o, lse


def fa_bwd_workspace_size(B, H, N, d):
    return int(load().fa_bwd_workspace_size(B, H, N, d))


def _bwd_outputs(q, dq, dk, dv, workspace):
    """(dq, dk, dv, workspace, allocated): the caller's buffers checked, or
    new ones."""
    torch = _torch()
    B, H, N, d = q.shape
    made = []
    grads = []
    for g in (dq, dk, dv):
        if g is None:
            g = torch.empty_like(q, memory_format=torch.contiguous_format)
            made.append(g)
        grads.append(g)
    _check_qkv(q, *grads)
    need = fa_bwd_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=q.device)
        made.append(workspace)
    _check_workspace(workspace, q, need)
    return (*grads, workspace, made)


def fa_bwd(q, k, v, o, lse, dO, scale=None, causal=False, key_len=None, dq=None, dk=None,
           dv=None, workspace=None, stream=None):
    """dq, dk, dv of sum(dO * O); see include/fa.h (fa_bwd)."""
    _check_qkv(q, k, v, o, dO)
    _check_lse(lse, q)
    B, H, N, d = q.shape
    kl = _key_len(key_len, q)
    dq, dk, dv, ws, made = _bwd_outputs(q, dq, dk, dv, workspace)
    st = _call(q, "fa_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
               _ptr(dk), _ptr(dv), B, H, N, d, _scale(scale, d), int(bool(causal)), _ptr(kl),
               _ptr(ws), ws.numel() * ws.element_size(), _dtype_code(q), _stream(stream, q))
    check("fa_bwd", st)
    _keep(stream, q, kl, *made)
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, scale=None, causal=False, key_len=None,
                   stream=None):
    """fa_bwd with the library's fixed workspace array; dq, dk, dv are the
    caller's (contiguous [B, H, N, d], q's dtype and device), and nothing is
    allocated on the way to the C call (key_len must be contiguous); see
    include/fa.h (fa_bwd_noalloc)."""
    _check_qkv(q, k, v, o, dO, dq, dk, dv)
    _check_lse(lse, q)
    B, H, N, d = q.shape
    if key_len is not None and not key_len.is_contiguous():
        raise ValueError("key_len must be contiguous (fa_bwd_noalloc makes no copies)")
    kl = _key_len(key_len, q)
    st = _call(q, "fa_bwd_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, _scale(scale, d), int(bool(causal)),
               _ptr(kl), _dtype_code(q), _stream(stream, q))
    check("fa_bwd_noalloc", st)
    return dq, dk, dv


def fa_fwd_blocksparse(q, k, v, block_mask, block_size=128, scale=None, out=None, lse=None,
                       stream=None):
    """Block-sparse forward; see include/fa.h (fa_fwd_blocksparse)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    bm = _block_mask(block_mask, q, block_size)
    o, lse, made = _fwd_outputs(q, out, lse)
    st = _call(q, "fa_fwd_blocksparse", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
               _scale(scale, d), _ptr(bm), block_size, _dtype_code(q), _stream(stream, q))
    check("fa_fwd_blocksparse", st)
    _keep(stream, q, bm, *made)
    return o, lse


def fa_bwd_blocksparse(q, k, v, o, lse, dO, block_mask, block_size=128, scale=None, dq=None,
                       dk=None, dv=None, workspace=None, stream=None):
    """Block-sparse backward; see include/fa.h (fa_bwd_blocksparse)."""
    _check_qkv(q, k, v, o, dO)
    _check_lse(lse, q)
    B, H, N, d = q.shape
    bm = _block_mask(block_mask, q, block_size)
    dq, dk, dv, ws, made = _bwd_outputs(q, dq, dk, dv, workspace)
    st = _call(q, "fa_bwd_blocksparse", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, _scale(scale, d), _ptr(bm), block_size,
               _ptr(ws), ws.numel() * ws.element_size(), _dtype_code(q), _stream(stream, q))
    check("fa_bwd_blocksparse", st)
    _keep(stream, q, bm, *made)
    return dq, dk, dv


def fa_bwd_stage(stage, q, k, v, o, lse, dO, dq, dk, dv, workspace, scale=None, causal=False,
                 key_len=None, block_mask=None, block_size=128, stream=None):
    """One stage of the backward (FA_BWD_STAGE_D, _DKDV, _DQ or _GRADS); outputs and
    workspace are caller-allocated; see include/fa.h (fa_bwd_stage)."""
    _check_qkv(q, k, v, o, dO, dq, dk, dv)
    _check_lse(lse, q)
    B, H, N, d = q.shape
    _check_workspace(workspace, q, fa_bwd_workspace_size(B, H, N, d))
    kl = _key_len(key_len, q)
    bm = None if block_mask is None else _block_mask(block_mask, q, block_size)
    st = _call(q, "fa_bwd_stage", int(stage), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
               _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, _scale(scale, d),
               int(bool(causal)), _ptr(kl), _ptr(bm), block_size, _ptr(workspace),
               workspace.numel() * workspace.element_size(), _dtype_code(q), _stream(stream, q))
    check("fa_bwd_stage", st)
    _keep(stream, q, kl, bm)


def fa_decode_workspace_size(B, H, Nq, Nk, d):
    return int(load().fa_decode_workspace_size(B, H, Nq, Nk, d))


def fa_decode(q, k, v, scale=None, key_len=None, out=None, lse=None, workspace=None,
              stream=None):
    """Nq new queries [B, H, Nq, d] against keys/values [B, H, Nk, d] (keys
    j >= key_len[b] hidden, no causal order); see include/fa.h (fa_decode).
    Returns (O [B, H, Nq, d], lse [B, H, Nq])."""
    torch = _torch()
    for t in (q, k, v):
        if t.dim() != 4 or t.dtype != q.dtype or not t.is_cuda or t.device != q.device:
            raise ValueError("q, k, v must be [B, H, n, d] tensors of one dtype on one GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    kl = _key_len(key_len, q)
    o, lse, made = _fwd_outputs(q, out, lse)
    need = fa_decode_workspace_size(B, H, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=q.device)
        made.append(workspace)
    _check_workspace(workspace, q, need)
    st = _call(q, "fa_decode", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
               _scale(scale, d), _ptr(kl), _ptr(workspace),
               workspace.numel() * workspace.element_size(), _dtype_code(q), _stream(stream, q))
    check("fa_decode", st)
    _keep(stream, q, kl, *made)
    return o, lse


def _seed(seed, offset):
    seed, offset = int(seed), int(offset)
    if not (0 <= seed < 1 << 64 and 0 <= offset < 1 << 32):
        raise ValueError("seed must fit 64 bits and offset 32 bits (unsigned)")
    return seed, offset


def fa_fwd_dropout(q, k, v, dropout_p, seed, offset=0, scale=None, causal=False, key_len=None,
                   out=None, lse=None, stream=None):
    """fa_fwd with dropout on the probabilities; see include/fa.h
    (fa_fwd_dropout).  Returns (O, lse)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    kl = _key_len(key_len, q)
    sd, off = _seed(seed, offset)
    o, lse, made = _fwd_outputs(q, out, lse)
    st = _call(q, "fa_fwd_dropout", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
               _scale(scale, d), int(bool(causal)), _ptr(kl), float(dropout_p), sd, off,
               _dtype_code(q), _stream(stream, q))
    check("fa_fwd_dropout", st)
    _keep(stream, q, kl, *made)
    return o, lse


def fa_bwd_dropout(q, k, v, o, lse, dO, dropout_p, seed, offset=0, scale=None, causal=False,
                   key_len=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward of fa_fwd_dropout (same dropout_p, seed, offset); see
    include/fa.h (fa_bwd_dropout).  Returns (dq, dk, dv)."""
    _check_qkv(q, k, v, o, dO)
    _check_lse(lse, q)
    B, H, N, d = q.shape
    kl = _key_len(key_len, q)
    sd, off = _seed(seed, offset)
    dq, dk, dv, ws, made = _bwd_outputs(q, dq, dk, dv, workspace)
    st = _call(q, "fa_bwd_dropout", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, _scale(scale, d), int(bool(causal)),
               _ptr(kl), float(dropout_p), sd, off, _ptr(ws), ws.numel() * ws.element_size(),
               _dtype_code(q), _stream(stream, q))
    check("fa_bwd_dropout", st)
    _keep(stream, q, kl, *made)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Strided views (fa_fwd_strided, fa_bwd_strided)
# ---------------------------------------------------------------------------

def _view_ok(t):
    """Whether the kernels can read or write the [B, H, N, d] view t in
    place: d contiguous, every other stride and the base 16-byte aligned."""
    align = 16 // t.element_size()
    st = t.stride()
    return (st[3] == 1 and all(x >= 0 and x % align == 0 for x in st[:3])
            and t.data_ptr() % 16 == 0 and st[2] < (1 << 24))


def _as_view(t):
    """t itself when the kernels take it in place, else a packed copy (a
    layout they cannot address: d not contiguous, or unaligned strides)."""
    return t if _view_ok(t) else t.contiguous()


def _check_views(*ts):
    """Tensors of q's shape, dtype and device (any strides)."""
    q = ts[0]
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in ts:
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, dO and the gradients must share shape and dtype")
        if not t.is_cuda or t.device != q.device:
            raise ValueError("tensors must be on the same GPU")


def _strides(t):
    return FaStrides(*t.stride()[:3]) if t is not None else FaStrides(0, 0, 1)


def _layout(q=None, k=None, v=None, o=None, dO=None, dq=None, dk=None, dv=None):
    return FaLayout(*(_strides(t) for t in (q, k, v, o, dO, dq, dk, dv)))


def _out_view(like, out):
    """The caller's output view (checked: writable in place, rows apart), or
    a new tensor with like's memory order (a [B, N, H, d]-ordered input gives
    a [B, N, H, d]-ordered output)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(like)  # keeps the stride order of dense views
        if not _view_ok(out):
            out = torch.empty(like.shape, dtype=like.dtype, device=like.device)
        return out, [out]
    _check_views(like, out)
    if not _view_ok(out) or out.stride(2) < out.shape[3]:
        raise ValueError("output views need a contiguous d, 16-byte aligned strides and rows "
                         "at least d elements apart")
    return out, []


def _mask_args(q, causal, key_len, block_mask, block_size):
    kl = _key_len(key_len, q)
    bm = None if block_mask is None else _block_mask(block_mask, q, block_size)
    if bm is not None and (causal or kl is not None):
        raise ValueError("block_mask is not combined with causal or key_len")
    return kl, bm


def fa_fwd_strided(q, k, v, scale=None, causal=False, key_len=None, block_mask=None,
                   block_size=128, dropout_p=0.0, seed=0, offset=0, out=None, lse=None,
                   stream=None):
    """The forward on [B, H, N, d] views of any strides (e.g. the transpose of
    [B, N, H, d] activations), read and written in place; every mask and
    dropout option in one call.  See include/fa.h (fa_fwd_strided).
    Returns (O, lse); O has q's memory order unless `out` is given."""
    torch = _torch()
    _check_views(q, k, v)
    q, k, v = (_as_view(t) for t in (q, k, v))
    B, H, N, d = q.shape
    kl, bm = _mask_args(q, causal, key_len, block_mask, block_size)
    sd, off = _seed(seed, offset)
    o, made = _out_view(q, out)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        made.append(lse)
    _check_lse(lse, q)
    lay = _layout(q=q, k=k, v=v, o=o)
    st = _call(q, "fa_fwd_strided", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
               _scale(scale, d), int(bool(causal)), _ptr(kl), _ptr(bm), block_size,
               float(dropout_p), sd, off, lay, _dtype_code(q), _stream(stream, q))
    check("fa_fwd_strided", st)
    _keep(stream, q, kl, bm, *made)
    return o, lse


def fa_bwd_strided(q, k, v, o, lse, dO, scale=None, causal=False, key_len=None, block_mask=None,
                   block_size=128, dropout_p=0.0, seed=0, offset=0, dq=None, dk=None, dv=None,
                   workspace=None, stream=None):
    """The backward of fa_fwd_strided on views of any strides; dq, dk, dv
    take the memory order of q, k, v unless given.  See include/fa.h
    (fa_bwd_strided).  Returns (dq, dk, dv)."""
    torch = _torch()
    _check_views(q, k, v, o, dO)
    q, k, v, o, dO = (_as_view(t) for t in (q, k, v, o, dO))
    _check_lse(lse, q)
    B, H, N, d = q.shape
    kl, bm = _mask_args(q, causal, key_len, block_mask, block_size)
    sd, off = _seed(seed, offset)
    dq, m1 = _out_view(q, dq)
    dk, m2 = _out_view(k, dk)
    dv, m3 = _out_view(v, dv)
    made = m1 + m2 + m3
    need = fa_bwd_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16) // 4 + 4, dtype=torch.float32, device=q.device)
        made.append(workspace)
    _check_workspace(workspace, q, need)
    lay = _layout(q=q, k=k, v=v, o=o, dO=dO, dq=dq, dk=dk, dv=dv)
    st = _call(q, "fa_bwd_strided", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
               _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, _scale(scale, d), int(bool(causal)),
               _ptr(kl), _ptr(bm), block_size, float(dropout_p), sd, off, lay, _ptr(workspace),
               workspace.numel() * workspace.element_size(), _dtype_code(q), _stream(stream, q))
    check("fa_bwd_strided", st)
    _keep(stream, q, kl, bm, *made)
    return dq, dk, dv

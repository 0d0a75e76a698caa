"""Torch-facing wrappers of the C ABI (device memory and streams come from PyTorch).

Two layers:
  * gbsa_metadata / gbsa_workspace_size / gbsa_forward / gbsa_forward_tnd / gbsa_num_workers /
    gbsa_check_params:
    the C entry points with the same names, taking a GbsaParams block and tensors;
  * generic_block_sparse_attention_metadata / generic_block_sparse_attention: the keyword
    interface of the GenericBlockSparseAttention article's PyTorch section (TND query,
    PA_BBND key/value, returns metadata, then (attention_out, softmax_lse)).
Only argument marshalling happens here; all computation runs in libgbsa's HIP kernels.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import GbsaParams, check

_DTYPE_CODE = {torch.float16: _lib.DTYPE_F16, torch.bfloat16: _lib.DTYPE_BF16,
               torch.float8_e4m3fn: _lib.DTYPE_FP8_E4M3}
_CODE_DTYPE = {v: k for k, v in _DTYPE_CODE.items()}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, contiguous=True):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_params(*, batch: int, num_heads_q: int, num_heads_kv: int, total_q: int,
                total_q_blocks: int, top_k: int, block_x: int, max_blocks_per_seq: int,
                num_pages: int, kv_page_stride: int = 0, dtype=torch.float16,
                out_dtype=None, mask_mode: int = 1, win_left: int = -1, win_right: int = -1,
                quant_mode: int = 0, softmax_precision: int = 0, return_lse: bool = False,
                has_seqused_q: bool = False, scale: float = 0.0, num_workers: int = 0,
                block_y: int = 128, head_dim: int = 128, kv_layout: int = 0,
                max_seqlen_q: int = -1, max_seqlen_kv: int = -1,
                dst_type_max: float = 0.0) -> GbsaParams:
    """kv_layout 0 = PA_BBND (num_pages pages), 1 = TND (num_pages = rows of key/value).
    max_seqlen_q / max_seqlen_kv: -1 (not given) or bounds that gbsa_validate checks.
    softmax_precision: 0 (fp32, the default here) or 1 (the 16-bit online softmax with f16;
    the keyword interface keeps the article's default of 1)."""
    p = GbsaParams()
    p.batch = batch
    p.num_heads_q = num_heads_q
    p.num_heads_kv = num_heads_kv
    p.head_dim = head_dim
    p.total_q = total_q
    p.total_q_blocks = total_q_blocks
    p.top_k = top_k
    p.block_x = block_x
    p.block_y = block_y
    p.page_size = 128
    p.max_blocks_per_seq = max_blocks_per_seq
    p.num_pages = num_pages
    p.kv_page_stride = kv_page_stride
    p.dtype = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    od = dtype if out_dtype is None else out_dtype
    p.out_dtype = _DTYPE_CODE[od] if isinstance(od, torch.dtype) else int(od)
    p.mask_mode = int(mask_mode)
    p.win_left = int(win_left)
    p.win_right = int(win_right)
    p.quant_mode = int(quant_mode)
    p.softmax_precision = int(softmax_precision)
    p.dst_type_max = float(dst_type_max)
    p.return_lse = int(bool(return_lse))
    p.is_packed_gqa = 1
    p.has_seqused_q = int(bool(has_seqused_q))
    p.scale = float(scale)
    p.num_workers = int(num_workers)
    p.kv_layout = int(kv_layout)
    p.max_seqlen_q = int(max_seqlen_q)
    p.max_seqlen_kv = int(max_seqlen_kv)
    return p


# ---------------------------------------------------------------------------
# C entry points
# ---------------------------------------------------------------------------

def gbsa_check_params(params: GbsaParams) -> int:
    return _lib.load().gbsa_check_params(ctypes.byref(params))


def gbsa_num_workers(params: GbsaParams) -> int:
    n = ctypes.c_int32(0)
    check("gbsa_num_workers", _lib.load().gbsa_num_workers(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def gbsa_workspace_size(params: GbsaParams) -> int:
    n = ctypes.c_size_t(0)
    check("gbsa_workspace_size",
          _lib.load().gbsa_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def gbsa_metadata(params: GbsaParams, sparse_block_count: torch.Tensor,
                  cu_seqlens_q: torch.Tensor, seqused_q: Optional[torch.Tensor],
                  seqused_kv: Optional[torch.Tensor], metadata: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    _need(sparse_block_count, "sparse_block_count", torch.int32)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int64)
    if seqused_kv is not None:
        _need(seqused_kv, "seqused_kv", torch.int32)
    if seqused_q is not None:
        _need(seqused_q, "seqused_q", torch.int32)
    if metadata is None:
        metadata = torch.empty(_lib.METADATA_SIZE, dtype=torch.int32,
                               device=sparse_block_count.device)
    _need(metadata, "metadata", torch.int32)
    if metadata.numel() != _lib.METADATA_SIZE:
        raise ValueError("metadata must hold 1024 int32")
    code = _lib.load().gbsa_metadata(ctypes.byref(params), _ptr(sparse_block_count),
                                     _ptr(cu_seqlens_q), _ptr(seqused_q), _ptr(seqused_kv),
                                     _ptr(metadata), _stream(stream))
    check("gbsa_metadata", code)
    return metadata


def gbsa_forward(params: GbsaParams, q, k, v, sparse_block_idx, sparse_block_count, metadata,
                 cu_seqlens_q, seqused_q, seqused_kv, block_table, q_scale=None, k_scale=None,
                 v_scale=None, p_scale=None, out=None, lse=None, workspace=None,
                 stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """Returns (attention_out, softmax_lse or None, workspace)."""
    _need(q, "query")
    for name, t in (("key", k), ("value", v)):
        _need(t, name, contiguous=False)
        D, N2 = t.shape[3], t.shape[2]
        if t.stride(3) != 1 or t.stride(2) != D or t.stride(1) != N2 * D:
            raise ValueError(f"{name}: only the page axis (dim 0) may be strided")
    if k.stride(0) != v.stride(0):
        raise ValueError("key and value must share the page stride")
    _need(sparse_block_idx, "sparse_block_idx", torch.int32)
    _need(sparse_block_count, "sparse_block_count", torch.int32)
    _need(block_table, "block_table", torch.int32)
    if out is None:
        out = torch.empty(q.shape, dtype=_CODE_DTYPE[params.out_dtype], device=q.device)
    if lse is None and params.return_lse:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.zeros(gbsa_workspace_size(params), dtype=torch.uint8, device=q.device)
    code = _lib.load().gbsa_forward(
        ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(sparse_block_idx),
        _ptr(sparse_block_count), _ptr(metadata), _ptr(cu_seqlens_q), _ptr(seqused_q),
        _ptr(seqused_kv), _ptr(block_table), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
        _ptr(p_scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
        _stream(stream))
    check("gbsa_forward", code)
    return out, lse, workspace


def gbsa_forward_tnd(params: GbsaParams, q, k, v, sparse_block_idx, sparse_block_count,
                     metadata, cu_seqlens_q, seqused_q, cu_seqlens_kv, seqused_kv=None,
                     q_scale=None, k_scale=None, v_scale=None, p_scale=None, out=None, lse=None,
                     workspace=None, stream=None
                     ) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """Token-major key/value [T_kv, N2, D]; returns (attention_out, softmax_lse or None,
    workspace)."""
    _need(q, "query")
    _need(k, "key")
    _need(v, "value")
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("key and value must both be [T_kv, N2, D]")
    _need(sparse_block_idx, "sparse_block_idx", torch.int32)
    _need(sparse_block_count, "sparse_block_count", torch.int32)
    _need(cu_seqlens_kv, "cu_seqlens_kv", torch.int64)
    if seqused_kv is not None:
        _need(seqused_kv, "seqused_kv", torch.int32)
    if out is None:
        out = torch.empty(q.shape, dtype=_CODE_DTYPE[params.out_dtype], device=q.device)
    if lse is None and params.return_lse:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.zeros(gbsa_workspace_size(params), dtype=torch.uint8, device=q.device)
    code = _lib.load().gbsa_forward_tnd(
        ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(sparse_block_idx),
        _ptr(sparse_block_count), _ptr(metadata), _ptr(cu_seqlens_q), _ptr(seqused_q),
        _ptr(cu_seqlens_kv), _ptr(seqused_kv), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
        _ptr(p_scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
        _stream(stream))
    check("gbsa_forward_tnd", code)
    return out, lse, workspace


def _mask_geometry(atten_mask: torch.Tensor):
    """(batch stride, row stride, rows, cols) of a uint8 or bool mask [rows, cols] or
    [B, rows, cols] whose last axis is dense."""
    if atten_mask.dtype not in (torch.uint8, torch.bool):
        raise ValueError("atten_mask must be uint8 or bool")
    if atten_mask.dim() not in (2, 3) or atten_mask.stride(-1) != 1:
        raise ValueError("atten_mask must be [rows, cols] or [B, rows, cols] with dense rows")
    rows, cols = atten_mask.shape[-2], atten_mask.shape[-1]
    bstride = 0 if atten_mask.dim() == 2 else atten_mask.stride(0)
    return bstride, atten_mask.stride(-2), rows, cols


def aligned_mask(atten_mask: torch.Tensor) -> torch.Tensor:
    """A copy of the mask as uint8 with its row stride padded to a multiple of 4 (the layout
    gbsa_forward_ex requires), or the mask itself when it already qualifies."""
    m = atten_mask.view(torch.uint8) if atten_mask.dtype == torch.bool else atten_mask
    bs, rs, rows, cols = _mask_geometry(m)
    if rs % 4 == 0 and bs % 4 == 0 and m.data_ptr() % 4 == 0:
        return m
    stride = -(-max(cols, 1) // 4) * 4
    shape = m.shape[:-1] + (stride,)
    out = torch.zeros(shape, dtype=torch.uint8, device=m.device)
    out[..., :cols] = m
    return out[..., :cols]


def gbsa_validate(params: GbsaParams, sparse_block_idx, sparse_block_count, cu_seqlens_q,
                  seqused_q=None, *, cu_seqlens_kv=None, seqused_kv=None, block_table=None,
                  atten_mask=None, stream=None) -> int:
    """Opt-in check of the tensor values the forward calls trust; returns the violation bits
    (0 = none; names in _lib.VALIDATE_BITS). Synchronises the stream to read the result."""
    g = _lib.GbsaForwardArgs()
    ptr = lambda t: None if t is None else t.data_ptr()
    g.sparse_block_idx = ptr(sparse_block_idx)
    g.sparse_block_count = ptr(sparse_block_count)
    g.cu_seqlens_q = ptr(cu_seqlens_q)
    g.seqused_q = ptr(seqused_q)
    g.cu_seqlens_kv = ptr(cu_seqlens_kv)
    g.seqused_kv = ptr(seqused_kv)
    g.block_table = ptr(block_table)
    if atten_mask is not None:
        m = atten_mask.view(torch.uint8) if atten_mask.dtype == torch.bool else atten_mask
        bs, rs, rows, cols = _mask_geometry(m)
        g.atten_mask = m.data_ptr()
        g.mask_batch_stride, g.mask_row_stride, g.mask_rows, g.mask_cols = bs, rs, rows, cols
    flags = torch.zeros(1, dtype=torch.int32, device=sparse_block_count.device)
    check("gbsa_validate", _lib.load().gbsa_validate(ctypes.byref(params), ctypes.byref(g),
                                                     _ptr(flags), _stream(stream)))
    return int(flags.item())


def gbsa_forward_ex(params: GbsaParams, q, k, v, sparse_block_idx, sparse_block_count,
                    metadata, cu_seqlens_q, seqused_q=None, *, cu_seqlens_kv=None,
                    seqused_kv=None, block_table=None, q_scale=None, k_scale=None,
                    v_scale=None, p_scale=None, atten_mask=None, out=None, lse=None,
                    workspace=None, stream=None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """Either key/value layout (params.kv_layout) with an optional user attention mask
    (uint8 or bool [rows, cols] or [B, rows, cols], nonzero = masked out; rows must be dense
    and 4-byte aligned, see aligned_mask). Returns (attention_out, softmax_lse or None,
    workspace)."""
    _need(q, "query")
    _need(sparse_block_idx, "sparse_block_idx", torch.int32)
    _need(sparse_block_count, "sparse_block_count", torch.int32)
    if out is None:
        out = torch.empty(q.shape, dtype=_CODE_DTYPE[params.out_dtype], device=q.device)
    if lse is None and params.return_lse:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.zeros(gbsa_workspace_size(params), dtype=torch.uint8, device=q.device)
    g = _lib.GbsaForwardArgs()
    g.query, g.key, g.value = q.data_ptr(), k.data_ptr(), v.data_ptr()
    ptr = lambda t: None if t is None else t.data_ptr()
    g.sparse_block_idx = ptr(sparse_block_idx)
    g.sparse_block_count = ptr(sparse_block_count)
    g.metadata = ptr(metadata)
    g.cu_seqlens_q = ptr(cu_seqlens_q)
    g.seqused_q = ptr(seqused_q)
    g.cu_seqlens_kv = ptr(cu_seqlens_kv)
    g.seqused_kv = ptr(seqused_kv)
    g.block_table = ptr(block_table)
    g.q_scale, g.k_scale, g.v_scale, g.p_scale = (ptr(q_scale), ptr(k_scale), ptr(v_scale),
                                                  ptr(p_scale))
    if atten_mask is not None:
        _need(atten_mask, "atten_mask", contiguous=False)
        m = atten_mask.view(torch.uint8) if atten_mask.dtype == torch.bool else atten_mask
        bs, rs, rows, cols = _mask_geometry(m)
        g.atten_mask = m.data_ptr()
        g.mask_batch_stride, g.mask_row_stride, g.mask_rows, g.mask_cols = bs, rs, rows, cols
    g.attention_out = out.data_ptr()
    g.softmax_lse = ptr(lse)
    g.workspace = workspace.data_ptr()
    g.workspace_bytes = workspace.numel()
    check("gbsa_forward_ex", _lib.load().gbsa_forward_ex(ctypes.byref(params), ctypes.byref(g),
                                                         _stream(stream)))
    return out, lse, workspace


def gbsa_forward_ex_noalloc(params: GbsaParams, q, k, v, sparse_block_idx, sparse_block_count,
                            metadata, cu_seqlens_q, seqused_q=None, *, cu_seqlens_kv=None,
                            seqused_kv=None, block_table=None, q_scale=None, k_scale=None,
                            v_scale=None, p_scale=None, atten_mask=None, out, lse=None,
                            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """gbsa_forward_ex without a workspace: the library's fixed device array holds the split
    partial results. The caller passes the outputs (out, and lse when params.return_lse);
    nothing is allocated here or in the library. Returns (attention_out, softmax_lse)."""
    _need(q, "query")
    _need(sparse_block_idx, "sparse_block_idx", torch.int32)
    _need(sparse_block_count, "sparse_block_count", torch.int32)
    _need(out, "out")
    g = _lib.GbsaForwardArgs()
    g.query, g.key, g.value = q.data_ptr(), k.data_ptr(), v.data_ptr()
    ptr = lambda t: None if t is None else t.data_ptr()
    g.sparse_block_idx = ptr(sparse_block_idx)
    g.sparse_block_count = ptr(sparse_block_count)
    g.metadata = ptr(metadata)
    g.cu_seqlens_q = ptr(cu_seqlens_q)
    g.seqused_q = ptr(seqused_q)
    g.cu_seqlens_kv = ptr(cu_seqlens_kv)
    g.seqused_kv = ptr(seqused_kv)
    g.block_table = ptr(block_table)
    g.q_scale, g.k_scale, g.v_scale, g.p_scale = (ptr(q_scale), ptr(k_scale), ptr(v_scale),
                                                  ptr(p_scale))
    if atten_mask is not None:
        _need(atten_mask, "atten_mask", contiguous=False)
        m = atten_mask.view(torch.uint8) if atten_mask.dtype == torch.bool else atten_mask
        bs, rs, rows, cols = _mask_geometry(m)
        g.atten_mask = m.data_ptr()
        g.mask_batch_stride, g.mask_row_stride, g.mask_rows, g.mask_cols = bs, rs, rows, cols
    g.attention_out = out.data_ptr()
    g.softmax_lse = ptr(lse)
    check("gbsa_forward_ex_noalloc",
          _lib.load().gbsa_forward_ex_noalloc(ctypes.byref(params), ctypes.byref(g),
                                              _stream(stream)))
    return out, lse


def workspace_status(workspace: torch.Tensor) -> int:
    """Word 0 of the workspace: non-zero after a metadata/parameter mismatch (sticky)."""
    return int(workspace[:4].view(torch.int32)[0].item())


# ---------------------------------------------------------------------------
# keyword interface of the article's PyTorch section
# ---------------------------------------------------------------------------

def _common_params(sparse_block_idx, num_heads_q, num_heads_kv, head_dim, block_shape,
                   cu_seqlens_q, seqused_q, mask_mode, quant_mode, softmax_precision,
                   win_left, win_right, is_packed_gqa, layout_q, layout_kv, cu_seqlens_kv):
    if layout_q != "TND" or layout_kv not in ("PA_BBND", "TND"):
        raise ValueError("layout_q must be 'TND' and layout_kv 'PA_BBND' or 'TND'")
    if layout_kv == "PA_BBND" and cu_seqlens_kv is not None:
        raise ValueError("PA_BBND takes seqused_kv, not cu_seqlens_kv")
    if layout_kv == "TND" and cu_seqlens_kv is None:
        raise ValueError("layout_kv 'TND' requires cu_seqlens_kv")
    if not is_packed_gqa:
        raise ValueError("only is_packed_gqa=True is supported")
    if cu_seqlens_q is None:
        raise ValueError("cu_seqlens_q is required with layout TND")
    bx, by = int(block_shape[0]), int(block_shape[1])
    return dict(batch=cu_seqlens_q.numel() - 1, num_heads_q=int(num_heads_q),
                num_heads_kv=int(num_heads_kv), head_dim=int(head_dim),
                total_q_blocks=sparse_block_idx.shape[1], top_k=sparse_block_idx.shape[2],
                block_x=bx, block_y=by, mask_mode=int(mask_mode), win_left=int(win_left),
                win_right=int(win_right), quant_mode=int(quant_mode),
                softmax_precision=int(softmax_precision), has_seqused_q=seqused_q is not None,
                kv_layout=_lib.KV_TND if layout_kv == "TND" else _lib.KV_PA_BBND)


def generic_block_sparse_attention_metadata(
        sparse_block_idx, sparse_block_count, num_heads_q, num_heads_kv, head_dim, block_shape,
        *, cu_seqlens_q=None, cu_seqlens_kv=None, seqused_q=None, seqused_kv=None,
        max_seqlen_q=-1, max_seqlen_kv=-1, is_packed_gqa=True, layout_q="TND",
        layout_kv="PA_BBND", mask_mode=1, quant_mode=0, softmax_precision=1, win_left=-1,
        win_right=-1, num_workers: int = 0) -> torch.Tensor:
    c = _common_params(sparse_block_idx, num_heads_q, num_heads_kv, head_dim, block_shape,
                       cu_seqlens_q, seqused_q, mask_mode, quant_mode, softmax_precision,
                       win_left, win_right, is_packed_gqa, layout_q, layout_kv, cu_seqlens_kv)
    if seqused_kv is None and layout_kv == "PA_BBND":
        raise ValueError("seqused_kv is required with PA_BBND")
    dt = torch.float8_e4m3fn if int(quant_mode) == 5 else torch.float16
    # total_q, max_blocks_per_seq and num_pages do not enter the task split: they only have to
    # hold the given length bounds, which are range-checked like the main call's
    msq, mskv = int(max_seqlen_q), int(max_seqlen_kv)
    p = make_params(total_q=max(1, msq), max_blocks_per_seq=max(1, -(-mskv // 128)),
                    num_pages=max(1, mskv), dtype=dt,
                    out_dtype=torch.bfloat16 if int(quant_mode) == 5 else None,
                    num_workers=num_workers, max_seqlen_q=msq, max_seqlen_kv=mskv, **c)
    return gbsa_metadata(p, sparse_block_count.contiguous(), cu_seqlens_q.contiguous(),
                         None if seqused_q is None else seqused_q.contiguous(),
                         None if seqused_kv is None else seqused_kv.contiguous())


def generic_block_sparse_attention(
        q, k, v, sparse_block_idx, sparse_block_count, block_shape, *, metadata=None,
        attn_mask=None, q_dequant_scale=None, k_dequant_scale=None, v_dequant_scale=None,
        p_quant_scale=None, cu_seqlens_q=None, cu_seqlens_kv=None, seqused_q=None,
        seqused_kv=None, block_table=None, is_packed_gqa=True, layout_q="TND",
        layout_kv="PA_BBND", softmax_scale=0.0, mask_mode=1, quant_mode=0, dst_type_max=0.0,
        softmax_precision=1, win_left=-1, win_right=-1, return_softmax_lse=False,
        attention_out_dtype=None, num_workers: int = 0):
    """Returns (attention_out, softmax_lse) with softmax_lse of shape (T, N1, 1) or empty.

    attn_mask: optional uint8/bool [rows, cols] (shared by all sequences) or [B, rows, cols];
    a nonzero entry (t, p) removes key position p for the batch-local query row t, on top of
    mask_mode (0 none, 1 causal bottom-right, 2 causal top-left) and the window.
    """
    if metadata is None:
        raise ValueError("metadata from generic_block_sparse_attention_metadata is required")
    tnd = layout_kv == "TND"
    if not tnd and (block_table is None or seqused_kv is None):
        raise ValueError("PA_BBND requires block_table and seqused_kv")
    if tnd and block_table is not None:
        raise ValueError("layout_kv 'TND' takes cu_seqlens_kv, not block_table")
    c = _common_params(sparse_block_idx, q.shape[1], k.shape[1 if tnd else 2], q.shape[2],
                       block_shape,
                       cu_seqlens_q, seqused_q, mask_mode, quant_mode, softmax_precision,
                       win_left, win_right, is_packed_gqa, layout_q, layout_kv, cu_seqlens_kv)
    if int(quant_mode) == 0:
        out_dtype = q.dtype
    else:
        if attention_out_dtype is None:
            raise ValueError("attention_out_dtype is required when quant_mode != 0")
        out_dtype = attention_out_dtype
    squ = None if seqused_q is None else seqused_q.contiguous()
    if attn_mask is not None:
        p = make_params(total_q=q.shape[0],
                        max_blocks_per_seq=0 if tnd else block_table.shape[1],
                        num_pages=k.shape[0], kv_page_stride=0 if tnd else k.stride(0),
                        dtype=q.dtype, out_dtype=out_dtype, return_lse=return_softmax_lse,
                        scale=float(softmax_scale), num_workers=num_workers,
                        dst_type_max=float(dst_type_max), **c)
        out, lse, _ = gbsa_forward_ex(
            p, q.contiguous(), k.contiguous() if tnd else k, v.contiguous() if tnd else v,
            sparse_block_idx.contiguous(), sparse_block_count.contiguous(), metadata,
            cu_seqlens_q.contiguous(), squ,
            cu_seqlens_kv=cu_seqlens_kv.contiguous() if tnd else None,
            seqused_kv=None if seqused_kv is None else seqused_kv.contiguous(),
            block_table=None if tnd else block_table.contiguous(), q_scale=q_dequant_scale,
            k_scale=k_dequant_scale, v_scale=v_dequant_scale, p_scale=p_quant_scale,
            atten_mask=aligned_mask(attn_mask))
    elif tnd:
        p = make_params(total_q=q.shape[0], max_blocks_per_seq=0, num_pages=k.shape[0],
                        dtype=q.dtype, out_dtype=out_dtype, return_lse=return_softmax_lse,
                        scale=float(softmax_scale), num_workers=num_workers,
                        dst_type_max=float(dst_type_max), **c)
        out, lse, _ = gbsa_forward_tnd(
            p, q.contiguous(), k.contiguous(), v.contiguous(), sparse_block_idx.contiguous(),
            sparse_block_count.contiguous(), metadata, cu_seqlens_q.contiguous(), squ,
            cu_seqlens_kv.contiguous(), None if seqused_kv is None else seqused_kv.contiguous(),
            q_dequant_scale, k_dequant_scale, v_dequant_scale, p_quant_scale)
    else:
        p = make_params(total_q=q.shape[0], max_blocks_per_seq=block_table.shape[1],
                        num_pages=k.shape[0], kv_page_stride=k.stride(0), dtype=q.dtype,
                        out_dtype=out_dtype, return_lse=return_softmax_lse,
                        scale=float(softmax_scale), num_workers=num_workers,
                        dst_type_max=float(dst_type_max), **c)
        out, lse, _ = gbsa_forward(
            p, q.contiguous(), k, v, sparse_block_idx.contiguous(),
            sparse_block_count.contiguous(), metadata, cu_seqlens_q.contiguous(), squ,
            seqused_kv.contiguous(), block_table.contiguous(), q_dequant_scale,
            k_dequant_scale, v_dequant_scale, p_quant_scale)
    if lse is None:
        lse = torch.empty(0, dtype=torch.float32, device=q.device)
    else:
        lse = lse.unsqueeze(-1)
    return out, lse

"""Seeded synthetic inputs for block-sparse attention over a paged KV cache.

This module only draws inputs: value tensors, page tables, per-query-block
selections and their lengths. It performs none of the attention arithmetic,
so both the float64 oracle and the HIP path consume exactly the same bytes
from here without sharing any computation.

Shapes follow the GenericBlockSparseAttention article (cf-1.com, CANN
ops-transformer GBSA), sections "parameters" and "general constraints":
query is TND [T, N1, D]; key/value are PA_BBND [num_pages, 128, N2, D];
sparse_block_idx is [N2, totalQBlocks, topK] and sparse_block_count is
[N2, totalQBlocks], where totalQBlocks sums ceil(storage_len / blockShapeX)
over the batch.

to_tnd() rewrites a problem's key/value into the token-major TND layout
[T_kv, N2, D] located by cu_seqlens_kv (the article's layoutKv "TND"): the same
logical sequences, copied out of their pages back to back.

Value tensors are drawn with a seeded torch.Generator on the requested
device (CPU for small problems, the GPU for the full-size ones); all integer
structure (lengths, page permutation, selections) is drawn with numpy PCG64
on the host so it is identical everywhere.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

PAGE = 128
HEAD_DIM = 128
FP8_MAX = 448.0

TORCH_DTYPES = {
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8": torch.float8_e4m3fn,
}


@dataclasses.dataclass
class Problem:
    """One block-sparse paged attention problem (inputs only)."""

    name: str
    batch: int
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    block_x: int
    block_y: int
    top_k: int
    dtype: str  # "f16" | "bf16" | "fp8"
    out_dtype: str  # "f16" | "bf16"
    mask_mode: int  # 0 none, 1 causal
    win_left: int
    win_right: int
    return_lse: bool
    scale: float
    cu_seqlens_q: np.ndarray  # int64 [B+1]
    seqused_q: Optional[np.ndarray]  # int32 [B] or None
    seqused_kv: Optional[np.ndarray]  # int32 [B]; None only with TND key/value
    block_table: Optional[np.ndarray]  # int32 [B, max_blocks]; None with TND key/value
    num_pages: int  # pages of the pool, or rows of TND key/value
    sparse_block_idx: np.ndarray  # int32 [N2, totalQBlocks, topK]
    sparse_block_count: np.ndarray  # int32 [N2, totalQBlocks]
    q: torch.Tensor  # [T, N1, D]
    k: torch.Tensor  # [num_pages, 128, N2, D] (page axis may be strided), or TND [T_kv, N2, D]
    v: torch.Tensor
    q_scale: Optional[np.ndarray] = None  # float32 [N1] (fp8 only)
    k_scale: Optional[np.ndarray] = None  # float32 [N2]
    v_scale: Optional[np.ndarray] = None  # float32 [N2]
    seed: int = 0
    kv_storage: Optional[np.ndarray] = None  # int64 [B]: cached KV length of each sequence
    kv_layout: str = "PA_BBND"  # or "TND"
    cu_seqlens_kv: Optional[np.ndarray] = None  # int64 [B+1] (TND only)
    # user attention mask: uint8 [1 or B, rows, row_stride], entries [:, :, :atten_mask_cols]
    # (nonzero = masked out); the bytes past atten_mask_cols are row padding
    atten_mask: Optional[np.ndarray] = None
    atten_mask_cols: int = 0

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def total_q_blocks(self) -> int:
        return int(self.sparse_block_count.shape[1])

    @property
    def group(self) -> int:
        return self.num_heads_q // self.num_heads_kv

    @property
    def quant_mode(self) -> int:
        return 5 if self.dtype == "fp8" else 0

    @property
    def kv_page_stride(self) -> int:
        if self.kv_layout == "TND":
            return 0
        if self.k is None:
            return PAGE * self.num_heads_kv * HEAD_DIM
        return int(self.k.stride(0))

    def kv_len(self, b: int) -> int:
        """Visible KV length of sequence b: seqused_kv, or the TND storage length."""
        if self.seqused_kv is not None:
            return int(self.seqused_kv[b])
        return int(self.cu_seqlens_kv[b + 1] - self.cu_seqlens_kv[b])


# ---------------------------------------------------------------------------
# small shape helpers (bookkeeping only)
# ---------------------------------------------------------------------------

def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def q_block_starts(cu_seqlens_q: np.ndarray, block_x: int) -> List[int]:
    """First global q-block index of every sequence (per the totalQBlocks rule)."""
    starts, acc = [], 0
    for b in range(len(cu_seqlens_q) - 1):
        starts.append(acc)
        acc += _ceil_div(int(cu_seqlens_q[b + 1] - cu_seqlens_q[b]), block_x)
    starts.append(acc)
    return starts


# ---------------------------------------------------------------------------
# value tensors
# ---------------------------------------------------------------------------

def _randn(shape, std: float, gen: torch.Generator, device, out_dtype) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 and cast with round-to-nearest-even, in chunks."""
    out = torch.empty(shape, dtype=out_dtype, device=device)
    flat = out.view(shape[0], -1)
    rows_per_chunk = max(1, (1 << 26) // max(1, flat.shape[1]))
    for r0 in range(0, shape[0], rows_per_chunk):
        r1 = min(shape[0], r0 + rows_per_chunk)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[r0:r1].copy_(x.to(out_dtype))
    return out


def _quantize_fp8_per_head(x: torch.Tensor, head_axis: int):
    """Per-head symmetric e4m3fn quantisation: scale = amax / 448 (dequant scale)."""
    dims = [d for d in range(x.dim()) if d != head_axis]
    amax = x.abs().amax(dim=dims).to(torch.float32)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    shape = [1] * x.dim()
    shape[head_axis] = -1
    q = (x / scale.view(shape)).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q, scale.cpu().numpy().astype(np.float32)


def _values(kind: str, shape, std, gen, device, head_axis):
    if kind == "fp8":
        x = _randn(shape, std, gen, device, torch.float32)
        q, s = _quantize_fp8_per_head(x, head_axis)
        del x
        return q, s
    return _randn(shape, std, gen, device, TORCH_DTYPES[kind]), None


def _paged_kv(num_pages, n2, kind, std, gen, device, page_pad: int):
    """K or V pool [num_pages, 128, N2, D]; page_pad extra elements per page (strided dim0)."""
    inner = PAGE * n2 * HEAD_DIM
    dense, s = _values(kind, (num_pages, PAGE, n2, HEAD_DIM), std, gen, device, 2)
    if page_pad == 0:
        return dense, s
    # padded page axis: only dim0 is strided, the page body stays dense
    stride = inner + page_pad
    backing = torch.zeros((num_pages, stride), dtype=torch.uint8 if kind == "fp8"
                          else TORCH_DTYPES[kind], device=device)
    if kind == "fp8":
        backing[:, :inner] = dense.reshape(num_pages, inner).view(torch.uint8)
        backing = backing.view(torch.float8_e4m3fn)
    else:
        backing[:, :inner] = dense.reshape(num_pages, inner)
    view = backing.as_strided((num_pages, PAGE, n2, HEAD_DIM), (stride, n2 * HEAD_DIM, HEAD_DIM, 1))
    return view, s


# ---------------------------------------------------------------------------
# selections
# ---------------------------------------------------------------------------

SelectFn = Callable[[np.random.Generator, int, int, int], np.ndarray]
"""(rng, q_block_local_index, last_row_local, n_eligible) -> sorted distinct block ids."""


def _fill_selection(n2: int, cu_seqlens_q, seqused_q, seqused_kv, block_x, top_k,
                    rng: np.random.Generator, select: SelectFn, causal_eligible: bool):
    starts = q_block_starts(cu_seqlens_q, block_x)
    tqb = starts[-1]
    idx = np.full((n2, tqb, top_k), -1, dtype=np.int32)
    cnt = np.zeros((n2, tqb), dtype=np.int32)
    for b in range(len(cu_seqlens_q) - 1):
        storage = int(cu_seqlens_q[b + 1] - cu_seqlens_q[b])
        sq = int(seqused_q[b]) if seqused_q is not None else storage
        skv = int(seqused_kv[b])
        off = skv - sq
        nkv = _ceil_div(skv, PAGE)
        for gl in range(starts[b + 1] - starts[b]):
            last = min((gl + 1) * block_x, storage) - 1
            if causal_eligible:
                n_elig = min(nkv, max(0, (last + off) // PAGE + 1))
            else:
                n_elig = nkv
            for h in range(n2):
                sel = select(rng, gl, last, n_elig)
                assert len(sel) <= top_k
                idx[h, starts[b] + gl, :len(sel)] = sel
                cnt[h, starts[b] + gl] = len(sel)
    return idx, cnt


def select_uniform_count(max_count: int) -> SelectFn:
    def f(rng, gl, last, n_elig):
        if n_elig <= 0:
            return np.zeros(0, dtype=np.int32)
        c = min(int(rng.integers(1, max_count + 1)), n_elig)
        return np.sort(rng.choice(n_elig, size=c, replace=False)).astype(np.int32)
    return f


def select_decode_last_plus(n_random: int) -> SelectFn:
    def f(rng, gl, last, n_elig):
        last_blk = n_elig - 1
        rest = rng.choice(last_blk, size=min(n_random, last_blk), replace=False)
        return np.sort(np.concatenate([rest, [last_blk]])).astype(np.int32)
    return f


def select_sink_recent_random(top_k: int, n_recent: int) -> SelectFn:
    def f(rng, gl, last, n_elig):
        if n_elig <= top_k:
            return np.arange(n_elig, dtype=np.int32)
        i = n_elig - 1
        fixed = [0] + list(range(i - n_recent + 1, i + 1))
        pool = np.arange(1, i - n_recent + 1)
        rnd = rng.choice(pool, size=top_k - len(fixed), replace=False)
        return np.sort(np.concatenate([fixed, rnd])).astype(np.int32)
    return f


def select_sink_window(n_sink: int, n_window: int) -> SelectFn:
    def f(rng, gl, last, n_elig):
        e = n_elig - 1
        s = set(range(0, min(n_sink, e + 1))) | set(range(max(0, e - n_window + 1), e + 1))
        return np.array(sorted(s), dtype=np.int32)
    return f


def select_all(rng, gl, last, n_elig):
    return np.arange(n_elig, dtype=np.int32)


# ---------------------------------------------------------------------------
# problem builder
# ---------------------------------------------------------------------------

def build_problem(name: str, *, seed: int, q_lens: Sequence[int], kv_lens: Sequence[int],
                  num_heads_q: int, num_heads_kv: int, block_x: int, top_k: int,
                  dtype: str, select: SelectFn, causal_eligible: bool = True,
                  seqused_q: Optional[Sequence[int]] = None, kv_storage: Optional[Sequence[int]] = None,
                  mask_mode: int = 0, win_left: int = -1, win_right: int = -1,
                  return_lse: bool = True, out_dtype: Optional[str] = None, std: float = 1.0,
                  scale: float = 0.0, device="cpu", extra_pages: int = 0, page_pad: int = 0,
                  shuffle_pages: bool = True, values: bool = True) -> Problem:
    """Assemble a problem. kv_lens are the seqused_kv values; kv_storage the cached lengths.

    values=False leaves q/k/v as None (integer structure only).
    """
    ss = np.random.SeedSequence(seed)
    s_sel, s_perm = [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(2)]
    B = len(q_lens)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(q_lens, dtype=np.int64))
    sk = np.asarray(kv_lens, dtype=np.int32)
    kv_storage = list(kv_storage) if kv_storage is not None else list(kv_lens)
    pages_per_seq = [_ceil_div(int(x), PAGE) for x in kv_storage]
    maxb = max(1, max(pages_per_seq))
    num_pages = sum(pages_per_seq) + extra_pages
    perm = s_perm.permutation(num_pages) if shuffle_pages else np.arange(num_pages)
    table = np.full((B, maxb), -1, dtype=np.int32)
    p = 0
    for b in range(B):
        table[b, :pages_per_seq[b]] = perm[p:p + pages_per_seq[b]]
        p += pages_per_seq[b]
    squ = None if seqused_q is None else np.asarray(seqused_q, dtype=np.int32)
    idx, cnt = _fill_selection(num_heads_kv, cu, squ, sk, block_x, top_k, s_sel, select,
                               causal_eligible)
    T = int(cu[-1])
    q = k = v = qs = ks = vs = None
    if values:
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        q, qs = _values(dtype, (T, num_heads_q, HEAD_DIM), std, gen, device, 1)
        k, ks = _paged_kv(num_pages, num_heads_kv, dtype, std, gen, device, page_pad)
        v, vs = _paged_kv(num_pages, num_heads_kv, dtype, std, gen, device, page_pad)
    if out_dtype is None:
        out_dtype = "bf16" if dtype == "fp8" else dtype
    return Problem(name=name, batch=B, num_heads_q=num_heads_q, num_heads_kv=num_heads_kv,
                   head_dim=HEAD_DIM, block_x=block_x, block_y=PAGE, top_k=top_k, dtype=dtype,
                   out_dtype=out_dtype, mask_mode=mask_mode, win_left=win_left,
                   win_right=win_right, return_lse=return_lse, scale=scale, cu_seqlens_q=cu,
                   seqused_q=squ, seqused_kv=sk, block_table=table, num_pages=num_pages,
                   sparse_block_idx=idx, sparse_block_count=cnt, q=q, k=k, v=v,
                   q_scale=qs, k_scale=ks, v_scale=vs, seed=seed,
                   kv_storage=np.asarray(kv_storage, dtype=np.int64))


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny_prefill_f16",
    2: "decode_bf16",
    3: "block_sparse_prefill_bf16",
    4: "long_context_varlen_f16",
    5: "dense_equivalent_fp8",
}


def decode_workload(batch: int = 64, top_k: int = 16, device="cpu",
                    values: bool = True) -> Problem:
    """Workload 2 and its variants: `batch` single-token queries over 32768-token paged
    sequences (N1=32, N2=8, bf16), each selecting its last page plus top_k - 1 random ones.
    Smaller batches and longer selections cut each unit over several workers (split-KV)."""
    name = CONFIG_NAMES[2] if (batch, top_k) == (64, 16) else f"decode_bf16_b{batch}_top{top_k}"
    return build_problem(name, seed=1002, q_lens=[1] * batch, kv_lens=[32768] * batch,
                         num_heads_q=32, num_heads_kv=8, block_x=1, top_k=top_k, dtype="bf16",
                         select=select_decode_last_plus(top_k - 1), causal_eligible=False,
                         mask_mode=0, return_lse=False, scale=1.0 / math.sqrt(HEAD_DIM),
                         device=device, values=values)


def block_sparse_prefill(block_x: int = 128, device="cpu", values: bool = True) -> Problem:
    """Workload 3 and its variants: 4 x 32768 causal tokens (N1=32, N2=4, bf16), each q-block
    of block_x rows selecting block 0, its 8 most recent eligible blocks and random others, 64
    in all. Smaller block_x gives fewer packed rows per unit (block_x * 8), which moves the
    work to the kernels for 17-64 and 65-256 rows."""
    name = CONFIG_NAMES[3] if block_x == 128 else f"block_sparse_prefill_bf16_x{block_x}"
    return build_problem(name, seed=1003, q_lens=[32768] * 4, kv_lens=[32768] * 4,
                         num_heads_q=32, num_heads_kv=4, block_x=block_x, top_k=64, dtype="bf16",
                         select=select_sink_recent_random(64, 8), mask_mode=1, return_lse=False,
                         scale=1.0 / math.sqrt(HEAD_DIM), device=device, values=values)


def config(cfg_id: int, device="cpu", values: bool = True) -> Problem:
    """Workloads 1..5: seeds 1000 + id, shapes and selection recipes as documented."""
    seed = 1000 + cfg_id
    sc = 1.0 / math.sqrt(HEAD_DIM)
    if cfg_id == 1:
        return build_problem(CONFIG_NAMES[1], seed=seed, q_lens=[256, 384], kv_lens=[256, 384],
                             num_heads_q=8, num_heads_kv=2, block_x=64, top_k=4, dtype="f16",
                             select=select_uniform_count(4), mask_mode=0, return_lse=True,
                             scale=sc, device=device, values=values)
    if cfg_id == 2:
        return decode_workload(64, 16, device=device, values=values)
    if cfg_id == 3:
        return block_sparse_prefill(128, device=device, values=values)
    if cfg_id == 4:
        return build_problem(CONFIG_NAMES[4], seed=seed, q_lens=[131072], kv_lens=[120000],
                             kv_storage=[131072], seqused_q=[120000], num_heads_q=64,
                             num_heads_kv=8, block_x=64, top_k=256, dtype="f16",
                             select=select_sink_window(4, 252), mask_mode=1, win_left=32256,
                             win_right=0, return_lse=True, std=0.5, scale=sc, device=device, values=values)
    if cfg_id == 5:
        B = 2
        return build_problem(CONFIG_NAMES[5], seed=seed, q_lens=[32768] * B, kv_lens=[32768] * B,
                             num_heads_q=16, num_heads_kv=16, block_x=128, top_k=256,
                             dtype="fp8", out_dtype="bf16", select=select_all, mask_mode=1,
                             return_lse=False, scale=sc, device=device, values=values)
    raise ValueError(f"unknown workload {cfg_id}")


def random_problem(seed: int, *, device="cpu", dtype: str = "f16", batch: int = 2,
                   max_len: int = 300, num_heads_q: int = 4, num_heads_kv: int = 2,
                   block_x: int = 32, top_k: int = 4, mask_mode: int = 1,
                   win_left: int = -1, win_right: int = -1, use_seqused_q: bool = False,
                   decode: bool = False, page_pad: int = 0, extra_pages: int = 3,
                   return_lse: bool = True, std: float = 1.0, out_dtype: Optional[str] = None,
                   causal_eligible: Optional[bool] = None, values: bool = True) -> Problem:
    """A small ragged problem for fuzzing: random lengths, selections, optional dual lengths."""
    rng = np.random.Generator(np.random.PCG64(seed + 7_000_000))
    if decode:
        q_lens = [int(rng.integers(1, 3)) for _ in range(batch)]
    else:
        q_lens = [int(rng.integers(1, max_len + 1)) for _ in range(batch)]
    seqused_q = None
    if use_seqused_q:
        seqused_q = [int(rng.integers(max(1, L // 2), L + 1)) for L in q_lens]
    sq = seqused_q if seqused_q is not None else q_lens
    kv_lens = [int(s + rng.integers(0, 200)) for s in sq]
    kv_storage = [int(k + rng.integers(0, 130)) for k in kv_lens]
    if causal_eligible is None:
        causal_eligible = mask_mode == 1
    return build_problem(f"random_{seed}", seed=seed, q_lens=q_lens, kv_lens=kv_lens,
                         kv_storage=kv_storage, seqused_q=seqused_q, num_heads_q=num_heads_q,
                         num_heads_kv=num_heads_kv, block_x=block_x, top_k=top_k, dtype=dtype,
                         select=select_uniform_count(top_k), causal_eligible=causal_eligible,
                         mask_mode=mask_mode, win_left=win_left, win_right=win_right,
                         return_lse=return_lse, std=std, scale=1.0 / math.sqrt(HEAD_DIM),
                         device=device, extra_pages=extra_pages, page_pad=page_pad,
                         out_dtype=out_dtype, values=values)


def to_device(p: Problem, device) -> Problem:
    """Same problem with its value tensors moved (bytes unchanged, strides kept)."""
    def mv(t):
        if t.stride(0) == t[0].numel():
            return t.to(device)
        base = t.as_strided((t.shape[0], t.stride(0)), (t.stride(0), 1))
        nb = base.to(device)
        return nb.as_strided(t.shape, t.stride())
    if p.kv_layout == "TND":
        return dataclasses.replace(p, q=p.q.to(device), k=p.k.to(device), v=p.v.to(device))
    return dataclasses.replace(p, q=p.q.to(device), k=mv(p.k), v=mv(p.v))


def to_tnd(p: Problem, keep_seqused_kv: bool = True, tail_rows: int = 0) -> Problem:
    """The same problem with token-major key/value [T_kv, N2, D] (layoutKv "TND").

    Sequence b's rows are its logical KV positions 0 .. storage_b - 1, copied out of its
    pages; sequences follow each other and cu_seqlens_kv holds the prefix of the storage
    lengths. keep_seqused_kv=False trims every storage to seqused_kv and drops seqused_kv
    (the single-length form). tail_rows extra rows follow the last sequence (zeros); with
    none, the last block of the last sequence runs past the tensor unless its length is a
    multiple of 128.
    """
    assert p.kv_layout == "PA_BBND"
    storage = (np.asarray(p.kv_storage, dtype=np.int64) if p.kv_storage is not None
               else np.asarray(p.seqused_kv, dtype=np.int64))
    if not keep_seqused_kv:
        storage = np.minimum(storage, np.asarray(p.seqused_kv, dtype=np.int64))
    cu_kv = np.zeros(p.batch + 1, dtype=np.int64)
    cu_kv[1:] = np.cumsum(storage)
    fp8 = p.k.dtype == torch.float8_e4m3fn

    def rows(t: torch.Tensor) -> torch.Tensor:
        src = t.view(torch.uint8) if fp8 else t
        out = torch.zeros((int(cu_kv[-1]) + tail_rows, p.num_heads_kv, HEAD_DIM),
                          dtype=src.dtype, device=src.device)
        for b in range(p.batch):
            st = int(storage[b])
            nblk = _ceil_div(st, PAGE)
            if nblk == 0:
                continue
            pages = torch.as_tensor(p.block_table[b, :nblk].astype(np.int64), device=src.device)
            out[int(cu_kv[b]):int(cu_kv[b]) + st] = src[pages].reshape(-1, p.num_heads_kv,
                                                                        HEAD_DIM)[:st]
        return out.view(torch.float8_e4m3fn) if fp8 else out

    return dataclasses.replace(
        p, name=p.name + "_tnd", k=rows(p.k), v=rows(p.v), block_table=None,
        num_pages=int(cu_kv[-1]) + tail_rows, kv_storage=storage, kv_layout="TND",
        cu_seqlens_kv=cu_kv, seqused_kv=p.seqused_kv if keep_seqused_kv else None)


def with_atten_mask(p: Problem, seed: int, density: float = 0.3, per_batch: bool = True,
                    rows: Optional[int] = None, cols: Optional[int] = None,
                    pad: int = 4) -> Problem:
    """The same problem with a random user attention mask.

    Entry (t, p) is masked (a random nonzero byte) with probability `density`. rows / cols
    default to the longest query storage / visible KV length; smaller values leave the rest
    unmasked. Each row is followed by `pad` padding bytes (row stride rounded up to 4) set to
    0xFF, which must never be read as mask entries.
    """
    rng = np.random.Generator(np.random.PCG64(seed + 9_000_000))
    qlen = np.diff(p.cu_seqlens_q)
    kvl = [p.kv_len(b) for b in range(p.batch)]
    rows = int(qlen.max()) if rows is None else int(rows)
    cols = int(max(kvl)) if cols is None else int(cols)
    stride = -(-(cols + pad) // 4) * 4
    nb = p.batch if per_batch else 1
    m = np.full((nb, rows, stride), 0xFF, dtype=np.uint8)
    body = rng.random((nb, rows, cols)) < density
    vals = rng.integers(1, 256, size=(nb, rows, cols), dtype=np.uint8)
    m[:, :, :cols] = np.where(body, vals, 0).astype(np.uint8)
    return dataclasses.replace(p, name=p.name + "_umask", atten_mask=m, atten_mask_cols=cols)


def sweep_problem(seed: int, device="cpu", max_len: int = 300) -> Problem:
    """A random combination of every option (dtype, GQA shape, rows per q-block, selection
    size, mask mode, window, dual lengths, KV layout, user mask, page padding), for sweeps."""
    rng = np.random.Generator(np.random.PCG64(seed + 11_000_000))
    dtype = str(rng.choice(["f16", "bf16", "fp8"]))
    n2 = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    kw = dict(dtype=dtype, num_heads_q=n2 * g, num_heads_kv=n2,
              block_x=int(rng.choice([1, 2, 5, 16, 32, 64, 100, 128])),
              top_k=int(rng.integers(1, 9)), mask_mode=int(rng.integers(0, 3)),
              use_seqused_q=bool(rng.random() < 0.4), batch=int(rng.integers(1, 4)),
              max_len=max_len, return_lse=bool(rng.random() < 0.7),
              std=float(rng.choice([0.5, 1.0])))
    if dtype == "fp8":
        kw["out_dtype"] = str(rng.choice(["f16", "bf16"]))
        kw["std"] = 0.7
    if rng.random() < 0.3:
        kw["win_left"] = int(rng.integers(0, 200))
    if rng.random() < 0.2:
        kw["win_right"] = int(rng.integers(0, 50))
    if kw["mask_mode"] != 1:  # selections over every block, not only causal-eligible ones
        kw["causal_eligible"] = False
    layout = str(rng.choice(["paged", "paged", "tnd", "tnd_single"]))
    if layout == "paged" and rng.random() < 0.4:
        kw["page_pad"] = int(rng.choice([128, 512]))
    p = random_problem(seed, device=device, **kw)
    if layout != "paged":
        p = to_tnd(p, keep_seqused_kv=(layout == "tnd"), tail_rows=int(rng.integers(0, 2)) * 7)
    if rng.random() < 0.3:
        p = with_atten_mask(p, seed, density=float(rng.choice([0.1, 0.5])),
                            per_batch=bool(rng.random() < 0.5))
    return dataclasses.replace(p, name=f"sweep_{seed}")

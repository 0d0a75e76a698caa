"""Plain float64 definition of block-sparse attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring). No online softmax, no
tiling, no fusion: for every query row the selected KV blocks are gathered
through the page table (or, for token-major key/value, from the sequence's rows),
the scaled logits are formed, masked positions are set to -inf and an explicit
full-row softmax is applied.

Sources (GenericBlockSparseAttention article, cf-1.com, CANN ops-transformer):
  * "sparse attention mechanism": out = softmax(scale * q * k_sparse^T + mask) * v_sparse,
    where k_sparse / v_sparse are the KV blocks that sparseBlockIdx /
    sparseBlockCount pick from the paged cache; each Q block of blockShapeX rows
    has its own selection, shared by the query heads of one KV head (packed GQA).
  * "general constraints": q-blocks are cut on each sequence's storage length
    (cu_seqlens_q differences); the task space uses seqused; KV pages are 128
    tokens; N1 % N2 == 0.
  * "mask": the built-in causal mask; win_left / win_right with -1 = unbounded.
  * "quantisation": fp8 e4m3 inputs with dequant scales; output in fp16/bf16.
  * "return values": softmax_lse is float32 of shape (T, N1, 1).
FlashAttention article (ai6s.net), "three steps": the blockwise result equals
the full softmax exactly, so the oracle is the full softmax.

Readings where the pages are silent (each is listed in the design notes):
  * sparse_block_idx holds LOGICAL block numbers of the sequence; the physical
    page is block_table[b, j]. Slots >= count are ignored; count is clamped to
    [0, topK]; negative indices select nothing; duplicates count twice.
  * Key position p = 128*j + r is visible iff p < seqused_kv[b] and the mask
    keeps it. With off = seqused_kv[b] - sq[b] (sq = seqused_q or the storage
    length), causal keeps p <= t + off; a window keeps
    t + off - win_left <= p <= t + off + win_right (a bound of -1 is absent).
  * scale <= 0 means 1/sqrt(D).
  * LSE is the natural log of the sum of exp of the scaled (dequantised) logits;
    a row with no visible key has O = 0 and LSE = -inf.
  * fp8: per-head dequant scales q_scale[N1], k_scale[N2], v_scale[N2]; the
    oracle works on exactly dequantised values and never quantises P.
  * Rows t >= sq[b] are not part of the output (left as NaN here).
  * Token-major (TND) key/value ("general constraints": layoutKv TND comes with
    cu_seqlens_kv, and the dual-length rule then holds on the KV side): sequence
    b owns rows cu_seqlens_kv[b] .. cu_seqlens_kv[b+1]-1, logical block j is its
    rows 128*j .. 128*j+127, and the visible length is seqused_kv[b] when given,
    else the storage length. A seqused_kv above the storage length (which the
    pages forbid) is read as the storage length.
  * mask_mode 2 (not on the pages, which support only the built-in causal mask) is
    causal aligned to the top-left corner: off = 0, keys p <= t (windows are then
    relative to the same diagonal).
  * The user attention mask (the pages list attenMaskOptional and require it to be
    absent): uint8 entries indexed by the batch-local query row t and key position
    p, one [rows, cols] array shared by every sequence or one per sequence; a
    nonzero entry removes the key for that row, on top of every other rule. Entries
    outside [0, rows) x [0, cols) do not mask.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np

from .formats import decode

PAGE = 128


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def q_block_starts(cu_seqlens_q: np.ndarray, block_x: int) -> List[int]:
    """Global index of each sequence's first q-block: prefix of ceil(storage_len / X)."""
    out, acc = [], 0
    for b in range(len(cu_seqlens_q) - 1):
        out.append(acc)
        acc += _ceil_div(int(cu_seqlens_q[b + 1]) - int(cu_seqlens_q[b]), block_x)
    out.append(acc)
    return out


def visible(p: np.ndarray, t: np.ndarray, skv: int, off: int, mask_mode: int,
            win_left: int, win_right: int) -> np.ndarray:
    """Boolean [len(t), len(p)]: key position p visible from batch-local query row t."""
    P = p[None, :]
    d = t[:, None] + off  # the diagonal position of each row
    ok = P < skv
    if mask_mode in (1, 2):  # causal (bottom-right or top-left: the caller's off)
        ok = ok & (P <= d)
    if win_left >= 0:
        ok = ok & (P >= d - win_left)
    if win_right >= 0:
        ok = ok & (P <= d + win_right)
    return np.broadcast_to(ok, (len(t), len(p)))


class Inputs:
    """The raw inputs (numpy; value tensors as storage bit patterns) plus scalars."""

    def __init__(self, q, k, v, sparse_block_idx, sparse_block_count, cu_seqlens_q, seqused_q,
                 seqused_kv, block_table, *, dtype: str, block_x: int, scale: float,
                 mask_mode: int, win_left: int = -1, win_right: int = -1,
                 q_scale=None, k_scale=None, v_scale=None, cu_seqlens_kv=None,
                 atten_mask=None):
        """Paged key/value [pages, 128, N2, D] with block_table and seqused_kv, or, when
        cu_seqlens_kv is given, token-major key/value [T_kv, N2, D] (block_table unused,
        seqused_kv optional). atten_mask: uint8 [rows, cols] (shared) or [B, rows, cols]."""
        self.q, self.k, self.v = q, k, v
        self.idx = np.asarray(sparse_block_idx)
        self.cnt = np.asarray(sparse_block_count)
        self.cu = np.asarray(cu_seqlens_q, dtype=np.int64)
        self.squ = None if seqused_q is None else np.asarray(seqused_q, dtype=np.int64)
        self.tnd = cu_seqlens_kv is not None
        self.cu_kv = np.asarray(cu_seqlens_kv, dtype=np.int64) if self.tnd else None
        if seqused_kv is None and not self.tnd:
            raise ValueError("paged key/value need seqused_kv")
        self.skv = None if seqused_kv is None else np.asarray(seqused_kv, dtype=np.int64)
        self.table = None if self.tnd else np.asarray(block_table)
        self.dtype = dtype
        self.X = int(block_x)
        self.D = int(q.shape[-1])
        self.scale = float(scale) if scale > 0 else 1.0 / math.sqrt(self.D)
        self.mask_mode = int(mask_mode)
        self.wl, self.wr = int(win_left), int(win_right)
        self.N1 = int(q.shape[1])
        self.N2 = int(k.shape[1] if self.tnd else k.shape[2])
        self.G = self.N1 // self.N2
        self.top_k = int(self.idx.shape[2])
        self.qs = None if q_scale is None else np.asarray(q_scale, dtype=np.float64)
        self.ks = None if k_scale is None else np.asarray(k_scale, dtype=np.float64)
        self.vs = None if v_scale is None else np.asarray(v_scale, dtype=np.float64)
        self.starts = q_block_starts(self.cu, self.X)
        self.umask = None
        if atten_mask is not None:
            m = np.asarray(atten_mask)
            self.umask = m[None] if m.ndim == 2 else m

    @property
    def B(self) -> int:
        return len(self.cu) - 1

    def storage(self, b: int) -> int:
        return int(self.cu[b + 1] - self.cu[b])

    def sq(self, b: int) -> int:
        return int(self.squ[b]) if self.squ is not None else self.storage(b)

    def kv_len(self, b: int) -> int:
        """Visible keys of sequence b (seqused_kv; token-major: capped at the storage)."""
        if not self.tnd:
            return int(self.skv[b])
        st = int(self.cu_kv[b + 1] - self.cu_kv[b])
        return st if self.skv is None else min(int(self.skv[b]), st)


def gather_unit(inp: Inputs, b: int, n2: int, g: int):
    """Visible-length-trimmed key positions, K rows and V rows selected for unit (b, n2, g).

    Returns positions [n], K [n, D] and V [n, D] in float64 (dequantised).
    """
    c = min(max(int(inp.cnt[n2, g]), 0), inp.top_k)
    skv = inp.kv_len(b)
    pos, ks, vs = [], [], []
    r = np.arange(PAGE)
    for s in range(c):
        j = int(inp.idx[n2, g, s])
        if j < 0:
            continue
        p = PAGE * j + r
        keep = p < skv
        if not keep.any():
            continue
        pos.append(p[keep])
        if inp.tnd:
            rows = int(inp.cu_kv[b]) + p[keep]
            if rows[-1] >= inp.k.shape[0]:
                raise ValueError(f"batch {b} block {j} reads past the key/value rows")
            ks.append(decode(np.asarray(inp.k[rows, n2, :]), inp.dtype))
            vs.append(decode(np.asarray(inp.v[rows, n2, :]), inp.dtype))
            continue
        page = int(inp.table[b, j])
        if page < 0 or page >= inp.k.shape[0]:
            raise ValueError(f"block table entry {page} for batch {b} block {j} out of range")
        ks.append(decode(np.asarray(inp.k[page, :, n2, :])[keep], inp.dtype))
        vs.append(decode(np.asarray(inp.v[page, :, n2, :])[keep], inp.dtype))
    if not pos:
        z = np.zeros((0, inp.D))
        return np.zeros(0, dtype=np.int64), z, z
    K = np.concatenate(ks)
    V = np.concatenate(vs)
    if inp.ks is not None:
        K = K * inp.ks[n2]
    if inp.vs is not None:
        V = V * inp.vs[n2]
    return np.concatenate(pos), K, V


def attention_unit(inp: Inputs, b: int, n2: int, gl: int, rows: Optional[np.ndarray] = None,
                   return_weights: bool = False):
    """Exact attention for the rows of q-block gl of batch b and the G heads of KV head n2.

    rows: batch-local query rows inside the q-block (default: every row < sq).
    Returns (rows, O [nrows, G, D], LSE [nrows, G]) and optionally the weights
    [nrows, G, n] with the key positions.
    """
    g = inp.starts[b] + gl
    X, G = inp.X, inp.G
    sq = inp.sq(b)
    lo, hi = gl * X, min((gl + 1) * X, sq, inp.storage(b))
    if rows is None:
        rows = np.arange(lo, hi)
    rows = np.asarray(rows, dtype=np.int64)
    assert np.all((rows >= lo) & (rows < hi)), "row outside the q-block's valid range"
    pos, K, V = gather_unit(inp, b, n2, g)
    heads = n2 * G + np.arange(G)
    qv = decode(np.asarray(inp.q[inp.cu[b] + rows][:, heads, :]), inp.dtype)  # [r, G, D]
    if inp.qs is not None:
        qv = qv * inp.qs[heads][None, :, None]
    z = inp.scale * np.einsum("rgd,nd->rgn", qv, K)  # [r, G, n]
    skv = inp.kv_len(b)
    off = 0 if inp.mask_mode == 2 else skv - sq
    vis = visible(pos, rows, skv, off, inp.mask_mode, inp.wl, inp.wr)  # [r, n]
    if inp.umask is not None:
        um = inp.umask[b if inp.umask.shape[0] > 1 else 0]
        inside = (rows[:, None] < um.shape[0]) & (pos[None, :] < um.shape[1])
        r_i = np.minimum(rows, um.shape[0] - 1)[:, None]
        p_i = np.minimum(pos, um.shape[1] - 1)[None, :]
        if um.size:
            vis = vis & ~(inside & (um[r_i, p_i] != 0))
    z = np.where(vis[:, None, :], z, -np.inf)
    O = np.zeros((len(rows), G, inp.D))
    lse = np.full((len(rows), G), -np.inf)
    w = np.zeros_like(z)
    any_vis = vis.any(axis=1)
    if any_vis.any():
        zr = z[any_vis]
        m = zr.max(axis=2, keepdims=True)
        e = np.exp(zr - m)
        ssum = e.sum(axis=2, keepdims=True)
        wr = e / ssum
        w[any_vis] = wr
        O[any_vis] = np.einsum("rgn,nd->rgd", wr, V)
        lse[any_vis] = (m + np.log(ssum))[..., 0]
    if return_weights:
        return rows, O, lse, w, pos
    return rows, O, lse


def sparse_attention(inp: Inputs, rows: Optional[Iterable[int]] = None
                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """O [T, N1, D] and LSE [T, N1] in float64, plus a boolean [T] of computed rows.

    rows: global token indices to compute (default: every row < seqused_q).
    Rows not computed are NaN.
    """
    T = int(inp.cu[-1])
    O = np.full((T, inp.N1, inp.D), np.nan)
    L = np.full((T, inp.N1), np.nan)
    done = np.zeros(T, dtype=bool)
    want: Dict[Tuple[int, int], List[int]] = {}
    if rows is None:
        for b in range(inp.B):
            for t in range(min(inp.sq(b), inp.storage(b))):
                want.setdefault((b, t // inp.X), []).append(t)
    else:
        for tg in rows:
            tg = int(tg)
            b = int(np.searchsorted(inp.cu, tg, side="right") - 1)
            t = tg - int(inp.cu[b])
            if t < min(inp.sq(b), inp.storage(b)):
                want.setdefault((b, t // inp.X), []).append(t)
    for (b, gl), ts in sorted(want.items()):
        ts = np.array(sorted(set(ts)), dtype=np.int64)
        for n2 in range(inp.N2):
            r, o, lse = attention_unit(inp, b, n2, gl, ts)
            heads = n2 * inp.G + np.arange(inp.G)
            tg = inp.cu[b] + r
            O[tg[:, None], heads[None, :]] = o
            L[tg[:, None], heads[None, :]] = lse
        done[inp.cu[b] + ts] = True
    return O, L, done

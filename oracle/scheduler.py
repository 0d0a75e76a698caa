"""Reference task split for the fixed-size metadata buffer (oracle; test infrastructure only).

GenericBlockSparseAttention article (cf-1.com), "two-stage call": a metadata
operator runs first and writes the AICore task split (load-balancing schedule)
into a (1024,) int32 tensor that the main operator consumes; it must be
regenerated for every call and match the main call's parameters. The pages do
not give the buffer's contents; this module is the written specification of
our format, implemented plainly, so the device scheduler can be compared with
it word for word.

Work units, in order: for each batch b, for each KV head n2, for each active
q-block gl < ceil(sq_b / blockShapeX) (sq_b = seqused_q[b], else the storage
length; "general constraints": the task space follows seqused while blocking
follows the storage length). The unit's global q-block is
g = sum_{i<b} ceil(storage_i / X) + gl.

Cost of a unit: c(u) = min(max(count[n2, g], 0), topK) + 1 (one per selected
block plus one for loading Q and writing the result). Prefix costs
C[0] = 0, C[u+1] = C[u] + c(u); W = C[U].

Cut positions: (u, s) "before slot s of unit u", with 0 <= s < max(count_u, 1),
ordered lexicographically, plus the end position (U, 0). The cost consumed
before (u, s) is C[u] + s. Worker w (0 <= w < P) owns the positions from
boundary w up to boundary w+1, where boundary w is the first position whose
consumed cost is >= floor(w * W / P) (integer arithmetic; boundary P = end).

Buffer layout (int32 words):
  [0] magic 0x41534247 ("GBSA" in little-endian bytes)   [1] version (1)
  [2] P   [3] U   [4] W mod 2^32   [5] W div 2^32   [6] number of split units
  [7] N1  [8] N2  [9] D  [10] blockShapeX  [11] blockShapeY  [12] topK
  [13] mask_mode  [14] quant_mode  [15] totalQBlocks  [16] B  [17] win_left
  [18] win_right  [19] seqused_q given (0/1)  [20] is_packed_gqa  [21] kv_layout (0 paged, 1 TND)  [22..23] 0
  [24 + w] boundary w for w = 0..P, packed as (u << 9) | s
  remaining words 0.
A unit is "split" when a boundary falls strictly inside it (s > 0).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

META_WORDS = 1024
HEADER_WORDS = 24
MAX_WORKERS = META_WORDS - HEADER_WORDS - 1  # 999
MAGIC = 0x41534247
VERSION = 1
SLOT_BITS = 9
MAX_UNITS = 1 << (32 - SLOT_BITS - 1)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def units(cu_seqlens_q: Sequence[int], seqused_q: Optional[Sequence[int]], block_x: int,
          num_heads_kv: int) -> List[Tuple[int, int, int]]:
    """Ordered work units (b, n2, g_global)."""
    out = []
    base = 0
    B = len(cu_seqlens_q) - 1
    for b in range(B):
        storage = int(cu_seqlens_q[b + 1]) - int(cu_seqlens_q[b])
        sq = storage if seqused_q is None else min(int(seqused_q[b]), storage)
        nact = _ceil_div(max(sq, 0), block_x)
        for n2 in range(num_heads_kv):
            for gl in range(nact):
                out.append((b, n2, base + gl))
        base += _ceil_div(storage, block_x)
    return out


def effective_count(count: np.ndarray, n2: int, g: int, top_k: int) -> int:
    return min(max(int(count[n2, g]), 0), top_k)


def unit_costs(unit_list, count: np.ndarray, top_k: int) -> List[int]:
    return [effective_count(count, n2, g, top_k) + 1 for (_, n2, g) in unit_list]


def prefix(costs: Sequence[int]) -> List[int]:
    C = [0]
    for c in costs:
        C.append(C[-1] + c)
    return C


def boundary(C: Sequence[int], counts: Sequence[int], target: int) -> Tuple[int, int]:
    """First cut position whose consumed cost is >= target (binary search on C)."""
    U = len(counts)
    if target >= C[U]:
        return (U, 0)
    lo, hi = 0, U  # largest u with C[u] <= target
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if C[mid] <= target:
            lo = mid
        else:
            hi = mid
    u = lo
    s = target - C[u]
    if s < max(counts[u], 1):
        return (u, s)
    return (u + 1, 0)


def boundaries(costs: Sequence[int], counts: Sequence[int], P: int) -> List[Tuple[int, int]]:
    C = prefix(costs)
    W = C[-1]
    return [boundary(C, counts, (w * W) // P) for w in range(P + 1)]


def reference_metadata(*, cu_seqlens_q, seqused_q, sparse_block_count: np.ndarray,
                       num_heads_q: int, num_heads_kv: int, head_dim: int, block_x: int,
                       block_y: int, top_k: int, mask_mode: int, quant_mode: int,
                       win_left: int, win_right: int, num_workers: int,
                       is_packed_gqa: int = 1, kv_layout: int = 0) -> np.ndarray:
    """The full 1024-word metadata buffer for the given inputs and worker count.

    kv_layout (0 paged, 1 token-major) is recorded in the header only: the split depends
    on the selection counts and the query lengths alone."""
    P = int(num_workers)
    assert 1 <= P <= MAX_WORKERS
    cnt = np.asarray(sparse_block_count)
    ul = units(cu_seqlens_q, seqused_q, block_x, num_heads_kv)
    assert len(ul) < MAX_UNITS
    counts = [effective_count(cnt, n2, g, top_k) for (_, n2, g) in ul]
    costs = [c + 1 for c in counts]
    bnd = boundaries(costs, counts, P)
    W = sum(costs)
    split_units = sorted({u for (u, s) in bnd if s > 0})
    meta = np.zeros(META_WORDS, dtype=np.int64)
    meta[0] = MAGIC
    meta[1] = VERSION
    meta[2] = P
    meta[3] = len(ul)
    meta[4] = W & 0xFFFFFFFF
    meta[5] = W >> 32
    meta[6] = len(split_units)
    meta[7:21] = [num_heads_q, num_heads_kv, head_dim, block_x, block_y, top_k, mask_mode,
                  quant_mode, cnt.shape[1], len(cu_seqlens_q) - 1, win_left, win_right,
                  0 if seqused_q is None else 1, is_packed_gqa]
    meta[21] = kv_layout
    for w, (u, s) in enumerate(bnd):
        meta[HEADER_WORDS + w] = (u << SLOT_BITS) | s
    return meta.astype(np.uint32).view(np.int32)


def decode_boundaries(meta: np.ndarray) -> List[Tuple[int, int]]:
    m = np.asarray(meta).astype(np.int64) & 0xFFFFFFFF
    P = int(m[2])
    words = m[HEADER_WORDS:HEADER_WORDS + P + 1]
    return [(int(x) >> SLOT_BITS, int(x) & ((1 << SLOT_BITS) - 1)) for x in words]


def expand_tasks(meta: np.ndarray, counts: Sequence[int]):
    """Tasks (worker, unit, s0, s1) that the buffer assigns, in worker order."""
    bnd = decode_boundaries(meta)
    U = len(counts)
    tasks = []
    for w in range(len(bnd) - 1):
        (u0, s0), (u1, s1) = bnd[w], bnd[w + 1]
        u = u0
        while u < U:
            a = s0 if u == u0 else 0
            if (u, a) >= (u1, s1):
                break
            e = s1 if u == u1 else counts[u]
            tasks.append((w, u, a, e))
            u += 1
    return tasks

"""Pins for the reference task split: hand-worked example, brute force, coverage, balance."""
import json
import os

import numpy as np
import pytest

import gbsa_inputs as gi
from oracle import scheduler as sch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _positions(counts):
    """Every cut position in order with its consumed cost (brute-force enumeration)."""
    out = []
    acc = 0
    for u, c in enumerate(counts):
        for s in range(max(c, 1)):
            out.append(((u, s), acc + s))
        acc += c + 1
    out.append(((len(counts), 0), acc))
    return out


def _brute_boundaries(counts, P):
    pos = _positions(counts)
    W = pos[-1][1]
    res = []
    for w in range(P + 1):
        target = (w * W) // P
        res.append(next(p for p, cost in pos if cost >= target))
    return res


def test_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "scheduler_worked_example.json")))
    counts = ex["counts"]
    costs = [c + 1 for c in counts]
    assert costs == ex["costs"] and sch.prefix(costs) == ex["prefix"]
    bnd = sch.boundaries(costs, counts, ex["num_workers"])
    assert [list(b) for b in bnd] == ex["boundaries"]
    meta = np.zeros(1024, dtype=np.int64)
    meta[2] = ex["num_workers"]
    for w, (u, s) in enumerate(bnd):
        meta[sch.HEADER_WORDS + w] = (u << sch.SLOT_BITS) | s
    assert [list(t) for t in sch.expand_tasks(meta, counts)] == ex["tasks"]


@pytest.mark.parametrize("seed", range(40))
def test_boundaries_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    U = int(rng.integers(1, 40))
    counts = [int(x) for x in rng.integers(0, 9, size=U)]
    if seed % 5 == 0:
        counts = [0] * U
    P = int(rng.integers(1, 3 * U + 5))
    assert sch.boundaries([c + 1 for c in counts], counts, P) == _brute_boundaries(counts, P)


def _counts_for(p):
    ul = sch.units(p.cu_seqlens_q, p.seqused_q, p.block_x, p.num_heads_kv)
    return ul, [sch.effective_count(p.sparse_block_count, n2, g, p.top_k) for (_, n2, g) in ul]


def _meta(p, P):
    return sch.reference_metadata(
        cu_seqlens_q=p.cu_seqlens_q, seqused_q=p.seqused_q,
        sparse_block_count=p.sparse_block_count, num_heads_q=p.num_heads_q,
        num_heads_kv=p.num_heads_kv, head_dim=128, block_x=p.block_x, block_y=128,
        top_k=p.top_k, mask_mode=p.mask_mode, quant_mode=p.quant_mode, win_left=p.win_left,
        win_right=p.win_right, num_workers=P)


@pytest.mark.parametrize("seed,P", [(1, 1), (2, 7), (3, 64), (4, 999), (5, 3), (6, 200)])
def test_coverage_and_balance(seed, P):
    p = gi.random_problem(seed, mask_mode=1, use_seqused_q=seed % 2 == 0, top_k=6, batch=3)
    ul, counts = _counts_for(p)
    meta = _meta(p, P)
    tasks = sch.expand_tasks(meta, counts)
    # coverage: every selected (unit, slot) exactly once; every unit visited
    seen = {}
    for (w, u, a, e) in tasks:
        assert 0 <= a <= e <= counts[u]
        for s in range(a, e):
            seen[(u, s)] = seen.get((u, s), 0) + 1
    want = {(u, s) for u, c in enumerate(counts) for s in range(c)}
    assert set(seen) == want and all(v == 1 for v in seen.values())
    assert {u for (_, u, _, _) in tasks} == set(range(len(counts)))
    # zero-count units are visited exactly once
    for u, c in enumerate(counts):
        if c == 0:
            assert sum(1 for t in tasks if t[1] == u) == 1
    # balance: each worker's consumed cost is within 2 of W/P
    bnd = sch.decode_boundaries(meta)
    C = sch.prefix([c + 1 for c in counts])
    W = C[-1]
    consumed = [C[u] + s if u < len(counts) else W for (u, s) in bnd]
    for w in range(P):
        assert abs((consumed[w + 1] - consumed[w]) - W / P) <= 2 + 1e-9
    # header words
    m = meta.astype(np.int64)
    assert m[0] == sch.MAGIC and m[1] == 1 and m[2] == P and m[3] == len(ul)
    assert m[4] + (m[5] << 32) == W
    assert m[6] == len({u for (u, s) in bnd if s > 0})
    assert np.all(m[sch.HEADER_WORDS + P + 1:] == 0)


def test_units_follow_seqused_not_storage():
    p = gi.config(1)
    ul, counts = _counts_for(p)
    # workload 1: storage lengths 256 and 384 with blockShapeX 64 -> 4 + 6 q-blocks per head
    assert len(ul) == 2 * (4 + 6)
    assert ul[0] == (0, 0, 0) and ul[4] == (0, 1, 0) and ul[8] == (1, 0, 4)
    import dataclasses
    p2 = dataclasses.replace(p, seqused_q=np.array([100, 384], dtype=np.int32))
    ul2, _ = _counts_for(p2)
    # ceil(100/64) = 2 active q-blocks for the first sequence; the second keeps its 6
    assert len(ul2) == 2 * (2 + 6) and ul2[2] == (0, 1, 0) and ul2[4] == (1, 0, 4)

"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small problems are compared on every row; the full-size workloads on sampled rows, with the
same launch configuration the benchmark times. The task split is compared word for word
with the oracle's reference scheduler.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import gbsa_inputs as gi
from helpers import (TOL, GpuProblem, compact_oracle_inputs, compare, compare_rows,
                     gpu_params, oracle_inputs, oracle_rows, out_f64, record_margin)
from oracle import attention as oa
from oracle import scheduler as sch

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_paged_gbsa_amd import _lib
    _lib.load()


def _ref_meta(p, P):
    return sch.reference_metadata(
        cu_seqlens_q=p.cu_seqlens_q, seqused_q=p.seqused_q,
        sparse_block_count=p.sparse_block_count, num_heads_q=p.num_heads_q,
        num_heads_kv=p.num_heads_kv, head_dim=128, block_x=p.block_x, block_y=128,
        top_k=p.top_k, mask_mode=p.mask_mode, quant_mode=p.quant_mode, win_left=p.win_left,
        win_right=p.win_right, num_workers=P, kv_layout=1 if p.kv_layout == "TND" else 0)


def _full_check(p, num_workers=0, label=""):
    _log(f"[parity] {label or p.name} workers={num_workers}")
    gp = GpuProblem(p)
    params, meta, out, lse, ws = gp.run(num_workers)
    assert int(ws[:4].view(torch.int32)[0].item()) == 0
    P = params.num_workers if num_workers else __import__(
        "block_sparse_paged_gbsa_amd").gbsa_num_workers(params)
    np.testing.assert_array_equal(meta.cpu().numpy(), _ref_meta(p, P))
    O, L, done = oa.sparse_attention(oracle_inputs(p))
    return compare(p, out, lse if p.return_lse else None, O, L, done, label or p.name)


# ---------------------------------------------------------------------------
# task split
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_metadata_bit_exact_workloads(cfg):
    p = gi.config(cfg, values=False)
    _log(f"[meta] workload {cfg}")
    gp = GpuProblem(p)
    params = gpu_params(p)
    from block_sparse_paged_gbsa_amd import gbsa_num_workers
    P = gbsa_num_workers(params)
    meta = gp.metadata(params).cpu().numpy()
    np.testing.assert_array_equal(meta, _ref_meta(p, P))
    for P2 in (1, 37, 999):
        meta = gp.metadata(gpu_params(p, P2)).cpu().numpy()
        np.testing.assert_array_equal(meta, _ref_meta(p, P2))


@pytest.mark.parametrize("seed", range(12))
def test_metadata_bit_exact_random(seed):
    rng = np.random.default_rng(seed)
    p = gi.random_problem(seed, values=False, batch=int(rng.integers(1, 6)),
                          use_seqused_q=bool(seed % 2), block_x=int(rng.choice([1, 16, 64, 100])),
                          top_k=int(rng.integers(1, 9)), num_heads_q=8,
                          num_heads_kv=int(rng.choice([1, 2, 4, 8])))
    if seed % 3 == 0:  # some zero-count units
        p.sparse_block_count[:, ::3] = 0
    P = int(rng.integers(1, 1000))
    _log(f"[meta] random seed={seed} P={P}")
    meta = GpuProblem(p).metadata(gpu_params(p, P)).cpu().numpy()
    np.testing.assert_array_equal(meta, _ref_meta(p, P))


@pytest.mark.parametrize("case", ["many_sequences", "large_tables", "max_batch", "huge_units"])
def test_metadata_bit_exact_beyond_lds(case):
    """More than 1024 sequences (up to GBSA_MAX_BATCH, whose tables fill the LDS), or N2 x
    q-block tables larger than LDS (up to 65536 units: workload 3 with 8-row q-blocks): the
    scheduler's chunked path, which must give the same split word for word."""
    if case == "huge_units":
        p = gi.block_sparse_prefill(8, values=False)
    elif case == "many_sequences":
        p = gi.random_problem(31, values=False, decode=True, batch=1500, num_heads_q=8,
                              num_heads_kv=2, block_x=1, top_k=4, use_seqused_q=True)
    elif case == "max_batch":
        p = gi.random_problem(33, values=False, decode=True, batch=16384, num_heads_q=8,
                              num_heads_kv=2, block_x=1, top_k=4, use_seqused_q=True)
    else:
        p = gi.random_problem(32, values=False, batch=12, max_len=4096, block_x=8,
                              num_heads_q=16, num_heads_kv=16, top_k=6, use_seqused_q=True)
    from block_sparse_paged_gbsa_amd import gbsa_num_workers
    gp = GpuProblem(p)
    for P in (1, 999, gbsa_num_workers(gpu_params(p))):
        _log(f"[meta] {case} P={P}")
        meta = gp.metadata(gpu_params(p, P)).cpu().numpy()
        np.testing.assert_array_equal(meta, _ref_meta(p, P))


# ---------------------------------------------------------------------------
# small problems: every row
# ---------------------------------------------------------------------------

def test_workload1_tiny_prefill_all_rows():
    p = gi.config(1, device="cuda")
    err, lerr = _full_check(p, label="workload1")
    _log(f"workload1 O max-abs {err:.3e} LSE rel {lerr:.3e}")


@pytest.mark.parametrize("P", [1, 3, 64, 999])
def test_workload1_any_worker_count(P):
    _full_check(gi.config(1, device="cuda"), num_workers=P, label=f"workload1 P={P}")


CASES = [
    dict(seed=101, dtype="f16", mask_mode=1),
    dict(seed=102, dtype="bf16", mask_mode=0, block_x=16),
    dict(seed=103, dtype="f16", mask_mode=1, win_left=90, win_right=0, use_seqused_q=True),
    dict(seed=104, dtype="bf16", mask_mode=0, win_left=40, win_right=30, num_heads_q=8,
         num_heads_kv=2, block_x=48),
    dict(seed=105, dtype="fp8", mask_mode=1, std=0.7),
    dict(seed=106, dtype="fp8", mask_mode=0, out_dtype="f16", block_x=64, num_heads_q=4,
         num_heads_kv=4),
    dict(seed=107, dtype="bf16", decode=True, batch=5, block_x=1, num_heads_q=16,
         num_heads_kv=4, mask_mode=1),
    dict(seed=108, dtype="f16", decode=True, batch=3, block_x=1, num_heads_q=32,
         num_heads_kv=2, mask_mode=0, top_k=8),
    dict(seed=109, dtype="f16", page_pad=512, mask_mode=1, use_seqused_q=True, block_x=40),
    dict(seed=110, dtype="bf16", num_heads_q=16, num_heads_kv=1, block_x=8, top_k=6),
    dict(seed=111, dtype="f16", num_heads_q=12, num_heads_kv=4, block_x=5, top_k=3,
         mask_mode=1, win_left=0, win_right=0),
    dict(seed=112, dtype="fp8", decode=True, batch=4, block_x=2, num_heads_q=8,
         num_heads_kv=1, top_k=5),
    dict(seed=113, dtype="bf16", batch=1, max_len=700, block_x=128, num_heads_q=8,
         num_heads_kv=1, top_k=6, mask_mode=1),
    dict(seed=114, dtype="f16", batch=4, block_x=17, num_heads_q=2, num_heads_kv=2,
         top_k=4, mask_mode=1, return_lse=False),
    # 256-row subtiles (row-split ping-pong): fp8, and f16 with a window and dual lengths
    dict(seed=115, dtype="fp8", batch=1, max_len=600, block_x=128, num_heads_q=8,
         num_heads_kv=2, top_k=5, mask_mode=1),
    dict(seed=116, dtype="f16", batch=2, max_len=500, block_x=40, num_heads_q=16,
         num_heads_kv=2, top_k=6, mask_mode=1, win_left=100, win_right=0, use_seqused_q=True),
    # 128-row subtiles (key-split ping-pong): 65 and 96 rows, fp8 with f16 output, 2 x 128 rows
    dict(seed=117, dtype="bf16", batch=2, max_len=400, block_x=65, num_heads_q=2,
         num_heads_kv=2, top_k=5, mask_mode=0),
    dict(seed=118, dtype="fp8", batch=2, max_len=500, block_x=96, num_heads_q=4,
         num_heads_kv=4, top_k=4, mask_mode=1, out_dtype="f16"),
    dict(seed=119, dtype="f16", batch=3, max_len=300, block_x=32, num_heads_q=8,
         num_heads_kv=1, top_k=4, mask_mode=1, win_left=50, win_right=-1),
    # 17-32 rows (every page's keys in four slices): fp8 causal with dual lengths, bf16 with a
    # two-sided window
    dict(seed=120, dtype="fp8", block_x=12, mask_mode=1, use_seqused_q=True),
    dict(seed=121, dtype="bf16", block_x=16, mask_mode=1, win_left=70, win_right=10),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c["seed"]) for c in CASES])
def test_random_problem_all_rows(case):
    kw = dict(case)
    seed = kw.pop("seed")
    p = gi.random_problem(seed, device="cuda", **kw)
    for P in (0, 5, 200):
        _full_check(p, num_workers=P, label=f"random{seed} P={P}")


@pytest.mark.parametrize("block_x,dtype", [(1, "bf16"), (2, "f16"), (3, "fp8")],
                         ids=["rows128", "rows256", "rows384"])
def test_maximum_group_and_top_k(block_x, dtype):
    """The largest packed GQA group (128 query heads on one KV head) with top_k = 256 slots:
    128, 256 and 384 packed rows per unit, long selections split across workers."""
    p = gi.build_problem("group128", seed=171, q_lens=[7, 4], kv_lens=[33000, 20000],
                         kv_storage=[33100, 20000], num_heads_q=128, num_heads_kv=1,
                         block_x=block_x, top_k=256, dtype=dtype,
                         select=gi.select_uniform_count(256), causal_eligible=False,
                         mask_mode=0, return_lse=True, scale=1.0 / 128 ** 0.5, device="cuda")
    assert p.sparse_block_count.max() > 200
    for P in (0, 3):
        _full_check(p, num_workers=P, label=f"group128 x{block_x} P={P}")


@pytest.mark.parametrize("num_heads_kv", [1, 4])
def test_unit_split_into_many_pieces(num_heads_kv):
    """One decode query over a 256-slot selection per KV head, cut into hundreds of pieces:
    with one KV head most of the 999 workers are empty (pieces are separated by empty
    workers); with four, nearly every worker holds a one-slot piece, so a unit's pieces span
    more than 64 consecutive workers. The merge must find and combine all of them."""
    p = gi.build_problem("many_pieces", seed=181, q_lens=[1], kv_lens=[32768],
                         num_heads_q=4 * num_heads_kv, num_heads_kv=num_heads_kv, block_x=1,
                         top_k=256, dtype="bf16", select=gi.select_decode_last_plus(255),
                         causal_eligible=False, mask_mode=0, return_lse=True,
                         scale=1.0 / 128 ** 0.5, device="cuda")
    for P in (999, 300, 0):
        _full_check(p, num_workers=P, label=f"many pieces N2={num_heads_kv} P={P}")


def test_maximum_batch():
    """GBSA_MAX_BATCH = 16384 decode-shaped sequences (the scheduler's chunked path), checked
    on sampled sequences including the first and the last."""
    rng = np.random.default_rng(172)
    B = 16384
    kv = rng.integers(1, 400, size=B)
    p = gi.build_problem("max_batch", seed=172, q_lens=[1] * B, kv_lens=kv.tolist(),
                         num_heads_q=4, num_heads_kv=2, block_x=1, top_k=3, dtype="bf16",
                         select=gi.select_uniform_count(3), causal_eligible=False, mask_mode=0,
                         return_lse=True, scale=1.0 / 128 ** 0.5, device="cuda")
    _log("[parity] max batch: gpu")
    params, meta, out, lse, ws = GpuProblem(p).run(0)
    assert int(ws[:4].view(torch.int32)[0].item()) == 0
    from block_sparse_paged_gbsa_amd import gbsa_num_workers
    np.testing.assert_array_equal(meta.cpu().numpy(), _ref_meta(p, gbsa_num_workers(params)))
    rows = sorted({0, 1, B - 1, B - 2} | set(rng.choice(B, 200, replace=False).tolist()))
    inp = compact_oracle_inputs(p, [(b, 0) for b in rows])  # row b is sequence b's only row
    O, L, done = oa.sparse_attention(inp, rows=rows)
    err, lerr = compare(p, out, lse, O, L, done, "max batch")
    _log(f"max batch: rows {int(done.sum())} O max-abs {err:.3e} LSE rel {lerr:.3e}")


# The fp8 key-split kernel with K and V moved by LDS DMA (65-256 rows per unit, no user mask,
# no P scale): two 128-row subtiles, a ragged second subtile with f16 output, one-page units
# (every move past the unit's stream clamped), a sliding window with dual lengths, token-major
# key/value; at the library's worker count, three workers and 200 (split units merged).
DMA8_CASES = [
    dict(seed=181, batch=2, max_len=700, block_x=128, num_heads_q=4, num_heads_kv=2, top_k=6,
         mask_mode=1),
    dict(seed=182, batch=2, max_len=600, block_x=100, num_heads_q=4, num_heads_kv=2, top_k=5,
         mask_mode=1, out_dtype="f16"),
    dict(seed=183, batch=3, max_len=500, block_x=128, num_heads_q=2, num_heads_kv=2, top_k=1,
         mask_mode=0),
    dict(seed=184, batch=2, max_len=900, block_x=80, num_heads_q=8, num_heads_kv=8, top_k=7,
         mask_mode=1, win_left=200, win_right=0, use_seqused_q=True),
    dict(seed=185, batch=2, max_len=600, block_x=128, num_heads_q=4, num_heads_kv=4, top_k=5,
         mask_mode=1, tnd=True),
]


@pytest.mark.parametrize("case", DMA8_CASES, ids=[str(c["seed"]) for c in DMA8_CASES])
def test_fp8_dma_key_split_all_rows(case):
    kw = dict(case)
    seed, tnd = kw.pop("seed"), kw.pop("tnd", False)
    p = gi.random_problem(seed, device="cuda", dtype="fp8", **kw)
    if tnd:
        p = gi.to_tnd(p, keep_seqused_kv=True, tail_rows=0)
    rows = p.block_x * p.num_heads_q // p.num_heads_kv
    assert 64 < rows <= 256
    for P in (0, 3, 200):
        _full_check(p, num_workers=P, label=f"dma8 {seed} rows={rows} P={P}")


@pytest.mark.parametrize("seed", range(200, 232))
def test_random_sweep(seed):
    """Random combinations of every option (see gbsa_inputs.sweep_problem) on every kernel,
    at the library's worker count and at a small random one (forcing split-KV merges)."""
    p = gi.sweep_problem(seed, device="cuda")
    P = int(np.random.default_rng(seed).integers(1, 40))
    for workers in (0, P):
        _full_check(p, num_workers=workers, label=f"sweep{seed} P={workers}")


def test_empty_selections_and_inactive_sequences():
    p = gi.random_problem(120, device="cuda", batch=4, use_seqused_q=True, mask_mode=1)
    cnt = p.sparse_block_count.copy()
    cnt[:, ::2] = 0
    squ = p.seqused_q.copy()
    squ[1] = 0  # a sequence with no active rows
    p = dataclasses.replace(p, sparse_block_count=cnt, seqused_q=squ)
    for P in (0, 7):
        _full_check(p, num_workers=P, label=f"empty P={P}")


def test_rows_beyond_seqused_are_not_written():
    p = gi.random_problem(121, device="cuda", batch=3, use_seqused_q=True, mask_mode=1)
    gp = GpuProblem(p)
    params = gpu_params(p, 9)
    meta = gp.metadata(params)
    out = torch.full(p.q.shape, 7.0, dtype=gi.TORCH_DTYPES[p.out_dtype], device="cuda")
    lse = torch.full(p.q.shape[:2], 7.0, dtype=torch.float32, device="cuda")
    gp.forward(params, meta, out, lse)
    torch.cuda.synchronize()
    o, l = out_f64(out), lse.cpu().numpy()
    for b in range(p.batch):
        c0, c1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        sq = int(p.seqused_q[b])
        assert np.all(o[c0 + sq:c1] == 7.0) and np.all(l[c0 + sq:c1] == 7.0)
        assert not np.any(o[c0:c0 + sq] == 7.0)


def test_deterministic_and_page_shuffle_invariant():
    p = gi.random_problem(122, device="cuda", batch=3, mask_mode=1, extra_pages=6)
    _, _, o1, l1, _ = GpuProblem(p).run(11)
    _, _, o2, l2, _ = GpuProblem(p).run(11)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rng = np.random.default_rng(3)
    perm = rng.permutation(p.num_pages)
    inv = torch.as_tensor(np.argsort(perm), device="cuda")
    table2 = np.where(p.block_table >= 0, perm[np.maximum(p.block_table, 0)], -1).astype(np.int32)
    p2 = dataclasses.replace(p, k=p.k[inv].contiguous(), v=p.v[inv].contiguous(),
                             block_table=table2)
    _, _, o3, l3, _ = GpuProblem(p2).run(11)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


# ---------------------------------------------------------------------------
# token-major (TND) key/value, and rows past the visible KV length
# ---------------------------------------------------------------------------

# one case per kernel: decode (M <= 16), 16-row waves (M <= 64), key-split (M <= 256) and
# row-split (M > 256) ping-pong; `keep` passes seqused_kv below the storage length (dual
# lengths), else none; tail rows follow the last sequence (0: its last block runs past the
# tensor's end)
TND_CASES = [
    dict(seed=131, dtype="f16", mask_mode=1, use_seqused_q=True, block_x=32, keep=True, tail=0),
    dict(seed=132, dtype="bf16", decode=True, batch=5, block_x=1, num_heads_q=16,
         num_heads_kv=4, mask_mode=1, keep=False, tail=0),
    dict(seed=133, dtype="fp8", batch=2, max_len=500, block_x=96, num_heads_q=4,
         num_heads_kv=4, top_k=4, mask_mode=1, out_dtype="f16", keep=True, tail=0),
    dict(seed=134, dtype="f16", batch=2, max_len=500, block_x=40, num_heads_q=16,
         num_heads_kv=2, top_k=6, mask_mode=1, win_left=100, win_right=0, use_seqused_q=True,
         keep=True, tail=0),
    dict(seed=135, dtype="bf16", batch=3, max_len=400, block_x=64, num_heads_q=4,
         num_heads_kv=2, top_k=5, mask_mode=0, keep=False, tail=64),
    dict(seed=136, dtype="fp8", decode=True, batch=4, block_x=2, num_heads_q=8,
         num_heads_kv=2, top_k=5, keep=True, tail=0),
    dict(seed=137, dtype="bf16", batch=1, max_len=700, block_x=128, num_heads_q=8,
         num_heads_kv=1, top_k=6, mask_mode=1, keep=True, tail=0),
]


@pytest.mark.parametrize("case", TND_CASES, ids=[str(c["seed"]) for c in TND_CASES])
def test_tnd_layout_all_rows(case):
    kw = dict(case)
    seed, keep, tail = kw.pop("seed"), kw.pop("keep"), kw.pop("tail")
    p = gi.to_tnd(gi.random_problem(seed, device="cuda", **kw), keep_seqused_kv=keep,
                  tail_rows=tail)
    assert p.num_pages == p.k.shape[0]
    for P in (0, 5, 200):
        _full_check(p, num_workers=P, label=f"tnd{seed} P={P}")


def test_tnd_matches_paged_bit_exact():
    """The kernels see the same bytes in the same order in either layout."""
    p = gi.random_problem(138, device="cuda", batch=3, mask_mode=1, use_seqused_q=True)
    res = []
    for prob in (p, gi.to_tnd(p)):
        # rows past seqused_q are not written: start both outputs from the same bytes
        out = torch.zeros(p.q.shape, dtype=gi.TORCH_DTYPES[p.out_dtype], device="cuda")
        lse = torch.zeros(p.q.shape[:2], dtype=torch.float32, device="cuda")
        res.append(GpuProblem(prob).run(9, out=out, lse=lse)[2:4])
    (o1, l1), (o2, l2) = res
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


POISON_CASES = [
    dict(seed=141, dtype="bf16", decode=True, batch=4, block_x=1, num_heads_q=8, num_heads_kv=2),
    dict(seed=142, dtype="f16", block_x=32, mask_mode=0),
    dict(seed=143, dtype="fp8", batch=2, max_len=400, block_x=100, num_heads_q=2,
         num_heads_kv=2, mask_mode=0),
    dict(seed=144, dtype="f16", batch=2, max_len=400, block_x=40, num_heads_q=8,
         num_heads_kv=1, mask_mode=0),
]


def _poison(t, dtype, rows_of):
    """NaN (fp8: its NaN byte) into the given KV positions of every head."""
    if dtype == "fp8":
        u = t.view(torch.uint8)
        for idx in rows_of:
            u[idx] = 0x7F
    else:
        for idx in rows_of:
            t[idx] = float("nan")


@pytest.mark.parametrize("layout", ["PA_BBND", "TND"])
@pytest.mark.parametrize("case", POISON_CASES, ids=[str(c["seed"]) for c in POISON_CASES])
def test_keys_past_visible_length_never_reach_the_output(case, layout):
    """NaN in every cached key/value row past seqused_kv (the page tails, or the TND storage
    rows past seqused_kv) leaves the output equal to the oracle's, which never reads them."""
    kw = dict(case)
    seed = kw.pop("seed")
    p = gi.random_problem(seed, device="cuda", mask_mode=kw.pop("mask_mode", 1), **kw)
    if layout == "TND":
        p = gi.to_tnd(p)
        k, v = p.k.clone(), p.v.clone()
        idx = []
        for b in range(p.batch):
            r0, r1 = int(p.cu_seqlens_kv[b]) + p.kv_len(b), int(p.cu_seqlens_kv[b + 1])
            if r1 > r0:
                idx.append(slice(r0, r1))
    else:
        k, v = p.k.clone(), p.v.clone()
        idx = []
        for b in range(p.batch):
            skv = int(p.seqused_kv[b])
            for j in range(skv // 128, (int(p.kv_storage[b]) + 127) // 128):
                page = int(p.block_table[b, j])
                idx.append((page, slice(max(skv - 128 * j, 0), 128)))
    assert idx, "the case has no rows past the visible length"
    _poison(k, p.dtype, idx)
    _poison(v, p.dtype, idx)
    pp = dataclasses.replace(p, k=k, v=v)
    for P in (0, 7):
        _full_check(pp, num_workers=P, label=f"poison{seed} {layout} P={P}")


# ---------------------------------------------------------------------------
# running max that jumps: the softmax item's exact path (block max taken, O rescaled)
# ---------------------------------------------------------------------------

# one case per kernel with the 32-row softmax item: 256-row DMA (bf16, f16, with a user mask),
# 16-bit key-split, fp8 DMA key-split and fp8 register-staged 256-row
JUMP_CASES = [
    dict(seed=181, dtype="bf16", block_x=64, num_heads_q=16, num_heads_kv=2),
    dict(seed=182, dtype="f16", block_x=64, num_heads_q=16, num_heads_kv=2, mask_mode=0),
    dict(seed=183, dtype="bf16", block_x=64, num_heads_q=16, num_heads_kv=2, umask=True),
    dict(seed=184, dtype="bf16", block_x=32, num_heads_q=8, num_heads_kv=2),
    dict(seed=185, dtype="fp8", block_x=32, num_heads_q=8, num_heads_kv=2),
    dict(seed=186, dtype="fp8", block_x=64, num_heads_q=16, num_heads_kv=2, out_dtype="f16"),
]


def _jumping_logits(p):
    """The same problem with logits that grow along each sequence: K of logical block j scaled
    by (1 + j) and Q by 3 (fp8: K of block j re-quantised at (1 + j) / blocks, and the Q
    dequant scales times 12, so that no byte leaves the e4m3 range), so that block maxima rise
    by several log2 units from one selected block to the next and most softmax items leave the
    lazy bound of the running max (the oracle reads the rescaled values). P is then close to
    one-hot and O close to single rows of V, so V is scaled by 1/4 (exactly; fp8 through its
    dequant scales): with |O| up to 4.5 one rounding of a bf16 output alone costs up to 2^-6,
    the whole bf16 bar, while below 2 it costs at most 2^-8 and the bar measures the kernel."""
    k = p.k.clone()
    seen = set()
    for b in range(p.batch):
        for j, phys in enumerate(p.block_table[b]):
            if phys < 0 or int(phys) in seen:
                continue
            seen.add(int(phys))
            f = float(1 + j) if p.dtype != "fp8" else float(1 + j) / float(len(p.block_table[b]))
            k[int(phys)] = (k[int(phys)].float() * f).to(k.dtype)
    if p.dtype == "fp8":
        return dataclasses.replace(p, k=k, q_scale=(p.q_scale * 12.0).astype(np.float32),
                                   v_scale=(p.v_scale * 0.25).astype(np.float32),
                                   name=p.name + "_jump")
    q = (p.q.float() * 3.0).to(p.q.dtype)
    v = (p.v.float() * 0.25).to(p.v.dtype)
    return dataclasses.replace(p, q=q, k=k, v=v, name=p.name + "_jump")


@pytest.mark.parametrize("case", JUMP_CASES, ids=[str(c["seed"]) for c in JUMP_CASES])
def test_running_max_jumps(case):
    kw = dict(case)
    seed, umask = kw.pop("seed"), kw.pop("umask", False)
    kw.setdefault("mask_mode", 1)
    p = _jumping_logits(gi.random_problem(seed, device="cuda", batch=2, max_len=700, top_k=6,
                                          **kw))
    if umask:
        p = gi.with_atten_mask(p, seed, density=0.2)
    for P in (0, 7):
        _full_check(p, num_workers=P, label=f"jump{seed} P={P}")


# ---------------------------------------------------------------------------
# user attention masks and the top-left causal mask
# ---------------------------------------------------------------------------

# one case per kernel (decode, 16-row waves, key-split, row-split), both layouts, shared and
# per-sequence masks, masks covering only part of the rows / keys, mask modes 0, 1 and 2
UMASK_CASES = [
    dict(seed=151, prob=dict(dtype="bf16", decode=True, batch=5, block_x=1, num_heads_q=16,
                             num_heads_kv=4, mask_mode=1),
         mask=dict(density=0.3, per_batch=True), tnd=False),
    dict(seed=152, prob=dict(dtype="f16", block_x=32, mask_mode=2, use_seqused_q=True),
         mask=dict(density=0.5, per_batch=False), tnd=True),
    dict(seed=153, prob=dict(dtype="fp8", batch=2, max_len=500, block_x=96, num_heads_q=4,
                             num_heads_kv=4, top_k=4, mask_mode=0, out_dtype="f16"),
         mask=dict(density=0.2, per_batch=True, rows=300, cols=333), tnd=False),
    dict(seed=154, prob=dict(dtype="f16", batch=2, max_len=500, block_x=40, num_heads_q=16,
                             num_heads_kv=2, top_k=6, mask_mode=1, win_left=100, win_right=0,
                             use_seqused_q=True),
         mask=dict(density=0.4, per_batch=True), tnd=True),
    dict(seed=155, prob=dict(dtype="bf16", batch=1, max_len=700, block_x=128, num_heads_q=8,
                             num_heads_kv=1, top_k=6, mask_mode=2),
         mask=dict(density=0.7, per_batch=False, cols=257), tnd=False),
    dict(seed=156, prob=dict(dtype="fp8", decode=True, batch=4, block_x=2, num_heads_q=8,
                             num_heads_kv=2, top_k=5, mask_mode=0),
         mask=dict(density=0.5, per_batch=True, rows=1), tnd=True),
]


@pytest.mark.parametrize("case", UMASK_CASES, ids=[str(c["seed"]) for c in UMASK_CASES])
def test_user_mask_all_rows(case):
    p = gi.random_problem(case["seed"], device="cuda", **case["prob"])
    if case["tnd"]:
        p = gi.to_tnd(p)
    p = gi.with_atten_mask(p, case["seed"], **case["mask"])
    for P in (0, 7):
        _full_check(p, num_workers=P, label=f"umask{case['seed']} P={P}")


@pytest.mark.parametrize("kw", [
    dict(dtype="bf16", decode=True, batch=4, block_x=1, num_heads_q=8, num_heads_kv=2),
    dict(dtype="f16", block_x=32, use_seqused_q=True),
    dict(dtype="bf16", batch=2, max_len=400, block_x=64, num_heads_q=4, num_heads_kv=2),
    dict(dtype="f16", batch=2, max_len=500, block_x=40, num_heads_q=16, num_heads_kv=2,
         win_left=60, win_right=0),
], ids=["decode", "rows64", "rows128", "rows320"])
def test_top_left_causal_all_rows(kw):
    p = gi.random_problem(157, device="cuda", mask_mode=2, **kw)
    for P in (0, 5):
        _full_check(p, num_workers=P, label=f"topleft P={P}")


def test_keyword_interface_bool_mask():
    """The article-style keyword call with a bool mask whose rows are not 4-byte multiples."""
    from block_sparse_paged_gbsa_amd import (generic_block_sparse_attention,
                                             generic_block_sparse_attention_metadata)
    p = gi.random_problem(158, device="cuda", dtype="f16", batch=2, mask_mode=1)
    cols = max(p.kv_len(b) for b in range(p.batch)) | 1  # odd: needs padding
    rows = int(np.diff(p.cu_seqlens_q).max())
    rng = np.random.default_rng(5)
    m = rng.random((rows, cols)) < 0.3
    pm = dataclasses.replace(p, atten_mask=np.where(m, 1, 0).astype(np.uint8)[None],
                             atten_mask_cols=cols)
    gp = GpuProblem(pm)
    meta = generic_block_sparse_attention_metadata(
        gp.idx, gp.cnt, p.num_heads_q, p.num_heads_kv, 128, [p.block_x, 128],
        cu_seqlens_q=gp.cu, seqused_kv=gp.skv, mask_mode=1, num_workers=6)
    out, lse = generic_block_sparse_attention(
        p.q, p.k, p.v, gp.idx, gp.cnt, [p.block_x, 128], metadata=meta,
        attn_mask=torch.as_tensor(m, device="cuda"), cu_seqlens_q=gp.cu, seqused_kv=gp.skv,
        block_table=gp.table, softmax_scale=p.scale, mask_mode=1, return_softmax_lse=True,
        num_workers=6)
    torch.cuda.synchronize()
    O, L, done = oa.sparse_attention(oracle_inputs(pm))
    compare(pm, out, lse[..., 0], O, L, done, "keyword bool mask")


@pytest.mark.parametrize("kw", [dict(decode=True, batch=4, block_x=1, num_heads_q=8,
                                     num_heads_kv=2),
                                dict(batch=2, max_len=500, block_x=40, num_heads_q=16,
                                     num_heads_kv=2, top_k=6)], ids=["decode", "prefill"])
def test_workspace_reuse(kw):
    """Split-KV units leave their arrival counters at zero: a workspace reused by several calls
    (same worker count) gives bit-identical results to a fresh one every time."""
    p = gi.random_problem(181, device="cuda", mask_mode=1, **kw)
    gp = GpuProblem(p)
    params = gpu_params(p, 7)  # few workers: most units are split
    meta = gp.metadata(params)
    ref, lref, _ = gp.forward(params, meta)
    ws = None
    for i in range(3):
        out, lse, ws = gp.forward(params, meta, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32)[0].item()) == 0
        assert torch.equal(out, ref) and torch.equal(lse, lref), f"call {i}"


def _validate(p, max_seqlen=(-1, -1), **over):
    from block_sparse_paged_gbsa_amd import gbsa_validate
    gp = GpuProblem(p)
    t = dict(cnt=gp.cnt, idx=gp.idx, cu=gp.cu, squ=gp.squ, skv=gp.skv, table=gp.table,
             cu_kv=gp.cu_kv, umask=gp.umask)
    t.update(over)
    params = gpu_params(p)
    params.max_seqlen_q, params.max_seqlen_kv = max_seqlen
    return gbsa_validate(params, t["idx"], t["cnt"], t["cu"], t["squ"],
                         cu_seqlens_kv=t["cu_kv"], seqused_kv=t["skv"], block_table=t["table"],
                         atten_mask=t["umask"])


def test_validate_reports_each_broken_rule():
    """The opt-in value check is silent on valid inputs and names each planted violation."""
    from block_sparse_paged_gbsa_amd._lib import VALIDATE_BITS
    bit = {v: k for k, v in VALIDATE_BITS.items()}
    p = gi.random_problem(191, device="cuda", batch=3, mask_mode=1, use_seqused_q=True)
    assert _validate(p) == 0
    gp = GpuProblem(p)
    dev = lambda a: torch.as_tensor(np.ascontiguousarray(a)).to("cuda")
    cu = p.cu_seqlens_q.copy(); cu[1] = cu[2] + 1  # decreasing
    assert _validate(p, cu=dev(cu)) & bit["cu_seqlens_q"]
    squ = p.seqused_q.copy(); squ[0] = np.diff(p.cu_seqlens_q)[0] + 1
    assert _validate(p, squ=dev(squ)) == bit["seqused_q"]
    skv = p.seqused_kv.copy(); skv[2] = p.block_table.shape[1] * 128 + 1
    assert _validate(p, skv=dev(skv)) & bit["kv_length"]
    tab = p.block_table.copy(); tab[1, 0] = p.num_pages
    assert _validate(p, table=dev(tab)) == bit["block_table"]
    cnt = p.sparse_block_count.copy(); cnt[0, 0] = p.top_k + 1
    assert _validate(p, cnt=dev(cnt)) == bit["count"]
    idx = p.sparse_block_idx.copy(); c0 = int(p.sparse_block_count[0, 0])
    assert c0 > 0
    idx[0, 0, 0] = 10_000
    assert _validate(p, idx=dev(idx)) == bit["selection"]
    # token-major key/value: cu_seqlens_kv past the tensor
    t = gi.to_tnd(p)
    assert _validate(t) == 0
    cukv = t.cu_seqlens_kv.copy(); cukv[-1] = t.num_pages + 5
    assert _validate(t, cu_kv=dev(cukv)) & bit["cu_seqlens_kv"]
    # a user mask that covers too few keys
    m = gi.with_atten_mask(p, 191, cols=10)
    assert _validate(m) == bit["mask_extent"]
    assert _validate(gi.with_atten_mask(p, 191)) == 0
    # length bounds: exact bounds pass, one below the longest sequence is reported
    lq = int(np.diff(p.cu_seqlens_q).max())
    lkv = int(max(p.kv_len(b) for b in range(p.batch)))
    assert _validate(p, max_seqlen=(lq, lkv)) == 0
    assert _validate(p, max_seqlen=(lq - 1, lkv)) == bit["max_seqlen"]
    assert _validate(p, max_seqlen=(lq, lkv - 1)) == bit["max_seqlen"]


def test_metadata_mismatch_is_refused():
    p = gi.random_problem(123, device="cuda", mask_mode=1)
    gp = GpuProblem(p)
    good = gpu_params(p, 8)
    other = gpu_params(p, 8)
    other.mask_mode = 0  # metadata built for different attributes
    meta = gp.metadata(other)
    out = torch.full(p.q.shape, 3.0, dtype=gi.TORCH_DTYPES[p.out_dtype], device="cuda")
    lse = torch.zeros(p.q.shape[:2], dtype=torch.float32, device="cuda") if p.return_lse else None
    _, _, ws = gp.forward(good, meta, out, lse)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32)[0].item()) != 0
    # nothing computed: every output entry is NaN, whatever the buffer held
    assert torch.isnan(out.float()).all()
    if lse is not None:
        assert torch.isnan(lse).all()


def test_metadata_mismatch_keyword_path_gives_nan():
    """The article-style keyword call returns no workspace, so a refused call must show in its
    outputs: metadata built for causal attention, main call without a mask."""
    from block_sparse_paged_gbsa_amd import (generic_block_sparse_attention,
                                             generic_block_sparse_attention_metadata)
    p = gi.random_problem(124, device="cuda", mask_mode=1)
    gp = GpuProblem(p)
    bs = [p.block_x, 128]
    meta = generic_block_sparse_attention_metadata(
        gp.idx, gp.cnt, p.num_heads_q, p.num_heads_kv, 128, bs, cu_seqlens_q=gp.cu,
        seqused_q=gp.squ, seqused_kv=gp.skv, mask_mode=1)
    kw = dict(metadata=meta, cu_seqlens_q=gp.cu, seqused_q=gp.squ, seqused_kv=gp.skv,
              block_table=gp.table, softmax_scale=p.scale, return_softmax_lse=True)
    out, lse = generic_block_sparse_attention(p.q, p.k, p.v, gp.idx, gp.cnt, bs, mask_mode=1,
                                              **kw)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any()
    out, lse = generic_block_sparse_attention(p.q, p.k, p.v, gp.idx, gp.cnt, bs, mask_mode=0,
                                              **kw)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()


# ---------------------------------------------------------------------------
# full-size workloads, sampled rows, benchmark launch configuration
# ---------------------------------------------------------------------------

def _sampled_rows(p, units, rows_per_unit, rng):
    """Global rows of the given (b, q-block) units: every active row, or rows_per_unit of
    them always including the q-block's first and last active rows."""
    rows = []
    for (b, gl) in units:
        storage = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
        sq = storage if p.seqused_q is None else min(int(p.seqused_q[b]), storage)
        lo, hi = gl * p.block_x, min((gl + 1) * p.block_x, sq)
        assert lo < hi, f"q-block {gl} of sequence {b} has no active row"
        ts = np.arange(lo, hi)
        if rows_per_unit is not None and len(ts) > rows_per_unit:
            ts = np.unique(np.concatenate([[lo, hi - 1], rng.choice(ts[1:-1], rows_per_unit - 2,
                                                                    replace=False)]))
        rows += list(int(p.cu_seqlens_q[b]) + ts)
    return rows


def _sampled_check(cfg, units, rows_per_unit=None, seed=0, tnd=False, problem=None,
                   p_scale=None, o_tol=None):
    """A full-size workload in the benchmark's launch configuration, checked against the
    oracle on the rows of the given q-blocks (all KV heads, so every query head), plus an
    all-finite check of every active row. Records the error margins."""
    label = f"workload{cfg}{'_tnd' if tnd else ''}" if problem is None else problem.name
    if p_scale is not None:
        label += "_p8"
    _log(f"[parity] {label}: generating on the GPU")
    p = gi.config(cfg, device="cuda") if problem is None else problem
    if tnd:
        p = gi.to_tnd(p)
    gp = GpuProblem(p)
    if p_scale is not None:
        gp.ps = torch.full((p.num_heads_q,), p_scale, dtype=torch.float32, device="cuda")
    params, meta, out, lse, ws = gp.run(0)
    words = ws[:256].view(torch.int32).cpu()
    assert int(words[0]) == 0
    # the prefill task queue counters (status page words 16..48) are back at zero
    assert not bool(words[16:49].any()), f"{label}: task counters left at {words[16:49]}"
    # every active row finite (checked on the device, rows past seqused_q are never written)
    for b in range(p.batch):
        c0 = int(p.cu_seqlens_q[b])
        storage = int(p.cu_seqlens_q[b + 1]) - c0
        sq = storage if p.seqused_q is None else min(int(p.seqused_q[b]), storage)
        assert bool(torch.isfinite(out[c0:c0 + sq].float()).all()), f"{label}: sequence {b}"
    _log(f"[parity] {label}: gpu done, oracle on {len(units)} q-blocks")
    inp = compact_oracle_inputs(p, units)
    rows = _sampled_rows(p, units, rows_per_unit, np.random.default_rng(seed))
    idx, O, L = oracle_rows(inp, rows, p.block_x, p.cu_seqlens_q)
    assert len(idx) == len(set(rows)), "a sampled row is not active"
    err, lerr = compare_rows(p, out, lse if p.return_lse else None, idx, O, L, label,
                             o_tol=o_tol)
    _log(f"[parity] {label}: {len(idx)} rows x {p.num_heads_q} heads, O max-abs "
         f"{err:.3e} (bar {TOL[p.dtype]:.1e}), LSE rel {lerr:.3e}")
    record_margin(label, rows=len(idx), heads=p.num_heads_q, q_blocks=len(units),
                  o_max_abs=err, o_bar=TOL[p.dtype], lse_rel=lerr if p.return_lse else None)
    return p, out, err


def _qblocks(n_active, extra=()):
    """First, second, middle, second-to-last and last q-block, plus the given ones."""
    return sorted({0, 1, n_active // 2, n_active - 2, n_active - 1, *extra})


def test_workload2_decode_sampled():
    _sampled_check(2, [(b, 0) for b in range(64)])


@pytest.mark.parametrize("batch,top_k", [(8, 16), (1, 256)], ids=["b8_top16", "b1_top256"])
def test_split_kv_decode_sampled(batch, top_k):
    """The split-KV decode shapes the benchmark times (`--batch`, `--top-k`): every unit cut
    over several of the default workers and merged in the kernel; all queries checked."""
    p = gi.decode_workload(batch, top_k, device="cuda")
    _sampled_check(2, [(b, 0) for b in range(batch)], problem=p)


def test_workload3_block_sparse_prefill_sampled():
    """Every sequence: first, middle and last q-blocks, and both sides of q-block 64 where
    the selection stops being every causal block (sink + 8 recent + random after it)."""
    units = [(b, gl) for b in range(4) for gl in _qblocks(256, (63, 64, 65))]
    _sampled_check(3, units, rows_per_unit=32)


@pytest.mark.parametrize("block_x", [8, 4], ids=["x8", "x4"])
def test_small_qblock_prefill_sampled(block_x):
    """Workload 3 with 8- and 4-row q-blocks (`--block-x`), as the benchmark times them: 64 and
    32 packed rows per unit, the in-phase kernel with every page's keys in two or four slices.
    First q-blocks, both sides of a 128-token block edge, and q-blocks in later sequences up to
    the last one; every row of each."""
    n = 32768 // block_x
    e = 128 // block_x
    units = [(0, 0), (0, 1), (0, e - 1), (0, e), (1, n // 4), (2, n // 2 + 1), (3, n - 1)]
    _sampled_check(3, units, problem=gi.block_sparse_prefill(block_x, device="cuda"))


def test_workload4_long_context_sampled():
    """First q-blocks (the sinks are the whole selection), both sides of the window edge
    (from row 32256 the sink blocks leave the window while still selected), a middle
    q-block, the q-blocks whose diagonal is the partial last KV block (seqused_kv = 120000,
    block 937 holds 64 keys) and the last active q-block (rows 119936..119999)."""
    units = [(0, gl) for gl in (0, 1, 2, 3, 503, 504, 505, 937, 1872, 1873, 1874)]
    _sampled_check(4, units, rows_per_unit=32)


def test_workload5_dense_equivalent_fp8_sampled():
    """Both sequences: first, middle and last q-blocks and a few in between (every causal
    block selected: the result must be dense causal attention)."""
    units = [(b, gl) for b in range(2) for gl in _qblocks(256, (100, 128))]
    _sampled_check(5, units, rows_per_unit=32)


def test_unit_tasks_repeat_bit_identical():
    """The fp8 dense-equivalent workload runs as whole units taken from the per-XCD task
    queues (its units outnumber the resident workgroups many times over). Which workgroup
    takes which unit changes from call to call; the result must not: three more calls on the
    same workspace give the same bytes, and leave the queue counters at zero."""
    p = gi.config(5, device="cuda")
    gp = GpuProblem(p)
    params, meta, ref, _, ws = gp.run(0)
    for i in range(3):
        out, _, ws = gp.forward(params, meta, workspace=ws)
        torch.cuda.synchronize()
        words = ws[:256].view(torch.int32).cpu()
        assert int(words[0]) == 0 and not bool(words[16:49].any()), f"call {i}"
        assert torch.equal(out, ref), f"call {i}"


# Softmax precision 1 (GBSA article, "softmax precision": online softmax in the output's 16-bit
# type, rescale in fp32; it may overflow). With f16 the two ping-pong kernels compute it in f16;
# bf16 and fp8 keep fp32 there. Bars: the logits rounded to f16 (relative 2^-11) and the f16
# scaling, subtraction and exponential (2^-11 each, the exponential's approximation within one
# ulp) give each exponential a relative error of at most eps = ln2 * 2^-11 * (2|t| + |x|) +
# 3 * 2^-11 (t the logit in log2 units, x = t - m); the weighted mean of those errors moves LSE
# by at most eps and O by at most 2 eps max|v|. For these inputs (unit-variance Q/K/V, D = 128)
# the logits stay within |t| <= 8 and the weight of keys with x < -16 is negligible, so
# eps <= 0.013: LSE within 1e-3 |LSE| + 1.3e-2, O within the bf16 bar of a 16-bit softmax
# stage, 1.6e-2 (the margins recorded show how far inside they stay).
HALF_SM_CASES = [
    dict(seed=161, num_heads_q=16, num_heads_kv=2, block_x=16, top_k=6, mask_mode=1,
         max_len=600),
    dict(seed=162, num_heads_q=32, num_heads_kv=4, block_x=64, top_k=5, mask_mode=1,
         max_len=900, use_seqused_q=True),
    dict(seed=163, num_heads_q=64, num_heads_kv=2, block_x=16, top_k=4, mask_mode=0,
         win_left=200, win_right=50, max_len=700),
    dict(seed=116, num_heads_q=16, num_heads_kv=2, block_x=32, top_k=6, mask_mode=1,
         max_len=500),
]


@pytest.mark.parametrize("case", HALF_SM_CASES, ids=[str(c["seed"]) for c in HALF_SM_CASES])
def test_half_precision_softmax_f16(case):
    """Both ping-pong kernels (128 and 512 packed rows per unit) in softmax precision 1, every
    row against the oracle; the same problem in precision 0 for comparison."""
    kw = {k: v for k, v in case.items() if k != "seed"}
    p = gi.random_problem(case["seed"], device="cuda", dtype="f16", return_lse=True, **kw)
    gp = GpuProblem(p)
    O, L, done = oa.sparse_attention(oracle_inputs(p))
    errs = {}
    for mode in (1, 0):
        params = gpu_params(p)
        params.softmax_precision = mode
        meta = gp.metadata(params)
        out, lse, ws = gp.forward(params, meta)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32)[0].item()) == 0
        label = f"half_softmax_{case['seed']}_mode{mode}"
        bars = dict(o_tol=1.6e-2, lse_atol=1.3e-2) if mode == 1 else {}
        errs[mode] = compare(p, out, lse, O, L, done, label, **bars)
        record_margin(label, rows=int(done.sum()), heads=p.num_heads_q, o_max_abs=errs[mode][0],
                      o_bar=bars.get("o_tol", TOL["f16"]), lse_rel=errs[mode][1])
    _log(f"[parity] half softmax {case['seed']}: O {errs[1][0]:.2e} (fp32 {errs[0][0]:.2e}), "
         f"LSE rel {errs[1][1]:.2e} (fp32 {errs[0][1]:.2e})")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_half_precision_softmax_other_dtypes_compute_fp32(dtype):
    """Softmax precision 1 with bf16 or fp8 is computed in fp32 (the mode permits the lower
    precision; only the f16 kernels use it): bit-identical to precision 0."""
    p = gi.random_problem(164, device="cuda", dtype=dtype, num_heads_q=16, num_heads_kv=2,
                          block_x=32, top_k=5, mask_mode=1, max_len=500, return_lse=True)
    gp = GpuProblem(p)
    res = []
    for mode in (0, 1):
        params = gpu_params(p)
        params.softmax_precision = mode
        out, lse, _ = gp.forward(params, gp.metadata(params))
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


# Quant mode 5 with p_quant_scale (GBSA article, "quantisation": FP8_E4M3_STATIC_CAST_P): P is
# cast to e4m3 after scaling and P·V runs on fp8 MFMA in the 65-256-row and 256-row fp8
# kernels. The oracle never quantises P (the definition is the same attention), so the result is
# held to the fp8 bar, 6e-2; LSE uses the unquantised row sums and keeps its bar.
P8_CASES = [
    dict(seed=171, num_heads_q=16, num_heads_kv=2, block_x=16, top_k=6, mask_mode=1,
         max_len=600, scale=448.0),
    dict(seed=172, num_heads_q=32, num_heads_kv=4, block_x=64, top_k=5, mask_mode=1,
         max_len=900, use_seqused_q=True, scale=448.0),
    dict(seed=173, num_heads_q=8, num_heads_kv=1, block_x=32, top_k=8, mask_mode=0,
         win_left=150, win_right=20, max_len=700, scale=None),  # per-head scales (below)
    dict(seed=174, num_heads_q=16, num_heads_kv=4, block_x=128, top_k=4, mask_mode=1,
         max_len=500, scale=1000.0, dst_type_max=240.0),  # the scale clamped to 240
]


@pytest.mark.parametrize("case", P8_CASES, ids=[str(c["seed"]) for c in P8_CASES])
def test_fp8_p_quantised_pv(case):
    """fp8 P·V (both fp8 ping-pong kernels), every row against the oracle, at one and at three
    worker counts' splits; without p_quant_scale the same problem keeps P in bf16."""
    kw = {k: v for k, v in case.items() if k not in ("seed", "scale", "dst_type_max")}
    p = gi.random_problem(case["seed"], device="cuda", dtype="fp8", return_lse=True, **kw)
    gp = GpuProblem(p)
    O, L, done = oa.sparse_attention(oracle_inputs(p))
    scale = case["scale"]
    # per-head scales that e4m3 holds exactly, so that each row's largest weight (P = 1) is cast
    # without error (a scale such as 100 puts a 4 % error on it, and the O error of that case
    # doubles: a property of the cast, reproduced by a CPU emulation of it)
    per_head = [448.0, 256.0, 224.0, 192.0, 160.0, 128.0, 112.0, 96.0]
    gp.ps = (torch.full((p.num_heads_q,), scale, dtype=torch.float32, device="cuda")
             if scale is not None else
             torch.tensor([per_head[h % 8] for h in range(p.num_heads_q)], dtype=torch.float32,
                          device="cuda"))
    for workers in (0, 5):
        params = gpu_params(p, workers)
        params.dst_type_max = case.get("dst_type_max", 0.0)
        meta = gp.metadata(params)
        out, lse, ws = gp.forward(params, meta)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32)[0].item()) == 0
        label = f"fp8_p_{case['seed']}_w{workers}"
        err, lerr = compare(p, out, lse, O, L, done, label)
        record_margin(label, rows=int(done.sum()), heads=p.num_heads_q, o_max_abs=err,
                      o_bar=TOL["fp8"], lse_rel=lerr)
    gp.ps = None
    params = gpu_params(p)
    out16, _, _ = gp.forward(params, gp.metadata(params))
    err16, _ = compare(p, out16, None, O, L, done, f"fp8_p_{case['seed']}_bf16P")
    _log(f"[parity] fp8 P {case['seed']}: O {err:.2e} (bf16 P {err16:.2e}), LSE rel {lerr:.2e}")


def test_fp8_p_scale_ignored_where_p_stays_bf16():
    """The decode and 17-64-row kernels keep P in bf16: p_quant_scale leaves their output bit
    for bit as without it."""
    for kw in (dict(decode=True, batch=4, block_x=1, num_heads_q=8, num_heads_kv=2),
               dict(batch=2, max_len=400, block_x=8, num_heads_q=8, num_heads_kv=2)):
        p = gi.random_problem(175, device="cuda", dtype="fp8", top_k=5, mask_mode=1, **kw)
        gp = GpuProblem(p)
        params = gpu_params(p)
        meta = gp.metadata(params)
        ref, _, _ = gp.forward(params, meta)
        gp.ps = torch.full((p.num_heads_q,), 448.0, dtype=torch.float32, device="cuda")
        out, _, _ = gp.forward(params, meta)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), kw


@pytest.mark.xfail(strict=True, reason="casting P to e4m3 (3 mantissa bits: up to 6 % per weight) "
                   "puts workload 5's largest O error at 0.066, over the 6e-2 fp8 bar; the "
                   "default keeps P in bf16 (0.009)")
def test_workload5_fp8_p_quantised_sampled():
    """Workload 5 with p_quant_scale 448 for every head: P cast to e4m3 and P·V on fp8 MFMA,
    in the benchmark's launch configuration; the same q-blocks as the bf16-P check. The error
    is measured and recorded first, then held to the fp8 bar (which it misses: expected)."""
    units = [(b, gl) for b in range(2) for gl in _qblocks(256, (100, 128))]
    _, _, err = _sampled_check(5, units, rows_per_unit=32, p_scale=448.0, o_tol=float("inf"))
    assert err <= TOL["fp8"], f"fp8 P: O max-abs {err}"


def test_workload2_decode_tnd_sampled():
    _sampled_check(2, [(b, 0) for b in range(64)], tnd=True)


def test_workload3_block_sparse_prefill_tnd_sampled():
    units = [(b, gl) for b in range(4) for gl in (0, 64, 255)]
    _sampled_check(3, units, rows_per_unit=32, tnd=True)


def test_workload5_dense_equivalent_fp8_tnd_sampled():
    units = [(b, gl) for b in range(2) for gl in (0, 1, 128, 255)]
    _sampled_check(5, units, rows_per_unit=32, tnd=True)


GRAPH_CASES = [
    dict(decode=True, batch=6, num_heads_q=16, num_heads_kv=4, block_x=1, top_k=8, workers=7),
    dict(batch=2, max_len=300, block_x=64, num_heads_q=8, num_heads_kv=2, top_k=4, workers=5),
]


@pytest.mark.parametrize("case", GRAPH_CASES, ids=["decode_split", "prefill_split"])
def test_graph_capture_replays_match_eager(case):
    """Metadata + forward captured in one HIP graph (no allocation, memset or host sync on the
    path) replay to the eager result, bit for bit, several times with eager work and host
    synchronisations in between; split units reset their arrival counters each time."""
    kw = dict(case)
    P = kw.pop("workers")
    p = gi.random_problem(191, device="cuda", mask_mode=1, **kw)
    gp = GpuProblem(p)
    params = gpu_params(p, P)
    meta = gp.metadata(params)
    ref, lref, ws = gp.forward(params, meta)
    torch.cuda.synchronize()
    out, lse = torch.empty_like(ref), torch.empty_like(lref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        gp.metadata(params, meta)
        gp.forward(params, meta, out, lse, ws)  # warm-up on the capture stream
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            gp.metadata(params, meta)
            gp.forward(params, meta, out, lse, ws)
    torch.cuda.current_stream().wait_stream(side)
    for i in range(4):
        out.fill_(0)
        lse.fill_(0)
        gp.metadata(params, meta)  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32)[0].item()) == 0
        assert torch.equal(out, ref) and torch.equal(lse, lref), f"replay {i}"

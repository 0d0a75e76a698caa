"""The allocation-free forward (gbsa_forward_ex_noalloc) against gbsa_forward_ex: two calls in
a row on the library's fixed device array, the second with a smaller problem, each
bit-identical to the workspace path and within the bars of the oracle."""
import numpy as np
import pytest
import torch

import gbsa_inputs as gi
from helpers import GpuProblem, compare, gpu_params, oracle_inputs
from oracle import attention as oa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc(gp, params, meta, out, lse):
    from block_sparse_paged_gbsa_amd import gbsa_forward_ex_noalloc
    p = gp.p
    return gbsa_forward_ex_noalloc(params, p.q, p.k, p.v, gp.idx, gp.cnt, meta, gp.cu, gp.squ,
                                   cu_seqlens_kv=gp.cu_kv, seqused_kv=gp.skv,
                                   block_table=gp.table, q_scale=gp.qs, k_scale=gp.ks,
                                   v_scale=gp.vs, atten_mask=gp.umask, out=out, lse=lse)


def _check_case(p, workers, label):
    print(f"[no-alloc] {label}: workers={workers}", flush=True)
    gp = GpuProblem(p)
    params = gpu_params(p, workers)
    meta = gp.metadata(params)
    ref, lref, ws = gp.forward(params, meta)  # the workspace path, fresh zeroed workspace
    out = torch.full_like(ref, 5.0)
    lse = torch.full_like(lref, 5.0) if lref is not None else None
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    _noalloc(gp, params, meta, out, lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before, "the call allocated through torch"
    assert int(ws[:4].view(torch.int32)[0].item()) == 0
    # rows past seqused_q are written by neither path: compare the active rows
    rows = np.zeros(p.total_q, dtype=bool)
    for b in range(p.batch):
        c0, c1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        sq = c1 - c0 if p.seqused_q is None else min(int(p.seqused_q[b]), c1 - c0)
        rows[c0:c0 + sq] = True
    r = torch.as_tensor(rows, device="cuda")
    assert torch.equal(out[r], ref[r]), f"{label}: output differs from gbsa_forward_ex"
    if lse is not None:
        assert torch.equal(lse[r], lref[r]), f"{label}: LSE differs from gbsa_forward_ex"
    O, L, done = oa.sparse_attention(oracle_inputs(p))
    err, lerr = compare(p, out, lse, O, L, done, label)
    print(f"[no-alloc] {label}: bit-identical to the workspace path; oracle O max-abs "
          f"{err:.3e}, LSE rel {lerr:.3e}", flush=True)


def test_noalloc_matches_workspace_path_twice():
    """First a prefill problem whose units are split over 9 workers (partials and arrival
    counters in the fixed array), then a smaller decode problem with split units on 5
    workers: the second call must not see anything the first one left behind."""
    big = gi.random_problem(301, device="cuda", batch=3, max_len=300, num_heads_q=8,
                            num_heads_kv=2, block_x=32, top_k=6, mask_mode=1,
                            use_seqused_q=True)
    _check_case(big, 9, "prefill, 9 workers")
    small = gi.random_problem(302, device="cuda", batch=2, decode=True, num_heads_q=8,
                              num_heads_kv=2, block_x=1, top_k=5, mask_mode=0)
    _check_case(small, 5, "decode, 5 workers")


def test_noalloc_refuses_oversized_and_workspace_arguments():
    """Shapes whose partial results exceed the fixed array, and a call that brings a
    workspace, are refused with GBSA_ERR_WORKSPACE before anything is enqueued."""
    from block_sparse_paged_gbsa_amd import GbsaError
    p = gi.random_problem(303, device="cuda", batch=2, max_len=300, num_heads_q=16,
                          num_heads_kv=2, block_x=64, top_k=4, mask_mode=1)
    gp = GpuProblem(p)
    params = gpu_params(p, 999)  # 999 workers x 512 rows per unit: 2 x 999 x 512 x 512 B
    meta = gp.metadata(params)
    out = torch.empty(p.q.shape, dtype=gi.TORCH_DTYPES[p.out_dtype], device="cuda")
    lse = torch.empty(p.q.shape[:2], dtype=torch.float32, device="cuda")
    with pytest.raises(GbsaError) as e:
        _noalloc(gp, params, meta, out, lse)
    assert e.value.code == 6

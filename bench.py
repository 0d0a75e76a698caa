"""Benchmark: block-sparse attention over a paged KV cache on one MI355X.

One step = the whole hot path on one batch: gbsa_metadata (task split) + gbsa_forward
(main kernel and split-KV combine), inputs resident in HBM. The default workload is the
decode-shaped one (64 sequences x 1 query token, 32768-token paged KV each, N1=32, N2=8,
bf16, 16 selected pages per query): bound by HBM bytes, so the headline value is GB/s of
algorithmic traffic. Effective TFLOP/s (selected blocks only) is reported beside it.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "block_sparse_paged_gbsa_amd", "csrc")
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "fp8": 5000.0}
ESIZE = {"f16": 2, "bf16": 2, "fp8": 1}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# HIP sources each main kernel is compiled from (its own file plus the shared headers)
KERNEL_SOURCES = {
    "fwd_decode_kernel": ["fwd_decode.hip"],
    "fwd_prefill_kernel": ["fwd_prefill.hip"],
    "fwd_prefill_pp32_kernel": ["fwd_prefill.hip"],
    "fwd_prefill_pp32d_kernel": ["fwd_prefill.hip"],
    "fwd_prefill_ks32_kernel": ["fwd_prefill.hip"],
    "fwd_prefill_ks32d_kernel": ["fwd_prefill.hip"],
}
SHARED_SOURCES = ["device_common.hpp", "gbsa_internal.hpp", "split_merge.hpp"]


def kernel_source_hash(kernel: str) -> str:
    """sha256 over the sources of one kernel; its counter summary is valid only for them."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES[kernel] + SHARED_SOURCES):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it matches these sources."""
    path = os.path.join(PROFILES, f"{kernel}__{workload}__pmc.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if kernel not in KERNEL_SOURCES or vals.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


TRACE_EVENTS = {1: "softmax start", 2: "softmax end", 3: "softmax barrier in",
                4: "softmax barrier out", 5: "MFMA start", 6: "MFMA end", 7: "MFMA barrier out",
                8: "K stored", 9: "MFMA issued"}
TRACED_KERNELS = ("fwd_prefill_pp32d_kernel", "fwd_prefill_ks32_kernel", "fwd_prefill_ks32d_kernel")


def slot_trace(w, p) -> int:
    """Forward launches on the slot-trace build; per group (waves 0-3 and 4-7), the median
    shader-clock cycles between consecutive events of the traced unit, and the cycles per slot
    pair (one MFMA and one softmax item of every wave)."""
    import ctypes
    import numpy as np
    import torch
    from block_sparse_paged_gbsa_amd import _lib
    if w.kernel not in TRACED_KERNELS:
        print(f"--slot-trace traces {', '.join(TRACED_KERNELS)}; this workload runs {w.kernel}",
              file=sys.stderr)
        return 2
    lib = ctypes.CDLL(_lib.LIB_PATH)
    lib.gbsa_slot_trace_read.argtypes = [ctypes.c_void_p]
    w.step()
    torch.cuda.synchronize()
    out = {"workload": p.name, "kernel": w.kernel, "clock": "s_memtime (shader clock)",
           "launches": []}
    for rep in range(3):
        assert lib.gbsa_slot_trace_reset() == 0
        w.forward()
        torch.cuda.synchronize()
        rec = np.zeros(8 * 1024, dtype=np.uint64)
        assert lib.gbsa_slot_trace_read(rec.ctypes.data) == 0
        rec = rec.reshape(8, 1024)
        code = (rec >> np.uint64(56)).astype(np.int64)
        clk = (rec & np.uint64((1 << 56) - 1)).astype(np.int64)
        launch = {}
        for grp, waves in ((0, range(0, 4)), (1, range(4, 8))):
            pairs, periods = {}, []
            for wv in waves:
                n = int((code[wv] > 0).sum())
                c, t = code[wv, :n], clk[wv, :n]
                for i in range(1, n):
                    key = f"{TRACE_EVENTS[int(c[i - 1])]} -> {TRACE_EVENTS[int(c[i])]}"
                    pairs.setdefault(key, []).append(int(t[i] - t[i - 1]))
                starts = t[c == 5]
                periods += list(np.diff(starts))
            launch[f"group{grp}"] = {k: int(np.median(v)) for k, v in sorted(pairs.items())}
            launch[f"group{grp}"]["slot pair"] = int(np.median(periods)) if periods else None
            launch[f"group{grp}"]["items traced"] = len(periods) // len(waves)
        out["launches"].append(launch)
    assert w.status() == 0, "metadata mismatch flagged by the kernels"
    print(json.dumps(out), flush=True)
    return 0


def copy_calibration(mib: int) -> int:
    """A plain device-to-device copy of a known size (scale reference for FETCH/WRITE_SIZE)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_dispatch": n}), flush=True)
    return 0


def algorithmic_work(p, units=None):
    """(bytes, flops) the method must move / compute, from the selection structure only.

    bytes: K and V rows of every selected block below seqused_kv (once per unit and KV head),
    Q and O rows of active queries, LSE if returned, the used index / count / page-table
    entries. flops: 4 * D per (active query row, head, visible-length key) of selected blocks.
    units: optional set of (b, q-block) to restrict the count to (a sample).
    """
    import gbsa_inputs as gi
    D = 128
    es = ESIZE[p.dtype]
    G = p.num_heads_q // p.num_heads_kv
    starts = gi.q_block_starts(p.cu_seqlens_q, p.block_x)
    kv_bytes = flops = meta_bytes = q_rows = 0
    for b in range(p.batch):
        storage = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
        sq = storage if p.seqused_q is None else min(int(p.seqused_q[b]), storage)
        skv = p.kv_len(b)
        gls = np.arange(-(-sq // p.block_x))
        if units is not None:
            gls = np.array([gl for gl in gls if (b, int(gl)) in units], dtype=np.int64)
        if len(gls) == 0:
            continue
        g = starts[b] + gls
        rows = np.minimum((gls + 1) * p.block_x, sq) - gls * p.block_x
        q_rows += int(rows.sum())
        cnt = np.clip(p.sparse_block_count[:, g], 0, p.top_k)  # [N2, n]
        idx = p.sparse_block_idx[:, g, :]  # [N2, n, topK]
        slot = np.arange(p.top_k)[None, None, :]
        used = slot < cnt[:, :, None]
        j = np.where(used, idx, -1).astype(np.int64)
        valid_tok = np.clip(skv - 128 * j, 0, 128) * (j >= 0)
        tok = (valid_tok * used).sum(axis=2)  # [N2, n]
        kv_bytes += int(tok.sum()) * 2 * D * es
        flops += int((tok * rows[None, :]).sum()) * 4 * D * G
        # indices (+ page-table entries for paged key/value) and counts
        meta_bytes += int(used.sum()) * (4 if p.kv_layout == "TND" else 8) + cnt.size * 4
    out_es = 2
    qo_bytes = q_rows * p.num_heads_q * D * (es + out_es)
    lse_bytes = q_rows * p.num_heads_q * 4 if p.return_lse else 0
    return kv_bytes + qo_bytes + lse_bytes + meta_bytes, flops


def gather_offsets(p):
    """Byte offsets (into key and value) of every selected, visible block's head slice: the
    decode kernel's reads, in task order."""
    import gbsa_inputs as gi
    es = ESIZE[p.dtype]
    starts = gi.q_block_starts(p.cu_seqlens_q, p.block_x)
    unit_bytes = (p.kv_page_stride * es if p.kv_layout != "TND"
                  else p.num_heads_kv * 128 * es)
    offs = []
    for b in range(p.batch):
        storage = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
        sq = storage if p.seqused_q is None else min(int(p.seqused_q[b]), storage)
        skv = p.kv_len(b)
        for gl in range(-(-sq // p.block_x)):
            g = starts[b] + gl
            for n2 in range(p.num_heads_kv):
                c = min(max(int(p.sparse_block_count[n2, g]), 0), p.top_k)
                for j in p.sparse_block_idx[n2, g, :c]:
                    if j < 0 or 128 * int(j) >= skv:
                        continue
                    unit = (int(p.block_table[b, j]) if p.kv_layout != "TND"
                            else int(p.cu_seqlens_kv[b]) + 128 * int(j))
                    offs.append(unit * unit_bytes + n2 * 128 * es)
    return np.asarray(offs, dtype=np.int64)


def timed(fn, iters: int, stream) -> float:
    """Average ms of `iters` calls of fn launched back to back between two events."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def ceilings(p, hbm_bound: bool, stream):
    """What this GPU delivers for the same kind of work, measured beside the kernel.

    HBM-bound workloads: a gather-only kernel reading exactly the selected K/V head slices
    (the decode kernel's bytes and pattern, nothing computed) and a contiguous read of the same
    byte count. MFMA-bound ones: a dense square GEMM in the workload's dtype (hipBLASLt via
    torch; fp8 through torch._scaled_mm when this torch build offers it)."""
    import torch
    from block_sparse_paged_gbsa_amd import probe
    out = {}
    if hbm_bound:
        offs = torch.as_tensor(gather_offsets(p), device=p.k.device)
        es = ESIZE[p.dtype]
        row_bytes, row_stride = 128 * es, p.num_heads_kv * 128 * es
        nbytes = int(offs.numel()) * 2 * 128 * row_bytes
        sink = torch.empty(max(int(offs.numel()), 1024) * 4096, dtype=torch.uint8,
                           device=p.k.device)
        ms = timed(lambda: probe.gather(p.k, p.v, offs, row_bytes, row_stride, sink, stream),
                   50, stream)
        out["gather_GBs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        flat = p.k.reshape(-1).view(torch.uint8)
        n = min(nbytes, flat.numel()) // 16 * 16
        ms = timed(lambda: probe.stream_read(flat, n, 2048, sink, stream), 50, stream)
        out["contiguous_read_GBs"] = round(n / (ms * 1e-3) / 1e9, 1)
        out["bytes"] = nbytes
    else:
        n = 8192
        if p.dtype == "fp8":
            a = torch.randn(n, n, device=p.q.device).to(torch.float8_e4m3fn)
            b = torch.randn(n, n, device=p.q.device).to(torch.float8_e4m3fn).t()
            one = torch.ones((), device=p.q.device)
            try:
                ms = timed(lambda: torch._scaled_mm(a, b, scale_a=one, scale_b=one,
                                                    out_dtype=torch.bfloat16), 20, stream)
                out["gemm_fp8_TFLOPs"] = round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)
            except (RuntimeError, AttributeError) as e:  # not offered by this build
                out["gemm_fp8_TFLOPs"] = None
                out["gemm_fp8_note"] = str(e).splitlines()[0][:120]
        dt = torch.float16 if p.dtype == "f16" else torch.bfloat16
        a = torch.randn(n, n, device=p.q.device, dtype=dt)
        b = torch.randn(n, n, device=p.q.device, dtype=dt)
        ms = timed(lambda: torch.matmul(a, b), 20, stream)
        out[f"gemm_{'f16' if dt == torch.float16 else 'bf16'}_TFLOPs"] = round(
            2 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    return out


# --- CPU baseline: the float64 oracle over units on a pool of forked processes ------------
_CPU_INPUTS = None  # set before the fork: the workers share the host inputs without a copy


def _cpu_unit(task):
    """One q-block (all KV heads) through the oracle's per-unit definition; seconds spent."""
    from threadpoolctl import threadpool_limits

    from oracle.attention import attention_unit
    b, gl, ts = task
    with threadpool_limits(limits=1):  # one BLAS thread per process: the pool owns the cores
        t0 = time.perf_counter()
        for n2 in range(_CPU_INPUTS.N2):
            attention_unit(_CPU_INPUTS, b, n2, gl, ts)
        return time.perf_counter() - t0


def host_cpu():
    """(cores usable by this process, CPU model) of the host."""
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return int(cores or 1), model


def cpu_baseline(p, budget_s: float, max_workers: int = 16):
    """The float64 oracle on a bounded sample of the same workload (whole q-blocks, every KV
    head), one q-block per task on a pool of processes over the host's cores. The sample grows
    until about budget_s seconds of wall time have been spent; a workload the pool finishes
    early is timed over repeated passes of all of it. Input preparation and the pool's start
    are outside the timed region."""
    import multiprocessing

    import torch

    import gbsa_inputs as gi
    from oracle import attention as oa
    global _CPU_INPUTS

    starts = gi.q_block_starts(p.cu_seqlens_q, p.block_x)
    units = []
    for b in range(p.batch):
        storage = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
        sq = storage if p.seqused_q is None else min(int(p.seqused_q[b]), storage)
        for gl in range(-(-sq // p.block_x)):
            lo, hi = gl * p.block_x, min((gl + 1) * p.block_x, sq)
            units.append((b, gl, np.arange(lo, hi, dtype=np.int64)))
    rng = np.random.default_rng(7)
    order = rng.permutation(len(units))
    units = [units[i] for i in order]

    def host(t):
        t = t.detach()
        if p.dtype == "bf16":
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        if p.dtype == "fp8":
            return t.view(torch.uint8).cpu().numpy()
        return t.cpu().numpy()

    def host_inputs(sample):
        """Oracle inputs holding only what the sampled units read."""
        common = dict(dtype=p.dtype, block_x=p.block_x, scale=p.scale, mask_mode=p.mask_mode,
                      win_left=p.win_left, win_right=p.win_right, q_scale=p.q_scale,
                      k_scale=p.k_scale, v_scale=p.v_scale)
        if p.kv_layout == "TND":
            seqs = {b for (b, _, _) in sample}
            cu = p.cu_seqlens_kv
            new_cu = np.zeros(p.batch + 1, dtype=np.int64)
            for b in range(p.batch):
                new_cu[b + 1] = new_cu[b] + (int(cu[b + 1] - cu[b]) if b in seqs else 0)
            sel = torch.cat([torch.arange(int(cu[b]), int(cu[b + 1]), device=p.k.device)
                             for b in sorted(seqs)])
            return oa.Inputs(host(p.q), host(p.k[sel]), host(p.v[sel]), p.sparse_block_idx,
                             p.sparse_block_count, p.cu_seqlens_q, p.seqused_q, p.seqused_kv,
                             None, cu_seqlens_kv=new_cu, **common)
        pages = set()
        for (b, gl, _) in sample:
            g = starts[b] + gl
            for n2 in range(p.num_heads_kv):
                c = min(max(int(p.sparse_block_count[n2, g]), 0), p.top_k)
                for j in p.sparse_block_idx[n2, g, :c]:
                    if j >= 0 and 128 * int(j) < int(p.seqused_kv[b]):
                        pages.add(int(p.block_table[b, j]))
        pages = sorted(pages)
        remap = np.full(p.num_pages, -1, dtype=np.int64)
        remap[pages] = np.arange(len(pages))
        sel = torch.as_tensor(pages, dtype=torch.long, device=p.k.device)
        table = np.where(p.block_table >= 0, remap[np.maximum(p.block_table, 0)], -1)
        return oa.Inputs(host(p.q), host(p.k[sel]), host(p.v[sel]), p.sparse_block_idx,
                         p.sparse_block_count, p.cu_seqlens_q, p.seqused_q, p.seqused_kv,
                         table, **common)

    cores, model = host_cpu()
    workers = max(1, min(cores, max_workers))
    _CPU_INPUTS = host_inputs(units)
    # units in growing chunks (at least one per process) until the budget is spent; a workload
    # the pool finishes early is timed over repeated passes of all of it
    done, passes, elapsed, k = [], 0, 0.0, workers
    with multiprocessing.get_context("fork").Pool(workers) as pool:
        pool.map(_cpu_unit, units[:workers], chunksize=1)  # start every worker (untimed)
        while elapsed < budget_s:
            if len(done) < len(units):
                batch = units[len(done):len(done) + k]
                k *= 2
            else:
                batch = units
            t0 = time.perf_counter()
            pool.map(_cpu_unit, batch, chunksize=1)
            elapsed += time.perf_counter() - t0
            if len(done) < len(units):
                done += batch
            else:
                passes += 1
    _CPU_INPUTS = None
    bytes_s, flops_s = algorithmic_work(p, {(b, gl) for (b, gl, _) in done})
    whole = len(done) == len(units)
    if whole:
        passes += 1
    return dict(units=len(done), seconds=elapsed, bytes=bytes_s * max(passes, 1),
                flops=flops_s * max(passes, 1), passes=max(passes, 1), whole=whole,
                cores=workers, host_cores=cores, cpu_model=model)


# --- one workload on the GPU ------------------------------------------------------------------
class Workload:
    """A problem's tensors on the GPU and the two calls of the path (marshalling only)."""

    def __init__(self, p, dev, tnd=False, umask=None):
        import torch

        import gbsa_inputs as gi
        from block_sparse_paged_gbsa_amd import gbsa_num_workers, gbsa_workspace_size, make_params
        self.p, self.tnd, self.umask = p, tnd, umask
        self.params = make_params(
            batch=p.batch, num_heads_q=p.num_heads_q, num_heads_kv=p.num_heads_kv,
            total_q=p.total_q, total_q_blocks=p.total_q_blocks, top_k=p.top_k,
            block_x=p.block_x, max_blocks_per_seq=0 if tnd else p.block_table.shape[1],
            num_pages=p.num_pages, kv_page_stride=p.kv_page_stride,
            dtype=gi.TORCH_DTYPES[p.dtype], out_dtype=gi.TORCH_DTYPES[p.out_dtype],
            mask_mode=p.mask_mode, win_left=p.win_left, win_right=p.win_right,
            quant_mode=p.quant_mode, return_lse=p.return_lse,
            has_seqused_q=p.seqused_q is not None, scale=p.scale, kv_layout=1 if tnd else 0)
        t = lambda x: None if x is None else torch.as_tensor(x).to(dev)
        self.idx, self.cnt, self.cu, self.skv = (t(p.sparse_block_idx), t(p.sparse_block_count),
                                                 t(p.cu_seqlens_q), t(p.seqused_kv))
        self.table = None if tnd else t(p.block_table)
        self.cu_kv = t(p.cu_seqlens_kv) if tnd else None
        self.squ = None if p.seqused_q is None else t(p.seqused_q)
        f32 = lambda s: None if s is None else torch.as_tensor(s, dtype=torch.float32).to(dev)
        self.qs, self.ks, self.vs = f32(p.q_scale), f32(p.k_scale), f32(p.v_scale)
        self.ps = None  # [N1] P quantisation scales (quant mode 5: fp8 P·V), `--p-scale`
        self.meta = torch.empty(1024, dtype=torch.int32, device=dev)
        self.out = torch.empty(p.q.shape, dtype=gi.TORCH_DTYPES[p.out_dtype], device=dev)
        self.lse = (torch.empty(p.q.shape[:2], dtype=torch.float32, device=dev)
                    if p.return_lse else None)
        self.ws = torch.zeros(gbsa_workspace_size(self.params), dtype=torch.uint8, device=dev)
        self.P = gbsa_num_workers(self.params)
        self.rows = p.block_x * p.num_heads_q // p.num_heads_kv  # packed GQA rows per unit

    @property
    def kernel(self):
        """The main kernel the library picks for this workload (rows per unit, dtype, options)."""
        rows, fp8 = self.rows, self.p.dtype == "fp8"
        if rows <= 16:
            return "fwd_decode_kernel"
        if rows > 256:
            return "fwd_prefill_pp32_kernel" if fp8 else "fwd_prefill_pp32d_kernel"
        if rows > 64:
            # fp8 without a user mask or P quantisation scale: the DMA key-split kernel
            dma = fp8 and self.umask is None and self.ps is None
            return "fwd_prefill_ks32d_kernel" if dma else "fwd_prefill_ks32_kernel"
        return "fwd_prefill_kernel"

    def metadata(self):
        from block_sparse_paged_gbsa_amd import gbsa_metadata
        gbsa_metadata(self.params, self.cnt, self.cu, self.squ, self.skv, self.meta)

    def forward(self):
        from block_sparse_paged_gbsa_amd import gbsa_forward, gbsa_forward_ex, gbsa_forward_tnd
        p = self.p
        if self.umask is not None:
            gbsa_forward_ex(self.params, p.q, p.k, p.v, self.idx, self.cnt, self.meta, self.cu,
                            self.squ, cu_seqlens_kv=self.cu_kv, seqused_kv=self.skv,
                            block_table=self.table, q_scale=self.qs, k_scale=self.ks,
                            v_scale=self.vs, p_scale=self.ps, atten_mask=self.umask,
                            out=self.out, lse=self.lse, workspace=self.ws)
        elif self.tnd:
            gbsa_forward_tnd(self.params, p.q, p.k, p.v, self.idx, self.cnt, self.meta, self.cu,
                             self.squ, self.cu_kv, self.skv, self.qs, self.ks, self.vs, self.ps,
                             self.out, self.lse, self.ws)
        else:
            gbsa_forward(self.params, p.q, p.k, p.v, self.idx, self.cnt, self.meta, self.cu,
                         self.squ, self.skv, self.table, self.qs, self.ks, self.vs, self.ps,
                         self.out, self.lse, self.ws)

    def step(self):
        self.metadata()
        self.forward()

    def status(self) -> int:
        return int(self.ws[:4].view(__import__("torch").int32)[0].item())


def cache_flusher(dev):
    """A read of 1 GiB that evicts the L2s and the Infinity Cache (256 MiB) without leaving
    dirty lines behind, so the next kernel finds none of its data cached and has no unrelated
    write-back to do."""
    import torch
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    acc = torch.empty((), dtype=torch.int64, device=dev)
    return lambda: torch.sum(flush, dim=0, dtype=torch.int64, out=acc)


def cold_forward_ms(w, flush, iters: int, stream) -> float:
    """The forward's average duration when every launch follows a cache-evicting read: each
    launch timed on its own between two events on its stream, recorded after the read has
    finished there (subtracting a separately timed read would add that read's jitter)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    flush()
    w.forward()
    for e0, e1 in ev:
        flush()
        e0.record(stream)
        w.forward()
        e1.record(stream)
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in ev) / iters


def roofline(w, alg_bytes, alg_flops, fwd_ms):
    """roofline object of the workload's dominant kernel from the forward's duration."""
    p = w.p
    if w.kernel == "fwd_decode_kernel":
        achieved = alg_bytes / (fwd_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    achieved = alg_flops / (fwd_ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[p.dtype]
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4)}


def config_sweep(dev, stream, iters: int, skip=None, known=None):
    """Every workload in the benchmark's launch configuration: forward ms (launches back to
    back), rate and roofline fraction of its kernel. `known` carries a workload already timed
    in this run (reused as is)."""
    import torch

    import gbsa_inputs as gi
    out = {}
    for cfg in sorted(gi.CONFIG_NAMES):
        name = gi.CONFIG_NAMES[cfg]
        if known is not None and name in known:
            out[name] = known[name]
            continue
        log(f"[bench] sweep: workload {cfg} ({name})")
        p = gi.config(cfg, device=dev)
        w = Workload(p, dev)
        alg_bytes, alg_flops = algorithmic_work(p)
        w.step()
        torch.cuda.synchronize()
        per = timed(w.forward, 1, stream)
        n = int(min(iters, max(3, 2000.0 / max(per, 1e-3))))  # about 2 s per workload at most
        w.metadata()
        fwd_ms = timed(w.forward, n, stream)
        meta_ms = timed(w.metadata, n, stream)
        assert w.status() == 0, f"{name}: metadata mismatch flagged by the kernels"
        roof = roofline(w, alg_bytes, alg_flops, fwd_ms)
        out[name] = {"kernel": w.kernel, "forward_ms": round(fwd_ms, 5),
                     "metadata_ms": round(meta_ms, 5), "launches": n, "workers": w.P,
                     "dtype": p.dtype, "tflops": round(alg_flops / (fwd_ms * 1e-3) / 1e12, 2),
                     "gbs": round(alg_bytes / (fwd_ms * 1e-3) / 1e9, 1), "roofline": roof}
        log(f"[bench] sweep: {name} forward {fwd_ms:.4f} ms, {roof['achieved']} "
            f"{roof['unit']} = {roof['frac']} of peak")
        del w, p
        torch.cuda.empty_cache()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload id 1..5 (default 2)")
    ap.add_argument("--kv-layout", choices=["pa_bbnd", "tnd"], default="pa_bbnd",
                    help="key/value layout: paged (default) or token-major TND")
    ap.add_argument("--user-mask", choices=["none", "causal"], default="none",
                    help="causal: replace the built-in causal mask of a causal workload with an "
                         "equal user attention mask (same visible keys, timed through the "
                         "per-element mask path)")
    ap.add_argument("--batch", type=int, default=64,
                    help="workload 2 only: number of decode queries (fewer than 64 splits "
                         "each unit over several workers)")
    ap.add_argument("--top-k", type=int, default=16,
                    help="workload 2 only: pages selected per query (at most 256)")
    ap.add_argument("--block-x", type=int, default=128,
                    help="workload 3 only: query rows per q-block (fewer than 16 packs fewer "
                         "rows per unit and selects the 17-64 or 65-256 row kernels)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle wall time for the CPU baseline (0 = skip)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip timing the other workloads (the `configs` object)")
    ap.add_argument("--forward-only", type=int, default=0, metavar="N",
                    help="only run the metadata and N forward launches of the workload back to "
                         "back (for counter and kernel-trace profiles) and print their count")
    ap.add_argument("--cold-only", action="store_true",
                    help="only run cache-flushed forward launches of the workload (for a "
                         "kernel-trace profile of them) and print their count")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter scale reference)")
    ap.add_argument("--p-scale", type=float, default=0.0, metavar="S",
                    help="fp8 workloads: pass p_quant_scale S for every query head, so that P is "
                         "cast to e4m3 and P·V runs on fp8 MFMA (name suffixed `_p8`)")
    ap.add_argument("--slot-trace", action="store_true",
                    help="run the workload on the slot-trace build of the library "
                         "(libgbsa_slot_trace.so, include/gbsa_slot_trace.h) and print the "
                         "item durations of one traced unit of the 256-row DMA kernel")
    a = ap.parse_args(argv)
    if a.slot_trace:
        from block_sparse_paged_gbsa_amd import _lib
        _lib.LIB_PATH = os.path.join(os.path.dirname(_lib.LIB_PATH), "libgbsa_slot_trace.so")
        if not os.path.exists(_lib.LIB_PATH):
            print(f"{_lib.LIB_PATH} is missing: build it with "
                  "`python -m block_sparse_paged_gbsa_amd.build`", file=sys.stderr)
            return 2
    if a.copy_calibration:
        return copy_calibration(a.copy_calibration)
    if (a.batch, a.top_k) != (64, 16) and (a.config != 2 or not 1 <= a.batch <= 4096 or
                                           not 1 <= a.top_k <= 256):
        print("--batch / --top-k apply to workload 2 (1..4096 queries, 1..256 pages)",
              file=sys.stderr)
        return 2
    if a.block_x != 128 and (a.config != 3 or not 1 <= a.block_x <= 128):
        print("--block-x applies to workload 3 (1..128 rows)", file=sys.stderr)
        return 2
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the kernel has no cross-GPU path in this build "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import gbsa_inputs as gi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    log(f"[bench] generating workload {a.config} on the GPU")
    if (a.batch, a.top_k) != (64, 16):
        p = gi.decode_workload(a.batch, a.top_k, device=dev)
    elif a.block_x != 128:
        p = gi.block_sparse_prefill(a.block_x, device=dev)
    else:
        p = gi.config(a.config, device=dev)
    tnd = a.kv_layout == "tnd"
    if tnd:
        log("[bench] rewriting key/value into the token-major TND layout")
        p = gi.to_tnd(p)
        torch.cuda.empty_cache()
    umask = None
    if a.user_mask == "causal":
        offs = {p.kv_len(b) - (int(p.seqused_q[b]) if p.seqused_q is not None
                               else int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b]))
                for b in range(p.batch)}
        if p.mask_mode != 1 or p.win_left >= 0 or p.win_right >= 0 or len(offs) != 1:
            print("--user-mask causal needs a causal workload without a window whose "
                  "sequences share one diagonal (workloads 3 and 5)", file=sys.stderr)
            return 2
        off = offs.pop()
        rows = int((p.cu_seqlens_q[1:] - p.cu_seqlens_q[:-1]).max())
        cols = max(p.kv_len(b) for b in range(p.batch))
        log(f"[bench] user mask [{rows}, {cols}] uint8 equal to the causal mask")
        t_idx = torch.arange(rows, device=dev, dtype=torch.int32)[:, None]
        p_idx = torch.arange(cols, device=dev, dtype=torch.int32)[None, :]
        umask = (p_idx > t_idx + off).to(torch.uint8)
        del t_idx, p_idx
        p.mask_mode = 0
    w = Workload(p, dev, tnd, umask)
    if a.p_scale > 0:
        if p.dtype != "fp8":
            print("--p-scale applies to fp8 workloads (workload 5)", file=sys.stderr)
            return 2
        w.ps = torch.full((p.num_heads_q,), a.p_scale, dtype=torch.float32, device=dev)
        p.name += "_p8"
    stream = torch.cuda.current_stream()
    hbm_bound = w.kernel == "fwd_decode_kernel"

    if a.forward_only > 0:
        w.step()
        for _ in range(a.forward_only):
            w.forward()
        torch.cuda.synchronize()
        assert w.status() == 0, "metadata mismatch flagged by the kernels"
        print(json.dumps({"forward_launches": a.forward_only + 1, "kernel": w.kernel,
                          "workload": p.name}), flush=True)
        return 0
    if a.slot_trace:
        return slot_trace(w, p)
    if a.cold_only:
        flush = cache_flusher(dev)
        w.step()
        for _ in range(a.steps):
            flush()
            w.forward()
        torch.cuda.synchronize()
        assert w.status() == 0, "metadata mismatch flagged by the kernels"
        print(json.dumps({"cold_forward_launches": a.steps, "kernel": w.kernel,
                          "workload": p.name}), flush=True)
        return 0

    alg_bytes, alg_flops = algorithmic_work(p)
    log(f"[bench] workers={w.P} algorithmic bytes={alg_bytes} flops={alg_flops}")
    for _ in range(a.warmup):
        w.step()
    torch.cuda.synchronize()

    # whole steps, back to back
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        w.step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / a.steps

    # the forward launch alone (main kernel with its fused split-KV combine): K launches back
    # to back between two events on their stream, so the average is the kernel's duration
    # without per-launch gaps
    fwd_ms = timed(w.forward, a.steps, stream)

    # the same step replayed from a HIP graph (metadata + forward captured once): what a serving
    # loop that captures its step pays, without per-call launch work
    graph_ms = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            w.step()
            side.synchronize()
            with torch.cuda.graph(graph, stream=side):
                w.step()
        stream.wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        graph_ms = timed(graph.replay, a.steps, stream)
        del graph
    except RuntimeError as e:  # capture unavailable: report the eager figures only
        log(f"[bench] graph capture failed: {e}")
    meta_ms = timed(w.metadata, a.steps, stream)
    assert w.status() == 0, "metadata mismatch flagged by the kernels"
    log(f"[bench] step {ms_step:.4f} ms, forward {fwd_ms:.4f} ms, wall {wall:.3f} s")

    # every forward launch after a 1 GiB read that evicts the L2s and the Infinity Cache: the
    # selected K/V bytes then come from HBM
    flush = cache_flusher(dev)
    fwd_cold_ms = cold_forward_ms(w, flush, a.steps, stream)
    del flush
    torch.cuda.empty_cache()
    ceil = ceilings(p, hbm_bound, stream)
    log(f"[bench] metadata {meta_ms:.4f} ms, cold forward {fwd_cold_ms:.4f} ms, ceilings {ceil}")

    gbs = alg_bytes / (ms_step * 1e-3) / 1e9
    tflops = alg_flops / (ms_step * 1e-3) / 1e12
    # the name carries "_tnd" after the layout rewrite
    workload = p.name + ("_user_mask" if umask is not None else "")
    traffic = measured_traffic(w.kernel, workload)
    if hbm_bound:
        # the roofline of the HBM-bound kernel is taken on cache-flushed launches; the warm
        # figure (launches back to back) is reported beside it
        roof = roofline(w, alg_bytes, alg_flops, fwd_cold_ms)
        roof["timing"] = "cache-flushed launches"
        roof["achieved_warm"] = roofline(w, alg_bytes, alg_flops, fwd_ms)["achieved"]
        metric_value, unit = gbs, "GB/s"
    else:
        roof = roofline(w, alg_bytes, alg_flops, fwd_ms)
        roof["timing"] = "launches back to back"
        metric_value, unit = tflops, "TFLOP/s"
    roof["traffic"] = traffic
    main_entry = {"kernel": w.kernel, "forward_ms": round(fwd_ms, 5),
                  "forward_cold_ms": round(fwd_cold_ms, 5), "metadata_ms": round(meta_ms, 5),
                  "launches": a.steps, "workers": w.P, "dtype": p.dtype,
                  "tflops": round(alg_flops / (fwd_ms * 1e-3) / 1e12, 2),
                  "gbs": round(alg_bytes / (fwd_ms * 1e-3) / 1e9, 1),
                  "roofline": roofline(w, alg_bytes, alg_flops,
                                       fwd_cold_ms if hbm_bound else fwd_ms)}
    default_shape = (not tnd and umask is None and (a.batch, a.top_k) == (64, 16) and
                     a.block_x == 128)
    config = {"workload": workload, "kv_layout": "TND" if tnd else "PA_BBND",
              "mask": "user (causal pattern)" if umask is not None else
                      {0: "none", 1: "causal", 2: "causal top-left"}[p.mask_mode],
              "batch": p.batch, "num_heads_q": p.num_heads_q, "num_heads_kv": p.num_heads_kv,
              "head_dim": 128, "block_shape": [p.block_x, 128], "top_k": p.top_k,
              ("kv_rows" if tnd else "kv_pages"): p.num_pages, "workers": w.P}

    cpu = None
    if a.cpu_budget > 0 and umask is None:
        log("[bench] timing the float64 oracle on a sample, all host cores")
        cb = cpu_baseline(p, a.cpu_budget)
        v = (cb["bytes"] / cb["seconds"] / 1e9) if hbm_bound else (cb["flops"] / cb["seconds"] / 1e12)
        cpu = {"value": round(v, 6), "unit": unit, "cores": cb["cores"], "kind": "oracle",
               "sample": (f"all {cb['units']} q-blocks (all KV heads) of the workload, "
                          f"{cb['passes']} passes" if cb["whole"] else
                          f"{cb['units']} q-blocks (all KV heads) of the same workload") +
                         f", {cb['seconds']:.1f} s wall of float64 numpy on a pool of "
                         f"{cb['cores']} processes, one q-block per task",
               "cpu_model": cb["cpu_model"], "host_cores": cb["host_cores"],
               "blas_threads_per_process": 1}
        log(f"[bench] oracle: {cpu}")

    configs = None
    if not a.no_sweep:
        del w
        torch.cuda.empty_cache()
        known = {p.name: main_entry} if default_shape else None
        del p
        torch.cuda.empty_cache()
        configs = config_sweep(dev, stream, a.steps, known=known)
        p = None
    res = {
        "metric": "block-sparse attn effective TFLOP/s + HBM GB/s, % of roofline, 1 MI355X",
        "value": round(metric_value, 3), "unit": unit, "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": main_entry["dtype"],
        "data": "synthetic",
        "config": config,
        "effective_tflops": round(tflops, 3), "hbm_gbs": round(gbs, 2),
        "forward_ms": round(fwd_ms, 5), "metadata_ms": round(meta_ms, 5),
        "ms_per_step_graph": None if graph_ms is None else round(graph_ms, 5),
        "forward_cold_ms": round(fwd_cold_ms, 5),
        "ceilings": ceil, "kernel": main_entry["kernel"], "algorithmic_bytes": alg_bytes,
        "algorithmic_flops": alg_flops, "roofline": roof, "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

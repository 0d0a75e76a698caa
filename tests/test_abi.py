"""The C-ABI library loads, exports what include/gbsa.h declares, matches its struct layout
and rejects invalid attributes before touching a device (CPU only)."""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_paged_gbsa_amd import _lib
from block_sparse_paged_gbsa_amd.api import make_params

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gbsa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gbsa_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (gbsa_\w+)", out))
    assert set(names) <= exported


@pytest.mark.parametrize("cname,pystruct", [("gbsa_params", _lib.GbsaParams),
                                             ("gbsa_forward_args", _lib.GbsaForwardArgs)])
def test_struct_layouts_match_c(cname, pystruct):
    """Compile a tiny C program against the header and compare sizeof/offsetof."""
    fields = [f for f, _ in pystruct._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "gbsa.h"', 'int main(void){',
           f'printf("%zu\\n", sizeof({cname}));']
    src += [f'printf("%zu\\n", offsetof({cname}, {f}));' for f in fields]
    src += ['return 0;}']
    tmp = os.path.join("/tmp", f"gbsa_layout_{cname}_{os.getpid()}")
    with open(tmp + ".c", "w") as fh:
        fh.write("\n".join(src))
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", tmp + ".c", "-o", tmp], check=True)
    vals = [int(x) for x in subprocess.run([tmp], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(pystruct)
    for f, off in zip(fields, vals[1:]):
        assert getattr(pystruct, f).offset == off, f


def _good(**kw):
    base = dict(batch=2, num_heads_q=8, num_heads_kv=2, total_q=640, total_q_blocks=10,
                top_k=4, block_x=64, max_blocks_per_seq=3, num_pages=5, mask_mode=1,
                num_workers=7)
    base.update(kw)
    return make_params(**base)


def _check(p):
    return _lib.load().gbsa_check_params(ctypes.byref(p))


def test_valid_params_pass():
    assert _check(_good()) == 0


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, 2), ("block_y", 64, 2), ("page_size", 256, 2), ("num_heads_kv", 3, 2),
    ("top_k", 257, 2), ("win_left", -2, 2), ("num_workers", 1000, 2), ("kv_page_stride", 100, 2),
    ("batch", 0, 5), ("total_q", 0, 5), ("top_k", 0, 5), ("num_pages", 0, 5),
    ("quant_mode", 3, 4), ("mask_mode", 3, 4), ("is_packed_gqa", 0, 4), ("softmax_precision", 2, 4),
    ("dtype", 2, 3), ("out_dtype", 2, 3), ("batch", 20000, 4),
])
def test_rejections(field, value, code):
    p = _good()
    setattr(p, field, value)
    assert _check(p) == code


def test_group_limit_and_quant_dtype_rules():
    assert _check(_good(num_heads_q=258, num_heads_kv=2)) == 2  # group 129 > 128
    assert _check(_good(num_heads_q=256, num_heads_kv=2)) == 0  # group 128
    import torch
    assert _check(_good(quant_mode=5)) == 3  # quant 5 needs fp8 inputs
    assert _check(_good(quant_mode=5, dtype=torch.float8_e4m3fn, out_dtype=torch.bfloat16)) == 0
    assert _check(_good(dtype=torch.bfloat16, out_dtype=torch.float16)) == 3  # quant 0: out=q
    assert _check(_good(kv_page_stride=128 * 2 * 128 + 256)) == 0
    assert _check(_good(kv_page_stride=128 * 2 * 128 + 100)) == 2


def test_max_seqlen_bounds():
    """max_seqlen_q / max_seqlen_kv (the metadata operator's keyword arguments): -1 or 0 mean
    "not given"; a given bound must fit the query rows and the KV storage (3 pages of 128)."""
    assert _check(_good(max_seqlen_q=-1, max_seqlen_kv=-1)) == 0
    assert _check(_good(max_seqlen_q=0, max_seqlen_kv=0)) == 0
    assert _check(_good(max_seqlen_q=384, max_seqlen_kv=384)) == 0
    assert _check(_good(max_seqlen_q=640)) == 0
    assert _check(_good(max_seqlen_q=641)) == 2  # longer than total_q
    assert _check(_good(max_seqlen_kv=385)) == 2  # more than max_blocks_per_seq * 128 keys
    assert _check(_good(max_seqlen_q=-2)) == 2
    assert _check(_good(max_seqlen_kv=-5)) == 2
    tnd = _good(kv_layout=_lib.KV_TND, max_blocks_per_seq=0, num_pages=1000)
    assert _check(tnd) == 0
    tnd.max_seqlen_kv = 1000
    assert _check(tnd) == 0
    tnd.max_seqlen_kv = 1001  # more than the T_kv rows
    assert _check(tnd) == 2
    for bad in (-1.0, float("nan"), float("inf")):
        p = _good()
        p.dst_type_max = bad
        assert _check(p) == 4
    p = _good()
    p.dst_type_max = 240.0
    assert _check(p) == 0


def test_entry_points_validate_before_device_work():
    lib = _lib.load()
    bad = _good(head_dim=64)
    dummy = ctypes.c_void_p(0x1000)
    assert lib.gbsa_metadata(ctypes.byref(bad), dummy, dummy, None, dummy, dummy, None) == 2
    assert lib.gbsa_forward(ctypes.byref(bad), *([dummy] * 17), 0, None) == 2
    good = _good()
    # missing metadata buffer / workspace / inconsistent optional pointers
    assert lib.gbsa_metadata(ctypes.byref(good), dummy, dummy, None, dummy, None, None) == 7
    assert lib.gbsa_metadata(ctypes.byref(good), dummy, dummy, dummy, dummy, dummy, None) == 1
    args = [dummy] * 17
    # order: q k v idx cnt meta cu squ skv table qs ks vs ps out lse ws
    args[7] = None  # seqused_q
    args[10] = args[11] = args[12] = None  # dequant scales (quant 0)
    args[13] = None  # p_scale
    args[15] = None  # lse (return_lse 0)
    assert lib.gbsa_forward(ctypes.byref(good), *args, 0, None) == 6  # workspace too small
    args2 = list(args)
    args2[11] = dummy  # a dequant scale with quant 0
    assert lib.gbsa_forward(ctypes.byref(good), *args2, 1 << 40, None) == 3
    args3 = list(args)
    args3[13] = dummy  # p_scale needs quant mode 5
    assert lib.gbsa_forward(ctypes.byref(good), *args3, 1 << 40, None) == 3
    sz = ctypes.c_size_t(0)
    assert lib.gbsa_workspace_size(ctypes.byref(good), ctypes.byref(sz)) == 0 and sz.value > 0
    n = ctypes.c_int32(0)
    assert lib.gbsa_num_workers(ctypes.byref(good), ctypes.byref(n)) == 0 and n.value == 7


def test_status_strings():
    for code in range(9):
        assert len(_lib.status_string(code)) >= 2


def test_tnd_layout_rules():
    """Token-major key/value: rows in num_pages, no page stride, block table not needed."""
    tnd = _lib.KV_TND
    assert _check(_good(kv_layout=tnd, max_blocks_per_seq=0, num_pages=1000)) == 0
    assert _check(_good(kv_layout=2)) == 4
    assert _check(_good(kv_layout=tnd, kv_page_stride=128 * 2 * 128)) == 2
    assert _check(_good(kv_layout=tnd, num_pages=_lib.MAX_KV_ROWS)) == 0
    assert _check(_good(kv_layout=tnd, num_pages=_lib.MAX_KV_ROWS + 1)) == 2
    assert _check(_good(max_blocks_per_seq=0)) == 5  # the paged layout needs a block table


def test_tnd_entry_point_validation():
    lib = _lib.load()
    dummy = ctypes.c_void_p(0x1000)
    paged = _good()
    tnd = _good(kv_layout=_lib.KV_TND, max_blocks_per_seq=0, num_pages=1000)
    # order: q k v idx cnt meta cu squ cu_kv skv qs ks vs ps out lse ws
    args = [dummy] * 17
    args[7] = None  # seqused_q
    args[10] = args[11] = args[12] = args[13] = None  # scales
    args[15] = None  # lse
    # each layout has its own entry point
    assert lib.gbsa_forward(ctypes.byref(tnd), *args, 1 << 40, None) == 4
    assert lib.gbsa_forward_tnd(ctypes.byref(paged), *args, 1 << 40, None) == 4
    assert lib.gbsa_forward_tnd(ctypes.byref(tnd), *args, 0, None) == 6  # workspace too small
    a2 = list(args)
    a2[8] = None  # cu_seqlens_kv is required
    assert lib.gbsa_forward_tnd(ctypes.byref(tnd), *a2, 1 << 40, None) == 1
    a3 = list(args)
    a3[9] = None  # seqused_kv is optional with TND
    assert lib.gbsa_forward_tnd(ctypes.byref(tnd), *a3, 0, None) == 6
    # metadata: seqused_kv optional with TND, required with PA_BBND
    assert lib.gbsa_metadata(ctypes.byref(tnd), dummy, dummy, None, None, None, None) == 7
    assert lib.gbsa_metadata(ctypes.byref(paged), dummy, dummy, None, None, dummy, None) == 1


def _args(**kw):
    g = _lib.GbsaForwardArgs()
    for f in ("query", "key", "value", "sparse_block_idx", "sparse_block_count", "metadata",
              "cu_seqlens_q", "seqused_kv", "block_table", "attention_out", "workspace"):
        setattr(g, f, 0x1000)
    for k, v in kw.items():
        setattr(g, k, v)
    return g


def test_forward_ex_validation():
    """The all-options entry point: mask geometry rules, one layout's tensors only, mask
    mode 2 accepted; every case stops before any device work."""
    lib = _lib.load()
    good = _good()
    fx = lambda p, g: lib.gbsa_forward_ex(ctypes.byref(p), None if g is None else ctypes.byref(g),
                                         None)
    assert fx(good, None) == 1
    assert fx(good, _args(workspace_bytes=0)) == 6  # reaches the workspace check
    mask = dict(atten_mask=0x2000, mask_rows=64, mask_cols=100, mask_row_stride=100)
    assert fx(good, _args(workspace_bytes=0, **mask)) == 6  # a valid mask
    assert fx(good, _args(workspace_bytes=0, **dict(mask, atten_mask=0x2001))) == 2  # alignment
    assert fx(good, _args(workspace_bytes=0, **dict(mask, mask_row_stride=102))) == 2
    assert fx(good, _args(workspace_bytes=0, **dict(mask, mask_row_stride=96))) == 2  # < cols
    assert fx(good, _args(workspace_bytes=0, **dict(mask, mask_batch_stride=6))) == 2
    assert fx(good, _args(workspace_bytes=0, **dict(mask, mask_rows=1 << 24,
                                                    mask_row_stride=1 << 8))) == 2  # 2^32 B
    assert fx(good, _args(workspace_bytes=0, **dict(mask, mask_cols=-1))) == 2
    # the layout not in use takes no tensors
    assert fx(good, _args(workspace_bytes=0, cu_seqlens_kv=0x3000)) == 1
    tnd = _good(kv_layout=_lib.KV_TND, max_blocks_per_seq=0, num_pages=1000)
    assert fx(tnd, _args(workspace_bytes=0)) == 1  # block_table given with TND
    assert fx(tnd, _args(workspace_bytes=0, block_table=None, cu_seqlens_kv=0x3000)) == 6
    assert fx(tnd, _args(workspace_bytes=0, block_table=None)) == 1  # cu_seqlens_kv missing
    # mask mode 2 (causal, top-left) is accepted
    assert _check(_good(mask_mode=_lib.MASK_CAUSAL_TOP_LEFT)) == 0


def test_probe_library_exports_its_header():
    from block_sparse_paged_gbsa_amd import probe
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "gbsa_probe.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(gbsa_probe_[a-z_]+)\s*\(", text)))
    assert set(names) == set(probe.EXPORTED)
    lib = probe.load()
    for n in names:
        assert hasattr(lib, n)
    # invalid arguments are refused before any launch
    assert lib.gbsa_probe_gather(None, None, None, 0, 256, 2048, None, None) == -1
    assert lib.gbsa_probe_stream(ctypes.c_void_p(0x1000), 15, 1, ctypes.c_void_p(0x1000),
                                 None) == -1


def test_slot_trace_library_exports_both_headers():
    """The diagnostic build is the library plus the two readout calls of gbsa_slot_trace.h;
    the normal build has neither."""
    trace = os.path.join(os.path.dirname(_lib.LIB_PATH), "libgbsa_slot_trace.so")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "gbsa_slot_trace.h")).read(),
                  flags=re.S)
    extra = sorted(set(re.findall(r"\b(gbsa_slot_trace_[a-z_]+)\s*\(", text)))
    assert extra == ["gbsa_slot_trace_read", "gbsa_slot_trace_reset"]

    def exports(path):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                             text=True, check=True).stdout
        return set(re.findall(r" T (gbsa_\w+)", out))
    assert exports(trace) == exports(_lib.LIB_PATH) | set(extra)
    assert not exports(_lib.LIB_PATH) & set(extra)


def test_noalloc_forward_argument_checks():
    """gbsa_forward_ex_noalloc takes no workspace and refuses shapes whose partial results do
    not fit its fixed array, before touching a device."""
    lib = _lib.load()
    fx = lambda p, g: lib.gbsa_forward_ex_noalloc(ctypes.byref(p), ctypes.byref(g), None)
    assert lib.gbsa_forward_ex_noalloc(ctypes.byref(_good()), None, None) == 1
    assert fx(_good(head_dim=64), _args()) == 2  # parameter errors first
    assert fx(_good(), _args()) == 6  # a workspace is given
    # 999 workers x 256 rows per unit: 2 * 999 * 256 rows of 128 floats > 32 MiB
    big = _good(num_workers=999)
    assert fx(big, _args(workspace=None, workspace_bytes=0)) == 6
    assert _lib.NOALLOC_SCRATCH_BYTES == 32 << 20


def test_validate_argument_checks():
    """gbsa_validate refuses missing or inconsistent pointers before any device work."""
    lib = _lib.load()
    good = _good()
    d = ctypes.c_void_p(0x1000)
    v = lambda p, g, out: lib.gbsa_validate(ctypes.byref(p), None if g is None else
                                            ctypes.byref(g), out, None)
    assert v(good, _args(), None) == 1  # violations pointer
    assert v(good, None, d) == 1
    assert v(good, _args(block_table=None), d) == 1  # paged needs the block table
    assert v(good, _args(cu_seqlens_kv=0x3000), d) == 1  # and no cu_seqlens_kv
    assert v(_good(head_dim=64), _args(), d) == 2  # parameter errors first

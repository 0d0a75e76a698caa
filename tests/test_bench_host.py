"""Host-side checks of bench.py (CPU only): the one-GPU contract and the work accounting that
turns a launch time into GB/s and TFLOP/s, pinned to closed forms of two workloads."""
import os
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(__file__), ".."))
import bench  # noqa: E402
import gbsa_inputs as gi  # noqa: E402


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("argv", [["--config", "3", "--batch", "8"], ["--top-k", "300"],
                                  ["--batch", "0"]])
def test_decode_shape_options_are_checked_first(argv, capsys):
    assert bench.main(argv) == 2  # before any GPU work
    assert "--batch" in capsys.readouterr().err


def test_decode_workload_bytes_and_flops():
    """64 queries x 8 KV heads select 16 full 128-token pages each: K and V rows are
    512 * 16 * 128 * 2 * 128 * 2 bytes; Q and O rows 64 * 32 * 128 * (2 + 2); each selected
    block costs its index and its page-table entry (8 bytes), each unit its count (4 bytes);
    no LSE. FLOPs: 4 * 128 per (query row, query head, key): 64 * 32 * 2048 keys."""
    p = gi.config(2, values=False)
    nbytes, flops = bench.algorithmic_work(p)
    kv = 512 * 16 * 128 * 2 * 128 * 2
    qo = 64 * 32 * 128 * 4
    meta = 512 * 16 * 8 + 512 * 4
    assert nbytes == kv + qo + meta == 537_987_072
    assert flops == 64 * 32 * 2048 * 4 * 128
    offs = bench.gather_offsets(p)
    assert len(offs) == 512 * 16 and len(set(offs.tolist())) == 512 * 16


def test_dense_equivalent_fp8_flops():
    """Every causal block selected: q-block g of each (sequence, head) sees g + 1 full blocks
    (the counted keys are the selected blocks' visible length; the causal cut inside the
    diagonal block is not subtracted), 128 query rows each."""
    p = gi.config(5, values=False)
    _, flops = bench.algorithmic_work(p)
    per_pair = sum(g + 1 for g in range(256)) * 128 * 128 * 4 * 128
    assert flops == 2 * 16 * per_pair == 8_830_452_760_576


def test_small_decode_variant_accounting():
    p = gi.decode_workload(8, 16, values=False)
    assert p.name == "decode_bf16_b8_top16" and p.batch == 8
    nbytes, _ = bench.algorithmic_work(p)
    assert nbytes == 64 * 16 * 65536 + 8 * 32 * 128 * 4 + 64 * 16 * 8 + 64 * 4

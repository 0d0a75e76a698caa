"""Pins for the float64 oracle: library routines, closed forms, invariants, hand-worked values.

None of these re-types the oracle's own formula: each compares it with something
fixed independently (torch's SDPA and logsumexp, torch's dtype conversions, the
OCP format table, exact closed forms, brute-force enumeration, or hand-worked
fixtures under tests/golden/).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import gbsa_inputs as gi
from helpers import dequant, oracle_inputs, user_mask
from oracle import attention as oa
from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# formats
# ---------------------------------------------------------------------------

def test_e4m3fn_matches_torch_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3fn_to_f64(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_e4m3fn_golden_table():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e4m3fn_values.txt"))
            if ln.strip() and not ln.startswith("#")]
    for byte, val in rows:
        got = formats.e4m3fn_to_f64(np.array([int(byte, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_bf16_and_f16_decode_match_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = formats.bf16_to_f64(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok]) and np.array_equal(np.isnan(ours), ~ok)
    ref16 = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    ours16 = formats.f16_to_f64(bits)
    ok = ~np.isnan(ref16)
    assert np.array_equal(ours16[ok], ref16[ok])


# ---------------------------------------------------------------------------
# mask reading (hand-worked)
# ---------------------------------------------------------------------------

def test_visibility_golden():
    spec = json.load(open(os.path.join(GOLDEN, "mask_example.json")))
    for c in spec["cases"]:
        t = np.arange(c["sq"])
        p = np.arange(c["skv"] + 3)  # a few positions past seqused must never be visible
        vis = oa.visible(p, t, c["skv"], c["skv"] - c["sq"], c["mask_mode"], c["win_left"],
                         c["win_right"])
        for ti, want in c["visible"].items():
            assert sorted(p[vis[int(ti)]].tolist()) == want, (c, ti)


# ---------------------------------------------------------------------------
# against torch SDPA on logically re-assembled sequences
# ---------------------------------------------------------------------------

def _logical_kv(p, b, n2):
    """K, V of sequence b / head n2 as a contiguous float64 [skv, D] via torch indexing."""
    skv = p.kv_len(b)
    if p.kv_layout == "TND":  # the sequence's own rows of the token-major tensor
        r0 = int(p.cu_seqlens_kv[b])
        k = dequant(p.k, p.dtype, p.k_scale, 1)[r0:r0 + skv, n2, :]
        v = dequant(p.v, p.dtype, p.v_scale, 1)[r0:r0 + skv, n2, :]
        return k, v
    nblk = -(-skv // 128)
    pages = torch.as_tensor(p.block_table[b, :nblk].astype(np.int64))
    k = dequant(p.k, p.dtype, p.k_scale, 2)[pages, :, n2, :].reshape(-1, 128)[:skv]
    v = dequant(p.v, p.dtype, p.v_scale, 2)[pages, :, n2, :].reshape(-1, 128)[:skv]
    return k, v


def _sdpa_reference(p):
    """Per row: SDPA over the logical sequence with a boolean mask built from the selection."""
    G = p.num_heads_q // p.num_heads_kv
    q = dequant(p.q, p.dtype, p.q_scale, 1)
    starts = gi.q_block_starts(p.cu_seqlens_q, p.block_x)
    T = int(p.cu_seqlens_q[-1])
    O = np.full((T, p.num_heads_q, 128), np.nan)
    L = np.full((T, p.num_heads_q), np.nan)
    scale = p.scale if p.scale > 0 else 1 / math.sqrt(128)
    for b in range(p.batch):
        c0 = int(p.cu_seqlens_q[b])
        storage = int(p.cu_seqlens_q[b + 1]) - c0
        sq = storage if p.seqused_q is None else int(p.seqused_q[b])
        skv = p.kv_len(b)
        off = 0 if p.mask_mode == 2 else skv - sq
        for n2 in range(p.num_heads_kv):
            k, v = _logical_kv(p, b, n2)
            mask = torch.zeros((sq, skv), dtype=torch.bool)
            for t in range(sq):
                g = starts[b] + t // p.block_x
                cnt = int(p.sparse_block_count[n2, g])
                for j in p.sparse_block_idx[n2, g, :cnt]:
                    if j >= 0:
                        mask[t, 128 * j:128 * (j + 1)] = True
            tt = torch.arange(sq)[:, None] + off
            pp = torch.arange(skv)[None, :]
            if p.mask_mode in (1, 2):
                mask &= pp <= tt
            if p.atten_mask is not None:  # user mask entries inside its extent
                um = torch.as_tensor(user_mask(p)[b if p.atten_mask.shape[0] > 1 else 0])
                r, c = min(sq, um.shape[0]), min(skv, um.shape[1])
                mask[:r, :c] &= um[:r, :c] == 0
            if p.win_left >= 0:
                mask &= pp >= tt - p.win_left
            if p.win_right >= 0:
                mask &= pp <= tt + p.win_right
            for gi_ in range(G):
                h = n2 * G + gi_
                qq = q[c0:c0 + sq, h, :]
                out = torch.nn.functional.scaled_dot_product_attention(
                    qq[None, None], k[None, None], v[None, None], attn_mask=mask[None, None],
                    scale=scale)[0, 0]
                logits = (qq @ k.T) * scale
                lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=1)
                empty = ~mask.any(dim=1)
                out[empty] = 0.0
                O[c0:c0 + sq, h] = out.numpy()
                L[c0:c0 + sq, h] = lse.numpy()
    return O, L


@pytest.mark.parametrize("seed,kw", [
    (1, dict(mask_mode=1)),
    (2, dict(mask_mode=0)),
    (3, dict(mask_mode=1, win_left=100, win_right=0, use_seqused_q=True)),
    (4, dict(mask_mode=0, win_left=50, win_right=20, num_heads_q=8, num_heads_kv=2)),
    (5, dict(mask_mode=1, dtype="fp8", std=0.7)),
    (6, dict(mask_mode=1, dtype="bf16", decode=True, batch=3, block_x=1)),
    (7, dict(mask_mode=1, page_pad=256, use_seqused_q=True, block_x=48)),
])
def test_oracle_matches_sdpa(seed, kw):
    p = gi.random_problem(seed, **kw)
    inp = oracle_inputs(p)
    O, L, done = oa.sparse_attention(inp)
    Or, Lr = _sdpa_reference(p)
    rows = done
    assert rows.sum() > 0
    np.testing.assert_allclose(O[rows], Or[rows], rtol=0, atol=1e-12)
    fin = np.isfinite(Lr[rows])
    assert np.array_equal(fin, np.isfinite(L[rows]))
    np.testing.assert_allclose(L[rows][fin], Lr[rows][fin], rtol=1e-12, atol=1e-12)
    # rows beyond seqused_q are not part of the output
    assert np.isnan(O[~rows]).all()


@pytest.mark.parametrize("seed,kw,keep", [
    (51, dict(mask_mode=1, use_seqused_q=True), True),
    (52, dict(mask_mode=0, win_left=70, win_right=10, num_heads_q=8, num_heads_kv=2), True),
    (53, dict(mask_mode=1, batch=3), False),
    (54, dict(mask_mode=1, dtype="fp8", std=0.7), True),
    (55, dict(mask_mode=1, dtype="bf16", decode=True, batch=4, block_x=1), True),
])
def test_tnd_oracle_matches_sdpa(seed, kw, keep):
    """Token-major key/value: SDPA over each sequence's own rows, with seqused_kv below the
    storage length (dual lengths) or without seqused_kv (keep=False)."""
    p = gi.to_tnd(gi.random_problem(seed, **kw), keep_seqused_kv=keep)
    assert p.cu_seqlens_kv[-1] == p.k.shape[0]
    O, L, done = oa.sparse_attention(oracle_inputs(p))
    Or, Lr = _sdpa_reference(p)
    assert done.sum() > 0
    np.testing.assert_allclose(O[done], Or[done], rtol=0, atol=1e-12)
    fin = np.isfinite(Lr[done])
    assert np.array_equal(fin, np.isfinite(L[done]))
    np.testing.assert_allclose(L[done][fin], Lr[done][fin], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("keep", [True, False])
def test_tnd_equals_paged_bit_identical(keep):
    """Layout independence: the same logical keys give bit-identical results."""
    p = gi.random_problem(56, mask_mode=1, use_seqused_q=True, batch=3, extra_pages=4)
    t = gi.to_tnd(p, keep_seqused_kv=keep, tail_rows=5)
    O1, L1, _ = oa.sparse_attention(oracle_inputs(p))
    O2, L2, _ = oa.sparse_attention(oracle_inputs(t))
    assert np.array_equal(O1, O2, equal_nan=True) and np.array_equal(L1, L2, equal_nan=True)


def test_tnd_rows_of_other_sequences_are_never_used():
    """Poisoning every row outside [cu_kv[b], cu_kv[b] + kv_len[b]) changes nothing."""
    p = gi.to_tnd(gi.random_problem(57, mask_mode=0, batch=3))
    O1, L1, _ = oa.sparse_attention(oracle_inputs(p))
    used = np.zeros(p.k.shape[0], dtype=bool)
    for b in range(p.batch):
        used[int(p.cu_seqlens_kv[b]):int(p.cu_seqlens_kv[b]) + p.kv_len(b)] = True
    k, v = p.k.clone(), p.v.clone()
    k[torch.as_tensor(~used)] = 1000.0
    v[torch.as_tensor(~used)] = float("nan")
    O2, L2, _ = oa.sparse_attention(oracle_inputs(_set(p, k=k, v=v)))
    assert (~used).any()
    assert np.array_equal(O1, O2, equal_nan=True) and np.array_equal(L1, L2, equal_nan=True)


def test_tnd_seqused_kv_above_storage_reads_as_storage():
    p = gi.to_tnd(gi.random_problem(58, mask_mode=1, batch=2))
    st = np.diff(p.cu_seqlens_kv)
    a = oa.sparse_attention(oracle_inputs(_set(p, seqused_kv=st.astype(np.int32))))
    b = oa.sparse_attention(oracle_inputs(_set(p, seqused_kv=(st + 300).astype(np.int32))))
    c = oa.sparse_attention(oracle_inputs(_set(p, seqused_kv=None)))
    for x, y in ((a, b), (a, c)):
        assert np.array_equal(x[0], y[0], equal_nan=True)
        assert np.array_equal(x[1], y[1], equal_nan=True)


@pytest.mark.parametrize("seed,kw,mk", [
    (61, dict(mask_mode=1, use_seqused_q=True), dict(density=0.3, per_batch=True)),
    (62, dict(mask_mode=0, num_heads_q=8, num_heads_kv=2), dict(density=0.6, per_batch=False)),
    (63, dict(mask_mode=2, use_seqused_q=True), dict(density=0.2, per_batch=True, rows=50,
                                                     cols=150)),
    (64, dict(mask_mode=0, win_left=60, win_right=10, dtype="bf16"), dict(density=0.5)),
    (65, dict(mask_mode=1, dtype="fp8", std=0.7, decode=True, batch=3, block_x=1),
     dict(density=0.4)),
])
def test_user_mask_and_top_left_causal_match_sdpa(seed, kw, mk):
    """User attention masks (shared or per sequence, full or partial extent) and mask mode 2
    against SDPA with an independently built boolean mask."""
    p = gi.with_atten_mask(gi.random_problem(seed, **kw), seed, **mk)
    O, L, done = oa.sparse_attention(oracle_inputs(p))
    Or, Lr = _sdpa_reference(p)
    assert done.sum() > 0
    np.testing.assert_allclose(O[done], Or[done], rtol=0, atol=1e-12)
    fin = np.isfinite(Lr[done])
    assert np.array_equal(fin, np.isfinite(L[done]))
    np.testing.assert_allclose(L[done][fin], Lr[done][fin], rtol=1e-12, atol=1e-12)


def test_user_mask_encoding_causal_equals_built_in_causal():
    """A user mask holding exactly the bottom-right causal pattern, with mask mode 0, is
    bit-identical to mask mode 1 (pins the mask's row/column orientation and offset)."""
    p = gi.random_problem(66, mask_mode=1, use_seqused_q=True, batch=3)
    rows = int(np.diff(p.cu_seqlens_q).max())
    cols = max(p.kv_len(b) for b in range(p.batch))
    m = np.zeros((p.batch, rows, cols), dtype=np.uint8)
    for b in range(p.batch):
        sq, skv = int(p.seqused_q[b]), p.kv_len(b)
        t = np.arange(rows)[:, None]
        q = np.arange(cols)[None, :]
        m[b] = np.where(q > t + (skv - sq), 7, 0)
    a = oa.sparse_attention(oracle_inputs(p))
    bm = oa.sparse_attention(oracle_inputs(_set(p, mask_mode=0, atten_mask=m,
                                                atten_mask_cols=cols)))
    assert np.array_equal(a[0], bm[0], equal_nan=True) and np.array_equal(a[1], bm[1],
                                                                           equal_nan=True)


def test_top_left_causal():
    """Mode 2 equals mode 1 when query and KV lengths agree, and a user mask p > t otherwise."""
    p = gi.random_problem(67, mask_mode=1, batch=3)  # kv lengths exceed the query lengths
    same = _set(p, seqused_kv=np.diff(p.cu_seqlens_q).astype(np.int32), kv_storage=None)
    x = oa.sparse_attention(oracle_inputs(same))
    y = oa.sparse_attention(oracle_inputs(_set(same, mask_mode=2)))
    assert np.array_equal(x[0], y[0], equal_nan=True) and np.array_equal(x[1], y[1],
                                                                         equal_nan=True)
    rows = int(np.diff(p.cu_seqlens_q).max())
    cols = max(p.kv_len(b) for b in range(p.batch))
    m = np.where(np.arange(cols)[None, None, :] > np.arange(rows)[None, :, None], 1, 0)
    u = oa.sparse_attention(oracle_inputs(_set(p, mask_mode=0, atten_mask=m.astype(np.uint8),
                                               atten_mask_cols=cols)))
    v = oa.sparse_attention(oracle_inputs(_set(p, mask_mode=2)))
    assert np.array_equal(u[0], v[0], equal_nan=True) and np.array_equal(u[1], v[1],
                                                                         equal_nan=True)
    assert not np.array_equal(v[0], oa.sparse_attention(oracle_inputs(p))[0], equal_nan=True)


@pytest.mark.parametrize("seed", range(10))
def test_oracle_sweep_matches_sdpa(seed):
    """Random combinations of every option against SDPA with an independently built mask."""
    p = gi.sweep_problem(seed, max_len=150)
    O, L, done = oa.sparse_attention(oracle_inputs(p))
    Or, Lr = _sdpa_reference(p)
    np.testing.assert_allclose(O[done], Or[done], rtol=0, atol=1e-12)
    fin = np.isfinite(Lr[done])
    assert np.array_equal(fin, np.isfinite(L[done]))
    np.testing.assert_allclose(L[done][fin], Lr[done][fin], rtol=1e-12, atol=1e-12)


def test_all_causal_blocks_equal_dense_causal():
    """Selecting every causal block with a causal mask equals dense causal attention."""
    p = gi.build_problem("dense", seed=11, q_lens=[300, 130], kv_lens=[300, 130],
                         num_heads_q=4, num_heads_kv=2, block_x=64, top_k=3, dtype="bf16",
                         select=gi.select_all, mask_mode=1, scale=0.05)
    O, L, _ = oa.sparse_attention(oracle_inputs(p))
    q = dequant(p.q, "bf16")
    for b in range(2):
        c0, c1 = int(p.cu_seqlens_q[b]), int(p.cu_seqlens_q[b + 1])
        for h in range(4):
            k, v = _logical_kv(p, b, h // 2)
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[c0:c1, h][None, None], k[None, None], v[None, None], is_causal=True,
                scale=0.05)[0, 0].numpy()
            np.testing.assert_allclose(O[c0:c1, h], ref, atol=1e-12, rtol=0)


def test_dense_equivalent_fp8_small():
    """Same property with e4m3fn inputs and per-head dequant scales."""
    p = gi.build_problem("dense8", seed=12, q_lens=[256], kv_lens=[256], num_heads_q=2,
                         num_heads_kv=2, block_x=128, top_k=2, dtype="fp8",
                         select=gi.select_all, mask_mode=1, scale=1 / math.sqrt(128))
    O, _, _ = oa.sparse_attention(oracle_inputs(p))
    q = dequant(p.q, "fp8", p.q_scale, 1)
    for h in range(2):
        k, v = _logical_kv(p, 0, h)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[:, h][None, None], k[None, None], v[None, None], is_causal=True,
            scale=1 / math.sqrt(128))[0, 0].numpy()
        np.testing.assert_allclose(O[:, h], ref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# invariants and closed forms
# ---------------------------------------------------------------------------

def test_softmax_rows_sum_to_one():
    p = gi.random_problem(21, mask_mode=1, win_left=80)
    inp = oracle_inputs(p)
    for b in range(p.batch):
        for gl in range(2):
            if gl * p.block_x >= inp.sq(b):
                continue
            rows, O, L, w, pos = oa.attention_unit(inp, b, 0, gl, return_weights=True)
            s = w.sum(axis=2)
            nonempty = np.isfinite(L)
            np.testing.assert_allclose(s[nonempty], 1.0, atol=1e-12)
            assert np.all(s[~nonempty] == 0)


def test_page_shuffle_invariance_bit_identical():
    p = gi.random_problem(31, mask_mode=1, extra_pages=5)
    O1, L1, _ = oa.sparse_attention(oracle_inputs(p))
    rng = np.random.default_rng(5)
    perm = rng.permutation(p.num_pages)  # new physical slot of each old page
    inv = np.argsort(perm)
    k2 = p.k[torch.as_tensor(inv)].contiguous()
    v2 = p.v[torch.as_tensor(inv)].contiguous()
    table2 = np.where(p.block_table >= 0, perm[np.maximum(p.block_table, 0)], -1).astype(np.int32)
    import dataclasses
    p2 = dataclasses.replace(p, k=k2, v=v2, block_table=table2)
    O2, L2, _ = oa.sparse_attention(oracle_inputs(p2))
    assert np.array_equal(O1, O2, equal_nan=True) and np.array_equal(L1, L2, equal_nan=True)


def _set(p, **fields):
    import dataclasses
    return dataclasses.replace(p, **fields)


def test_constant_v_gives_constant_output():
    p = gi.random_problem(41, mask_mode=1, dtype="f16")
    v = torch.full_like(p.v, 0.625)
    O, L, done = oa.sparse_attention(oracle_inputs(_set(p, v=v)))
    fin = np.isfinite(L[done])
    Od = O[done]
    np.testing.assert_allclose(Od[fin], 0.625, rtol=0, atol=1e-13)
    assert np.all(Od[~fin] == 0.0)


def test_zero_q_gives_mean_and_log_count():
    p = gi.random_problem(42, mask_mode=1, win_left=70, use_seqused_q=True)
    O, L, done = oa.sparse_attention(oracle_inputs(_set(p, q=torch.zeros_like(p.q))))
    # brute force: enumerate visible positions from the selection by hand
    starts = gi.q_block_starts(p.cu_seqlens_q, p.block_x)
    vv = dequant(p.v, "f16")
    for b in range(p.batch):
        c0 = int(p.cu_seqlens_q[b])
        sq = int(p.seqused_q[b])
        skv = int(p.seqused_kv[b])
        for t in range(sq):
            g = starts[b] + t // p.block_x
            for h in range(p.num_heads_q):
                n2 = h // (p.num_heads_q // p.num_heads_kv)
                vis = []
                for j in p.sparse_block_idx[n2, g, :p.sparse_block_count[n2, g]]:
                    for r in range(128):
                        pos = 128 * int(j) + r
                        d = t + skv - sq
                        if pos < skv and pos <= d and pos >= d - 70:
                            vis.append(vv[p.block_table[b, j], r, n2].numpy())
                if not vis:
                    assert L[c0 + t, h] == -np.inf and np.all(O[c0 + t, h] == 0)
                    continue
                assert abs(L[c0 + t, h] - math.log(len(vis))) < 1e-12
                np.testing.assert_allclose(O[c0 + t, h], np.mean(vis, axis=0), atol=1e-12)


def test_single_visible_key():
    """A one-token window leaves exactly one key: O = v_p and LSE = its logit."""
    p = gi.build_problem("single", seed=51, q_lens=[200], kv_lens=[200], num_heads_q=2,
                         num_heads_kv=1, block_x=32, top_k=2, dtype="f16", select=gi.select_all,
                         mask_mode=1, win_left=0, win_right=0, scale=0.1)
    O, L, _ = oa.sparse_attention(oracle_inputs(p))
    q = dequant(p.q, "f16")
    k, v = _logical_kv(p, 0, 0)
    for t in range(200):
        for h in range(2):
            np.testing.assert_array_equal(O[t, h], v[t].numpy())
            assert abs(L[t, h] - 0.1 * float(q[t, h] @ k[t])) < 1e-12


def test_single_key_identifies_logical_position():
    """With V encoding each key's logical position, a one-key window reads the right page."""
    p = gi.build_problem("pos", seed=52, q_lens=[384], kv_lens=[384], num_heads_q=1,
                         num_heads_kv=1, block_x=64, top_k=3, dtype="f16", select=gi.select_all,
                         mask_mode=1, win_left=0, win_right=0, extra_pages=4)
    v = torch.zeros_like(p.v)
    for j in range(3):
        page = int(p.block_table[0, j])
        v[page, :, 0, 0] = torch.arange(128 * j, 128 * (j + 1), dtype=torch.float16)
    O, _, _ = oa.sparse_attention(oracle_inputs(_set(p, v=v)))
    np.testing.assert_array_equal(O[:, 0, 0], np.arange(384, dtype=np.float64))


def test_hand_worked_three_key_softmax():
    """Logits (0, 0, 1): weights (1, 1, e)/(2+e); LSE = ln(2+e)."""
    p = gi.build_problem("hand", seed=53, q_lens=[1], kv_lens=[3], num_heads_q=1,
                         num_heads_kv=1, block_x=1, top_k=1, dtype="f16", select=gi.select_all,
                         causal_eligible=False, mask_mode=0, scale=1.0, shuffle_pages=False)
    q = torch.zeros_like(p.q)
    q[0, 0, 0] = 1.0
    k = torch.zeros_like(p.k)
    k[0, 2, 0, 0] = 1.0
    v = torch.zeros_like(p.v)
    v[0, 0, 0, 0], v[0, 1, 0, 0], v[0, 2, 0, 0] = 2.0, -4.0, 3.0
    O, L, _ = oa.sparse_attention(oracle_inputs(_set(p, q=q, k=k, v=v)))
    e = math.e
    assert abs(O[0, 0, 0] - (2.0 - 4.0 + 3.0 * e) / (2 + e)) < 1e-15
    assert abs(L[0, 0] - math.log(2 + e)) < 1e-15
    assert np.all(O[0, 0, 1:] == 0)


def test_merge_identity_over_disjoint_selections():
    """Attention over A u B is the LSE-weighted merge of attention over A and over B."""
    p = gi.random_problem(61, mask_mode=1, top_k=4)
    cnt = p.sparse_block_count
    idx = p.sparse_block_idx
    idxA = np.full_like(idx, -1)
    idxB = np.full_like(idx, -1)
    cA = cnt // 2
    cB = cnt - cA
    for h in range(idx.shape[0]):
        for g in range(idx.shape[1]):
            idxA[h, g, :cA[h, g]] = idx[h, g, :cA[h, g]]
            idxB[h, g, :cB[h, g]] = idx[h, g, cA[h, g]:cnt[h, g]]
    O, L, done = oa.sparse_attention(oracle_inputs(p))
    OA, LA, _ = oa.sparse_attention(oracle_inputs(_set(p, sparse_block_idx=idxA,
                                                       sparse_block_count=cA)))
    OB, LB, _ = oa.sparse_attention(oracle_inputs(_set(p, sparse_block_idx=idxB,
                                                       sparse_block_count=cB)))
    Lm = np.logaddexp(LA, LB)
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isfinite(LA), np.exp(LA - Lm), 0.0)
        wb = np.where(np.isfinite(LB), np.exp(LB - Lm), 0.0)
    Om = wa[..., None] * np.nan_to_num(OA) + wb[..., None] * np.nan_to_num(OB)
    fin = np.isfinite(L) & done[:, None]
    np.testing.assert_allclose(O[fin], Om[fin], atol=1e-12)
    np.testing.assert_allclose(L[fin], Lm[fin], atol=1e-12)


def test_packed_gqa_equals_replicated_mha():
    p = gi.random_problem(71, mask_mode=1, num_heads_q=6, num_heads_kv=2)
    G = 3
    O, L, _ = oa.sparse_attention(oracle_inputs(p))
    k = p.k.repeat_interleave(G, dim=2).contiguous()
    v = p.v.repeat_interleave(G, dim=2).contiguous()
    idx = np.repeat(p.sparse_block_idx, G, axis=0)
    cnt = np.repeat(p.sparse_block_count, G, axis=0)
    O2, L2, _ = oa.sparse_attention(oracle_inputs(_set(p, k=k, v=v, num_heads_kv=6,
                                                      sparse_block_idx=idx,
                                                      sparse_block_count=cnt)))
    assert np.array_equal(O, O2, equal_nan=True) and np.array_equal(L, L2, equal_nan=True)


def test_slot_order_changes_only_rounding():
    p = gi.random_problem(81, mask_mode=0, top_k=4)
    O, L, done = oa.sparse_attention(oracle_inputs(p))
    idx = p.sparse_block_idx.copy()
    for h in range(idx.shape[0]):
        for g in range(idx.shape[1]):
            c = p.sparse_block_count[h, g]
            idx[h, g, :c] = idx[h, g, :c][::-1]
    O2, L2, _ = oa.sparse_attention(oracle_inputs(_set(p, sparse_block_idx=idx)))
    np.testing.assert_allclose(O[done], O2[done], atol=1e-13)


def test_pooled_oracle_equals_one_call():
    """The tests' process-pool evaluation of many q-blocks (one q-block per task) gives the
    oracle's own single-call result bit for bit: q-blocks are independent units."""
    from helpers import oracle_rows
    p = gi.random_problem(77, batch=3, max_len=200, block_x=16, mask_mode=1)
    inp = oracle_inputs(p)
    rows = [t for t in range(int(p.cu_seqlens_q[-1])) if t % 3 != 1]
    O1, L1, d1 = oa.sparse_attention(inp, rows=rows)
    idx, O2, L2 = oracle_rows(inp, rows, p.block_x, p.cu_seqlens_q, workers=4)
    assert np.array_equal(np.nonzero(d1)[0], idx) and len(idx) > 0
    assert np.array_equal(O1[d1], O2) and np.array_equal(L1[d1], L2)

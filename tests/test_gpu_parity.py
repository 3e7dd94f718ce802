"""GPU parity of the HIP path against the fp64 oracle, through the C ABI (MI355X only).

Small cases are compared element by element over every row; they span several
32-token tiles, ragged page tails, empty contexts, odd row counts and forced
split counts. The pools' unused slots and the extra fill page hold bf16 NaN,
so a stale-slot leak shows up as a non-finite output.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import Case
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def case(idx, *, batch=2, K=3, hq=4, hkv=1, D=64, P=32, ctx=100, ctx_range=None, wl=-1, wr=-1, outliers=0.0):
    return Case(f"g{idx}", 80, idx, batch=batch, block_size=K, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
                page_size=P, context=ctx, context_range=ctx_range, window_left=wl, window_right=wr,
                outlier_rate=outliers)


def check_full(c, label, **run_kw):
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    out, lse, info = H.run(dc, **run_kw)
    wl = run_kw.get("window_left", c.window_left)
    wr = run_kw.get("window_right", c.window_right)
    ref_out, ref_lse = oracle.attention_case(inp, window_left=wl, window_right=wr)
    res = H.compare(out, lse, ref_out, ref_lse, label=label)
    print(f"{label}: {res} info={info}", flush=True)
    return out, lse, info


def test_cfg1_tiny():
    c = synth.cases_for_config(1)[0]
    check_full(c, "cfg1")


SMALL = [
    # (idx, kwargs)
    (1, dict(batch=1, K=3, hq=4, hkv=1, D=64, P=32, ctx=0)),          # empty context: only block keys
    (2, dict(batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=1000)),       # R = 28, ragged tail
    (3, dict(batch=3, K=3, hq=6, hkv=3, D=64, P=16, ctx_range=(40, 300))),  # R = 6, P = 16, mixed lengths
    (4, dict(batch=2, K=4, hq=10, hkv=2, D=64, P=64, ctx=513)),       # group 5, R = 20
    (5, dict(batch=1, K=7, hq=16, hkv=1, D=64, P=32, ctx=777)),       # R = 112 on D = 64
    (6, dict(batch=2, K=1, hq=16, hkv=1, D=128, P=64, ctx=300)),      # R = 16, D = 128
    (7, dict(batch=2, K=3, hq=16, hkv=1, D=128, P=64, ctx=2100)),     # R = 48
    (8, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=128, ctx=950)),     # R = 112, P = 128
    (9, dict(batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=4096)),       # page-aligned end
    (10, dict(batch=2, K=5, hq=16, hkv=1, D=128, P=16, ctx=1500)),    # R = 80: three row-waves, 16-token pages
    (11, dict(batch=3, K=3, hq=16, hkv=1, D=64, P=16, ctx_range=(30, 700))),  # R = 48 on D = 64, mixed lengths
    (12, dict(batch=1, K=8, hq=16, hkv=1, D=128, P=32, ctx=2222)),    # R = 128: every row block live
]


@pytest.mark.parametrize("idx,kw", SMALL, ids=[f"s{i}" for i, _ in SMALL])
def test_unwindowed_small(idx, kw):
    check_full(case(idx, **kw), f"unwindowed s{idx}")


WSMALL = [
    (21, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=64, ctx=3000, wl=256, wr=-1)),
    (22, dict(batch=3, K=3, hq=64, hkv=4, D=128, P=64, ctx_range=(100, 1500), wl=300, wr=-1, outliers=0.01)),
    (23, dict(batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=500, wl=33, wr=2)),
    (24, dict(batch=2, K=3, hq=16, hkv=1, D=128, P=64, ctx=10, wl=4096, wr=-1)),  # window longer than cache
    (25, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=64, ctx=700, wl=1, wr=-1)),    # self + later keys only
    (26, dict(batch=2, K=5, hq=16, hkv=1, D=128, P=64, ctx=5000, wl=4096, wr=-1)),  # R = 80, window inside
    (27, dict(batch=3, K=7, hq=16, hkv=1, D=64, P=32, ctx_range=(10, 2000), wl=100, wr=3)),  # R = 112, D = 64
]


@pytest.mark.parametrize("idx,kw", WSMALL, ids=[f"w{i}" for i, _ in WSMALL])
def test_windowed_small(idx, kw):
    _, _, info = check_full(case(idx, **kw), f"windowed w{idx}")
    assert info["merge_active"] == 1


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 1000])
def test_split_invariance(splits):
    c = case(30, batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=3000)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    ref_out, ref_lse = oracle.attention_case(inp)
    out, lse, info = H.run(dc, splits=splits)
    H.compare(out, lse, ref_out, ref_lse, label=f"splits={splits}")
    assert info["max_splits"] == min(splits, (3000 + 7 + 31) // 32)
    assert info["combine_launch"] == (1 if info["max_splits"] > 1 else 0)
    base, base_lse, _ = H.run(dc, splits=1)
    # different split counts only reorder fp32 sums: agreement well inside the parity bar
    assert np.abs(out - base).max() <= 4 * H.ulp_bf16(float(np.abs(base).max()))


@pytest.mark.parametrize("waves,groups", [(0, 1), (8, 2)])
@pytest.mark.parametrize("splits", [1, 3, 1000])
def test_split_invariance_shared_tiles(splits, waves, groups):
    c = case(36, batch=2, K=7, hq=16, hkv=1, D=128, P=64, ctx=3000, wl=2000, wr=-1)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    ref_out, ref_lse = oracle.attention_case(inp)
    out, lse, info = H.run(dc, splits=splits, waves=waves)
    assert info["shared_tiles"] == 1 and info["token_groups"] == groups
    assert info["row_waves"] == (7 if groups == 1 else 4)
    H.compare(out, lse, ref_out, ref_lse, label=f"shared splits={splits} groups={groups}")
    base, _, _ = H.run(dc, splits=1, waves=waves)
    assert np.abs(out - base).max() <= 4 * H.ulp_bf16(float(np.abs(base).max()))


@pytest.mark.parametrize("K,waves,row_waves,groups",
                         [(7, 4, 4, 1), (5, 3, 3, 1), (3, 3, 3, 1), (3, 2, 2, 1), (3, 0, 4, 1), (7, 7, 7, 1),
                          (7, 8, 4, 2), (7, 0, 7, 1), (8, 0, 8, 1), (4, 0, 4, 1)])
def test_rows_per_wave_variants(K, waves, row_waves, groups):
    """Every row-blocks-per-wave choice of the shared-tile kernel at D = 128 meets the bar,
    with one token group or two (seven or eight row blocks); four row-waves load one
    16-row half of K or V each (at three row blocks the fourth wave owns no rows)."""
    c = case(37 + K, batch=2, K=K, hq=16, hkv=1, D=128, P=64, ctx=2500, wl=1000, wr=-1)
    inp = synth.make_inputs(c)
    ref_out, ref_lse = oracle.attention_case(inp)
    out, lse, info = H.run(H.upload(inp), waves=waves)
    assert info["shared_tiles"] == 1 and info["row_waves"] == row_waves and info["token_groups"] == groups
    H.compare(out, lse, ref_out, ref_lse, label=f"K={K} waves={waves}")


# Two token groups (seven or eight row blocks at D = 128): odd and even tile counts per unit (the
# second group idles through the last step of an odd one), forced splits, the all-on eight-block
# form, and the size rule that picks them without an override.
TWO_GROUPS = [
    (90, dict(batch=3, K=7, hq=16, hkv=1, D=128, P=32, ctx_range=(0, 2000)), 8),              # unwindowed, ragged
    (91, dict(batch=2, K=7, hq=32, hkv=2, D=128, P=128, ctx=3333, wl=1500, wr=3), 8),         # W_r = 3
    (92, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=16, ctx_range=(100, 2500), wl=64, wr=-1), 8),  # short window
    (93, dict(batch=16, K=7, hq=16, hkv=1, D=128, P=64, ctx=4200, wl=4096, wr=-1), 0),        # 2064 tiles: default
    (94, dict(batch=3, K=8, hq=64, hkv=4, D=128, P=64, ctx_range=(5000, 9000)), 0),          # all on, default
]


@pytest.mark.parametrize("idx,kw,waves", TWO_GROUPS, ids=[f"groups_{i}" for i, *_ in TWO_GROUPS])
def test_two_token_groups(idx, kw, waves):
    _, _, info = check_full(case(idx, **kw), f"groups_{idx}", waves=waves)
    assert info["token_groups"] == 2 and info["row_waves"] == 4
    check_full(case(idx, **kw), f"groups_{idx} splits=3", waves=waves, splits=3)


# Three row blocks (R = 48) as two token groups of four one-block waves, one of them
# rowless: forced here with a wave count above the blocks (automatic for fp8 pools of
# at least 64 tiles per CU, covered in the fp8 tests).
TWO_GROUPS_3 = [
    (95, dict(batch=3, K=3, hq=16, hkv=1, D=128, P=32, ctx_range=(0, 2000))),                 # unwindowed, ragged
    (96, dict(batch=2, K=3, hq=32, hkv=2, D=128, P=128, ctx=3333, wl=1500, wr=1)),            # W_r = 1
    (97, dict(batch=2, K=3, hq=16, hkv=1, D=128, P=16, ctx_range=(100, 2500), wl=64, wr=-1)),  # short window
]


@pytest.mark.parametrize("idx,kw", TWO_GROUPS_3, ids=[f"groups3_{i}" for i, _ in TWO_GROUPS_3])
def test_two_token_groups_three_blocks(idx, kw):
    _, _, info = check_full(case(idx, **kw), f"groups3_{idx}", waves=8)
    assert info["token_groups"] == 2 and info["row_waves"] == 4 and info["waves_per_unit"] == 8
    check_full(case(idx, **kw), f"groups3_{idx} splits=5", waves=8, splits=5)


def test_empty_splits_from_shorter_live_lengths():
    """Plan with long host lengths, run with shorter device lengths: trailing splits get no tiles."""
    c = case(31, batch=2, K=3, hq=4, hkv=1, D=64, P=32, ctx=2000)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    short = inp.seq_lens.copy()
    short[:] = [500, 37]
    dc.seq_lens = torch.from_numpy(short).cuda()
    out, lse, info = H.run(dc, plan_lens=inp.seq_lens, splits=16)
    inp2 = synth.Inputs(c, inp.q, inp.k_pool, inp.v_pool, inp.page_table, short)
    ref_out, ref_lse = oracle.attention_case(inp2)
    H.compare(out, lse, ref_out, ref_lse, label="empty splits")


def test_windowed_full_window_equals_unwindowed():
    c = case(32, batch=2, K=7, hq=16, hkv=1, D=128, P=64, ctx=2048, wl=4096, wr=-1)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    w_out, w_lse, _ = H.run(dc)
    u_out, u_lse, _ = H.run(dc, window_left=-1, window_right=-1)
    ref_out, ref_lse = oracle.attention_case(inp)
    H.compare(w_out, w_lse, ref_out, ref_lse, label="windowed W>=N")
    H.compare(u_out, u_lse, ref_out, ref_lse, label="unwindowed")
    assert np.abs(w_out - u_out).max() <= 2 * H.ulp_bf16(float(np.abs(u_out).max()))


def test_block_of_one_skips_merge_bit_identical():
    c = case(33, batch=3, K=1, hq=16, hkv=1, D=128, P=64, ctx=5000, wl=4096, wr=-1)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    out_a, lse_a, info_a = H.run(dc)
    out_b, lse_b, info_b = H.run(dc, window_right=0)
    assert info_a["merge_active"] == 0 and info_b["merge_active"] == 0
    np.testing.assert_array_equal(out_a, out_b)
    np.testing.assert_array_equal(lse_a, lse_b)
    ref_out, ref_lse = oracle.attention_case(inp)
    H.compare(out_a, lse_a, ref_out, ref_lse, label="K=1 windowed")


def test_page_permutation_and_batch_independence():
    c = case(34, batch=3, K=7, hq=8, hkv=2, D=64, P=32, ctx_range=(200, 900))
    inp = synth.make_inputs(c)
    base, base_lse, _ = H.run(H.upload(inp))
    rng = np.random.default_rng(5)
    perm = rng.permutation(inp.num_pages)
    inv = np.argsort(perm)
    moved = synth.Inputs(c, inp.q, inp.k_pool[perm].copy(), inp.v_pool[perm].copy(),
                         inv[inp.page_table].astype(np.int32), inp.seq_lens)
    out, lse, _ = H.run(H.upload(moved))
    np.testing.assert_array_equal(out, base)
    np.testing.assert_array_equal(lse, base_lse)
    one = Case("g34b", 80, 34, batch=1, block_size=7, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
               context=int(inp.seq_lens[1]) - 7)
    single = synth.Inputs(one, inp.q[1:2].copy(), inp.k_pool, inp.v_pool, inp.page_table[1:2].copy(),
                          inp.seq_lens[1:2].copy())
    out1, lse1, _ = H.run(H.upload(single))
    ref_out, ref_lse = oracle.attention_case(single)
    H.compare(out1, lse1, ref_out, ref_lse, label="request alone")
    H.compare(base[1:2], base_lse[1:2], ref_out, ref_lse, label="request in batch")


def test_workspace_canary_and_no_nan_leak():
    c = case(35, batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=1234)
    inp = synth.make_inputs(c)
    assert (inp.k_pool[-1] == synth.BF16_NAN).all()
    out, lse, _ = H.run(H.upload(inp), canary=True)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


# 256-token pages: the size of a target model's pool when the draft context lives in it.
PAGES_256 = [
    (60, dict(batch=3, K=7, hq=8, hkv=2, D=64, P=256, ctx_range=(0, 1500))),                 # streaming
    (61, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=256, ctx=2000, wl=300, wr=-1)),          # shared tiles
    (62, dict(batch=2, K=3, hq=16, hkv=1, D=128, P=256, ctx_range=(200, 900), wl=4096, wr=1)),
    (63, dict(batch=1, K=16, hq=2, hkv=1, D=64, P=256, ctx=255)),                          # block across a page edge
]


@pytest.mark.parametrize("idx,kw", PAGES_256, ids=[f"p256_{i}" for i, _ in PAGES_256])
def test_pages_of_256_tokens(idx, kw):
    check_full(case(idx, **kw), f"p256_{idx}")
    check_full(case(idx, **kw), f"p256_{idx} splits=3", splits=3)


# More than 128 query rows per kv head: row groups of at most 128 rows, each its own unit.
ROW_GROUPS = [
    (80, dict(batch=2, K=16, hq=16, hkv=1, D=128, P=64, ctx=900)),                          # R = 256: 2 x 128
    (81, dict(batch=2, K=9, hq=32, hkv=2, D=128, P=32, ctx_range=(0, 700), wl=200, wr=-1)),  # R = 144, ragged
    (82, dict(batch=1, K=16, hq=40, hkv=2, D=64, P=16, ctx=300, wl=64, wr=3)),              # R = 320: 3 groups
    (83, dict(batch=3, K=12, hq=24, hkv=2, D=64, P=128, ctx_range=(10, 500))),              # R = 144 at D = 64
]


@pytest.mark.parametrize("idx,kw", ROW_GROUPS, ids=[f"rows_{i}" for i, _ in ROW_GROUPS])
def test_more_than_128_rows(idx, kw):
    _, _, info = check_full(case(idx, **kw), f"rows_{idx}")
    assert info["row_groups"] > 1
    check_full(case(idx, **kw), f"rows_{idx} splits=3", splits=3)


# The split combine packs 256 / (D / 4 * SL) output rows into a workgroup, with SL split
# streams per row chosen from the largest split count (1 up to 4 splits, 2 up to 8, ...,
# at most 16 at D = 64 and 8 at D = 128). Each case forces a split count that selects one
# SL, with a row count that leaves the last workgroup partly empty; the mixed-length
# cases give requests different split counts (the per-pair table instead of a uniform S).
COMBINE = [
    # (idx, splits, kwargs)
    (70, 2, dict(batch=3, K=3, hq=10, hkv=2, D=64, P=32, ctx=900)),              # SL 1, 90 rows over 16 per group
    (71, 6, dict(batch=2, K=7, hq=6, hkv=2, D=64, P=32, ctx=3000)),              # SL 2, 84 rows over 8
    (72, 30, dict(batch=1, K=5, hq=3, hkv=3, D=64, P=16, ctx=4000)),             # SL 8, 15 rows over 2
    (73, 60, dict(batch=1, K=7, hq=8, hkv=2, D=64, P=32, ctx=5000)),             # SL 16
    (74, 130, dict(batch=1, K=3, hq=4, hkv=1, D=64, P=32, ctx=8000)),            # SL 16, 33 splits per stream
    (75, 3, dict(batch=3, K=1, hq=12, hkv=1, D=128, P=64, ctx=2500)),            # SL 1 at D = 128, 36 rows over 8
    (76, 40, dict(batch=2, K=1, hq=16, hkv=1, D=128, P=64, ctx=3000)),           # SL 8 at D = 128
    (79, 7, dict(batch=2, K=3, hq=10, hkv=2, D=128, P=64, ctx=2000)),            # SL 2 at D = 128, 60 rows over 4
    (77, 9, dict(batch=3, K=5, hq=6, hkv=2, D=64, P=32, ctx_range=(20, 600))),   # mixed split counts, SL 4
    (78, 3, dict(batch=3, K=3, hq=48, hkv=3, D=128, P=64, ctx_range=(0, 700), wl=200, wr=-1)),  # shared tiles
]


@pytest.mark.parametrize("idx,splits,kw", COMBINE, ids=[f"comb{i}" for i, _, _ in COMBINE])
def test_combine_row_packing(idx, splits, kw):
    _, _, info = check_full(case(idx, **kw), f"combine {idx} splits={splits}", splits=splits)
    assert info["combine_launch"] == 1

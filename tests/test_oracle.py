"""Pins for the fp64 oracle: brute force, closed forms, identities (CPU only).

None of these re-type the oracle's loops. Each pins it to something else:
dense library routines on tiny inputs, values derived by hand for special
inputs, or identities the pages state (windowed = causal + merge, K = 1 is a
plain decode, a window covering everything is the unwindowed form).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import Case
from tests import bruteforce

LOG2E = 1.0 / math.log(2.0)


def tiny(batch=1, K=3, hq=4, hkv=1, D=16, P=8, ctx=20, ctx_range=None, wl=-1, wr=-1, idx=0, scale=0.0):
    return Case(f"tiny{idx}", 90, idx, batch=batch, block_size=K, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
                page_size=P, context=ctx, context_range=ctx_range, window_left=wl, window_right=wr, sm_scale=scale)


def run(inp, **kw):
    return oracle.attention_case(inp, threads=2, **kw)


GRID = []
_i = 0
for ctx in (0, 1, 31, 32, 33, 70):
    for K in (1, 2, 3, 7):
        for P in (16, 32):
            for (hq, hkv) in ((1, 1), (4, 1), (8, 2), (5, 1)):
                _i += 1
                if _i % 3:  # a deterministic third of the cross product keeps the CPU suite short
                    continue
                GRID.append((ctx, K, P, hq, hkv))


@pytest.mark.parametrize("ctx,K,P,hq,hkv", GRID)
def test_unwindowed_matches_bruteforce(ctx, K, P, hq, hkv):
    inp = synth.make_inputs(tiny(batch=2, K=K, hq=hq, hkv=hkv, D=16, P=P, ctx=ctx, idx=ctx * 100 + K * 10 + P))
    out, lse = run(inp)
    ref_out, ref_lse = bruteforce.attention(inp)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


WGRID = [(ctx, K, W, wr) for ctx in (0, 5, 40) for K in (1, 3, 7) for W in (1, 2, 3, 8, 200) for wr in (-1, 0, 1)
         if (ctx + K + W + wr) % 2 == 0]


@pytest.mark.parametrize("ctx,K,W,wr", WGRID)
def test_windowed_matches_bruteforce(ctx, K, W, wr):
    inp = synth.make_inputs(tiny(batch=2, K=K, hq=4, hkv=2, D=16, P=16, ctx=ctx, wl=W, wr=wr, idx=7 + ctx + K * W))
    for part, name in ((oracle.PART_ALL, "all"), (oracle.PART_CAUSAL, "causal"), (oracle.PART_FUTURE, "future")):
        out, lse = run(inp, part=part)
        ref_out, ref_lse = bruteforce.attention(inp, part=name)
        np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_mixed_lengths_and_library_sdpa():
    """Unequal context lengths; cross-checked against torch's fp64 SDPA with the same boolean mask."""
    case = tiny(batch=3, K=3, hq=8, hkv=2, D=32, P=16, ctx_range=(10, 90), idx=3)
    inp = synth.make_inputs(case)
    assert len(set(inp.seq_lens.tolist())) > 1
    out, lse = run(inp)
    q = synth.bf16_bits_to_float(inp.q).astype(np.float64)
    for b in range(case.batch):
        n = int(inp.seq_lens[b])
        kd = torch.from_numpy(bruteforce.dense_kv(inp.k_pool, inp.page_table, b, n))
        vd = torch.from_numpy(bruteforce.dense_kv(inp.v_pool, inp.page_table, b, n))
        for h in range(case.num_q_heads):
            hk = h // case.group
            qq = torch.from_numpy(q[b, :, h, :])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq, kd[:, hk][None, None].contiguous(), vd[:, hk][None, None].contiguous(), scale=case.scale)
            np.testing.assert_allclose(out[b, :, h, :], ref[0, 0].numpy(), rtol=1e-10, atol=1e-12)


# Key-set sizes derived by hand from the window reading (W keys including the
# query's own position, W_r later keys): p = N - K + i, lo = max(0, p - W + 1),
# hi = min(N - 1, p + W_r) with -1 meaning "no limit"; |S| = hi - lo + 1.
#   (N, K, W, W_r): [(lo, hi) for i = 0..K-1]
KEYSETS = {
    (259, 3, -1, -1): [(0, 258)] * 3,            # unwindowed: every key
    (10, 3, 4, -1): [(4, 9), (5, 9), (6, 9)],     # p = 7, 8, 9
    (10, 3, 4, 0): [(4, 7), (5, 8), (6, 9)],      # causal window only
    (10, 3, 4, 1): [(4, 8), (5, 9), (6, 9)],      # one later key where it exists
    (5, 3, 100, -1): [(0, 4)] * 3,                # window longer than the cache
    (5, 3, 1, 0): [(2, 2), (3, 3), (4, 4)],       # self only
    (3, 3, 2, -1): [(0, 2), (0, 2), (1, 2)],      # empty context, p = 0, 1, 2
    (1, 1, -1, -1): [(0, 0)],                     # a single key
}


@pytest.mark.parametrize("key", list(KEYSETS))
def test_zero_query_gives_uniform_average(key):
    """q = 0 makes every score 0: out is the plain mean of V over S and lse2 = log2 |S|."""
    N, K, W, wr = key
    case = tiny(batch=1, K=K, hq=2, hkv=1, D=8, P=4, ctx=N - K, wl=W, wr=wr, idx=11)
    inp = synth.make_inputs(case)
    inp.q[...] = 0
    out, lse = run(inp)
    vd = bruteforce.dense_kv(inp.v_pool, inp.page_table, 0, N)
    for i, (lo, hi) in enumerate(KEYSETS[key]):
        for h in range(2):
            assert lse[0, i, h] == pytest.approx(math.log2(hi - lo + 1), abs=1e-13)
            np.testing.assert_allclose(out[0, i, h], vd[lo:hi + 1, 0].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_constant_values_and_equal_keys():
    case = tiny(batch=2, K=3, hq=4, hkv=2, D=16, P=8, ctx=37, idx=12)
    inp = synth.make_inputs(case)
    inp.v_pool[...] = 0x3FC0  # 1.5 everywhere, fill page included: out must be exactly 1.5
    out, _ = run(inp)
    np.testing.assert_allclose(out, 1.5, rtol=0, atol=1e-13)
    inp = synth.make_inputs(case)
    inp.k_pool[...] = inp.k_pool[0, 0, 0, :]  # all keys equal: softmax is uniform
    out, lse = run(inp)
    q = synth.bf16_bits_to_float(inp.q).astype(np.float64)
    k0 = synth.bf16_bits_to_float(inp.k_pool[0, 0, 0, :]).astype(np.float64)
    n = int(inp.seq_lens[0])
    for b in range(2):
        vd = bruteforce.dense_kv(inp.v_pool, inp.page_table, b, n)
        for h in range(4):
            s = case.scale * float(q[b, 0, h] @ k0)
            assert lse[b, 0, h] == pytest.approx(s * LOG2E + math.log2(n), rel=1e-12)
            np.testing.assert_allclose(out[b, 0, h], vd[:, h // 2].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_single_key_and_two_key_sigmoid():
    case = tiny(batch=1, K=1, hq=1, hkv=1, D=16, P=8, ctx=0, idx=13)
    inp = synth.make_inputs(case)
    out, lse = run(inp)
    q = synth.bf16_bits_to_float(inp.q[0, 0, 0]).astype(np.float64)
    k = bruteforce.dense_kv(inp.k_pool, inp.page_table, 0, 1)[0, 0]
    v = bruteforce.dense_kv(inp.v_pool, inp.page_table, 0, 1)[0, 0]
    np.testing.assert_array_equal(out[0, 0, 0], v)
    assert lse[0, 0, 0] == pytest.approx(case.scale * float(q @ k) * LOG2E, rel=1e-14)

    case = tiny(batch=1, K=2, hq=1, hkv=1, D=16, P=8, ctx=0, idx=14)
    inp = synth.make_inputs(case)
    out, lse = run(inp)
    q = synth.bf16_bits_to_float(inp.q[0, :, 0]).astype(np.float64)
    kd = bruteforce.dense_kv(inp.k_pool, inp.page_table, 0, 2)[:, 0]
    vd = bruteforce.dense_kv(inp.v_pool, inp.page_table, 0, 2)[:, 0]
    for i in range(2):
        s0, s1 = case.scale * (q[i] @ kd[0]), case.scale * (q[i] @ kd[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(out[0, i, 0], w0 * vd[0] + (1 - w0) * vd[1], rtol=1e-12, atol=1e-14)
        assert lse[0, i, 0] == pytest.approx(math.log2(math.exp(s0) + math.exp(s1)), rel=1e-13)


def test_merge_closed_forms():
    rng = np.random.default_rng(0)
    a, b = rng.normal(size=(5, 8)), rng.normal(size=(5, 8))
    la = rng.normal(size=5)
    out, lse = oracle.merge(a, la, b, la.copy())
    np.testing.assert_allclose(out, (a + b) / 2, rtol=1e-14)
    np.testing.assert_allclose(lse, la + 1.0, rtol=1e-14)
    out, lse = oracle.merge(a, la, b, np.full(5, -np.inf))
    np.testing.assert_array_equal(out, a)
    np.testing.assert_array_equal(lse, la)
    lb = la + np.log2(3.0)  # weights 1/4 and 3/4
    out, lse = oracle.merge(a, la, b, lb)
    np.testing.assert_allclose(out, 0.25 * a + 0.75 * b, rtol=1e-13)
    np.testing.assert_allclose(lse, la + 2.0, rtol=1e-13)


@pytest.mark.parametrize("W,wr", [(1, -1), (4, -1), (9, 2), (64, 0), (300, -1)])
def test_windowed_is_causal_merged_with_future(W, wr):
    """PR #21130's decomposition: causal windowed decode, then the LSE merge of the later block keys."""
    case = tiny(batch=2, K=7, hq=8, hkv=2, D=16, P=16, ctx=50, wl=W, wr=wr, idx=15)
    inp = synth.make_inputs(case)
    direct = run(inp)
    oc, lc = run(inp, part=oracle.PART_CAUSAL)
    of, lf = run(inp, part=oracle.PART_FUTURE)
    out, lse = oracle.merge(oc, lc, of, lf)
    np.testing.assert_allclose(out, direct[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, direct[1], rtol=1e-12)


def test_full_window_equals_unwindowed():
    case = tiny(batch=2, K=7, hq=8, hkv=2, D=16, P=16, ctx=60, wl=4096, wr=-1, idx=16)
    inp = synth.make_inputs(case)
    w = run(inp)
    u = run(inp, window_left=-1, window_right=-1)
    np.testing.assert_array_equal(w[0], u[0])
    np.testing.assert_array_equal(w[1], u[1])


def test_block_of_one_is_plain_decode():
    """K = 1: nothing follows the query, so the windowed form is the causal decode (merge skipped)."""
    case = tiny(batch=3, K=1, hq=4, hkv=1, D=16, P=8, ctx=45, wl=16, wr=-1, idx=17)
    inp = synth.make_inputs(case)
    w = run(inp)
    c = run(inp, part=oracle.PART_CAUSAL)
    f = run(inp, part=oracle.PART_FUTURE)
    np.testing.assert_array_equal(w[0], c[0])
    np.testing.assert_array_equal(w[1], c[1])
    assert np.all(f[1] == -np.inf)
    # and the unwindowed K = 1 form is a single-query decode over all N keys
    u = run(inp, window_left=-1, window_right=-1)
    ref = bruteforce.attention(inp, window_left=-1, window_right=-1)
    np.testing.assert_allclose(u[0], ref[0], rtol=1e-12, atol=1e-13)


def test_page_permutation_invariance():
    case = tiny(batch=2, K=3, hq=4, hkv=1, D=16, P=8, ctx=40, idx=18)
    inp = synth.make_inputs(case)
    base = run(inp)
    rng = np.random.default_rng(1)
    perm = rng.permutation(inp.k_pool.shape[0])
    inv = np.argsort(perm)
    inp.k_pool = inp.k_pool[perm].copy()
    inp.v_pool = inp.v_pool[perm].copy()
    inp.page_table = inv[inp.page_table].astype(np.int32)
    moved = run(inp)
    np.testing.assert_array_equal(base[0], moved[0])
    np.testing.assert_array_equal(base[1], moved[1])


def test_gqa_replication():
    """Repeating each kv head g times and using Hq kv heads gives the same result."""
    case = tiny(batch=2, K=3, hq=8, hkv=2, D=16, P=8, ctx=30, idx=19)
    inp = synth.make_inputs(case)
    base = run(inp)
    g = case.group
    inp.k_pool = np.repeat(inp.k_pool, g, axis=1)
    inp.v_pool = np.repeat(inp.v_pool, g, axis=1)
    rep = oracle.attention(inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, block_size=3,
                           num_q_heads=8, num_kv_heads=8, head_dim=16, page_size=8, sm_scale=case.scale, threads=2)
    np.testing.assert_array_equal(base[0], rep[0])
    np.testing.assert_array_equal(base[1], rep[1])


def test_batch_independence_and_pair_selection():
    case = tiny(batch=3, K=3, hq=4, hkv=2, D=16, P=8, ctx_range=(5, 40), idx=20)
    inp = synth.make_inputs(case)
    full = run(inp)
    part = run(inp, pairs=[(1, 0), (2, 1)])
    np.testing.assert_array_equal(part[0][1, :, 0:2], full[0][1, :, 0:2])
    np.testing.assert_array_equal(part[0][2, :, 2:4], full[0][2, :, 2:4])
    assert np.isnan(part[0][0]).all()
    # request 1 alone, with its own page-table row, gives the same rows
    sub = oracle.attention(inp.q[1:2], inp.k_pool, inp.v_pool, inp.page_table[1:2], inp.seq_lens[1:2],
                           block_size=3, num_q_heads=4, num_kv_heads=2, head_dim=16, page_size=8,
                           sm_scale=case.scale, threads=2)
    np.testing.assert_array_equal(sub[0][0], full[0][1])


def test_rejects_invalid_arguments():
    case = tiny(batch=1, K=3, hq=4, hkv=1, D=16, P=8, ctx=10, idx=21)
    inp = synth.make_inputs(case)
    with pytest.raises(ValueError):
        oracle.attention(inp.q, inp.k_pool, inp.v_pool, inp.page_table, np.array([2], np.int32), block_size=3,
                         num_q_heads=4, num_kv_heads=1, head_dim=16, page_size=8, sm_scale=0.25)
    bad = inp.page_table.copy()
    bad[0, 0] = inp.k_pool.shape[0]
    with pytest.raises(ValueError):
        oracle.attention(inp.q, inp.k_pool, inp.v_pool, bad, inp.seq_lens, block_size=3, num_q_heads=4,
                         num_kv_heads=1, head_dim=16, page_size=8, sm_scale=0.25)


def test_bf16_widening():
    assert oracle.bf16_to_double(0x3F80) == 1.0
    assert oracle.bf16_to_double(0xC000) == -2.0
    assert oracle.bf16_to_double(0x0001) == 2.0 ** -133
    assert oracle.bf16_to_double(0x7F80) == math.inf
    assert oracle.bf16_to_double(0x3FC0) == 1.5


def test_planted_mistakes_are_caught(monkeypatch):
    """A wrong scale, sign or off-by-one window in a copy of the inputs shows up in the pins above."""
    case = tiny(batch=1, K=3, hq=4, hkv=1, D=16, P=8, ctx=20, wl=4, wr=-1, idx=22)
    inp = synth.make_inputs(case)
    ref_out, ref_lse = bruteforce.attention(inp)
    # an off-by-one window (W + 1 keys) must disagree with the brute force
    out, lse = run(inp, window_left=5)
    assert np.abs(lse - ref_lse).max() > 1e-3
    # a dropped scale must disagree
    out2, lse2 = oracle.attention(inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, block_size=3,
                                  num_q_heads=4, num_kv_heads=1, head_dim=16, page_size=8, sm_scale=1.0,
                                  window_left=4, threads=2)
    assert np.abs(out2 - ref_out).max() > 1e-3

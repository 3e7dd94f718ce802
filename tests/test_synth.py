"""The seeded input generator: determinism, layout and distribution (CPU only)."""
import numpy as np

import synth
from synth.configs import Case, all_cases


def test_case_inventory():
    cases = all_cases()
    by_cfg = {}
    for c in cases:
        by_cfg[c.cfg] = by_cfg.get(c.cfg, 0) + 1
    assert by_cfg == {1: 1, 2: 12, 3: 8, 4: 27, 5: 2}
    assert len({c.name for c in cases}) == 50
    assert len({c.seed for c in cases}) == 50
    c1 = cases[0]
    assert (c1.batch, c1.block_size, c1.num_q_heads, c1.num_kv_heads, c1.head_dim, c1.page_size) == (1, 3, 4, 1, 64, 32)
    assert c1.rows == 12 and c1.scale == 0.125


def test_deterministic_and_disjoint_pages():
    case = Case("t", 91, 0, batch=4, block_size=7, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
                context_range=(100, 400))
    a = synth.make_inputs(case)
    b = synth.make_inputs(case)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.k_pool, b.k_pool)
    np.testing.assert_array_equal(a.page_table, b.page_table)
    used = []
    for r in range(case.batch):
        n = int(a.seq_lens[r])
        np_ = (n + 31) // 32
        used.extend(a.page_table[r, :np_].tolist())
        assert (a.page_table[r, np_:] == a.num_pages - 1).all()
    assert len(used) == len(set(used)) == a.num_pages - 1
    assert sorted(used) != used  # shuffled
    # unused slots and the fill page hold bf16 NaN
    assert (a.k_pool[-1] == synth.BF16_NAN).all()
    r0 = int(a.seq_lens[0])
    last = a.page_table[0, (r0 - 1) // 32]
    if r0 % 32:
        assert (a.v_pool[last, :, r0 % 32:, :] == synth.BF16_NAN).all()


def test_normal_moments_and_outliers():
    case = Case("t", 92, 0, batch=2, block_size=3, num_q_heads=4, num_kv_heads=4, head_dim=128, page_size=64,
                context=4000, outlier_rate=0.01)
    inp = synth.make_inputs(case)
    v = synth.bf16_bits_to_float(inp.v_pool[:-1]).astype(np.float64)
    v = v[np.isfinite(v)]
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01
    k = synth.bf16_bits_to_float(inp.k_pool[:-1]).astype(np.float64)
    k = k[np.isfinite(k)]
    assert abs(k.std() - 1.0) > 0.05  # 1 % of tokens scaled by 8 lifts the spread
    # q differs from k and v streams
    assert not np.array_equal(inp.q.ravel()[:64], inp.k_pool.ravel()[:64])


def test_dense_block_draws():
    case = Case("t", 92, 1, batch=4, block_size=7, num_q_heads=16, num_kv_heads=2, head_dim=128, page_size=64,
                context=100)
    kb, vb = synth.make_block(case)
    assert kb.shape == vb.shape == (4, 7, 2, 128) and kb.dtype == np.uint16
    kb2, vb2 = synth.make_block(case)
    assert np.array_equal(kb, kb2) and np.array_equal(vb, vb2)
    q = synth.make_q(case)
    for a in (kb, vb):
        x = synth.bf16_bits_to_float(a).astype(np.float64)
        assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05
    # three different streams
    assert not np.array_equal(kb.ravel()[:64], vb.ravel()[:64])
    assert not np.array_equal(kb.ravel()[:64], q.ravel()[:64])
    # the query stream is the generic normal fill of tensor 1
    q2 = np.empty_like(q)
    synth._load().synth_fill_normal(case.seed, 1, q2.size, q2.ctypes.data, 3)
    assert np.array_equal(q, q2)


def test_bf16_rounding_is_nearest_even():
    lib = synth._load()
    assert lib.synth_bf16_from_double(1.0) == 0x3F80
    assert lib.synth_bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80  # tie to even
    assert lib.synth_bf16_from_double(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie to even (up)
    assert lib.synth_bf16_from_double(-2.5) == 0xC020

"""GPU parity of the dense-block form and the fused append (MI355X only).

The block's keys and values come from dense bf16 arrays. The cache's own block
slots are poisoned with NaN to prove they are not read; the oracle reads the same
arrays. With append, the cache's block slots must afterwards hold exactly the
oracle's encoding of the arrays (bf16, or saturating E4M3 by nearest-even, after
the fp32 division by the pool scale), every other cache byte must be unchanged,
and a plain forward over the updated cache must match the oracle.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_draft_paged_amd as ba
import synth
from synth.configs import Case, fp8_variant
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def bcase(idx, *, fp8=False, batch=2, K=3, hq=4, hkv=1, D=64, P=32, ctx=100, ctx_range=None, wl=-1, wr=-1,
          ks=None, vs=None):
    """A small case; ks / vs: pool scales (fp8 default 1/16, bf16 default 1)."""
    c = Case(f"bk{idx}", 82, idx, batch=batch, block_size=K, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=P,
             context=ctx, context_range=ctx_range, window_left=wl, window_right=wr)
    if fp8:
        return fp8_variant(c, 0.0625 if ks is None else ks, 0.0625 if vs is None else vs)
    return replace(c, k_scale=1.0 if ks is None else ks, v_scale=1.0 if vs is None else vs)


def block_slots(inp):
    """(page, slot) of every block key, per request."""
    c = inp.case
    out = []
    for b in range(c.batch):
        n = int(inp.seq_lens[b])
        out.append([(int(inp.page_table[b, j // c.page_size]), j % c.page_size) for j in range(n - c.block_size, n)])
    return out


def poison_block_slots(inp):
    nan = synth.FP8_NAN if inp.k_pool.dtype == np.uint8 else synth.BF16_NAN
    for row in block_slots(inp):
        for page, slot in row:
            inp.k_pool[page, :, slot, :] = nan
            inp.v_pool[page, :, slot, :] = nan


def random_block(c, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    shape = (c.batch, c.block_size, c.num_kv_heads, c.head_dim)
    mk = lambda: torch.from_numpy(rng.normal(0, scale, shape).astype(np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    return mk(), mk()


def run_block(dc, kb, vb, *, append, splits=0, waves=0):
    c = dc.inputs.case
    prm = H.params_for(dc, splits=splits, waves=waves)
    lens = dc.inputs.seq_lens
    nbytes = ba.blockattn_workspace_size(prm, lens)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    plan = ba.blockattn_plan(prm, lens, ws, nbytes)
    out = torch.empty(c.batch, c.block_size, c.num_q_heads, c.head_dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(c.batch, c.block_size, c.num_q_heads, dtype=torch.float32, device="cuda")
    to = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    ba.blockattn_forward_block(plan, dc.q, to(kb), to(vb), dc.k, dc.v, dc.page_table, dc.seq_lens, ws, out, lse,
                               append=append)
    torch.cuda.synchronize()
    plan.destroy()
    return out.float().cpu().numpy(), lse.cpu().numpy()


CASES = [
    (1, dict(batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=1000)),                       # streaming kernel
    (2, dict(batch=3, K=3, hq=6, hkv=3, D=64, P=16, ctx_range=(0, 300))),             # 16-token pages, C = 0 allowed
    (3, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=64, ctx=3000, wl=256, wr=-1)),      # shared tiles, windowed
    (4, dict(batch=2, K=3, hq=16, hkv=1, D=128, P=64, ctx=700, wl=4096, wr=1)),       # two blocks per wave, W_r = 1
    (5, dict(fp8=True, batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=900, ks=0.5, vs=2.0)),  # fp8 cache
    (6, dict(fp8=True, batch=2, K=7, hq=16, hkv=1, D=128, P=64, ctx=2500, wl=1000, wr=-1)),
    (7, dict(batch=1, K=5, hq=4, hkv=1, D=64, P=32, ctx=0)),                          # the block is every key
    # scales that are not powers of two (block probabilities rounded after the 1 / v_scale product)
    (10, dict(fp8=True, batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=600, ks=0.3, vs=-0.7)),
    (11, dict(batch=2, K=5, hq=32, hkv=2, D=128, P=64, ctx=1500, ks=0.37, vs=1.9)),    # bf16 cache with scales
    (12, dict(batch=2, K=16, hq=2, hkv=1, D=64, P=128, ctx=700, wl=300, wr=-1)),      # largest block, 128-token pages
    (13, dict(batch=3, K=16, hq=8, hkv=1, D=128, P=16, ctx_range=(0, 400), wl=50, wr=3)),  # R = 128, 8 row-waves
    (14, dict(fp8=True, batch=2, K=2, hq=48, hkv=2, D=64, P=32, ctx=333, wl=40, wr=0)),   # shared tiles at D = 64, causal
    (15, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=256, ctx=250, wl=1000, wr=-1)),   # 256-token pages, block over an edge
    (16, dict(fp8=True, batch=3, K=5, hq=8, hkv=1, D=64, P=256, ctx_range=(0, 700))),
    (17, dict(batch=2, K=16, hq=16, hkv=1, D=128, P=32, ctx=600, wl=300, wr=-1)),   # R = 256: two row groups
    (18, dict(fp8=True, batch=2, K=9, hq=32, hkv=2, D=64, P=64, ctx_range=(0, 400))),  # R = 144 at D = 64
    # fp8 pools through the streaming kernel at D = 128 (paired contraction layout, two 16-byte K
    # loads per row block): unwindowed R = 16, and windowed R = 30 with mixed lengths
    (19, dict(fp8=True, batch=2, K=2, hq=16, hkv=2, D=128, P=64, ctx=700, ks=0.25, vs=0.5)),
    (20, dict(fp8=True, batch=3, K=3, hq=30, hkv=3, D=128, P=32, ctx_range=(0, 900), wl=200, wr=-1)),
]


@pytest.mark.parametrize("idx,kw", CASES, ids=[f"bk{i}" for i, _ in CASES])
def test_dense_block_reads_the_arrays_not_the_cache(idx, kw):
    c = bcase(idx, **kw)
    inp = synth.make_inputs(c)
    poison_block_slots(inp)
    kb, vb = random_block(c, idx)
    dc = H.upload(inp)
    k_before, v_before = dc.k.clone(), dc.v.clone()
    out, lse = run_block(dc, kb, vb, append=False)
    ref_out, ref_lse = oracle.attention_case(inp, k_block=kb, v_block=vb)
    res = H.compare(out, lse, ref_out, ref_lse, label=f"block bk{idx}")
    print(f"bk{idx}: {res}", flush=True)
    assert torch.equal(dc.k.view(torch.uint8), k_before.view(torch.uint8))
    assert torch.equal(dc.v.view(torch.uint8), v_before.view(torch.uint8))


@pytest.mark.parametrize("splits", [1, 5])
def test_dense_block_split_invariance(splits):
    c = bcase(8, batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=2000)
    inp = synth.make_inputs(c)
    poison_block_slots(inp)
    kb, vb = random_block(c, 8)
    out, lse = run_block(H.upload(inp), kb, vb, append=False, splits=splits)
    ref_out, ref_lse = oracle.attention_case(inp, k_block=kb, v_block=vb)
    H.compare(out, lse, ref_out, ref_lse, label=f"block splits={splits}")


def expected_append(inp, kb, vb):
    """Host copies of the pools with the block stored by the oracle's encoding."""
    c = inp.case
    k, v = inp.k_pool.copy(), inp.v_pool.copy()
    for b, row in enumerate(block_slots(inp)):
        for i, (page, slot) in enumerate(row):
            for h in range(c.num_kv_heads):
                k[page, h, slot, :] = [oracle.encode_kv(c.kv_dtype, c.k_scale, int(x)) for x in kb[b, i, h]]
                v[page, h, slot, :] = [oracle.encode_kv(c.kv_dtype, c.v_scale, int(x)) for x in vb[b, i, h]]
    return k, v


APPEND = [CASES[i] for i in (0, 2, 4, 5, 7, 8, 9, 10, 11, 12, 13, 14, 15)]


@pytest.mark.parametrize("idx,kw", APPEND, ids=[f"bk{i}" for i, _ in APPEND])
def test_fused_append_stores_the_encoded_block(idx, kw):
    c = bcase(idx, **kw)
    inp = synth.make_inputs(c)
    poison_block_slots(inp)
    kb, vb = random_block(c, 100 + idx, scale=3.0)
    want_k, want_v = expected_append(inp, kb, vb)
    dc = H.upload(inp)
    out, lse = run_block(dc, kb, vb, append=True)
    ref_out, ref_lse = oracle.attention_case(inp, k_block=kb, v_block=vb)
    H.compare(out, lse, ref_out, ref_lse, label=f"append bk{idx}")
    got_k = dc.k.view(torch.uint8).cpu().numpy().view(want_k.dtype).reshape(want_k.shape)
    got_v = dc.v.view(torch.uint8).cpu().numpy().view(want_v.dtype).reshape(want_v.shape)
    np.testing.assert_array_equal(got_k, want_k)
    np.testing.assert_array_equal(got_v, want_v)
    # the next step reads the block from the cache like any other key
    after = synth.Inputs(c, inp.q, want_k, want_v, inp.page_table, inp.seq_lens)
    out2, lse2, _ = H.run(H.upload(after))
    ref2_out, ref2_lse = oracle.attention_case(after)
    H.compare(out2, lse2, ref2_out, ref2_lse, label=f"after append bk{idx}")


# Seven and eight (or three) row blocks at D = 128 as two token groups (waves_override 8 or a large batch):
# the block tile is consumed by the first group only, the append by every wave.
TWO_GROUPS = [
    (30, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=64, ctx=2500, wl=1000, wr=-1), 8, False),
    (31, dict(fp8=True, batch=3, K=7, hq=16, hkv=1, D=128, P=32, ctx_range=(0, 900)), 8, True),
    (32, dict(batch=2, K=7, hq=32, hkv=2, D=128, P=64, ctx=1300, wl=700, wr=2), 8, True),
    (33, dict(batch=16, K=8, hq=16, hkv=1, D=128, P=64, ctx=4100, wl=4096, wr=-1), 0, False),
    # three row blocks: two groups of four one-block waves, one rowless
    (34, dict(fp8=True, batch=3, K=3, hq=16, hkv=1, D=128, P=32, ctx_range=(0, 900)), 8, True),
    (35, dict(batch=2, K=3, hq=32, hkv=2, D=128, P=64, ctx=1300, wl=700, wr=2), 8, False),
]


@pytest.mark.parametrize("idx,kw,waves,append", TWO_GROUPS, ids=[f"bk{i}" for i, *_ in TWO_GROUPS])
def test_dense_block_and_append_with_two_token_groups(idx, kw, waves, append):
    c = bcase(idx, **kw)
    inp = synth.make_inputs(c)
    poison_block_slots(inp)
    kb, vb = random_block(c, 200 + idx, scale=2.0)
    want_k, want_v = expected_append(inp, kb, vb) if append else (inp.k_pool, inp.v_pool)
    dc = H.upload(inp)
    prm = H.params_for(dc, waves=waves)
    info = ba.blockattn_plan(prm, inp.seq_lens, None).info()
    assert info["token_groups"] == 2 and info["row_waves"] == 4
    out, lse = run_block(dc, kb, vb, append=append, waves=waves)
    ref_out, ref_lse = oracle.attention_case(inp, k_block=kb, v_block=vb)
    H.compare(out, lse, ref_out, ref_lse, label=f"two groups bk{idx}")
    got_k = dc.k.view(torch.uint8).cpu().numpy().view(want_k.dtype).reshape(want_k.shape)
    got_v = dc.v.view(torch.uint8).cpu().numpy().view(want_v.dtype).reshape(want_v.shape)
    np.testing.assert_array_equal(got_k, want_k)
    np.testing.assert_array_equal(got_v, want_v)


def test_append_encoding_of_special_values():
    """Ties, saturation, subnormals and signed zeros through the kernels' E4M3 encoder, bit for bit."""
    c = bcase(9, fp8=True, batch=1, K=16, hq=1, hkv=1, D=64, P=16, ctx=40, ks=1.0, vs=0.25)
    inp = synth.make_inputs(c)
    e4 = [oracle.fp8_e4m3_to_double(x) for x in range(0x7F)]
    vals = []
    for a, b in zip(e4[:-1], e4[1:]):
        vals += [a, (a + b) / 2, -((a + b) / 2)]  # codes, and midpoints between neighbours (ties)
    vals += [448.0, 460.0, 464.0, 470.0, 1e4, -1e4, 0.0, -0.0, 2.0 ** -12, -(2.0 ** -11), 3 * 2.0 ** -10]
    vals = np.resize(np.array(vals, dtype=np.float32), 16 * 64)
    bits = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kb = bits.reshape(1, 16, 1, 64).copy()
    vb = np.roll(bits, 17).reshape(1, 16, 1, 64).copy()
    want_k, want_v = expected_append(inp, kb, vb)
    dc = H.upload(inp)
    run_block(dc, kb, vb, append=True)
    got_k = dc.k.cpu().numpy().reshape(want_k.shape)
    got_v = dc.v.cpu().numpy().reshape(want_v.shape)
    np.testing.assert_array_equal(got_k, want_k)
    np.testing.assert_array_equal(got_v, want_v)


@pytest.mark.parametrize("ks,vs", [(0.997, 0.75), (1.01, 7.0), (0.5, 0.0625)])
def test_append_bf16_special_values(ks, vs):
    """The bf16 encoder at its corners, bit for bit with the oracle: quotients on both sides of
    the overflow midpoint (rounded to infinity past it), +-inf, NaNs of either sign and any
    payload (all become 0x7FC0), subnormals, signed zeros and the smallest normal."""
    c = bcase(21, batch=1, K=16, hq=1, hkv=1, D=64, P=16, ctx=40, ks=ks, vs=vs)
    inp = synth.make_inputs(c)
    special = [0x7F7F, 0xFF7F, 0x7F7E, 0xFF7E, 0x7F7D, 0x7F70, 0x7F00, 0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81,
               0xFF81, 0x7FFF, 0xFFFF, 0x7FA5, 0x0001, 0x8001, 0x0003, 0x007F, 0x8040, 0x0080, 0x8080, 0x0000,
               0x8000, 0x3F80, 0xBF80, 0x3F81, 0x4049]
    rng = np.random.default_rng(21)
    top = (rng.integers(0x7F00, 0x7F80, 512, dtype=np.uint32) | (rng.integers(0, 2, 512, dtype=np.uint32) << 15))
    bits = np.resize(np.concatenate([np.array(special, np.uint32), top]).astype(np.uint16), 16 * 64)
    kb = bits.reshape(1, 16, 1, 64).copy()
    vb = np.roll(bits, 29).reshape(1, 16, 1, 64).copy()
    want_k, want_v = expected_append(inp, kb, vb)
    assert ((want_k & 0x7FFF) == 0x7F80).any() and (want_k == 0x7FC0).any()
    if 0.99 < ks < 1:  # quotients on both sides of the overflow midpoint
        assert ((want_k & 0x7FFF) == 0x7F7F).any() or ((want_k & 0x7FFF) == 0x7F7E).any()
    dc = H.upload(inp)
    run_block(dc, kb, vb, append=True)  # outputs are NaN here (the block holds NaN and inf): only the cache counts
    got_k = dc.k.view(torch.int16).cpu().numpy().view(np.uint16).reshape(want_k.shape)
    got_v = dc.v.view(torch.int16).cpu().numpy().view(np.uint16).reshape(want_v.shape)
    np.testing.assert_array_equal(got_k, want_k)
    np.testing.assert_array_equal(got_v, want_v)

"""Pins for the dense block keys and the append encoding in the oracle (CPU only).

The block keys may come from dense bf16 arrays instead of the cache (the
dense-suffix form); appending stores them into the cache encoded for its
element type and scale. The oracle's encoder is held to torch's fp32 division
and its bf16 / float8_e4m3fn casts; the dense block to identities (arrays equal
to the cache give the cache's result exactly; writing the arrays into a bf16
cache gives the same result) and to the brute force.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import Case, fp8_variant
from tests import bruteforce


def tiny(idx, *, fp8=False, batch=2, K=3, hq=4, hkv=1, D=16, P=8, ctx=20, ctx_range=None, wl=-1, wr=-1,
         ks=0.0625, vs=0.0625):
    c = Case(f"blk{idx}", 92, idx, batch=batch, block_size=K, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
             page_size=P, context=ctx, context_range=ctx_range, window_left=wl, window_right=wr)
    return fp8_variant(c, ks, vs) if fp8 else c


def random_bf16(rng, shape, scale=1.0):
    x = torch.from_numpy(rng.normal(0, scale, shape).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def block_of_cache(inp):
    """The cache's own block keys/values as bf16 bits [B, K, Hkv, D] (bf16 pools only)."""
    c = inp.case
    kb = np.empty((c.batch, c.block_size, c.num_kv_heads, c.head_dim), np.uint16)
    vb = np.empty_like(kb)
    for b in range(c.batch):
        n = int(inp.seq_lens[b])
        for i in range(c.block_size):
            j = n - c.block_size + i
            page, slot = inp.page_table[b, j // c.page_size], j % c.page_size
            kb[b, i] = inp.k_pool[page, :, slot, :]
            vb[b, i] = inp.v_pool[page, :, slot, :]
    return kb, vb


@pytest.mark.parametrize("scale", [1.0, 0.0625, 0.3, 7.0])
def test_encode_bf16_matches_library(scale):
    rng = np.random.default_rng(11)
    bits = random_bf16(rng, 3000, 3.0)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    want = (x / torch.tensor(scale, dtype=torch.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.encode_kv("bf16", scale, int(b)) for b in bits], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("scale", [1.0, 0.0625, 0.3, 0.01])
def test_encode_fp8_matches_library_in_range(scale):
    rng = np.random.default_rng(12)
    bits = random_bf16(rng, 3000, 2.0)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    q = x / torch.tensor(scale, dtype=torch.float32)
    keep = (q.abs() < 464).numpy()  # torch's cast turns the rest into NaN; the cache saturates instead
    want = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.encode_kv("fp8_e4m3", scale, int(b)) for b in bits], dtype=np.uint8)
    np.testing.assert_array_equal(got[keep], want[keep])
    assert keep.sum() > 2000


def test_encode_fp8_saturation_ties_and_nan():
    enc = lambda v, s=1.0: oracle.encode_kv("fp8_e4m3", s, int(torch.tensor(v).to(torch.bfloat16).view(torch.int16)) & 0xFFFF)
    assert enc(1000.0) == 0x7E and enc(-1000.0) == 0xFE and enc(480.0) == 0x7E
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A  # ties to the even code
    assert enc(float("nan")) == 0x7F
    assert enc(3.0, 0.5) == oracle.encode_kv("fp8_e4m3", 1.0, int(torch.tensor(6.0).to(torch.bfloat16).view(torch.int16)))


def test_block_arrays_equal_to_the_cache_change_nothing():
    c = tiny(1, batch=2, K=3, ctx=37)
    inp = synth.make_inputs(c)
    kb, vb = block_of_cache(inp)
    a_out, a_lse = oracle.attention_case(inp, threads=2)
    b_out, b_lse = oracle.attention_case(inp, threads=2, k_block=kb, v_block=vb)
    np.testing.assert_array_equal(a_out, b_out)
    np.testing.assert_array_equal(a_lse, b_lse)


@pytest.mark.parametrize("kw", [dict(ctx=0), dict(ctx=45, wl=9, wr=-1), dict(ctx=70, K=7, hq=8, hkv=2),
                                dict(batch=3, ctx_range=(1, 60), K=2, hq=6, hkv=3, wl=5, wr=1)])
def test_block_arrays_read_instead_of_the_cache(kw):
    c = tiny(2 + len(str(kw)), **kw)
    inp = synth.make_inputs(c)
    rng = np.random.default_rng(3)
    shape = (c.batch, c.block_size, c.num_kv_heads, c.head_dim)
    kb, vb = random_bf16(rng, shape), random_bf16(rng, shape)
    out, lse = oracle.attention_case(inp, threads=2, k_block=kb, v_block=vb)
    # writing the arrays into the (bf16, unscaled) cache gives the same answer
    for b in range(c.batch):
        n = int(inp.seq_lens[b])
        for i in range(c.block_size):
            j = n - c.block_size + i
            page, slot = inp.page_table[b, j // c.page_size], j % c.page_size
            inp.k_pool[page, :, slot, :] = kb[b, i]
            inp.v_pool[page, :, slot, :] = vb[b, i]
    ref_out, ref_lse = oracle.attention_case(inp, threads=2)
    np.testing.assert_array_equal(out, ref_out)
    np.testing.assert_array_equal(lse, ref_lse)


def test_block_arrays_with_an_fp8_cache_match_bruteforce():
    c = tiny(20, fp8=True, batch=2, K=3, ctx=29, ks=0.5, vs=2.0)
    inp = synth.make_inputs(c)
    rng = np.random.default_rng(4)
    shape = (c.batch, c.block_size, c.num_kv_heads, c.head_dim)
    kb, vb = random_bf16(rng, shape), random_bf16(rng, shape)
    out, lse = oracle.attention_case(inp, threads=2, k_block=kb, v_block=vb)
    ref_out, ref_lse = bruteforce.attention(inp, k_block=kb, v_block=vb)
    np.testing.assert_allclose(out, ref_out, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_block_arrays_go_together():
    c = tiny(21)
    inp = synth.make_inputs(c)
    kb, _ = block_of_cache(inp)
    with pytest.raises(ValueError):
        oracle.attention_case(inp, k_block=kb)

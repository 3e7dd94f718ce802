"""Pins for the dense block keys and the append encoding in the oracle (CPU only).

The block keys may come from dense bf16 arrays instead of the cache (the
dense-suffix form); appending stores them into the cache encoded for its
element type and scale. The oracle's encoder is held to torch's fp32 division
and its bf16 / float8_e4m3fn casts; the dense block to identities (arrays equal
to the cache give the cache's result exactly; writing the arrays into a bf16
cache gives the same result) and to the brute force.
"""
import math

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


def _bf16_bits(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_encode_bf16_overflow_matches_library():
    """Quotients near FLT_MAX: past the midpoint between the largest finite bf16 and 2^128
    they round to infinity, below it to 0x7F7F (torch's fp32 -> bf16 cast decides)."""
    top = [0x7F7F, 0x7F7E, 0x7F70, 0x7F00, 0xFF7F, 0xFF7E, 0xFF00]
    scales = [1.0, 0.999, 0.998, 0.9975, 0.997, 0.996, 0.99, 0.9, 0.75, 0.5, 0.25, 1.01]
    hit_inf = hit_top = 0
    for s in scales:
        bits = np.array(top, dtype=np.uint16)
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
        want = (x / torch.tensor(s, dtype=torch.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        got = np.array([oracle.encode_kv("bf16", s, int(b)) for b in bits], dtype=np.uint16)
        np.testing.assert_array_equal(got, want, err_msg=f"scale {s}")
        hit_inf += int(((want & 0x7FFF) == 0x7F80).sum())
        hit_top += int(((want & 0x7FFF) == 0x7F7F).sum())
    assert hit_inf >= 10 and hit_top >= 4  # both sides of the overflow midpoint are exercised
    # quotients spread over the last binade, drawn so that many land within 1 % of FLT_MAX
    rng = np.random.default_rng(13)
    s = np.float32(0.9921875)  # 1 - 2^-7: exact, so the fp32 quotients stay distinct
    mant = rng.integers(0x7F7000, 0x7F8000, 4000, dtype=np.uint32)
    bits = (mant >> 8).astype(np.uint16) | (rng.integers(0, 2, 4000, dtype=np.uint16) << 15)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    want = (x / torch.tensor(float(s), dtype=torch.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.encode_kv("bf16", float(s), int(b)) for b in bits], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)
    assert ((want & 0x7FFF) == 0x7F80).sum() > 100


def test_encode_bf16_infinities_and_nan():
    """+-inf stay +-inf (torch's cast agrees); every NaN becomes the canonical quiet NaN 0x7FC0
    (the reading taken for the append: torch's CPU cast gives another NaN code, so only its
    NaN-ness is a library fact)."""
    inf = float("inf")
    for v, s, want in [(inf, 1.0, 0x7F80), (-inf, 1.0, 0xFF80), (inf, 0.01, 0x7F80), (-inf, 7.0, 0xFF80)]:
        b = int(_bf16_bits([v])[0])
        lib = int((torch.tensor([v]).to(torch.bfloat16).float() / s).to(torch.bfloat16).view(torch.int16)) & 0xFFFF
        assert oracle.encode_kv("bf16", s, b) == want == lib
    for nan_bits in (0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x7FFF, 0xFFFF, 0x7FA5):
        got = oracle.encode_kv("bf16", 0.3, nan_bits)
        assert got == 0x7FC0
        assert math.isnan(oracle.bf16_to_double(got))
    # finite / scale overflowing fp32 itself: the quotient is inf
    assert oracle.encode_kv("bf16", 0.5, 0x7F7F) == 0x7F80 and oracle.encode_kv("bf16", 0.5, 0xFF7F) == 0xFF80


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

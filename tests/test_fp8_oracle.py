"""Pins for the fp8 (OCP E4M3) context storage in the oracle and the input generator (CPU only).

The oracle decodes pool bytes with its own code; these tests hold it to
torch's float8_e4m3fn conversion (a library routine), to values the format's
definition fixes by hand, and to the dense brute force, whose decode goes
through torch. The generator's encoder is held to torch's float -> e4m3 cast.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import Case, fp8_variant
from tests import bruteforce


def tiny8(idx, *, batch=1, K=3, hq=4, hkv=1, D=16, P=8, ctx=20, ctx_range=None, wl=-1, wr=-1, ks=0.0625, vs=0.0625):
    c = Case(f"tiny8_{idx}", 91, idx, batch=batch, block_size=K, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
             page_size=P, context=ctx, context_range=ctx_range, window_left=wl, window_right=wr)
    return fp8_variant(c, ks, vs)


def test_decode_matches_library_for_every_code():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    for c in range(256):
        got = oracle.fp8_e4m3_to_double(c)
        assert (math.isnan(got) and math.isnan(ref[c])) or got == ref[c], (c, got, ref[c])


def test_decode_values_the_format_fixes():
    d = oracle.fp8_e4m3_to_double
    assert d(0x38) == 1.0 and d(0xB8) == -1.0 and d(0x40) == 2.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0        # largest finite: 1.75 * 2^8
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9  # smallest normal, smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9 and d(0x3F) == 1.875
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))   # no infinities in E4M3


def test_encoder_round_trips_every_finite_code():
    for c in range(256):
        v = oracle.fp8_e4m3_to_double(c)
        if math.isnan(v):
            continue
        assert synth.e4m3_from_double(v) == c, (c, v)


def test_encoder_matches_library_cast():
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.normal(0, 1, 4000) * 16, rng.normal(0, 1e-2, 1000), rng.uniform(-440, 440, 1000)])
    lib = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([synth.e4m3_from_double(x) for x in xs], dtype=np.uint8)
    np.testing.assert_array_equal(ours, lib)


def test_encoder_ties_saturation_and_nan():
    enc = synth.e4m3_from_double
    assert enc(1.0 + 1 / 16) == 0x38          # halfway between 1 and 1.125: to the even mantissa (1)
    assert enc(1.0 + 3 / 16) == 0x3A          # halfway between 1.125 and 1.25: to even (1.25)
    assert enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02  # subnormal ties to even
    assert enc(1000.0) == 0x7E and enc(-1e9) == 0xFE and enc(464.0) == 0x7E
    assert enc(float("nan")) == 0x7F


@pytest.mark.parametrize("kw", [
    dict(ctx=0), dict(ctx=37, P=16), dict(ctx=70, K=7, hq=8, hkv=2), dict(ctx=45, K=3, wl=9, wr=-1),
    dict(ctx=60, K=7, hq=16, hkv=1, wl=20, wr=2, ks=0.5, vs=2.0), dict(batch=3, ctx_range=(5, 90), K=2, hq=6, hkv=3),
])
def test_fp8_oracle_matches_bruteforce(kw):
    c = tiny8(len(str(kw)), **kw)
    inp = synth.make_inputs(c)
    assert inp.k_pool.dtype == np.uint8 and (inp.k_pool[-1] == synth.FP8_NAN).all()
    out, lse = oracle.attention_case(inp, threads=2)
    ref_out, ref_lse = bruteforce.attention(inp)
    np.testing.assert_allclose(out, ref_out, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_fp8_zero_query_is_uniform_average_of_scaled_values():
    c = tiny8(50, ctx=25, K=3, hq=2, hkv=1, vs=0.25)
    inp = synth.make_inputs(c)
    inp.q[:] = 0
    out, lse = oracle.attention_case(inp, threads=2)
    n = int(inp.seq_lens[0])
    vals = bruteforce.dense_kv(inp.v_pool, inp.page_table, 0, n, 0.25)[:, 0, :]
    np.testing.assert_allclose(out[0, :, 0, :], np.broadcast_to(vals.mean(axis=0), (3, c.head_dim)), rtol=1e-12)
    np.testing.assert_allclose(lse, np.log2(n), rtol=1e-12)


def test_scales_act_as_logit_and_output_factors():
    c = tiny8(51, ctx=40, K=3, hq=4, hkv=1, ks=1.0, vs=1.0)
    inp = synth.make_inputs(c)
    base_out, base_lse = oracle.attention_case(inp, threads=2)
    kw = dict(block_size=c.block_size, num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads, head_dim=c.head_dim,
              page_size=c.page_size, kv_dtype="fp8_e4m3", threads=2)
    args = (inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens)
    # k_scale multiplies every logit, exactly like sm_scale
    a_out, a_lse = oracle.attention(*args, sm_scale=c.scale, k_scale=0.5, **kw)
    b_out, b_lse = oracle.attention(*args, sm_scale=c.scale * 0.5, k_scale=1.0, **kw)
    np.testing.assert_allclose(a_out, b_out, rtol=1e-13)
    np.testing.assert_allclose(a_lse, b_lse, rtol=1e-13)
    # v_scale multiplies the output and leaves the LSE alone
    v_out, v_lse = oracle.attention(*args, sm_scale=c.scale, v_scale=3.0, **kw)
    np.testing.assert_allclose(v_out, 3.0 * base_out, rtol=1e-13)
    np.testing.assert_array_equal(v_lse, base_lse)


def test_rejects_unknown_kv_dtype_code():
    c = tiny8(52)
    inp = synth.make_inputs(c)
    with pytest.raises(KeyError):
        oracle.attention(inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, block_size=3, num_q_heads=4,
                         num_kv_heads=1, head_dim=16, page_size=8, sm_scale=0.25, kv_dtype="fp16")

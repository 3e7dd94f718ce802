"""GPU parity of the fp8 (OCP E4M3) context path against the fp64 oracle (MI355X only).

The same rule as the bf16 path: the oracle decodes every pool byte exactly and
applies the per-pool scales in fp64. Small cases compare every row; the
full-size configuration variants compare sampled (request, kv head) pairs. One
test walks all 256 codes through the kernels' own conversions: a single-key
request's output is exactly v_scale times its value, and with one-hot queries
each row's LSE exposes one key element.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth.configs import Case, find_case, fp8_variant
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def case8(idx, *, batch=2, K=3, hq=4, hkv=1, D=64, P=32, ctx=100, ctx_range=None, wl=-1, wr=-1, outliers=0.0,
          ks=0.0625, vs=0.0625):
    c = Case(f"f{idx}", 81, idx, batch=batch, block_size=K, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=P,
             context=ctx, context_range=ctx_range, window_left=wl, window_right=wr, outlier_rate=outliers)
    return fp8_variant(c, ks, vs)


def check_full(c, label, **run_kw):
    inp = synth.make_inputs(c)
    assert inp.k_pool.dtype == np.uint8
    out, lse, info = H.run(H.upload(inp), **run_kw)
    ref_out, ref_lse = oracle.attention_case(inp)
    res = H.compare(out, lse, ref_out, ref_lse, label=label)
    print(f"{label}: {res} info={info}", flush=True)
    return out, lse, info


SMALL8 = [
    (1, dict(batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=1000)),                # streaming kernel, D = 64
    (2, dict(batch=3, K=3, hq=6, hkv=3, D=64, P=16, ctx_range=(40, 300))),     # 16-token pages, mixed lengths
    (3, dict(batch=2, K=1, hq=16, hkv=1, D=128, P=64, ctx=300)),               # streaming kernel, D = 128
    (4, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=128, ctx=950)),              # shared tiles, one block per wave
    (5, dict(batch=1, K=7, hq=16, hkv=1, D=64, P=32, ctx=777)),                # shared tiles, D = 64
    (6, dict(batch=2, K=3, hq=16, hkv=1, D=128, P=64, ctx=2100, ks=0.5, vs=2.0)),  # two blocks per wave; scales
    (7, dict(batch=1, K=3, hq=4, hkv=1, D=64, P=32, ctx=0)),                   # block keys only
]

W8 = [
    (21, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=64, ctx=3000, wl=256, wr=-1, ks=0.25, vs=4.0)),
    (22, dict(batch=3, K=3, hq=64, hkv=4, D=128, P=64, ctx_range=(100, 1500), wl=300, wr=-1, outliers=0.01)),
    (23, dict(batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=500, wl=33, wr=2)),
]


@pytest.mark.parametrize("idx,kw", SMALL8 + W8, ids=[f"f{i}" for i, _ in SMALL8 + W8])
def test_fp8_small(idx, kw):
    check_full(case8(idx, **kw), f"fp8 f{idx}")


def test_fp8_three_blocks_two_token_groups():
    """R = 48 with fp8 pools: two token groups of four one-block waves (one rowless), chosen
    automatically once the batch holds at least 64 tiles per CU (here 256 (request, kv head)
    pairs of 129 window tiles), and forced on a small ragged batch with forced splits."""
    big = case8(30, batch=64, K=3, hq=64, hkv=4, D=128, P=64, ctx_range=(4200, 5000), wl=4096, wr=-1, outliers=0.01)
    _, _, info = check_full(big, "fp8 f30")
    assert info["token_groups"] == 2 and info["row_waves"] == 4 and info["max_splits"] == 1
    small = case8(31, batch=3, K=3, hq=16, hkv=1, D=128, P=32, ctx_range=(0, 1800), ks=0.5, vs=2.0)
    _, _, info = check_full(small, "fp8 f31", waves=8, splits=3)
    assert info["token_groups"] == 2 and info["row_waves"] == 4


@pytest.mark.parametrize("splits", [1, 3, 1000])
def test_fp8_split_invariance(splits):
    c = case8(30, batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=3000)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    ref_out, ref_lse = oracle.attention_case(inp)
    out, lse, info = H.run(dc, splits=splits)
    H.compare(out, lse, ref_out, ref_lse, label=f"fp8 splits={splits}")
    base, _, _ = H.run(dc, splits=1)
    assert np.abs(out - base).max() <= 4 * H.ulp_bf16(float(np.abs(base).max()))


def _single_key_case(idx, *, batch, hq, D, ks=1.0, vs=1.0):
    return case8(idx, batch=batch, K=1, hq=hq, hkv=1, D=D, P=16, ctx=0, ks=ks, vs=vs)


def test_fp8_every_value_code_decodes_exactly():
    """Single-key requests: out = v_scale * v exactly; 4 requests x 64 dims hold all 256 codes."""
    c = _single_key_case(40, batch=4, hq=1, D=64, vs=2.0)
    inp = synth.make_inputs(c)
    codes = np.arange(256, dtype=np.uint8).reshape(4, 64)
    for b in range(4):
        page = inp.page_table[b, 0]
        inp.v_pool[page, 0, 0, :] = codes[b]
        inp.k_pool[page, 0, 0, :] = 0
    out, _, _ = H.run(H.upload(inp))
    want = np.array([[2.0 * oracle.fp8_e4m3_to_double(int(x)) for x in row] for row in codes])
    got = out[:, 0, 0, :].astype(np.float64)
    nan = np.isnan(want)
    assert nan.sum() == 2 and np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan], want[~nan])


def test_fp8_every_key_code_decodes_exactly():
    """One-hot queries: row h's LSE is log2(e) * sm_scale * k_scale * k[h]. Requests 0-7 hold the 254 finite
    codes (two slots repeat code 0); request 8 holds the two NaN codes, and since a NaN key element makes every
    dot product with that key NaN (0 * NaN), all its rows must come out NaN, as in the oracle."""
    c = _single_key_case(41, batch=9, hq=32, D=64, ks=0.5)
    inp = synth.make_inputs(c)
    finite = [x for x in range(256) if x not in (0x7F, 0xFF)] + [0, 0]
    codes = np.array(finite + [0x7F, 0xFF] + [0] * 30, dtype=np.uint8).reshape(9, 32)
    one = 0x3F80  # bf16 1.0
    inp.q[:] = 0
    for b in range(9):
        page = inp.page_table[b, 0]
        inp.k_pool[page, 0, 0, :] = 0
        inp.k_pool[page, 0, 0, :32] = codes[b]
        inp.v_pool[page, 0, 0, :] = 0x38  # 1.0
        for h in range(32):
            inp.q[b, 0, h, h] = one
    _, lse, _ = H.run(H.upload(inp))
    _, ref_lse = oracle.attention_case(inp)
    got = lse[:, 0, :].astype(np.float64)
    want = ref_lse[:, 0, :]
    assert np.isfinite(want[:8]).all() and np.isnan(want[8]).all()
    assert np.isnan(got[8]).all(), got[8].tolist()
    np.testing.assert_allclose(got[:8], want[:8], rtol=2e-7, atol=1e-6)


FP8_CONFIGS = ["cfg1_fp8", "cfg2_b1_128k_fp8", "cfg2_b8_128k_fp8", "cfg3_b4_32k_fp8", "cfg4_b8_k7_16k_fp8",
               "cfg4_b64_k3_8k_fp8", "cfg5_k3_fp8", "cfg5_k7_fp8"]


@pytest.mark.parametrize("name", FP8_CONFIGS)
def test_fp8_config_case(name):
    case = find_case(name)
    print(f"[{name}] generating", flush=True)
    inp = synth.make_inputs(case)
    dc = H.upload(inp)
    out, lse, info = H.run(dc)
    del dc
    ref_out, ref_lse = oracle.attention_case(inp)  # every row of the call
    res = H.compare(out, lse, ref_out, ref_lse, label=name)
    print(f"[{name}] {res} units={info['units']}", flush=True)


@pytest.mark.parametrize("idx,kw", [(70, dict(batch=2, K=7, hq=8, hkv=2, D=64, P=256, ctx_range=(0, 1200))),
                                     (71, dict(batch=2, K=7, hq=16, hkv=1, D=128, P=256, ctx=1800, wl=500, wr=-1))],
                         ids=["p256_stream", "p256_shared"])
def test_fp8_pages_of_256_tokens(idx, kw):
    check_full(case8(idx, **kw), f"fp8 p256_{idx}")


def test_fp8_more_than_128_rows():
    c = case8(72, batch=2, K=16, hq=16, hkv=1, D=128, P=64, ctx=1100, wl=700, wr=-1)  # R = 256
    check_full(c, "fp8 rows 256")

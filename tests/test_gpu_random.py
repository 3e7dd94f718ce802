"""Seeded random shapes across the parameter space, each against the fp64 oracle (MI355X only).

Every case draws, from its own seed: block size K in 1..16, a GQA group with R = K * g
rows at most 128, D in {64, 128}, P in {16, 32, 64, 128}, one to four kv heads, mixed
context lengths (empty contexts included), the unwindowed or the windowed form (any W,
W_r in {-1, 0, 1..K}), a bf16 or fp8 cache with scales, forced split and wave counts,
and the block's keys from the cache or from dense arrays (with or without the append).
"""
import numpy as np
import pytest
import torch
from dataclasses import replace

import oracle
import speculative_decoding_draft_paged_amd as ba
import synth
from synth.configs import Case, fp8_variant
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

N_CASES = 256


def draw(seed, max_rows=128):
    rng = np.random.default_rng(7000 + seed)
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64, 128]))
    K = int(rng.integers(1, 17))
    g = int(rng.integers(1, max(2, max_rows // K + 1)))
    g = max(1, min(g, max_rows // K))
    hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 5))
    lo = int(rng.integers(0, 400))
    hi = lo + int(rng.integers(0, 2500))
    windowed = bool(rng.integers(0, 2))
    wl, wr = -1, -1
    if windowed:
        wl = int(rng.choice([1, 2, 7, 64, 500, 3000, 100000]))
        wr = int(rng.choice([-1, 0, 1, max(1, K // 2), K]))
    c = Case(f"rnd{seed}", 84, seed, batch=B, block_size=K, num_q_heads=g * hkv, num_kv_heads=hkv, head_dim=D,
             page_size=P, context_range=(lo, hi), window_left=wl, window_right=wr,
             outlier_rate=float(rng.choice([0.0, 0.02])))
    if rng.integers(0, 3) == 0:
        c = fp8_variant(c, float(rng.choice([0.0625, 0.5, 0.3])), float(rng.choice([0.0625, 2.0, -0.7])))
    elif rng.integers(0, 3) == 0:
        c = replace(c, k_scale=float(rng.choice([0.5, 1.7])), v_scale=float(rng.choice([0.25, 3.0])))
    splits = int(rng.choice([0, 0, 1, 2, 5, 13]))
    waves = int(rng.choice([0, 0, 0, 1, 2, 3, 4, 8]))
    block = str(rng.choice(["cache", "cache", "dense", "append"]))
    return c, splits, waves, block


def block_arrays(c, seed):
    rng = np.random.default_rng(9000 + seed)
    shape = (c.batch, c.block_size, c.num_kv_heads, c.head_dim)
    mk = lambda: torch.from_numpy(rng.normal(0, 1.5, shape).astype(np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    return mk(), mk()


def run_case(seed, max_rows):
    c, splits, waves, block = draw(seed, max_rows)
    print(f"rnd{seed}: K={c.block_size} Hq={c.num_q_heads} Hkv={c.num_kv_heads} D={c.head_dim} P={c.page_size} "
          f"B={c.batch} ctx={c.context_range} W={c.window_left}/{c.window_right} kv={c.kv_dtype} "
          f"scales={c.k_scale}/{c.v_scale} splits={splits} waves={waves} block={block}", flush=True)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    if block == "cache":
        out, lse, _ = H.run(dc, splits=splits, waves=waves)
        ref_out, ref_lse = oracle.attention_case(inp)
    else:
        kb, vb = block_arrays(c, seed)
        prm = H.params_for(dc, splits=splits, waves=waves)
        nbytes = ba.blockattn_workspace_size(prm, inp.seq_lens)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        plan = ba.blockattn_plan(prm, inp.seq_lens, ws, nbytes)
        o = torch.empty(c.batch, c.block_size, c.num_q_heads, c.head_dim, dtype=torch.bfloat16, device="cuda")
        l = torch.empty(c.batch, c.block_size, c.num_q_heads, dtype=torch.float32, device="cuda")
        to = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        ba.blockattn_forward_block(plan, dc.q, to(kb), to(vb), dc.k, dc.v, dc.page_table, dc.seq_lens, ws, o, l,
                                   append=block == "append")
        torch.cuda.synchronize()
        plan.destroy()
        out, lse = o.float().cpu().numpy(), l.cpu().numpy()
        ref_out, ref_lse = oracle.attention_case(inp, k_block=kb, v_block=vb)
    H.compare(out, lse, ref_out, ref_lse, label=f"rnd{seed}")


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    run_case(seed, 128)


@pytest.mark.parametrize("seed", range(N_CASES, N_CASES + 64))
def test_random_shape_up_to_512_rows(seed):
    """Row groups: R up to 512 query rows per kv head."""
    run_case(seed, 512)

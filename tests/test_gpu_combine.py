"""The split combine inside the attention kernel (last arriver) against the combine kernel (MI355X only).

A split (request, kv head) is combined either by the separate combine kernel or, inside the
attention kernel, by whichever of its units finishes last (found by an arrival counter in the
workspace, reset by that unit for the next call). Both must meet the parity rule against the
oracle on every row, give the same bits on a second call with the same plan (so the counters
were left at zero), agree with each other within a few ulp, and behave under graph replay
and with splits left empty by shorter device lengths.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_draft_paged_amd as ba
import synth
from synth.configs import Case, fp8_variant
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def ccase(idx, *, fp8=False, batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx=3000, ctx_range=None, wl=-1, wr=-1):
    c = Case(f"cb{idx}", 85, idx, batch=batch, block_size=K, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
             page_size=P, context=ctx, context_range=ctx_range, window_left=wl, window_right=wr)
    return fp8_variant(c, 0.0625, 0.0625) if fp8 else c


CASES = [
    (1, dict(), 8),                                                       # stream kernel, D = 64, R = 28
    (2, dict(batch=3, ctx_range=(500, 9000)), 0),                          # mixed lengths: per-request splits
    (3, dict(K=3, hq=16, hkv=2, D=128, P=64, ctx=5000), 6),                # stream kernel, D = 128, R = 24
    (4, dict(K=7, hq=16, hkv=1, D=128, P=64, ctx=6000, wl=2000, wr=-1), 5),  # shared tiles, R = 112, windowed
    (5, dict(K=3, hq=48, hkv=3, D=64, P=32, ctx=4000), 4),                 # shared tiles at D = 64, R = 144
    (6, dict(K=16, hq=16, hkv=1, D=128, P=32, ctx=3000, wl=900, wr=3), 3),  # R = 256: two row groups
    (7, dict(fp8=True, batch=2, ctx=7000), 12),                            # fp8 pools
    (8, dict(batch=1, ctx=20000), 125),                                    # many splits
    (9, dict(K=1, hq=8, hkv=2, ctx=2500, wl=700, wr=-1), 7),               # one query: windowed decode
    # R = 112 over 2064 tiles: two token groups of the shared-tile kernel
    (10, dict(batch=16, K=7, hq=16, hkv=1, D=128, P=64, ctx=4200, wl=4096, wr=-1), 3),
]


@pytest.mark.parametrize("idx,kw,splits", CASES, ids=[f"cb{i}" for i, _, _ in CASES])
def test_last_arriver_combine_matches_oracle_and_kernel_combine(idx, kw, splits):
    c = ccase(idx, **kw)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    ref_out, ref_lse = oracle.attention_case(inp)
    out_f, lse_f, info_f = H.run(dc, splits=splits, combine="last_arriver", canary=True)
    out_k, lse_k, info_k = H.run(dc, splits=splits, combine="kernel")
    assert info_f["fused_combine"] == 1 and info_f["combine_launch"] == 0 and info_f["max_splits"] > 1
    assert info_k["fused_combine"] == 0 and info_k["combine_launch"] == 1
    rf = H.compare(out_f, lse_f, ref_out, ref_lse, label=f"cb{idx} last arriver")
    rk = H.compare(out_k, lse_k, ref_out, ref_lse, label=f"cb{idx} combine kernel")
    amax = float(np.abs(ref_out).max())
    assert np.abs(out_f - out_k).max() <= 4 * H.ulp_bf16(amax)
    assert np.abs(lse_f - lse_k).max() <= 1e-5
    print(f"cb{idx}: last arriver {rf}, kernel {rk}, splits {info_f['max_splits']}", flush=True)


def test_last_arriver_with_two_token_groups_of_one_block_waves():
    """Three row blocks as two token groups (one rowless wave each): the groups merge in LDS,
    then the last split of each pair combines the pair's partials."""
    c = ccase(11, fp8=True, batch=2, K=3, hq=16, hkv=1, D=128, P=64, ctx=5000, wl=3000, wr=-1)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    ref_out, ref_lse = oracle.attention_case(inp)
    out_f, lse_f, info_f = H.run(dc, splits=6, waves=8, combine="last_arriver", canary=True)
    assert info_f["fused_combine"] == 1 and info_f["token_groups"] == 2 and info_f["row_waves"] == 4
    H.compare(out_f, lse_f, ref_out, ref_lse, label="cb11 last arriver, two groups")


def test_last_arriver_with_empty_splits():
    """Device lengths far shorter than the plan's leave some splits with no tiles (m = -inf, l = 0)."""
    c = ccase(20, batch=2, ctx=8000)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    short = inp.seq_lens.copy()
    short[:] = [600, 40]
    dc.seq_lens = torch.from_numpy(short).cuda()
    out, lse, info = H.run(dc, plan_lens=inp.seq_lens, splits=24, combine="last_arriver", canary=True)
    assert info["fused_combine"] == 1 and info["max_splits"] == 24
    ref_out, ref_lse = oracle.attention_case(synth.Inputs(c, inp.q, inp.k_pool, inp.v_pool, inp.page_table, short))
    H.compare(out, lse, ref_out, ref_lse, label="empty splits, last arriver")


def test_last_arriver_under_graph_replay():
    """Captured calls replayed several times, with eager calls and synchronisations between the
    replays: every replay matches the eager result bit for bit (the counters start at zero each time)."""
    c = ccase(21, batch=3, ctx_range=(2000, 12000))
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    prm = H.params_for(dc, combine="last_arriver")
    n = ba.blockattn_workspace_size(prm, inp.seq_lens)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    plan = ba.blockattn_plan(prm, inp.seq_lens, ws, n)
    assert plan.info()["fused_combine"] == 1
    shape = (c.batch, c.block_size, c.num_q_heads, c.head_dim)
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    ba.blockattn_forward(plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, ws, out, lse)
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()
    ref_out, ref_lse = oracle.attention_case(inp)
    H.compare(eager_out.float().cpu().numpy(), eager_lse.cpu().numpy(), ref_out, ref_lse, label="eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            ba.blockattn_forward(plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, ws, out, lse)
    for rep in range(4):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16)), f"replay {rep}"
        assert torch.equal(lse.view(torch.int32), eager_lse.view(torch.int32)), f"replay {rep}"
        ba.blockattn_forward(plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, ws, out, lse)  # eager in between
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16))
    plan.destroy()


def test_last_arriver_through_the_scratch_entry_point():
    c = ccase(22, batch=2, ctx_range=(3000, 9000))
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    prm = H.params_for(dc, combine="last_arriver")
    plan = ba.blockattn_plan(prm, inp.seq_lens)
    assert plan.info()["fused_combine"] == 1
    shape = (c.batch, c.block_size, c.num_q_heads, c.head_dim)
    ref_out, ref_lse = oracle.attention_case(inp)
    for rep in range(2):
        out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
        ba.blockattn_forward_scratch(plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, out, lse)
        torch.cuda.synchronize()
        H.compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, label=f"scratch call {rep}")
    plan.destroy()

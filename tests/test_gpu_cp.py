"""A context split into shards, each attended on its own, then merged (MI355X only).

Context parallelism gives each GPU a contiguous shard of a request's pages; each computes
its (out, LSE) over its keys, and after an all-gather every GPU merges the G parts. Here one
GPU plays every shard in turn: the unwindowed forward runs on each page-aligned shard (its
own page-table slice and length), blockattn_merge combines the parts, and the result must
match the fp64 oracle over the whole context. The merge is also checked on its own against
the oracle's pairwise LSE merge, with empty and NaN parts.
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


def shard_call(dc, c, G, splits=0):
    """Forward on G page-aligned shards of every request; returns stacked (out, lse) on the device."""
    inp = dc.inputs
    P = c.page_size
    outs, lses = [], []
    for g in range(G):
        lens_g = np.zeros(c.batch, dtype=np.int32)
        first = np.zeros(c.batch, dtype=np.int64)
        for b in range(c.batch):
            n = int(inp.seq_lens[b])
            pages = (n + P - 1) // P
            p0, p1 = pages * g // G, pages * (g + 1) // G
            first[b] = p0
            lens_g[b] = min(p1 * P, n) - p0 * P
        stride = int(((lens_g + P - 1) // P).max()) + 1
        pt_g = np.zeros((c.batch, stride), dtype=np.int32)
        for b in range(c.batch):
            np_b = (int(lens_g[b]) + P - 1) // P
            pt_g[b, :np_b] = inp.page_table[b, first[b]:first[b] + np_b]
        assert (lens_g >= c.block_size).all()
        prm = ba.make_params(batch=c.batch, block_size=c.block_size, num_q_heads=c.num_q_heads,
                             num_kv_heads=c.num_kv_heads, head_dim=c.head_dim, page_size=P, page_table_stride=stride,
                             num_pages=inp.num_pages, sm_scale=c.scale, splits_override=splits, kv_dtype=c.kv_dtype,
                             k_scale=c.k_scale, v_scale=c.v_scale)
        nbytes = ba.blockattn_workspace_size(prm, lens_g)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        plan = ba.blockattn_plan(prm, lens_g, ws, nbytes)
        out = torch.empty(c.batch, c.block_size, c.num_q_heads, c.head_dim, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(c.batch, c.block_size, c.num_q_heads, dtype=torch.float32, device="cuda")
        ba.blockattn_forward(plan, dc.q, dc.k, dc.v, torch.from_numpy(pt_g).cuda(), torch.from_numpy(lens_g).cuda(),
                             ws, out, lse)
        torch.cuda.synchronize()
        plan.destroy()
        outs.append(out)
        lses.append(lse)
    return torch.stack(outs), torch.stack(lses)


SHARDS = [
    (1, 2, dict(batch=2, K=7, hq=8, hkv=2, D=64, P=32, ctx_range=(600, 3000))),
    (2, 3, dict(batch=3, K=3, hq=16, hkv=1, D=128, P=64, ctx_range=(900, 2500))),
    (3, 8, dict(batch=2, K=7, hq=8, hkv=2, D=64, P=16, ctx=4000)),
    (4, 4, dict(fp8=True, batch=2, K=7, hq=16, hkv=1, D=128, P=32, ctx=2000)),
]


@pytest.mark.parametrize("idx,G,kw", SHARDS, ids=[f"cp{i}_G{G}" for i, G, _ in SHARDS])
def test_context_shards_merge_to_the_full_result(idx, G, kw):
    kw = dict(kw)
    fp8 = kw.pop("fp8", False)
    c = Case(f"cp{idx}", 85, idx, batch=kw["batch"], block_size=kw["K"], num_q_heads=kw["hq"],
             num_kv_heads=kw["hkv"], head_dim=kw["D"], page_size=kw["P"], context=kw.get("ctx", 0),
             context_range=kw.get("ctx_range"))
    c = fp8_variant(c) if fp8 else c
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    ref_out, ref_lse = oracle.attention_case(inp)
    for splits in (0, 2):
        part_out, part_lse = shard_call(dc, c, G, splits)
        out = torch.empty_like(part_out[0])
        lse = torch.empty_like(part_lse[0])
        ba.blockattn_merge(part_out, part_lse, out, lse)
        torch.cuda.synchronize()
        H.compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, label=f"cp{idx} G={G}")


def test_merge_of_special_parts():
    rng = np.random.default_rng(5)
    G, rows, D = 5, 300, 128
    po = rng.normal(0, 1, (G, rows, D)).astype(np.float32)
    pl = rng.normal(0, 4, (G, rows)).astype(np.float32)
    pl[1, :40] = -np.inf             # empty parts
    pl[:, 40:45] = -np.inf           # rows no part has keys for
    pl[2, 45:50] = np.nan            # a NaN part poisons its rows
    po_bf = torch.from_numpy(po).to(torch.bfloat16)
    out = torch.empty(rows, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    ba.blockattn_merge(po_bf.cuda(), torch.from_numpy(pl).cuda(), out, lse)
    torch.cuda.synchronize()
    got, got_lse = out.float().cpu().numpy(), lse.cpu().numpy()
    parts = po_bf.float().numpy().astype(np.float64)
    ok = np.ones(rows, dtype=bool)
    ok[40:50] = False
    ref, ref_lse = parts[0][ok], pl[0][ok].astype(np.float64)
    for g in range(1, G):
        ref, ref_lse = oracle.merge(ref, ref_lse, parts[g][ok], pl[g][ok].astype(np.float64))
    H.compare(got[ok], got_lse[ok], ref, ref_lse, label="merge")
    assert (got[40:45] == 0).all() and np.isneginf(got_lse[40:45]).all()
    assert np.isnan(got[45:50]).all() and np.isnan(got_lse[45:50]).all()
    # one part: the result is the part itself
    one = torch.empty(rows, D, dtype=torch.bfloat16, device="cuda")
    one_lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    ba.blockattn_merge(po_bf[:1].cuda(), torch.from_numpy(pl[:1]).cuda(), one, one_lse)
    torch.cuda.synchronize()
    finite = np.isfinite(pl[0])
    assert torch.equal(one.cpu()[finite], po_bf[0][finite])
    assert np.array_equal(one_lse.cpu().numpy()[finite], pl[0][finite])

"""blockattn_forward_scratch: the forward for callers that cannot allocate (MI355X only).

The entry point keeps its work list and partial softmax states in the library's per-GPU
scratch array instead of a caller's workspace. Its output must match the workspace
forward on the same plan (the same decomposition, so bit for bit) and the fp64 oracle
(the parity rule), over two calls in a row, the second with a smaller input, so nothing
the first call left in the shared array reaches the second. (A plan too large for the
array is refused before anything launches: tests/test_abi_host.py, on the CPU.)
"""
import pytest
import torch

import oracle
import speculative_decoding_draft_paged_amd as ba
import synth
from synth.configs import Case
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _forward_both(c):
    """(scratch out, scratch lse, workspace out, workspace lse, inputs, plan info) for one case."""
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    prm = H.params_for(dc)
    n = ba.blockattn_workspace_size(prm, inp.seq_lens)
    assert n <= ba.BLOCKATTN_SCRATCH_BYTES
    shape = (c.batch, c.block_size, c.num_q_heads, c.head_dim)
    # the plan for the scratch call has no workspace at all
    plan = ba.blockattn_plan(prm, inp.seq_lens)
    out_s = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_s = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    ba.blockattn_forward_scratch(plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, out_s, lse_s)
    torch.cuda.synchronize()
    info = plan.info()
    plan.destroy()
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    wplan = ba.blockattn_plan(prm, inp.seq_lens, ws, n)
    out_w = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse_w = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    fwd = ba.blockattn_forward if c.window_left == -1 else ba.blockattn_windowed_forward
    fwd(wplan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, ws, out_w, lse_w)
    torch.cuda.synchronize()
    wplan.destroy()
    return out_s, lse_s, out_w, lse_w, inp, info


def _check(c, label):
    print(f"[no-alloc] {label}: {c}", flush=True)
    out_s, lse_s, out_w, lse_w, inp, info = _forward_both(c)
    assert torch.equal(out_s.view(torch.int16), out_w.view(torch.int16)), f"{label}: scratch and workspace outputs differ"
    assert torch.equal(lse_s.view(torch.int32), lse_w.view(torch.int32)), f"{label}: scratch and workspace LSE differ"
    ref, ref_lse = oracle.attention_case(inp)
    res = H.compare(out_s.float().cpu().numpy(), lse_s.cpu().numpy(), ref, ref_lse, label=label)
    print(f"[no-alloc] {label}: {res} units={info['units']} splits={info['max_splits']}", flush=True)
    return info


def test_scratch_forward_two_calls_second_smaller():
    # first: mixed long contexts, so requests get different split counts and the call copies
    # its work list into the array; second: a smaller windowed call through the shared-tile
    # kernel with another layout of the array
    big = Case("na1", 84, 1, batch=4, block_size=7, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
               context=0, context_range=(20000, 40000))
    small = Case("na2", 84, 2, batch=2, block_size=3, num_q_heads=16, num_kv_heads=1, head_dim=128, page_size=64,
                 context=0, context_range=(900, 2500), window_left=500, window_right=-1)
    info = _check(big, "first call")
    assert info["combine_launch"] == 1
    _check(small, "second, smaller call")


def test_scratch_forward_equal_lengths_and_single_split():
    # equal lengths (no work-list copy), then one split per request (no partials at all)
    _check(Case("na3", 84, 3, batch=2, block_size=7, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
                context=9000), "equal lengths")
    _check(Case("na4", 84, 4, batch=64, block_size=1, num_q_heads=16, num_kv_heads=1, head_dim=128, page_size=64,
                context=300, window_left=4096, window_right=-1), "one split per request")

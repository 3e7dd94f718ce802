"""Boundary behaviour on the GPU: stream ordering after the plan's upload, and the input-error word.

- A forward on a stream other than the plan's must not read the work list before the
  plan's upload has landed: the library orders it after the copy with an event wait.
- Out-of-range device inputs (a length past page_table_stride * P, a page id outside
  [0, num_pages)) are clamped so that no read leaves the caller's buffers, and the
  clamp is reported by blockattn_input_errors (checked mode).
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_draft_paged_amd as ba
import synth
from synth.configs import Case
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _case(idx, **kw):
    base = dict(batch=3, block_size=7, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32, context=0,
                context_range=(2000, 20000))
    base.update(kw)
    return Case(f"chk{idx}", 83, idx, **base)


def test_forward_on_another_stream_waits_for_the_plan_upload():
    c = _case(1)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    lens = inp.seq_lens
    assert len(set(lens.tolist())) > 1  # mixed lengths: the kernel reads the work list
    # A stale plan for longer, equal lengths first fills the workspace head with another
    # (valid) work list; its partials region is then poisoned with NaN bytes.
    stale_lens = np.full_like(lens, int(lens.max()))
    prm = H.params_for(dc)
    n_stale = ba.blockattn_workspace_size(prm, stale_lens)
    n_live = ba.blockattn_workspace_size(prm, lens)
    ws = torch.empty(max(n_stale, n_live), dtype=torch.uint8, device="cuda")
    a = torch.cuda.Stream()
    b = torch.cuda.Stream()
    with torch.cuda.stream(a):
        ws.fill_(0xFF)
        stale = ba.blockattn_plan(prm, stale_lens, ws, n_stale, stream=a)
    torch.cuda.synchronize()
    live_units = ba.blockattn_plan(prm, lens, None).info()["units"]
    assert stale.info()["units"] >= live_units  # stale items cover every unit index the live plan launches
    stale.destroy()
    out = torch.empty(c.batch, c.block_size, c.num_q_heads, c.head_dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(c.batch, c.block_size, c.num_q_heads, dtype=torch.float32, device="cuda")
    big = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(a):
        for _ in range(30):  # several milliseconds of work queued ahead of the upload
            big.mul_(1.0)
        plan = ba.blockattn_plan(prm, lens, ws, n_live, stream=a)
    with torch.cuda.stream(b):
        ba.blockattn_forward(plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, ws, out, lse, stream=b)
    torch.cuda.synchronize()
    got, got_lse = out.float().cpu().numpy(), lse.cpu().numpy()
    ref, ref_lse = oracle.attention_case(inp)
    H.compare(got, got_lse, ref, ref_lse, label="forward on a second stream")
    # the same plan on its own stream gives the same bits
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    with torch.cuda.stream(a):
        ba.blockattn_forward(plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, ws, out2, lse2, stream=a)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    plan.destroy()


def _run(dc, plan, ws, lens_dev, pt_dev):
    c = dc.inputs.case
    out = torch.empty(c.batch, c.block_size, c.num_q_heads, c.head_dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(c.batch, c.block_size, c.num_q_heads, dtype=torch.float32, device="cuda")
    fwd = ba.blockattn_forward if c.window_left == -1 else ba.blockattn_windowed_forward
    fwd(plan, dc.q, dc.k, dc.v, pt_dev, lens_dev, ws, out, lse)
    return out, lse


@pytest.mark.parametrize("windowed", [False, True])
def test_input_errors_report_clamped_lengths_and_pages(windowed):
    kw = dict(window_left=900, window_right=-1) if windowed else {}
    c = _case(2 + windowed, context_range=(100, 3000), **kw)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    prm = H.params_for(dc)
    n = ba.blockattn_workspace_size(prm, inp.seq_lens)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    plan = ba.blockattn_plan(prm, inp.seq_lens, ws, n)
    stride, P = inp.page_table.shape[1], c.page_size

    # clean inputs: no record, and the result matches the oracle
    out, lse = _run(dc, plan, ws, dc.seq_lens, dc.page_table)
    assert ba.blockattn_input_errors(plan, ws) == 0
    ref, ref_lse = oracle.attention_case(inp)
    H.compare(out.float().cpu().numpy(), lse.cpu().numpy(), ref, ref_lse, label="clean")

    # a device length past the page table's reach: clamped to stride * P and reported
    bad_lens = dc.seq_lens.clone()
    bad_lens[1] = stride * P + 100
    _run(dc, plan, ws, bad_lens, dc.page_table)
    assert ba.blockattn_input_errors(plan, ws) == ba.BLOCKATTN_INPUT_BAD_LENGTH
    assert ba.blockattn_input_errors(plan, ws) == 0  # the record was cleared

    # a length below the block size
    bad_lens = dc.seq_lens.clone()
    bad_lens[0] = c.block_size - 1
    _run(dc, plan, ws, bad_lens, dc.page_table)
    assert ba.blockattn_input_errors(plan, ws) == ba.BLOCKATTN_INPUT_BAD_LENGTH

    # page ids past the pool and negative ones, inside the pages a request reads
    bad_pt = dc.page_table.clone()
    last = (int(inp.seq_lens[2]) - 1) // P
    bad_pt[2, last] = inp.num_pages + 5
    bad_pt[0, 0] = -3
    _run(dc, plan, ws, dc.seq_lens, bad_pt)
    assert ba.blockattn_input_errors(plan, ws) == ba.BLOCKATTN_INPUT_BAD_PAGE

    # both at once
    _run(dc, plan, ws, bad_lens, bad_pt)
    got = ba.blockattn_input_errors(plan, ws)
    assert got == ba.BLOCKATTN_INPUT_BAD_LENGTH | ba.BLOCKATTN_INPUT_BAD_PAGE

    # an entry past a request's pages is never read, so it is not an error
    spare = dc.page_table.clone()
    used = (int(inp.seq_lens[0]) + P - 1) // P
    if used < stride:
        spare[0, used:] = inp.num_pages + 1000
        _run(dc, plan, ws, dc.seq_lens, spare)
        assert ba.blockattn_input_errors(plan, ws) == 0
    plan.destroy()

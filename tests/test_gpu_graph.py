"""HIP graph capture of the forward calls (MI355X only).

A plan fixes the split counts from host lengths; every forward reads the live
lengths from device memory, so a captured graph replays correctly after the
lengths change in place (within the page table's capacity). Each replay is
checked against the oracle, with eager work and host synchronisation between
replays. The decode-loop test captures the dense-block call with the fused
append and replays it as a drafting loop would: each step appends the new block
at the accepted position and the next step reads it back from the cache.
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


def gcase(idx, *, fp8=False, batch=3, K=4, hq=8, hkv=2, D=64, P=32, ctx=700, wl=-1, wr=-1):
    c = Case(f"gr{idx}", 83, idx, batch=batch, block_size=K, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
             page_size=P, context=ctx, window_left=wl, window_right=wr)
    return fp8_variant(c) if fp8 else c


class Captured:
    """Plan + buffers + one captured forward; lengths live in dc.seq_lens."""

    def __init__(self, dc, kb=None, vb=None, append=False):
        c = dc.inputs.case
        prm = H.params_for(dc)
        lens = dc.inputs.seq_lens
        nbytes = ba.blockattn_workspace_size(prm, lens)
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        self.plan = ba.blockattn_plan(prm, lens, self.ws, nbytes)
        self.out = torch.empty(c.batch, c.block_size, c.num_q_heads, c.head_dim, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(c.batch, c.block_size, c.num_q_heads, dtype=torch.float32, device="cuda")
        self.dc, self.kb, self.vb, self.append = dc, kb, vb, append
        self.call()  # warm-up outside the capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.call()

    def call(self):
        dc = self.dc
        if self.kb is not None:
            ba.blockattn_forward_block(self.plan, dc.q, self.kb, self.vb, dc.k, dc.v, dc.page_table, dc.seq_lens,
                                       self.ws, self.out, self.lse, append=self.append)
        else:
            fwd = ba.blockattn_forward if self.plan.params.window_left == -1 else ba.blockattn_windowed_forward
            fwd(self.plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, self.ws, self.out, self.lse)

    def replay(self):
        self.graph.replay()
        torch.cuda.synchronize()
        return self.out.float().cpu().numpy(), self.lse.cpu().numpy()


GRAPH_CASES = [
    (1, dict()),                                                               # stream kernel, unwindowed
    (2, dict(wl=200, wr=-1)),                                                  # stream kernel, windowed
    (3, dict(K=7, hq=16, hkv=1, D=128, P=64, ctx=1500, wl=300, wr=2)),         # shared tiles
    (4, dict(fp8=True, K=7, hq=16, hkv=1, D=128, P=64, ctx=1500)),
]


@pytest.mark.parametrize("idx,kw", GRAPH_CASES, ids=[f"gr{i}" for i, _ in GRAPH_CASES])
def test_graph_replay_follows_live_lengths(idx, kw):
    c = gcase(idx, **kw)
    inp = synth.make_inputs(c)
    dc = H.upload(inp)
    cap = Captured(dc)
    n0 = inp.seq_lens.copy()
    K = c.block_size
    # shorter live lengths (down to a block alone), and back to the planned ones
    for lens in (n0, n0 - 37, np.maximum(n0 // 3, K), np.full_like(n0, K), n0 - np.arange(len(n0)) * 5, n0):
        lens = lens.astype(np.int32)
        dc.seq_lens.copy_(torch.from_numpy(lens))
        out, lse = cap.replay()
        now = replace(inp, seq_lens=lens)
        ref_out, ref_lse = oracle.attention_case(now)
        H.compare(out, lse, ref_out, ref_lse, label=f"gr{idx} lens={lens.tolist()}")
        # eager call on the same lengths: the same bits
        eager_out, eager_lse, _ = H.run(H.DeviceCase(now, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens),
                                        plan_lens=n0)
        assert np.array_equal(out.view(np.uint32), eager_out.view(np.uint32))
        assert np.array_equal(lse.view(np.uint32), eager_lse.view(np.uint32))
    cap.plan.destroy()


def encode_block(c, kb, vb, k_pool, v_pool, page_table, lens):
    """Store the oracle's encoding of the block at positions lens - K .. lens - 1 of each request."""
    for b in range(c.batch):
        for i in range(c.block_size):
            j = int(lens[b]) - c.block_size + i
            page, slot = int(page_table[b, j // c.page_size]), j % c.page_size
            for h in range(c.num_kv_heads):
                k_pool[page, h, slot, :] = [oracle.encode_kv(c.kv_dtype, c.k_scale, int(x)) for x in kb[b, i, h]]
                v_pool[page, h, slot, :] = [oracle.encode_kv(c.kv_dtype, c.v_scale, int(x)) for x in vb[b, i, h]]


@pytest.mark.parametrize("idx,kw", [(5, dict()), (6, dict(fp8=True, wl=150, wr=-1)),
                                     (7, dict(K=7, hq=16, hkv=1, D=128, P=64, ctx=900, wl=256, wr=-1))],
                         ids=["gr5", "gr6_fp8", "gr7_shared"])
def test_graph_decode_loop_with_fused_append(idx, kw):
    c = gcase(idx, **kw)
    K = c.block_size
    steps = 6
    # pools and page table sized for the longest step (each step accepts 1..K tokens)
    big = replace(c, context=c.context + steps * K)
    inp = synth.make_inputs(big)
    inp = replace(inp, case=c)
    rng = np.random.default_rng(idx)
    ctx = np.full(c.batch, c.context, dtype=np.int32) - rng.integers(0, 50, c.batch).astype(np.int32)
    lens = ctx + K
    k_exp, v_exp = inp.k_pool.copy(), inp.v_pool.copy()
    dc = H.upload(replace(inp, seq_lens=lens))
    shape = (c.batch, K, c.num_kv_heads, c.head_dim)
    kb_dev = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    vb_dev = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    # capture on a copy of the cache, so the warm-up call's append does not touch the tracked one
    k_live, v_live = dc.k.clone(), dc.v.clone()
    cap = Captured(dc, kb_dev, vb_dev, append=True)
    dc.k.copy_(k_live)
    dc.v.copy_(v_live)
    for step in range(steps):
        kb = torch.from_numpy(rng.normal(0, 1.5, shape).astype(np.float32)).to(torch.bfloat16)
        vb = torch.from_numpy(rng.normal(0, 1.5, shape).astype(np.float32)).to(torch.bfloat16)
        kb_bits = kb.view(torch.int16).numpy().view(np.uint16)
        vb_bits = vb.view(torch.int16).numpy().view(np.uint16)
        kb_dev.copy_(kb)
        vb_dev.copy_(vb)
        dc.seq_lens.copy_(torch.from_numpy(lens))
        out, lse = cap.replay()
        now = replace(inp, k_pool=k_exp, v_pool=v_exp, seq_lens=lens.copy())
        ref_out, ref_lse = oracle.attention_case(now, k_block=kb_bits, v_block=vb_bits)
        H.compare(out, lse, ref_out, ref_lse, label=f"gr{idx} step {step}")
        encode_block(c, kb_bits, vb_bits, k_exp, v_exp, inp.page_table, lens)
        got_k = dc.k.view(torch.uint8).cpu().numpy().view(k_exp.dtype).reshape(k_exp.shape)
        got_v = dc.v.view(torch.uint8).cpu().numpy().view(v_exp.dtype).reshape(v_exp.shape)
        np.testing.assert_array_equal(got_k, k_exp, err_msg=f"step {step}")
        np.testing.assert_array_equal(got_v, v_exp, err_msg=f"step {step}")
        lens = lens + rng.integers(1, K + 1, c.batch).astype(np.int32)  # accepted drafts
    cap.plan.destroy()

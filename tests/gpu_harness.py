"""Helpers for the GPU parity tests: upload a case, run the library, compare with the oracle."""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

import speculative_decoding_draft_paged_amd as ba
import synth

# Parity rule: TensorRT-LLM PR #20374, Test Coverage: relative L2 error < 1e-2 and
# max abs difference <= 8 bf16 ulp at the largest expected magnitude. LSE bound 1e-3
# absolute (base 2).
REL_L2 = 1e-2
MAX_ULP = 8
LSE_ABS = 1e-3


def ulp_bf16(x: float) -> float:
    """Spacing of bf16 numbers at magnitude x (8 significand bits)."""
    if x <= 0:
        return 2.0 ** -133
    return 2.0 ** (math.floor(math.log2(x)) - 7)


@dataclass
class DeviceCase:
    inputs: synth.Inputs
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    page_table: torch.Tensor
    seq_lens: torch.Tensor


def upload(inputs: synth.Inputs, device="cuda") -> DeviceCase:
    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    def kv(a):  # bf16 bits, or fp8 E4M3 bytes kept as uint8
        return torch.from_numpy(np.ascontiguousarray(a)).to(device) if a.dtype == np.uint8 else bf(a)

    return DeviceCase(inputs, bf(inputs.q), kv(inputs.k_pool), kv(inputs.v_pool),
                      torch.from_numpy(np.ascontiguousarray(inputs.page_table)).to(device),
                      torch.from_numpy(np.ascontiguousarray(inputs.seq_lens)).to(device))


def params_for(dc: DeviceCase, *, window_left=None, window_right=None, splits=0, scale=None, waves=0,
               combine="auto"):
    c = dc.inputs.case
    return ba.make_params(batch=c.batch, block_size=c.block_size, num_q_heads=c.num_q_heads,
                          num_kv_heads=c.num_kv_heads, head_dim=c.head_dim, page_size=c.page_size,
                          page_table_stride=dc.inputs.page_table.shape[1], num_pages=dc.inputs.num_pages,
                          sm_scale=c.scale if scale is None else scale,
                          window_left=c.window_left if window_left is None else window_left,
                          window_right=c.window_right if window_right is None else window_right,
                          splits_override=splits, waves_override=waves, kv_dtype=c.kv_dtype, k_scale=c.k_scale,
                          v_scale=c.v_scale, combine=combine)


def run(dc: DeviceCase, *, window_left=None, window_right=None, splits=0, plan_lens=None, with_lse=True,
        canary=False, waves=0, combine="auto"):
    """Plan + forward on the current stream; returns (out float32 np, lse np or None, info)."""
    c = dc.inputs.case
    prm = params_for(dc, window_left=window_left, window_right=window_right, splits=splits, waves=waves,
                     combine=combine)
    lens = dc.inputs.seq_lens if plan_lens is None else plan_lens
    nbytes = ba.blockattn_workspace_size(prm, lens)
    guard = 4096 if canary else 0
    ws_all = torch.empty(nbytes + guard, dtype=torch.uint8, device=dc.q.device)
    if canary:
        ws_all[nbytes:] = 0xA5
    ws = ws_all[:nbytes] if nbytes else ws_all[:1]
    plan = ba.blockattn_plan(prm, lens, ws, nbytes)
    out = torch.empty(c.batch, c.block_size, c.num_q_heads, c.head_dim, dtype=torch.bfloat16, device=dc.q.device)
    lse = torch.empty(c.batch, c.block_size, c.num_q_heads, dtype=torch.float32, device=dc.q.device) \
        if (with_lse or prm.window_left != -1) else None
    fwd = ba.blockattn_forward if prm.window_left == -1 else ba.blockattn_windowed_forward
    fwd(plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, ws, out, lse)
    torch.cuda.synchronize()
    # A second call on the same plan and workspace must give the same bits (compared as
    # bits, so NaN outputs of NaN inputs compare equal): nothing a call leaves in the
    # workspace may leak into the next one.
    first = out.clone()
    first_lse = lse.clone() if lse is not None else None
    fwd(plan, dc.q, dc.k, dc.v, dc.page_table, dc.seq_lens, ws, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), first.view(torch.int16)), "second call on the same plan differs"
    if lse is not None:
        assert torch.equal(lse.view(torch.int32), first_lse.view(torch.int32)), \
            "second call on the same plan differs (lse)"
    info = plan.info()
    if canary:
        assert bool((ws_all[nbytes:] == 0xA5).all()), "workspace guard bytes were overwritten"
    plan.destroy()
    return out.float().cpu().numpy(), (lse.cpu().numpy() if lse is not None else None), info


def compare(out, lse, ref_out, ref_lse, *, sel=None, label=""):
    """Apply the parity rule; sel restricts to rows (a boolean mask over [B, K, Hq]) the oracle computed."""
    if sel is not None:
        out, ref_out = out[sel], ref_out[sel]
        if lse is not None:
            lse, ref_lse = lse[sel], ref_lse[sel]
    assert np.isfinite(out).all(), f"{label}: non-finite output"
    diff = np.abs(out.astype(np.float64) - ref_out)
    rel_l2 = float(np.linalg.norm(out.astype(np.float64) - ref_out) / max(np.linalg.norm(ref_out), 1e-300))
    amax = float(np.abs(ref_out).max())
    max_ulp = float(diff.max() / ulp_bf16(amax))
    res = {"rel_l2": rel_l2, "max_abs": float(diff.max()), "max_ulp": max_ulp}
    if lse is not None:
        assert np.isfinite(lse).all(), f"{label}: non-finite lse"
        res["lse_err"] = float(np.abs(lse.astype(np.float64) - ref_lse).max())
    assert rel_l2 < REL_L2, f"{label}: rel L2 {rel_l2:.3e} >= {REL_L2} ({res})"
    assert max_ulp <= MAX_ULP, f"{label}: max abs {res['max_abs']:.3e} = {max_ulp:.2f} ulp > {MAX_ULP} ({res})"
    if lse is not None:
        assert res["lse_err"] <= LSE_ABS, f"{label}: lse error {res['lse_err']:.3e} > {LSE_ABS} ({res})"
    return res

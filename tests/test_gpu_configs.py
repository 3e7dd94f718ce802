"""Parity at the five workload configurations' full sizes (MI355X only).

Every case of every configuration (50 cases) runs through the C ABI in the
default plan, the launch configuration bench.py times. The fp64 oracle then
recomputes a sample of (request, kv head) pairs one by one (the first, the
last and a middle one; more for the small windowed cases) and the sampled
rows must meet the parity rule. A per-case summary line (JSON) is appended to
the file that the environment variable BLOCKATTN_PARITY_LOG names, if set.
"""
import json
import os
import time

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

CASES = synth.all_cases()


def sample_pairs(case):
    B, H_ = case.batch, case.num_kv_heads
    pairs = {(0, 0), (B - 1, H_ - 1), (B // 2, H_ // 2)}
    if case.windowed:  # cheap rows: take more of them, spread over the batch
        rng = np.random.default_rng(case.seed)
        for _ in range(5):
            pairs.add((int(rng.integers(B)), int(rng.integers(H_))))
    return sorted(pairs)


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_config_case(case):
    t0 = time.perf_counter()
    print(f"[{case.name}] generating", flush=True)
    inp = synth.make_inputs(case)
    dc = H.upload(inp)
    t1 = time.perf_counter()
    out, lse, info = H.run(dc)
    del dc
    pairs = sample_pairs(case)
    ref_out, ref_lse = oracle.attention_case(inp, pairs=pairs)
    g = case.group
    sel = np.zeros(out.shape[:3], dtype=bool)
    for b, h in pairs:
        sel[b, :, h * g:(h + 1) * g] = True
    res = H.compare(out, lse, ref_out, ref_lse, sel=sel, label=case.name)
    res.update(case=case.name, pairs=len(pairs), units=info["units"], max_splits=info["max_splits"],
               merge=info["merge_active"], seconds=round(time.perf_counter() - t0, 1),
               gen_seconds=round(t1 - t0, 1))
    print(f"[{case.name}] {res}", flush=True)
    log_path = os.environ.get("BLOCKATTN_PARITY_LOG")
    if log_path:
        with open(log_path, "a") as f:
            f.write(json.dumps(res) + "\n")

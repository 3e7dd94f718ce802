"""Parity at the five workload configurations' full sizes (MI355X only).

Every case of every configuration (50 cases) runs through the C ABI in the
default plan, the launch configuration bench.py times. The fp64 oracle then
recomputes every output row of the call (all (request, kv head) pairs; about
60 ms per pair at 128K on 16 host threads, under two minutes for all cases) and
the whole output and LSE must meet the parity rule. A per-case summary line
(JSON) is appended to the file that the environment variable
BLOCKATTN_PARITY_LOG names, if set.
"""
import json
import os
import time

import pytest

import oracle
import synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

CASES = synth.all_cases()


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_config_case(case):
    t0 = time.perf_counter()
    print(f"[{case.name}] generating", flush=True)
    inp = synth.make_inputs(case)
    dc = H.upload(inp)
    t1 = time.perf_counter()
    out, lse, info = H.run(dc)
    del dc
    print(f"[{case.name}] GPU done after {t1 - t0:.1f}s of generation; oracle on every row", flush=True)
    t2 = time.perf_counter()
    ref_out, ref_lse = oracle.attention_case(inp)
    res = H.compare(out, lse, ref_out, ref_lse, label=case.name)
    res.update(case=case.name, pairs=case.batch * case.num_kv_heads, units=info["units"],
               max_splits=info["max_splits"], merge=info["merge_active"], seconds=round(time.perf_counter() - t0, 1),
               gen_seconds=round(t1 - t0, 1), oracle_seconds=round(time.perf_counter() - t2, 1))
    print(f"[{case.name}] {res}", flush=True)
    log_path = os.environ.get("BLOCKATTN_PARITY_LOG")
    if log_path:
        with open(log_path, "a") as f:
            f.write(json.dumps(res) + "\n")

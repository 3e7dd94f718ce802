"""The benchmark's host-side accounting (no GPU): algorithmic bytes, the multi-GPU refusal and the
HBM-counter summary."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth
from synth.configs import Case, find_case, fp8_variant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bytes_by_key(case, seq_lens, block):
    """Count every key a row of the call needs, one by one, from the key-set definition."""
    eb = 1 if case.kv_dtype == "fp8_e4m3" else 2
    K, D, H = case.block_size, case.head_dim, case.num_kv_heads
    total = 0
    for n in seq_lens.tolist():
        c = n - K
        needed = set()
        for i in range(K):
            p = c + i
            if case.window_left > 0:
                right = K if case.window_right < 0 else case.window_right
                needed.update(range(max(0, p - case.window_left + 1), min(n - 1, p + right) + 1))
            else:
                needed.update(range(n))
        for j in needed:
            from_arrays = block != "cache" and j >= c
            total += H * 2 * D * (2 if from_arrays else eb)  # K and V of key j
        if block == "append":
            total += H * K * 2 * D * eb  # the block written into the cache
    return total


CASES = [
    Case("h1", 91, 1, batch=3, block_size=7, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32,
         context_range=(0, 900)),
    Case("h2", 91, 2, batch=2, block_size=3, num_q_heads=16, num_kv_heads=1, head_dim=128, page_size=64,
         context_range=(100, 2000), window_left=300, window_right=-1),
    Case("h3", 91, 3, batch=2, block_size=5, num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16,
         context_range=(0, 50), window_left=2, window_right=0),
]


@pytest.mark.parametrize("block", ["cache", "dense", "append"])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("idx", range(len(CASES)))
def test_algorithmic_bytes_match_the_key_sets(idx, fp8, block):
    c = fp8_variant(CASES[idx]) if fp8 else CASES[idx]
    lens = synth.seq_lens_for(c)
    assert bench.kv_bytes(c, lens, block) == bytes_by_key(c, lens, block)


def test_headline_bytes():
    c = find_case("cfg2_b8_128k")
    assert bench.kv_bytes(c, synth.seq_lens_for(c)) == 8 * 2 * 131079 * 4 * 64


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_reference_copy(tmp_path):
    # the reference copy reads 1 GiB and writes 1 GiB; its counters read half and all of that
    gib_kib = bench.COPY_ELEMS * 4 / 1024
    write_counters(str(tmp_path / "f"), "FETCH_SIZE", [("void at::native::neg_kernel", gib_kib / 2),
                                                       ("stream_kernel<64>", 1000.0), ("stream_kernel<64>", 1200.0),
                                                       ("combine_kernel<64>", 5.0)])
    write_counters(str(tmp_path / "w"), "WRITE_SIZE", [("void at::native::neg_kernel", gib_kib),
                                                       ("shared_kernel<128>", 10.0)])
    rec = bench.pmc_summary("x", str(tmp_path / "f"), str(tmp_path / "w"))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == int(1100.0 * 1024 * 2.0)
    assert rec["write_bytes_per_launch"] == 10 * 1024
    assert rec["hbm_bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["kernel_digest"] == bench.kernel_source_digest()


def test_mfma_summary_averages_the_attention_kernel_only(tmp_path):
    path = str(tmp_path / "m")
    os.makedirs(path)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, util in (("stream_kernel<64>", 6.0), ("stream_kernel<64>", 7.0), ("combine_kernel<64>", 50.0)):
            for counter, value in (("MfmaUtil", util), ("VALUBusy", 2 * util), ("LdsUtil", util / 2),
                                   ("GRBM_GUI_ACTIVE", 1000.0)):
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
    rec = bench.mfma_summary("x", path)
    assert rec["MfmaUtil"] == pytest.approx(6.5) and rec["VALUBusy"] == pytest.approx(13.0)
    assert rec["LdsUtil"] == pytest.approx(3.25) and rec["dispatches"] == 2
    assert rec["kernel_digest"] == bench.kernel_source_digest()


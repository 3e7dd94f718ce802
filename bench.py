#!/usr/bin/env python3
"""Benchmark of draft-block paged attention on one MI355X.

Workload (default): the Kimi-style TP8 rank of a 64q/16kv GQA drafter, i.e.
8 q / 2 kv heads, head_dim 64, block K = 7, 128K-token contexts, page 32, HND
bf16 pools, B = 8 requests with disjoint shuffled page ranges; synthetic N(0,1)
data from the seeded generator. One step = one blockattn_forward call for the
whole batch (plan once, outside timing): the paged attention kernel and, when
the plan splits a request's keys, the LSE combine.

Timing: the K timed steps are one captured HIP graph, replayed R >= 10 times,
each replay between two device synchronisations and timed with HIP events; the
per-call time is the median replay / K. Each step reads the next of M copies of
the K/V pools (M * bytes read per call >= 1 GiB, M at most the step count) so
the 256 MB Infinity Cache cannot serve repeats. HIP events recorded around every
attention-kernel launch give that kernel's average duration (a separate pass of
K eager calls), from which the roofline fraction is computed. HBM traffic per
launch comes from a committed rocprofv3 counter summary of the same kernel
source (null when the source has changed since).

Output: one JSON line (metric, value in GB/s of algorithmic KV bytes, ...,
roofline, cpu_baseline, read_reference, cases). The cpu_baseline leg times the
fp64 oracle on a bounded sample of the same workload on the host cores;
read_reference is the read-only streaming kernel over 2 GiB (the achievable HBM
read rate); cases repeats the measurement for every 128K-context configuration
case (per-call time, kernel time, fraction of 8 TB/s).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "us per block-attention call and achieved HBM GB/s (KV read) vs MI355X peak"
# Pages' number for this workload (TensorRT-LLM PR #20374, B > 1 comment): 8q/2kv heads, D 64,
# page 32, K 7, 128K context, B = 8, decode-row form: 252.4 us per attention op on SM107.
# Unique KV bytes / time = 536.9 MB / 252.4 us = 2127 GB/s. Another machine: context only.
PAGES_CONTEXT = {"cfg2_b8_128k": 536_895_488 / 252.4e-6 / 1e9, "cfg2_b16_128k": 1_073_790_976 / 492.9e-6 / 1e9,
                 "cfg2_b8_32k": 134_246_400 / 65.7e-6 / 1e9, "cfg2_b16_32k": 268_492_800 / 131.3e-6 / 1e9}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kv_bytes(case, seq_lens, block="cache") -> int:
    """Algorithmic KV bytes of one call: every key a row needs, read once (K and V, 2 B each for bf16, 1 for fp8).

    block "dense": the K block keys and values come from dense bf16 arrays (2 B each) instead of the
    cache; "append": the same, plus writing them into the cache (K and V, at the cache's element size).
    """
    eb = 1 if case.kv_dtype == "fp8_e4m3" else 2
    K, D = case.block_size, case.head_dim
    total = 0
    for n in seq_lens.tolist():
        c = n - K
        lo = max(0, c - case.window_left + 1) if case.window_left > 0 else 0
        if block == "cache":
            total += case.num_kv_heads * (n - lo) * 2 * eb * D
        else:
            total += case.num_kv_heads * ((c - lo) * 2 * eb * D + K * 2 * 2 * D)
            if block == "append":
                total += case.num_kv_heads * K * 2 * eb * D
    return total


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch loaded (shared with the library)."""

    def __init__(self):
        import torch

        lib_dir = os.path.join(os.path.dirname(torch.__file__), "lib")
        path = os.path.join(lib_dir, "libamdhip64.so")
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in ("attention_kernels.h", "kernels_bf16.hip", "kernels_fp8.hip", "api.cpp", "internal.h"):
        with open(os.path.join(ROOT, "speculative_decoding_draft_paged_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(case_name: str, per_launch_bytes: int):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, if it matches the current kernels."""
    path = os.path.join(ROOT, "profiles", f"pmc_partial_{case_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_digest") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


TRACE_PHASES = ("entry", "length", "pages", "loop", "epilogue", "stored")


def phase_stats(calls):
    """Per-unit phase timestamps (100 MHz ticks, [units, 8] per traced call) as a timeline in us.

    For each call, times are taken from the earliest unit entry; each statistic is the median
    over units (and the max for the ends), then the median over calls."""
    import numpy as np

    per_call = []
    for tr in calls:
        tr = tr.astype(np.int64)
        e, ln, pg, lp, ep, st = (tr[:, k] for k in range(6))
        ok = (e > 0) & (ln > 0) & (pg > 0) & (lp > 0) & (st > 0)
        e, ln, pg, lp, ep, st = e[ok], ln[ok], pg[ok], lp[ok], ep[ok], st[ok]
        t0 = e.min()
        us = lambda x: x * 0.01  # 10 ns per tick
        has_ep = bool((ep > 0).all())
        row = {
            "units_traced": int(ok.sum()),
            "entry_spread_us": us(e.max() - t0),
            "entry_median_us": us(np.median(e - t0)),
            "length_latency_us": us(np.median(ln - e)),
            "pages_latency_us": us(np.median(pg - ln)),
            "loop_us": us(np.median(lp - pg)),
            "slowest_group_wait_us": us(np.median(ep - lp)) if has_ep else 0.0,
            "epilogue_us": us(np.median(st - (ep if has_ep else lp))),
            "unit_end_median_us": us(np.median(st - t0)),
            "unit_end_max_us": us(st.max() - t0),
            "unit_end_p10_us": us(np.percentile(st - t0, 10)),
            "unit_end_p90_us": us(np.percentile(st - t0, 90)),
        }
        per_call.append(row)
    out = {k: (round(float(np.median([r[k] for r in per_call])), 3) if k != "units_traced" else per_call[0][k])
           for k in per_call[0]}
    out["calls"] = len(per_call)
    return out


def run_case(case, steps, warmup, threads, graph=True, splits=0, waves=0, block="cache", replays=10,
             trace_calls=0, combine="auto"):
    import numpy as np
    import torch

    import speculative_decoding_draft_paged_amd as ba
    import synth

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    inp = synth.make_inputs(case, threads=threads)
    log(f"[bench] {case.name}: inputs generated in {time.perf_counter() - t0:.1f}s "
        f"(pool {inp.k_pool.nbytes / 2**20:.0f} MiB per tensor)")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    q = bf(inp.q)
    kv = (lambda a: torch.from_numpy(a).to(dev)) if inp.k_pool.dtype == np.uint8 else bf
    k0, v0 = kv(inp.k_pool), kv(inp.v_pool)
    pt = torch.from_numpy(inp.page_table).to(dev)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    # Copies of the pools, rotated call by call, so that the calls between two reads of
    # one copy read at least 1 GiB: the 256 MB Infinity Cache then cannot serve repeats.
    # A call reads only its key sets (a windowed call far less than the pools hold), so
    # the count follows the bytes read per call, up to one copy per timed call and 16 GiB
    # of copies. Below about 50 MB per call the timed calls' whole read set fits the
    # cache at the default step count; those cases are latency-bound either way.
    pool_bytes = 2 * inp.k_pool.nbytes
    read_bytes = max(1, kv_bytes(case, inp.seq_lens, block))
    copies = max(1, min(math.ceil((1 << 30) / read_bytes), max(steps, 1), (16 << 30) // pool_bytes))
    ks, vs = [k0], [v0]
    for _ in range(copies - 1):
        ks.append(k0.clone())
        vs.append(v0.clone())
    prm = ba.make_params(batch=case.batch, block_size=case.block_size, num_q_heads=case.num_q_heads,
                         num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, page_size=case.page_size,
                         page_table_stride=inp.page_table.shape[1], num_pages=inp.num_pages, sm_scale=case.scale,
                         window_left=case.window_left, window_right=case.window_right, splits_override=splits,
                         waves_override=waves, kv_dtype=case.kv_dtype, k_scale=case.k_scale, v_scale=case.v_scale,
                         combine=combine)
    nbytes = ba.blockattn_workspace_size(prm, inp.seq_lens)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    plan = ba.blockattn_plan(prm, inp.seq_lens, ws, nbytes)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    fwd = ba.blockattn_windowed_forward if case.windowed else ba.blockattn_forward
    blocks = None
    if block != "cache":
        blocks = synth.make_block(case, threads=threads)
        kb, vb = bf(blocks[0]), bf(blocks[1])

    def step(i):
        if blocks is None:
            fwd(plan, q, ks[i % copies], vs[i % copies], pt, lens, ws, out, lse)
        else:
            ba.blockattn_forward_block(plan, q, kb, vb, ks[i % copies], vs[i % copies], pt, lens, ws, out, lse,
                                       append=block == "append")

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ref_out = out.clone()

    hip = HipEvents()
    ga, gb = hip.create(2)
    stream = torch.cuda.current_stream()
    used_graph = False
    if graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    step(i)
            g.replay()  # untimed: warms the graph; its result must equal the eager result
            torch.cuda.synchronize()
            if not torch.equal(out, ref_out):
                raise RuntimeError("graph replay output differs from the eager output")
            used_graph = True
        except Exception as e:
            log(f"[bench] graph capture unavailable ({e}); timing eager launches")
            torch.cuda.synchronize()

    # Timed regions: `replays` runs of exactly `steps` forward calls (one graph replay, or the
    # eager calls), each between two device synchronisations and timed with HIP events on the
    # launch stream; the per-call time is the median over the runs.
    run_ms, walls = [], []
    for _ in range(max(1, replays)):
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        hip.hip.hipEventRecord(ctypes.c_void_p(ga), ctypes.c_void_p(stream.cuda_stream))
        if used_graph:
            g.replay()
        else:
            for i in range(steps):
                step(i)
        hip.hip.hipEventRecord(ctypes.c_void_p(gb), ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t_start)
        run_ms.append(hip.elapsed_ms(ga, gb))
    if not torch.equal(out, ref_out):
        raise RuntimeError("timed run output differs from the warm-up output")
    total_ms = float(np.median(run_ms))
    wall = float(np.median(walls))

    # Kernel timing: HIP events recorded by the library right around every attention-kernel
    # launch, on the stream it launches on, over `steps` eager calls.
    before, after = hip.create(steps), hip.create(steps)
    for i in range(steps):
        ba.blockattn_plan_set_profile_events(plan, before[i], after[i])
        step(i)
    ba.blockattn_plan_set_profile_events(plan, None, None)
    torch.cuda.synchronize()
    kern_ms = [hip.elapsed_ms(before[i], after[i]) for i in range(steps)]
    timing = "eager"
    hip.destroy(before + after + [ga, gb])
    info = plan.info()
    phases = None
    if trace_calls > 0:
        # Traced eager calls: per-unit phase timestamps, and the attention kernel's event time of
        # the same calls (the trace's waits make them a little slower than untraced calls).
        tr = torch.zeros(info["units"] * 8, dtype=torch.int64, device=dev)
        ba.blockattn_plan_set_phase_trace(plan, tr)
        tb, ta = hip.create(trace_calls), hip.create(trace_calls)
        calls = []
        for i in range(trace_calls):
            tr.zero_()
            ba.blockattn_plan_set_profile_events(plan, tb[i], ta[i])
            step(i)
            torch.cuda.synchronize()
            calls.append(tr.view(info["units"], 8).cpu().numpy())
        ba.blockattn_plan_set_profile_events(plan, None, None)
        ba.blockattn_plan_set_phase_trace(plan, None)
        phases = phase_stats(calls)
        phases["traced_kernel_event_us"] = round(float(np.median([hip.elapsed_ms(tb[i], ta[i]) for i in
                                                                   range(trace_calls)])) * 1e3, 2)
        hip.destroy(tb + ta)
    res = {
        "case": case.name,
        "kv_bytes": kv_bytes(case, inp.seq_lens, block),
        "block": block,
        "step_ms": total_ms / steps,
        "step_ms_min": min(run_ms) / steps,
        "step_ms_max": max(run_ms) / steps,
        "replays": len(run_ms),
        "wall_ms": wall * 1e3 / steps,
        "partial_ms": sum(kern_ms) / len(kern_ms),
        "partial_ms_min": min(kern_ms),
        "graph": used_graph,
        "kernel_timing": timing,
        "copies": copies,
        "units": info["units"],
        "max_splits": info["max_splits"],
        "waves_per_unit": info["waves_per_unit"],
        "shared_tiles": info["shared_tiles"],
        "combine_launch": info["combine_launch"],
        "fused_combine": info["fused_combine"],
        "phases": phases,
    }
    plan.destroy()
    return res, inp, out, blocks


READ_BYTES = 2 << 30  # the read-only streaming reference reads 2 GiB per launch


def read_reference(reps=20):
    """The read-only streaming reference: blockattn_stream_read over 2 GiB (every byte read once with
    the attention kernels' 16-byte non-temporal loads), median of `reps` launches timed with HIP
    events, at five launch widths; the best median is the box's achievable HBM read rate."""
    import numpy as np
    import torch

    import speculative_decoding_draft_paged_amd as ba

    src = torch.ones(READ_BYTES // 4, dtype=torch.int32, device="cuda")
    acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    hip = HipEvents()
    evs = hip.create(2 * reps)
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for wg in (256, 512, 1024, 2048, 4096):
        for _ in range(3):
            ba.blockattn_stream_read(src, acc, wg)
        torch.cuda.synchronize()
        for r in range(reps):
            hip.hip.hipEventRecord(ctypes.c_void_p(evs[2 * r]), ctypes.c_void_p(stream))
            ba.blockattn_stream_read(src, acc, wg)
            hip.hip.hipEventRecord(ctypes.c_void_p(evs[2 * r + 1]), ctypes.c_void_p(stream))
        torch.cuda.synchronize()
        us = float(np.median([hip.elapsed_ms(evs[2 * r], evs[2 * r + 1]) for r in range(reps)])) * 1e3
        if best is None or us < best["us"]:
            best = {"kernel": "blockattn_stream_read, 2 GiB read once (16-byte non-temporal loads, a contiguous "
                              "range per workgroup)", "workgroups": wg,
                    "us": round(us, 1), "gbs": round(READ_BYTES / (us * 1e-6) / 1e9, 1), "reps": reps}
    hip.destroy(evs)
    best["frac_of_peak"] = round(best["gbs"] / HBM_PEAK_GBS, 4)
    del src, acc
    torch.cuda.empty_cache()
    log(f"[bench] read reference: {best}")
    return best


COPY_ELEMS = 1 << 28  # float32 elements of the reference copy: 1 GiB read + 1 GiB written per launch


def copy_reference(reps=10):
    """A plain elementwise kernel of known traffic: y = -x over 1 GiB of float32.

    Its HBM rate (read + written bytes / time) is the box's achievable streaming
    reference, and its PMC byte counters calibrate FETCH_SIZE / WRITE_SIZE (the
    kernel moves exactly 1 GiB each way per launch)."""
    import torch

    x = torch.ones(COPY_ELEMS, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    res = {"kernel": "torch.neg float32, 1 GiB in + 1 GiB out", "us": round(dt * 1e6, 1),
           "gbs_read_plus_write": round(2 * x.numel() * 4 / dt / 1e9, 1)}
    del x, y
    torch.cuda.empty_cache()
    log(f"[bench] copy reference: {res}")
    return res


def _counter_rows(path):
    """Rows (kernel name, counter, value) of a rocprofv3 counter_collection.csv (file or folder)."""
    import csv
    import glob

    files = [path] if os.path.isfile(path) else sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"),
                                                                 recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def pmc_summary(case_name, fetch_path, write_path):
    """Turn a FETCH_SIZE run and a WRITE_SIZE run into HBM bytes per attention-kernel launch.

    Both counters are KiB per dispatch. Each is scaled by the factor that maps the
    reference copy's reading onto its known 1 GiB, then averaged over the
    attention-kernel dispatches (stream_kernel or shared_kernel) of the run."""
    out = {"case": case_name, "kernel_digest": kernel_source_digest()}
    for tag, path, counter in (("fetch", fetch_path, "FETCH_SIZE"), ("write", write_path, "WRITE_SIZE")):
        rows = [r for r in _counter_rows(path) if r[1] == counter]
        att = [v for k, _, v in rows if "stream_kernel" in k or "shared_kernel" in k]
        ref = [v for k, _, v in rows if "neg" in k.lower()]
        if not att or not ref:
            raise SystemExit(f"{path}: {counter} rows for the attention kernel ({len(att)}) or the copy ({len(ref)}) missing")
        ref_kib = sum(ref) / len(ref)
        factor = (COPY_ELEMS * 4 / 1024) / ref_kib
        out[f"{tag}_kib_raw"] = round(sum(att) / len(att), 1)
        out[f"{tag}_copy_kib_raw"] = round(ref_kib, 1)
        out[f"{tag}_scale"] = round(factor, 5)
        out[f"{tag}_bytes_per_launch"] = int(sum(att) / len(att) * 1024 * factor)
        out[f"{tag}_dispatches"] = len(att)
    out["hbm_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    return out


MFMA_COUNTERS = ("MfmaUtil", "VALUBusy", "LdsUtil", "GRBM_GUI_ACTIVE")


def mfma_summary(case_name, path):
    """Matrix-core, vector-ALU and LDS utilisation of the attention kernel from one rocprofv3
    --pmc run of MFMA_COUNTERS (rocprofv3's derived metrics: MfmaUtil = MFMA-busy cycles
    summed over SIMDs / (GPU-active cycles x SIMDs), in percent; VALUBusy and LdsUtil
    likewise per CU), averaged over the attention-kernel dispatches of the run."""
    out = {"case": case_name, "kernel_digest": kernel_source_digest()}
    rows = _counter_rows(path)
    for counter in MFMA_COUNTERS:
        att = [v for k, c, v in rows if c == counter and ("stream_kernel" in k or "shared_kernel" in k)]
        if not att:
            raise SystemExit(f"{path}: no {counter} rows for the attention kernel")
        out[counter] = round(sum(att) / len(att), 3)
        out["dispatches"] = len(att)
    return out


def load_mfma(case_name: str):
    """MfmaUtil (percent) of the attention kernel from a committed summary of the current kernels."""
    path = os.path.join(ROOT, "profiles", f"pmc_mfma_{case_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_digest") != kernel_source_digest():
        return None
    return rec.get("MfmaUtil")


def cpu_baseline(case, inp, gpu_out, kv_total, budget_s, blocks=None):
    """Time the fp64 oracle on a bounded sample of (request, kv head) pairs of the same call."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    pairs_all = [(b, h) for b in range(case.batch) for h in range(case.num_kv_heads)]
    kb, vb = blocks if blocks is not None else (None, None)
    t0 = time.perf_counter()
    out, lse = oracle.attention_case(inp, pairs=pairs_all[:1], threads=threads, k_block=kb, v_block=vb)
    t1 = time.perf_counter() - t0
    n = max(1, min(len(pairs_all), int(budget_s / max(t1, 1e-3))))
    sample = pairs_all[:n]
    if n > 1:
        t0 = time.perf_counter()
        out, lse = oracle.attention_case(inp, pairs=sample, threads=threads, k_block=kb, v_block=vb)
        t1 = time.perf_counter() - t0
    per_pair = t1 / len(sample)
    full_s = per_pair * len(pairs_all)
    g = case.group
    sel = np.zeros(out.shape[:3], dtype=bool)
    for b, h in sample:
        sel[b, :, h * g:(h + 1) * g] = True
    got = gpu_out.float().cpu().numpy().astype(np.float64)
    diff = got[sel] - out[sel]
    amax = float(np.abs(out[sel]).max())
    ulp = 2.0 ** (math.floor(math.log2(amax)) - 7)
    return {
        "value": kv_total / full_s / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(sample)} of {len(pairs_all)} (request, kv head) pairs of the same call, "
                  f"{t1:.1f} s fp64, scaled to the whole call ({full_s * 1e6:.0f} us per call)",
        "us_per_call": full_s * 1e6,
        "sample_parity": {"rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(out[sel])),
                          "max_ulp": float(np.abs(diff).max() / ulp)},
    }


def write_phase_summary(name, row, args):
    """profiles/phases_<case>.md: the traced phase timeline of the attention kernel for one case."""
    ph = row["phases"]
    cmd = "python bench.py " + " ".join(sys.argv[1:])
    lines = [
        f"# Phase timeline of the attention kernel: {name}",
        "",
        f"Command: `{cmd}`",
        "",
        f"Kernel source digest {kernel_source_digest()}. One traced eager call = one `blockattn_forward` for the "
        f"whole batch; {ph['calls']} traced calls, {ph['units_traced']} work units each; every figure is the "
        "median over units (ends also as p10 / p90 / max), then the median over calls. Times in us from the "
        "earliest unit's first instruction, in the GPU's 100 MHz constant clock. Each phase ends when the "
        "unit's memory operations in flight have completed, so traced calls run a little slower than untraced ones.",
        "",
        "| phase | us |",
        "|---|---|",
        f"| untraced call (graph replays, median) | {row['us_per_call']} |",
        f"| untraced attention kernel (HIP events) | {row['kernel_us']} |",
        f"| traced attention kernel (HIP events) | {ph['traced_kernel_event_us']} |",
        f"| last unit entry after the first (dispatch spread) | {ph['entry_spread_us']} |",
        f"| sequence length loaded, after entry | {ph['length_latency_us']} |",
        f"| first page ids staged, after the length | {ph['pages_latency_us']} |",
        f"| token group 0's tile loop | {ph['loop_us']} |",
        f"| wait for the unit's slowest token group | {ph['slowest_group_wait_us']} |",
        f"| epilogue (merge of token groups, stores complete) | {ph['epilogue_us']} |",
        f"| unit end: median / p10 / p90 / max | {ph['unit_end_median_us']} / {ph['unit_end_p10_us']} / "
        f"{ph['unit_end_p90_us']} / {ph['unit_end_max_us']} |",
        "",
        f"Per call: {row['kv_bytes']} bytes of KV, {row['units']} units, at most {row['max_splits']} splits per "
        f"(request, kv head); combine launch: {'yes' if row['combine_launch'] else 'no'}.",
        "",
    ]
    with open(os.path.join(ROOT, args.summary_dir, f"phases_{name}.md"), "w") as f:
        f.write("\n".join(lines))


def case_list(spec):
    """Names of the per-case array: the ten 128K-context cases by default."""
    from synth.configs import all_cases

    if spec == "none":
        return []
    if spec == "128k":
        return [c.name for c in all_cases() if c.context == 131072]
    if spec == "all":
        return [c.name for c in all_cases()]
    return [n for n in spec.split(",") if n]


def per_case_array(names, head_case, head_res, args, threads):
    """One entry per case: median per-call time over graph replays, the attention kernel's HIP-event
    time, and both as GB/s of algorithmic KV bytes and as a fraction of 8 TB/s. The headline case is
    not run again."""
    import torch

    from synth.configs import find_case

    rows = []
    for name in names:
        c = find_case(name)
        if name == head_case.name and args.block == "cache" and not args.splits and not args.waves:
            r = head_res
        else:
            r, _, _, _ = run_case(c, args.case_steps, 3, threads, graph=not args.eager, replays=args.replays,
                                  trace_calls=args.phase_trace, combine=args.combine)
            torch.cuda.empty_cache()
        gbs = r["kv_bytes"] / (r["step_ms"] * 1e-3) / 1e9
        kgbs = r["kv_bytes"] / (r["partial_ms"] * 1e-3) / 1e9
        row = {"case": name, "kv_dtype": c.kv_dtype, "batch": c.batch, "context": c.context, "kv_bytes": r["kv_bytes"],
               "us_per_call": round(r["step_ms"] * 1e3, 2), "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
               "kernel_us": round(r["partial_ms"] * 1e3, 2), "kernel_frac": round(kgbs / HBM_PEAK_GBS, 4),
               "us_min": round(r["step_ms_min"] * 1e3, 2), "us_max": round(r["step_ms_max"] * 1e3, 2),
               "steps": args.case_steps if r is not head_res else args.steps, "replays": r["replays"],
               "units": r["units"], "max_splits": r["max_splits"], "combine_launch": r["combine_launch"],
               "fused_combine": r["fused_combine"]}
        if r.get("phases"):
            row["phases"] = r["phases"]
            if args.phase_summary:
                write_phase_summary(name, row, args)
        rows.append(row)
        log(f"[case] {name:16s} {row['us_per_call']:9.2f} us/call  {gbs:7.0f} GB/s  ({100 * row['frac']:5.1f} % of 8 TB/s)"
            f"  kernel {row['kernel_us']:9.2f} us ({100 * row['kernel_frac']:5.1f} %)  units {row['units']}")
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--case", default="cfg2_b8_128k", help="workload case name (see synth/configs.py)")
    ap.add_argument("--sweep", action="store_true", help="also time every case of the same config (stderr)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU budget of the oracle sample")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--splits", type=int, default=0, help="force the split count per (request, kv head)")
    ap.add_argument("--waves", type=int, default=0, help="force the tile-streaming waves per workgroup")
    ap.add_argument("--combine", choices=("auto", "kernel", "last_arriver"), default="auto",
                    help="split combine: the plan's choice, the combine kernel, or the last split inside the "
                         "attention kernel")
    ap.add_argument("--block", choices=("cache", "dense", "append"), default="cache",
                    help="where the block's keys and values come from: the cache (default), dense arrays, or "
                         "dense arrays also appended into the cache in the same call")
    ap.add_argument("--replays", type=int, default=10,
                    help="timed runs of the K steps (graph replays); the per-call time is their median")
    ap.add_argument("--cases", default="128k",
                    help="per-case array in the same line: '128k' (the ten 128K-context cases, default), 'all', "
                         "'none', or a comma-separated list of case names")
    ap.add_argument("--case-steps", type=int, default=50,
                    help="calls per timed run for the per-case array (the headline's count by default)")
    ap.add_argument("--no-read-reference", action="store_true", help="skip the read-only 2 GiB streaming reference")
    ap.add_argument("--phase-trace", type=int, default=0, metavar="CALLS",
                    help="also trace CALLS eager calls of each timed case (per-unit phase timestamps) and report "
                         "the phase timeline; with --phase-summary, write it to profiles/phases_<case>.md")
    ap.add_argument("--phase-summary", action="store_true",
                    help="write the phase timelines to <summary-dir>/phases_<case>.md (needs --phase-trace)")
    ap.add_argument("--summary-dir", default="profiles", help="folder (under the repository) for --phase-summary")
    ap.add_argument("--copy-reference", action="store_true",
                    help="also time a plain 1 GiB elementwise copy (achievable HBM rate; PMC calibration kernel)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH", "WRITE"),
                    help="no GPU: read two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) of a --copy-reference "
                         "run of --case (and --block) and write profiles/pmc_partial_<case>[_<block>].json")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="no GPU: read a rocprofv3 --pmc run of " + " ".join(MFMA_COUNTERS) + " of --case (and "
                         "--block) and write profiles/pmc_mfma_<case>[_<block>].json")
    args = ap.parse_args()

    label = args.case if args.block == "cache" else f"{args.case}_{args.block}"
    if args.pmc_summary:
        rec = pmc_summary(label, *args.pmc_summary)
        with open(os.path.join(ROOT, "profiles", f"pmc_partial_{label}.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.mfma_summary:
        rec = mfma_summary(label, args.mfma_summary)
        with open(os.path.join(ROOT, "profiles", f"pmc_mfma_{label}.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; the path shards by request or kv head "
                                   "with no exchange, so no multi-GPU figure is measured", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from synth.configs import cases_for_config, find_case, fp8_variant

    threads = min(16, len(os.sched_getaffinity(0)))

    case = find_case(args.case)
    res, inp, out, blocks = run_case(case, args.steps, args.warmup, threads, graph=not args.eager,
                                     splits=args.splits, waves=args.waves, block=args.block, replays=args.replays,
                                     trace_calls=args.phase_trace, combine=args.combine)
    kvb = res["kv_bytes"]
    value = kvb / (res["step_ms"] * 1e-3) / 1e9
    achieved = kvb / (res["partial_ms"] * 1e-3) / 1e9
    log(f"[bench] {case.name}: step {res['step_ms'] * 1e3:.1f} us, attention kernel {res['partial_ms'] * 1e3:.1f} us "
        f"(min {res['partial_ms_min'] * 1e3:.1f}), {value:.0f} GB/s per step, {achieved:.0f} GB/s in the partial "
        f"kernel, units {res['units']}, splits {res['max_splits']}, graph {res['graph']}")

    sweep = None
    if args.sweep:
        sweep = []
        for c in cases_for_config(case.cfg):
            if case.kv_dtype != "bf16":
                c = fp8_variant(c, case.k_scale, case.v_scale)
            r, _, _, _ = run_case(c, max(10, args.steps // 2), 3, threads, graph=not args.eager,
                                  splits=args.splits, waves=args.waves, block=args.block, replays=args.replays,
                                  combine=args.combine)
            r["gbs"] = r["kv_bytes"] / (r["step_ms"] * 1e-3) / 1e9
            r["frac"] = r["gbs"] / HBM_PEAK_GBS
            r["partial_gbs"] = r["kv_bytes"] / (r["partial_ms"] * 1e-3) / 1e9
            sweep.append(r)
            log(f"[sweep] {c.name:16s} {r['step_ms'] * 1e3:9.1f} us  {r['gbs']:7.0f} GB/s  "
                f"({100 * r['frac']:5.1f} % of 8 TB/s)  partial {r['partial_ms'] * 1e3:9.1f} us "
                f"{r['partial_gbs']:7.0f} GB/s  units {r['units']}")
            torch.cuda.empty_cache()

    copy_ref = copy_reference() if args.copy_reference else None
    read_ref = None if args.no_read_reference else read_reference()
    traffic = load_traffic(label, kvb)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "us_per_call": round(res["step_ms"] * 1e3, 2),
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / PAGES_CONTEXT[case.name], 3) if case.name in PAGES_CONTEXT else None),
        "vs_baseline_note": "ratio to the pages' SM107 decode-row figure for the same shape (another GPU: context)"
                            if case.name in PAGES_CONTEXT else None,
        "dtype": case.kv_dtype,
        "data": "synthetic",
        "config": {"workload": f"{case.name}: draft-block attention, {case.num_q_heads}q/{case.num_kv_heads}kv heads, "
                               f"head_dim {case.head_dim}, K={case.block_size}, page {case.page_size}, "
                               f"{'windowed W=%d' % case.window_left if case.windowed else 'unwindowed'}"
                               + {"cache": "", "dense": ", block K/V from dense arrays",
                                  "append": ", block K/V from dense arrays and appended to the cache"}[args.block],
                   "block_kv": args.block,
                   "batch": case.batch, "context": case.context, "kv_dtype": case.kv_dtype,
                   "k_scale": case.k_scale, "v_scale": case.v_scale, "kv_bytes_per_call": kvb,
                   "pool_copies_rotated": res["copies"], "hip_graph": res["graph"], "units": res["units"],
                   "max_splits": res["max_splits"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": ("shared_kernel" if res["shared_tiles"] else "stream_kernel") +
                               " (split-KV paged attention)",
                     "kernel_us": round(res["partial_ms"] * 1e3, 2), "kernel_events": res["kernel_timing"],
                     "mfma_busy_pct": load_mfma(label)},
        "cpu_baseline": None,
    }
    if read_ref is not None:
        line["read_reference"] = read_ref
    if copy_ref is not None:
        line["copy_reference"] = copy_ref
    if sweep is not None:
        line["sweep"] = [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in sweep]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, inp, out, kvb, args.cpu_seconds, blocks)
    del inp, out, blocks
    names = case_list(args.cases)
    if names:
        line["cases"] = per_case_array(names, case, res, args, threads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

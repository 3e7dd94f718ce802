"""Seeded synthetic inputs shared by the oracle, the GPU tests and the benchmark.

The arrays come from ``synth.c`` (a counter-based SplitMix64 stream, Box-Muller
normals rounded to bf16). Nothing here computes attention: it draws numbers and
lays them out in the paged "HND" pools the kernels read.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

from .configs import Case, all_cases, cases_for_config  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

BF16_NAN = 0x7FC0
FP8_NAN = 0x7F  # OCP E4M3 NaN


def build() -> str:
    """Compile ``libsynth.so`` with gcc (plain C, pthreads)."""
    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-o", _LIB_PATH + ".tmp", src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    ptr = ctypes.c_void_p
    lib.synth_key.argtypes = [u64, u64]
    lib.synth_key.restype = u64
    lib.synth_draw.argtypes = [u64, u64]
    lib.synth_draw.restype = u64
    lib.synth_normal.argtypes = [u64, u64]
    lib.synth_normal.restype = dbl
    lib.synth_bf16_from_double.argtypes = [dbl]
    lib.synth_bf16_from_double.restype = ctypes.c_uint16
    lib.synth_fill_q.argtypes = [u64, i64, ptr, i32]
    lib.synth_fill_q.restype = None
    lib.synth_fill_normal.argtypes = [u64, i32, i64, ptr, i32]
    lib.synth_fill_normal.restype = None
    lib.synth_context_lengths.argtypes = [u64, i32, i32, i32, ptr]
    lib.synth_context_lengths.restype = None
    lib.synth_pages_needed.argtypes = [i32, ptr, i32]
    lib.synth_pages_needed.restype = i64
    lib.synth_page_table.argtypes = [u64, i32, ptr, i32, i32, ptr]
    lib.synth_page_table.restype = i32
    lib.synth_fill_kv.argtypes = [u64, i32, i32, ptr, i32, i32, i32, i32, ptr, i64, dbl, dbl, i32, dbl, ctypes.c_uint16,
                                  ptr, i32]
    lib.synth_e4m3_from_double.argtypes = [dbl]
    lib.synth_e4m3_from_double.restype = ctypes.c_uint8
    lib.synth_fill_kv.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


@dataclass
class Inputs:
    """One case's inputs, all host numpy arrays.

    q            uint16 (bf16 bits) [B, K, Hq, D]
    k_pool       [num_pages, Hkv, P, D]: uint16 bf16 bits, or uint8 fp8 E4M3 bytes
    v_pool       same as k_pool (case.kv_dtype; elements stand for scale * value)
    page_table   int32 [B, stride]
    seq_lens     int32 [B]   keys in cache per request, block included (C_b + K)
    """

    case: Case
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    page_table: np.ndarray
    seq_lens: np.ndarray

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])


def seq_lens_for(case: Case) -> np.ndarray:
    """Per-request key counts C_b + K for a case (fixed, or drawn for mixed batches)."""
    if case.context_range is None:
        return np.full(case.batch, case.context + case.block_size, dtype=np.int32)
    lib = _load()
    ctx = np.empty(case.batch, dtype=np.int32)
    lo, hi = case.context_range
    lib.synth_context_lengths(case.seed, case.batch, lo, hi, _p(ctx))
    return ctx + np.int32(case.block_size)


def make_page_table(case: Case, seq_lens: np.ndarray, stride: int | None = None) -> np.ndarray:
    lib = _load()
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    need = int(((seq_lens.astype(np.int64) + case.page_size - 1) // case.page_size).max())
    if stride is None:
        stride = need + 1
    pt = np.empty((case.batch, stride), dtype=np.int32)
    rc = lib.synth_page_table(case.seed, case.batch, _p(seq_lens), case.page_size, stride, _p(pt))
    if rc != 0:
        raise ValueError(f"synth_page_table failed ({rc})")
    return pt


def make_q(case: Case, threads: int | None = None) -> np.ndarray:
    lib = _load()
    q = np.empty((case.batch, case.block_size, case.num_q_heads, case.head_dim), dtype=np.uint16)
    lib.synth_fill_q(case.seed, q.size, _p(q), threads or default_threads())
    return q


def make_block(case: Case, threads: int | None = None):
    """Dense block keys and values, bf16 bits [B, K, Hkv, D] each (N(0, 1) draws, unscaled)."""
    lib = _load()
    shape = (case.batch, case.block_size, case.num_kv_heads, case.head_dim)
    out = []
    for tensor_id in (7, 8):
        a = np.empty(shape, dtype=np.uint16)
        lib.synth_fill_normal(case.seed, tensor_id, a.size, _p(a), threads or default_threads())
        out.append(a)
    return out[0], out[1]


def make_pool(case: Case, tensor_id: int, seq_lens: np.ndarray, page_table: np.ndarray, num_pages: int,
              fill: int | None = None, threads: int | None = None) -> np.ndarray:
    lib = _load()
    fp8 = case.kv_dtype == "fp8_e4m3"
    if fill is None:
        fill = FP8_NAN if fp8 else BF16_NAN
    scale = case.k_scale if tensor_id == 2 else case.v_scale
    pool = np.empty((num_pages, case.num_kv_heads, case.page_size, case.head_dim), dtype=np.uint8 if fp8 else np.uint16)
    rc = lib.synth_fill_kv(case.seed, tensor_id, case.batch, _p(seq_lens), case.num_kv_heads, case.head_dim,
                           case.page_size, page_table.shape[1], _p(page_table), num_pages,
                           float(case.outlier_rate), float(case.outlier_scale), 1 if fp8 else 0, 1.0 / float(scale),
                           fill, _p(pool), threads or default_threads())
    if rc != 0:
        raise ValueError(f"synth_fill_kv failed ({rc})")
    return pool


def make_inputs(case: Case, fill: int | None = None, threads: int | None = None) -> Inputs:
    """Generate every input of a case (pools include one fill page; see synth.c)."""
    lib = _load()
    seq_lens = seq_lens_for(case)
    pt = make_page_table(case, seq_lens)
    num_pages = int(lib.synth_pages_needed(case.batch, _p(seq_lens), case.page_size))
    q = make_q(case, threads)
    k_pool = make_pool(case, 2, seq_lens, pt, num_pages, fill, threads)
    v_pool = make_pool(case, 3, seq_lens, pt, num_pages, fill, threads)
    return Inputs(case, q, k_pool, v_pool, pt, seq_lens)


def e4m3_from_double(x: float) -> int:
    """OCP fp8 E4M3 encoding (round to nearest even, saturating at +-448) of one value."""
    return int(_load().synth_e4m3_from_double(float(x)))


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (a layout helper, no arithmetic)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)

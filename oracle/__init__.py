"""fp64 CPU oracle for draft-block paged attention (ctypes binding of oracle.c).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The GPU library
never uses it, and it shares no code with the library.

Every function here is a direct, slow definition; see oracle.c for the
passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

PART_ALL, PART_CAUSAL, PART_FUTURE = 0, 1, 2
KV_BF16, KV_FP8_E4M3 = 0, 1
_KV_CODES = {"bf16": KV_BF16, "fp8_e4m3": KV_FP8_E4M3}


class _Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("page_table_stride", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("sm_scale", ctypes.c_double),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_double),
        ("v_scale", ctypes.c_double),
        ("k_block", ctypes.c_void_p),
        ("v_block", ctypes.c_void_p),
    ]


def build() -> str:
    """Compile ``liboracle.so`` with gcc: plain C99 loops, no vector intrinsics."""
    src = os.path.join(_HERE, "oracle.c")
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
    p = ctypes.c_void_p
    lib.oracle_attention.argtypes = [ctypes.POINTER(_Params), ctypes.c_int, p, p, p, p, p, p, ctypes.c_int, p, p,
                                     ctypes.c_int]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_merge.argtypes = [ctypes.c_int64, ctypes.c_int32, p, p, p, p, p, p]
    lib.oracle_merge.restype = None
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_fp8_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_encode_kv.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_uint16]
    lib.oracle_encode_kv.restype = ctypes.c_uint16
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def attention(q, k_pool, v_pool, page_table, seq_lens, *, block_size, num_q_heads, num_kv_heads, head_dim,
              page_size, sm_scale, window_left=-1, window_right=-1, part=PART_ALL, pairs=None, threads=None,
              kv_dtype="bf16", k_scale=1.0, v_scale=1.0, k_block=None, v_block=None):
    """Return (out [B,K,Hq,D] float64, lse2 [B,K,Hq] float64) straight from the definition.

    ``q`` holds bf16 bit patterns (uint16); ``k_pool`` and ``v_pool`` hold bf16
    bits (uint16) or OCP fp8 e4m3 bytes (uint8, ``kv_dtype="fp8_e4m3"``) that
    stand for ``k_scale`` / ``v_scale`` times their value. ``k_block`` /
    ``v_block`` (bf16 bits [B, K, Hkv, D], both or neither) replace the cache as the
    source of the K block keys. ``pairs`` optionally restricts the work to a list
    of (b, h_kv); other rows are NaN.
    """
    lib = _load()
    code = _KV_CODES[kv_dtype]
    el = np.uint8 if code == KV_FP8_E4M3 else np.uint16
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_pool = np.ascontiguousarray(k_pool, dtype=el)
    v_pool = np.ascontiguousarray(v_pool, dtype=el)
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = int(seq_lens.shape[0])
    if (k_block is None) != (v_block is None):
        raise ValueError("k_block and v_block go together")
    if k_block is not None:
        k_block = np.ascontiguousarray(k_block, dtype=np.uint16)
        v_block = np.ascontiguousarray(v_block, dtype=np.uint16)
        if k_block.shape != (B, block_size, num_kv_heads, head_dim) or v_block.shape != k_block.shape:
            raise ValueError("block arrays must be [B, K, Hkv, D]")
    prm = _Params(B, block_size, num_q_heads, num_kv_heads, head_dim, page_size, int(page_table.shape[1]),
                  int(k_pool.shape[0]), window_left, window_right, float(sm_scale), code, float(k_scale),
                  float(v_scale), None if k_block is None else k_block.ctypes.data,
                  None if v_block is None else v_block.ctypes.data)
    out = np.full((B, block_size, num_q_heads, head_dim), np.nan)
    lse2 = np.full((B, block_size, num_q_heads), np.nan)
    if pairs is not None:
        pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        pptr, npairs = pr.ctypes.data, int(pr.shape[0])
    else:
        pr, pptr, npairs = None, None, 0
    rc = lib.oracle_attention(ctypes.byref(prm), part, q.ctypes.data, k_pool.ctypes.data, v_pool.ctypes.data,
                              page_table.ctypes.data, seq_lens.ctypes.data, pptr, npairs, out.ctypes.data,
                              lse2.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return out, lse2


def attention_case(inputs, *, part=PART_ALL, pairs=None, threads=None, window_left=None, window_right=None,
                   k_block=None, v_block=None):
    """Oracle on a ``synth.Inputs`` object with the case's own parameters."""
    c = inputs.case
    return attention(inputs.q, inputs.k_pool, inputs.v_pool, inputs.page_table, inputs.seq_lens,
                     block_size=c.block_size, num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
                     head_dim=c.head_dim, page_size=c.page_size, sm_scale=c.scale,
                     window_left=c.window_left if window_left is None else window_left,
                     window_right=c.window_right if window_right is None else window_right,
                     part=part, pairs=pairs, threads=threads, kv_dtype=c.kv_dtype, k_scale=c.k_scale,
                     v_scale=c.v_scale, k_block=k_block, v_block=v_block)


def merge(out_a, lse_a, out_b, lse_b):
    """LSE merge of two normalised results over disjoint key sets (base-2 LSEs)."""
    lib = _load()
    out_a = np.ascontiguousarray(out_a, dtype=np.float64)
    out_b = np.ascontiguousarray(out_b, dtype=np.float64)
    lse_a = np.ascontiguousarray(lse_a, dtype=np.float64)
    lse_b = np.ascontiguousarray(lse_b, dtype=np.float64)
    D = int(out_a.shape[-1])
    rows = int(lse_a.size)
    out = np.empty_like(out_a)
    lse = np.empty_like(lse_a)
    lib.oracle_merge(rows, D, out_a.ctypes.data, lse_a.ctypes.data, out_b.ctypes.data, lse_b.ctypes.data,
                     out.ctypes.data, lse.ctypes.data)
    return out, lse


def bf16_to_double(bits: int) -> float:
    return float(_load().oracle_bf16_to_double(bits))


def fp8_e4m3_to_double(code: int) -> float:
    return float(_load().oracle_fp8_e4m3_to_double(code))


def encode_kv(kv_dtype: str, scale: float, bits: int) -> int:
    """The cache element appending bf16 `bits` stores in a `kv_dtype` pool with `scale`."""
    return int(_load().oracle_encode_kv(_KV_CODES[kv_dtype], float(scale), int(bits)))

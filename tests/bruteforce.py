"""Brute-force dense fp64 attention used to pin the oracle on tiny inputs.

It takes a different route from the oracle: the request's K/V are gathered
into dense arrays with numpy fancy indexing over the page table, an explicit
boolean [rows x keys] mask is built, and the result comes from library
routines (matmul, scipy's logsumexp and softmax). Only tests import it.
"""
from __future__ import annotations

import math

import numpy as np
import torch
from scipy.special import logsumexp, softmax

from synth import bf16_bits_to_float


def decode_pool(raw: np.ndarray) -> np.ndarray:
    """Element values of pool pages: bf16 bits (uint16) by bit widening, OCP fp8 E4M3 bytes
    (uint8) through torch's float8_e4m3fn conversion (a library decoder, not the oracle's)."""
    if raw.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(raw)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return bf16_bits_to_float(raw).astype(np.float64)


def dense_kv(pool: np.ndarray, page_table: np.ndarray, b: int, n: int, scale: float = 1.0) -> np.ndarray:
    """[n, Hkv, D] float64 view of request b's keys (or values) in logical order, times the pool scale."""
    P = pool.shape[2]
    pages = page_table[b, : (n + P - 1) // P]
    blk = scale * decode_pool(pool[pages])  # [np, Hkv, P, D]
    blk = np.transpose(blk, (0, 2, 1, 3)).reshape(-1, pool.shape[1], pool.shape[3])
    return blk[:n]


def key_mask(n: int, K: int, g: int, window_left: int, window_right: int, part: str = "all") -> np.ndarray:
    """Boolean [K*g, n]: row r = i*g + l may see key j."""
    R = K * g
    j = np.arange(n)[None, :]
    i = (np.arange(R) // g)[:, None]
    p = n - K + i
    m = np.ones((R, n), dtype=bool)
    if window_left != -1:
        m &= j > p - window_left
    if window_right != -1:
        m &= j <= p + window_right
    if part == "causal":
        m &= j <= p
    elif part == "future":
        m &= j > p
    return m


def attention(inputs, window_left=None, window_right=None, part="all", k_block=None, v_block=None):
    """Dense masked attention for every row; returns (out, lse2) like the oracle. With k_block / v_block
    (bf16 bits [B, K, Hkv, D]) the last K keys of each request come from them instead of the cache."""
    c = inputs.case
    wl = c.window_left if window_left is None else window_left
    wr = c.window_right if window_right is None else window_right
    B, K, Hq, D = inputs.q.shape
    Hkv = inputs.k_pool.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, K, Hq, D))
    lse2 = np.full((B, K, Hq), -np.inf)
    q = bf16_bits_to_float(inputs.q).astype(np.float64)
    for b in range(B):
        n = int(inputs.seq_lens[b])
        kd = dense_kv(inputs.k_pool, inputs.page_table, b, n, c.k_scale)
        vd = dense_kv(inputs.v_pool, inputs.page_table, b, n, c.v_scale)
        if k_block is not None:
            kd[n - K:] = bf16_bits_to_float(k_block[b]).astype(np.float64)
            vd[n - K:] = bf16_bits_to_float(v_block[b]).astype(np.float64)
        mask = key_mask(n, K, g, wl, wr, part)
        for hk in range(Hkv):
            qr = q[b, :, hk * g:(hk + 1) * g, :].reshape(K * g, D)
            s = c.scale * (qr @ kd[:, hk, :].T)
            s = np.where(mask, s, -np.inf)
            has = mask.any(axis=1)
            lse = np.full(K * g, -np.inf)
            lse[has] = logsumexp(s[has], axis=1) / math.log(2.0)
            o = np.zeros((K * g, D))
            o[has] = softmax(s[has], axis=1) @ vd[:, hk, :]
            out[b, :, hk * g:(hk + 1) * g, :] = o.reshape(K, g, D)
            lse2[b, :, hk * g:(hk + 1) * g] = lse.reshape(K, g)
    return out, lse2

"""Dense paged GQA decode ("pa_decode"), plain and slow -- test infrastructure
only.  Neither the GPU path nor anything a user calls imports this module.

The aiter page "[FlyDSL] [Perf] pa_decode: K/V streaming, MTP query split and
sparse split-major on gfx950" (Summary, Motivation, Performance) measures a
paged decode of grouped-query attention with separate K and V rows ("K/V
streaming"), MTP query positions and split plans, over a matrix of head dims,
GQA ratios, batches and context lengths, but does not print its definition.
The reading used here is the usual paged decode:

* q is bf16 [B * mtp, Hq, D]; token t = b * mtp + i is MTP position i of
  sequence b; query head h uses KV head g = h // (Hq // Hkv);
* the caches are bf16 [num_blocks, page_size, Hkv, D] (K and V alike);
  position p of sequence b lives in physical block block_tables[b, p //
  page_size], slot p % page_size;
* the last mtp positions of a sequence's context are its MTP tokens, causal
  among themselves: token i attends to positions p < context_lens[b] -
  (mtp - 1 - i);
* s_p = scale * <q, k_p>, out = sum_p softmax(s)_p v_p, lse = ln sum_p e^{s_p}
  (natural log, no sink); a token with no position gets out = 0, lse = -inf;
* a block-table entry outside [0, num_blocks) names no block: the positions
  of that page are masked (a reading; the page does not say);
* split partials as in ``oracle.ref``: split r covers positions [a_r, e_r)
  of ``ref.split_bounds(max_context_len, s)`` (one plan per call, cut at each
  token's own limit); lse_r = ln sum_{p in r} e^{s_p}, o_r = sum_{p in r}
  e^{s_p - lse_r} v_p, and o_r = 0, lse_r = -inf for an empty split.

float64 throughout, from the exact bf16 values; no blocking, no online
softmax: gather, scores, one full softmax, PV.
"""
from __future__ import annotations

import numpy as np

from oracle import ref


def _positions(block_tables, b: int, n: int, page_size: int, num_blocks: int):
    """Physical (block, slot) of positions 0 .. n-1 of sequence b, and whether
    the block-table entry names a block (block 0 stands in where it does not)."""
    p = np.arange(n)
    blk = np.asarray(block_tables)[b, p // page_size].astype(np.int64)
    ok = (blk >= 0) & (blk < num_blocks)
    return np.where(ok, blk, 0), p % page_size, ok


def gather_kv(cache: np.ndarray, block_tables, b: int, g: int, n: int, page_size: int):
    """float64 [n, D] rows of KV head g at positions 0 .. n-1 of sequence b,
    and bool [n]: the position's page names a block (rows of the others are
    placeholders, never attended)."""
    cache = np.asarray(cache)
    blk, slot, ok = _positions(block_tables, b, n, page_size, cache.shape[0])
    return ref.bf16_to_f64(cache[blk, slot, g]), ok


def _attend_kv(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """q [D], k/v [n, D] float64 -> (o [D], lse)."""
    if k.shape[0] == 0:
        return np.zeros(q.shape[0]), -np.inf
    s = float(np.float32(scale)) * (k @ q)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    return (e / z) @ v, m + np.log(z)


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, page_size: int, mtp: int, softmax_scale: float):
    """Returns out float64 [B*mtp, Hq, D] and lse float64 [B*mtp, Hq]."""
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = np.asarray(k_cache).shape[2]
    R = Hq // Hkv
    qf = ref.bf16_to_f64(q)
    out = np.zeros((T, Hq, D))
    lse = np.zeros((T, Hq))
    for b in range(T // mtp):
        L = int(context_lens[b])
        for g in range(Hkv):
            kk, ok = gather_kv(k_cache, block_tables, b, g, L, page_size)
            vv, _ = gather_kv(v_cache, block_tables, b, g, L, page_size)
            for i in range(mtp):
                n = max(L - (mtp - 1 - i), 0)
                t = b * mtp + i
                sel = ok[:n]
                for j in range(R):
                    h = g * R + j
                    out[t, h], lse[t, h] = _attend_kv(qf[t, h], kk[:n][sel], vv[:n][sel], softmax_scale)
    return out, lse


def paged_decode_partials(q, k_cache, v_cache, block_tables, context_lens, page_size: int, mtp: int,
                          softmax_scale: float, num_splits: int, max_context_len: int):
    """FP32-partial semantics in float64: o [T, Hq, s, D], lse [T, Hq, s].
    Split r covers positions ``ref.split_bounds(max_context_len, s)[r]`` of
    every sequence, cut at each token's own limit."""
    q = np.asarray(q)
    T, Hq, D = q.shape
    Hkv = np.asarray(k_cache).shape[2]
    R = Hq // Hkv
    qf = ref.bf16_to_f64(q)
    bounds = ref.split_bounds(max_context_len, num_splits)
    o = np.zeros((T, Hq, num_splits, D))
    lse = np.zeros((T, Hq, num_splits))
    for b in range(T // mtp):
        L = int(context_lens[b])
        for g in range(Hkv):
            kk, ok = gather_kv(k_cache, block_tables, b, g, L, page_size)
            vv, _ = gather_kv(v_cache, block_tables, b, g, L, page_size)
            for i in range(mtp):
                n = max(L - (mtp - 1 - i), 0)
                t = b * mtp + i
                for r, (a, e) in enumerate(bounds):
                    a2, e2 = min(a, n), min(e, n)
                    sel = ok[a2:e2]
                    for j in range(R):
                        h = g * R + j
                        o[t, h, r], lse[t, h, r] = _attend_kv(qf[t, h], kk[a2:e2][sel], vv[a2:e2][sel],
                                                              softmax_scale)
    return o, lse

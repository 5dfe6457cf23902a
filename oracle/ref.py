"""Float64 reference of sparse MLA decode -- test infrastructure only.

Definitions follow the pages:

* vLLM "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA decode on gfx950",
  section Design: a 512-wide QK dot made of 448 NoPE and 64 RoPE dims; the
  PV product runs over the same 512-wide latent row (V is the row itself);
  attention sinks; an invalid index contributes zero probability; main
  (top-k) and sliding-window work run as ordered tiles of one softmax, read
  here as two sources (a main pool and an SWA pool, each with its own index
  list) whose rows all enter one softmax, main positions first.
* aiter "[ASM][HIP][MLA v4 nm] Split plan helper and persistent decode
  kernel", Summary: split-KV with FP32 partials reduced by a stage-2 merge;
  rows with K = 0 are left unwritten.

Readings where the pages are silent (each listed in the design notes):
the sink is a logit in the already-scaled score domain that adds e^sink to
the softmax denominator and has no value row; the final LSE includes the
sink, split partial LSEs do not; logs are natural; any index outside
[0, N) is invalid; duplicate indices are separate terms; a row with no
valid entry gives out = 0 and lse = sink (or -inf without a sink).

Everything is computed in float64 from the exact values of the stored bf16
and fp8 inputs, without blocking or an online softmax: gather, scores, one
full softmax, PV.
"""
from __future__ import annotations

import math

import numpy as np

NOPE = 448
ROPE = 64
DIM = 512


# ----------------------------------------------------------------------------
# element decoding
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN bytes -> float64: sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
    there is no infinity.  Pinned against torch.float8_e4m3fn for all 256 codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    v = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)


def ue8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    """UE8M0 scale byte c -> 2^(c - 127); c = 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def pool_rows(pool: dict, rows: np.ndarray) -> np.ndarray:
    """Decode pool rows `rows` (already valid) into float64 [len(rows), 512]:
    NoPE dims 0..447 then RoPE dims 448..511.

    bf16 pool: {"kv": uint16 [N, 512]} or {"nope": uint16 [N,448], "rope": uint16 [N,64]}.
    fp8 pool:  {"nope": uint8 [N,448], "scale": uint8 [N,>=7], "rope": uint16 [N,64]};
               NoPE dim d = e4m3(byte_d) * 2^(code_(d // 64) - 127); RoPE is plain bf16.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if "kv" in pool:
        return bf16_to_f64(pool["kv"][rows])
    if pool["nope"].dtype == np.uint16:
        return np.concatenate([bf16_to_f64(pool["nope"][rows]), bf16_to_f64(pool["rope"][rows])], axis=1)
    x = e4m3fn_to_f64(pool["nope"][rows])                      # [n, 448]
    s = ue8m0_to_f64(pool["scale"][rows][:, :NOPE // 64])       # [n, 7]
    x = x * np.repeat(s, 64, axis=1)
    r = bf16_to_f64(pool["rope"][rows])
    return np.concatenate([x, r], axis=1)


def pool_size(pool: dict) -> int:
    return (pool["kv"] if "kv" in pool else pool["nope"]).shape[0]


def queries(q_nope: np.ndarray, q_rope: np.ndarray) -> np.ndarray:
    """[T,H,448] and [T,H,64] bf16 bits -> float64 [T, H, 512]."""
    return np.concatenate([bf16_to_f64(q_nope), bf16_to_f64(q_rope)], axis=-1)


def valid_mask(idx: np.ndarray, n: int) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.int64)
    return (idx >= 0) & (idx < n)


def _scale64(softmax_scale: float) -> float:
    """The scale is a float32 argument of the library; widen that float32 value."""
    return float(np.float32(softmax_scale))


# ----------------------------------------------------------------------------
# attention of a block of query rows over one gathered row set
# ----------------------------------------------------------------------------
def attend(q: np.ndarray, k: np.ndarray, softmax_scale: float, sink: np.ndarray | None):
    """q [M,512] float64, k [n,512] float64 (valid gathered rows, duplicates kept),
    sink [M] float64 or None.

    s_j = scale * <q, k_j>;  Z = sum_j e^{s_j} + e^{sink};  out = sum_j (e^{s_j}/Z) k_j;
    lse = ln Z.  Computed with the usual max shift.  No valid row: out = 0,
    lse = sink (or -inf without a sink)."""
    M = q.shape[0]
    if k.shape[0] == 0:
        out = np.zeros((M, DIM))
        lse = np.full(M, -np.inf) if sink is None else np.array(sink, dtype=np.float64).copy()
        return out, lse
    s = _scale64(softmax_scale) * (q @ k.T)                      # [M, n]
    m = s.max(axis=1)
    if sink is not None:
        m = np.maximum(m, sink)
    e = np.exp(s - m[:, None])
    z = e.sum(axis=1)
    if sink is not None:
        z = z + np.exp(sink - m)
    out = (e / z[:, None]) @ k
    lse = m + np.log(z)
    return out, lse


def _sink64(sink, H):
    if sink is None:
        return None
    return np.asarray(sink, dtype=np.float32).astype(np.float64).reshape(H)


def sparse_mla_decode(q_nope, q_rope, pool: dict, indices, sink, softmax_scale: float, q_per_seq: int = 1, *,
                      queries64=None):
    """Dense-index decode: token t uses index row t // q_per_seq.  queries64
    (float64 [T, H, 512]) replaces the queries that q_nope / q_rope encode.

    Returns out float64 [T, H, 512] and lse float64 [T, H]."""
    q = queries(q_nope, q_rope) if queries64 is None else np.asarray(queries64, dtype=np.float64)
    T, H, _ = q.shape
    n = pool_size(pool)
    sk = _sink64(sink, H)
    out = np.zeros((T, H, DIM))
    lse = np.zeros((T, H))
    idx_all = np.asarray(indices)
    for b in range(idx_all.shape[0]):
        idx = idx_all[b]
        rows = idx[valid_mask(idx, n)]
        k = pool_rows(pool, rows)
        t0, t1 = b * q_per_seq, (b + 1) * q_per_seq
        qb = q[t0:t1].reshape(-1, DIM)                            # [(t,h) rows]
        skb = None if sk is None else np.tile(sk, q_per_seq)
        o, l = attend(qb, k, softmax_scale, skb)
        out[t0:t1] = o.reshape(q_per_seq, H, DIM)
        lse[t0:t1] = l.reshape(q_per_seq, H)
    return out, lse


def sparse_mla_decode_ragged(q_nope, q_rope, pool: dict, kv_indptr, kv_indices, sink, softmax_scale: float,
                             q_per_seq: int, *, queries64=None):
    """Ragged decode: sequence b owns kv_indices[kv_indptr[b]:kv_indptr[b+1]] and
    tokens b*q_per_seq .. (b+1)*q_per_seq-1, which all share that index list.

    Returns (out, lse, written): rows of sequences with K_b = 0 are not written
    (the pages leave them untouched); `written` is a bool [T] mask.
    queries64 as in sparse_mla_decode."""
    q = queries(q_nope, q_rope) if queries64 is None else np.asarray(queries64, dtype=np.float64)
    T, H, _ = q.shape
    n = pool_size(pool)
    sk = _sink64(sink, H)
    ptr = np.asarray(kv_indptr, dtype=np.int64)
    out = np.full((T, H, DIM), np.nan)
    lse = np.full((T, H), np.nan)
    written = np.zeros(T, dtype=bool)
    for b in range(len(ptr) - 1):
        if ptr[b + 1] == ptr[b]:
            continue
        idx = np.asarray(kv_indices[ptr[b]:ptr[b + 1]])
        rows = idx[valid_mask(idx, n)]
        k = pool_rows(pool, rows)
        t0, t1 = b * q_per_seq, (b + 1) * q_per_seq
        skb = None if sk is None else np.tile(sk, q_per_seq)
        o, l = attend(q[t0:t1].reshape(-1, DIM), k, softmax_scale, skb)
        out[t0:t1] = o.reshape(q_per_seq, H, DIM)
        lse[t0:t1] = l.reshape(q_per_seq, H)
        written[t0:t1] = True
    return out, lse, written


# ----------------------------------------------------------------------------
# split-KV partials and their merge
# ----------------------------------------------------------------------------
SPLIT_ALIGN = 64


def split_bounds(kv_len: int, num_splits: int):
    """Uniform split of index positions [0, kv_len) into `num_splits` pieces.

    Reading of the uniform split_indptr of the aiter page (Summary, part 1):
    chunk = ceil(ceil(kv_len / s) / 64) * 64 and split r covers
    [min(r*chunk, K), min((r+1)*chunk, K)); trailing splits may be empty."""
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    per = -(-kv_len // num_splits)
    chunk = -(-per // SPLIT_ALIGN) * SPLIT_ALIGN
    return [(min(r * chunk, kv_len), min((r + 1) * chunk, kv_len)) for r in range(num_splits)]


def partial_one(q: np.ndarray, k: np.ndarray, softmax_scale: float):
    """Partial result of one split (no sink): lse_r = ln sum_j e^{s_j},
    o_r = sum_j e^{s_j - lse_r} k_j; an empty split gives o_r = 0, lse_r = -inf."""
    M = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((M, DIM)), np.full(M, -np.inf)
    s = _scale64(softmax_scale) * (q @ k.T)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    z = e.sum(axis=1)
    return (e / z[:, None]) @ k, m + np.log(z)


def sparse_mla_decode_partials(q_nope, q_rope, pool: dict, indices, softmax_scale: float, num_splits: int,
                               q_per_seq: int = 1, *, queries64=None):
    """Per-split FP32-partial semantics in float64: o [T, H, s, 512], lse [T, H, s].
    Split r of index row b covers positions split_bounds(K, s)[r] of that row.
    queries64 as in sparse_mla_decode."""
    q = queries(q_nope, q_rope) if queries64 is None else np.asarray(queries64, dtype=np.float64)
    T, H, _ = q.shape
    n = pool_size(pool)
    idx_all = np.asarray(indices)
    K = idx_all.shape[1]
    bounds = split_bounds(K, num_splits)
    o = np.zeros((T, H, num_splits, DIM))
    lse = np.zeros((T, H, num_splits))
    for b in range(idx_all.shape[0]):
        t0, t1 = b * q_per_seq, (b + 1) * q_per_seq
        qb = q[t0:t1].reshape(-1, DIM)
        for r, (a, e) in enumerate(bounds):
            idx = idx_all[b, a:e]
            k = pool_rows(pool, idx[valid_mask(idx, n)])
            orr, lr = partial_one(qb, k, softmax_scale)
            o[t0:t1, :, r] = orr.reshape(q_per_seq, H, DIM)
            lse[t0:t1, :, r] = lr.reshape(q_per_seq, H)
    return o, lse


def merge_partials(o: np.ndarray, lse: np.ndarray, sink):
    """Stage-2 merge: LSE = ln(sum_r e^{lse_r} + e^{sink_h}); out = sum_r e^{lse_r - LSE} o_r.

    o [T, H, s, 512], lse [T, H, s]; sink [H] or None.  All terms -inf and no
    sink gives out = 0, LSE = -inf."""
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    T, H, S, _ = o.shape
    terms = lse
    if sink is not None:
        sk = np.broadcast_to(_sink64(sink, H)[None, :, None], (T, H, 1))
        terms = np.concatenate([lse, sk], axis=2)
    m = terms.max(axis=2)
    finite = np.isfinite(m)
    ms = np.where(finite, m, 0.0)
    z = np.exp(terms - ms[:, :, None]).sum(axis=2)
    L = np.where(finite, ms + np.log(z), -np.inf)
    w = np.where(finite[:, :, None], np.exp(lse - np.where(finite, L, 0.0)[:, :, None]), 0.0)
    out = (w[..., None] * o).sum(axis=2)
    return out, L


# ----------------------------------------------------------------------------
# two sources: the compressed main cache and the sliding-window (SWA) cache
# ----------------------------------------------------------------------------
def two_source_rows(main_pool: dict, main_idx, swa_pool: dict, swa_idx) -> np.ndarray:
    """Rows one index row attends to when its main (top-k) entries index the
    main pool and its SWA entries index the SWA pool (the vLLM page, Design:
    main and SWA work run as ordered tiles of one softmax).  Each entry is
    valid against its own pool's size; the main rows come first."""
    main_idx = np.asarray(main_idx)
    swa_idx = np.asarray(swa_idx)
    km = pool_rows(main_pool, main_idx[valid_mask(main_idx, pool_size(main_pool))])
    ks = pool_rows(swa_pool, swa_idx[valid_mask(swa_idx, pool_size(swa_pool))])
    return np.concatenate([km, ks], axis=0)


def sparse_mla_decode_two_source(q_nope, q_rope, main_pool: dict, main_indices, swa_pool: dict, swa_indices, sink,
                                 softmax_scale: float, q_per_seq: int = 1):
    """Decode over both sources: token t uses main row t // q_per_seq of
    main_indices (into main_pool) and the same row of swa_indices (into
    swa_pool), all of them terms of one softmax with the sink.

    Returns out float64 [T, H, 512] and lse float64 [T, H]."""
    q = queries(q_nope, q_rope)
    T, H, _ = q.shape
    sk = _sink64(sink, H)
    out = np.zeros((T, H, DIM))
    lse = np.zeros((T, H))
    mi, si = np.asarray(main_indices), np.asarray(swa_indices)
    for b in range(mi.shape[0]):
        k = two_source_rows(main_pool, mi[b], swa_pool, si[b])
        t0, t1 = b * q_per_seq, (b + 1) * q_per_seq
        skb = None if sk is None else np.tile(sk, q_per_seq)
        o, l = attend(q[t0:t1].reshape(-1, DIM), k, softmax_scale, skb)
        out[t0:t1] = o.reshape(q_per_seq, H, DIM)
        lse[t0:t1] = l.reshape(q_per_seq, H)
    return out, lse


def sparse_mla_decode_two_source_partials(q_nope, q_rope, main_pool: dict, main_indices, swa_pool: dict,
                                          swa_indices, softmax_scale: float, num_splits: int, q_per_seq: int = 1):
    """Split partials over the ordered positions of both sources: position p
    of an index row is main entry p for p < K_main, else SWA entry p - K_main;
    split r covers split_bounds(K_main + K_swa, s)[r] of those positions."""
    q = queries(q_nope, q_rope)
    T, H, _ = q.shape
    mi, si = np.asarray(main_indices), np.asarray(swa_indices)
    k_main, k_swa = mi.shape[1], si.shape[1]
    bounds = split_bounds(k_main + k_swa, num_splits)
    o = np.zeros((T, H, num_splits, DIM))
    lse = np.zeros((T, H, num_splits))
    for b in range(mi.shape[0]):
        t0, t1 = b * q_per_seq, (b + 1) * q_per_seq
        qb = q[t0:t1].reshape(-1, DIM)
        for r, (a, e) in enumerate(bounds):
            # positions [a, e): the main part [a, min(e, K_main)), the SWA part from max(a, K_main)
            k = two_source_rows(main_pool, mi[b, a:min(e, k_main)], swa_pool,
                                si[b, max(a, k_main) - k_main:max(e, k_main) - k_main])
            orr, lr = partial_one(qb, k, softmax_scale)
            o[t0:t1, :, r] = orr.reshape(q_per_seq, H, DIM)
            lse[t0:t1, :, r] = lr.reshape(q_per_seq, H)
    return o, lse


# ----------------------------------------------------------------------------
# bf16 rounding of the output (fp32 -> bf16, round to nearest even)
# ----------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest float32 -> bf16 (RNE), returned as float64 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


LN2 = math.log(2.0)

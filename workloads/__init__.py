"""Seeded synthetic inputs for sparse MLA decode.

This module only draws inputs.  It holds none of the decode arithmetic: no
score, softmax, merge or split rule lives here.  Both the float64 oracle and
the HIP path consume exactly the arrays it returns, so a parity test compares
the two on identical bytes.

Layout of every workload (NumPy arrays, bf16 stored as uint16 bit patterns):

* ``q_nope``  uint16 [T, H, 448]   bf16 bits
* ``q_rope``  uint16 [T, H, 64]    bf16 bits
* pool, bf16:  ``kv``    uint16 [N, 512]  (448 NoPE dims then 64 RoPE dims)
* pool, fp8:   ``nope``  uint8  [N, 448]  OCP E4M3FN bytes
               ``scale`` uint8  [N, 8]    UE8M0 codes of the seven 64-dim
                                          NoPE blocks, byte 7 is padding (0)
               ``rope``  uint16 [N, 64]   bf16 bits
* ``sink``    float32 [H]
* dense index rows: ``indices`` int32 [T // q_per_seq, K] (-1 = invalid)
* ragged rows: ``kv_indptr`` int32 [B + 1], ``kv_indices`` int32 [sum K_b]

The workload shapes follow the DeepSeek-V4 sparse-MLA decode statement on the
vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA decode on gfx950"
(Design: 448 NoPE + 64 RoPE dims in one 512-wide row; invalid index -1) and
the aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and persistent decode
kernel" (Summary part 2: ragged kv_indptr + flat kv_page_indices, K=0 rows).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

NOPE = 448
ROPE = 64
DIM = NOPE + ROPE
FP8_BLOCK = 64
FP8_BLOCKS = NOPE // FP8_BLOCK  # 7
SCALE_STRIDE = 8  # 7 codes + 1 pad byte per row


# ----------------------------------------------------------------------------
# float32 -> bf16 bits, round to nearest even (a storage conversion of the
# generator, not part of the decode)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.  The 32-bit
    sum cannot wrap for any non-NaN input (the largest, -inf, gives 0xFF807FFF)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def _normal_bf16(rng: np.random.Generator, shape, chunk_rows: int = 65536) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16, generated in row chunks to bound memory."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.uint16)
    if len(shape) == 0 or shape[0] == 0:
        return out
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = f32_to_bf16_bits(rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32))
    return out


def quantize_e4m3_ue8m0(x: np.ndarray):
    """Cache-writer stand-in: float32 [N, 448] -> (e4m3fn bytes [N,448], codes [N,8]).

    Per 64-element block: code c = clamp(ceil(log2(amax / 448)) + 127, 0, 254)
    (a zero block gets c = 0), byte = RNE_e4m3fn(x / 2^(c-127)).  The cap at 254
    follows the vLLM page's Design section (writers never emit the NaN code 255).
    The decode never sees the float32 input, only these bytes and codes.
    """
    import torch

    n = x.shape[0]
    xb = x.reshape(n, FP8_BLOCKS, FP8_BLOCK).astype(np.float64)
    amax = np.abs(xb).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.ceil(np.log2(amax / 448.0)), -127.0)
    codes = np.clip(e + 127.0, 0, 254).astype(np.int64)
    scaled = xb / np.exp2((codes - 127).astype(np.float64))[:, :, None]
    t = torch.from_numpy(scaled.reshape(n, NOPE).astype(np.float32))
    q = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    sc = np.zeros((n, SCALE_STRIDE), dtype=np.uint8)
    sc[:, :FP8_BLOCKS] = codes.astype(np.uint8)
    return q, sc


def _fp8_pool(rng: np.random.Generator, n: int, chunk_rows: int = 65536):
    nope = np.empty((n, NOPE), dtype=np.uint8)
    scale = np.empty((n, SCALE_STRIDE), dtype=np.uint8)
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        q, sc = quantize_e4m3_ue8m0(rng.standard_normal((r1 - r0, NOPE), dtype=np.float32))
        nope[r0:r1] = q
        scale[r0:r1] = sc
    return nope, scale


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    num_tokens: int
    num_heads: int
    q_per_seq: int
    kv_dtype: str  # "bf16" | "fp8"
    pool_rows: int
    softmax_scale: float
    arrays: dict = field(default_factory=dict)
    ragged: bool = False
    two_source: bool = False
    note: str = ""

    @property
    def num_index_rows(self) -> int:
        return self.num_tokens // self.q_per_seq

    def row_bytes(self) -> int:
        return 2 * DIM if self.kv_dtype == "bf16" else NOPE + SCALE_STRIDE + 2 * ROPE


def _queries(rng, T, H):
    q_nope = _normal_bf16(rng, (T, H, NOPE))
    q_rope = _normal_bf16(rng, (T, H, ROPE))
    return q_nope, q_rope


def _pool(rng, kv_dtype, n):
    if kv_dtype == "bf16":
        nope = _normal_bf16(rng, (n, NOPE))
        rope = _normal_bf16(rng, (n, ROPE))
        kv = np.empty((n, DIM), dtype=np.uint16)
        kv[:, :NOPE] = nope
        kv[:, NOPE:] = rope
        return {"kv": kv}
    nope, scale = _fp8_pool(rng, n)
    rope = _normal_bf16(rng, (n, ROPE))
    return {"nope": nope, "scale": scale, "rope": rope}


def _set_invalid(rng, idx: np.ndarray, count: int):
    if count <= 0:
        return
    for r in range(idx.shape[0]):
        pos = rng.choice(idx.shape[1], size=count, replace=False)
        idx[r, pos] = -1


_POOL_CACHE: dict = {}


def _own_pool(kv_dtype: str, n: int, seed: int) -> dict:
    """A pool drawn from its own generator (PCG64(seed)); the last one of each
    (dtype, size, seed) is kept, so table sweeps over T reuse it."""
    key = (kv_dtype, n, seed)
    if key not in _POOL_CACHE:
        _POOL_CACHE.clear()
        _POOL_CACHE[key] = _pool(np.random.Generator(np.random.PCG64(seed)), kv_dtype, n)
    return _POOL_CACHE[key]


def dense_workload(name: str, *, T: int, H: int, kv_dtype: str, pool_rows: int, topk: int,
                   swa: int = 0, invalid: int = 0, sorted_topk: bool = False, q_per_seq: int = 1,
                   seed: int = 0, pool_seed: int | None = None, softmax_scale: float | None = None,
                   note: str = "") -> Workload:
    """One index row per q_per_seq tokens: `topk` indices drawn uniformly without
    replacement from the pool, then the last `swa` pool rows appended in order,
    then `invalid` positions per row set to -1 (uniformly chosen).

    Draw order: q_nope, q_rope, pool, sink, indices, invalid positions.  With
    pool_seed the pool comes from its own generator instead (and is not drawn
    from the main one)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q_nope, q_rope = _queries(rng, T, H)
    pool = _pool(rng, kv_dtype, pool_rows) if pool_seed is None else _own_pool(kv_dtype, pool_rows, pool_seed)
    sink = rng.standard_normal(H, dtype=np.float32)
    R = T // q_per_seq
    K = topk + swa
    idx = np.empty((R, K), dtype=np.int32)
    for r in range(R):
        top = rng.choice(pool_rows, size=topk, replace=False)
        if sorted_topk:
            top = np.sort(top)
        idx[r, :topk] = top
        if swa:
            idx[r, topk:] = np.arange(pool_rows - swa, pool_rows, dtype=np.int32)
    _set_invalid(rng, idx, invalid)
    arrays = {"q_nope": q_nope, "q_rope": q_rope, "sink": sink, "indices": idx, **pool}
    scale = 1.0 / math.sqrt(DIM) if softmax_scale is None else softmax_scale
    return Workload(name, T, H, q_per_seq, kv_dtype, pool_rows, scale, arrays, note=note)


def ragged_workload(name: str, *, B: int, q_per_seq: int, H: int, kv_dtype: str, pool_rows: int,
                    max_k: int, zero_rows: int = 0, indptr_offset: int = 0, seed: int = 0,
                    softmax_scale: float | None = None, note: str = "") -> Workload:
    """Ragged index lists: K_b ~ U{0..max_k}, `zero_rows` sequences forced to K_b = 0,
    indices uniform without replacement (unsorted, none invalid).  kv_indptr[0] =
    indptr_offset (the flat array then starts with that many padding entries).

    Draw order: q_nope, q_rope, pool, sink, K_b, zero rows, indices."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = B * q_per_seq
    q_nope, q_rope = _queries(rng, T, H)
    pool = _pool(rng, kv_dtype, pool_rows)
    sink = rng.standard_normal(H, dtype=np.float32)
    ks = rng.integers(0, max_k, size=B, endpoint=True).astype(np.int64)
    if zero_rows:
        ks[rng.choice(B, size=zero_rows, replace=False)] = 0
    indptr = np.empty(B + 1, dtype=np.int64)
    indptr[0] = indptr_offset
    indptr[1:] = indptr_offset + np.cumsum(ks)
    flat = np.full(int(indptr[-1]), -7, dtype=np.int32)  # padding before the offset is never read
    for b in range(B):
        flat[indptr[b]:indptr[b + 1]] = rng.choice(pool_rows, size=int(ks[b]), replace=False)
    arrays = {"q_nope": q_nope, "q_rope": q_rope, "sink": sink,
              "kv_indptr": indptr.astype(np.int32), "kv_indices": flat, **pool}
    scale = 1.0 / math.sqrt(DIM) if softmax_scale is None else softmax_scale
    return Workload(name, T, H, q_per_seq, kv_dtype, pool_rows, scale, arrays, ragged=True, note=note)


def two_source_workload(name: str, *, T: int, H: int, kv_dtype: str, main_rows: int, topk: int, window: int,
                        invalid: int = 0, swa_invalid: int = 0, q_per_seq: int = 1, seed: int = 0,
                        softmax_scale: float | None = None, note: str = "") -> Workload:
    """Main + SWA sources.  Index row b draws `topk` main indices uniformly
    without replacement from a main pool of main_rows rows (`invalid` of them
    then set to -1), and owns block b of a sliding-window pool of
    R * window rows, a ring: its window list is that block's rows starting at
    a random ring position, the first `swa_invalid` entries -1 (a window not
    yet full).  Both pools have the same format.

    Draw order: q_nope, q_rope, main pool, SWA pool, sink, main indices,
    invalid main positions, ring positions."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q_nope, q_rope = _queries(rng, T, H)
    R = T // q_per_seq
    main = _pool(rng, kv_dtype, main_rows)
    swa = _pool(rng, kv_dtype, max(R * window, 1))
    sink = rng.standard_normal(H, dtype=np.float32)
    midx = np.empty((R, topk), dtype=np.int32)
    for r in range(R):
        midx[r] = rng.choice(main_rows, size=topk, replace=False)
    _set_invalid(rng, midx, invalid)
    sidx = np.empty((R, window), dtype=np.int32)
    for r in range(R if window else 0):
        start = int(rng.integers(0, window))
        sidx[r] = r * window + (start + np.arange(window)) % window
        sidx[r, :swa_invalid] = -1
    arrays = {"q_nope": q_nope, "q_rope": q_rope, "sink": sink, "main": main, "swa": swa,
              "main_indices": midx, "swa_indices": sidx}
    scale = 1.0 / math.sqrt(DIM) if softmax_scale is None else softmax_scale
    return Workload(name, T, H, q_per_seq, kv_dtype, main_rows, scale, arrays, two_source=True, note=note)


# ----------------------------------------------------------------------------
# the named configurations
# ----------------------------------------------------------------------------
CONFIG_NAMES = ("tiny_bf16", "bf16_topk_swa", "fp8_ue8m0", "long_context_bf16", "ragged_mtp4_fp8",
                "fp8_two_source")


def config(i: int, **over) -> Workload:
    """The five workloads of the statement, by position 0..4, and the
    two-source (main + SWA) decode as 5."""
    if i == 0:
        kw = dict(T=2, H=16, kv_dtype="bf16", pool_rows=512, topk=64, invalid=8, seed=0)
        kw.update(over)
        return dense_workload("tiny_bf16 T=2 H=16 K=64 pool=512", **kw)
    if i == 1:
        kw = dict(T=8, H=64, kv_dtype="bf16", pool_rows=32768, topk=2048, swa=128,
                  invalid=round(0.01 * 2176), seed=1)
        kw.update(over)
        return dense_workload("bf16 T=8 H=64 K=2048+128swa pool=32768", **kw)
    if i == 2:
        kw = dict(T=32, H=128, kv_dtype="fp8", pool_rows=131072, topk=2048,
                  invalid=round(0.005 * 2048), seed=2)
        kw.update(over)
        return dense_workload("fp8-e4m3/ue8m0 T=32 H=128 K=2048 pool=131072", **kw)
    if i == 3:
        kw = dict(T=1, H=128, kv_dtype="bf16", pool_rows=1 << 20, topk=65536, swa=128,
                  sorted_topk=True, seed=3)
        kw.update(over)
        return dense_workload("bf16 long context T=1 H=128 K=65536+128swa pool=1M", **kw)
    if i == 4:
        kw = dict(B=64, q_per_seq=4, H=128, kv_dtype="fp8", pool_rows=262144, max_k=8192,
                  zero_rows=4, seed=4)
        kw.update(over)
        return ragged_workload("ragged MTP4 fp8 B=64x4 H=128 K_b<=8192 pool=262144", **kw)
    if i == 5:
        kw = dict(T=32, H=128, kv_dtype="fp8", main_rows=131072, topk=2048, window=128,
                  invalid=round(0.005 * 2048), seed=5)
        kw.update(over)
        return two_source_workload("fp8 two-source T=32 H=128 K=2048 main + 128 swa", **kw)
    raise ValueError(i)


MATRIX_T = (1, 2, 4, 8, 16, 32, 48, 64)
MATRIX_CTX = (4096, 32768, 102400, 512000, 1048576)
MATRIX_VARIANTS = {"bf16_h128": ("bf16", 128), "fp8_h128": ("fp8", 128), "bf16_h16": ("bf16", 16)}


def matrix_cell(T: int, ctx: int, variant: str = "bf16_h128", seed: int | None = None) -> Workload:
    """T x context cell: pool of `ctx` rows, K = ctx/16 sorted unique top-k + the
    last 128 rows as a sliding window, q and sink ~ N(0,1), one index row per token.
    The pool depends on (ctx, variant) only: seed 100 + ctx index (+ 50 for fp8);
    q, sink and indices on the cell: seed 1000 + 10 * T index + ctx index."""
    kv_dtype, H = MATRIX_VARIANTS[variant]
    ic = MATRIX_CTX.index(ctx)
    if seed is None:
        seed = 1000 + 10 * MATRIX_T.index(T) + ic
    return dense_workload(f"{variant} T={T} ctx={ctx}", T=T, H=H, kv_dtype=kv_dtype, pool_rows=ctx,
                          topk=ctx // 16, swa=128, sorted_topk=True, seed=seed,
                          pool_seed=100 + ic + (50 if kv_dtype == "fp8" else 0))


def algorithmic_bytes(w: Workload) -> int:
    """Bytes the decode must move at least once: each valid gathered row once per
    index row, every index, q, out (bf16), lse (fp32) and sink."""
    a = w.arrays
    rb = w.row_bytes()
    if w.two_source:
        nidx = a["main_indices"].size + a["swa_indices"].size
        nvalid = _two_source_valid(w)
        written_tokens = w.num_tokens
    elif w.ragged:
        flat = a["kv_indices"][int(a["kv_indptr"][0]):]
        nidx = flat.size
        nvalid = int(np.count_nonzero((flat >= 0) & (flat < w.pool_rows)))
        written_tokens = int(np.count_nonzero(np.diff(a["kv_indptr"]) > 0)) * w.q_per_seq
    else:
        idx = a["indices"]
        nidx = idx.size
        nvalid = int(np.count_nonzero((idx >= 0) & (idx < w.pool_rows)))
        written_tokens = w.num_tokens
    H = w.num_heads
    q = written_tokens * H * DIM * 2
    out = written_tokens * H * DIM * 2 + written_tokens * H * 4
    return nvalid * rb + nidx * 4 + q + out + H * 4


def _two_source_valid(w: Workload) -> int:
    a = w.arrays
    n_swa = (a["swa"]["kv"] if "kv" in a["swa"] else a["swa"]["nope"]).shape[0]
    mi, si = a["main_indices"], a["swa_indices"]
    return int(np.count_nonzero((mi >= 0) & (mi < w.pool_rows)) + np.count_nonzero((si >= 0) & (si < n_swa)))


def algorithmic_flops(w: Workload) -> int:
    """2*512 (QK) + 2*512 (PV) flops per valid gathered row per query row."""
    a = w.arrays
    M = w.num_heads * w.q_per_seq
    if w.two_source:
        return 2048 * M * _two_source_valid(w)
    if w.ragged:
        ptr = a["kv_indptr"]
        tot = 0
        for b in range(len(ptr) - 1):
            seg = a["kv_indices"][ptr[b]:ptr[b + 1]]
            tot += int(np.count_nonzero((seg >= 0) & (seg < w.pool_rows)))
        return 2048 * M * tot
    idx = a["indices"]
    nvalid = int(np.count_nonzero((idx >= 0) & (idx < w.pool_rows)))
    return 2048 * M * nvalid


# ----------------------------------------------------------------------------
# fp8/UE8M0 cache writer
# ----------------------------------------------------------------------------
WRITER_ROW_READ = DIM * 2                             # one bf16 latent row
WRITER_ROW_WRITE = NOPE + SCALE_STRIDE + ROPE * 2     # 448 bytes + 8 code bytes + 128 RoPE bytes
WRITER_SLOT = 4                                       # int32 destination slot


def writer_workload(rows: int, pool_rows: int, seed: int = 7) -> dict:
    """Latent rows for the cache writer: N(0,1) rounded to bf16, each row
    scaled by 2^U{-8..8} (so the seven blocks of a row take different codes
    across rows), written to distinct random slots of a pool_rows-row pool."""
    assert rows <= pool_rows
    rng = np.random.default_rng(seed)
    kv = np.empty((rows, DIM), dtype=np.uint16)
    for r0 in range(0, rows, 65536):
        r1 = min(rows, r0 + 65536)
        x = rng.standard_normal((r1 - r0, DIM), dtype=np.float32)
        x *= np.exp2(rng.integers(-8, 9, size=(r1 - r0, 1))).astype(np.float32)
        kv[r0:r1] = f32_to_bf16_bits(x)
    slots = rng.permutation(pool_rows)[:rows].astype(np.int32)
    return {"kv": kv, "slots": slots, "pool_rows": pool_rows,
            "name": f"fp8 cache write rows={rows} pool={pool_rows}"}


def writer_algorithmic_bytes(rows: int) -> int:
    """Each latent row read once, its fp8 row (bytes, codes, RoPE) written once, one slot read."""
    return rows * (WRITER_ROW_READ + WRITER_ROW_WRITE + WRITER_SLOT)


# ----------------------------------------------------------------------------
# dense paged GQA decode (pa_decode)
# ----------------------------------------------------------------------------
def paged_workload(name: str, *, B: int, mtp: int, Hq: int, Hkv: int, max_ctx: int, page: int, seed: int,
                   lens=None, spare_blocks: int = 3, softmax_scale: float | None = None) -> dict:
    """q ~ N(0,1) bf16 [B*mtp, Hq, 512]; K and V caches ~ N(0,1) bf16
    [num_blocks, page, Hkv, 512] with every sequence's pages at distinct
    random blocks (a random permutation, spare_blocks never referenced);
    context lengths `lens` (default: every sequence at max_ctx)."""
    rng = np.random.default_rng(seed)
    pages = -(-max_ctx // page)
    nblk = B * pages + spare_blocks
    q = _normal_bf16(rng, (B * mtp, Hq, DIM))
    k = _normal_bf16(rng, (nblk, page, Hkv, DIM))
    v = _normal_bf16(rng, (nblk, page, Hkv, DIM))
    bt = rng.permutation(nblk)[:B * pages].reshape(B, pages).astype(np.int32)
    cl = np.full(B, max_ctx, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
    return {"name": name, "q": q, "k": k, "v": v, "block_tables": bt, "context_lens": cl, "B": B, "mtp": mtp,
            "Hq": Hq, "Hkv": Hkv, "max_ctx": max_ctx, "page": page, "num_blocks": nblk,
            "softmax_scale": float(np.float32(1.0 / np.sqrt(DIM))) if softmax_scale is None else softmax_scale}


def paged_config() -> dict:
    """The pa_decode page's BF16 D512 MTP4 GQA16 case at batch 16 and an 8K
    context, with one KV head (the page does not print the KV head count) and
    16-row pages; every sequence at the full 8192 positions."""
    return paged_workload("paged bf16 D512 MTP4 GQA16 B16 ctx8K", B=16, mtp=4, Hq=16, Hkv=1, max_ctx=8192, page=16,
                          seed=41)


def paged_algorithmic_bytes(w: dict) -> int:
    """Each position's K and V row of every KV head read once (MTP-causal
    positions included once), q read, out (bf16) and lse (fp32) written, the
    block-table entries and lengths read."""
    cl = np.minimum(np.maximum(w["context_lens"], 0), w["max_ctx"]).astype(np.int64)
    rows = int(cl.sum()) * w["Hkv"]
    T, Hq = w["B"] * w["mtp"], w["Hq"]
    pages = int(np.sum(-(-cl // w["page"])))
    return rows * 2 * DIM * 2 + T * Hq * DIM * 2 * 2 + T * Hq * 4 + pages * 4 + w["B"] * 4


def paged_algorithmic_flops(w: dict) -> int:
    """2*512 (QK) + 2*512 (PV) flops per (query row, visible position)."""
    cl = np.minimum(np.maximum(w["context_lens"], 0), w["max_ctx"]).astype(np.int64)
    mtp = w["mtp"]
    vis = sum(max(int(L) - (mtp - 1 - i), 0) for L in cl for i in range(mtp))
    return 2048 * w["Hq"] * vis

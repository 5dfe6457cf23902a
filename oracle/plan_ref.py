"""Integer plans of sparse MLA decode -- test infrastructure only.

* ``num_kv_splits`` -- the host split-count cost model.  The aiter page
  "[ASM][HIP][MLA v4 nm] Split plan helper and persistent decode kernel"
  (Summary, part 1) states what it minimises: workgroup waves times per-wave
  KV time, plus the partial-write / stage-2 cost of splitting, computed on the
  host from (num_seqs, num_heads, kv_len) only.  The vLLM page "[ROCm][DSV4]
  [Perf] Optimize Triton sparse-MLA decode on gfx950" (Design) caps short
  workloads at four splits and allows up to 32 for long contexts.  The fitted
  coefficients are not printed on either page; here they are an explicit
  argument, so the formula is pinned while the library's fitted values are
  parity unpinned.
* ``split_bounds`` lives in ``oracle.ref`` (it defines the partial semantics).
"""
from __future__ import annotations

from dataclasses import dataclass

SPLIT_ALIGN = 64
MAX_SPLITS = 32


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class PlanModel:
    fixed_ps: int
    tile_ps: tuple  # (bf16, fp8)
    merge_ps: int
    part_ps: int
    wg_per_cu: int
    short_cap: int
    long_cap: int
    long_kv: int


def num_kv_splits(num_seqs: int, num_heads: int, q_per_seq: int, kv_len: int, kv_dtype: int, num_cus: int,
                  model: PlanModel) -> int:
    """argmin over s of

        waves(s) * (fixed + tile[dtype] * tiles(s)) + [s > 1] * (merge + part * num_seqs * M * s)

    with M = num_heads * q_per_seq query rows per index row, G = ceil(M / min(M, 64))
    row groups, waves(s) = ceil(num_seqs * G * s / (num_cus * wg_per_cu)) and
    tiles(s) = ceil(ceil(kv_len / s) / 64).  s runs over 1 .. min(cap, ceil(kv_len / 64)),
    cap = short_cap below long_kv indices, long_cap from there on; ties keep the
    smaller s.  Empty problems plan one split."""
    if min(num_seqs, num_heads, q_per_seq, kv_len) < 0:
        raise ValueError("negative size")
    if num_seqs == 0 or kv_len == 0 or num_heads == 0 or q_per_seq == 0:
        return 1
    cus = num_cus if num_cus > 0 else 256
    M = num_heads * q_per_seq
    G = _cdiv(M, min(M, 64))
    slots = cus * model.wg_per_cu
    cap = model.short_cap if kv_len < model.long_kv else model.long_cap
    cap = min(cap, _cdiv(kv_len, SPLIT_ALIGN))
    best_s, best = 1, None
    for s in range(1, cap + 1):
        waves = _cdiv(num_seqs * G * s, slots)
        tiles = _cdiv(_cdiv(kv_len, s), SPLIT_ALIGN)
        cost = waves * (model.fixed_ps + model.tile_ps[kv_dtype] * tiles)
        if s > 1:
            cost += model.merge_ps + model.part_ps * num_seqs * M * s
        if best is None or cost < best:
            best, best_s = cost, s
    return best_s

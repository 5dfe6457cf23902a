"""Integer plans of sparse MLA decode -- test infrastructure only.

* ``num_kv_splits`` / ``plan_decode`` -- the host split-count cost model.  The
  aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and persistent decode
  kernel" (Summary, part 1) prices a split count by its rounds of workgroups
  times the KV time of one round, plus what splitting adds (writing the
  partials and merging them), from (num_seqs, num_heads, kv_len) alone, on
  the host.  The library has two kinds of decode workgroup (narrow: 16 query
  rows; wide: 128 query rows sharing each gathered row), so the modelled time
  of a split count is that of the cheaper kind, and the plan also names which
  kind won.  The vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA
  decode on gfx950" (Design) caps short workloads at four splits and allows
  more for long contexts (32 for its kernel; the caps are model fields
  here).  The fitted coefficients are not printed on
  either page; here they are an explicit argument, so the formula is pinned
  while the library's fitted values are parity unpinned.
* ``split_bounds`` lives in ``oracle.ref`` (it defines the partial semantics).
"""
from __future__ import annotations

from dataclasses import dataclass

SPLIT_ALIGN = 64
MAX_SPLITS = 256


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class PlanModel:
    fixed_ps: int
    step_ps: int
    step_load_ps: int
    merge_ps: int
    part_ps: int
    rows_per_wg: int
    waves_per_wg: int
    wg_per_cu: int
    short_cap: int
    long_cap: int
    long_kv: int
    wide_rows: int = 0
    wide_tile: int = 32
    wide_fixed_ps: int = 0
    wide_tile_ps: int = 0
    wide_tile_fp8_ps: int = 0
    wide_tile_load_ps: int = 0
    wide_cap: int = 0  # wide split cap from long_kv on; 0: long_cap


def split_cost(s: int, num_seqs: int, num_heads: int, q_per_seq: int, kv_len: int, num_cus: int,
               model: PlanModel) -> int:
    """Modelled picoseconds of a plan with s splits:

        waves(s) * (fixed + steps(s) * (step + floor(step_load * busy(s) / slots)))
          + [s > 1] * (merge + part * num_seqs * M * s)

    M = num_heads * q_per_seq query rows per index row, G = ceil(M / rows_per_wg)
    workgroups per index row and split, slots = num_cus * wg_per_cu,
    wgs(s) = num_seqs * G * s, waves(s) = ceil(wgs(s) / slots), busy(s) = min(wgs(s), slots),
    chunk(s) = the split length of ``ref.split_bounds`` (ceil(kv_len / s) rounded up
    to 64), steps(s) = ceil(ceil(min(chunk(s), kv_len) / 16) / waves_per_wg)."""
    cus = num_cus if num_cus > 0 else 256
    M = num_heads * q_per_seq
    G = _cdiv(M, model.rows_per_wg)
    slots = cus * model.wg_per_cu
    wgs = num_seqs * G * s
    waves = _cdiv(wgs, slots)
    busy = min(wgs, slots)
    chunk = _cdiv(_cdiv(kv_len, s), SPLIT_ALIGN) * SPLIT_ALIGN
    steps = _cdiv(_cdiv(min(chunk, kv_len), 16), model.waves_per_wg)
    cost = waves * (model.fixed_ps + steps * (model.step_ps + model.step_load_ps * busy // slots))
    if s > 1:
        cost += model.merge_ps + model.part_ps * num_seqs * M * s
    return cost


def wide_split_cost(s: int, num_seqs: int, num_heads: int, q_per_seq: int, kv_len: int, kv_dtype: int,
                    num_cus: int, model: PlanModel) -> int | None:
    """Modelled picoseconds of s splits on the wide workgroups, or None where
    they do not apply (wide_rows == 0 or M not a multiple of wide_rows):

        waves_w(s) * (wide_fixed + tiles(s) * (tile + floor(wide_tile_load * busy_w(s) / cus)))
          + [s > 1] * (merge + part * num_seqs * M * s)

    one workgroup per CU: wgs_w(s) = num_seqs * (M / wide_rows) * s,
    waves_w(s) = ceil(wgs_w(s) / cus), busy_w(s) = min(wgs_w(s), cus);
    tiles(s) = ceil(min(chunk(s), kv_len) / wide_tile) with chunk(s) as in
    ``split_cost``; tile = wide_tile_fp8 for kv_dtype 1 (fp8), else wide_tile."""
    M = num_heads * q_per_seq
    if model.wide_rows <= 0 or M % model.wide_rows != 0:
        return None
    cus = num_cus if num_cus > 0 else 256
    wgs = num_seqs * (M // model.wide_rows) * s
    waves = _cdiv(wgs, cus)
    busy = min(wgs, cus)
    chunk = _cdiv(_cdiv(kv_len, s), SPLIT_ALIGN) * SPLIT_ALIGN
    tiles = _cdiv(min(chunk, kv_len), model.wide_tile)
    tile = model.wide_tile_fp8_ps if kv_dtype == 1 else model.wide_tile_ps
    cost = waves * (model.wide_fixed_ps + tiles * (tile + model.wide_tile_load_ps * busy // cus))
    if s > 1:
        cost += model.merge_ps + model.part_ps * num_seqs * M * s
    return cost


def plan_decode(num_seqs: int, num_heads: int, q_per_seq: int, kv_len: int, kv_dtype: int, num_cus: int,
                model: PlanModel, two_source: bool = False) -> tuple[int, bool]:
    """(s, wide): s is the argmin over the split counts each family takes of
    the family's cost (``split_cost`` narrow, ``wide_split_cost`` wide); ties
    keep the smaller s, and at one s wide wins only when strictly cheaper.
    Below long_kv indices both families take s <= short_cap; from there on
    narrow takes s <= long_cap and wide s <= wide_cap (0: long_cap); every cap
    is also at most ceil(kv_len / 64).  A two-source call, or a model without
    wide workgroups, prices narrow alone.  Empty problems plan (1, False)."""
    if min(num_seqs, num_heads, q_per_seq, kv_len) < 0:
        raise ValueError("negative size")
    if num_seqs == 0 or kv_len == 0 or num_heads == 0 or q_per_seq == 0:
        return 1, False
    tiles = _cdiv(kv_len, SPLIT_ALIGN)
    short = kv_len < model.long_kv
    cap_n = min(model.short_cap if short else model.long_cap, tiles)
    cap_w = min(model.short_cap if short else (model.wide_cap or model.long_cap), tiles)
    best_s, best, best_wide = 1, None, False
    for s in range(1, max(cap_n, cap_w) + 1):
        cost, wide = None, False
        if s <= cap_n:
            cost = split_cost(s, num_seqs, num_heads, q_per_seq, kv_len, num_cus, model)
        if not two_source and s <= cap_w:
            cw = wide_split_cost(s, num_seqs, num_heads, q_per_seq, kv_len, kv_dtype, num_cus, model)
            if cw is not None and (cost is None or cw < cost):
                cost, wide = cw, True
        if cost is not None and (best is None or cost < best):
            best, best_s, best_wide = cost, s, wide
    return best_s, best_wide


def num_kv_splits(num_seqs: int, num_heads: int, q_per_seq: int, kv_len: int, kv_dtype: int, num_cus: int,
                  model: PlanModel) -> int:
    """The split count of ``plan_decode`` for a one-source call."""
    return plan_decode(num_seqs, num_heads, q_per_seq, kv_len, kv_dtype, num_cus, model)[0]


# ----------------------------------------------------------------------------
# persistent plan: balanced contiguous partition of all 64-position tiles
# ----------------------------------------------------------------------------
# The aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and persistent decode
# kernel" (Summary, part 2) has the persistent kernel derive its split plan
# inside the kernel from the live kv_indptr and merge split rows in the
# workgroup that arrives last.  The pages do not print the partition rule; the
# reading used here: every sequence b with tiles_b = ceil(K_b / 64) > 0
# takes tiles_b + SEQ_OVERHEAD plan units -- SEQ_OVERHEAD units charged for
# the fixed cost of a piece, then one unit per tile -- and a sequence with
# K_b = 0 takes none.  The units of all sequences are concatenated in
# sequence order, partition p of P owns the units [floor(p*total/P),
# floor((p+1)*total/P)), and a tile belongs to the partition owning its unit.
# (With SEQ_OVERHEAD = 0 this is the plain balanced split of the tiles.)  A
# sequence whose tiles fall in more than one partition is split; its pieces
# merge in partition order.  With fewer units than partitions some partitions
# are empty, and they may sit between two pieces of one sequence, so the piece
# count is the number of partitions that own a tile of the sequence, not the
# width of the partition span.  A partition holds at most two split pieces
# (one that starts at its first unit and one that continues past its end), so
# piece (p, b) has slot 2p when it starts at p's first unit and 2p+1
# otherwise.

PERSIST_TILE = 64
SEQ_OVERHEAD = 2  # plan units charged per sequence with tiles (a measured cost, not the pages')


@dataclass
class Piece:
    seq: int         # sequence b
    begin: int       # first index position of the piece within the sequence
    end: int         # one past the last position (<= K_b)
    split: bool      # the sequence has pieces in more than one partition
    slot: int        # partial slot of a split piece (2p or 2p+1), else -1
    first_part: int  # first partition holding a piece of the sequence
    num_pieces: int  # partitions owning a tile of the sequence


def partition(kv_indptr, num_partitions: int, seq_overhead: int = SEQ_OVERHEAD):
    """Returns (descriptors, pieces): descriptors[p] = (u0, u1, b_first, b_last)
    with [u0, u1) the units of partition p and b_first / b_last the first /
    last sequence with a tile in it (-1, -1 when it holds no tile); pieces[p] =
    the list of Piece of p in sequence order."""
    P = int(num_partitions)
    if P < 1:
        raise ValueError("num_partitions must be >= 1")
    if seq_overhead < 0:
        raise ValueError("seq_overhead must be >= 0")
    ptr = [int(x) for x in kv_indptr]
    B = len(ptr) - 1
    lens = [ptr[b + 1] - ptr[b] for b in range(B)]
    if any(k < 0 for k in lens):
        raise ValueError("kv_indptr must be non-decreasing")
    tiles = [_cdiv(k, PERSIST_TILE) for k in lens]
    units = [t + seq_overhead if t > 0 else 0 for t in tiles]
    first_tile = [0] * B  # global unit of each sequence's first tile
    u = 0
    for b in range(B):
        first_tile[b] = u + (units[b] - tiles[b])
        u += units[b]
    total = u
    bounds = [p * total // P for p in range(P + 1)]

    def owner(unit):  # the partition whose range holds `unit`
        p = 0
        while bounds[p + 1] <= unit:
            p += 1
        return p

    descs, pieces = [], []
    for p in range(P):
        u0, u1 = bounds[p], bounds[p + 1]
        mine = []
        for b in range(B):
            lo, hi = max(u0, first_tile[b]), min(u1, first_tile[b] + tiles[b])
            if lo >= hi:
                continue
            owners = sorted({owner(first_tile[b] + t) for t in range(tiles[b])})
            fp, lp = owners[0], owners[-1]
            mine.append(Piece(seq=b, begin=(lo - first_tile[b]) * PERSIST_TILE,
                              end=min((hi - first_tile[b]) * PERSIST_TILE, lens[b]),
                              split=lp > fp, slot=(2 * p + (0 if lo == u0 else 1)) if lp > fp else -1,
                              first_part=fp, num_pieces=len(owners)))
        descs.append((u0, u1, mine[0].seq, mine[-1].seq) if mine else (u0, u1, -1, -1))
        pieces.append(mine)
    return descs, pieces


def default_partitions(num_heads: int, q_per_seq: int, num_cus: int = 256, wg_per_cu: int = 1) -> int:
    """Partitions that fill the machine once: num_cus * wg_per_cu workgroups over
    the query-row groups of M = num_heads * q_per_seq rows.  A group is 128 rows
    when 128 divides M, else 64 when 64 does, else 32 when 32 does, else 16."""
    M = num_heads * q_per_seq
    rows = 128 if M % 128 == 0 else (64 if M % 64 == 0 else (32 if M % 32 == 0 else 16))
    return max(1, (num_cus * wg_per_cu) // (M // rows))

"""Pins of the oracle's persistent plan (the balanced contiguous partition of
the sequences' plan units -- two charged per sequence, then one per
64-position tile -- over P partitions) and of the piecewise merge it implies.
CPU only."""
import dataclasses

import numpy as np
import pytest

import workloads as wl
from oracle import plan_ref as pr
from oracle import ref


def test_partition_hand_example():
    # Without charged units (the plain split of the tiles):
    # K_b = 100, 0, 200, 1  ->  tiles 2, 0, 4, 1 (ceil(K/64)); total 7; P = 3:
    # bounds floor(7p/3) = 0, 2, 4, 7.  Partition 0 = seq 0 (whole); partition
    # 1 = tiles 2..3 = seq 2 positions [0, 128); partition 2 = tiles 4..6 =
    # seq 2 positions [128, 200) then seq 3 [0, 1).  Seq 2 is split over
    # partitions 1 and 2 and is the first sequence of both (slots 2 and 4).
    # The indptr starts at an offset: only differences matter.
    descs, pieces = pr.partition([50, 150, 150, 350, 351], 3, seq_overhead=0)
    assert descs == [(0, 2, 0, 0), (2, 4, 2, 2), (4, 7, 2, 3)]
    got = [[(x.seq, x.begin, x.end, x.split, x.slot, x.first_part, x.num_pieces) for x in p] for p in pieces]
    assert got == [[(0, 0, 100, False, -1, 0, 1)],
                   [(2, 0, 128, True, 2, 1, 2)],
                   [(2, 128, 200, True, 4, 1, 2), (3, 0, 1, False, -1, 2, 1)]]


def test_partition_hand_example_charged_units():
    # The same lists with two units charged per sequence with tiles: units
    # 4, 0, 6, 3 (seq 0 = units 0..3, its tiles at 2, 3; seq 2 = units 4..9,
    # tiles at 6..9; seq 3 = units 10..12, its tile at 12); total 13; P = 3:
    # bounds floor(13p/3) = 0, 4, 8, 13.  Partition 0 = seq 0 (whole).
    # Partition 1 = seq 2's charged units 4, 5 and its tiles 0, 1 (units 6, 7):
    # positions [0, 128), which start after the partition's first unit, so the
    # piece takes the odd slot 3.  Partition 2 = seq 2 tiles 2, 3 (units 8, 9:
    # positions [128, 200), starting at the partition's first unit: slot 4),
    # then seq 3 whole.
    descs, pieces = pr.partition([50, 150, 150, 350, 351], 3)
    assert pr.SEQ_OVERHEAD == 2
    assert descs == [(0, 4, 0, 0), (4, 8, 2, 2), (8, 13, 2, 3)]
    got = [[(x.seq, x.begin, x.end, x.split, x.slot, x.first_part, x.num_pieces) for x in p] for p in pieces]
    assert got == [[(0, 0, 100, False, -1, 0, 1)],
                   [(2, 0, 128, True, 3, 1, 2)],
                   [(2, 128, 200, True, 4, 1, 2), (3, 0, 1, False, -1, 2, 1)]]
    # K = 64, 64 -> units 3, 3; P = 6 gives one unit per partition: partitions
    # 0, 1, 3, 4 own only charged units and hold no piece.
    descs, pieces = pr.partition([0, 64, 128], 6)
    assert descs == [(0, 1, -1, -1), (1, 2, -1, -1), (2, 3, 0, 0), (3, 4, -1, -1), (4, 5, -1, -1), (5, 6, 1, 1)]
    assert [[(x.seq, x.begin, x.end, x.split) for x in p] for p in pieces] == [
        [], [], [(0, 0, 64, False)], [], [], [(1, 0, 64, False)]]


def test_partition_last_piece_takes_odd_slot():
    # K = 64, 128 -> tiles 1, 2; P = 2: bounds 0, 1, 3.  Partition 0 = seq 0 only;
    # partition 1 = seq 1 whole.  Now K = 128, 128, P = 3: bounds 0, 1, 2, 4:
    # partition 1 = tile 1 (seq 0 second half) -> first sequence, slot 2;
    # partition 0 = seq 0 first half, slot 0; partition 2 = seq 1 whole.
    _, pieces = pr.partition([0, 128, 256], 3, seq_overhead=0)
    assert [(x.seq, x.begin, x.end, x.slot) for x in pieces[0]] == [(0, 0, 64, 0)]
    assert [(x.seq, x.begin, x.end, x.slot) for x in pieces[1]] == [(0, 64, 128, 2)]
    assert [(x.seq, x.begin, x.end, x.split) for x in pieces[2]] == [(1, 0, 128, False)]
    # K = 64, 192, P = 2: tiles 1, 3; bounds 0, 2, 4: partition 0 = seq 0 then
    # seq 1 tile 0 -> seq 1's piece there is not the first sequence: slot 1.
    _, pieces = pr.partition([0, 64, 256], 2, seq_overhead=0)
    assert [(x.seq, x.slot) for x in pieces[0]] == [(0, -1), (1, 1)]
    assert [(x.seq, x.begin, x.end, x.slot) for x in pieces[1]] == [(1, 64, 192, 2)]


def _random_indptr(rng, B, kmax, zero_frac=0.2, offset=0):
    k = rng.integers(0, kmax + 1, size=B)
    k[rng.random(B) < zero_frac] = 0
    return np.concatenate([[offset], offset + np.cumsum(k)]).astype(np.int64)


@pytest.mark.parametrize("charged", [0, 2, 5])
@pytest.mark.parametrize("seed", range(24))
def test_partition_invariants(seed, charged):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    ptr = _random_indptr(rng, B, int(rng.choice([5, 64, 300, 3000])), offset=int(rng.integers(0, 1000)))
    P = int(rng.choice([1, 2, 3, 7, 32, 64, 300, 5000]))
    descs, pieces = pr.partition(ptr, P, seq_overhead=charged)
    lens = np.diff(ptr)
    tiles = -(-lens // 64)
    units = np.where(tiles > 0, tiles + charged, 0)
    total = int(units.sum())
    first_tile = np.cumsum(units) - tiles  # global unit of each sequence's first tile
    # partition sizes (in units) differ by at most one and cover the range in order
    sizes = [d[1] - d[0] for d in descs]
    assert sum(sizes) == total and max(sizes) - min(sizes) <= 1
    assert descs[0][0] == 0 and descs[-1][1] == total
    assert all(descs[p][1] == descs[p + 1][0] for p in range(P - 1))
    # every position of every sequence is covered exactly once, in (partition, seq) order
    seen = {b: [] for b in range(B)}
    for p, plist in enumerate(pieces):
        assert [x.seq for x in plist] == sorted({x.seq for x in plist})
        if plist:
            assert descs[p][2] == plist[0].seq and descs[p][3] == plist[-1].seq
        else:
            assert descs[p][2:] == (-1, -1)
        for x in plist:
            assert x.begin % 64 == 0 and 0 <= x.begin < x.end <= lens[x.seq]
            # the piece's tiles are units of this partition
            u_lo, u_hi = first_tile[x.seq] + x.begin // 64, first_tile[x.seq] + -(-x.end // 64)
            assert descs[p][0] <= u_lo < u_hi <= descs[p][1]
            seen[x.seq].append((p, x.begin, x.end))
    for b in range(B):
        segs = seen[b]
        if lens[b] == 0:
            assert segs == []  # K = 0 sequences get nothing
            continue
        ps = [s[0] for s in segs]
        assert ps == sorted(set(ps))  # increasing partitions ...
        for q in range(ps[0], ps[-1] + 1):  # ... and any partition between them owns no tile
            assert q in ps or descs[q][0] == descs[q][1]
        cover = [s[1:] for s in segs]
        assert cover[0][0] == 0 and cover[-1][1] == lens[b]
        assert all(cover[i][1] == cover[i + 1][0] for i in range(len(cover) - 1))
    # split flags, piece counts and slots
    slots = []
    for p, plist in enumerate(pieces):
        for i, x in enumerate(plist):
            n = len(seen[x.seq])
            assert x.num_pieces == n and x.split == (n > 1) and x.first_part == seen[x.seq][0][0]
            if x.split:
                starts_at_first_unit = first_tile[x.seq] + x.begin // 64 == descs[p][0]
                assert x.slot == 2 * p + (0 if starts_at_first_unit else 1)
                slots.append(x.slot)
            else:
                assert x.slot == -1
    assert len(slots) == len(set(slots)) and all(0 <= s < 2 * P for s in slots)


def test_partition_edge_cases():
    # no work at all: every partition empty
    descs, pieces = pr.partition([7, 7, 7], 4)
    assert all(d == (0, 0, -1, -1) for d in descs) and all(p == [] for p in pieces)
    # more partitions than tiles: bounds floor(4p/8) = 0,0,1,1,2,2,3,3,4, so the
    # odd partitions own one tile each and the even ones are empty -- empty
    # partitions sit between the pieces, which still number 4 (not 7 = 7 - 1 + 1)
    descs, pieces = pr.partition([0, 200], 8, seq_overhead=0)  # 4 tiles
    assert sum(1 for p in pieces if p) == 4
    assert [(x.begin, x.end, x.slot) for p in pieces for x in p] == [(0, 64, 2), (64, 128, 6), (128, 192, 10),
                                                                      (192, 200, 14)]
    assert all(x.num_pieces == 4 and x.first_part == 1 for p in pieces for x in p)
    # with the two charged units: 6 units, bounds floor(6p/8) = 0,0,1,2,3,3,4,5,6;
    # partitions 1, 2 own the charged units, 3, 5, 6, 7 one tile each
    descs, pieces = pr.partition([0, 200], 8)
    assert [d[:2] for d in descs] == [(0, 0), (0, 1), (1, 2), (2, 3), (3, 3), (3, 4), (4, 5), (5, 6)]
    assert [(x.begin, x.end, x.slot) for p in pieces for x in p] == [(0, 64, 6), (64, 128, 10), (128, 192, 12),
                                                                      (192, 200, 14)]
    assert all(x.num_pieces == 4 and x.first_part == 3 for p in pieces for x in p)
    with pytest.raises(ValueError):
        pr.partition([0, 5], 2, seq_overhead=-1)
    with pytest.raises(ValueError):
        pr.partition([0, 5], 0)
    with pytest.raises(ValueError):
        pr.partition([5, 0], 2)


def test_default_partitions():
    assert pr.default_partitions(128, 4) == 64  # M = 512: four 128-row groups
    assert pr.default_partitions(128, 1) == 256  # M = 128: one group
    assert pr.default_partitions(64, 2) == 256   # M = 128
    assert pr.default_partitions(64, 3) == 85    # M = 192: three 64-row groups
    assert pr.default_partitions(16, 1) == 256  # M = 16: one 16-row group
    assert pr.default_partitions(16, 3) == 85   # M = 48: three 16-row groups
    assert pr.default_partitions(32, 3) == 85   # M = 96: three 32-row groups
    assert pr.default_partitions(64, 1, num_cus=80) == 80


@pytest.mark.parametrize("seed,P", [(0, 5), (1, 32), (2, 3), (3, 200)])
def test_piecewise_merge_equals_unsplit(seed, P):
    """Partials of the pieces, merged in partition order with the sink, equal the
    unsplit ragged decode (the split-merge identity over the persistent plan)."""
    w = wl.ragged_workload("persist pin", B=6, q_per_seq=2, H=16, kv_dtype="fp8", pool_rows=700, max_k=400,
                           zero_rows=2, seed=seed)
    a = w.arrays
    pool = {"nope": a["nope"], "scale": a["scale"], "rope": a["rope"]}
    ptr, flat = a["kv_indptr"], a["kv_indices"]
    want_o, want_l, written = ref.sparse_mla_decode_ragged(a["q_nope"], a["q_rope"], pool, ptr, flat, a["sink"],
                                                           w.softmax_scale, 2)
    q = ref.queries(a["q_nope"], a["q_rope"])
    H = q.shape[1]
    n = ref.pool_size(pool)
    _, pieces = pr.partition(ptr, P)
    parts = {}
    for plist in pieces:
        for x in plist:
            idx = np.asarray(flat[ptr[x.seq] + x.begin:ptr[x.seq] + x.end])
            k = ref.pool_rows(pool, idx[ref.valid_mask(idx, n)])
            qb = q[x.seq * 2:(x.seq + 1) * 2].reshape(-1, 512)
            parts.setdefault(x.seq, []).append(ref.partial_one(qb, k, w.softmax_scale))
    for b, lst in parts.items():
        o = np.stack([p[0] for p in lst], axis=1).reshape(2, H, len(lst), 512)
        l = np.stack([p[1] for p in lst], axis=1).reshape(2, H, len(lst))
        mo, ml = ref.merge_partials(o, l, a["sink"])
        np.testing.assert_allclose(mo, want_o[b * 2:(b + 1) * 2], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, want_l[b * 2:(b + 1) * 2], rtol=0, atol=1e-12)
    assert set(parts) == {b for b in range(len(ptr) - 1) if ptr[b + 1] > ptr[b]}
    assert written.sum() == 2 * len(parts)


# ----------------------------------------------------------------------------
# host split planner: the cost formula worked out by hand
# ----------------------------------------------------------------------------
def _fitted_model(wide: bool = True):
    """The library's built-in coefficients; wide=False leaves out the wide
    family (wide_rows = 0), so that only the narrow formula prices a plan."""
    return pr.PlanModel(fixed_ps=7194000, step_ps=1971000, step_load_ps=569000, merge_ps=4065000,
                        part_ps=287, rows_per_wg=16, waves_per_wg=8, wg_per_cu=1, short_cap=128,
                        long_cap=128, long_kv=4096, wide_rows=128 if wide else 0, wide_tile=32,
                        wide_fixed_ps=13648000, wide_tile_ps=1774000, wide_tile_fp8_ps=2192000,
                        wide_tile_load_ps=536000, wide_cap=256)


def test_planner_wide_cap_worked_example():
    """4 index rows x 128 heads x 65664 bf16 indices: from long_kv on, narrow
    takes up to long_cap = 128 splits and wide up to wide_cap = 256.
      s=61: 4*61 = 244 workgroups, one round; ceil(65664/61) = 1077 -> chunk
            1088, 34 tiles at 1774000 + 536000*244//256 = 2284875:
            13648000 + 34*2284875 + 4065000 + 287*4*128*61          = 104362334
      s=60: chunk ceil(1095/64)*64 = 1152, 36 tiles at 2276500:
            13648000 + 36*2276500 + 4065000 + 287*4*128*60          = 108483640
      s=62: 248 workgroups, chunk 1088, 34 tiles at 2293250:
            13648000 + 34*2293250 + 4065000 + 287*4*128*62          = 104794028
      s=64: 256 workgroups, 34 tiles at 2310000                      = 105657416
      s=65: 260 workgroups take two rounds                           = 188752360
      s=128: 512 workgroups in two rounds, ceil(65664/128) = 513 -> chunk
            576, 18 tiles at 2310000:
            2*(13648000 + 18*2310000) + 4065000 + 287*4*128*128     = 133329832
    so the plan is 61 splits on the wide kernel.  With both caps at 32
    (long_cap = 32) it is 32 splits on the wide kernel (157187208), below the
    narrow family's best, s = 8 (177534552); with the narrow family at 32 and
    wide_cap = 128 it is 61 wide splits again."""
    m = _fitted_model()
    want = {61: 104362334, 60: 108483640, 62: 104794028, 64: 105657416, 65: 188752360, 128: 133329832}
    for s, c in want.items():
        assert pr.wide_split_cost(s, 4, 128, 1, 65664, 0, 256, m) == c, s
    assert pr.plan_decode(4, 128, 1, 65664, 0, 256, m) == (61, True)
    m32 = dataclasses.replace(m, long_cap=32, wide_cap=0)
    assert pr.wide_split_cost(32, 4, 128, 1, 65664, 0, 256, m32) == 157187208
    assert pr.split_cost(8, 4, 128, 1, 65664, 256, m32) == 177534552
    assert pr.plan_decode(4, 128, 1, 65664, 0, 256, m32) == (32, True)
    assert pr.plan_decode(4, 128, 1, 65664, 0, 256, dataclasses.replace(m32, wide_cap=128)) == (61, True)
    # a short list keeps both families within short_cap
    assert pr.plan_decode(4, 128, 1, 2176, 0, 256, dataclasses.replace(m, short_cap=4))[0] <= 4


def test_planner_cost_worked_example_short_list():
    """8 index rows x 64 heads x 2176 indices on 256 slots, every term by hand.
    G = 64 / 16 = 4 workgroups per row and split, so wgs(s) = 32 s, one wave.
      s=1: chunk 2176, 136 half-tiles -> 17 steps, step 1971000 + 569000*32//256
           = 2042125; 7194000 + 17*2042125                         = 41910125
      s=2: chunk 1088 -> 68 -> 9 steps, step 2113250; 7194000 + 9*2113250
           + merge 4065000 + 287*8*64*2                            = 30572138
      s=3: ceil(2176/3) = 726 -> chunk 768 -> 48 -> 6 steps, step 2184375;
           7194000 + 6*2184375 + 4065000 + 287*8*64*3                = 24806082
      s=4: 544 -> chunk 576 -> 36 -> 5 steps, step 2255500;
           7194000 + 5*2255500 + 4065000 + 287*8*64*4                = 23124276
    and a short-list cap of 4 (2176 < 4096; the library's default is 128) stops
    at s = 4."""
    m = dataclasses.replace(_fitted_model(wide=False), short_cap=4)
    want = {1: 41910125, 2: 30572138, 3: 24806082, 4: 23124276}
    for s, c in want.items():
        assert pr.split_cost(s, 8, 64, 1, 2176, 256, m) == c, s
    assert pr.num_kv_splits(8, 64, 1, 2176, 0, 256, m) == 4


def test_planner_cost_worked_example_long_list_and_waves():
    """One row x 128 heads x 65664 indices (beyond 32 splits its 8 s
    workgroups take two rounds, so the plan stays below 33):
      s=32: chunk ceil(65664/32)=2052 -> 2112, 132 half-tiles -> 17 steps, all
            256 slots busy (step 2540000): 7194000 + 17*2540000 + 4065000
            + 287*128*32                                            = 55614552
      s=31: 2119 -> 2176 -> 136 -> 17 steps, 248 busy, step 1971000 +
            569000*248//256 = 2522218: 7194000 + 17*2522218 + 4065000
            + 287*128*31                                            = 55275522
      s=30: 2189 -> 2240 -> 140 -> 18 steps, step 2504437            = 57440946
    so 31 splits beat 32 (and every s <= 30 needs 18 or more steps).
    300 rows x 128 heads x 2048 indices: s=1 runs 2400 workgroups in 10 waves
    of 16 full-load steps, 10*(7194000 + 16*2540000) = 478340000; s=2 needs 19
    waves of 8 steps plus the merge, 19*27514000 + 4065000 + 287*300*128*2
    = 548872600.  (Narrow family alone; the wide terms are in the next test.)"""
    m = _fitted_model(wide=False)
    assert pr.split_cost(32, 1, 128, 1, 65664, 256, m) == 55614552
    assert pr.split_cost(31, 1, 128, 1, 65664, 256, m) == 55275522
    assert pr.split_cost(30, 1, 128, 1, 65664, 256, m) == 57440946
    assert pr.num_kv_splits(1, 128, 1, 65664, 0, 256, m) == 31
    assert pr.split_cost(1, 300, 128, 1, 2048, 256, m) == 478340000
    assert pr.split_cost(2, 300, 128, 1, 2048, 256, m) == 548872600
    assert pr.num_kv_splits(300, 128, 1, 2048, 1, 256, m) == 1


def test_planner_cost_worked_example_wide_family():
    """The same calls with the wide terms (128 query rows per workgroup, tiles
    of 32 positions, one workgroup per CU; every tile at full load costs
    2192000 + 536000 = 2728000 for fp8).  300 rows x 128 heads x 2048 fp8
    indices:
      s=1: 300 workgroups, 2 waves of 64 tiles: 2*(13648000 + 64*2728000)   = 376480000
      s=2: 600 workgroups, 3 waves of 32 tiles: 3*(13648000 + 32*2728000)
           + 4065000 + 287*300*128*2                                        = 328938600
      s=3: 900 -> 4 waves; chunk 683 -> 704, 22 tiles: 4*(13648000 + 22*2728000)
           + 4065000 + 287*300*128*3                                        = 331783400
      s=4: 1200 -> 5 waves; chunk 512, 16 tiles: 5*(13648000 + 16*2728000)
           + 4065000 + 287*300*128*4                                        = 334628200
    all below the narrow 478340000 and 548872600 of s = 1, 2, so the plan is
    two splits on the wide kernel.  One row x 128 heads x 65664 bf16 indices,
    s=32: 32 workgroups of 66 tiles at 1774000 + 536000*32//256 = 1841000:
    13648000 + 66*1841000 + 4065000 + 287*128*32 = 140394552, far above the
    narrow 55275522 of s = 31.  Beyond 128 splits (wide_cap = 256) the wide
    family wins there: s=206, 206 workgroups in one round at 1774000 +
    536000*206//256 = 2205312 per tile; ceil(65664/206) = 319 -> chunk 320,
    10 tiles: 13648000 + 10*2205312 + 4065000 + 287*128*206 = 47333736
    (s=205: chunk 384, 12 tiles, 51682496; s=207: 47391412).  With wide_cap =
    128 the best wide plan is s=128 (59171208) and the plan stays 31 narrow."""
    m = _fitted_model()
    assert pr.wide_split_cost(1, 300, 128, 1, 2048, 1, 256, m) == 376480000
    assert pr.wide_split_cost(2, 300, 128, 1, 2048, 1, 256, m) == 328938600
    assert pr.wide_split_cost(3, 300, 128, 1, 2048, 1, 256, m) == 331783400
    assert pr.wide_split_cost(4, 300, 128, 1, 2048, 1, 256, m) == 334628200
    assert pr.plan_decode(300, 128, 1, 2048, 1, 256, m) == (2, True)
    assert pr.plan_decode(300, 128, 1, 2048, 1, 256, m, two_source=True) == (1, False)
    assert pr.wide_split_cost(32, 1, 128, 1, 65664, 0, 256, m) == 140394552
    assert pr.wide_split_cost(206, 1, 128, 1, 65664, 0, 256, m) == 47333736
    assert pr.wide_split_cost(205, 1, 128, 1, 65664, 0, 256, m) == 51682496
    assert pr.wide_split_cost(207, 1, 128, 1, 65664, 0, 256, m) == 47391412
    assert pr.split_cost(31, 1, 128, 1, 65664, 256, m) == 55275522
    assert pr.plan_decode(1, 128, 1, 65664, 0, 256, m) == (206, True)
    assert pr.wide_split_cost(128, 1, 128, 1, 65664, 0, 256, m) == 59171208
    assert pr.plan_decode(1, 128, 1, 65664, 0, 256, dataclasses.replace(m, wide_cap=128)) == (31, False)
    # M = 64 is not a multiple of 128: no wide cost at all
    assert pr.wide_split_cost(1, 8, 64, 1, 2176, 0, 256, m) is None


"""CPU tests of libsmd's C ABI: exported symbols, host-side argument checks
(which run before any HIP call, so no GPU is needed), and the integer host
logic -- split bounds and the planner -- bit-exact against the oracle."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import sparse_mla_decode_index_amd as smd
from oracle import plan_ref, ref

HEADER = Path(__file__).resolve().parents[1] / "include" / "smd.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smd_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = smd.lib()
    names = declared_functions()
    assert "smd_sparse_mla_decode" in names and "smd_merge_partials" in names
    assert "smd_plan_num_kv_splits" in names
    for n in names:
        assert hasattr(L, n), f"libsmd.so does not export {n}"


def test_split_bounds_bit_exact_vs_oracle():
    rng = np.random.default_rng(0)
    cases = [(0, 1), (1, 1), (63, 2), (64, 4), (2176, 4), (65664, 32), (2048, 8)]
    cases += [(int(rng.integers(0, 100000)), int(rng.integers(1, 33))) for _ in range(300)]
    for K, s in cases:
        want = ref.split_bounds(K, s)
        got = [smd.split_bounds(K, s, r) for r in range(s)]
        assert got == want, (K, s)


def test_split_bounds_rejects_bad_args():
    with pytest.raises(smd.SmdError):
        smd.split_bounds(10, 0, 0)
    with pytest.raises(smd.SmdError):
        smd.split_bounds(10, 4, 4)
    with pytest.raises(smd.SmdError):
        smd.split_bounds(-1, 4, 0)


def _model_pair(rng):
    v = dict(fixed_ps=int(rng.integers(1, 10_000_000)), step_ps=int(rng.integers(1, 3_000_000)),
             step_load_ps=int(rng.integers(0, 3_000_000)), merge_ps=int(rng.integers(0, 10_000_000)),
             part_ps=int(rng.integers(0, 5_000)), rows_per_wg=int(rng.choice([16, 32, 64])),
             waves_per_wg=int(rng.choice([1, 4, 8])), wg_per_cu=int(rng.integers(1, 4)),
             short_cap=int(rng.integers(1, 33)), long_cap=int(rng.integers(1, 33)),
             long_kv=int(rng.integers(1, 20000)), wide_rows=int(rng.choice([0, 64, 128, 256])),
             wide_tile=int(rng.choice([16, 32, 64])), wide_fixed_ps=int(rng.integers(0, 30_000_000)),
             wide_tile_ps=int(rng.integers(1, 4_000_000)), wide_tile_fp8_ps=int(rng.integers(1, 4_000_000)),
             wide_tile_load_ps=int(rng.integers(0, 2_000_000)), wide_cap=int(rng.choice([0, 1, 16, 64, 128, 256])))
    c = smd.PlanModel()
    for k, x in v.items():
        setattr(c, k, x)
    return c, plan_ref.PlanModel(**v)


def test_planner_formula_bit_exact_vs_oracle():
    rng = np.random.default_rng(1)
    for _ in range(400):
        cm, pm = _model_pair(rng)
        args = (int(rng.integers(0, 300)), int(rng.choice([16, 32, 64, 128])), int(rng.integers(1, 9)),
                int(rng.integers(0, 200000)), int(rng.integers(0, 2)), int(rng.choice([0, 80, 256, 304])))
        two = bool(rng.integers(0, 2))
        got = smd.plan_decode(args[0], args[1], args[3], args[2], args[4], args[5], model=cm, two_source=two)
        want = plan_ref.plan_decode(*args, pm, two_source=two)
        assert got == want, (args, two, pm)
        if not two:
            assert smd.plan_num_kv_splits(args[0], args[1], args[3], args[2], args[4], args[5],
                                          model=cm) == want[0]


def test_default_model_fields_round_trip():
    """Every coefficient of the built-in model reaches the oracle's mirror."""
    pm = _library_model()
    assert pm.wide_rows == 128 and pm.wide_tile == 32 and pm.rows_per_wg == 16 and pm.long_cap == 128
    assert smd.plan_default_model().reserved == 0
    assert set(vars(pm)) == {name for name, _ in smd.PlanModel._fields_ if name != "reserved"}


def test_default_planner_properties():
    """Properties of every plan; the exact fitted choice is parity unpinned."""
    for rows in [1, 2, 8, 32, 64, 256]:
        for H in [16, 64, 128]:
            for K in [64, 384, 2176, 6528, 32128, 65664]:
                s, wide = smd.plan_decode(rows, H, K)
                assert s == smd.plan_num_kv_splits(rows, H, K)
                assert 1 <= s <= 256
                assert s <= -(-K // 64)    # never more splits than 64-row chunks
    # depends only on its arguments
    assert smd.plan_num_kv_splits(8, 64, 2176) == smd.plan_num_kv_splits(8, 64, 2176)
    # a batch that already fills the machine with one split per row stays unsplit
    assert smd.plan_num_kv_splits(1024, 128, 2048) == 1
    assert smd.plan_num_kv_splits(0, 128, 2048) == 1 and smd.plan_num_kv_splits(4, 128, 0) == 1


def test_planner_rejects_bad_args():
    with pytest.raises(smd.SmdError):
        smd.plan_num_kv_splits(-1, 16, 100)
    with pytest.raises(smd.SmdError):
        smd.plan_num_kv_splits(1, 16, 100, kv_dtype=7)


# ----------------------------------------------------------------------------
# host validation of the decode entry points (no launch happens on failure)
# ----------------------------------------------------------------------------
def _pool(**kw):
    p = smd._KVPool()
    p.dtype = kw.get("dtype", smd.KV_BF16)
    p.num_rows = kw.get("num_rows", 1024)
    p.nope = kw.get("nope", 0x10000)
    p.nope_stride = kw.get("nope_stride", 512)
    p.rope = kw.get("rope", 0x10000 + 896)
    p.rope_stride = kw.get("rope_stride", 512)
    p.scale = kw.get("scale", None)
    p.scale_stride = kw.get("scale_stride", 0)
    return p


def _decode(pool=None, **kw):
    a = dict(q_nope=0x20000, q_rope=0x30000, T=4, H=64, qps=1, idx=0x40000, idx_stride=100, topk=100, sink=None,
             scale=0.04, s=1, po=None, pl=None, out=0x50000, lse=0x60000)
    a.update(kw)
    p = pool if pool is not None else _pool()
    rc = smd.lib().smd_sparse_mla_decode(a["q_nope"], a["q_rope"], a["T"], a["H"], a["qps"], ctypes.byref(p),
                                         a["idx"], a["idx_stride"], a["topk"], a["sink"], a["scale"], a["s"],
                                         a["po"], a["pl"], a["out"], a["lse"], None)
    return rc, smd.lib().smd_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(H=17), -2, "num_heads"),
    (dict(H=256), -2, "num_heads"),
    (dict(qps=0), -2, "q_per_seq"),
    (dict(qps=9), -2, "q_per_seq"),
    (dict(T=3, qps=2), -1, "multiple"),
    (dict(s=0), -1, "num_splits"),
    (dict(s=257), -1, "num_splits"),
    (dict(T=-1), -1, "negative"),
    (dict(topk=-5), -1, "negative"),
    (dict(s=2), -3, "partial_o"),
    (dict(out=None), -3, "partial_o"),
    (dict(q_nope=None), -1, "required"),
    (dict(q_nope=0x20008), -1, "aligned"),
    (dict(idx_stride=50), -1, "indices_stride"),
    (dict(scale=float("inf")), -1, "softmax_scale"),
    (dict(out=0x50008), -1, "aligned"),
])
def test_decode_rejects(kw, code, msg):
    rc, err = _decode(**kw)
    assert rc == code and msg in err, (rc, err)


@pytest.mark.parametrize("pkw,code,msg", [
    (dict(dtype=5), -2, "dtype"),
    (dict(num_rows=-1), -1, "num_rows"),
    (dict(nope=None), -1, "NULL"),
    (dict(nope=0x10004), -1, "aligned"),
    (dict(nope_stride=100), -1, "stride"),
    (dict(rope_stride=60), -1, "stride"),
    (dict(nope_stride=452), -1, "multiples of 16"),
    (dict(scale=0x70000, scale_stride=8), -1, "scale"),
    (dict(dtype=1, nope_stride=448, rope_stride=64), -1, "scale"),
    (dict(dtype=1, nope_stride=448, rope_stride=64, scale=0x70000, scale_stride=7), -1, "scale"),
    (dict(dtype=1, nope_stride=448, rope_stride=64, scale=0x70001, scale_stride=8), -1, "scale"),
])
def test_decode_rejects_bad_pool(pkw, code, msg):
    rc, err = _decode(pool=_pool(**pkw))
    assert rc == code and msg in err, (rc, err)


def test_decode_null_pool():
    L = smd.lib()
    rc = L.smd_sparse_mla_decode(0x20000, 0x30000, 4, 64, 1, None, 0x40000, 100, 100, None, 0.04, 1, None, None,
                                 0x50000, 0x60000, None)
    assert rc == -1


def test_empty_problems_launch_nothing():
    # T == 0 and topk == 0 return OK before any HIP call (so this runs without a GPU)
    assert _decode(T=0)[0] == 0
    assert _decode(topk=0, idx=None)[0] == 0


@pytest.mark.parametrize("args,code", [
    ((0x1000, 0x2000, 4, 64, 0, None, 0x3000, 0x4000), -1),     # s = 0
    ((0x1000, 0x2000, 4, 64, 1025, None, 0x3000, 0x4000), -1),  # s too large
    ((None, 0x2000, 4, 64, 2, None, 0x3000, 0x4000), -1),       # no partials
    ((0x1000, 0x2000, 4, 64, 2, None, None, 0x4000), -1),       # no out
    ((0x1004, 0x2000, 4, 64, 2, None, 0x3000, 0x4000), -1),     # misaligned
    ((0x1000, 0x2000, -1, 64, 2, None, 0x3000, 0x4000), -1),    # negative tokens
])
def test_merge_rejects(args, code):
    assert smd.lib().smd_merge_partials(*args, None) == code


# ----------------------------------------------------------------------------
# persistent entry points: sizing, defaults and host validation
# ----------------------------------------------------------------------------
def _up256(x):
    return -(-x // 256) * 256


@pytest.mark.parametrize("H,qps,P", [(128, 4, 32), (16, 1, 256), (64, 2, 7), (32, 8, 1), (128, 1, 16384)])
def test_persistent_workspace_bytes(H, qps, P):
    # plan 16 B per partition, counters 4 B per (16-row group, partition), then
    # 2P slots of M rows x (512 bf16 + one fp32 lse); each region starts
    # 256-byte aligned
    M = H * qps
    want = _up256(16 * P) + _up256(4 * (M // 16) * P) + 2 * P * M * (512 * 2 + 4)
    assert smd.persistent_workspace_bytes(H, qps, P) == want


def test_persistent_default_partitions_vs_oracle():
    for H in (16, 32, 64, 128):
        for qps in range(1, 9):
            for cus in (0, 80, 256, 304):
                want = plan_ref.default_partitions(H, qps, num_cus=cus or 256)
                assert smd.persistent_default_partitions(H, qps, cus) == want


@pytest.mark.parametrize("args", [(17, 1, 4), (128, 0, 4), (128, 9, 4), (128, 1, 0), (128, 1, 16385)])
def test_persistent_workspace_bytes_rejects(args):
    with pytest.raises(smd.SmdError):
        smd.persistent_workspace_bytes(*args)


def _persist(pool=None, **kw):
    a = dict(q_nope=0x20000, q_rope=0x30000, B=4, qps=1, H=64, ptr=0x40000, flat=0x48000, sink=None, scale=0.04,
             ws=0x100000, ws_bytes=1 << 30, P=8, out=0x50000, lse=0x60000)
    a.update(kw)
    p = pool if pool is not None else _pool()
    rc = smd.lib().smd_sparse_mla_decode_persistent(a["q_nope"], a["q_rope"], a["B"], a["qps"], a["H"],
                                                    ctypes.byref(p), a["ptr"], a["flat"], a["sink"], a["scale"],
                                                    a["ws"], a["ws_bytes"], a["P"], a["out"], a["lse"], None)
    return rc, smd.lib().smd_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(B=-1), -1, "negative"),
    (dict(H=48), -2, "num_heads"),
    (dict(qps=9), -2, "q_per_seq"),
    (dict(P=0), -1, "num_partitions"),
    (dict(P=16385), -1, "num_partitions"),
    (dict(scale=float("nan")), -1, "softmax_scale"),
    (dict(ws=None), -3, "workspace"),
    (dict(ws=0x100010), -3, "256-byte"),
    (dict(ws_bytes=1000), -3, "below"),
    (dict(ptr=None), -1, "required"),
    (dict(flat=None), -1, "required"),
    (dict(out=None), -1, "required"),
    (dict(out=0x50008), -1, "aligned"),
    (dict(ptr=0x40002), -1, "4-byte"),
])
def test_persistent_rejects(kw, code, msg):
    rc, err = _persist(**kw)
    assert rc == code and msg in err, (rc, err)


def test_persistent_rejects_bad_pool():
    rc, err = _persist(pool=_pool(dtype=1, nope_stride=448, rope_stride=64))
    assert rc == -1 and "scale" in err


def test_persistent_empty_batch_launches_nothing():
    assert _persist(B=0)[0] == 0


def _persist_ex(opts, **kw):
    a = dict(q_nope=0x20000, q_rope=0x30000, B=4, qps=1, H=64, ptr=0x40000, flat=0x48000, sink=None, scale=0.04,
             ws=0x100000, ws_bytes=1 << 30, P=8, out=0x50000, lse=0x60000)
    a.update(kw)
    p = _pool()
    rc = smd.lib().smd_sparse_mla_decode_persistent_ex(a["q_nope"], a["q_rope"], a["B"], a["qps"], a["H"],
                                                       ctypes.byref(p), a["ptr"], a["flat"], a["sink"], a["scale"],
                                                       a["ws"], a["ws_bytes"], a["P"], a["out"], a["lse"],
                                                       ctypes.byref(opts) if opts is not None else None, None)
    return rc, smd.lib().smd_last_error().decode()


@pytest.mark.parametrize("opts,msg", [
    (smd._DecodeOptions(kernel=smd.KERNEL_WIDE), "SMD_KERNEL_AUTO"),
    (smd._DecodeOptions(merge=2), "merge"),
    (smd._DecodeOptions(merge=-1), "merge"),
    (smd._DecodeOptions(reserved=(ctypes.c_int32 * 5)(0, 0, 1, 0, 0)), "reserved"),
    (smd._DecodeOptions(qk=2), "qk"),
])
def test_persistent_ex_rejects_bad_options(opts, msg):
    rc, err = _persist_ex(opts)
    assert rc == -1 and msg in err, (rc, err)


@pytest.mark.parametrize("merge", [smd.MERGE_AUTO, smd.MERGE_WORKSPACE])
def test_persistent_ex_empty_batch_launches_nothing(merge):
    assert _persist_ex(smd._DecodeOptions(merge=merge), B=0)[0] == 0
    assert _persist_ex(None, B=0)[0] == 0


def test_split_kv_rejects_merge_option():
    """SMD_MERGE_* belongs to the persistent decode; the split-KV entry points
    take SMD_MERGE_AUTO only."""
    opts = smd._DecodeOptions(merge=smd.MERGE_WORKSPACE)
    p = _pool()
    rc = smd.lib().smd_sparse_mla_decode_ex(0x20000, 0x30000, 4, 64, 1, ctypes.byref(p), 0x40000, 100, 100, None,
                                            0.04, 1, None, None, 0x50000, 0x60000, ctypes.byref(opts), None)
    assert rc == -1 and "persistent" in smd.lib().smd_last_error().decode()


def _fp8_pool():
    return _pool(dtype=smd.KV_FP8_E4M3_UE8M0, nope_stride=448, rope=0x80000, rope_stride=64, scale=0x90000,
                 scale_stride=8)


def _split_ex(opts, pool, H=128, T=4):
    rc = smd.lib().smd_sparse_mla_decode_ex(0x20000, 0x30000, T, H, 1, ctypes.byref(pool), 0x40000, 100, 100, None,
                                            0.04, 1, None, None, 0x50000, 0x60000, ctypes.byref(opts), None)
    return rc, smd.lib().smd_last_error().decode()


@pytest.mark.parametrize("case,code", [
    ("unknown qk", -1),
    ("bf16 pool", -2),
    ("M = 64", -2),
    ("rows16 kernel", -2),
    ("pairs kernel", -2),
])
def test_split_kv_rejects_qk_fp8_where_it_does_not_run(case, code):
    """The fp8 QK runs on the wide kernel over one fp8 pool with M a multiple
    of 128; any other call that asks for it is rejected before a launch."""
    opts = smd._DecodeOptions(qk=smd.QK_FP8)
    pool, H = _fp8_pool(), 128
    if case == "unknown qk":
        opts = smd._DecodeOptions(qk=3)
    elif case == "bf16 pool":
        pool = _pool()
    elif case == "M = 64":
        H = 64
    elif case == "rows16 kernel":
        opts = smd._DecodeOptions(kernel=smd.KERNEL_ROWS16, qk=smd.QK_FP8)
    else:
        opts = smd._DecodeOptions(kernel=smd.KERNEL_PAIRS, qk=smd.QK_FP8)
    rc, err = _split_ex(opts, pool, H=H)
    assert rc == code and "qk" in err, (rc, err)


def test_two_source_rejects_qk_fp8():
    opts = smd._DecodeOptions(qk=smd.QK_FP8)
    p = _fp8_pool()
    rc = smd.lib().smd_sparse_mla_decode_two_source_ex(0x20000, 0x30000, 4, 128, 1, ctypes.byref(p), 0x40000, 100,
                                                       100, ctypes.byref(p), 0x48000, 128, 128, None, 0.04, 1, None,
                                                       None, 0x50000, 0x60000, ctypes.byref(opts), None)
    assert rc == -2 and "qk" in smd.lib().smd_last_error().decode()


@pytest.mark.parametrize("H,fp8", [(128, False), (64, True)])
def test_persistent_rejects_qk_fp8_where_it_does_not_run(H, fp8):
    a = dict(q_nope=0x20000, q_rope=0x30000, B=4, qps=1, ptr=0x40000, flat=0x48000, sink=None, scale=0.04,
             ws=0x100000, ws_bytes=1 << 30, P=8, out=0x50000, lse=0x60000)
    p = _fp8_pool() if fp8 else _pool()
    opts = smd._DecodeOptions(qk=smd.QK_FP8)
    rc = smd.lib().smd_sparse_mla_decode_persistent_ex(a["q_nope"], a["q_rope"], a["B"], a["qps"], H,
                                                       ctypes.byref(p), a["ptr"], a["flat"], a["sink"], a["scale"],
                                                       a["ws"], a["ws_bytes"], a["P"], a["out"], a["lse"],
                                                       ctypes.byref(opts), None)
    assert rc == -2 and "qk" in smd.lib().smd_last_error().decode()


def test_persistent_workspace_reset_rejects_null():
    assert smd.lib().smd_persistent_workspace_reset(None, 100, None) == -1


def test_library_default_model_is_the_fitted_one():
    """The built-in coefficients are those the oracle's worked examples use."""
    from tests.test_oracle_persistent import _fitted_model
    d = smd.plan_default_model()
    m = _fitted_model()
    for k in m.__dataclass_fields__:
        assert getattr(d, k) == getattr(m, k), k


def test_partials_bytes():
    """513 fp32 values (o and lse) per token, head and split."""
    assert smd.partials_bytes(8, 64, 4) == 8 * 64 * 4 * 513 * 4
    assert smd.partials_bytes(1, 128, 32) == 128 * 32 * 2052
    assert smd.partials_bytes(0, 16, 1) == 0
    assert smd.partials_bytes(2, 16, 0) == 0 and "num_splits" in smd.lib().smd_last_error().decode()
    # the merge's range: up to SMD_MAX_MERGE_SPLITS pieces
    assert smd.partials_bytes(2, 16, 33) == 2 * 16 * 33 * 2052
    assert smd.partials_bytes(1, 16, smd.MAX_MERGE_SPLITS) == 16 * smd.MAX_MERGE_SPLITS * 2052
    assert smd.partials_bytes(1, 16, smd.MAX_MERGE_SPLITS + 1) == 0


# ----------------------------------------------------------------------------
# host validation of the cache writer (no launch happens on failure)
# ----------------------------------------------------------------------------
def _fp8_pool(**kw):
    base = dict(dtype=smd.KV_FP8_E4M3_UE8M0, nope_stride=448, rope_stride=64, scale=0x70000, scale_stride=8)
    base.update(kw)
    return _pool(**base)


def _write(pool=None, kv=0x20000, kv_stride=512, n=4, slots=None):
    p = pool if pool is not None else _fp8_pool()
    rc = smd.lib().smd_write_kv_fp8(kv, kv_stride, n, slots, ctypes.byref(p), None)
    return rc, smd.lib().smd_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n=-1), -1, "negative num_rows"),
    (dict(kv=None), -1, "kv must be"),
    (dict(kv=0x20008), -1, "16-byte aligned"),
    (dict(kv_stride=511), -1, "stride"),
    (dict(kv_stride=516), -1, "multiple of 8"),
    (dict(slots=0x80002), -1, "slots must be 4-byte aligned"),
])
def test_writer_rejects(kw, code, msg):
    rc, err = _write(**kw)
    assert rc == code and msg in err, (rc, err)


@pytest.mark.parametrize("pkw,code,msg", [
    (dict(dtype=smd.KV_BF16, nope_stride=512, rope_stride=512, scale=None), -2, "must be fp8"),
    (dict(scale=None), -1, "scale"),
    (dict(nope_stride=440), -1, "below the row widths"),
    (dict(rope=0x10000 + 900), -1, "16-byte aligned"),
])
def test_writer_rejects_bad_pool(pkw, code, msg):
    rc, err = _write(pool=_fp8_pool(**pkw))
    assert rc == code and msg in err, (rc, err)


def test_writer_empty_launches_nothing():
    assert _write(n=0, kv=None)[0] == 0


# ----------------------------------------------------------------------------
# host validation of the two-source decode
# ----------------------------------------------------------------------------
def _two(main=None, swa=None, **kw):
    a = dict(q_nope=0x20000, q_rope=0x30000, T=4, H=64, qps=1, mi=0x40000, ms=100, km=100, si=0x48000, ss=128,
             ks=128, sink=None, scale=0.04, s=1, po=None, pl=None, out=0x50000, lse=0x60000)
    a.update(kw)
    mp = main if main is not None else _pool()
    sp = swa if swa is not None else _pool(nope=0x90000, rope=0x90000 + 896, num_rows=512)
    rc = smd.lib().smd_sparse_mla_decode_two_source(
        a["q_nope"], a["q_rope"], a["T"], a["H"], a["qps"], ctypes.byref(mp), a["mi"], a["ms"], a["km"],
        ctypes.byref(sp), a["si"], a["ss"], a["ks"], a["sink"], a["scale"], a["s"], a["po"], a["pl"], a["out"],
        a["lse"], None)
    return rc, smd.lib().smd_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(ks=-1), -1, "negative"),
    (dict(ss=-4), -1, "negative"),
    (dict(si=None), -1, "index lists are required"),
    (dict(mi=None), -1, "index lists are required"),
    (dict(ss=100), -1, "swa indices stride"),
    (dict(ms=50), -1, "indices_stride"),
    (dict(km=2 ** 31 - 100, ms=2 ** 31), -1, "exceed"),
    (dict(H=24), -2, "num_heads"),
    (dict(s=2), -3, "partial_o"),
])
def test_two_source_rejects(kw, code, msg):
    rc, err = _two(**kw)
    assert rc == code and msg in err, (rc, err)


@pytest.mark.parametrize("skw,code,msg", [
    (dict(dtype=smd.KV_FP8_E4M3_UE8M0, nope_stride=448, rope_stride=64, scale=0x70000, scale_stride=8), -2,
     "same dtype"),
    (dict(nope=0x90000, rope=0xA0000), -2, "RoPE placement"),        # split arrays against a packed main pool
    (dict(nope=0x90000, rope=0x90000 + 896, nope_stride=520, rope_stride=520), -2, "row strides"),
    (dict(nope=0x90008), -1, "16-byte aligned"),
])
def test_two_source_rejects_bad_swa_pool(skw, code, msg):
    rc, err = _two(swa=_pool(**skw))
    assert rc == code and msg in err, (rc, err)


def test_two_source_null_swa_pool():
    L = smd.lib()
    p = _pool()
    rc = L.smd_sparse_mla_decode_two_source(0x20000, 0x30000, 4, 64, 1, ctypes.byref(p), 0x40000, 100, 100, None,
                                            0x48000, 128, 128, None, 0.04, 1, None, None, 0x50000, 0x60000, None)
    assert rc == -1 and "NULL" in L.smd_last_error().decode()


def test_two_source_empty_launches_nothing():
    assert _two(km=0, ks=0, mi=None, si=None)[0] == 0
    assert _two(T=0)[0] == 0


def _library_model():
    c = smd.plan_default_model()
    return plan_ref.PlanModel(**{name: getattr(c, name) for name, _ in smd.PlanModel._fields_ if name != "reserved"})


@pytest.mark.parametrize("T,H,qps,s,K,kvd,two,req,want", [
    (64, 128, 1, 4, 65664, 1, False, None, "wide"),   # 256 wide workgroups of 514 tiles each
    (32, 128, 1, 1, 2176, 0, False, None, "rows16"),  # 32 wide workgroups: the narrow grid is cheaper
    (1, 128, 1, 31, 65664, 0, False, None, "rows16"),  # low batch, long list: narrow, 248 workgroups
    (4, 128, 1, 61, 65664, 0, False, None, "wide"),   # beyond the narrow cap of 32: a wide plan
    (4, 64, 1, 61, 65664, 0, False, None, "pairs"),   # M = 64 has no wide family: narrow at any s
    (256, 128, 4, 1, 4096, 1, False, None, "wide"),   # MTP4: M = 512, 64 rows x 4 groups
    (64, 128, 1, 1, 384, 0, False, None, "pairs"),    # short list: wide's fixed cost loses; pairs pay
    (32, 128, 1, 8, 65664, 1, True, None, "pairs"),   # two sources never take the wide kernel
    (8, 64, 1, 1, 2176, 0, False, None, "rows16"),    # M = 64: no wide; 16 pair workgroups do not pay
    (32, 128, 1, 1, 2176, 0, False, "rows16", "rows16"),
    (4, 64, 1, 1, 100, 0, False, "pairs", "pairs"),
    (1, 128, 1, 1, 64, 0, False, "wide", "wide"),
])
def test_decode_kernel_choice(T, H, qps, s, K, kvd, two, req, want):
    """smd_decode_kernel_choice applies the documented rule: wide when 128
    divides M, one source and the planner's model prices it below the narrow
    kernels at this s; else pairs when they pay; else rows16; a named family
    is returned as is when it fits."""
    assert smd.decode_kernel_choice(T, H, qps, s, K, kvd, two_source=two, kernel=req) == want


def test_decode_kernel_choice_follows_the_cost_model():
    """AUTO picks wide exactly where the oracle's cost formula, with the
    library's coefficients, prices the wide workgroups strictly below the
    narrow ones or the split count is beyond the narrow family's cap, and the
    planner's own family agrees at its chosen s."""
    pm = _library_model()
    rng = np.random.default_rng(5)
    for _ in range(300):
        rows = int(rng.integers(1, 200))
        H = int(rng.choice([16, 64, 128]))
        qps = int(rng.choice([1, 2, 4]))
        K = int(rng.integers(1, 70000))
        kvd = int(rng.integers(0, 2))
        s = int(rng.integers(1, 257))
        cw = plan_ref.wide_split_cost(s, rows, H, qps, K, kvd, 256, pm)
        narrow_cap = pm.short_cap if K < pm.long_kv else pm.long_cap
        wide = cw is not None and (s > narrow_cap or cw < plan_ref.split_cost(s, rows, H, qps, K, 256, pm))
        got = smd.decode_kernel_choice(rows * qps, H, qps, s, K, kvd)
        assert (got == "wide") == wide, (rows, H, qps, K, kvd, s)
        ps, pw = smd.plan_decode(rows, H, K, qps, kvd)
        assert (ps, pw) == plan_ref.plan_decode(rows, H, qps, K, kvd, 0, pm)
        assert (smd.decode_kernel_choice(rows * qps, H, qps, ps, K, kvd) == "wide") == pw


@pytest.mark.parametrize("args,code", [
    ((32, 64, 1, 1, 100, 0, 0, smd.KERNEL_WIDE), -2),   # M = 64 cannot take the wide kernel
    ((32, 128, 1, 1, 100, 0, 1, smd.KERNEL_WIDE), -2),  # nor two sources
    ((32, 16, 1, 1, 100, 0, 0, smd.KERNEL_PAIRS), -2),  # M = 16: no pairs
    ((4, 16, 1, 1, 100, 5, 0, 0), -2),                  # unknown kv dtype
    ((3, 16, 2, 1, 100, 0, 0, 0), -1),                  # tokens not a multiple of q_per_seq
    ((4, 16, 1, 0, 100, 0, 0, 0), -1),                  # no split
    ((4, 16, 1, 1, -1, 0, 0, 0), -1),                   # negative index count
    ((4, 16, 1, 1, 100, 0, 0, 9), -1),                  # unknown family
])
def test_decode_kernel_choice_rejects(args, code):
    assert smd.lib().smd_decode_kernel_choice(*args) == code


def _paged(**kw):
    a = dict(q=0x20000, B=2, mtp=4, Hq=16, k=0x30000, v=0x40000, nblk=100, page=16, Hkv=1, bt=0x50000, bts=64,
             cl=0x60000, max_ctx=1000, scale=0.04, s=1, po=None, pl=None, out=0x70000, lse=0x80000)
    a.update(kw)
    rc = smd.lib().smd_paged_decode(a["q"], a["B"], a["mtp"], a["Hq"], a["k"], a["v"], a["nblk"], a["page"], a["Hkv"],
                                    a["bt"], a["bts"], a["cl"], a["max_ctx"], a["scale"], a["s"], a["po"], a["pl"],
                                    a["out"], a["lse"], None)
    return rc, smd.lib().smd_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(Hq=8), -2, "64"),                       # GQA 8 x MTP 4 = 32 rows
    (dict(Hq=16, Hkv=3), -2, "64"),               # heads not a multiple of the KV heads
    (dict(page=24), -2, "page_size"),             # not a power of two
    (dict(page=8), -2, "page_size"),              # below 16
    (dict(s=0), -1, "num_splits"),
    (dict(s=257), -1, "num_splits"),
    (dict(bts=10), -1, "block_tables_stride"),    # 1000 positions need 63 pages
    (dict(max_ctx=1 << 20, bts=1 << 16), -1, "splits"),  # one split spanning 65536 pages
    (dict(scale=float("nan")), -1, "softmax_scale"),
    (dict(s=2), -1, "partials"),                  # a split plan without partials
    (dict(q=0x20008), -1, "aligned"),
    (dict(mtp=0), -1, "size"),
])
def test_paged_decode_rejects(kw, code, msg):
    rc, err = _paged(**kw)
    assert rc == code and msg in err, (rc, err)


def test_paged_decode_empty_launches_nothing():
    assert _paged(B=0)[0] == 0
    assert _paged(max_ctx=0)[0] == 0


def test_paged_num_splits():
    """Enough splits to cover 256 CUs once, capped at 32 and ceil(ctx / 64),
    raised until a split spans at most 4095 pages."""
    assert smd.paged_num_splits(16, 1, 8192, 16) == 16
    assert smd.paged_num_splits(64, 8, 32768, 16) == 1
    assert smd.paged_num_splits(1, 1, 100, 16) == 2        # ceil(100 / 64)
    assert smd.paged_num_splits(300, 1, 1 << 20, 16) == 17  # 1M / 16 pages needs >= 17 splits of <= 65520
    assert smd.paged_num_splits(2, 1, 0, 16) == 1
    with pytest.raises(smd.SmdError):
        smd.paged_num_splits(1, 1, 1 << 30, 16)

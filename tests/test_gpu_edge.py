"""GPU edge cases of the split-KV decode, through the C ABI:

* one-hot gather probe: q = 0 and pool row r = e_r, so the output recovers the
  exact multiset of gathered rows (and, per split, the split's multiset, which
  pins the split bounds) -- integer work, compared exactly;
* NaN-poisoned unreferenced rows, all-invalid and out-of-range entries;
* repeat-launch bit-exactness and HIP-graph replay of the split path;
* empty problems, the largest query-row count per index row (q_per_seq = 8),
  and the bf16 pool given as separate NoPE / RoPE arrays.
"""
import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import ref
from tests.helpers import bf16_tensor, check_lse, check_out, device_inputs, oracle_pool

pytestmark = pytest.mark.gpu

BF16_ONE = 0x3F80


def _one_hot_pool(n):
    kv = np.zeros((n, 512), dtype=np.uint16)
    kv[np.arange(n), np.arange(n)] = BF16_ONE
    return kv


@pytest.mark.parametrize("K,s", [(64, 1), (200, 3), (777, 4), (1500, 7)])
def test_one_hot_gather_probe(gpu, K, s):
    """Recovered counts per split equal the multiset of valid indices that
    smd_split_bounds assigns to that split."""
    n, T, H = 512, 3, 16
    rng = np.random.default_rng(K + s)
    idx = rng.integers(-40, n + 40, size=(T, K)).astype(np.int32)  # duplicates and invalid entries
    idx[1, ::7] = -1
    kv = _one_hot_pool(n)
    pool = smd.KVPool.bf16(bf16_tensor(kv, gpu))
    q_nope = torch.zeros((T, H, 448), dtype=torch.bfloat16, device=gpu)
    q_rope = torch.zeros((T, H, 64), dtype=torch.bfloat16, device=gpu)
    print(f"one-hot probe K={K} s={s}", flush=True)
    po, pl = smd.sparse_mla_decode(q_nope, q_rope, pool, torch.from_numpy(idx).to(gpu), None, 0.0442,
                                   num_splits=s, partials_only=True)
    torch.cuda.synchronize()
    po = po.cpu().numpy().astype(np.float64)
    pl = pl.cpu().numpy().astype(np.float64)
    for t in range(T):
        for r in range(s):
            a0, a1 = smd.split_bounds(K, s, r)
            seg = idx[t, a0:a1]
            seg = seg[(seg >= 0) & (seg < n)]
            want = np.bincount(seg, minlength=n).astype(np.float64)
            if seg.size == 0:
                assert np.all(po[t, :, r] == 0) and np.all(np.isneginf(pl[t, :, r]))
                continue
            # o_r[d] = count(d) / K_r and lse_r = ln K_r (all scores 0)
            kr = np.exp(pl[t, :, r])
            assert np.allclose(kr, seg.size, rtol=1e-5)
            got = np.rint(po[t, :, r, :n] * seg.size)
            assert np.array_equal(got, np.broadcast_to(want, got.shape)), (t, r)
            assert np.all(po[t, :, r, n:] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_nan_in_unreferenced_rows(gpu, dtype):
    """Rows that no index selects hold NaN; the output must not see them."""
    w = wl.dense_workload("nan pool", T=4, H=64, kv_dtype=dtype, pool_rows=2048, topk=333, invalid=7, seed=121)
    a = w.arrays
    used = np.unique(a["indices"][(a["indices"] >= 0) & (a["indices"] < 2048)])
    unused = np.setdiff1d(np.arange(2048), used)
    if dtype == "bf16":
        a["kv"][unused] = 0x7FC0  # bf16 NaN
    else:
        a["nope"][unused] = 0x7F  # e4m3fn NaN
        a["rope"][unused] = 0x7FC0
        a["scale"][unused] = 0xFF  # UE8M0 NaN
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(a["indices"]).to(gpu)
    o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"], a["sink"],
                                         w.softmax_scale)
    for s in (1, 3):
        print(f"nan pool {dtype} s={s}", flush=True)
        out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s)
        torch.cuda.synchronize()
        check_out(out, o_ref, f"{dtype} s={s}")
        check_lse(lse, l_ref, f"{dtype} s={s}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_all_invalid_and_out_of_range(gpu, dtype):
    w = wl.dense_workload("invalid rows", T=3, H=32, kv_dtype=dtype, pool_rows=1024, topk=130, invalid=0, seed=131)
    a = w.arrays
    a["indices"][0, :] = -1                      # every entry invalid
    a["indices"][1, ::3] = 1024                  # == N: out of range
    a["indices"][1, 1::5] = np.iinfo(np.int32).min
    a["indices"][2, :] = 5                       # one row, 130 times
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(a["indices"]).to(gpu)
    for use_sink in (True, False):
        o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"],
                                             a["sink"] if use_sink else None, w.softmax_scale)
        for s in (1, 2):
            print(f"invalid {dtype} sink={use_sink} s={s}", flush=True)
            out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink if use_sink else None, w.softmax_scale,
                                             num_splits=s)
            torch.cuda.synchronize()
            check_out(out, o_ref)
            check_lse(lse, l_ref)
            assert torch.all(out[0] == 0)
            if use_sink:  # ln(e^sink) (exact through the merge; one rounding in the exp2 domain at s=1)
                assert torch.allclose(lse[0].cpu(), sink.cpu(), rtol=1e-6, atol=1e-6)
            else:
                assert torch.all(torch.isneginf(lse[0]))


def test_repeat_launch_bit_exact(gpu):
    w = wl.config(1)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    ref_out = None
    for i in range(3):
        out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=4)
        torch.cuda.synchronize()
        if ref_out is None:
            ref_out, ref_lse = out.clone(), lse.clone()
        else:
            assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
            assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))


def test_graph_replay_split_path(gpu):
    """The planner + decode + merge step captured once and replayed several
    times, with eager work and synchronisation between replays; every replay
    equals the eager result."""
    w = wl.config(1)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    T, H = w.num_tokens, w.num_heads
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=gpu)
    lse = torch.empty((T, H), dtype=torch.float32, device=gpu)
    po = torch.empty((T, H, 4, 512), dtype=torch.float32, device=gpu)
    pl = torch.empty((T, H, 4), dtype=torch.float32, device=gpu)
    eager_out, eager_lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=4)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=4, out=out, lse=lse,
                              partial_o=po, partial_lse=pl)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        print(f"split-path graph replay {i}", flush=True)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16))
        assert torch.equal(lse, eager_lse)


def test_empty_problems_leave_outputs(gpu):
    w = wl.dense_workload("empty", T=2, H=16, kv_dtype="bf16", pool_rows=64, topk=8, seed=141)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    out = torch.full((2, 16, 512), 7.0, dtype=torch.bfloat16, device=gpu)
    lse = torch.full((2, 16), 7.0, dtype=torch.float32, device=gpu)
    idx0 = torch.empty((2, 0), dtype=torch.int32, device=gpu)
    smd.sparse_mla_decode(q_nope, q_rope, pool, idx0, sink, w.softmax_scale, num_splits=1, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


def test_largest_query_group(gpu):
    """q_per_seq = 8 with 128 heads: 1024 query rows share each index list."""
    w = wl.dense_workload("mtp8", T=16, H=128, kv_dtype="bf16", pool_rows=4096, topk=300, invalid=3, q_per_seq=8,
                          seed=151)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    o_ref, l_ref = ref.sparse_mla_decode(w.arrays["q_nope"], w.arrays["q_rope"], oracle_pool(w),
                                         w.arrays["indices"], w.arrays["sink"], w.softmax_scale, 8)
    for s in (1, 2):
        print(f"mtp8 s={s}", flush=True)
        out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s, q_per_seq=8)
        torch.cuda.synchronize()
        check_out(out, o_ref)
        check_lse(lse, l_ref)


def test_bf16_split_layout_pool(gpu):
    """A bf16 pool given as separate NoPE and RoPE arrays with padded strides."""
    w = wl.dense_workload("split layout", T=3, H=32, kv_dtype="bf16", pool_rows=3000, topk=410, invalid=4, seed=161)
    kv = w.arrays["kv"]
    nope = torch.zeros((3000, 512), dtype=torch.bfloat16, device=gpu)   # row stride 1024 B, 448 used
    rope = torch.zeros((3000, 72), dtype=torch.bfloat16, device=gpu)    # row stride 144 B, 64 used
    nope[:, :448] = bf16_tensor(np.ascontiguousarray(kv[:, :448]), gpu)
    rope[:, :64] = bf16_tensor(np.ascontiguousarray(kv[:, 448:]), gpu)
    pool = smd.KVPool(smd.KV_BF16, nope[:, :448], rope[:, :64])
    q_nope, q_rope, sink, _ = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    o_ref, l_ref = ref.sparse_mla_decode(w.arrays["q_nope"], w.arrays["q_rope"], oracle_pool(w),
                                         w.arrays["indices"], w.arrays["sink"], w.softmax_scale)
    for s in (1, 3):
        print(f"split layout s={s}", flush=True)
        out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s)
        torch.cuda.synchronize()
        check_out(out, o_ref)
        check_lse(lse, l_ref)

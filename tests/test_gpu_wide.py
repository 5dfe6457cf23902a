"""GPU parity of the wide split-KV decode kernel (128 query rows per workgroup
on 32x32 MFMAs), through the C ABI.

The library picks that kernel when the query rows per index row (heads x MTP
positions) are a multiple of 128 and its grid holds at least 128 workgroups;
the cases below name it explicitly (kernel="wide", the C ABI's
smd_decode_options) so that it runs on sizes the oracle finishes quickly.
The bars are those of every parity test: bf16 out atol = rtol = 2e-2, FP32
partials and LSE 1e-3, the one-hot gather probe exact, repeated launches and
graph replays bit-identical.
"""
import functools

import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import ref
from tests.helpers import bf16_tensor, check_lse, check_out, check_partials, device_inputs, oracle_pool

pytestmark = pytest.mark.gpu

# every call below names the wide kernel
_dec = functools.partial(smd.sparse_mla_decode, kernel="wide")


def _run(w, gpu, s, partials=False, sink=True):
    q_nope, q_rope, sk, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    a = w.arrays
    print(f"wide {w.name} s={s} partials={partials} sink={sink}", flush=True)
    if partials:
        po, pl = _dec(q_nope, q_rope, pool, idx, None, w.softmax_scale, num_splits=s, q_per_seq=w.q_per_seq,
                      partials_only=True)
        torch.cuda.synchronize()
        po_ref, pl_ref = ref.sparse_mla_decode_partials(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"],
                                                        w.softmax_scale, s, w.q_per_seq)
        check_partials(po, pl, po_ref, pl_ref)
        return
    out, lse = _dec(q_nope, q_rope, pool, idx, sk if sink else None, w.softmax_scale, num_splits=s,
                    q_per_seq=w.q_per_seq)
    torch.cuda.synchronize()
    o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"],
                                         a["sink"] if sink else None, w.softmax_scale, w.q_per_seq)
    check_out(out, o_ref)
    check_lse(lse, l_ref)


@pytest.mark.parametrize("H,qps,T,s", [(128, 1, 3, 1), (128, 1, 3, 3), (64, 2, 4, 2), (32, 4, 8, 1),
                                       (128, 2, 4, 2), (16, 8, 8, 4)])
def test_wide_bf16_ragged_tail(gpu, H, qps, T, s):
    """Lists of 687 positions (21 full tiles and a tail of 15), MTP rows
    sharing one list, more than one 128-row group per list (H=128, qps=2)."""
    w = wl.dense_workload("wide bf16", T=T, H=H, kv_dtype="bf16", pool_rows=4096, topk=650, swa=37, invalid=9,
                          q_per_seq=qps, seed=611 + H + qps + s)
    _run(w, gpu, s)


@pytest.mark.parametrize("H,qps,s", [(128, 1, 1), (128, 1, 2), (128, 1, 7), (64, 2, 3)])
def test_wide_fp8_ragged_tail(gpu, H, qps, s):
    w = wl.dense_workload("wide fp8", T=2 * qps, H=H, kv_dtype="fp8", pool_rows=4096, topk=700, invalid=4,
                          q_per_seq=qps, seed=631 + H + qps + s)
    _run(w, gpu, s)


@pytest.mark.parametrize("kv_dtype,s", [("bf16", 61), ("bf16", 128), ("fp8", 100), ("bf16", 256), ("fp8", 200)])
def test_wide_beyond_32_splits(gpu, kv_dtype, s):
    """The wide family's split counts above 32: 8250 positions cut into
    splits of 192 (s = 61: 43 non-empty, 18 empty), of 128 (s = 128: 65
    non-empty, 63 empty; s = 100: 65 and 35) and of 64 (s = 256: 129 and 127;
    s = 200: 129 and 71); bf16 out through the merge of up to 256 partials."""
    w = wl.dense_workload("wide many splits", T=2, H=128, kv_dtype=kv_dtype, pool_rows=16384, topk=8200, swa=50,
                          invalid=40, seed=671 + s)
    _run(w, gpu, s)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_wide_partials(gpu, kv_dtype):
    """FP32 partials (two-part P) and an empty trailing split (K=300, s=6)."""
    w = wl.dense_workload("wide partials", T=2, H=128, kv_dtype=kv_dtype, pool_rows=2048, topk=300, invalid=3,
                          seed=641)
    _run(w, gpu, 6, partials=True)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_wide_no_sink_and_invalid_rows(gpu, kv_dtype):
    """An all-invalid row (out = 0, lse = sink or -inf), out-of-range entries,
    one row repeated (duplicates are separate terms)."""
    w = wl.dense_workload("wide invalid", T=3, H=128, kv_dtype=kv_dtype, pool_rows=1024, topk=130, seed=661)
    a = w.arrays
    a["indices"][0, :] = -1
    a["indices"][1, ::3] = 1024
    a["indices"][2, :] = 5
    for sink in (True, False):
        _run(w, gpu, 2, sink=sink)


def test_wide_nan_in_unreferenced_rows(gpu):
    w = wl.dense_workload("wide nan pool", T=2, H=128, kv_dtype="fp8", pool_rows=2048, topk=333, invalid=7,
                          seed=671)
    a = w.arrays
    used = np.unique(a["indices"][(a["indices"] >= 0) & (a["indices"] < 2048)])
    unused = np.setdiff1d(np.arange(2048), used)
    a["nope"][unused] = 0x7F
    a["rope"][unused] = 0x7FC0
    a["scale"][unused] = 0xFF
    _run(w, gpu, 3)


def test_wide_split_layout_pool(gpu):
    """bf16 NoPE / RoPE in separate arrays with padded strides."""
    w = wl.dense_workload("wide split layout", T=2, H=128, kv_dtype="bf16", pool_rows=3000, topk=410, invalid=4,
                          seed=681)
    kv = w.arrays["kv"]
    nope = torch.zeros((3000, 512), dtype=torch.bfloat16, device=gpu)
    rope = torch.zeros((3000, 72), dtype=torch.bfloat16, device=gpu)
    nope[:, :448] = bf16_tensor(np.ascontiguousarray(kv[:, :448]), gpu)
    rope[:, :64] = bf16_tensor(np.ascontiguousarray(kv[:, 448:]), gpu)
    pool = smd.KVPool(smd.KV_BF16, nope[:, :448], rope[:, :64])
    q_nope, q_rope, sink, _ = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    o_ref, l_ref = ref.sparse_mla_decode(w.arrays["q_nope"], w.arrays["q_rope"], oracle_pool(w),
                                         w.arrays["indices"], w.arrays["sink"], w.softmax_scale)
    for s in (1, 3):
        print(f"wide split layout s={s}", flush=True)
        out, lse = _dec(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s)
        torch.cuda.synchronize()
        check_out(out, o_ref)
        check_lse(lse, l_ref)


@pytest.mark.parametrize("kv_dtype,K,s", [("bf16", 64, 1), ("bf16", 777, 4), ("fp8", 1500, 7)])
def test_wide_one_hot_gather_probe(gpu, kv_dtype, K, s):
    """q = 0 and pool row r = e_r: each split's partial recovers the exact
    multiset of its valid indices, in every one of the 128 query rows."""
    n, T, H = 512, 2, 128
    rng = np.random.default_rng(700 + K + s)
    idx = rng.integers(-40, n + 40, size=(T, K)).astype(np.int32)
    if kv_dtype == "bf16":
        kv = np.zeros((n, 512), dtype=np.uint16)
        kv[np.arange(n), np.arange(n)] = 0x3F80
        pool = smd.KVPool.bf16(bf16_tensor(kv, gpu))
    else:  # e4m3 1.0 = 0x38 with code 127 in NoPE dims; bf16 1.0 in RoPE dims
        nope = np.zeros((n, 448), dtype=np.uint8)
        rope = np.zeros((n, 64), dtype=np.uint16)
        r = np.arange(n)
        nope[r[r < 448], r[r < 448]] = 0x38
        rope[r[r >= 448], r[r >= 448] - 448] = 0x3F80
        codes = np.full((n, 8), 127, dtype=np.uint8)
        codes[:, 7] = 0
        pool = smd.KVPool.fp8(torch.from_numpy(nope).to(gpu), torch.from_numpy(codes).to(gpu),
                              bf16_tensor(rope, gpu))
    q_nope = torch.zeros((T, H, 448), dtype=torch.bfloat16, device=gpu)
    q_rope = torch.zeros((T, H, 64), dtype=torch.bfloat16, device=gpu)
    print(f"wide one-hot {kv_dtype} K={K} s={s}", flush=True)
    po, pl = _dec(q_nope, q_rope, pool, torch.from_numpy(idx).to(gpu), None, 0.0442, num_splits=s,
                  partials_only=True)
    torch.cuda.synchronize()
    po = po.cpu().numpy().astype(np.float64)
    pl = pl.cpu().numpy().astype(np.float64)
    for t in range(T):
        for r in range(s):
            a0, a1 = smd.split_bounds(K, s, r)
            seg = idx[t, a0:a1]
            seg = seg[(seg >= 0) & (seg < n)]
            if seg.size == 0:
                assert np.all(po[t, :, r] == 0) and np.all(np.isneginf(pl[t, :, r]))
                continue
            want = np.bincount(seg, minlength=n).astype(np.float64)
            assert np.allclose(np.exp(pl[t, :, r]), seg.size, rtol=1e-5)
            got = np.rint(po[t, :, r, :n] * seg.size)
            assert np.array_equal(got, np.broadcast_to(want, got.shape)), (t, r)


def test_wide_graph_replay(gpu):
    w = wl.dense_workload("wide graph", T=4, H=128, kv_dtype="bf16", pool_rows=4096, topk=900, invalid=5, seed=691)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    out = torch.empty((4, 128, 512), dtype=torch.bfloat16, device=gpu)
    lse = torch.empty((4, 128), dtype=torch.float32, device=gpu)
    po = torch.empty((4, 128, 3, 512), dtype=torch.float32, device=gpu)
    pl = torch.empty((4, 128, 3), dtype=torch.float32, device=gpu)
    eager_out, eager_lse = _dec(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=3)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        _dec(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=3, out=out, lse=lse, partial_o=po,
             partial_lse=pl)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        print(f"wide graph replay {i}", flush=True)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16))
        assert torch.equal(lse, eager_lse)


def test_wide_rejected_where_it_does_not_fit(gpu):
    """The wide family needs M % 128 == 0: a named wide call on M = 64 fails
    on the host (nothing launched), the library's choice still runs."""
    w = wl.dense_workload("wide misfit", T=2, H=64, kv_dtype="bf16", pool_rows=1024, topk=100, seed=695)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    with pytest.raises(smd.SmdError) as e:
        _dec(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=1)
    assert e.value.code == -2
    out, _ = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=1)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


@pytest.mark.slow
@pytest.mark.parametrize("s", [2, 8])
def test_wide_config3_full_size(gpu, s):
    """The fp8 workload of 32 tokens x 128 heads, 2048 indices (0.5% invalid)
    into a 131072-row pool, on the wide kernel at 2 and 8 splits: every
    output against the float64 oracle, and three launches bit-identical."""
    w = wl.config(2)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    runs = []
    for i in range(3):
        print(f"wide config 3 s={s} launch {i}", flush=True)
        runs.append(_dec(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s))
        torch.cuda.synchronize()
    for o, l in runs[1:]:
        assert torch.equal(o.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(l, runs[0][1])
    a = w.arrays
    o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"], a["sink"],
                                         w.softmax_scale)
    check_out(runs[0][0], o_ref)
    check_lse(runs[0][1], l_ref)

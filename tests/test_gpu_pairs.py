"""GPU parity of the dim-split (wave-pair) decode kernel, through the C ABI.

The library picks that kernel when the query rows per index row are a multiple
of 32 and its grid of 32-row blocks fills whole rounds of the GPU (the rule in
the header); the cases below name it explicitly (kernel="pairs", the C ABI's
smd_decode_options) so that it runs on sizes the oracle finishes quickly.  The same bars as the other parity tests:
bf16 out atol = rtol = 2e-2, FP32 partials and LSE 1e-3, the one-hot gather
probe exact.
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


# every call below names the dim-split kernel
_dec = functools.partial(smd.sparse_mla_decode, kernel="pairs")


def _run(w, gpu, s, partials=False, sink=True):
    q_nope, q_rope, sk, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    a = w.arrays
    print(f"pairs {w.name} s={s} partials={partials} sink={sink}", flush=True)
    if partials:
        po, pl = _dec(q_nope, q_rope, pool, idx, None, w.softmax_scale, num_splits=s,
                                       q_per_seq=w.q_per_seq, partials_only=True)
        torch.cuda.synchronize()
        po_ref, pl_ref = ref.sparse_mla_decode_partials(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"],
                                                        w.softmax_scale, s, w.q_per_seq)
        check_partials(po, pl, po_ref, pl_ref)
        return
    out, lse = _dec(q_nope, q_rope, pool, idx, sk if sink else None, w.softmax_scale,
                                     num_splits=s, q_per_seq=w.q_per_seq)
    torch.cuda.synchronize()
    o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"],
                                         a["sink"] if sink else None, w.softmax_scale, w.q_per_seq)
    check_out(out, o_ref)
    check_lse(lse, l_ref)


@pytest.mark.parametrize("H,s", [(32, 1), (32, 3), (64, 2), (128, 1), (128, 5)])
def test_pairs_bf16_ragged_tail(gpu, H, s):
    w = wl.dense_workload("pairs bf16", T=3, H=H, kv_dtype="bf16", pool_rows=4096, topk=650, swa=37, invalid=9,
                          seed=211 + H + s)
    _run(w, gpu, s)


@pytest.mark.parametrize("H,s", [(64, 1), (128, 2), (128, 7)])
def test_pairs_fp8_ragged_tail(gpu, H, s):
    w = wl.dense_workload("pairs fp8", T=2, H=H, kv_dtype="fp8", pool_rows=4096, topk=700, invalid=4,
                          seed=231 + H + s)
    _run(w, gpu, s)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_pairs_partials(gpu, kv_dtype):
    """FP32 partials (two-part P) and an empty trailing split (K=300, s=6)."""
    w = wl.dense_workload("pairs partials", T=2, H=64, kv_dtype=kv_dtype, pool_rows=2048, topk=300, invalid=3,
                          seed=241)
    _run(w, gpu, 6, partials=True)


@pytest.mark.parametrize("qps", [2, 4])
def test_pairs_mtp_shared_rows(gpu, qps):
    w = wl.dense_workload("pairs mtp", T=2 * qps, H=32, kv_dtype="bf16", pool_rows=2048, topk=300, invalid=3,
                          q_per_seq=qps, seed=251 + qps)
    _run(w, gpu, 2)


def test_pairs_no_sink_and_invalid_rows(gpu):
    w = wl.dense_workload("pairs invalid", T=3, H=32, kv_dtype="bf16", pool_rows=1024, topk=130, seed=261)
    a = w.arrays
    a["indices"][0, :] = -1
    a["indices"][1, ::3] = 1024
    a["indices"][2, :] = 5
    for sink in (True, False):
        _run(w, gpu, 2, sink=sink)


def test_pairs_nan_in_unreferenced_rows(gpu):
    w = wl.dense_workload("pairs nan pool", T=2, H=64, kv_dtype="fp8", pool_rows=2048, topk=333, invalid=7,
                          seed=271)
    a = w.arrays
    used = np.unique(a["indices"][(a["indices"] >= 0) & (a["indices"] < 2048)])
    unused = np.setdiff1d(np.arange(2048), used)
    a["nope"][unused] = 0x7F
    a["rope"][unused] = 0x7FC0
    a["scale"][unused] = 0xFF
    _run(w, gpu, 3)


def test_pairs_split_layout_pool(gpu):
    """bf16 NoPE / RoPE in separate arrays: the RoPE dims come from their own
    array in the upper dims half."""
    w = wl.dense_workload("pairs split layout", T=2, H=32, kv_dtype="bf16", pool_rows=3000, topk=410, invalid=4,
                          seed=281)
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
        print(f"pairs split layout s={s}", flush=True)
        out, lse = _dec(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s)
        torch.cuda.synchronize()
        check_out(out, o_ref)
        check_lse(lse, l_ref)


@pytest.mark.parametrize("K,s", [(64, 1), (777, 4), (1500, 7)])
def test_pairs_one_hot_gather_probe(gpu, K, s):
    """q = 0 and pool row r = e_r: each split's partial recovers the exact
    multiset of its valid indices (both dims halves: r < 256 and r >= 256)."""
    n, T, H = 512, 2, 32
    rng = np.random.default_rng(300 + K + s)
    idx = rng.integers(-40, n + 40, size=(T, K)).astype(np.int32)
    kv = np.zeros((n, 512), dtype=np.uint16)
    kv[np.arange(n), np.arange(n)] = 0x3F80
    pool = smd.KVPool.bf16(bf16_tensor(kv, gpu))
    q_nope = torch.zeros((T, H, 448), dtype=torch.bfloat16, device=gpu)
    q_rope = torch.zeros((T, H, 64), dtype=torch.bfloat16, device=gpu)
    print(f"pairs one-hot K={K} s={s}", flush=True)
    po, pl = _dec(q_nope, q_rope, pool, torch.from_numpy(idx).to(gpu), None, 0.0442,
                                   num_splits=s, partials_only=True)
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


def test_pairs_graph_replay(gpu):
    w = wl.dense_workload("pairs graph", T=4, H=64, kv_dtype="bf16", pool_rows=4096, topk=900, invalid=5, seed=291)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    out = torch.empty((4, 64, 512), dtype=torch.bfloat16, device=gpu)
    lse = torch.empty((4, 64), dtype=torch.float32, device=gpu)
    po = torch.empty((4, 64, 3, 512), dtype=torch.float32, device=gpu)
    pl = torch.empty((4, 64, 3), dtype=torch.float32, device=gpu)
    eager_out, eager_lse = _dec(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=3)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        _dec(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=3, out=out, lse=lse,
                              partial_o=po, partial_lse=pl)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        print(f"pairs graph replay {i}", flush=True)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16))
        assert torch.equal(lse, eager_lse)


@pytest.mark.slow
def test_pairs_selected_at_full_size(gpu):
    """With the library's choice: the fp8 workload of 32 tokens x 128 heads at 2 splits
    (32 x 2 x 4 = 256 blocks of 32 rows) runs the dim-split kernel -- its
    output is bit-identical to the forced dim-split run -- and meets the
    oracle."""
    w = wl.config(2)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    runs = {}
    for mode in (None, "1"):
        print(f"pairs full size mode={mode}", flush=True)
        dec = smd.sparse_mla_decode if mode is None else _dec
        runs[mode] = dec(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=2)
        torch.cuda.synchronize()
    assert torch.equal(runs[None][0].view(torch.int16), runs["1"][0].view(torch.int16))
    assert torch.equal(runs[None][1], runs["1"][1])
    a = w.arrays
    o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"], a["sink"],
                                         w.softmax_scale)
    check_out(runs[None][0], o_ref)
    check_lse(runs[None][1], l_ref)

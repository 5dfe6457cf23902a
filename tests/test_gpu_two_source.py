"""GPU parity of the two-source (main + sliding-window) decode against the
oracle, through the C ABI: bf16 and fp8 pools, segment boundaries inside a
half-tile and inside a split, every split count tried, both kernels (16-row
and dim-split), per-source validity, one empty source, the one-hot gather
probe, NaN in unreferenced rows, and the fp8 T=32 H=128 top-k 2048 + 128-row
window workload at full size.  Bars: bf16 out atol = rtol = 2e-2, FP32
partials and LSE 1e-3."""
import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import ref
from tests.helpers import bf16_tensor, check_lse, check_out, check_partials

pytestmark = pytest.mark.gpu


# the kernel family of the calls below (None: the library's choice); set by
# the `kernel` fixture for the tests that take it
_KERNEL = {"name": None}


@pytest.fixture(params=["auto", "pairs", "rows16"])
def kernel(request):
    _KERNEL["name"] = None if request.param == "auto" else request.param
    yield request.param
    _KERNEL["name"] = None


def _dev_pool(p: dict, gpu) -> smd.KVPool:
    if "kv" in p:
        return smd.KVPool.bf16(bf16_tensor(p["kv"], gpu))
    return smd.KVPool.fp8(torch.from_numpy(p["nope"]).to(gpu), torch.from_numpy(p["scale"]).to(gpu),
                          bf16_tensor(p["rope"], gpu))


def _inputs(w, gpu):
    a = w.arrays
    return (bf16_tensor(a["q_nope"], gpu), bf16_tensor(a["q_rope"], gpu), torch.from_numpy(a["sink"]).to(gpu),
            _dev_pool(a["main"], gpu), torch.from_numpy(a["main_indices"]).to(gpu), _dev_pool(a["swa"], gpu),
            torch.from_numpy(a["swa_indices"]).to(gpu))


def _check(w, gpu, s, partials=False, sink=True):
    a = w.arrays
    qn, qr, sk, mp, mi, sp, si = _inputs(w, gpu)
    print(f"two-source {w.name} s={s} partials={partials} sink={sink} "
          f"kernel={_KERNEL['name']}", flush=True)
    if partials:
        po, pl = smd.sparse_mla_decode_two_source(qn, qr, mp, mi, sp, si, None, w.softmax_scale, num_splits=s,
                                                  kernel=_KERNEL['name'],
                                                  q_per_seq=w.q_per_seq, partials_only=True)
        torch.cuda.synchronize()
        po_ref, pl_ref = ref.sparse_mla_decode_two_source_partials(
            a["q_nope"], a["q_rope"], a["main"], a["main_indices"], a["swa"], a["swa_indices"], w.softmax_scale,
            s, w.q_per_seq)
        check_partials(po, pl, po_ref, pl_ref)
        return
    out, lse = smd.sparse_mla_decode_two_source(qn, qr, mp, mi, sp, si, sk if sink else None, w.softmax_scale,
                                                kernel=_KERNEL['name'],
                                                num_splits=s, q_per_seq=w.q_per_seq)
    torch.cuda.synchronize()
    o_ref, l_ref = ref.sparse_mla_decode_two_source(a["q_nope"], a["q_rope"], a["main"], a["main_indices"],
                                                    a["swa"], a["swa_indices"], a["sink"] if sink else None,
                                                    w.softmax_scale, w.q_per_seq)
    check_out(out, o_ref)
    check_lse(lse, l_ref)


def _w(kv_dtype, T=3, H=64, topk=650, window=37, main_rows=4096, invalid=9, swa_invalid=5, qps=1, seed=0):
    return wl.two_source_workload(f"{kv_dtype} T={T} H={H} {topk}+{window}", T=T, H=H, kv_dtype=kv_dtype,
                                  main_rows=main_rows, topk=topk, window=window, invalid=invalid,
                                  swa_invalid=swa_invalid, q_per_seq=qps, seed=seed)


@pytest.mark.parametrize("s", [1, 2, 5, 11])
def test_two_source_bf16(gpu, kernel, s):
    _check(_w("bf16"), gpu, s)


@pytest.mark.parametrize("s", [1, 3])
def test_two_source_fp8(gpu, kernel, s):
    _check(_w("fp8", T=2, H=128, topk=700, window=128, main_rows=8192, seed=1), gpu, s)


@pytest.mark.parametrize("kv_dtype,s", [("bf16", 3), ("fp8", 4)])
def test_two_source_partials(gpu, kernel, kv_dtype, s):
    """The main/SWA boundary (position 650) falls inside split 1 for s = 3
    (chunk 256) and inside split 2 for s = 4 (chunk 192)."""
    _check(_w(kv_dtype, H=32, seed=2), gpu, s, partials=True)


def test_two_source_mtp_no_sink(gpu):
    _check(_w("bf16", T=4, H=16, topk=300, window=64, qps=2, seed=3), gpu, 2, sink=False)


@pytest.mark.parametrize("k_main,window", [(0, 100), (500, 0)])
def test_one_empty_source(gpu, k_main, window):
    w = _w("bf16", topk=k_main, window=window, invalid=0, swa_invalid=0, seed=4)
    _check(w, gpu, 1)
    _check(w, gpu, 2)


def test_per_source_validity(gpu):
    """The SWA pool is far smaller than the main pool: SWA entries that are
    valid main rows but not SWA rows contribute nothing, and main entries are
    checked against the main pool only."""
    w = _w("bf16", seed=5)
    a = w.arrays
    n_swa = a["swa"]["kv"].shape[0]
    a["swa_indices"][:, 1] = n_swa + 3          # a main row, not an SWA row
    a["swa_indices"][:, 2] = 2 ** 31 - 1
    a["main_indices"][:, 0] = n_swa - 1          # in range for both; it is a main row here
    a["main_indices"][:, 5] = w.pool_rows        # just past the main pool
    _check(w, gpu, 1)
    _check(w, gpu, 3)


def test_nan_in_unreferenced_rows(gpu):
    w = _w("bf16", seed=6)
    a = w.arrays
    used_m = set(a["main_indices"].ravel().tolist())
    used_s = set(a["swa_indices"].ravel().tolist())
    for pool, used in ((a["main"]["kv"], used_m), (a["swa"]["kv"], used_s)):
        free = [r for r in range(pool.shape[0]) if r not in used][:50]
        pool[free] = 0x7FC1  # NaN
    _check(w, gpu, 2)


def test_one_hot_gather_probe(gpu, kernel):
    """Main row r is e_r and SWA row r is e_(256 + r); with q = 0 the partial
    of a split is the mean of the rows it gathered, which shows exactly which
    rows of which pool each split read."""
    T, H, topk, window = 2, 32, 150, 70
    n_main, n_swa = 200, 180
    rng = np.random.default_rng(7)
    main = np.zeros((n_main, 512), dtype=np.uint16)
    main[np.arange(n_main), np.arange(n_main)] = 0x3F80
    swa = np.zeros((n_swa, 512), dtype=np.uint16)
    swa[np.arange(n_swa), 256 + np.arange(n_swa)] = 0x3F80
    mi = rng.integers(-2, n_main + 2, size=(T, topk)).astype(np.int32)
    si = rng.integers(-2, n_swa + 40, size=(T, window)).astype(np.int32)
    q0 = np.zeros((T, H, 448), dtype=np.uint16)
    r0 = np.zeros((T, H, 64), dtype=np.uint16)
    for s in (1, 2, 4):
        print(f"two-source one-hot s={s} kernel={_KERNEL['name']}", flush=True)
        po, pl = smd.sparse_mla_decode_two_source(
            bf16_tensor(q0, gpu), bf16_tensor(r0, gpu), smd.KVPool.bf16(bf16_tensor(main, gpu)),
            torch.from_numpy(mi).to(gpu), smd.KVPool.bf16(bf16_tensor(swa, gpu)), torch.from_numpy(si).to(gpu),
            None, 1.0, num_splits=s, partials_only=True, kernel=_KERNEL['name'])
        torch.cuda.synchronize()
        po_ref, pl_ref = ref.sparse_mla_decode_two_source_partials(q0, r0, {"kv": main}, mi, {"kv": swa}, si, 1.0, s)
        g = po.cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(g, po_ref, rtol=1e-6, atol=1e-7)
        check_lse(pl, pl_ref, "partial_lse")


def test_fullsize_fp8_top2048_window128(gpu):
    """The fp8 two-source workload at full size, in the launch the bench
    times (the planner's split count)."""
    w = wl.config(5)
    a = w.arrays
    qn, qr, sk, mp, mi, sp, si = _inputs(w, gpu)
    K = a["main_indices"].shape[1] + a["swa_indices"].shape[1]
    s = smd.plan_num_kv_splits(w.num_index_rows, w.num_heads, K, 1, smd.KV_FP8_E4M3_UE8M0, two_source=True)
    print(f"two-source full size s={s}", flush=True)
    out, lse = smd.sparse_mla_decode_two_source(qn, qr, mp, mi, sp, si, sk, w.softmax_scale, num_splits=s)
    torch.cuda.synchronize()
    o_ref, l_ref = ref.sparse_mla_decode_two_source(a["q_nope"], a["q_rope"], a["main"], a["main_indices"],
                                                    a["swa"], a["swa_indices"], a["sink"], w.softmax_scale)
    check_out(out, o_ref)
    check_lse(lse, l_ref)


def test_rejects_mismatched_pools(gpu):
    w = _w("bf16", seed=8)
    qn, qr, sk, mp, mi, sp, si = _inputs(w, gpu)
    nope = torch.zeros((64, 448), dtype=torch.uint8, device=gpu)
    fp8 = smd.KVPool.fp8(nope, torch.zeros((64, 8), dtype=torch.uint8, device=gpu),
                         torch.zeros((64, 64), dtype=torch.bfloat16, device=gpu))
    with pytest.raises(smd.SmdError):
        smd.sparse_mla_decode_two_source(qn, qr, mp, mi, fp8, si, sk, w.softmax_scale, num_splits=1)

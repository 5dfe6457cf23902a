"""GPU parity of the fp8 QK ("a8w8", options qk = SMD_QK_FP8), through the C ABI.

q_nope is quantised the way the cache writer quantises a latent row's NoPE
and the NoPE half of QK runs on the block-scaled fp8 MFMA straight from the
pool's bytes and codes; the oracle is the float64 decode with those quantised
queries (oracle.a8_ref), so the bars are the ordinary ones: bf16 out
atol = rtol = 2e-2, FP32 partials and LSE 1e-3, repeated launches
bit-identical.  Covered: the wide split-KV kernel (one split and several,
FP32 partials, MTP rows, ragged tails, invalid indices, no sink), the exact-
max redo, the persistent kernel on small ragged batches and on the ragged
MTP4 workload at full size (sampled sequences), and the calls the option
rejects.
"""
import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import a8_ref, ref
from tests.helpers import check_lse, check_out, check_partials, device_inputs, oracle_pool
from tests.test_gpu_persistent import SENTINEL, _check_plan, _filled, _ragged_inputs

pytestmark = pytest.mark.gpu


# The scaled fp8 MFMA does not sum its 64 products in full fp32: on gfx950 its
# result is off by up to 1.4e-4 of the block's largest |product| (an in-bounds
# probe against exact sums; the bf16 MFMA on the same products is within fp32
# rounding).  So the fp8 QK carries a score error of up to
# EPS8 * scale * sum_b max_{d in b} |q_d k_d| over the 7 NoPE blocks, which
# the float64 oracle does not have.  At the workloads' scale (1/sqrt(512)) it
# is ~1e-4; the redo test's scale of 3.0 makes it ~1e-2.  The FP32-partial
# bar adds twice that bound per row to its 1e-3 (a score error d moves each
# weight by a factor within e^(+-d) and the normaliser too), and the LSE bar
# adds it once.
EPS8 = 2.0 ** -12


def _score_error_bound(w, q64, t, rows):
    """Per head of token t: EPS8 * scale * max_j sum_b max_d |q_d k_jd| over the
    gathered rows j."""
    k = ref.pool_rows(oracle_pool(w), rows)[:, :448]                     # [n, 448]
    q = q64[t, :, :448]                                                  # [H, 448]
    prod = np.abs(q[:, None, :] * k[None, :, :]).reshape(q.shape[0], k.shape[0], 7, 64)
    return EPS8 * abs(w.softmax_scale) * prod.max(axis=3).sum(axis=2).max(axis=1)


def _check_partials_fp8(w, po, pl, po_ref, pl_ref):
    """FP32 partials and their LSE against the oracle's, with the fp8-QK score
    error bound added to the 1e-3 bars (see EPS8)."""
    a = w.arrays
    q64 = a8_ref.queries_a8(a["q_nope"], a["q_rope"])
    g = po.cpu().numpy().astype(np.float64)
    gl = pl.cpu().numpy().astype(np.float64)
    assert not np.isnan(g).any()
    for t in range(w.num_tokens):
        row = a["indices"][t // w.q_per_seq]
        rows = row[(row >= 0) & (row < w.pool_rows)]
        d = _score_error_bound(w, q64, t, rows)[:, None]                 # [H, 1]
        rowmax = np.abs(po_ref[t]).max(axis=-1)                          # [H, s]
        err = np.abs(g[t] - po_ref[t])
        tol = 1e-3 * np.abs(po_ref[t]) + ((1e-3 + 2 * d) * rowmax)[..., None]
        assert not (err > tol).any(), f"partial_o token {t}: {(err > tol).sum()} out of tolerance"
        lr = pl_ref[t]
        both = np.isneginf(gl[t]) & np.isneginf(lr)
        lerr = np.where(both, 0.0, np.abs(gl[t] - lr))
        ltol = 1e-3 * np.maximum(1.0, np.abs(np.where(np.isfinite(lr), lr, 0.0))) + d
        assert not (~(lerr <= ltol)).any(), f"partial_lse token {t} out of tolerance"


def _dense(w, gpu, s, partials=False, sink=True, repeats=1):
    q_nope, q_rope, sk, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    a = w.arrays
    print(f"qk fp8 {w.name} s={s} partials={partials} sink={sink}", flush=True)
    if partials:
        po, pl = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, None, w.softmax_scale, num_splits=s,
                                       q_per_seq=w.q_per_seq, partials_only=True, qk="fp8")
        torch.cuda.synchronize()
        po_ref, pl_ref = a8_ref.sparse_mla_decode_partials(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"],
                                                           w.softmax_scale, s, w.q_per_seq)
        if abs(w.softmax_scale) * 512 ** 0.5 <= 1.0:
            check_partials(po, pl, po_ref, pl_ref)  # the plain bars at the workloads' scale
        _check_partials_fp8(w, po, pl, po_ref, pl_ref)
        return
    first = None
    for rep in range(repeats):
        out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sk if sink else None, w.softmax_scale,
                                         num_splits=s, q_per_seq=w.q_per_seq, qk="fp8")
        torch.cuda.synchronize()
        if first is None:
            first = (out, lse)
            continue
        assert torch.equal(out.view(torch.int16), first[0].view(torch.int16)), f"launch {rep} differs (out)"
        assert torch.equal(lse, first[1]), f"launch {rep} differs (lse)"
    o_ref, l_ref = a8_ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"],
                                            a["sink"] if sink else None, w.softmax_scale, w.q_per_seq)
    check_out(first[0], o_ref)
    check_lse(first[1], l_ref)
    return first


@pytest.mark.parametrize("qps,T,s", [(1, 2, 1), (1, 3, 3), (1, 2, 7), (2, 4, 2), (4, 4, 1)])
def test_split_kv_ragged_tail(gpu, qps, T, s):
    """700 positions (21 full 32-row tiles and a tail of 28), 4 invalid, one
    or more splits, MTP rows sharing a list (M = 128, 256, 512)."""
    w = wl.dense_workload("qk fp8", T=T, H=128, kv_dtype="fp8", pool_rows=4096, topk=700, invalid=4,
                          q_per_seq=qps, seed=851 + qps + s)
    _dense(w, gpu, s)


def test_split_kv_partials_and_no_sink(gpu):
    """FP32 partials with an empty trailing split (K = 300, s = 6), and the
    output without a sink."""
    w = wl.dense_workload("qk fp8 partials", T=2, H=128, kv_dtype="fp8", pool_rows=2048, topk=300, invalid=3,
                          seed=861)
    _dense(w, gpu, 6, partials=True)
    _dense(w, gpu, 2, sink=False)


def test_split_kv_repeat_launches_bit_exact(gpu):
    w = wl.dense_workload("qk fp8 repeat", T=4, H=128, kv_dtype="fp8", pool_rows=8192, topk=2176, invalid=20,
                          seed=862)
    _dense(w, gpu, 4, repeats=10)


def test_close_to_the_exact_decode(gpu):
    """The quantisation moves the result by far less than the tolerance
    scale: against the exact (bf16 QK) oracle the fp8-QK output stays within
    0.05 everywhere on N(0,1) data (a sanity bound, not the parity bar)."""
    w = wl.dense_workload("qk fp8 vs exact", T=2, H=128, kv_dtype="fp8", pool_rows=4096, topk=1000, seed=863)
    out, _ = _dense(w, gpu, 2)
    a = w.arrays
    o_ex, _ = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"], a["sink"],
                                    w.softmax_scale)
    assert np.abs(out.float().cpu().numpy() - o_ex).max() < 0.05


def test_redo_path(gpu):
    """A softmax scale of 3.0 spreads the scores so widely that the exact-max
    redo runs; outputs and LSE meet the oracle at the plain bars, the FP32
    partials at the bars plus the fp8 MFMA's score error bound (EPS8)."""
    w = wl.dense_workload("qk fp8 redo", T=4, H=128, kv_dtype="fp8", pool_rows=4096, topk=900, invalid=7,
                          seed=864, softmax_scale=3.0)
    q = a8_ref.queries_a8(w.arrays["q_nope"][:1], w.arrays["q_rope"][:1])[0]
    row = w.arrays["indices"][0]
    k = ref.pool_rows(oracle_pool(w), row[row >= 0][:256])
    sc = 3.0 * (q @ k.T) * 1.4426950408889634
    assert np.any(sc[:, 16:].max(axis=1) - sc[:, :16].max(axis=1) > 32.0), "inputs do not force the redo"
    for s in (1, 3):
        _dense(w, gpu, s)
    _dense(w, gpu, 3, partials=True)


@pytest.mark.parametrize("qps,P", [(1, 7), (2, 5), (4, 64)])
def test_persistent_small(gpu, qps, P):
    """Ragged batches on the persistent kernel (split and unsplit sequences,
    K = 0 rows untouched, the plan bit-exact)."""
    w = wl.ragged_workload("qk fp8 persist", B=6, q_per_seq=qps, H=128, kv_dtype="fp8", pool_rows=3000, max_k=900,
                           zero_rows=1, seed=870 + qps + P)
    q_nope, q_rope, sink, pool, ptr, flat = _ragged_inputs(w, gpu)
    ws = smd.PersistentWorkspace(128, qps, P, device=gpu)
    out, lse = _filled(w, gpu)
    print(f"qk fp8 persistent qps={qps} P={P}", flush=True)
    smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink, w.softmax_scale, q_per_seq=qps,
                                     workspace=ws, out=out, lse=lse, qk="fp8")
    torch.cuda.synchronize()
    _check_plan(ws, w.arrays["kv_indptr"], P)
    _check_ragged(w, out, lse)


def _check_ragged(w, out, lse, seqs=None):
    a = w.arrays
    ptr = a["kv_indptr"]
    qps = w.q_per_seq
    o_gpu = out.float().cpu().numpy()
    l_gpu = lse.cpu().numpy()
    checked = 0
    for b in (range(len(ptr) - 1) if seqs is None else seqs):
        t0, t1 = b * qps, (b + 1) * qps
        if ptr[b + 1] == ptr[b]:
            assert np.all(o_gpu[t0:t1] == SENTINEL) and np.all(l_gpu[t0:t1] == SENTINEL), f"sequence {b} written"
            continue
        o_ref, l_ref, _ = a8_ref.sparse_mla_decode_ragged(a["q_nope"][t0:t1], a["q_rope"][t0:t1], oracle_pool(w),
                                                          np.array([0, ptr[b + 1] - ptr[b]]),
                                                          a["kv_indices"][ptr[b]:ptr[b + 1]], a["sink"],
                                                          w.softmax_scale, qps)
        check_out(out[t0:t1], o_ref, f"out of sequence {b}")
        check_lse(lse[t0:t1], l_ref, f"lse of sequence {b}")
        checked += 1
    return checked


@pytest.mark.slow
def test_persistent_config5_full_size(gpu):
    """The ragged MTP4 workload at full size with the fp8 QK, in the launch
    `bench.py --qk fp8` times: ten launches bit-identical, the workspace merge
    giving the same bits, the plan bit-exact, K = 0 rows untouched, and a
    sample of sequences (the longest, the shortest non-empty, and every
    eighth) against the oracle."""
    w = wl.config(4)
    a = w.arrays
    q_nope, q_rope, sink, pool, ptr, flat = _ragged_inputs(w, gpu)
    P = smd.persistent_default_partitions(128, 4)
    ws = smd.PersistentWorkspace(128, 4, P, device=gpu)
    first = None
    for rep in range(10):
        out, lse = _filled(w, gpu)
        print(f"qk fp8 config 5 full size launch {rep}", flush=True)
        smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink, w.softmax_scale, q_per_seq=4,
                                         workspace=ws, out=out, lse=lse, qk="fp8")
        torch.cuda.synchronize()
        if first is None:
            first = (out, lse)
            continue
        assert torch.equal(out.view(torch.int16), first[0].view(torch.int16)), f"launch {rep} differs (out)"
        assert torch.equal(lse, first[1]), f"launch {rep} differs (lse)"
    out, lse = _filled(w, gpu)
    smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink, w.softmax_scale, q_per_seq=4,
                                     workspace=ws, out=out, lse=lse, qk="fp8", merge="workspace")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), first[0].view(torch.int16)), "workspace merge differs (out)"
    out, lse = first
    _check_plan(ws, a["kv_indptr"], P)
    lens = np.diff(a["kv_indptr"])
    nz = np.flatnonzero(lens)
    sample = sorted({int(nz[np.argmax(lens[nz])]), int(nz[np.argmin(lens[nz])]), *range(0, len(lens), 8)})
    _check_ragged(w, out, lse, seqs=sample)
    zero = np.flatnonzero(lens == 0)
    o_gpu = out.float().cpu().numpy()
    for b in zero:
        assert np.all(o_gpu[4 * b:4 * b + 4] == SENTINEL), f"sequence {b} has K=0 but was written"

"""GPU parity of the split-KV decode and the merge against the float64 oracle.

Every case runs through the C ABI (Python binding -> libsmd.so) on seeded
inputs from `workloads` and compares element by element with `oracle.ref`.
"""
import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import ref
from tests.helpers import (check_lse, check_out, check_partials, device_inputs, oracle_pool)

pytestmark = pytest.mark.gpu


def run_case(w, gpu, num_splits, sink=True, partials=False):
    q_nope, q_rope, sink_t, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    sk = sink_t if sink else None
    print(f"case {w.name} s={num_splits} sink={sink} partials={partials}", flush=True)
    if partials:
        po, pl = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sk, w.softmax_scale,
                                       num_splits=num_splits, q_per_seq=w.q_per_seq, partials_only=True)
        torch.cuda.synchronize()
        po_ref, pl_ref = ref.sparse_mla_decode_partials(w.arrays["q_nope"], w.arrays["q_rope"], oracle_pool(w),
                                                        w.arrays["indices"], w.softmax_scale, num_splits,
                                                        w.q_per_seq)
        check_partials(po, pl, po_ref, pl_ref)
        return
    out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sk, w.softmax_scale,
                                     num_splits=num_splits, q_per_seq=w.q_per_seq)
    torch.cuda.synchronize()
    o_ref, l_ref = ref.sparse_mla_decode(w.arrays["q_nope"], w.arrays["q_rope"], oracle_pool(w),
                                         w.arrays["indices"], w.arrays["sink"] if sink else None,
                                         w.softmax_scale, w.q_per_seq)
    check_out(out, o_ref)
    check_lse(lse, l_ref)


@pytest.mark.parametrize("s", [1, 2, 3, 4, 7, 32])
def test_tiny_bf16(gpu, s):
    run_case(wl.config(0), gpu, s)


def test_tiny_bf16_no_sink(gpu):
    run_case(wl.config(0), gpu, 1, sink=False)


@pytest.mark.parametrize("H,s", [(16, 1), (32, 2), (64, 1), (64, 3), (128, 5)])
def test_bf16_ragged_tail(gpu, H, s):
    w = wl.dense_workload("bf16 ragged", T=3, H=H, kv_dtype="bf16", pool_rows=4096, topk=650, swa=37,
                          invalid=9, seed=11 + H + s)
    run_case(w, gpu, s)


@pytest.mark.parametrize("H,kv_dtype,s,partials", [(16, "bf16", 103, False), (16, "fp8", 128, False),
                                                    (32, "bf16", 64, False), (16, "bf16", 77, True)])
def test_narrow_beyond_32_splits(gpu, H, kv_dtype, s, partials):
    """The narrow kernels at the split counts the planner reaches for grids of
    few query rows (16 heads, one or two tokens): 8300 positions in splits of
    128 (s = 103, 128 and 77: 65 non-empty) or of 192 (s = 64: 44 non-empty),
    the empty ones included, through the merge or as FP32 partials."""
    w = wl.dense_workload("narrow many splits", T=2, H=H, kv_dtype=kv_dtype, pool_rows=16384, topk=8250, swa=50,
                          invalid=40, seed=21 + H + s)
    run_case(w, gpu, s, partials=partials)


@pytest.mark.parametrize("s", [1, 4])
def test_bf16_partials(gpu, s):
    w = wl.dense_workload("bf16 partials", T=2, H=64, kv_dtype="bf16", pool_rows=2048, topk=500, invalid=5,
                          seed=21 + s)
    run_case(w, gpu, s, partials=True)


@pytest.mark.parametrize("H,s", [(128, 1), (64, 3), (16, 2)])
def test_fp8_ragged_tail(gpu, H, s):
    w = wl.dense_workload("fp8 ragged", T=2, H=H, kv_dtype="fp8", pool_rows=4096, topk=700, invalid=4,
                          seed=31 + H + s)
    run_case(w, gpu, s)


def test_fp8_partials(gpu):
    w = wl.dense_workload("fp8 partials", T=2, H=128, kv_dtype="fp8", pool_rows=2048, topk=300, invalid=3,
                          seed=41)
    run_case(w, gpu, 3, partials=True)


@pytest.mark.parametrize("qps", [2, 4])
def test_mtp_shared_rows(gpu, qps):
    w = wl.dense_workload("mtp", T=2 * qps, H=32, kv_dtype="bf16", pool_rows=2048, topk=300, invalid=3,
                          q_per_seq=qps, seed=51 + qps)
    run_case(w, gpu, 2)


@pytest.mark.parametrize("S,topk,sink", [(6, 200, True), (13, 700, True), (13, 130, False), (32, 2100, True),
                                          (32, 130, False), (100, 4000, True), (300, 2000, False)])
def test_merge_kernel_alone(gpu, S, topk, sink):
    """smd_merge_partials on oracle-computed partials: one to sixteen waves
    per row, including splits that are all empty and a token with no valid
    index."""
    w = wl.dense_workload("merge", T=3, H=32, kv_dtype="bf16", pool_rows=4096, topk=topk, invalid=2, seed=61 + S)
    w.arrays["indices"][1, :] = -1
    po, pl = ref.sparse_mla_decode_partials(w.arrays["q_nope"], w.arrays["q_rope"], oracle_pool(w),
                                            w.arrays["indices"], w.softmax_scale, S)
    o_ref, l_ref = ref.merge_partials(po, pl, w.arrays["sink"] if sink else None)
    print(f"merge S={S} topk={topk} sink={sink}", flush=True)
    out, lse = smd.merge_partials(torch.from_numpy(po.astype(np.float32)).to(gpu),
                                  torch.from_numpy(pl.astype(np.float32)).to(gpu),
                                  torch.from_numpy(w.arrays["sink"]).to(gpu) if sink else None)
    torch.cuda.synchronize()
    check_out(out, o_ref)
    check_lse(lse, l_ref)
    if not sink:
        assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))

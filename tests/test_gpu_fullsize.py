"""GPU parity at the full sizes of the named workloads, in the launch
configuration bench.py times (the host planner's split count, decode + merge
into bf16), plus the extreme split counts.  Every output element is compared
with the float64 oracle."""
import functools

import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import ref
from tests.helpers import check_lse, check_out, check_partials, device_inputs, oracle_pool

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@functools.lru_cache(maxsize=2)
def _workload(i):
    return wl.config(i)


@functools.lru_cache(maxsize=2)
def _oracle(i):
    w = _workload(i)
    return ref.sparse_mla_decode(w.arrays["q_nope"], w.arrays["q_rope"], oracle_pool(w), w.arrays["indices"],
                                 w.arrays["sink"], w.softmax_scale, w.q_per_seq)


def _run(i, gpu, splits):
    w = _workload(i)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    K = idx.shape[1]
    kvd = smd.KV_BF16 if w.kv_dtype == "bf16" else smd.KV_FP8_E4M3_UE8M0
    s = smd.plan_num_kv_splits(w.num_index_rows, w.num_heads, K, w.q_per_seq, kvd) if splits == "planner" else splits
    print(f"full size {w.name} s={s}", flush=True)
    out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s,
                                     q_per_seq=w.q_per_seq)
    torch.cuda.synchronize()
    o_ref, l_ref = _oracle(i)
    check_out(out, o_ref, f"{w.name} s={s}")
    check_lse(lse, l_ref, f"{w.name} s={s}")


@pytest.mark.parametrize("i,splits", [(0, "planner"), (1, "planner"), (1, 1), (1, 4), (2, "planner"), (2, 1),
                                      (3, "planner"), (3, 32)])
def test_config_full_size(gpu, i, splits):
    _run(i, gpu, splits)


def test_long_context_partials_full_size(gpu):
    """The long-context workload's FP32 partials at 32 splits against the
    oracle's per-split partials (1e-3 relative)."""
    w = _workload(3)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    print("long-context partials s=32", flush=True)
    po, pl = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, None, w.softmax_scale, num_splits=32,
                                   partials_only=True)
    torch.cuda.synchronize()
    po_ref, pl_ref = ref.sparse_mla_decode_partials(w.arrays["q_nope"], w.arrays["q_rope"], oracle_pool(w),
                                                    w.arrays["indices"], w.softmax_scale, 32)
    check_partials(po, pl, po_ref, pl_ref)

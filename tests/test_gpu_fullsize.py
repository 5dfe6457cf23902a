"""GPU parity at the full sizes of the named workloads, in the launch
configuration bench.py times (the host planner's split count, decode + merge
into bf16), plus the extreme split counts and every kernel family.  Every
output element is compared with the float64 oracle, and repeated launches
must give bit-identical outputs (the aiter page "[FlyDSL] [Perf] pa_decode:
K/V streaming, MTP query split and sparse split-major on gfx950", PR
Self-Review: every changed case bit-exact over repeated launches)."""
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


def _run(i, gpu, splits, kernel=None, repeats=1):
    w = _workload(i)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    K = idx.shape[1]
    kvd = smd.KV_BF16 if w.kv_dtype == "bf16" else smd.KV_FP8_E4M3_UE8M0
    s = smd.plan_num_kv_splits(w.num_index_rows, w.num_heads, K, w.q_per_seq, kvd) if splits == "planner" else splits
    first = None
    for rep in range(repeats):
        print(f"full size {w.name} s={s} kernel={kernel} launch {rep}", flush=True)
        out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s,
                                         q_per_seq=w.q_per_seq, kernel=kernel)
        torch.cuda.synchronize()
        if first is None:
            first = (out, lse)
            continue
        assert torch.equal(out.view(torch.int16), first[0].view(torch.int16)), f"launch {rep} differs (out)"
        assert torch.equal(lse, first[1]), f"launch {rep} differs (lse)"
    o_ref, l_ref = _oracle(i)
    check_out(first[0], o_ref, f"{w.name} s={s}")
    check_lse(first[1], l_ref, f"{w.name} s={s}")


@pytest.mark.parametrize("i,splits", [(0, "planner"), (1, "planner"), (1, 1), (1, 4), (2, "planner"), (2, 1),
                                      (3, "planner"), (3, 32)])
def test_config_full_size(gpu, i, splits):
    _run(i, gpu, splits)


@pytest.mark.parametrize("i,splits,kernel", [(1, 4, "rows16"), (1, 2, "pairs"), (2, 1, "rows16"), (2, 2, "pairs"),
                                             (2, 8, "wide"), (3, 31, "rows16")])
def test_config_repeat_launches_bit_exact(gpu, i, splits, kernel):
    """Twenty launches of the same call give bit-identical out and lse, on
    each kernel family at the bf16 (T=8, H=64), fp8 (T=32, H=128) and
    long-context (T=1, 65664 indices) workloads; the first launch also meets
    the oracle."""
    _run(i, gpu, splits, kernel=kernel, repeats=20)


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


@pytest.mark.parametrize("T,ctx,var", [(64, 1048576, "fp8_h128"), (16, 102400, "bf16_h128"),
                                       (64, 32768, "bf16_h128")])
def test_matrix_cell_wide_plan_sampled(gpu, T, ctx, var):
    """T x ctx matrix cells where the host planner prices the wide kernel
    cheapest, in the launch `bench.py --matrix` times (the planner's split
    count, the library's kernel choice, decode + merge): the first, a middle
    and the last token, every head, against the oracle, and a second launch
    bit-identical to the first."""
    w = wl.matrix_cell(T, ctx, var)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    K = idx.shape[1]
    kvd = smd.KV_BF16 if w.kv_dtype == "bf16" else smd.KV_FP8_E4M3_UE8M0
    s, wide = smd.plan_decode(w.num_index_rows, w.num_heads, K, 1, kvd)
    assert wide and smd.decode_kernel_choice(T, w.num_heads, 1, s, K, kvd) == "wide"
    runs = []
    for rep in range(2):
        print(f"matrix cell {w.name} K={K} s={s} wide launch {rep}", flush=True)
        runs.append(smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s))
        torch.cuda.synchronize()
    out, lse = runs[0]
    assert torch.equal(out.view(torch.int16), runs[1][0].view(torch.int16))
    assert torch.equal(lse, runs[1][1])
    a = w.arrays
    for t in (0, T // 2, T - 1):
        o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"][t:t + 1], a["q_rope"][t:t + 1], oracle_pool(w),
                                             a["indices"][t:t + 1], a["sink"], w.softmax_scale)
        check_out(out[t:t + 1], o_ref, f"{w.name} token {t}")
        check_lse(lse[t:t + 1], l_ref, f"{w.name} token {t}")

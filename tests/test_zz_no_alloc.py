"""The allocation-free split-KV decode (smd_sparse_mla_decode_noalloc), through
the C ABI: its output must equal the usual entry point's (same kernels, same
partials, the merge reading them back) bit for bit and meet the oracle, on two
calls in a row -- the second with a smaller input, so the per-GPU scratch
array holds the first call's partials when the second begins -- and sizes
beyond the array are rejected on the host."""
import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import ref
from tests.helpers import check_lse, check_out, device_inputs, oracle_pool

pytestmark = pytest.mark.gpu


def _case(w, gpu, s, kernel):
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    T, H = w.num_tokens, w.num_heads
    out = torch.full((T, H, 512), 7.0, dtype=torch.bfloat16, device=gpu)
    lse = torch.full((T, H), 7.0, dtype=torch.float32, device=gpu)
    print(f"no-alloc {w.name} s={s} kernel={kernel}", flush=True)
    smd.sparse_mla_decode_noalloc(q_nope, q_rope, pool, idx, sink, w.softmax_scale, out=out, lse=lse, num_splits=s,
                                  q_per_seq=w.q_per_seq, kernel=kernel)
    ref_out, ref_lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s,
                                             q_per_seq=w.q_per_seq, kernel=kernel)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "out differs from smd_sparse_mla_decode"
    assert torch.equal(lse, ref_lse), "lse differs from smd_sparse_mla_decode"
    a = w.arrays
    o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"], a["sink"],
                                         w.softmax_scale, w.q_per_seq)
    check_out(out, o_ref)
    check_lse(lse, l_ref)


@pytest.mark.parametrize("kernel,H,kv_dtype", [("rows16", 64, "bf16"), ("pairs", 64, "fp8"), ("wide", 128, "fp8")])
def test_noalloc_matches_decode_twice(gpu, kernel, H, kv_dtype):
    big = wl.dense_workload("no-alloc big", T=8, H=H, kv_dtype=kv_dtype, pool_rows=4096, topk=1500, invalid=9,
                            seed=901)
    small = wl.dense_workload("no-alloc small", T=2, H=H, kv_dtype=kv_dtype, pool_rows=4096, topk=333, invalid=3,
                              seed=902)
    _case(big, gpu, 6, kernel)
    _case(small, gpu, 3, kernel)


def test_noalloc_rejects_oversize(gpu):
    """Partials beyond the scratch array: SMD_ERR_WORKSPACE, nothing written."""
    w = wl.dense_workload("no-alloc oversize", T=64, H=128, kv_dtype="bf16", pool_rows=1024, topk=64, seed=903)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    s = 8  # 64 x 128 x 8 x 2052 bytes > 32 MiB
    assert smd.partials_bytes(64, 128, s) > smd.NOALLOC_SCRATCH_BYTES
    out = torch.full((64, 128, 512), 7.0, dtype=torch.bfloat16, device=gpu)
    with pytest.raises(smd.SmdError) as e:
        smd.sparse_mla_decode_noalloc(q_nope, q_rope, pool, idx, sink, w.softmax_scale, out=out, num_splits=s)
    assert e.value.code == -3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all())
    # one split needs no scratch
    smd.sparse_mla_decode_noalloc(q_nope, q_rope, pool, idx, sink, w.softmax_scale, out=out, num_splits=1)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())

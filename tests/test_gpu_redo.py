"""GPU parity when scores spread far beyond each row's reference max.

Every kernel fixes a query row's reference max at its first valid tile (or
half-tile) and, when a later score exceeds that reference by more than 2^32,
redoes its range with the exact max found by a scores-only sweep.  A large
softmax scale (3.0 instead of 1/sqrt(512)) spreads the scores so widely that
the redo runs for nearly every row; the inputs are checked to have that
property.  Outputs, lse and FP32 partials are compared with the float64
oracle, on every kernel: the 16-row split-KV kernel, the dim-split pair kernel,
and the persistent kernel's 16-, 64- and 128-row groups.
"""

import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import ref
from tests.helpers import check_lse, check_out, check_partials, device_inputs, oracle_pool
from tests.test_gpu_persistent import SENTINEL, _check_against_oracle, _filled, _ragged_inputs

pytestmark = pytest.mark.gpu

SCALE = 3.0
LOG2E = 1.4426950408889634


def _assert_spread(w, idx_row, t=0):
    """Some head of token t has a score, beyond the list's first 16 entries,
    more than 32 (log2 units) above the best of those 16."""
    pool = oracle_pool(w)
    k = ref.pool_rows(pool, np.asarray(idx_row[:256]))
    q = ref.queries(w.arrays["q_nope"][t:t + 1], w.arrays["q_rope"][t:t + 1])[0]
    s = SCALE * (q @ k.T) * LOG2E
    assert np.any(s[:, 16:].max(axis=1) - s[:, :16].max(axis=1) > 32.0), "inputs do not force the redo"


@pytest.mark.parametrize("kv_dtype,H,kernel", [("bf16", 16, "rows16"), ("fp8", 64, "rows16"), ("fp8", 64, "pairs"),
                                               ("bf16", 128, "pairs"), ("bf16", 128, "wide"), ("fp8", 128, "wide")])
@pytest.mark.parametrize("s", [1, 3])
def test_split_kv_redo(gpu, kv_dtype, H, kernel, s):
    w = wl.dense_workload("redo split-kv", T=4, H=H, kv_dtype=kv_dtype, pool_rows=4096, topk=900, invalid=7,
                          seed=300 + H + s, softmax_scale=SCALE)
    _assert_spread(w, w.arrays["indices"][0][w.arrays["indices"][0] >= 0])
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    print(f"redo split-kv {kv_dtype} H={H} kernel={kernel} s={s}", flush=True)
    out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s, kernel=kernel)
    po, pl = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, None, w.softmax_scale, num_splits=s,
                                   partials_only=True, kernel=kernel)
    torch.cuda.synchronize()
    a = w.arrays
    o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"], a["sink"],
                                         w.softmax_scale)
    check_out(out, o_ref)
    check_lse(lse, l_ref)
    po_ref, pl_ref = ref.sparse_mla_decode_partials(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"],
                                                    w.softmax_scale, s)
    check_partials(po, pl, po_ref, pl_ref)


@pytest.mark.parametrize("H,qps,kv_dtype,P", [(16, 1, "fp8", 5), (64, 1, "bf16", 6), (128, 1, "fp8", 9),
                                              (128, 2, "bf16", 4)])
def test_persistent_redo(gpu, H, qps, kv_dtype, P):
    w = wl.ragged_workload("redo persistent", B=4, q_per_seq=qps, H=H, kv_dtype=kv_dtype, pool_rows=4096,
                           max_k=1000, zero_rows=1, seed=310 + H + qps, softmax_scale=SCALE)
    ptr = w.arrays["kv_indptr"]
    b = int(np.argmax(np.diff(ptr)))
    _assert_spread(w, w.arrays["kv_indices"][ptr[b]:ptr[b + 1]], t=b * qps)
    q_nope, q_rope, sink, pool, ptr_t, flat = _ragged_inputs(w, gpu)
    ws = smd.PersistentWorkspace(H, qps, P, device=gpu)
    out, lse = _filled(w, gpu)
    print(f"redo persistent H={H} qps={qps} {kv_dtype} P={P}", flush=True)
    smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr_t, flat, sink, w.softmax_scale, q_per_seq=qps,
                                     workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    assert _check_against_oracle(w, out, lse) > 0
    assert SENTINEL not in out.float()[torch.from_numpy(np.repeat(np.diff(ptr) > 0, qps)).to(gpu)]

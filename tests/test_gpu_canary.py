"""Guard zones around every buffer the library writes (the aiter page
"[ASM][HIP][MLA v4 nm] Split plan helper and persistent decode kernel", Test
plan: guard-page out-of-bounds checks).

Each output is a view into a larger allocation whose margins before and after
are filled with a sentinel; after the call (and its merge) the margins must
hold the sentinel bit for bit, and the outputs themselves must meet the
oracle.  Covered: out, lse and the FP32 partials of the split-KV decode on
every kernel family, partials-only calls, the stand-alone merge, the
two-source decode, the persistent decode's out, lse and workspace, and the
fp8 cache writer's pool arrays.
"""
import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import ref
from tests.helpers import bf16_tensor, check_lse, check_out, device_inputs, oracle_pool

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements of margin on each side (a multiple of 256 bytes for every dtype used)


def _fill(t: torch.Tensor, value: int):
    """Fill t with an integer bit pattern of its element width."""
    if t.dtype == torch.uint8:
        t.fill_(value)
    else:
        t.view(torch.int16 if t.element_size() == 2 else torch.int32).fill_(value)


class Guarded:
    """A contiguous view of `shape` inside an allocation with GUARD elements of
    a sentinel bit pattern on each side."""

    def __init__(self, shape, dtype, gpu, fill):
        self.n = int(np.prod(shape))
        self.base = torch.empty(self.n + 2 * GUARD, dtype=dtype, device=gpu)
        _fill(self.base, fill)
        self.view = self.base[GUARD:GUARD + self.n].view(*shape)
        margin = torch.empty(GUARD, dtype=dtype, device=gpu)
        _fill(margin, fill)
        self.margin = margin.view(torch.uint8)

    def check(self, what):
        torch.cuda.synchronize()
        raw = self.base.view(torch.uint8)
        es = self.base.element_size()
        assert torch.equal(raw[:GUARD * es], self.margin), f"{what}: bytes before the buffer were written"
        assert torch.equal(raw[(GUARD + self.n) * es:], self.margin), f"{what}: bytes after the buffer were written"


def guarded(shape, dtype, gpu, fill=-21555):
    """Default sentinel: 0xABCD per 16-bit element; pass an int32 NaN pattern
    (0x7FBADBAD) for fp32 buffers and a byte for uint8 ones."""
    return Guarded(shape, dtype, gpu, fill)


@pytest.mark.parametrize("kernel,H,kv_dtype", [("rows16", 64, "bf16"), ("pairs", 64, "fp8"), ("wide", 128, "bf16"),
                                               ("wide", 128, "fp8")])
@pytest.mark.parametrize("s", [1, 3])
def test_split_kv_outputs_guarded(gpu, kernel, H, kv_dtype, s):
    T = 3
    w = wl.dense_workload("canary", T=T, H=H, kv_dtype=kv_dtype, pool_rows=2048, topk=500, invalid=5, seed=800 + s)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    idx = torch.from_numpy(w.arrays["indices"]).to(gpu)
    out = guarded((T, H, 512), torch.bfloat16, gpu)
    lse = guarded((T, H), torch.float32, gpu, fill=0x7FBADBAD)
    po = guarded((T, H, s, 512), torch.float32, gpu, fill=0x7FBADBAD)
    pl = guarded((T, H, s), torch.float32, gpu, fill=0x7FBADBAD)
    print(f"canary split-kv {kernel} H={H} {kv_dtype} s={s}", flush=True)
    smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=s, out=out.view, lse=lse.view,
                          partial_o=po.view if s > 1 else None, partial_lse=pl.view if s > 1 else None, kernel=kernel)
    for g, name in ((out, "out"), (lse, "lse"), (po, "partial_o"), (pl, "partial_lse")):
        g.check(name)
    a = w.arrays
    o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], oracle_pool(w), a["indices"], a["sink"],
                                         w.softmax_scale)
    check_out(out.view, o_ref)
    check_lse(lse.view, l_ref)
    # partials only (FP32 partials are the result)
    po2 = guarded((T, H, s, 512), torch.float32, gpu, fill=0x7FBADBAD)
    pl2 = guarded((T, H, s), torch.float32, gpu, fill=0x7FBADBAD)
    smd.sparse_mla_decode(q_nope, q_rope, pool, idx, None, w.softmax_scale, num_splits=s, partial_o=po2.view,
                          partial_lse=pl2.view, partials_only=True, kernel=kernel)
    po2.check("partial_o (partials only)")
    pl2.check("partial_lse (partials only)")
    # the stand-alone merge of those partials
    out3 = guarded((T, H, 512), torch.bfloat16, gpu)
    lse3 = guarded((T, H), torch.float32, gpu, fill=0x7FBADBAD)
    smd.merge_partials(po2.view, pl2.view, sink, out=out3.view, lse=lse3.view)
    out3.check("merge out")
    lse3.check("merge lse")
    check_out(out3.view, o_ref, "merge out")


def test_two_source_outputs_guarded(gpu):
    T, H = 2, 64
    w = wl.two_source_workload("canary two-source", T=T, H=H, kv_dtype="fp8", main_rows=2048, topk=300, window=40,
                               invalid=3, swa_invalid=2, seed=820)
    a = w.arrays

    def dev_pool(p):
        return smd.KVPool.fp8(torch.from_numpy(p["nope"]).to(gpu), torch.from_numpy(p["scale"]).to(gpu),
                              bf16_tensor(p["rope"], gpu))

    out = guarded((T, H, 512), torch.bfloat16, gpu)
    lse = guarded((T, H), torch.float32, gpu, fill=0x7FBADBAD)
    po = guarded((T, H, 2, 512), torch.float32, gpu, fill=0x7FBADBAD)
    pl = guarded((T, H, 2), torch.float32, gpu, fill=0x7FBADBAD)
    print("canary two-source", flush=True)
    smd.sparse_mla_decode_two_source(bf16_tensor(a["q_nope"], gpu), bf16_tensor(a["q_rope"], gpu),
                                     dev_pool(a["main"]), torch.from_numpy(a["main_indices"]).to(gpu),
                                     dev_pool(a["swa"]), torch.from_numpy(a["swa_indices"]).to(gpu),
                                     torch.from_numpy(a["sink"]).to(gpu), w.softmax_scale, num_splits=2,
                                     out=out.view, lse=lse.view, partial_o=po.view, partial_lse=pl.view)
    for g, name in ((out, "out"), (lse, "lse"), (po, "partial_o"), (pl, "partial_lse")):
        g.check(name)
    o_ref, l_ref = ref.sparse_mla_decode_two_source(a["q_nope"], a["q_rope"], a["main"], a["main_indices"], a["swa"],
                                                    a["swa_indices"], a["sink"], w.softmax_scale)
    check_out(out.view, o_ref)
    check_lse(lse.view, l_ref)


@pytest.mark.parametrize("H,qps,kv_dtype,P", [(128, 4, "fp8", 16), (128, 1, "bf16", 7), (64, 1, "fp8", 5)])
def test_persistent_outputs_and_workspace_guarded(gpu, H, qps, kv_dtype, P):
    w = wl.ragged_workload("canary persistent", B=6, q_per_seq=qps, H=H, kv_dtype=kv_dtype, pool_rows=4096,
                           max_k=1500, zero_rows=1, seed=830 + H + qps)
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    ptr = torch.from_numpy(w.arrays["kv_indptr"]).to(gpu)
    flat = torch.from_numpy(w.arrays["kv_indices"]).to(gpu)
    T = w.num_tokens
    ws = smd.PersistentWorkspace(H, qps, P, device=gpu)
    # the same workspace inside a guarded allocation (256-byte aligned, zeroed once)
    gws = guarded((ws.nbytes,), torch.uint8, gpu, fill=0xA5)
    assert gws.view.data_ptr() % 256 == 0
    gws.view.zero_()
    ws.view = gws.view
    out = guarded((T, H, 512), torch.bfloat16, gpu)
    lse = guarded((T, H), torch.float32, gpu, fill=0x7FBADBAD)
    print(f"canary persistent H={H} qps={qps} {kv_dtype} P={P}", flush=True)
    for _ in range(2):  # a second call reuses the workspace (self-reset counters)
        smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink, w.softmax_scale, q_per_seq=qps,
                                         workspace=ws, out=out.view, lse=lse.view)
        gws.check("workspace")
        out.check("out")
        lse.check("lse")
    a = w.arrays
    p = a["kv_indptr"]
    o_ref, l_ref, _ = ref.sparse_mla_decode_ragged(a["q_nope"], a["q_rope"], oracle_pool(w), p, a["kv_indices"],
                                                   a["sink"], w.softmax_scale, qps)
    rows = np.repeat(np.diff(p) > 0, qps)
    check_out(out.view[torch.from_numpy(rows).to(gpu)], o_ref[rows])
    check_lse(lse.view[torch.from_numpy(rows).to(gpu)], l_ref[rows])


def test_writer_pool_guarded(gpu):
    rows, n_pool = 300, 1000
    wk = wl.writer_workload(rows, n_pool, seed=840)
    kv = torch.from_numpy(wk["kv"].view(np.int16)).to(gpu).view(torch.bfloat16)
    slots = torch.from_numpy(wk["slots"]).to(gpu)
    nope = guarded((n_pool, 448), torch.uint8, gpu, fill=0x5A)
    scale = guarded((n_pool, 8), torch.uint8, gpu, fill=0x5A)
    rope = guarded((n_pool, 64), torch.bfloat16, gpu)
    print("canary writer", flush=True)
    smd.write_kv_fp8(kv, smd.KVPool.fp8(nope.view, scale.view, rope.view), slots)
    nope.check("nope")
    scale.check("scale")
    rope.check("rope")

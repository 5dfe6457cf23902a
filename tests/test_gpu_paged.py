"""GPU parity of the dense paged GQA decode (smd_paged_decode) against the
float64 oracle (oracle.paged_ref), through the C ABI: ragged context lengths
(tails of every size, contexts shorter than the MTP span), GQA x MTP shapes
of 64 query rows per KV head, several KV heads, page sizes 16 to 128, one
split and several, FP32 partials, block-table entries that name no block,
repeated launches bit-identical, the
pa_decode page's BF16 D512 MTP4 GQA16 B16 ctx8K case at full size (sampled
tokens), and the calls the entry point rejects.  Bars: bf16 out
atol = rtol = 2e-2, FP32 partials and LSE 1e-3 (as for the sparse decode)."""
import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import paged_ref
from tests.helpers import bf16_tensor, check_lse, check_out, check_partials

pytestmark = pytest.mark.gpu


def _dev(w, gpu):
    return (bf16_tensor(w["q"], gpu), bf16_tensor(w["k"], gpu), bf16_tensor(w["v"], gpu),
            torch.from_numpy(w["block_tables"]).to(gpu), torch.from_numpy(w["context_lens"]).to(gpu))


def _run(w, gpu, s, partials=False, repeats=1):
    q, k, v, bt, cl = _dev(w, gpu)
    print(f"paged {w['name']} s={s} partials={partials}", flush=True)
    if partials:
        po, pl = smd.paged_decode(q, k, v, bt, cl, w["max_ctx"], w["softmax_scale"], mtp=w["mtp"], num_splits=s,
                                  partials_only=True)
        torch.cuda.synchronize()
        po_ref, pl_ref = paged_ref.paged_decode_partials(w["q"], w["k"], w["v"], w["block_tables"], w["context_lens"],
                                                         w["page"], w["mtp"], w["softmax_scale"], s, w["max_ctx"])
        check_partials(po, pl, po_ref, pl_ref)
        return
    first = None
    for rep in range(repeats):
        out, lse = smd.paged_decode(q, k, v, bt, cl, w["max_ctx"], w["softmax_scale"], mtp=w["mtp"], num_splits=s)
        torch.cuda.synchronize()
        if first is None:
            first = (out, lse)
            continue
        assert torch.equal(out.view(torch.int16), first[0].view(torch.int16)), f"launch {rep} differs"
        assert torch.equal(lse, first[1]), f"launch {rep} differs (lse)"
    o_ref, l_ref = paged_ref.paged_decode(w["q"], w["k"], w["v"], w["block_tables"], w["context_lens"], w["page"],
                                          w["mtp"], w["softmax_scale"])
    check_out(first[0], o_ref)
    check_lse(first[1], l_ref)


@pytest.mark.parametrize("Hq,Hkv,mtp", [(16, 1, 4), (32, 2, 4), (64, 1, 1), (128, 2, 1), (32, 1, 2)])
@pytest.mark.parametrize("s", [1, 3])
def test_shapes_and_ragged_contexts(gpu, Hq, Hkv, mtp, s):
    """Context lengths 300 (18 half-tiles and a tail of 12), 177, 16, 2 and 1
    (shorter than some MTP spans: those tokens see nothing)."""
    w = wl.paged_workload("paged", B=5, mtp=mtp, Hq=Hq, Hkv=Hkv, max_ctx=300, page=16, seed=900 + Hq + mtp + s,
                          lens=[300, 177, 16, 2, 1])
    _run(w, gpu, s)


@pytest.mark.parametrize("page", [32, 128])
def test_page_sizes(gpu, page):
    w = wl.paged_workload("paged pages", B=3, mtp=4, Hq=16, Hkv=1, max_ctx=777, page=page, seed=920 + page,
                          lens=[777, 640, 129])
    _run(w, gpu, 2)


def test_partials_with_empty_splits(gpu):
    """FP32 partials at s = 6 over contexts of 700 and 90: the second
    sequence's later splits are empty (o = 0, lse = -inf)."""
    w = wl.paged_workload("paged partials", B=2, mtp=4, Hq=16, Hkv=1, max_ctx=700, page=16, seed=931, lens=[700, 90])
    _run(w, gpu, 6, partials=True)


@pytest.mark.parametrize("s", [1, 4])
def test_invalid_block_entries_are_masked(gpu, s):
    """Block-table entries -1, num_blocks, num_blocks + 7 and INT32_MIN name no
    block: their pages are masked, including a page that holds the MTP
    tokens' limits and the last page of a ragged context."""
    w = wl.paged_workload("paged bad blocks", B=3, mtp=4, Hq=16, Hkv=1, max_ctx=400, page=16, seed=940 + s,
                          lens=[400, 250, 37])
    bt = w["block_tables"].copy()
    nblk = w["num_blocks"]
    bt[0, 3] = -1
    bt[0, 24] = nblk          # positions 384..399: the page of every MTP limit
    bt[1, 0] = nblk + 7
    bt[1, 15] = np.iinfo(np.int32).min  # positions 240..255, the ragged tail's page
    bt[2, 1] = -1
    w["block_tables"] = bt
    _run(w, gpu, s)


def test_graph_replays_match_eager(gpu):
    """A captured call (split plan: decode + merge, caller buffers, nothing
    allocated) replays bit-identically to the eager call, four times, with
    the outputs cleared between replays."""
    w = wl.paged_workload("paged graph", B=3, mtp=4, Hq=32, Hkv=2, max_ctx=900, page=32, seed=951,
                          lens=[900, 513, 40])
    q, k, v, bt, cl = _dev(w, gpu)
    T, Hq, s = w["B"] * w["mtp"], w["Hq"], 5
    eager_out, eager_lse = smd.paged_decode(q, k, v, bt, cl, w["max_ctx"], w["softmax_scale"], mtp=w["mtp"],
                                            num_splits=s)
    out = torch.empty((T, Hq, 512), dtype=torch.bfloat16, device=gpu)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=gpu)
    po = torch.empty((T, Hq, s, 512), dtype=torch.float32, device=gpu)
    pl = torch.empty((T, Hq, s), dtype=torch.float32, device=gpu)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        smd.paged_decode(q, k, v, bt, cl, w["max_ctx"], w["softmax_scale"], mtp=w["mtp"], num_splits=s, out=out,
                         lse=lse, partial_o=po, partial_lse=pl)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        print(f"paged graph replay {i}", flush=True)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16))
        assert torch.equal(lse, eager_lse)


def test_many_splits(gpu):
    """More splits than the heuristic picks (s = 40 over 2500 positions:
    splits of 64, the last ones empty), merged from bf16 scratch partials."""
    w = wl.paged_workload("paged many splits", B=2, mtp=4, Hq=16, Hkv=1, max_ctx=2500, page=16, seed=952,
                          lens=[2500, 1100])
    _run(w, gpu, 40)


def test_repeat_launches_bit_exact(gpu):
    w = wl.paged_workload("paged repeat", B=4, mtp=4, Hq=32, Hkv=2, max_ctx=1500, page=16, seed=932)
    _run(w, gpu, 4, repeats=10)


@pytest.mark.slow
def test_pa_decode_case_full_size(gpu):
    """The page's BF16 D512 MTP4 GQA16 B16 ctx8K case (one KV head, pages of
    16), in the launch bench.py --paged times (the library's split count):
    two launches bit-identical; tokens of the first, a middle and the last
    sequence against the oracle."""
    w = wl.paged_config()
    q, k, v, bt, cl = _dev(w, gpu)
    s = smd.paged_num_splits(w["B"], w["Hkv"], w["max_ctx"], w["page"])
    runs = []
    for rep in range(2):
        print(f"paged full size s={s} launch {rep}", flush=True)
        runs.append(smd.paged_decode(q, k, v, bt, cl, w["max_ctx"], w["softmax_scale"], mtp=w["mtp"], num_splits=s))
        torch.cuda.synchronize()
    out, lse = runs[0]
    assert torch.equal(out.view(torch.int16), runs[1][0].view(torch.int16))
    mtp = w["mtp"]
    for b in (0, w["B"] // 2, w["B"] - 1):
        sl = slice(b * mtp, (b + 1) * mtp)
        o_ref, l_ref = paged_ref.paged_decode(w["q"][sl], w["k"], w["v"], w["block_tables"][b:b + 1],
                                              w["context_lens"][b:b + 1], w["page"], mtp, w["softmax_scale"])
        check_out(out[sl], o_ref, f"sequence {b}")
        check_lse(lse[sl], l_ref, f"sequence {b}")

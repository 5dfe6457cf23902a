"""GPU parity of the persistent, graph-safe decode over ragged sequences.

Through the C ABI on seeded ragged workloads: outputs against the float64
oracle, rows of K_b = 0 sequences left untouched, the in-kernel plan (the
workspace plan region) bit-exact against the oracle's partition, workspace
reuse across batch sizes, offset kv_indptr, and graph replay with kv_indptr
and kv_indices changing between replays.
"""
import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import plan_ref, ref
from tests.helpers import bf16_tensor, check_lse, check_out, device_inputs, oracle_pool

pytestmark = pytest.mark.gpu

SENTINEL = 12288.0  # 1.5 * 2^13, exact in bf16; pre-fills out and lse to detect writes


def _ragged_inputs(w, gpu):
    q_nope, q_rope, sink, pool = device_inputs(w, gpu)
    ptr = torch.from_numpy(w.arrays["kv_indptr"]).to(gpu)
    flat = torch.from_numpy(w.arrays["kv_indices"]).to(gpu)
    return q_nope, q_rope, sink, pool, ptr, flat


def _filled(w, gpu):
    out = torch.full((w.num_tokens, w.num_heads, 512), SENTINEL, dtype=torch.bfloat16, device=gpu)
    lse = torch.full((w.num_tokens, w.num_heads), SENTINEL, dtype=torch.float32, device=gpu)
    return out, lse


def _check_against_oracle(w, out, lse, sink=True, seqs=None):
    a = w.arrays
    ptr = a["kv_indptr"]
    qps = w.q_per_seq
    B = len(ptr) - 1
    seqs = range(B) if seqs is None else seqs
    o_gpu = out.float().cpu().numpy()
    l_gpu = lse.cpu().numpy()
    checked = 0
    for b in seqs:
        t0, t1 = b * qps, (b + 1) * qps
        if ptr[b + 1] == ptr[b]:
            assert np.all(o_gpu[t0:t1] == SENTINEL) and np.all(l_gpu[t0:t1] == SENTINEL), \
                f"sequence {b} has K=0 but its rows were written"
            continue
        sub_ptr = np.array([0, ptr[b + 1] - ptr[b]])
        o_ref, l_ref, _ = ref.sparse_mla_decode_ragged(a["q_nope"][t0:t1], a["q_rope"][t0:t1], oracle_pool(w),
                                                       sub_ptr, a["kv_indices"][ptr[b]:ptr[b + 1]],
                                                       a["sink"] if sink else None, w.softmax_scale, qps)
        check_out(out[t0:t1], o_ref, f"out of sequence {b}")
        check_lse(lse[t0:t1], l_ref, f"lse of sequence {b}")
        checked += 1
    return checked


def _check_plan(ws, ptr_np, P):
    descs, _ = plan_ref.partition(ptr_np, P)
    got = ws.plan().cpu().numpy()
    assert got.tolist() == [list(d) for d in descs]


def run_persistent(w, gpu, P, sink=True):
    q_nope, q_rope, sink_t, pool, ptr, flat = _ragged_inputs(w, gpu)
    ws = smd.PersistentWorkspace(w.num_heads, w.q_per_seq, P, device=gpu)
    out, lse = _filled(w, gpu)
    print(f"persistent case {w.name} P={P} sink={sink}", flush=True)
    smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink_t if sink else None, w.softmax_scale,
                                     q_per_seq=w.q_per_seq, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    _check_plan(ws, w.arrays["kv_indptr"], P)
    _check_against_oracle(w, out, lse, sink)
    return ws


@pytest.mark.parametrize("P", [1, 3, 7, 64])
def test_fp8_mtp_small(gpu, P):
    w = wl.ragged_workload("persist fp8 mtp2", B=6, q_per_seq=2, H=16, kv_dtype="fp8", pool_rows=3000, max_k=700,
                           zero_rows=2, seed=70 + P)
    run_persistent(w, gpu, P)


@pytest.mark.parametrize("H,qps,P", [(16, 1, 6), (16, 3, 5), (16, 5, 9), (32, 3, 7), (16, 6, 4), (128, 3, 7)])
def test_row_groups_of_every_width(gpu, H, qps, P):
    """M = 16, 48, 80 (16-row groups), 96 (32-row groups), 96 via H=16 x 6,
    384 (three 128-row groups of wide waves): every row of every sequence is
    written."""
    w = wl.ragged_workload("persist row groups", B=5, q_per_seq=qps, H=H, kv_dtype="fp8", pool_rows=3000,
                           max_k=600, zero_rows=1, seed=70 + H + qps + P)
    run_persistent(w, gpu, P)


@pytest.mark.parametrize("H,qps,P", [(64, 1, 5), (128, 1, 16), (32, 1, 9), (16, 4, 11), (64, 4, 9)])
def test_bf16_shapes(gpu, H, qps, P):
    w = wl.ragged_workload("persist bf16", B=5, q_per_seq=qps, H=H, kv_dtype="bf16", pool_rows=4096, max_k=900,
                           zero_rows=1, indptr_offset=37, seed=80 + H + qps + P)
    run_persistent(w, gpu, P)


@pytest.mark.parametrize("P", [7, 300, 1500])
def test_many_sequences(gpu, P):
    """More sequences than a workgroup has threads, so the in-kernel plan scans
    kv_indptr in several chunks: 600 short lists (40 of them empty), from one
    partition holding many sequences to partitions holding only charged units."""
    w = wl.ragged_workload("persist many", B=600, q_per_seq=1, H=16, kv_dtype="bf16", pool_rows=4096, max_k=200,
                           zero_rows=40, indptr_offset=5, seed=120 + P)
    run_persistent(w, gpu, P)


def test_no_sink(gpu):
    w = wl.ragged_workload("persist no sink", B=4, q_per_seq=1, H=64, kv_dtype="fp8", pool_rows=2048, max_k=500,
                           zero_rows=1, seed=91)
    run_persistent(w, gpu, 6, sink=False)


@pytest.mark.parametrize("H,kv_dtype,P", [(128, "bf16", 64), (128, "bf16", 100), (16, "fp8", 130), (128, "fp8", 12),
                                          (128, "fp8", 40), (128, "fp8", 100)])
def test_long_sequence_many_pieces(gpu, H, kv_dtype, P):
    """One long sequence spread over every partition: a merge of up to 64
    pieces (at most one per lane) and of more than 64 (several per lane); on
    the fp8 wide path, up to 18 pieces (staged in LDS) and more."""
    w = wl.ragged_workload("persist long", B=1, q_per_seq=1, H=H, kv_dtype=kv_dtype, pool_rows=65536, max_k=1,
                           seed=92)
    K = 20000
    w.arrays["kv_indptr"] = np.array([0, K], dtype=np.int32)
    w.arrays["kv_indices"] = np.random.default_rng(2).choice(65536, K, replace=False).astype(np.int32)
    run_persistent(w, gpu, P)


@pytest.mark.parametrize("qps,kv_dtype,P,B", [(4, "fp8", 16, 12), (1, "bf16", 9, 8), (2, "fp8", 40, 30),
                                              (1, "fp8", 5, 1)])
def test_register_merge_matches_workspace_merge(gpu, qps, kv_dtype, P, B):
    """Wide row groups (H = 128): a split row group is merged either by the
    piece that finds every other piece arrived, straight from its registers,
    or from the workspace by the last to arrive; which one happens depends on
    timing, so both must give the same bits.  Five launches of each way agree
    bit for bit, and the outputs meet the oracle.  (B = 1, P = 5: one
    sequence in five pieces, most of them finishing together.)"""
    w = wl.ragged_workload("persist merge ways", B=B, q_per_seq=qps, H=128, kv_dtype=kv_dtype, pool_rows=8192,
                           max_k=3000, zero_rows=0, seed=140 + P + qps)
    if B == 1:
        K = 2500
        w.arrays["kv_indptr"] = np.array([0, K], dtype=np.int32)
        w.arrays["kv_indices"] = np.random.default_rng(5).choice(8192, K, replace=False).astype(np.int32)
    q_nope, q_rope, sink, pool, ptr, flat = _ragged_inputs(w, gpu)
    ws = smd.PersistentWorkspace(128, qps, P, device=gpu)
    first = None
    for merge in ("auto", "workspace"):
        for rep in range(5):
            out, lse = _filled(w, gpu)
            print(f"merge ways qps={qps} {kv_dtype} P={P} B={B} {merge} launch {rep}", flush=True)
            smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink, w.softmax_scale, q_per_seq=qps,
                                             workspace=ws, out=out, lse=lse, merge=merge)
            torch.cuda.synchronize()
            if first is None:
                first = (out, lse)
                continue
            assert torch.equal(out.view(torch.int16), first[0].view(torch.int16)), f"{merge} {rep} differs (out)"
            assert torch.equal(lse, first[1]), f"{merge} {rep} differs (lse)"
    _check_against_oracle(w, first[0], first[1])


def test_all_sequences_empty(gpu):
    w = wl.ragged_workload("persist empty", B=4, q_per_seq=2, H=16, kv_dtype="bf16", pool_rows=512, max_k=10,
                           zero_rows=4, seed=93)
    ws = run_persistent(w, gpu, 8)
    assert (ws.plan().cpu().numpy()[:, 2:] == -1).all()


@pytest.mark.parametrize("H,kv_dtype", [(32, "fp8"), (128, "fp8"), (128, "bf16")])
def test_invalid_entries_in_ragged_lists(gpu, H, kv_dtype):
    """Entries -1 and >= N inside the flat list are masked; an all-invalid
    sequence gives out = 0 and lse = sink.  H = 128 runs the wide waves (fp8:
    the direct-to-LDS ring, where masked rows read the zero row)."""
    w = wl.ragged_workload("persist invalid", B=5, q_per_seq=1, H=H, kv_dtype=kv_dtype, pool_rows=2048,
                           max_k=400, zero_rows=0, seed=94 + H)
    a = w.arrays
    ptr, flat = a["kv_indptr"], a["kv_indices"]
    rng = np.random.default_rng(0)
    for b in range(4):
        seg = np.arange(ptr[b], ptr[b + 1])
        if len(seg):
            bad = rng.choice(seg, size=max(1, len(seg) // 10), replace=False)
            flat[bad] = np.where(rng.random(len(bad)) < 0.5, -1, 2048 + 5)
    flat[ptr[4]:ptr[5]] = -1  # sequence 4: every entry invalid
    run_persistent(w, gpu, 7)


def test_matches_split_kv_path(gpu):
    """Equal-length sequences: the persistent kernel against the split-KV entry
    point on the same data (dense index rows)."""
    w = wl.ragged_workload("persist vs dense", B=4, q_per_seq=2, H=64, kv_dtype="fp8", pool_rows=4096, max_k=1,
                           seed=95)
    K = 777
    rng = np.random.default_rng(1)
    dense = np.stack([rng.choice(4096, K, replace=False) for _ in range(4)]).astype(np.int32)
    w.arrays["kv_indptr"] = (np.arange(5) * K).astype(np.int32)
    w.arrays["kv_indices"] = dense.reshape(-1).copy()
    q_nope, q_rope, sink, pool, ptr, flat = _ragged_inputs(w, gpu)
    ws = smd.PersistentWorkspace(64, 2, 10, device=gpu)
    out_p, lse_p = smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink, w.softmax_scale,
                                                    q_per_seq=2, workspace=ws)
    out_d, lse_d = smd.sparse_mla_decode(q_nope, q_rope, pool, torch.from_numpy(dense).to(gpu), sink,
                                         w.softmax_scale, num_splits=3, q_per_seq=2)
    torch.cuda.synchronize()
    a, b = out_p.float(), out_d.float()
    assert torch.all((a - b).abs() <= 2e-2 + 2e-2 * b.abs())
    assert torch.all((lse_p - lse_d).abs() <= 1e-3 * torch.clamp(lse_d.abs(), min=1.0))
    _check_against_oracle(w, out_p, lse_p)


def test_workspace_reuse_across_batch_sizes(gpu):
    """One workspace, no reset between calls: B = 12, then 3, then 12 again with
    other data; every call matches the oracle (the counters self-reset)."""
    ws = smd.PersistentWorkspace(128, 1, 20, device=gpu)
    for i, B in enumerate((12, 3, 12)):
        w = wl.ragged_workload(f"persist reuse B={B}", B=B, q_per_seq=1, H=128, kv_dtype="fp8", pool_rows=4096,
                               max_k=1500, zero_rows=1, seed=100 + i)
        q_nope, q_rope, sink, pool, ptr, flat = _ragged_inputs(w, gpu)
        out, lse = _filled(w, gpu)
        print(f"reuse call {i} B={B}", flush=True)
        smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink, w.softmax_scale, q_per_seq=1,
                                         workspace=ws, out=out, lse=lse)
        torch.cuda.synchronize()
        _check_plan(ws, w.arrays["kv_indptr"], 20)
        _check_against_oracle(w, out, lse)


def test_graph_replay_with_changing_lengths(gpu):
    """Capture one persistent call, then change kv_indptr / kv_indices in place
    between replays (eager work and synchronisation in between); each replay
    matches the oracle for the data it saw."""
    B, qps, H, cap = 8, 2, 64, 8 * 1200
    base = wl.ragged_workload("persist graph", B=B, q_per_seq=qps, H=H, kv_dtype="bf16", pool_rows=8192,
                              max_k=1200, zero_rows=2, seed=110)
    q_nope, q_rope, sink, pool, _, _ = _ragged_inputs(base, gpu)
    ptr_buf = torch.zeros(B + 1, dtype=torch.int32, device=gpu)
    flat_buf = torch.full((cap,), -1, dtype=torch.int32, device=gpu)
    ws = smd.PersistentWorkspace(H, qps, 24, device=gpu)
    out, lse = _filled(base, gpu)

    def load(seed):
        w = wl.ragged_workload("persist graph", B=B, q_per_seq=qps, H=H, kv_dtype="bf16", pool_rows=8192,
                               max_k=1200, zero_rows=2, seed=seed)
        # the same queries, pool and sink as `base` (same seed prefix is not
        # guaranteed), so take those arrays from base and only the lists from w
        for k in ("q_nope", "q_rope", "kv", "sink"):
            w.arrays[k] = base.arrays[k]
        n = int(w.arrays["kv_indptr"][-1])
        ptr_buf.copy_(torch.from_numpy(w.arrays["kv_indptr"]))
        flat_buf[:n].copy_(torch.from_numpy(w.arrays["kv_indices"]))
        return w

    w0 = load(110)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):  # warm-up outside capture
        smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr_buf, flat_buf, sink, base.softmax_scale,
                                         q_per_seq=qps, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr_buf, flat_buf, sink, base.softmax_scale,
                                         q_per_seq=qps, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()
    for i, seed in enumerate((110, 111, 112, 113)):
        w = w0 if i == 0 else load(seed)
        out.fill_(SENTINEL)
        lse.fill_(SENTINEL)
        torch.cuda.synchronize()
        print(f"graph replay {i} (lists of seed {seed})", flush=True)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        _check_plan(ws, w.arrays["kv_indptr"], 24)
        _check_against_oracle(w, out, lse)


@pytest.mark.slow
def test_config5_full_size(gpu):
    """The ragged MTP4 workload at full size (64 x 4 tokens, H=128, fp8 pool of
    262144 rows, K_b <= 8192, 4 empty sequences) with the default partition
    count, in the launch configuration bench.py times.  Every non-empty
    sequence is checked against the float64 oracle (split sequences and the
    longest and shortest lists among them), every K=0 row is checked
    untouched, the plan bit-exact, and twenty launches give bit-identical
    outputs (the fixed merge order of the split sequences makes them
    deterministic).  As an extra check every sequence also matches the
    split-KV path."""
    w = wl.config(4)
    a = w.arrays
    q_nope, q_rope, sink, pool, ptr, flat = _ragged_inputs(w, gpu)
    P = smd.persistent_default_partitions(128, 4)
    ws = smd.PersistentWorkspace(128, 4, P, device=gpu)
    first = None
    for rep in range(20):
        out, lse = _filled(w, gpu)
        print(f"config 5 full size P={P} launch {rep}", flush=True)
        smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink, w.softmax_scale, q_per_seq=4,
                                         workspace=ws, out=out, lse=lse)
        torch.cuda.synchronize()
        if first is None:
            first = (out, lse)
            continue
        assert torch.equal(out.view(torch.int16), first[0].view(torch.int16)), f"launch {rep} differs (out)"
        assert torch.equal(lse, first[1]), f"launch {rep} differs (lse)"
    for rep in range(3):  # every split row group merged from the workspace: the same bits
        out, lse = _filled(w, gpu)
        print(f"config 5 full size P={P} workspace merge launch {rep}", flush=True)
        smd.sparse_mla_decode_persistent(q_nope, q_rope, pool, ptr, flat, sink, w.softmax_scale, q_per_seq=4,
                                         workspace=ws, out=out, lse=lse, merge="workspace")
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), first[0].view(torch.int16)), f"workspace merge {rep} differs (out)"
        assert torch.equal(lse, first[1]), f"workspace merge {rep} differs (lse)"
    out, lse = first
    _check_plan(ws, a["kv_indptr"], P)
    ptr_np = a["kv_indptr"]
    B = len(ptr_np) - 1
    _, pieces = plan_ref.partition(ptr_np, P)
    split = {x.seq for pl in pieces for x in pl if x.split}
    lens = np.diff(ptr_np)
    assert len(split) > 10, "the workload should split many sequences"
    checked = _check_against_oracle(w, out, lse)  # every sequence; K=0 rows must be untouched
    assert checked == int(np.count_nonzero(lens))
    # extra check: every sequence against the split-KV entry point
    o_all, l_all = out.float(), lse
    for b in range(B):
        if lens[b] == 0:
            continue
        t0, t1 = 4 * b, 4 * b + 4
        idx = flat[ptr_np[b]:ptr_np[b + 1]].view(1, -1)
        od, ld = smd.sparse_mla_decode(q_nope[t0:t1].contiguous(), q_rope[t0:t1].contiguous(), pool, idx, sink,
                                       w.softmax_scale, num_splits=1, q_per_seq=4)
        torch.cuda.synchronize()
        assert torch.all((o_all[t0:t1] - od.float()).abs() <= 2e-2 + 2e-2 * od.float().abs()), f"sequence {b}"
        assert torch.all((l_all[t0:t1] - ld).abs() <= 1e-3 * torch.clamp(ld.abs(), min=1.0)), f"sequence {b}"

"""Pins of the float64 oracle against facts that do not come from the oracle:
brute force, a library softmax, closed forms, the format definitions of bf16 /
E4M3FN / UE8M0 (cross-checked with torch's own conversions), the split-merge
identity and invariances the definition implies.  CPU only."""
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import ref

GOLDEN = Path(__file__).parent / "golden"


# ----------------------------------------------------------------------------
# element formats
# ----------------------------------------------------------------------------
def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = ref.e4m3fn_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(mine[ok], lib[ok])
    # spot values of the OCP format: 0x7E = 448 (max), 0x01 = 2^-9 (min subnormal), 0x38 = 1.0
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x38] == 1.0 and mine[0xB8] == -1.0


def test_ue8m0_closed_form():
    c = np.arange(256, dtype=np.uint8)
    v = ref.ue8m0_to_f64(c)
    assert np.isnan(v[255])
    assert v[127] == 1.0 and v[128] == 2.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    assert np.all(v[1:255] / v[:254] == 2.0)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    mine = ref.bf16_to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(mine[ok], lib[ok])


def test_fp8_row_decode_against_torch_scaling():
    w = wl.dense_workload("fp8 rows", T=1, H=16, kv_dtype="fp8", pool_rows=64, topk=8, seed=5)
    a = w.arrays
    rows = np.arange(64)
    mine = ref.pool_rows({"nope": a["nope"], "scale": a["scale"], "rope": a["rope"]}, rows)
    x = torch.from_numpy(a["nope"]).view(torch.float8_e4m3fn).to(torch.float64)
    e = torch.from_numpy(a["scale"][:, :7].astype(np.int64) - 127)
    x = torch.ldexp(x, e.repeat_interleave(64, dim=1))
    r = torch.from_numpy(a["rope"].view(np.int16)).view(torch.bfloat16).to(torch.float64)
    lib = torch.cat([x, r], dim=1).numpy()
    assert np.array_equal(mine, lib)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10000) * np.exp(rng.uniform(-20, 20, 10000))
    mine = ref.round_bf16(x)
    lib = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, lib)


# ----------------------------------------------------------------------------
# the decode against independent formulations
# ----------------------------------------------------------------------------
def _brute_dense(q, pool_f64, idx, n, scale, sink):
    """Dense attention over every pool row r with weight c_r * e^{s_r}, where c_r
    counts the valid occurrences of r in the index list (multiset semantics)."""
    counts = np.zeros(n)
    for i in idx:
        if 0 <= i < n:
            counts[i] += 1
    s = float(np.float32(scale)) * (q @ pool_f64.T)          # [M, n]
    out = np.zeros((q.shape[0], pool_f64.shape[1]))
    lse = np.zeros(q.shape[0])
    for m in range(q.shape[0]):
        terms = [(counts[r], s[m, r]) for r in range(n) if counts[r] > 0]
        z = sum(c * math.exp(v) for c, v in terms)
        if sink is not None:
            z += math.exp(sink[m])
        if not terms:
            out[m] = 0.0
            lse[m] = -math.inf if sink is None else sink[m]
            continue
        for r in range(n):
            if counts[r] > 0:
                out[m] += counts[r] * math.exp(s[m, r]) / z * pool_f64[r]
        lse[m] = math.log(z)
    return out, lse


@pytest.mark.parametrize("with_sink", [True, False])
def test_decode_matches_brute_force_dense(with_sink):
    w = wl.dense_workload("brute", T=2, H=16, kv_dtype="bf16", pool_rows=512, topk=64, invalid=8, seed=7)
    a = w.arrays
    idx = a["indices"].copy()
    idx[0, 5] = idx[0, 6]            # a duplicate
    idx[1, 3] = 512                  # out of range -> invalid
    idx[1, 4] = -5                   # negative -> invalid
    out, lse = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], {"kv": a["kv"]}, idx,
                                     a["sink"] if with_sink else None, w.softmax_scale)
    pool = ref.bf16_to_f64(a["kv"])
    q = ref.queries(a["q_nope"], a["q_rope"])
    for t in range(2):
        sk = a["sink"].astype(np.float64) if with_sink else None
        o2, l2 = _brute_dense(q[t], pool, idx[t], 512, w.softmax_scale, sk)
        np.testing.assert_allclose(out[t], o2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[t], l2, rtol=1e-12, atol=1e-12)


def test_decode_matches_torch_softmax():
    """Unique valid indices: torch SDPA (float64) without a sink, and a softmax
    over [scores, sink] with the sink column dropped afterwards."""
    w = wl.dense_workload("sdpa", T=3, H=32, kv_dtype="bf16", pool_rows=300, topk=100, seed=8)
    a = w.arrays
    q = torch.from_numpy(ref.queries(a["q_nope"], a["q_rope"]))
    pool = torch.from_numpy(ref.bf16_to_f64(a["kv"]))
    scale = float(np.float32(w.softmax_scale))
    out0, _ = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], {"kv": a["kv"]}, a["indices"], None, w.softmax_scale)
    out1, lse1 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], {"kv": a["kv"]}, a["indices"], a["sink"],
                                       w.softmax_scale)
    for t in range(3):
        k = pool[torch.from_numpy(a["indices"][t].astype(np.int64))]
        o = torch.nn.functional.scaled_dot_product_attention(q[t][None], k[None], k[None], scale=scale)[0]
        np.testing.assert_allclose(out0[t], o.numpy(), rtol=1e-10, atol=1e-12)
        s = scale * q[t] @ k.T
        sk = torch.from_numpy(a["sink"].astype(np.float64))[:, None]
        p = torch.softmax(torch.cat([s, sk], dim=1), dim=1)[:, :-1]
        np.testing.assert_allclose(out1[t], (p @ k).numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse1[t], torch.logsumexp(torch.cat([s, sk], 1), 1).numpy(), rtol=1e-12)


def test_hand_worked_example():
    """tests/golden/hand_example.json: scores and weights derived by hand."""
    ex = json.loads((GOLDEN / "hand_example.json").read_text())
    kv = np.array(ex["kv_bits"], dtype=np.uint16)
    qn = np.array(ex["q_nope_bits"], dtype=np.uint16).reshape(1, 1, 448)
    qr = np.array(ex["q_rope_bits"], dtype=np.uint16).reshape(1, 1, 64)
    idx = np.array([ex["indices"]], dtype=np.int32)
    sink = np.array([ex["sink"]], dtype=np.float32)
    out, lse = ref.sparse_mla_decode(qn, qr, {"kv": kv}, idx, sink, ex["softmax_scale"])
    w = np.array([math.exp(v) for v in ex["expected_scores"]])
    z = w.sum() + math.exp(ex["sink"])
    rows = ref.bf16_to_f64(kv)
    expect = sum(w[j] / z * rows[i] for j, i in enumerate(i for i in ex["indices"] if i >= 0))
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-14, atol=1e-15)
    assert abs(lse[0, 0] - math.log(z)) < 1e-14
    np.testing.assert_allclose(out[0, 0, :4], ex["expected_out_first4"], rtol=1e-12)
    assert abs(lse[0, 0] - ex["expected_lse"]) < 1e-12


# ----------------------------------------------------------------------------
# splits and merge
# ----------------------------------------------------------------------------
def test_split_bounds_examples_and_properties():
    assert ref.split_bounds(2176, 4) == [(0, 576), (576, 1152), (1152, 1728), (1728, 2176)]
    assert ref.split_bounds(64, 4) == [(0, 64), (64, 64), (64, 64), (64, 64)]
    assert ref.split_bounds(0, 3) == [(0, 0), (0, 0), (0, 0)]
    rng = np.random.default_rng(2)
    for _ in range(500):
        K = int(rng.integers(0, 70000))
        s = int(rng.integers(1, 33))
        b = ref.split_bounds(K, s)
        assert len(b) == s and b[0][0] == 0 and b[-1][1] == K
        for (a0, e0), (a1, e1) in zip(b, b[1:]):
            assert e0 == a1
        for a0, e0 in b:
            assert a0 <= e0 and (a0 % 64 == 0 or a0 == K)
            assert e0 == K or (e0 - a0) % 64 == 0


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_split_merge_identity(kv_dtype):
    rng = np.random.default_rng(3)
    w = wl.dense_workload("merge id", T=2, H=16, kv_dtype=kv_dtype, pool_rows=600, topk=333, swa=20, invalid=7,
                          seed=9)
    a = w.arrays
    pool = ref_pool(w)
    out, lse = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, a["indices"], a["sink"], w.softmax_scale)
    for s in [1, 2, 3, 5, 6, 17, 32] + list(rng.integers(1, 33, 3)):
        po, pl = ref.sparse_mla_decode_partials(a["q_nope"], a["q_rope"], pool, a["indices"], w.softmax_scale,
                                                int(s))
        o2, l2 = ref.merge_partials(po, pl, a["sink"])
        np.testing.assert_allclose(o2, out, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(l2, lse, rtol=1e-12)


def test_merge_degenerate():
    po = np.zeros((1, 2, 3, 512))
    pl = np.full((1, 2, 3), -np.inf)
    o, l = ref.merge_partials(po, pl, None)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    o, l = ref.merge_partials(po, pl, np.array([0.5, -1.0], dtype=np.float32))
    assert np.all(o == 0) and np.allclose(l[0], [0.5, -1.0])


def ref_pool(w):
    a = w.arrays
    return {"kv": a["kv"]} if w.kv_dtype == "bf16" else {"nope": a["nope"], "scale": a["scale"], "rope": a["rope"]}


# ----------------------------------------------------------------------------
# invariants and closed forms
# ----------------------------------------------------------------------------
def test_sink_only_rescales():
    w = wl.dense_workload("sink", T=2, H=16, kv_dtype="bf16", pool_rows=400, topk=90, invalid=4, seed=10)
    a = w.arrays
    o0, l0 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], {"kv": a["kv"]}, a["indices"], None, w.softmax_scale)
    o1, l1 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], {"kv": a["kv"]}, a["indices"], a["sink"],
                                   w.softmax_scale)
    sk = a["sink"].astype(np.float64)[None, :]
    np.testing.assert_allclose(o1, o0 / (1.0 + np.exp(sk - l0))[..., None], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, np.logaddexp(l0, sk), rtol=1e-13)
    # a very negative sink recovers the sink-free result; a very positive one drives out to 0
    o2, _ = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], {"kv": a["kv"]}, a["indices"],
                                  np.full(16, -1e4, np.float32), w.softmax_scale)
    np.testing.assert_allclose(o2, o0, rtol=1e-13, atol=1e-15)
    o3, _ = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], {"kv": a["kv"]}, a["indices"],
                                  np.full(16, 1e4, np.float32), w.softmax_scale)
    assert np.abs(o3).max() < 1e-300


def test_invalid_entries_contribute_nothing():
    w = wl.dense_workload("invalid", T=2, H=16, kv_dtype="bf16", pool_rows=256, topk=40, seed=11)
    a = w.arrays
    pool = {"kv": a["kv"]}
    o0, l0 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, a["indices"], a["sink"], w.softmax_scale)
    ext = np.concatenate([a["indices"], np.full((2, 9), -1, np.int32), np.full((2, 3), 256, np.int32)], axis=1)
    o1, l1 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, ext, a["sink"], w.softmax_scale)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    # NaN in rows nobody selects changes nothing
    kv = a["kv"].copy()
    unused = np.setdiff1d(np.arange(256), a["indices"].ravel())
    kv[unused] = 0x7FC0
    o2, l2 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], {"kv": kv}, a["indices"], a["sink"], w.softmax_scale)
    np.testing.assert_array_equal(o0, o2)
    # all invalid: zero output, lse = sink (or -inf without one)
    allbad = np.full((2, 12), -1, np.int32)
    o3, l3 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, allbad, a["sink"], w.softmax_scale)
    assert np.all(o3 == 0) and np.allclose(l3, a["sink"][None, :].astype(np.float64))
    o4, l4 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, allbad, None, w.softmax_scale)
    assert np.all(o4 == 0) and np.all(np.isneginf(l4))


def test_permutation_invariance():
    w = wl.dense_workload("perm", T=2, H=16, kv_dtype="fp8", pool_rows=300, topk=120, invalid=5, seed=12)
    a = w.arrays
    pool = ref_pool(w)
    o0, l0 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, a["indices"], a["sink"], w.softmax_scale)
    perm = np.random.default_rng(4).permutation(120)
    o1, l1 = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, a["indices"][:, perm], a["sink"],
                                   w.softmax_scale)
    np.testing.assert_allclose(o0, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l0, l1, rtol=1e-13)


def test_closed_forms():
    w = wl.dense_workload("closed", T=1, H=16, kv_dtype="bf16", pool_rows=100, topk=10, seed=13)
    a = w.arrays
    pool = {"kv": a["kv"]}
    rows = ref.bf16_to_f64(a["kv"])
    qz = np.zeros_like(a["q_nope"]), np.zeros_like(a["q_rope"])
    idx = a["indices"].copy()
    idx[0, 1] = idx[0, 0]                      # duplicate counts twice
    # q = 0, no sink -> mean of the gathered multiset
    o, l = ref.sparse_mla_decode(*qz, pool, idx, None, w.softmax_scale)
    np.testing.assert_allclose(o[0, 0], rows[idx[0]].mean(axis=0), rtol=1e-13, atol=1e-15)
    assert abs(l[0, 0] - math.log(10)) < 1e-13
    # scale = 0 is the same
    o, _ = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, idx, None, 0.0)
    np.testing.assert_allclose(o[0, 0], rows[idx[0]].mean(axis=0), rtol=1e-13, atol=1e-15)
    # one valid entry, no sink -> exactly that row
    one = np.full((1, 5), -1, np.int32)
    one[0, 3] = 42
    o, l = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, one, None, w.softmax_scale)
    assert np.array_equal(o[0], np.broadcast_to(rows[42], (16, 512)))
    # one valid entry with a sink -> row * sigmoid(s - sink)
    q = ref.queries(a["q_nope"], a["q_rope"])[0]
    s = float(np.float32(w.softmax_scale)) * (q @ rows[42])
    o, l = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], pool, one, a["sink"], w.softmax_scale)
    sig = 1.0 / (1.0 + np.exp(a["sink"].astype(np.float64) - s))
    np.testing.assert_allclose(o[0], sig[:, None] * rows[42][None, :], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l[0], np.logaddexp(s, a["sink"].astype(np.float64)), rtol=1e-14)


def test_ragged_matches_dense_and_skips_empty():
    w = wl.ragged_workload("ragged", B=5, q_per_seq=2, H=16, kv_dtype="bf16", pool_rows=500, max_k=80,
                           zero_rows=2, indptr_offset=3, seed=14)
    a = w.arrays
    out, lse, written = ref.sparse_mla_decode_ragged(a["q_nope"], a["q_rope"], {"kv": a["kv"]}, a["kv_indptr"],
                                                     a["kv_indices"], a["sink"], w.softmax_scale, 2)
    ptr = a["kv_indptr"]
    for b in range(5):
        t0, t1 = 2 * b, 2 * b + 2
        if ptr[b + 1] == ptr[b]:
            assert not written[t0:t1].any() and np.isnan(out[t0:t1]).all()
            continue
        idx = a["kv_indices"][ptr[b]:ptr[b + 1]][None]
        o, l = ref.sparse_mla_decode(a["q_nope"][t0:t1], a["q_rope"][t0:t1], {"kv": a["kv"]}, idx, a["sink"],
                                     w.softmax_scale, q_per_seq=2)
        np.testing.assert_array_equal(out[t0:t1], o)
        np.testing.assert_array_equal(lse[t0:t1], l)

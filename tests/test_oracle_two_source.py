"""Pins of the two-source (main + sliding-window) oracle, CPU only: brute
force over both pools with multiplicities, the reduction to the pinned
single-source decode, the split-merge identity over the ordered positions, the
merge of per-source partials, and a one-hot worked example that recovers
which rows of which pool each split gathered."""
import numpy as np
import pytest

import workloads as wl
from oracle import ref


def _bf16_pool(rng, n):
    return {"kv": wl.f32_to_bf16_bits(rng.standard_normal((n, 512), dtype=np.float32))}


def _case(seed=0, T=3, H=4, n_main=40, n_swa=24, k_main=30, k_swa=12):
    rng = np.random.default_rng(seed)
    q_nope = wl.f32_to_bf16_bits(rng.standard_normal((T, H, 448), dtype=np.float32))
    q_rope = wl.f32_to_bf16_bits(rng.standard_normal((T, H, 64), dtype=np.float32))
    main, swa = _bf16_pool(rng, n_main), _bf16_pool(rng, n_swa)
    mi = rng.integers(-3, n_main + 3, size=(T, k_main)).astype(np.int32)   # -1s, out of range, duplicates
    si = rng.integers(-3, n_swa + 3, size=(T, k_swa)).astype(np.int32)
    if k_swa:
        si[:, 0] = n_swa + 1  # valid for the main pool's size, not for the SWA pool's
    sink = rng.standard_normal(H).astype(np.float32)
    return q_nope, q_rope, main, swa, mi, si, sink


def _brute(q_nope, q_rope, main, swa, mi, si, sink, scale):
    """Attention over every row of both pools, row weight = its multiplicity
    among the valid entries of its own list."""
    q = np.concatenate([ref.bf16_to_f64(q_nope), ref.bf16_to_f64(q_rope)], axis=-1)
    km, ks = ref.bf16_to_f64(main["kv"]), ref.bf16_to_f64(swa["kv"])
    rows = np.concatenate([km, ks])
    T, H, _ = q.shape
    out, lse = np.zeros((T, H, 512)), np.zeros((T, H))
    sc = float(np.float32(scale))
    for t in range(T):
        c = np.zeros(len(rows))
        for i in mi[t]:
            if 0 <= i < len(km):
                c[i] += 1
        for i in si[t]:
            if 0 <= i < len(ks):
                c[len(km) + i] += 1
        for h in range(H):
            s = sc * (rows @ q[t, h])
            z = np.sum(c * np.exp(s)) + np.exp(float(sink[h]))
            out[t, h] = (c * np.exp(s)) @ rows / z
            lse[t, h] = np.log(z)
    return out, lse


def test_two_source_brute_force():
    q_nope, q_rope, main, swa, mi, si, sink = _case()
    o, l = ref.sparse_mla_decode_two_source(q_nope, q_rope, main, mi, swa, si, sink, 0.05)
    bo, bl = _brute(q_nope, q_rope, main, swa, mi, si, sink, 0.05)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, bl, rtol=0, atol=1e-12)


def test_one_pool_reduces_to_single_source():
    q_nope, q_rope, main, _, mi, _, sink = _case(seed=1)
    si = np.random.default_rng(5).integers(-1, 40, size=(3, 17)).astype(np.int32)
    o, l = ref.sparse_mla_decode_two_source(q_nope, q_rope, main, mi, main, si, sink, 0.07)
    so, sl = ref.sparse_mla_decode(q_nope, q_rope, main, np.concatenate([mi, si], axis=1), sink, 0.07)
    np.testing.assert_allclose(o, so, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, sl, rtol=0, atol=1e-13)


@pytest.mark.parametrize("k_main,k_swa", [(70, 60), (200, 128), (0, 50), (64, 0), (1, 1)])
def test_split_merge_identity(k_main, k_swa):
    q_nope, q_rope, main, swa, mi, si, sink = _case(seed=2, k_main=k_main, k_swa=k_swa)
    o, l = ref.sparse_mla_decode_two_source(q_nope, q_rope, main, mi, swa, si, sink, 0.05)
    for s in range(1, 9):
        po, pl = ref.sparse_mla_decode_two_source_partials(q_nope, q_rope, main, mi, swa, si, 0.05, s)
        mo, ml = ref.merge_partials(po, pl, sink)
        np.testing.assert_allclose(mo, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, l, rtol=0, atol=1e-12)


def test_merge_of_per_source_partials():
    """Each source decoded alone into one partial (no sink), the two merged
    with the sink, equals the two-source decode."""
    q_nope, q_rope, main, swa, mi, si, sink = _case(seed=3)
    pm, lm = ref.sparse_mla_decode_partials(q_nope, q_rope, main, mi, 0.05, 1)
    ps, ls = ref.sparse_mla_decode_partials(q_nope, q_rope, swa, si, 0.05, 1)
    mo, ml = ref.merge_partials(np.concatenate([pm, ps], axis=2), np.concatenate([lm, ls], axis=2), sink)
    o, l = ref.sparse_mla_decode_two_source(q_nope, q_rope, main, mi, swa, si, sink, 0.05)
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, l, rtol=0, atol=1e-12)


def test_one_hot_split_contents():
    """Worked example.  Main row r is e_r, SWA row r is e_(256+r), q = 0, so a
    split's o is the mean of the rows it gathered and exposes them exactly.
    K_main = 70, K_swa = 60, s = 2: chunk = roundup(ceil(130 / 2), 64) = 128,
    so split 0 holds positions 0..127 (main 0..69, SWA 0..57) and split 1 the
    positions 128, 129: SWA entries 58 and 59."""
    n_main, n_swa = 100, 200
    main = {"kv": np.zeros((n_main, 512), dtype=np.uint16)}
    swa = {"kv": np.zeros((n_swa, 512), dtype=np.uint16)}
    one = 0x3F80  # bf16 1.0
    main["kv"][np.arange(n_main), np.arange(n_main)] = one
    swa["kv"][np.arange(n_swa), 256 + np.arange(n_swa) % 256] = one
    mi = (np.arange(70, dtype=np.int32) * 3 % n_main)[None, :]
    si = (np.arange(60, dtype=np.int32) * 7 % 250)[None, :]   # entries >= 200 are invalid for the SWA pool
    q0 = np.zeros((1, 1, 448), dtype=np.uint16)
    r0 = np.zeros((1, 1, 64), dtype=np.uint16)
    po, pl = ref.sparse_mla_decode_two_source_partials(q0, r0, main, mi, swa, si, 1.0, 2)
    # split 1: SWA entries 58 and 59 are 406 % 250 = 156 and 413 % 250 = 163, both valid
    want1 = np.zeros(512)
    want1[256 + 156] = want1[256 + 163] = 0.5
    np.testing.assert_array_equal(po[0, 0, 1], want1)
    assert pl[0, 0, 1] == pytest.approx(np.log(2.0), abs=1e-15)
    # split 0: all 70 main entries (dims 3p % 100) and the valid SWA entries 0..57
    cnt = np.zeros(512)
    for p in range(70):
        cnt[3 * p % 100] += 1
    for p in range(58):
        v = 7 * p % 250
        if v < n_swa:
            cnt[256 + v] += 1
    np.testing.assert_allclose(po[0, 0, 0], cnt / cnt.sum(), rtol=0, atol=1e-15)
    assert pl[0, 0, 0] == pytest.approx(np.log(cnt.sum()), abs=1e-13)

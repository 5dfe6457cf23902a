"""Pins of the paged GQA decode oracle (oracle.paged_ref): float64 SDPA on
the gathered rows with the MTP-causal mask, the sparse decode oracle on a
one-head cache with K = V, invariance under a permutation of the physical
blocks, the MTP positions against shorter contexts, the split-merge
identity, empty contexts, and block-table entries that name no block against
the same sequence with that page taken out."""
import numpy as np
import torch

from oracle import paged_ref, ref


def _bf16(x):
    return (torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
            .view(np.uint16))


def _case(seed, B=3, mtp=2, Hq=4, Hkv=2, D=64, page=8, max_ctx=40, nblk=64, lens=None):
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((B * mtp, Hq, D)))
    k = _bf16(rng.standard_normal((nblk, page, Hkv, D)))
    v = _bf16(rng.standard_normal((nblk, page, Hkv, D)))
    pages = -(-max_ctx // page)
    bt = np.stack([rng.permutation(nblk)[:pages] for _ in range(B)]).astype(np.int32)
    cl = np.array(lens if lens is not None else rng.integers(1, max_ctx + 1, B), dtype=np.int32)
    return q, k, v, bt, cl


def test_against_sdpa_with_the_mtp_causal_mask():
    q, k, v, bt, cl = _case(1)
    B, mtp, page = 3, 2, 8
    out, lse = paged_ref.paged_decode(q, k, v, bt, cl, page, mtp, 0.11)
    T, Hq, D = q.shape
    Hkv = k.shape[2]
    for b in range(B):
        L = int(cl[b])
        blk, slot = bt[b, np.arange(L) // page], np.arange(L) % page
        kk = torch.from_numpy(ref.bf16_to_f64(k[blk, slot]))          # [L, Hkv, D]
        vv = torch.from_numpy(ref.bf16_to_f64(v[blk, slot]))
        qq = torch.from_numpy(ref.bf16_to_f64(q[b * mtp:(b + 1) * mtp]))  # [mtp, Hq, D]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            mask = torch.tensor([[p < L - (mtp - 1 - i) for p in range(L)] for i in range(mtp)])
            o = torch.nn.functional.scaled_dot_product_attention(qq[None, None, :, h], kk[None, None, :, g],
                                                                 vv[None, None, :, g], attn_mask=mask[None, None],
                                                                 scale=float(np.float32(0.11)))[0, 0]
            np.testing.assert_allclose(out[b * mtp:(b + 1) * mtp, h], o.numpy(), rtol=0, atol=1e-12)


def test_one_head_with_k_equal_v_is_the_sparse_decode():
    """Hq = Hkv = 1, mtp = 1, V = K: the sparse decode oracle over the
    physical rows the block table names (no sink)."""
    q, k, _, bt, cl = _case(2, B=4, mtp=1, Hq=1, Hkv=1, D=512, page=4, max_ctx=30, nblk=40)
    out, lse = paged_ref.paged_decode(q, k, k, bt, cl, 4, 1, 0.05)
    pool = {"kv": k.reshape(-1, 512)}                                   # row = block * 4 + slot
    for b in range(4):
        L = int(cl[b])
        rows = (bt[b, np.arange(L) // 4] * 4 + np.arange(L) % 4).astype(np.int32)[None]
        # the sparse oracle takes the 512 dims as 448 NoPE + 64 RoPE
        qn, qr = q[b:b + 1, :, :448], q[b:b + 1, :, 448:]
        o2, l2 = ref.sparse_mla_decode(qn, qr, pool, rows, None, 0.05)
        np.testing.assert_allclose(out[b], o2[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], l2[0], rtol=0, atol=1e-12)


def test_block_permutation_invariance():
    q, k, v, bt, cl = _case(3)
    perm = np.random.default_rng(9).permutation(k.shape[0])
    inv = np.argsort(perm)
    out1, lse1 = paged_ref.paged_decode(q, k, v, bt, cl, 8, 2, 0.2)
    out2, lse2 = paged_ref.paged_decode(q, k[perm], v[perm], inv[bt].astype(np.int32), cl, 8, 2, 0.2)
    np.testing.assert_array_equal(out1, out2)
    np.testing.assert_array_equal(lse1, lse2)


def test_mtp_positions_equal_shorter_contexts():
    """Token i of an mtp-token step is the one-token decode of the context cut
    mtp - 1 - i positions short."""
    q, k, v, bt, cl = _case(4, B=2, mtp=3, lens=[20, 33])
    out, lse = paged_ref.paged_decode(q, k, v, bt, cl, 8, 3, 0.1)
    for b in range(2):
        for i in range(3):
            t = 3 * b + i
            o1, l1 = paged_ref.paged_decode(q[t:t + 1], k, v, bt[b:b + 1], cl[b:b + 1] - (2 - i), 8, 1, 0.1)
            np.testing.assert_allclose(out[t], o1[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[t], l1[0], rtol=0, atol=1e-12)


def test_split_merge_identity():
    q, k, v, bt, cl = _case(5, lens=[40, 17, 1])
    out, lse = paged_ref.paged_decode(q, k, v, bt, cl, 8, 2, 0.1)
    for s in (1, 2, 3, 5):
        po, pl = paged_ref.paged_decode_partials(q, k, v, bt, cl, 8, 2, 0.1, s, 40)
        mo, ml = ref.merge_partials(po, pl, None)
        np.testing.assert_allclose(mo, out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)


def test_empty_context():
    """A context shorter than the MTP span leaves the early tokens with no
    position: out = 0, lse = -inf."""
    q, k, v, bt, cl = _case(6, B=1, mtp=3, lens=[1])
    out, lse = paged_ref.paged_decode(q, k, v, bt, cl, 8, 3, 0.1)
    assert np.all(out[:2] == 0) and np.all(np.isneginf(lse[:2]))
    assert np.all(np.isfinite(lse[2]))


def test_invalid_block_entries_equal_the_page_taken_out():
    """A page whose block-table entry is outside [0, num_blocks) is masked: a
    sequence with such a page below every token's limit decodes as the same
    sequence with that page removed (the table shifted left, the context one
    page shorter), bit for bit; the split partials still merge to it."""
    page, mtp = 8, 2
    q, k, v, bt, cl = _case(7, B=3, mtp=mtp, page=page, max_ctx=40, lens=[40, 33, 25])
    nblk = k.shape[0]
    bad = bt.copy()
    bad[0, 1] = -1            # page 1 of sequence 0
    bad[1, 0] = nblk + 3      # page 0 of sequence 1
    bad[2, 2] = np.iinfo(np.int32).min
    out, lse = paged_ref.paged_decode(q, k, v, bad, cl, page, mtp, 0.1)
    for b, j in ((0, 1), (1, 0), (2, 2)):
        short = np.concatenate([bt[b, :j], bt[b, j + 1:], bt[b, :1]])[None].astype(np.int32)
        sl = slice(b * mtp, (b + 1) * mtp)
        o2, l2 = paged_ref.paged_decode(q[sl], k, v, short, cl[b:b + 1] - page, page, mtp, 0.1)
        np.testing.assert_array_equal(out[sl], o2)
        np.testing.assert_array_equal(lse[sl], l2)
    po, pl = paged_ref.paged_decode_partials(q, k, v, bad, cl, page, mtp, 0.1, 3, 40)
    mo, ml = ref.merge_partials(po, pl, None)
    np.testing.assert_allclose(mo, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)

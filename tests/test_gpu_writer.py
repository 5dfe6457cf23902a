"""GPU parity of the fp8/UE8M0 cache writer (smd_write_kv_fp8) against the
oracle (oracle/writer_ref.py): bytes, codes and RoPE bits compared exactly,
on seeded rows over many magnitudes, on edge rows (zeros, signed zeros,
power-of-two boundaries, subnormals, the largest bf16, NaN, infinities), with
slots and padded strides; and a round trip through the decode."""
import numpy as np
import pytest
import torch

import sparse_mla_decode_index_amd as smd
import workloads as wl
from oracle import ref, writer_ref
from tests.helpers import bf16_tensor, check_lse, check_out

pytestmark = pytest.mark.gpu


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return wl.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _rows(n, seed):
    """Seeded rows: N(0,1) scaled per row by 2^U{-140..130} (clamped to the
    bf16 range by the rounding), so codes cover most of [0, 254]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 512))
    x *= np.exp2(rng.integers(-140, 121, size=(n, 1)).astype(np.float64))
    with np.errstate(over="ignore"):
        return _bf16_bits(x.astype(np.float32))


def _edge_rows():
    rows = []
    z = np.zeros(512, dtype=np.float32)
    rows.append(z.copy())                                   # all zeros
    r = z.copy(); r[::2] = -0.0; rows.append(r)            # signed zeros
    for k in (-12, 0, 7, 40):
        r = z.copy()
        r[:64] = 448.0 * 2.0 ** k                          # amax exactly 448 * 2^k
        r[64:128] = 450.0 * 2.0 ** k                       # one bf16 step above
        r[128:192] = np.linspace(-1, 1, 64) * 2.0 ** k     # interior values, ties
        r[192:256] = 464.0 * 2.0 ** (k - 8) * np.r_[1.0, np.ones(63) * 0.5]
        rows.append(r)
    r = z.copy()
    r[0:64] = np.float32(2.0 ** -133) * np.arange(64)      # bf16 subnormals
    r[64:128] = np.float32(3.3895314e38)                   # the largest finite bf16
    r[128] = np.nan; r[129:192] = 3.0                      # NaN among values
    r[192:256] = np.nan                                    # an all-NaN block
    r[256] = np.inf; r[257] = -np.inf; r[258] = 1.0        # infinities
    r[320:384] = np.float32(1e-40)                         # fp32-subnormal range
    r[448] = np.nan; r[449] = 1.0; r[511] = -np.inf        # RoPE
    rows.append(r)
    bits = _bf16_bits(np.array(rows, dtype=np.float32))
    bits[-1, 450] = 0xFF81                                 # a non-canonical RoPE NaN
    return bits


def _pool(n, gpu, nope_stride=448, scale_stride=8, rope_stride=64):
    nope = torch.full((n, nope_stride), 0xAA, dtype=torch.uint8, device=gpu)
    scale = torch.full((n, scale_stride), 0xAA, dtype=torch.uint8, device=gpu)
    rope = torch.full((n, rope_stride), 0x5555, dtype=torch.int16, device=gpu).view(torch.bfloat16)
    return nope, scale, rope, smd.KVPool.fp8(nope[:, :448], scale[:, :8], rope[:, :64])


def _expect(kv_bits, slots, n):
    nope = np.full((n, 448), 0xAA, dtype=np.uint8)
    codes = np.full((n, 8), 0xAA, dtype=np.uint8)
    rope = np.full((n, 64), 0x5555, dtype=np.uint16)
    writer_ref.write_cache(kv_bits, slots, n, nope, codes, rope)
    return nope, codes, rope


def _check(pool_t, kv_bits, slots, n):
    nope, scale, rope = pool_t
    e_nope, e_codes, e_rope = _expect(kv_bits, slots, n)
    g_nope = nope[:, :448].cpu().numpy()
    g_codes = scale[:, :8].cpu().numpy()
    g_rope = rope[:, :64].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.argwhere(g_nope != e_nope)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[0]}: {g_nope[tuple(bad[0])]:#x} vs " \
                          f"{e_nope[tuple(bad[0])]:#x}"
    assert np.array_equal(g_codes, e_codes)
    assert np.array_equal(g_rope, e_rope)


@pytest.mark.parametrize("n,seed", [(1, 1), (37, 2), (4096, 3)])
def test_writer_rows_exact(gpu, n, seed):
    kv_bits = _rows(n, seed)
    nope, scale, rope, pool = _pool(n, gpu)
    print(f"writer rows n={n}", flush=True)
    smd.write_kv_fp8(bf16_tensor(kv_bits, gpu), pool)
    torch.cuda.synchronize()
    _check((nope, scale, rope), kv_bits, None, n)


def test_writer_edge_rows_exact(gpu):
    kv_bits = _edge_rows()
    n = kv_bits.shape[0]
    nope, scale, rope, pool = _pool(n, gpu)
    print("writer edge rows", flush=True)
    smd.write_kv_fp8(bf16_tensor(kv_bits, gpu), pool)
    torch.cuda.synchronize()
    _check((nope, scale, rope), kv_bits, None, n)


def test_writer_slots_and_strides(gpu):
    """Rows go to their slots; -1 and slots past the pool are skipped and the
    rows no slot names keep their contents; padded strides on every array."""
    rng = np.random.default_rng(9)
    n_in, n_pool = 50, 64
    kv_bits = _rows(n_in, 4)
    slots = rng.permutation(n_pool)[:n_in].astype(np.int32)
    slots[::7] = -1
    slots[3] = n_pool
    kv_pad = torch.zeros((n_in, 520), dtype=torch.bfloat16, device=gpu)
    kv_pad[:, :512] = bf16_tensor(kv_bits, gpu)
    nope, scale, rope, pool = _pool(n_pool, gpu, nope_stride=512, scale_stride=16, rope_stride=72)
    print("writer slots", flush=True)
    smd.write_kv_fp8(kv_pad[:, :512], pool, torch.from_numpy(slots).to(gpu))
    torch.cuda.synchronize()
    _check((nope, scale, rope), kv_bits, slots, n_pool)
    # the padding columns are untouched
    assert torch.all(nope[:, 448:] == 0xAA) and torch.all(scale[:, 8:] == 0xAA)


def test_writer_two_rows_per_wave(gpu):
    """Large writes take two rows per wave: an odd row count leaves the last
    wave one row, and skipped slots fall on either row of a wave."""
    n_in, n_pool = 65537, 70000
    rng = np.random.default_rng(11)
    kv_bits = _rows(n_in, 5)
    edge = _edge_rows()
    kv_bits[1000:1000 + len(edge)] = edge      # NaN, infinities, zeros on both rows of a wave
    kv_bits[-len(edge) - 1:-1] = edge
    slots = rng.permutation(n_pool)[:n_in].astype(np.int32)
    slots[rng.choice(n_in, 300, replace=False)] = -1
    slots[-1] = n_pool + 5
    nope, scale, rope, pool = _pool(n_pool, gpu)
    print(f"writer two rows per wave n={n_in}", flush=True)
    smd.write_kv_fp8(bf16_tensor(kv_bits, gpu), pool, torch.from_numpy(slots).to(gpu))
    torch.cuda.synchronize()
    _check((nope, scale, rope), kv_bits, slots, n_pool)


def test_writer_round_trip_through_decode(gpu):
    """A pool written by the GPU writer decodes like the oracle's writer +
    oracle decode (the bytes are equal, so this checks the wiring)."""
    w = wl.dense_workload("writer round trip", T=2, H=64, kv_dtype="bf16", pool_rows=2048, topk=300, invalid=3,
                          seed=401)
    a = w.arrays
    nope, scale, rope, pool = _pool(2048, gpu)
    smd.write_kv_fp8(bf16_tensor(a["kv"], gpu), pool)
    e_nope, e_codes, e_rope = writer_ref.quantize_rows(a["kv"])
    q_nope = bf16_tensor(a["q_nope"], gpu)
    q_rope = bf16_tensor(a["q_rope"], gpu)
    idx = torch.from_numpy(a["indices"]).to(gpu)
    sink = torch.from_numpy(a["sink"]).to(gpu)
    print("writer round trip", flush=True)
    out, lse = smd.sparse_mla_decode(q_nope, q_rope, pool, idx, sink, w.softmax_scale, num_splits=2)
    torch.cuda.synchronize()
    o_ref, l_ref = ref.sparse_mla_decode(a["q_nope"], a["q_rope"], {"nope": e_nope, "scale": e_codes,
                                                                    "rope": e_rope},
                                         a["indices"], a["sink"], w.softmax_scale)
    check_out(out, o_ref)
    check_lse(lse, l_ref)


def test_writer_rejects_bf16_pool(gpu):
    kv = torch.zeros((4, 512), dtype=torch.bfloat16, device=gpu)
    with pytest.raises((ValueError, smd.SmdError)):
        smd.write_kv_fp8(kv, smd.KVPool.bf16(torch.zeros((4, 512), dtype=torch.bfloat16, device=gpu)))

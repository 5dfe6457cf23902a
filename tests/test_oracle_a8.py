"""Pins of the fp8-QK oracle (oracle.a8_ref), each independent of the
quantiser it checks: a brute-force nearest search over every E4M3FN code,
the block code as the smallest admissible exponent found by search, the
identity on queries that are already representable, and the decode on those
queries against the exact decode."""
import math

import numpy as np
import torch

from oracle import a8_ref, ref



def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values that are bf16-representable -> their bf16 bits."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _round_to_bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


# every finite E4M3FN value with its code, from the format's definition
def _e4m3_table():
    vals, codes = [], []
    for c in range(256):
        e, m = (c >> 3) & 0xF, c & 7
        if e == 0xF and m == 7:
            continue  # NaN
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.append(-v if c & 0x80 else v)
        codes.append(c)
    return np.array(vals), np.array(codes)


def _block_code_by_search(amax: float) -> int:
    """Smallest c in [0, 254] with amax <= 448 * 2^(c - 127) (0 for amax = 0)."""
    if amax == 0.0:
        return 0
    for c in range(255):
        if amax <= 448.0 * math.ldexp(1.0, c - 127):
            return c
    return 254


def test_block_codes_are_the_smallest_admissible_exponent():
    rng = np.random.default_rng(1)
    x = _round_to_bf16(rng.standard_normal((5, 448)) * np.exp2(rng.integers(-20, 20, (5, 1))))
    x[2, 64:128] = 0.0  # an all-zero block
    _, _, codes = a8_ref.quantized_q_nope(_bf16_bits(x))
    for r in range(5):
        for b in range(7):
            assert codes[r, b] == _block_code_by_search(float(np.abs(x[r, 64 * b:64 * b + 64]).max())), (r, b)


def test_quantized_values_are_the_nearest_e4m3_at_the_block_scale():
    """Each value is the representable e4m3 * 2^(c-127) nearest to x, ties to
    the code with an even mantissa, found by trying all 255 finite codes."""
    tv, tc = _e4m3_table()
    rng = np.random.default_rng(2)
    x = _round_to_bf16(rng.standard_normal((3, 448)) * 3.0)
    vals, nbytes, codes = a8_ref.quantized_q_nope(_bf16_bits(x))
    for r in range(3):
        for d in range(448):
            s = math.ldexp(1.0, int(codes[r, d // 64]) - 127)
            err = np.abs(tv * s - float(x[r, d]))
            best = np.flatnonzero(err == err.min())
            if len(best) > 1:  # a tie: the even mantissa wins
                best = [i for i in best if tc[i] & 1 == 0]
            assert len(best) == 1
            assert tv[np.flatnonzero(tc == nbytes[r, d])[0]] == tv[best[0]]  # (+0 and -0 are both zero)
            assert vals[r, d] == tv[best[0]] * s


def test_identity_on_representable_queries_and_decode_equals_exact():
    """Queries that already are e4m3 values times their block scale, each
    block holding one value of magnitude 448 * 2^(c-127) (so the block code
    is c), come back unchanged, and the fp8-QK decode equals the exact one."""
    tv, _ = _e4m3_table()
    rng = np.random.default_rng(3)
    T, H = 2, 4
    c = rng.integers(118, 124, (T, H, 7))
    v = rng.choice(tv[np.abs(tv) <= 448], size=(T, H, 7, 64))
    v[..., 0] = 448.0 * rng.choice([-1.0, 1.0], size=(T, H, 7))
    x = (v * np.exp2(c[..., None] - 127.0)).reshape(T, H, 448).astype(np.float32)
    qn = _bf16_bits(x)
    assert np.array_equal(ref.bf16_to_f64(qn), x.astype(np.float64))  # bf16 holds them exactly
    vals, _, codes = a8_ref.quantized_q_nope(qn)
    assert np.array_equal(codes, c.astype(np.uint8))
    assert np.array_equal(vals, x.astype(np.float64))
    qr = _bf16_bits(_round_to_bf16(rng.standard_normal((T, H, 64))))
    pool = {"kv": _bf16_bits(_round_to_bf16(rng.standard_normal((300, 512))))}
    idx = rng.integers(-1, 300, (T, 50)).astype(np.int32)
    sink = rng.standard_normal(H).astype(np.float32)
    o8, l8 = a8_ref.sparse_mla_decode(qn, qr, pool, idx, sink, 0.04)
    oe, le = ref.sparse_mla_decode(qn, qr, pool, idx, sink, 0.04)
    assert np.array_equal(o8, oe) and np.array_equal(l8, le)


def test_quantisation_error_bound():
    """|x - q(x)| <= 2^-4 |x| for values in the normal range of the block
    (e4m3 keeps 3 fraction bits, so a rounding moves a value by at most half
    an ulp, 2^-4 of it)."""
    rng = np.random.default_rng(4)
    x = _round_to_bf16(rng.standard_normal((4, 448)))
    vals, _, codes = a8_ref.quantized_q_nope(_bf16_bits(x))
    smallest_normal = np.repeat(np.exp2(codes.astype(np.float64) - 127.0 - 6.0), 64, axis=1)
    normal = np.abs(x) >= smallest_normal
    assert np.all(np.abs(vals - x)[normal] <= 2.0 ** -4 * np.abs(x[normal]))

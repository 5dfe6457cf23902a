"""CPU pins of the fp8/UE8M0 cache-writer oracle (oracle/writer_ref.py).

The byte of every value is checked against an exhaustive search over the 256
E4M3FN codes (nearest value, ties to the even mantissa, beyond 464 -> NaN),
the codes against closed forms at and next to the powers-of-two boundaries,
and the NaN rules directly.
"""
import numpy as np
import pytest

from oracle import ref, writer_ref as w

_CODES = np.arange(256, dtype=np.uint8)
_VALUES = ref.e4m3fn_to_f64(_CODES)  # decode, pinned against torch in test_oracle


def _bits(x):
    """float -> bf16 bits (the inputs are chosen exactly representable)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "test value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _nearest_code(y: float) -> int:
    """Brute force: the E4M3FN code nearest to y, ties to the even mantissa,
    NaN past the largest finite value's rounding range."""
    if np.isnan(y):
        return 0xFF if np.signbit(y) else 0x7F
    if abs(y) > 464.0:
        return 0xFF if y < 0 else 0x7F
    finite = ~np.isnan(_VALUES)
    cand = _CODES[finite]
    vals = _VALUES[finite]
    d = np.abs(vals - y)
    best = cand[d == d.min()]
    if y == 0.0:
        return 0x80 if np.signbit(y) else 0x00
    best = [c for c in best if (c < 0x80) == (y > 0)]  # same sign as y
    if len(best) > 1:  # a tie: the even mantissa
        best = [c for c in best if (c & 1) == 0]
    assert len(best) == 1
    return int(best[0])


def test_bytes_are_the_nearest_codes():
    rng = np.random.default_rng(5)
    rows = []
    for scale in (1e-3, 0.3, 1.0, 17.0, 1e4, 3e-30):
        rows.append(rng.standard_normal(512) * scale)
    rows.append(np.r_[np.linspace(-500, 500, 448), rng.standard_normal(64)])
    x = np.array(rows, dtype=np.float32)
    kv = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncate to bf16 bits: exact inputs
    nope, codes, _ = w.quantize_rows(kv)
    xf = (kv[:, :448].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for i in range(len(rows)):
        for b in range(7):
            c = int(codes[i, b])
            for d in range(64 * b, 64 * b + 64):
                y = xf[i, d] * 2.0 ** (127 - c)
                assert int(nope[i, d]) == _nearest_code(y), (i, d, y)


def test_code_closed_forms():
    """amax = 448 * 2^k gives code 127 + k and the max value byte 0x7E; one
    bf16 step above it gives the next code; a zero block gives code 0."""
    for k in (-9, -3, 0, 1, 5, 20):
        row = np.zeros(512, dtype=np.float32)
        row[:64] = 1.0 * 2.0 ** k            # block 0: amax 2^k < 448 * 2^k
        row[3] = 448.0 * 2.0 ** k            # amax = 448 * 2^k exactly
        row[64:128] = 450.0 * 2.0 ** k        # block 1: one bf16 step above
        row[128:192] = -448.0 * 2.0 ** k     # block 2: the sign does not matter
        nope, codes, _ = w.quantize_rows(_bits(row)[None])
        assert codes[0, 0] == 127 + k and nope[0, 3] == 0x7E
        assert codes[0, 1] == 128 + k
        assert codes[0, 2] == 127 + k and nope[0, 130] == 0xFE
        assert np.all(codes[0, 3:7] == 0) and np.all(nope[0, 192:] == 0)
        assert codes[0, 7] == 0
    # codes stay within [0, 254]: the smallest and largest bf16 magnitudes
    row = np.zeros(512, dtype=np.float32)
    row[0] = np.float32(2.0 ** -133)          # smallest bf16 subnormal
    row[64] = np.float32(3.3895314e38)        # largest finite bf16
    _, codes, _ = w.quantize_rows(_bits(row)[None])
    assert codes[0, 0] == 0 and codes[0, 1] == 247


def test_round_trip_of_representable_values():
    """Values of the form e4m3 x 2^(c - 127) come back unchanged."""
    rng = np.random.default_rng(6)
    finite = _CODES[~np.isnan(_VALUES)]
    for c in (90, 120, 127, 140):
        picks = rng.choice(finite, size=448)
        picks[0] = 0x7E  # make 448 the block maxima so the code is c
        for b in range(1, 7):
            picks[64 * b] = 0x7E
        x = _VALUES[picks] * 2.0 ** (c - 127)
        row = np.r_[x, np.zeros(64)].astype(np.float32)
        nope, codes, _ = w.quantize_rows(_bits(row)[None])
        assert np.all(codes[0, :7] == c)
        back = _VALUES[nope[0]] * 2.0 ** (c - 127)
        assert np.array_equal(back, x)


def test_nan_and_infinity_rules():
    row = np.zeros(512, dtype=np.float32)
    row[0:64] = 1.0
    row[5] = np.nan                            # NaN ignored in amax, stored as NaN
    row[64:128] = np.nan                       # an all-NaN block: code 0, bytes NaN
    row[128] = -np.inf                         # infinite amax: code 254, the inf -> NaN
    row[129] = 1.0
    row[448] = np.nan                          # RoPE NaN -> canonical
    row[449] = -np.nan
    row[450] = 2.5
    kv = (row.view(np.uint32) >> 16).astype(np.uint16)[None]
    kv[0, 449] = 0xFFC1                        # a non-canonical negative NaN
    nope, codes, rope = w.quantize_rows(kv)
    assert codes[0, 0] == 127 - 8 and nope[0, 5] in (0x7F, 0xFF) and nope[0, 0] == 0x78  # 1.0 * 2^8 = 256: exponent field 15
    assert codes[0, 1] == 0 and np.all((nope[0, 64:128] & 0x7F) == 0x7F)
    assert codes[0, 2] == 254 and nope[0, 128] == 0xFF and nope[0, 129] == 0x00
    assert rope[0, 0] == 0x7FC0 and rope[0, 1] == 0x7FC0 and rope[0, 2] == _bits(np.float32(2.5))
    assert np.all(codes < 255)


def test_cache_update_with_slots():
    rng = np.random.default_rng(7)
    kv = (rng.standard_normal((5, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nope_pool = np.full((8, 448), 0xAA, dtype=np.uint8)
    code_pool = np.full((8, 8), 0xAA, dtype=np.uint8)
    rope_pool = np.full((8, 64), 0xAAAA, dtype=np.uint16)
    w.write_cache(kv, [6, -1, 0, 8, 3], 8, nope_pool, code_pool, rope_pool)
    nope, codes, rope = w.quantize_rows(kv)
    for r, s in ((0, 6), (2, 0), (4, 3)):
        assert np.array_equal(nope_pool[s], nope[r]) and np.array_equal(code_pool[s], codes[r])
        assert np.array_equal(rope_pool[s], rope[r])
    for s in (1, 2, 4, 5, 7):  # untouched rows (slot -1 and 8 are skipped)
        assert np.all(nope_pool[s] == 0xAA) and np.all(code_pool[s] == 0xAA) and np.all(rope_pool[s] == 0xAAAA)

"""Writes hand_example.json: a one-head decode whose result follows by hand.

q = e_0 (the first NoPE dim is 1, every other dim 0) and softmax_scale = 1, so
the score of a row is that row's dim 0.  Rows 3, 7 and 5 carry dim-0 values
0, 1 and 2; the index list is [3, 7, -1, 5] (the -1 is invalid and contributes
nothing) and the sink logit is 0.  Hence (definition of the decode on the vLLM
page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA decode on gfx950", Design:
one 512-wide QK dot, softmax with a sink in the denominator, PV over the same
rows):

    weights  e^0, e^1, e^2 for rows 3, 7, 5;  Z = 1 + e + e^2 + e^0 (sink)
    out      = (row3 + e*row7 + e^2*row5) / Z
    lse      = ln Z = ln(2 + e + e^2)

Every stored input is an exactly representable bf16 value.  Uses only math.
"""
import json
import math
import struct
from pathlib import Path


def bf16_bits(x: float) -> int:
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    assert b & 0xFFFF == 0, x  # exactly representable
    return b >> 16


def row_value(r: int, d: int) -> float:
    if d == 0:
        return {3: 0.0, 7: 1.0, 5: 2.0}.get(r, -3.0)
    return (((r * 7 + d * 3) % 9) - 4) * 0.125


rows = [[row_value(r, d) for d in range(512)] for r in range(8)]
e = math.e
z = 1.0 + e + e * e + 1.0
out4 = [(rows[3][d] + e * rows[7][d] + e * e * rows[5][d]) / z for d in range(4)]
ex = {
    "source": "closed form derived by hand; see make_hand_example.py",
    "softmax_scale": 1.0,
    "sink": 0.0,
    "indices": [3, 7, -1, 5],
    "q_nope_bits": [bf16_bits(1.0)] + [0] * 447,
    "q_rope_bits": [0] * 64,
    "kv_bits": [[bf16_bits(v) for v in row] for row in rows],
    "expected_scores": [0.0, 1.0, 2.0],
    "expected_out_first4": out4,
    "expected_lse": math.log(z),
}
Path(__file__).with_name("hand_example.json").write_text(json.dumps(ex))
print("wrote hand_example.json", out4, math.log(z))

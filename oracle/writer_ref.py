"""fp8/UE8M0 KV-cache writer, plain and slow -- test infrastructure only.

Neither the GPU path nor anything a user calls imports this module; only
tests/ do.

What is computed (the vLLM page "[ROCm][DSV4][Perf] Optimize Triton sparse-MLA
decode on gfx950", Design: on gfx950 both cache writers cap the UE8M0 codes at
254 and canonicalise RoPE NaNs; the rest of the rule is a reading the pages
leave open):

* a latent row is 512 bf16 values, NoPE dims [0, 448) then RoPE dims
  [448, 512);
* NoPE block b (dims [64b, 64b + 64), b = 0..6): amax = the largest |x| of the
  block, NaN ignored; code c = clamp(ceil(log2(amax / 448)) + 127, 0, 254),
  and c = 0 when amax = 0 (or every value is NaN);
* each NoPE value is stored as the OCP E4M3FN byte nearest to x * 2^(127 - c),
  ties to an even mantissa, non-saturating (beyond 464 in magnitude, and
  infinities, give NaN 0x7F with the sign bit of x; NaN gives NaN with its
  sign);
* the code row holds the 7 codes and one zero pad byte;
* RoPE dims are copied as bf16, every NaN replaced by the canonical 0x7FC0.

x * 2^(127 - c) is exact in float64, and the float64 -> float8_e4m3fn cast of
torch rounds to nearest even; both the cast and the code rule are pinned by
tests (an exhaustive nearest-code search, closed forms).
"""
from __future__ import annotations

import numpy as np
import torch

NOPE = 448
ROPE = 64
BLOCK = 64
BLOCKS = NOPE // BLOCK
CODE_CAP = 254
E4M3_MAX = 448.0
ROPE_NAN = 0x7FC0


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def block_codes(x: np.ndarray) -> np.ndarray:
    """UE8M0 codes of NoPE values x [n, 448] (float64): [n, 7] uint8."""
    xb = x.reshape(-1, BLOCKS, BLOCK)
    a = np.abs(xb)
    amax = np.fmax.reduce(a, axis=2)          # fmax ignores NaN
    amax = np.where(np.isnan(amax), 0.0, amax)  # every value NaN
    with np.errstate(divide="ignore", over="ignore"):
        e = np.where(amax > 0, np.ceil(np.log2(amax / E4M3_MAX)), -np.inf)
    c = np.where(amax > 0, np.clip(e + 127, 0, CODE_CAP), 0)
    return c.astype(np.uint8)


def e4m3fn_rne(y: np.ndarray) -> np.ndarray:
    """float64 -> OCP E4M3FN bytes, round to nearest even, non-saturating."""
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float64)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy().copy()


def quantize_rows(kv: np.ndarray):
    """kv: bf16 bits [n, 512] uint16.  Returns (nope uint8 [n, 448],
    codes uint8 [n, 8], rope bf16 bits uint16 [n, 64])."""
    kv = np.asarray(kv, dtype=np.uint16)
    n = kv.shape[0]
    x = _bf16_to_f64(kv[:, :NOPE])
    c = block_codes(x)
    scale = np.exp2(127.0 - c.astype(np.float64))  # exact powers of two
    y = x.reshape(n, BLOCKS, BLOCK) * scale[:, :, None]
    nope = e4m3fn_rne(y.reshape(n, NOPE))
    codes = np.zeros((n, 8), dtype=np.uint8)
    codes[:, :BLOCKS] = c
    rope = kv[:, NOPE:].copy()
    is_nan = ((rope & 0x7F80) == 0x7F80) & ((rope & 0x007F) != 0)
    rope[is_nan] = ROPE_NAN
    return nope, codes, rope


def write_cache(kv: np.ndarray, slots, pool_rows: int, nope_pool: np.ndarray, code_pool: np.ndarray,
                rope_pool: np.ndarray) -> None:
    """The writer as a cache update: input row r goes to pool row slots[r]
    (slots None: row r); a slot outside [0, pool_rows) is skipped.  Valid
    slots are distinct (no order between rows is defined)."""
    nope, codes, rope = quantize_rows(kv)
    n = kv.shape[0]
    dst = np.arange(n) if slots is None else np.asarray(slots, dtype=np.int64)
    for r in range(n):
        s = int(dst[r])
        if 0 <= s < pool_rows:
            nope_pool[s, :NOPE] = nope[r]
            code_pool[s, :8] = codes[r]
            rope_pool[s, :ROPE] = rope[r]

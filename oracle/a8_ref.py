"""fp8 ("a8w8") QK of sparse MLA decode, plain and slow -- test infrastructure
only.  Neither the GPU path nor anything a user calls imports this module.

The aiter page "[ASM][HIP][MLA v4 nm] Split plan helper and persistent decode
kernel" (Summary, part 2) names its persistent decode object "a8w8": 8-bit
queries against the 8-bit cache.  The pages do not say how q is quantised.
The reading used here: q_nope is quantised exactly as the cache writer
quantises a latent row's NoPE (``writer_ref``: per 64-dim block a UE8M0 code
c = clamp(ceil(log2(amax / 448)) + 127, 0, 254), c = 0 for an all-zero block,
each value the E4M3FN byte nearest to x * 2^(127 - c), ties to even); q_rope
stays bf16; and the decode is then the exact one of ``ref`` with q_nope
replaced by the quantised values e4m3(byte) * 2^(c - 127).  Everything after
the quantisation (scores, softmax with the sink, PV, split partials) is
``ref``'s float64 arithmetic, unchanged.

Pinned by tests/test_oracle_a8.py: every quantised value against a
brute-force nearest search over all 256 E4M3FN codes at the block's code,
the block code against its closed form, the identity on inputs that are
already representable, and the decode against ``ref`` on those inputs.
"""
from __future__ import annotations

import numpy as np

from oracle import ref, writer_ref

NOPE = ref.NOPE


def quantized_q_nope(q_nope: np.ndarray):
    """q_nope bf16 bits [..., 448] -> (values float64 [..., 448], bytes uint8
    [..., 448], codes uint8 [..., 7]): the E4M3FN bytes and UE8M0 block codes
    of the cache writer's rule, and the values they stand for."""
    q = np.asarray(q_nope, dtype=np.uint16)
    lead = q.shape[:-1]
    x = ref.bf16_to_f64(q.reshape(-1, NOPE))
    codes = writer_ref.block_codes(x)                                   # [n, 7]
    scale = np.exp2(127.0 - codes.astype(np.float64))                   # exact powers of two
    y = (x.reshape(-1, 7, 64) * scale[:, :, None]).reshape(-1, NOPE)
    nbytes = writer_ref.e4m3fn_rne(y)
    vals = ref.e4m3fn_to_f64(nbytes) * np.repeat(ref.ue8m0_to_f64(codes), 64, axis=1)
    return vals.reshape(*lead, NOPE), nbytes.reshape(*lead, NOPE), codes.reshape(*lead, 7)


def queries_a8(q_nope: np.ndarray, q_rope: np.ndarray) -> np.ndarray:
    """float64 [T, H, 512] queries of the fp8 QK: quantised NoPE, exact RoPE."""
    return np.concatenate([quantized_q_nope(q_nope)[0], ref.bf16_to_f64(q_rope)], axis=-1)


def sparse_mla_decode(q_nope, q_rope, pool: dict, indices, sink, softmax_scale: float, q_per_seq: int = 1):
    """``ref.sparse_mla_decode`` with the fp8-QK queries."""
    return ref.sparse_mla_decode(q_nope, q_rope, pool, indices, sink, softmax_scale, q_per_seq,
                                 queries64=queries_a8(q_nope, q_rope))


def sparse_mla_decode_ragged(q_nope, q_rope, pool: dict, kv_indptr, kv_indices, sink, softmax_scale: float,
                             q_per_seq: int):
    """``ref.sparse_mla_decode_ragged`` with the fp8-QK queries."""
    return ref.sparse_mla_decode_ragged(q_nope, q_rope, pool, kv_indptr, kv_indices, sink, softmax_scale,
                                        q_per_seq, queries64=queries_a8(q_nope, q_rope))


def sparse_mla_decode_partials(q_nope, q_rope, pool: dict, indices, softmax_scale: float, num_splits: int,
                               q_per_seq: int = 1):
    """``ref.sparse_mla_decode_partials`` with the fp8-QK queries."""
    return ref.sparse_mla_decode_partials(q_nope, q_rope, pool, indices, softmax_scale, num_splits, q_per_seq,
                                          queries64=queries_a8(q_nope, q_rope))

"""Python binding of libsmd (sparse MLA decode for MI355X).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  Tensors supply device memory and the current HIP stream; shapes and
dtypes are checked here, everything else by the library before it launches.
The library is loaded from this package directory and must have been built
(``python -m sparse_mla_decode_index_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from pathlib import Path
from typing import Optional

import torch

NOPE = 448
ROPE = 64
DIM = 512
MAX_SPLITS = 256
MAX_MERGE_SPLITS = 1024
NOALLOC_SCRATCH_BYTES = 32 << 20
SPLIT_ALIGN = 64
MAX_PARTITIONS = 16384

KV_BF16 = 0
KV_FP8_E4M3_UE8M0 = 1

# Kernel families of the split-KV decode (include/smd.h, SMD_KERNEL_*).
KERNEL_AUTO = 0
KERNEL_ROWS16 = 1
KERNEL_PAIRS = 2
KERNEL_WIDE = 3
_KERNELS = {"auto": KERNEL_AUTO, "rows16": KERNEL_ROWS16, "pairs": KERNEL_PAIRS, "wide": KERNEL_WIDE}

_LIB_PATH = Path(__file__).resolve().parent / "libsmd.so"
_lib = None


class SmdError(RuntimeError):
    """A libsmd entry point returned a negative status."""

    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


class _KVPool(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("num_rows", ctypes.c_int64),
        ("nope", ctypes.c_void_p),
        ("nope_stride", ctypes.c_int64),
        ("rope", ctypes.c_void_p),
        ("rope_stride", ctypes.c_int64),
        ("scale", ctypes.c_void_p),
        ("scale_stride", ctypes.c_int64),
    ]


class _DecodeOptions(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("merge", ctypes.c_int32), ("qk", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 5)]


MERGE_AUTO = 0
MERGE_WORKSPACE = 1
_MERGES = {"auto": MERGE_AUTO, "workspace": MERGE_WORKSPACE}
QK_BF16 = 0
QK_FP8 = 1
_QKS = {"bf16": QK_BF16, "fp8": QK_FP8}


def _options(kernel=None, merge=None, qk=None) -> Optional[_DecodeOptions]:
    """A smd_decode_options for `kernel` (a KERNEL_* value or its name),
    `merge` (a MERGE_* value or its name) and `qk` (a QK_* value, "bf16" or
    "fp8"), or None for the library's defaults."""
    if kernel is None and merge is None and qk is None:
        return None
    k = 0 if kernel is None else (_KERNELS[kernel] if isinstance(kernel, str) else int(kernel))
    m = 0 if merge is None else (_MERGES[merge] if isinstance(merge, str) else int(merge))
    q = 0 if qk is None else (_QKS[qk] if isinstance(qk, str) else int(qk))
    return _DecodeOptions(kernel=k, merge=m, qk=q)


class PlanModel(ctypes.Structure):
    """Coefficients of the host split planner's cost model (picoseconds)."""

    _fields_ = [
        ("fixed_ps", ctypes.c_int64),
        ("step_ps", ctypes.c_int64),
        ("step_load_ps", ctypes.c_int64),
        ("merge_ps", ctypes.c_int64),
        ("part_ps", ctypes.c_int64),
        ("rows_per_wg", ctypes.c_int32),
        ("waves_per_wg", ctypes.c_int32),
        ("wg_per_cu", ctypes.c_int32),
        ("short_cap", ctypes.c_int32),
        ("long_cap", ctypes.c_int32),
        ("long_kv", ctypes.c_int32),
        ("wide_rows", ctypes.c_int32),
        ("wide_tile", ctypes.c_int32),
        ("wide_fixed_ps", ctypes.c_int64),
        ("wide_tile_ps", ctypes.c_int64),
        ("wide_tile_fp8_ps", ctypes.c_int64),
        ("wide_tile_load_ps", ctypes.c_int64),
        ("wide_cap", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def library_path() -> Path:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libsmd.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m sparse_mla_decode_index_amd.build`")
    L = ctypes.CDLL(str(_LIB_PATH))
    i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    L.smd_last_error.restype = ctypes.c_char_p
    L.smd_last_error.argtypes = []
    L.smd_plan_num_kv_splits.restype = ctypes.c_int
    L.smd_plan_num_kv_splits.argtypes = [i32, i32, i32, i32, i32, i32]
    L.smd_plan_num_kv_splits_model.restype = ctypes.c_int
    L.smd_plan_num_kv_splits_model.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(PlanModel)]
    L.smd_plan_decode.restype = ctypes.c_int
    L.smd_plan_decode.argtypes = [i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(PlanModel),
                                  ctypes.POINTER(i32)]
    L.smd_plan_default_model.restype = ctypes.c_int
    L.smd_plan_default_model.argtypes = [ctypes.POINTER(PlanModel)]
    L.smd_partials_bytes.restype = ctypes.c_size_t
    L.smd_partials_bytes.argtypes = [i32, i32, i32]
    L.smd_split_bounds.restype = ctypes.c_int
    L.smd_split_bounds.argtypes = [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.smd_sparse_mla_decode.restype = ctypes.c_int
    L.smd_sparse_mla_decode.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(_KVPool), vp, i64, i32,
                                        vp, f32, i32, vp, vp, vp, vp, vp]
    L.smd_sparse_mla_decode_ex.restype = ctypes.c_int
    L.smd_sparse_mla_decode_ex.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(_KVPool), vp, i64, i32,
                                           vp, f32, i32, vp, vp, vp, vp, ctypes.POINTER(_DecodeOptions), vp]
    L.smd_sparse_mla_decode_noalloc.restype = ctypes.c_int
    L.smd_sparse_mla_decode_noalloc.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(_KVPool), vp, i64, i32,
                                                vp, f32, i32, vp, vp, ctypes.POINTER(_DecodeOptions), vp]
    L.smd_sparse_mla_decode_two_source.restype = ctypes.c_int
    L.smd_sparse_mla_decode_two_source.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(_KVPool), vp, i64, i32,
                                                   ctypes.POINTER(_KVPool), vp, i64, i32,
                                                   vp, f32, i32, vp, vp, vp, vp, vp]
    L.smd_sparse_mla_decode_two_source_ex.restype = ctypes.c_int
    L.smd_sparse_mla_decode_two_source_ex.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(_KVPool), vp, i64,
                                                      i32, ctypes.POINTER(_KVPool), vp, i64, i32,
                                                      vp, f32, i32, vp, vp, vp, vp,
                                                      ctypes.POINTER(_DecodeOptions), vp]
    L.smd_merge_partials.restype = ctypes.c_int
    L.smd_merge_partials.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp]
    L.smd_write_kv_fp8.restype = ctypes.c_int
    L.smd_write_kv_fp8.argtypes = [vp, i64, i32, vp, ctypes.POINTER(_KVPool), vp]
    L.smd_persistent_default_partitions.restype = i32
    L.smd_persistent_default_partitions.argtypes = [i32, i32, i32]
    L.smd_persistent_workspace_bytes.restype = ctypes.c_size_t
    L.smd_persistent_workspace_bytes.argtypes = [i32, i32, i32]
    L.smd_persistent_workspace_reset.restype = ctypes.c_int
    L.smd_persistent_workspace_reset.argtypes = [vp, ctypes.c_size_t, vp]
    L.smd_sparse_mla_decode_persistent.restype = ctypes.c_int
    L.smd_sparse_mla_decode_persistent.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(_KVPool), vp, vp, vp, f32,
                                                   vp, ctypes.c_size_t, i32, vp, vp, vp]
    L.smd_sparse_mla_decode_persistent_ex.restype = ctypes.c_int
    L.smd_sparse_mla_decode_persistent_ex.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(_KVPool), vp, vp, vp,
                                                      f32, vp, ctypes.c_size_t, i32, vp, vp,
                                                      ctypes.POINTER(_DecodeOptions), vp]
    L.smd_paged_decode.restype = ctypes.c_int
    L.smd_paged_decode.argtypes = [vp, i32, i32, i32, vp, vp, i64, i32, i32, vp, i64, vp, i32, f32, i32, vp, vp, vp,
                                   vp, vp]
    L.smd_paged_num_splits.restype = ctypes.c_int32
    L.smd_paged_num_splits.argtypes = [i32, i32, i32, i32, i32]
    L.smd_decode_kernel_choice.restype = ctypes.c_int32
    L.smd_decode_kernel_choice.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    _lib = L
    return L


def _check(fn: str, rc: int) -> int:
    if rc < 0:
        raise SmdError(fn, rc, lib().smd_last_error().decode())
    return rc


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


# ----------------------------------------------------------------------------
# KV pools
# ----------------------------------------------------------------------------
@dataclass
class KVPool:
    """A latent KV pool on the device: rows of 448 NoPE dims then 64 RoPE dims.

    bf16:  nope bf16 [N, >=448] and rope bf16 [N, >=64] (row-strided views; a
           packed [N, 512] tensor gives nope = kv[:, :448], rope = kv[:, 448:]).
    fp8:   nope uint8 [N, >=448] OCP E4M3FN bytes, scale uint8 [N, >=7] UE8M0
           codes (one per 64-dim NoPE block), rope bf16 [N, >=64].
    """

    dtype: int
    nope: torch.Tensor
    rope: torch.Tensor
    scale: Optional[torch.Tensor] = None

    @staticmethod
    def bf16(kv: torch.Tensor) -> "KVPool":
        _need(kv, "kv", torch.bfloat16)
        if kv.dim() != 2 or kv.shape[1] < DIM or kv.stride(1) != 1:
            raise ValueError("kv must be a row-major [N, 512] bf16 tensor")
        return KVPool(KV_BF16, kv[:, :NOPE], kv[:, NOPE:DIM])

    @staticmethod
    def fp8(nope: torch.Tensor, scale: torch.Tensor, rope: torch.Tensor) -> "KVPool":
        _need(nope, "nope", torch.uint8)
        _need(scale, "scale", torch.uint8)
        _need(rope, "rope", torch.bfloat16)
        return KVPool(KV_FP8_E4M3_UE8M0, nope, rope, scale)

    @property
    def num_rows(self) -> int:
        return self.nope.shape[0]

    @property
    def device(self):
        return self.nope.device

    def _struct(self) -> _KVPool:
        if self.nope.stride(-1) != 1 or self.rope.stride(-1) != 1:
            raise ValueError("pool rows must be contiguous in their last dimension")
        s = _KVPool()
        s.dtype = self.dtype
        s.num_rows = self.num_rows
        s.nope = self.nope.data_ptr()
        s.nope_stride = self.nope.stride(0)
        s.rope = self.rope.data_ptr()
        s.rope_stride = self.rope.stride(0)
        if self.scale is not None:
            if self.scale.stride(-1) != 1:
                raise ValueError("scale rows must be contiguous")
            s.scale = self.scale.data_ptr()
            s.scale_stride = self.scale.stride(0)
        else:
            s.scale = None
            s.scale_stride = 0
        return s


# ----------------------------------------------------------------------------
# planner
# ----------------------------------------------------------------------------
def decode_kernel_choice(num_tokens: int, num_heads: int, q_per_seq: int = 1, num_splits: int = 1,
                         kv_len: int = 0, kv_dtype: int = KV_BF16, two_source: bool = False, kernel=None) -> str:
    """The kernel family ("rows16", "pairs" or "wide") a split-KV call with
    these shapes runs (smd.h smd_decode_kernel_choice); kv_len is the index
    count per index row."""
    k = 0 if kernel is None else (_KERNELS[kernel] if isinstance(kernel, str) else int(kernel))
    rc = lib().smd_decode_kernel_choice(num_tokens, num_heads, q_per_seq, num_splits, kv_len, kv_dtype,
                                        int(bool(two_source)), k)
    _check("smd_decode_kernel_choice", rc)
    return {KERNEL_ROWS16: "rows16", KERNEL_PAIRS: "pairs", KERNEL_WIDE: "wide"}[rc]


def plan_num_kv_splits(num_seqs: int, num_heads: int, kv_len: int, q_per_seq: int = 1,
                       kv_dtype: int = KV_BF16, num_cus: int = 0,
                       model: Optional[PlanModel] = None, two_source: bool = False) -> int:
    """Host split count in [1, 32] from the cost model (no device work)."""
    return plan_decode(num_seqs, num_heads, kv_len, q_per_seq, kv_dtype, num_cus, model, two_source)[0]


def plan_decode(num_seqs: int, num_heads: int, kv_len: int, q_per_seq: int = 1, kv_dtype: int = KV_BF16,
                num_cus: int = 0, model: Optional[PlanModel] = None,
                two_source: bool = False) -> tuple[int, bool]:
    """(split count, whether the wide family won the cost model at that count)
    (smd.h smd_plan_decode; model None = the built-in coefficients)."""
    k = ctypes.c_int32(-1)
    s = _check("smd_plan_decode",
               lib().smd_plan_decode(num_seqs, num_heads, q_per_seq, kv_len, kv_dtype, num_cus,
                                     int(bool(two_source)), ctypes.byref(model) if model is not None else None,
                                     ctypes.byref(k)))
    return s, k.value == KERNEL_WIDE


def partials_bytes(num_tokens: int, num_heads: int, num_splits: int) -> int:
    """Bytes of partial_o + partial_lse for a split-KV call (0 on bad sizes)."""
    return int(lib().smd_partials_bytes(num_tokens, num_heads, num_splits))


def plan_default_model() -> PlanModel:
    m = PlanModel()
    _check("smd_plan_default_model", lib().smd_plan_default_model(ctypes.byref(m)))
    return m


def split_bounds(kv_len: int, num_splits: int, split: int) -> tuple[int, int]:
    b, e = ctypes.c_int32(), ctypes.c_int32()
    _check("smd_split_bounds", lib().smd_split_bounds(kv_len, num_splits, split, ctypes.byref(b),
                                                       ctypes.byref(e)))
    return b.value, e.value


# ----------------------------------------------------------------------------
# decode and merge
# ----------------------------------------------------------------------------
def _decode_buffers(q_nope, q_rope, index_lists, sink, pools, q_per_seq, num_splits, out, lse, partial_o,
                    partial_lse, partials_only, allocate=True):
    """Shared checks and output allocation of the dense-index decodes.  With
    allocate=False nothing is allocated: out must be given, lse and the
    partials are checked only when given."""
    dev = q_nope.device
    _need(q_nope, "q_nope", torch.bfloat16, device=dev)
    if q_nope.dim() != 3 or q_nope.shape[2] != NOPE:
        raise ValueError("q_nope must be [T, H, 448]")
    T, H, _ = q_nope.shape
    _need(q_rope, "q_rope", torch.bfloat16, (T, H, ROPE), dev)
    if not (q_nope.is_contiguous() and q_rope.is_contiguous()):
        raise ValueError("q_nope and q_rope must be contiguous")
    for name, idx in index_lists:
        _need(idx, name, torch.int32, device=dev)
        if idx.dim() != 2 or idx.shape[0] * q_per_seq != T or (idx.shape[1] > 0 and idx.stride(1) != 1):
            raise ValueError(f"{name} must be [T / q_per_seq, K] with unit column stride")
    if sink is not None:
        _need(sink, "sink", torch.float32, (H,), dev)
    for kv in pools:
        if kv.device != dev:
            raise ValueError("kv pool must be on the same device as q")
    K = sum(idx.shape[1] for _, idx in index_lists)
    if num_splits is None:
        num_splits = plan_num_kv_splits(T // q_per_seq, H, K, q_per_seq, pools[0].dtype if K > 0 else KV_BF16,
                                        two_source=len(pools) > 1)
    need_partials = allocate and (partials_only or num_splits > 1)
    if need_partials:
        if partial_o is None:
            partial_o = torch.empty((T, H, num_splits, DIM), dtype=torch.float32, device=dev)
        if partial_lse is None:
            partial_lse = torch.empty((T, H, num_splits), dtype=torch.float32, device=dev)
        _need(partial_o, "partial_o", torch.float32, (T, H, num_splits, DIM), dev)
        _need(partial_lse, "partial_lse", torch.float32, (T, H, num_splits), dev)
    if not partials_only:
        if allocate and out is None:
            out = torch.empty((T, H, DIM), dtype=torch.bfloat16, device=dev)
        if allocate and lse is None:
            lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        if out is None:
            raise ValueError("out is required")
        _need(out, "out", torch.bfloat16, (T, H, DIM), dev)
        if lse is not None:
            _need(lse, "lse", torch.float32, (T, H), dev)
    return T, H, num_splits, out, lse, partial_o, partial_lse


def _idx_args(idx: torch.Tensor):
    K = idx.shape[1]
    return (idx.data_ptr() if idx.numel() else None), (idx.stride(0) if K > 0 else 0), K


def sparse_mla_decode(q_nope: torch.Tensor, q_rope: torch.Tensor, kv: KVPool, indices: torch.Tensor,
                      sink: Optional[torch.Tensor], softmax_scale: float, *,
                      num_splits: Optional[int] = None, q_per_seq: int = 1,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      partial_o: Optional[torch.Tensor] = None,
                      partial_lse: Optional[torch.Tensor] = None,
                      partials_only: bool = False, kernel=None, qk=None):
    """Split-KV sparse MLA decode.

    q_nope bf16 [T,H,448], q_rope bf16 [T,H,64], indices int32 [T/q_per_seq, K]
    (row stride free), sink fp32 [H] or None.  Returns (out, lse) — bf16
    [T,H,512] and fp32 [T,H] — or, with partials_only, (partial_o, partial_lse)
    of shapes [T,H,s,512] and [T,H,s].  num_splits=None asks the host planner.
    kernel: None (the library's choice) or a kernel family ("rows16", "pairs",
    "wide" or a KERNEL_* value).  qk: None / "bf16" (exact) or "fp8" (q_nope
    quantised like the cache, NoPE QK on the block-scaled fp8 MFMA; fp8 pools,
    M a multiple of 128; smd.h SMD_QK_*).
    """
    T, H, num_splits, out, lse, partial_o, partial_lse = _decode_buffers(
        q_nope, q_rope, [("indices", indices)], sink, [kv], q_per_seq, num_splits, out, lse, partial_o,
        partial_lse, partials_only)
    pool = kv._struct()
    opt = _options(kernel, qk=qk)
    rc = lib().smd_sparse_mla_decode_ex(
        q_nope.data_ptr(), q_rope.data_ptr(), T, H, q_per_seq, ctypes.byref(pool), *_idx_args(indices),
        _ptr(sink), float(softmax_scale), num_splits,
        _ptr(partial_o), _ptr(partial_lse),
        None if partials_only else out.data_ptr(), None if partials_only else lse.data_ptr(),
        ctypes.byref(opt) if opt is not None else None, _stream(q_nope))
    _check("smd_sparse_mla_decode", rc)
    if partials_only:
        return partial_o, partial_lse
    return out, lse


def sparse_mla_decode_noalloc(q_nope: torch.Tensor, q_rope: torch.Tensor, kv: KVPool, indices: torch.Tensor,
                              sink: Optional[torch.Tensor], softmax_scale: float, *, out: torch.Tensor,
                              lse: Optional[torch.Tensor] = None, num_splits: Optional[int] = None,
                              q_per_seq: int = 1, kernel=None, qk=None):
    """sparse_mla_decode through the allocation-free entry point: the FP32
    partials of a split plan stay in the library's per-GPU scratch array
    (NOALLOC_SCRATCH_BYTES), so neither this call nor the library allocates.
    out (bf16 [T,H,512]) must be given; lse (fp32 [T,H]) is optional; kernel
    and qk as in sparse_mla_decode."""
    T, H, num_splits, out, lse, _, _ = _decode_buffers(q_nope, q_rope, [("indices", indices)], sink, [kv], q_per_seq,
                                                       num_splits, out, lse, None, None, partials_only=False,
                                                       allocate=False)
    pool = kv._struct()
    opt = _options(kernel, qk=qk)
    rc = lib().smd_sparse_mla_decode_noalloc(
        q_nope.data_ptr(), q_rope.data_ptr(), T, H, q_per_seq, ctypes.byref(pool), *_idx_args(indices),
        _ptr(sink), float(softmax_scale), num_splits, out.data_ptr(), _ptr(lse),
        ctypes.byref(opt) if opt is not None else None, _stream(q_nope))
    _check("smd_sparse_mla_decode_noalloc", rc)
    return out, lse


def sparse_mla_decode_two_source(q_nope: torch.Tensor, q_rope: torch.Tensor, main_kv: KVPool,
                                 main_indices: torch.Tensor, swa_kv: KVPool, swa_indices: torch.Tensor,
                                 sink: Optional[torch.Tensor], softmax_scale: float, *,
                                 num_splits: Optional[int] = None, q_per_seq: int = 1,
                                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                                 partial_o: Optional[torch.Tensor] = None,
                                 partial_lse: Optional[torch.Tensor] = None,
                                 partials_only: bool = False, kernel=None):
    """Two-source decode: main_indices [T/q_per_seq, K_main] index main_kv,
    swa_indices [T/q_per_seq, K_swa] index swa_kv, all one softmax (main
    positions first).  Pools of the same dtype and strides.  Outputs as
    sparse_mla_decode (kernel likewise); the planner sees K_main + K_swa
    positions."""
    T, H, num_splits, out, lse, partial_o, partial_lse = _decode_buffers(
        q_nope, q_rope, [("main_indices", main_indices), ("swa_indices", swa_indices)], sink, [main_kv, swa_kv],
        q_per_seq, num_splits, out, lse, partial_o, partial_lse, partials_only)
    mp, sp = main_kv._struct(), swa_kv._struct()
    opt = _options(kernel)
    rc = lib().smd_sparse_mla_decode_two_source_ex(
        q_nope.data_ptr(), q_rope.data_ptr(), T, H, q_per_seq, ctypes.byref(mp), *_idx_args(main_indices),
        ctypes.byref(sp), *_idx_args(swa_indices), _ptr(sink), float(softmax_scale), num_splits,
        _ptr(partial_o), _ptr(partial_lse),
        None if partials_only else out.data_ptr(), None if partials_only else lse.data_ptr(),
        ctypes.byref(opt) if opt is not None else None, _stream(q_nope))
    _check("smd_sparse_mla_decode_two_source", rc)
    if partials_only:
        return partial_o, partial_lse
    return out, lse


def write_kv_fp8(kv: torch.Tensor, pool: KVPool, slots: Optional[torch.Tensor] = None) -> None:
    """fp8/UE8M0 cache writer: bf16 latent rows kv [n, 512] (unit column
    stride) into the fp8 pool's arrays, row r to pool row slots[r] (int32 [n];
    None: row r; rows outside the pool are skipped)."""
    _need(kv, "kv", torch.bfloat16, device=pool.device)
    if kv.dim() != 2 or kv.shape[1] != DIM or kv.stride(1) != 1:
        raise ValueError("kv must be [n, 512] bf16 with unit column stride")
    if pool.dtype != KV_FP8_E4M3_UE8M0:
        raise ValueError("write_kv_fp8 writes into an fp8 pool")
    n = kv.shape[0]
    if slots is not None:
        _need(slots, "slots", torch.int32, (n,), pool.device)
    st = pool._struct()
    rc = lib().smd_write_kv_fp8(kv.data_ptr() if n else None, kv.stride(0) if n else DIM, n, _ptr(slots),
                                ctypes.byref(st), _stream(kv))
    _check("smd_write_kv_fp8", rc)


def merge_partials(partial_o: torch.Tensor, partial_lse: torch.Tensor, sink: Optional[torch.Tensor], *,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Stage-2 merge of FP32 partials [T,H,s,512] + [T,H,s] into bf16 out and fp32 lse."""
    dev = partial_o.device
    _need(partial_o, "partial_o", torch.float32, device=dev)
    if partial_o.dim() != 4 or partial_o.shape[3] != DIM or not partial_o.is_contiguous():
        raise ValueError("partial_o must be contiguous [T, H, s, 512]")
    T, H, S, _ = partial_o.shape
    _need(partial_lse, "partial_lse", torch.float32, (T, H, S), dev)
    if not partial_lse.is_contiguous():
        raise ValueError("partial_lse must be contiguous")
    if sink is not None:
        _need(sink, "sink", torch.float32, (H,), dev)
    if out is None:
        out = torch.empty((T, H, DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, (T, H, DIM), dev)
    _need(lse, "lse", torch.float32, (T, H), dev)
    rc = lib().smd_merge_partials(partial_o.data_ptr(), partial_lse.data_ptr(), T, H, S, _ptr(sink),
                                  out.data_ptr(), lse.data_ptr(), _stream(partial_o))
    _check("smd_merge_partials", rc)
    return out, lse



# ----------------------------------------------------------------------------
# persistent, graph-safe decode over ragged sequences
# ----------------------------------------------------------------------------
def persistent_default_partitions(num_heads: int, q_per_seq: int = 1, num_cus: int = 0) -> int:
    """Partitions that fill num_cus CUs once (num_cus=0: 256)."""
    return _check("smd_persistent_default_partitions",
                  lib().smd_persistent_default_partitions(num_heads, q_per_seq, num_cus))


def persistent_workspace_bytes(num_heads: int, q_per_seq: int, num_partitions: int) -> int:
    n = lib().smd_persistent_workspace_bytes(num_heads, q_per_seq, num_partitions)
    if n == 0:
        raise SmdError("smd_persistent_workspace_bytes", -1, lib().smd_last_error().decode())
    return n


class PersistentWorkspace:
    """Device workspace of the persistent decode: allocated with torch and zeroed
    once (do both outside graph capture).  Calls sharing it must be ordered on
    the GPU; the kernel resets its counters itself, so it can be reused across
    batch sizes and graph replays."""

    def __init__(self, num_heads: int, q_per_seq: int = 1, num_partitions: Optional[int] = None,
                 device=None):
        dev = torch.device(device if device is not None else "cuda")
        self.num_heads, self.q_per_seq = num_heads, q_per_seq
        self.num_partitions = num_partitions or persistent_default_partitions(num_heads, q_per_seq)
        self.nbytes = persistent_workspace_bytes(num_heads, q_per_seq, self.num_partitions)
        self.buffer = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=dev)
        off = (-self.buffer.data_ptr()) % 256
        self.view = self.buffer[off:off + self.nbytes]
        _check("smd_persistent_workspace_reset",
               lib().smd_persistent_workspace_reset(self.view.data_ptr(), self.nbytes, _stream(self.view)))

    def plan(self) -> torch.Tensor:
        """The plan region: int32 [P, 4] = (t0, t1, first sequence, last sequence)."""
        return self.view[:16 * self.num_partitions].view(torch.int32).view(self.num_partitions, 4)


def sparse_mla_decode_persistent(q_nope: torch.Tensor, q_rope: torch.Tensor, kv: KVPool,
                                 kv_indptr: torch.Tensor, kv_indices: torch.Tensor,
                                 sink: Optional[torch.Tensor], softmax_scale: float, *,
                                 q_per_seq: int = 1, workspace: PersistentWorkspace,
                                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                                 merge=None, qk=None):
    """Persistent decode over ragged sequences: q bf16 [B*q_per_seq, H, 448/64],
    kv_indptr int32 [B+1], kv_indices int32 flat.  Returns (out, lse); rows of
    sequences with no index are left as they were in `out` / `lse`.  merge:
    None / "auto" or "workspace" (smd.h SMD_MERGE_*; both give the same bits).
    qk: None / "bf16" or "fp8" (as in sparse_mla_decode; fp8 pools, M a
    multiple of 128)."""
    dev = q_nope.device
    _need(q_nope, "q_nope", torch.bfloat16, device=dev)
    if q_nope.dim() != 3 or q_nope.shape[2] != NOPE:
        raise ValueError("q_nope must be [T, H, 448]")
    T, H, _ = q_nope.shape
    _need(q_rope, "q_rope", torch.bfloat16, (T, H, ROPE), dev)
    if not (q_nope.is_contiguous() and q_rope.is_contiguous()):
        raise ValueError("q_nope and q_rope must be contiguous")
    if T % q_per_seq:
        raise ValueError("the token count must be a multiple of q_per_seq")
    B = T // q_per_seq
    _need(kv_indptr, "kv_indptr", torch.int32, (B + 1,), dev)
    _need(kv_indices, "kv_indices", torch.int32, device=dev)
    if not (kv_indptr.is_contiguous() and kv_indices.is_contiguous()):
        raise ValueError("kv_indptr and kv_indices must be contiguous")
    if sink is not None:
        _need(sink, "sink", torch.float32, (H,), dev)
    if kv.device != dev:
        raise ValueError("kv pool must be on the same device as q")
    if (workspace.num_heads, workspace.q_per_seq) != (H, q_per_seq):
        raise ValueError("workspace was sized for other shapes")
    if out is None:
        out = torch.empty((T, H, DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, (T, H, DIM), dev)
    _need(lse, "lse", torch.float32, (T, H), dev)
    pool = kv._struct()
    opts = _options(merge=merge, qk=qk)
    rc = lib().smd_sparse_mla_decode_persistent_ex(
        q_nope.data_ptr(), q_rope.data_ptr(), B, q_per_seq, H, ctypes.byref(pool), kv_indptr.data_ptr(),
        kv_indices.data_ptr() if kv_indices.numel() else kv_indptr.data_ptr(), _ptr(sink), float(softmax_scale),
        workspace.view.data_ptr(), workspace.nbytes, workspace.num_partitions, out.data_ptr(), lse.data_ptr(),
        ctypes.byref(opts) if opts is not None else None, _stream(q_nope))
    _check("smd_sparse_mla_decode_persistent", rc)
    return out, lse

def paged_num_splits(num_seqs: int, num_kv_heads: int, max_context_len: int, page_size: int,
                     num_cus: int = 0) -> int:
    """Split count for paged_decode (smd.h smd_paged_num_splits)."""
    return _check("smd_paged_num_splits",
                  lib().smd_paged_num_splits(num_seqs, num_kv_heads, max_context_len, page_size, num_cus))


def paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                 context_lens: torch.Tensor, max_context_len: int, softmax_scale: float, *, mtp: int = 1,
                 num_splits: Optional[int] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, partial_o: Optional[torch.Tensor] = None,
                 partial_lse: Optional[torch.Tensor] = None, partials_only: bool = False):
    """Dense paged GQA decode (smd.h smd_paged_decode): q bf16 [B*mtp, Hq, 512],
    caches bf16 [num_blocks, page, Hkv, 512], block_tables int32 [B, >= pages],
    context_lens int32 [B].  Returns (out, lse), or with partials_only
    (partial_o, partial_lse) of shapes [T, Hq, s, 512] and [T, Hq, s]."""
    dev = q.device
    _need(q, "q", torch.bfloat16, device=dev)
    if q.dim() != 3 or q.shape[2] != DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B * mtp, Hq, 512] tensor")
    T, Hq, _ = q.shape
    if T % mtp:
        raise ValueError("the token count must be a multiple of mtp")
    B = T // mtp
    for name, c in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(c, name, torch.bfloat16, device=dev)
        if c.dim() != 4 or c.shape[3] != DIM or not c.is_contiguous() or c.shape != k_cache.shape:
            raise ValueError(f"{name} must be a contiguous [num_blocks, page, Hkv, 512] tensor like k_cache")
    nblk, page, Hkv, _ = k_cache.shape
    _need(block_tables, "block_tables", torch.int32, device=dev)
    _need(context_lens, "context_lens", torch.int32, (B,), dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be [B, pages] with unit column stride")
    if num_splits is None:
        num_splits = paged_num_splits(B, Hkv, max_context_len, page)
    s = num_splits
    need_partials = partials_only or s > 1
    if need_partials:
        if partial_o is None:
            partial_o = torch.empty((T, Hq, s, DIM), dtype=torch.float32, device=dev)
        if partial_lse is None:
            partial_lse = torch.empty((T, Hq, s), dtype=torch.float32, device=dev)
        _need(partial_o, "partial_o", torch.float32, (T, Hq, s, DIM), dev)
        _need(partial_lse, "partial_lse", torch.float32, (T, Hq, s), dev)
    if not partials_only:
        if out is None:
            out = torch.empty((T, Hq, DIM), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
        _need(out, "out", torch.bfloat16, (T, Hq, DIM), dev)
        _need(lse, "lse", torch.float32, (T, Hq), dev)
    rc = lib().smd_paged_decode(q.data_ptr(), B, mtp, Hq, k_cache.data_ptr(), v_cache.data_ptr(), nblk, page, Hkv,
                                block_tables.data_ptr(), block_tables.stride(0), context_lens.data_ptr(),
                                int(max_context_len), float(softmax_scale), s, _ptr(partial_o), _ptr(partial_lse),
                                None if partials_only else out.data_ptr(), None if partials_only else lse.data_ptr(),
                                _stream(q))
    _check("smd_paged_decode", rc)
    if partials_only:
        return partial_o, partial_lse
    return out, lse


__all__ = ["KVPool", "PlanModel", "SmdError", "plan_num_kv_splits", "plan_decode", "plan_default_model",
           "split_bounds", "partials_bytes", "write_kv_fp8", "sparse_mla_decode", "sparse_mla_decode_noalloc",
           "sparse_mla_decode_two_source", "merge_partials", "persistent_default_partitions",
           "persistent_workspace_bytes", "PersistentWorkspace", "sparse_mla_decode_persistent", "lib",
           "library_path", "KV_BF16", "KV_FP8_E4M3_UE8M0", "QK_BF16", "QK_FP8", "paged_decode",
           "paged_num_splits"]

if os.environ.get("SMD_EAGER_LOAD") == "1":
    lib()

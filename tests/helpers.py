"""Shared test helpers: moving seeded workloads to the device and comparing
the HIP results with the oracle at the documented tolerances."""
from __future__ import annotations

import numpy as np
import torch

import sparse_mla_decode_index_amd as smd

# Tolerances (see the design notes): bf16 out atol = rtol = 2e-2; FP32 partials
# rtol = 1e-3 with atol = 1e-3 * max |oracle row|; LSE |d| <= 1e-3 * max(1, |lse|).
OUT_ATOL = OUT_RTOL = 2e-2
PART_RTOL = 1e-3
LSE_TOL = 1e-3


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def pool_to_device(w, device) -> smd.KVPool:
    a = w.arrays
    if w.kv_dtype == "bf16":
        return smd.KVPool.bf16(bf16_tensor(a["kv"], device))
    return smd.KVPool.fp8(torch.from_numpy(a["nope"]).to(device), torch.from_numpy(a["scale"]).to(device),
                          bf16_tensor(a["rope"], device))


def oracle_pool(w) -> dict:
    a = w.arrays
    if w.kv_dtype == "bf16":
        return {"kv": a["kv"]}
    return {"nope": a["nope"], "scale": a["scale"], "rope": a["rope"]}


def device_inputs(w, device):
    a = w.arrays
    q_nope = bf16_tensor(a["q_nope"], device)
    q_rope = bf16_tensor(a["q_rope"], device)
    sink = torch.from_numpy(a["sink"]).to(device)
    pool = pool_to_device(w, device)
    return q_nope, q_rope, sink, pool


def check_out(out_gpu: torch.Tensor, out_ref: np.ndarray, what: str = "out"):
    g = out_gpu.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - out_ref)
    bad = err > OUT_ATOL + OUT_RTOL * np.abs(out_ref)
    assert not np.isnan(g).any(), f"{what}: NaN in GPU output"
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; "
                           f"max abs err {err.max():.3e}")
    return err.max()


def check_lse(lse_gpu: torch.Tensor, lse_ref: np.ndarray, what: str = "lse"):
    g = lse_gpu.cpu().numpy().astype(np.float64)
    both_inf = np.isneginf(g) & np.isneginf(lse_ref)
    err = np.where(both_inf, 0.0, np.abs(g - lse_ref))
    tol = LSE_TOL * np.maximum(1.0, np.abs(np.where(np.isfinite(lse_ref), lse_ref, 0.0)))
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} out of tolerance; max err {np.nanmax(err):.3e}"
    return np.nanmax(err) if err.size else 0.0


def check_partials(po_gpu, pl_gpu, po_ref, pl_ref):
    g = po_gpu.cpu().numpy().astype(np.float64)
    rowmax = np.abs(po_ref).max(axis=-1, keepdims=True)
    err = np.abs(g - po_ref)
    bad = err > PART_RTOL * np.abs(po_ref) + PART_RTOL * rowmax
    assert not np.isnan(g).any(), "partial_o: NaN"
    assert not bad.any(), f"partial_o: {bad.sum()} of {bad.size} out of tolerance; max err {err.max():.3e}"
    check_lse(pl_gpu, pl_ref, "partial_lse")

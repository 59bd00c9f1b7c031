"""Host-side plumbing for the GPU parity tests: moving seeded inputs to the
device in the library's padded layout and reading results back.  No step of
the method's arithmetic lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def say(*a):
    """Names the case before a GPU step (flushed, so it survives a crash)."""
    print(*a, file=sys.stderr, flush=True)


def to_dev_dense(x: np.ndarray, dtype: str = "f32"):
    """fp32 values, or bf16 bit patterns (uint16), into a padded device tensor."""
    import sparse_aggregation_gemm_amd as sag
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x, np.uint16).view(np.int16)).view(torch.bfloat16)
        td = torch.bfloat16
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
        td = torch.float32
    out = sag.empty_dense(x.shape[0], x.shape[1], td, DEV)
    out.copy_(t.to(DEV))
    return out


def to_dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor (fp32 or bf16) as exact float64 on the host."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def elementwise_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / |ref| over the entries with |ref| >= 1e-3 max |ref|
    (reported beside the bound-relative error; not a gate)."""
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    sel = np.abs(ref) >= 1e-3 * np.abs(ref).max()
    if not np.any(sel):
        return 0.0
    return float(np.max(np.abs(np.asarray(got, np.float64)[sel] - ref[sel]) / np.abs(ref[sel])))


def tol(dtype: str) -> float:
    """Error bound relative to the magnitude of the summed terms: fp32 1e-5;
    bf16 inputs with fp32 accumulation 2e-2."""
    return 1e-5 if dtype == "f32" else 2e-2


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values as the stored type's bits/values (input encoding only)."""
    import gen
    if dtype == "bf16":
        return gen.f32_to_bf16_bits(np.asarray(x, np.float32))
    return np.asarray(x, np.float32)

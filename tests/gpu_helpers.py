"""Helpers for the GPU parity tests: padded device copies, NaN-sentinel
outputs, and the two parity gates against the CPU oracle.

Gate for integer-valued inputs: bit-exact (+0 and -0 compare equal).
Gate for fp32 inputs: |C - C_ref| <= 1e-4 * sum_k |a_ik| |b_kj| per element,
no NaN, where C_ref and the sum of magnitudes come from the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

REL_TOL = 1e-4


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says which."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def padded_buffer(view: torch.Tensor) -> torch.Tensor:
    """The (rows x pitch) buffer behind a row-pitched CPU view."""
    rows, cols = view.shape
    pitch = view.stride(0) if rows > 1 else cols
    if pitch == cols:
        return view.contiguous()
    return torch.as_strided(view, (rows, pitch), (pitch, 1))


def to_device(view: torch.Tensor, device="cuda", offset: int = 0) -> torch.Tensor:
    """Copy a row-pitched CPU view to the GPU keeping its pitch.  ``offset``
    shifts the base by that many floats (to make it unaligned)."""
    rows, cols = view.shape
    buf = padded_buffer(view)
    pitch = buf.shape[1] if buf.dim() == 2 else cols
    flat = torch.full((rows * pitch + offset + 4,), float("nan"), dtype=torch.float32)
    flat[offset:offset + rows * pitch] = buf.reshape(-1)
    d = flat.to(device)
    return torch.as_strided(d, (rows, cols), (pitch, 1), storage_offset=offset)


def sentinel_output(M: int, N: int, ldc: int | None = None, device="cuda", offset: int = 0):
    """C (M x N, pitch ldc) inside a NaN-filled buffer; returns (view, flat buffer)."""
    ldc = N if ldc is None else ldc
    flat = torch.full((max(M, 1) * max(ldc, 1) + offset + 8,), float("nan"),
                      dtype=torch.float32, device=device)
    view = torch.as_strided(flat, (M, N), (max(ldc, 1), 1), storage_offset=offset)
    return view, flat


def window_mask(M, N, ldc, offset, total):
    """Boolean mask over the flat buffer: True inside the written window."""
    m = np.zeros(total, dtype=bool)
    for i in range(M):
        m[offset + i * ldc: offset + i * ldc + N] = True
    return m


def check_outside_untouched(flat: torch.Tensor, M, N, ldc, offset=0):
    f = flat.cpu().numpy()
    mask = window_mask(M, N, ldc, offset, f.size)
    outside = f[~mask]
    assert np.all(np.isnan(outside)), "a kernel wrote outside the M x N window of C"


def oracle_of(A_cpu: torch.Tensor, B_cpu: torch.Tensor):
    C, Cd, ABS = oracle.gemm(A_cpu.numpy(), B_cpu.numpy())
    return C, ABS


def assert_bitexact(C_gpu: np.ndarray, C_ref: np.ndarray, what: str = ""):
    assert C_gpu.shape == C_ref.shape
    bad = ~(C_gpu == C_ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} elements differ from the oracle on integer "
                             f"inputs, e.g. at {idx.tolist()}: gpu={C_gpu[tuple(idx[0])]}, "
                             f"oracle={C_ref[tuple(idx[0])]}")


def assert_within_tol(C_gpu: np.ndarray, C_ref: np.ndarray, ABS: np.ndarray, what: str = ""):
    assert C_gpu.shape == C_ref.shape
    assert not np.isnan(C_gpu).any(), f"{what}: NaN in the GPU result"
    err = np.abs(C_gpu.astype(np.float64) - C_ref.astype(np.float64))
    ok = err <= REL_TOL * ABS
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        i = tuple(idx[0])
        raise AssertionError(f"{what}: {(~ok).sum()} elements outside 1e-4*sum|a||b|, e.g. at "
                             f"{idx.tolist()}: gpu={C_gpu[i]}, oracle={C_ref[i]}, "
                             f"scale={ABS[i]}")
    return float(np.max(np.where(ABS > 0, err / np.where(ABS > 0, ABS, 1), 0)))

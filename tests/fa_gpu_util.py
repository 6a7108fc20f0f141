"""Helpers for the GPU parity tests: run libfa on seeded inputs and compare with
the oracle. The oracle side only ever sees the host inputs; nothing it uses
comes back from the GPU.
"""
from __future__ import annotations

import os

import numpy as np

import oracle

TOL_F32 = 1e-4     # max |gpu - oracle| on unit-scale data, fp32 KV cache
TOL_Q4 = 2e-4      # same, Q4_0 KV cache (oracle on the same dequantised K/V)
ORACLE_THREADS = min(16, os.cpu_count() or 1)


# Parity figures of this session (max |gpu - oracle| per compared output);
# tests/conftest.py prints them in the terminal summary, passing tests included.
PARITY_LINES: list[str] = []


def log(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)


def device():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def oracle_kv(fmt: int, k_rows: np.ndarray, head_dim: int) -> np.ndarray:
    """Cache view the oracle attends over: rows [rows][n_kv][hd] -> [n_kv][rows][hd],
    quantised and dequantised by the oracle itself for Q4_0."""
    if fmt == 1:
        k_rows = oracle.q4_dequantize(oracle.q4_quantize(k_rows), head_dim)
    return np.ascontiguousarray(k_rows.transpose(1, 0, 2))


def compare_rows(gpu: np.ndarray, ref: np.ndarray, tol: float, what: str) -> float:
    """max-abs bar plus the argmax rule over each output row (lowest index
    wins ties; rows whose oracle top-2 margin is within 2*tol are near-ties and
    are only reported)."""
    gpu = gpu.reshape(-1, gpu.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = float(np.abs(gpu - ref).max())
    assert err <= tol, f"{what}: max|gpu-oracle| = {err:.3e} > {tol:.1e}"
    srt = np.sort(ref, axis=1)
    margin = srt[:, -1] - srt[:, -2]
    decided = margin > 2 * tol
    am_g = np.argmax(gpu, axis=1)
    am_r = np.argmax(ref, axis=1)
    bad = np.nonzero(decided & (am_g != am_r))[0]
    assert bad.size == 0, f"{what}: argmax differs on rows {bad[:8]}"
    near = int((~decided).sum())
    line = f"{what}: max_abs={err:.3e} (bar {tol:.0e}) rows={gpu.shape[0]} near_ties={near}"
    PARITY_LINES.append(line)
    log(line)
    return err


def sample_positions(n: int, rng: np.random.Generator, extra=(), count: int = 48) -> np.ndarray:
    base = set(range(min(n, 6))) | set(range(max(0, n - 6), n))
    base |= {p for p in extra if 0 <= p < n}
    base |= set(rng.integers(0, n, size=count).tolist())
    return np.array(sorted(base), dtype=np.int64)

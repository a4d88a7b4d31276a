"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""

import os
import sys

import numpy as np
import pytest
import torch

# Tolerances: absolute, over every valid element, against the fp64 oracle.
TOL_O_BF16 = 2e-2     # bf16 storage, fp32 accumulation
TOL_O_F32 = 1e-5      # fp32 end to end
TOL_LSE = 1e-3


def device():
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU on this host")
    from io_aware_attention_02_amd import load_library
    load_library()  # raises if the HIP library is missing: no silent fallback
    return torch.device("cuda:0")


def f64(t):
    """Exact upcast of a (bf16 / fp32) torch tensor to a float64 numpy array."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def tile_rows(N, tile, head, seed=0, edges=True):
    """Query rows that reach every `tile`-row query tile: one row per tile, drawn per head (so the
    heads of a grid see different rows), plus the tile edges 0, tile - 1, tile and N - 1."""
    g = np.random.default_rng(1000 * seed + head)
    rows = {min(N - 1, t + int(g.integers(0, tile))) for t in range(0, N, tile)}
    if edges:
        rows |= {r for r in (0, tile - 1, tile, N - 1) if 0 <= r < N}
    return sorted(rows)

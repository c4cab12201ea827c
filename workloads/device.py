"""The calibration-input recipes of the workloads, drawn on the GPU.

Same recipes as ``make_x_chunk`` (the same distribution parameters, taken from
the same seeded host draws: the low-rank mixing matrix and outlier channels, the
power-law spectrum, signs, 3 x 3 rotation and permutation), but the per-row
random numbers come from torch's device generator instead of numpy's, so the
values differ from the host recipe's while following the same law.  The host
recipe needs minutes per 16384-row chunk at the 11008- and 49152-wide shapes
(about 160 s for the power-law recipe at 49152 columns); this one takes
milliseconds, which lets whole 262144-row calibration sets stream through a GPU
test.  Like the rest of this package it holds none of the solver's arithmetic.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from . import CHUNK_ROWS, T_X, LayerSpec, _lowrank_params, _powerlaw_params


def _generator(spec: LayerSpec, chunk: int, device) -> torch.Generator:
    seed = np.random.SeedSequence([1, spec.workload, spec.layer, T_X, chunk]).generate_state(1, np.uint64)[0]
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & ((1 << 63) - 1))
    return g


def _fwht_last(y: torch.Tensor) -> torch.Tensor:
    """Unnormalised Walsh-Hadamard transform along the last axis (length 2^m)."""
    n = y.shape[-1]
    h = 1
    while h < n:
        v = y.reshape(*y.shape[:-1], n // (2 * h), 2, h)
        a, b = v[..., 0, :], v[..., 1, :]
        y = torch.stack((a + b, a - b), dim=-2).reshape(*y.shape[:-1], n)
        h *= 2
    return y


def make_x_chunk_device(spec: LayerSpec, chunk: int, rows: Optional[int] = None,
                        device="cuda") -> torch.Tensor:
    """Rows of X for chunk ``chunk`` as a device tensor [rows x d_col] in the
    layer's dtype, by the layer's recipe (fp32 arithmetic, one rounding to the
    stored dtype at the end)."""
    d = spec.d_col
    start = chunk * CHUNK_ROWS
    nr = rows if rows is not None else min(CHUNK_ROWS, spec.n_rows - start)
    if nr <= 0:
        raise ValueError("chunk out of range")
    g = _generator(spec, chunk, device)
    dt = torch.float16 if spec.x_dtype == "f16" else torch.float32
    if spec.x_kind == "lowrank":
        a, ch = _lowrank_params(spec)
        z = torch.randn(nr, a.shape[0], generator=g, device=device)
        x = z @ torch.from_numpy(a.astype(np.float32)).to(device)
        chd = torch.from_numpy(ch).to(device)
        x[:, chd] *= 20.0
    elif spec.x_kind == "silu":
        a = torch.randn(nr, d, generator=g, device=device)
        b = torch.randn(nr, d, generator=g, device=device)
        x = a * torch.sigmoid(a) * b
    elif spec.x_kind == "powerlaw":
        m, s, signs, q3, perm = _powerlaw_params(spec)
        scale = torch.from_numpy((s * signs).astype(np.float32)).to(device)
        y = (torch.randn(nr, d, generator=g, device=device) * scale).reshape(nr, 3, 1 << m)
        # the 3 x 3 rotation across the three Hadamard blocks, as plain sums
        y = torch.stack([sum(float(q3[a, b]) * y[:, b] for b in range(3)) for a in range(3)], dim=1)
        y = _fwht_last(y) * (2.0 ** (-m / 2.0))
        x = torch.empty(nr, d, device=device)
        x[:, torch.from_numpy(perm).to(device)] = y.reshape(nr, d)
    else:
        raise ValueError(f"no device recipe for {spec.x_kind}")
    return x.to(dt)

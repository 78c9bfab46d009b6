"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module only draws random numbers and rounds them to the storage dtype; it holds
none of the method's arithmetic.  Every tensor is drawn from numpy's PCG64 generator
seeded by ``SeedSequence(seed, spawn_key=key + (block,))``, one stream per block of
``BLOCK_ROWS`` leading-dimension rows, so any row range of a tensor can be regenerated
on its own (sampled oracle checks of large problems regenerate only the rows they read).

Values are drawn as float32 standard normals, multiplied by the requested standard
deviation in float32 and rounded to the storage dtype (bf16 by round-to-nearest-even
through torch's CPU conversion).  The same stored bytes go to the GPU and, widened to
float64, to the oracle.
"""

from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np
import torch

BLOCK_ROWS = 2048

_TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name):
    return _TORCH_DTYPES[name]


def _generator(seed, key):
    ss = np.random.SeedSequence(int(seed), spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def gaussian(seed, key, shape, std=1.0, dtype="bf16", rows=None):
    """N(0, std^2) tensor of ``shape`` in storage dtype ``dtype`` on the CPU.

    rows=(r0, r1) returns only leading-dimension rows [r0, r1) -- bit-identical to the
    same slice of the full tensor.
    """
    shape = tuple(int(s) for s in shape)
    n_rows = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    r0, r1 = (0, n_rows) if rows is None else (int(rows[0]), int(rows[1]))
    assert 0 <= r0 <= r1 <= n_rows
    out = torch.empty((r1 - r0,) + shape[1:], dtype=_TORCH_DTYPES[dtype])
    if r1 == r0 or inner == 0:
        return out
    flat = out.view(r1 - r0, inner)
    std32 = np.float32(std)
    blocks = range(r0 // BLOCK_ROWS, (r1 - 1) // BLOCK_ROWS + 1)

    def fill(b):
        b0 = b * BLOCK_ROWS
        b1 = min(n_rows, b0 + BLOCK_ROWS)
        vals = np.empty((b1 - b0, inner), dtype=np.float32)
        _generator(seed, tuple(key) + (b,)).standard_normal(out=vals, dtype=np.float32)
        if std32 != np.float32(1.0):
            vals *= std32
        lo, hi = max(b0, r0), min(b1, r1)
        flat[lo - r0:hi - r0].copy_(torch.from_numpy(vals[lo - b0:hi - b0]))

    if len(blocks) == 1:
        fill(blocks[0])
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, blocks))
    return out


def integers(seed, key, low, high, size):
    """Integers uniform in [low, high] (inclusive), as int32."""
    return _generator(seed, key).integers(low, high + 1, size=size).astype(np.int32)


def to_f64(t):
    """Exact float64 view of stored values, for the oracle."""
    return t.to(torch.float64).numpy()

"""Helpers for the GPU-vs-checker parity tests (tolerances and comparisons)."""
from __future__ import annotations

import sys

import numpy as np

# Output tolerances of the layer: bf16 inputs -> max-abs 2e-2 and relative L2
# 5e-3; the float32 configuration -> 1e-5 for both.
TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-5, 1e-5)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in GPU result"
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(name, got, ref, max_abs, rel_l2):
    ma, rl = errors(got, ref)
    log("  %-28s max-abs %.3e (<= %.1e)  rel-L2 %.3e (<= %.1e)" % (name, ma, max_abs, rl, rel_l2))
    assert ma <= max_abs and rl <= rel_l2, "%s: max-abs %.3e rel-L2 %.3e" % (name, ma, rl)


def to_gpu(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()

"""Comparison metrics for parity checks (test infrastructure).

Acceptance scale: output relative RMS <= 5e-3 and max abs <= 2e-2, final-state relative RMS <= 1e-4, each
taken jointly over all compared elements of one call.
"""
from __future__ import annotations

import numpy as np

OUT_REL_RMS = 5e-3
OUT_MAX_ABS = 2e-2
STATE_REL_RMS = 1e-4


class Accum:
    """Streams sum(err^2), sum(ref^2) and max|err| over several blocks of one comparison."""

    def __init__(self):
        self.se = 0.0
        self.sr = 0.0
        self.mx = 0.0
        self.n = 0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        if got.size == 0:
            return
        e = got - ref
        self.se += float(np.sum(e * e))
        self.sr += float(np.sum(ref * ref))
        self.mx = max(self.mx, float(np.max(np.abs(e))))
        self.n += got.size

    def merge(self, other):
        """Fold in another Accum of the same comparison (e.g. a later batch of units)."""
        self.se += other.se
        self.sr += other.sr
        self.mx = max(self.mx, other.mx)
        self.n += other.n
        return self

    @property
    def rel_rms(self):
        if self.sr == 0.0:
            return 0.0 if self.se == 0.0 else float("inf")
        return (self.se / self.sr) ** 0.5

    @property
    def max_abs(self):
        return self.mx

    def __repr__(self):
        return f"Accum(n={self.n}, rel_rms={self.rel_rms:.3e}, max_abs={self.max_abs:.3e})"


def rel_rms(got, ref):
    a = Accum()
    a.add(got, ref)
    return a.rel_rms


def max_abs(got, ref):
    a = Accum()
    a.add(got, ref)
    return a.max_abs

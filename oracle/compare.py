"""Comparison metrics for parity checks (test infrastructure; only tests, the smoke check and the bench's CPU
baseline use this package).

The acceptance metrics are the two the prefill page reports for its accuracy comparison ("[Lightning
Attention] Add Hopper SM90 CuTe DSL prefill", Accuracy vs original C++ implementation): output max abs and
relative RMS, and the final state's relative RMS. Bars: output relative RMS <= 5e-3 and max abs <= 2e-2,
final-state relative RMS <= 1e-4.

    rel RMS = sqrt( sum (got - ref)^2 / sum ref^2 )        max abs = max |got - ref|

Each bar is applied twice: jointly over every compared element of a call, and separately to every unit
(a (sequence, value head) pair of outputs, or one state plane) that the caller names, so that a unit with small
values cannot hide its error under the joint sums of larger ones. NaN and Inf are never dropped: a NaN anywhere
makes rel RMS and max abs NaN, an Inf makes them Inf, and both fail every bar.
"""
from __future__ import annotations

import math

import numpy as np

OUT_REL_RMS = 5e-3
OUT_MAX_ABS = 2e-2
STATE_REL_RMS = 1e-4


def _max_nan(a: float, b: float) -> float:
    """max(a, b) that returns NaN when either side is NaN (Python's max() keeps whichever it saw first)."""
    return float(np.maximum(a, b))


def _rel(se: float, sr: float) -> float:
    if math.isnan(se) or math.isnan(sr):
        return float("nan")
    if sr == 0.0:
        return 0.0 if se == 0.0 else float("inf")
    return math.sqrt(se / sr)


class Accum:
    """Streams sum(err^2), sum(ref^2) and max|err| over blocks of one comparison. Blocks added with a `unit` key
    also keep their own sums, so that the bars can be checked per unit (`worst_unit`)."""

    def __init__(self):
        self.se = 0.0
        self.sr = 0.0
        self.mx = 0.0
        self.n = 0
        self.units = {}          # unit key -> [se, sr, mx, n]

    def add(self, got, ref, unit=None):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        if got.size == 0:
            return
        e = got - ref
        se = float(np.sum(e * e))
        sr = float(np.sum(ref * ref))
        mx = float(np.max(np.abs(e)))
        self.se += se
        self.sr += sr
        self.mx = _max_nan(self.mx, mx)
        self.n += got.size
        if unit is not None:
            u = self.units.setdefault(unit, [0.0, 0.0, 0.0, 0])
            u[0] += se
            u[1] += sr
            u[2] = _max_nan(u[2], mx)
            u[3] += got.size

    def merge(self, other):
        """Fold in another Accum of the same comparison (e.g. a later batch of units)."""
        self.se += other.se
        self.sr += other.sr
        self.mx = _max_nan(self.mx, other.mx)
        self.n += other.n
        for key, (se, sr, mx, n) in other.units.items():
            u = self.units.setdefault(key, [0.0, 0.0, 0.0, 0])
            u[0] += se
            u[1] += sr
            u[2] = _max_nan(u[2], mx)
            u[3] += n
        return self

    @property
    def rel_rms(self):
        return _rel(self.se, self.sr)

    @property
    def max_abs(self):
        return self.mx

    def unit_rel_rms(self, unit):
        se, sr, _, _ = self.units[unit]
        return _rel(se, sr)

    def worst_unit(self):
        """(key, rel RMS) of the unit with the largest relative RMS (NaN ranks above everything), or None."""
        worst = None
        for key in self.units:
            r = self.unit_rel_rms(key)
            rank = math.inf if math.isnan(r) else r
            if worst is None or rank > worst[2]:
                worst = (key, r, rank)
        return None if worst is None else (worst[0], worst[1])

    def __repr__(self):
        w = self.worst_unit()
        tail = "" if w is None else f", worst unit {w[0]} rel_rms={w[1]:.3e}"
        return f"Accum(n={self.n}, rel_rms={self.rel_rms:.3e}, max_abs={self.max_abs:.3e}{tail})"


def within(value: float, bar: float) -> bool:
    """value <= bar, false for NaN."""
    return bool(value <= bar)


def output_ok(acc: Accum) -> bool:
    """Output bars: joint rel RMS and max abs, and rel RMS of every named unit."""
    if not (within(acc.rel_rms, OUT_REL_RMS) and within(acc.max_abs, OUT_MAX_ABS)):
        return False
    w = acc.worst_unit()
    return w is None or within(w[1], OUT_REL_RMS)


def state_ok(acc: Accum) -> bool:
    """Final-state bar: joint rel RMS and rel RMS of every named plane."""
    if not within(acc.rel_rms, STATE_REL_RMS):
        return False
    w = acc.worst_unit()
    return w is None or within(w[1], STATE_REL_RMS)


def rel_rms(got, ref):
    a = Accum()
    a.add(got, ref)
    return a.rel_rms


def max_abs(got, ref):
    a = Accum()
    a.add(got, ref)
    return a.max_abs

"""Pins of the parity comparator (oracle/compare.py), CPU only.

Every acceptance number in the GPU tests passes through this comparator, so it is pinned on hand-computed
values -- relative RMS sqrt(sum e^2 / sum ref^2) and max |e| worked out by hand for tiny vectors -- and on the
behaviour the bars need: NaN and Inf fail, streaming in batches equals one pass, and one unit with a large
relative error fails the check even when the joint sums over all units pass. Planted mistakes in a copy of the
comparator's source (a dropped square root, a swallowed NaN, a wrong denominator, a dropped absolute value,
per-unit sums ignored or lost in a merge) must each fail at least one pin.
"""
import importlib.util
import math
import types

import numpy as np
import pytest

import oracle.compare as compare


def _pins(m):
    """Run every pin against comparator module m; return the names of the pins that fail."""
    failed = []

    def pin(name, cond):
        try:
            ok = bool(cond())
        except Exception:       # a mutant may raise instead of returning a wrong value
            ok = False
        if not ok:
            failed.append(name)

    def acc(got, ref, unit=None):
        a = m.Accum()
        a.add(np.array(got, np.float64), np.array(ref, np.float64), unit=unit)
        return a

    # e = [0, 2]: sum e^2 = 4, sum ref^2 = 2 -> rel RMS sqrt(2); max |e| = 2
    pin("hand_sqrt2", lambda: math.isclose(acc([1, 3], [1, 1]).rel_rms, math.sqrt(2.0), rel_tol=1e-15))
    pin("hand_max", lambda: acc([1, 3], [1, 1]).max_abs == 2.0)
    # e = [0, -3]: the largest magnitude is a negative error
    pin("hand_abs", lambda: acc([1, -2], [1, 1]).max_abs == 3.0)
    # got = 2 ref: sum e^2 = sum ref^2 = 25 -> rel RMS exactly 1 (the denominator is the reference)
    pin("hand_denominator", lambda: acc([6, 8], [3, 4]).rel_rms == 1.0)
    # got = 0: rel RMS exactly 1 whatever the reference
    pin("hand_zero_got", lambda: acc([0, 0], [3, 4]).rel_rms == 1.0)
    # e = [0.5, 0.5, 0.5, 0.5] on ref of ones: sqrt(1 / 4) = 0.5
    pin("hand_half", lambda: acc([1.5, 0.5, 1.5, 0.5], [1, 1, 1, 1]).rel_rms == 0.5)
    # an all-zero reference: exact agreement is 0, any error is infinite
    pin("zero_ref_exact", lambda: acc([0, 0], [0, 0]).rel_rms == 0.0)
    pin("zero_ref_error", lambda: math.isinf(acc([1e-3, 0], [0, 0]).rel_rms))
    # streaming: two batches merged equal one add (integers, so the sums are exact)
    def merged():
        a = acc([1, 2, 7], [1, 1, 1])
        b = acc([4, 5], [2, 9])
        one = acc([1, 2, 7, 4, 5], [1, 1, 1, 2, 9])
        a.merge(b)
        return a.se == one.se and a.sr == one.sr and a.mx == one.mx and a.n == one.n
    pin("merge_equals_one_pass", merged)
    # NaN and Inf in the result fail every bar
    pin("nan_max_abs", lambda: math.isnan(acc([float("nan"), 1], [1, 1]).max_abs))
    pin("nan_rel_rms", lambda: math.isnan(acc([float("nan"), 1], [1, 1]).rel_rms))
    pin("nan_fails_output", lambda: not m.output_ok(acc([float("nan"), 1], [1, 1])))
    pin("nan_merge", lambda: math.isnan(acc([1], [1]).merge(acc([float("nan")], [1])).max_abs))
    pin("nan_after_large", lambda: math.isnan(acc([5, float("nan")], [1, 1]).max_abs))
    pin("inf_fails_output", lambda: not m.output_ok(acc([float("inf"), 1], [1, 1])))
    pin("inf_fails_state", lambda: not m.state_ok(acc([float("inf"), 1], [1, 1])))

    # per-unit bar: a unit at 1e-1 relative error with |o| = 0.1 hides under the joint sums of a large unit
    def hidden_unit():
        a = m.Accum()
        a.add(np.full(1000, 100.0), np.full(1000, 100.0), unit=("big", 0))
        a.add(np.full(100, 0.11), np.full(100, 0.1), unit=("small", 1))
        joint_passes = a.rel_rms <= m.OUT_REL_RMS and a.max_abs <= m.OUT_MAX_ABS
        w = a.worst_unit()
        return (joint_passes and not m.output_ok(a) and w[0] == ("small", 1)
                and math.isclose(w[1], 0.1, rel_tol=1e-12))
    pin("per_unit_catches_hidden_error", hidden_unit)

    def per_unit_after_merge():
        a = m.Accum()
        a.add(np.full(1000, 100.0), np.full(1000, 100.0), unit=("big", 0))
        b = m.Accum()
        b.add(np.full(100, 0.11), np.full(100, 0.1), unit=("small", 1))
        a.merge(b)
        return not m.output_ok(a)
    pin("per_unit_survives_merge", per_unit_after_merge)

    def state_plane():
        a = m.Accum()
        a.add(np.ones(4096), np.ones(4096), unit=(0, 0))
        a.add(np.full(4, 1.001), np.ones(4), unit=(0, 1))      # 1e-3 relative on one plane
        return a.rel_rms < m.STATE_REL_RMS and not m.state_ok(a)
    pin("per_plane_state", state_plane)

    def nan_unit_is_worst():
        a = m.Accum()
        a.add([1.0, 2.0], [1.0, 1.0], unit="a")
        a.add([float("nan")], [1.0], unit="b")
        return a.worst_unit()[0] == "b"
    pin("nan_unit_is_worst", nan_unit_is_worst)
    # a passing comparison passes
    pin("clean_passes", lambda: m.output_ok(acc([1.001, 2.002], [1.0, 2.0], unit=0))
        and m.state_ok(acc([1.0, 2.0], [1.0, 2.0], unit=0)))
    return failed


def test_comparator_pins():
    assert _pins(compare) == []


def test_bars_are_the_acceptance_values():
    assert (compare.OUT_REL_RMS, compare.OUT_MAX_ABS, compare.STATE_REL_RMS) == (5e-3, 2e-2, 1e-4)


MUTANTS = {
    "sqrt_dropped": ("return math.sqrt(se / sr)", "return se / sr"),
    "nan_swallowed": ("return float(np.maximum(a, b))", "return max(a, b)"),
    "nan_swallowed_by_nanmax": ("mx = float(np.max(np.abs(e)))", "mx = float(np.nanmax(np.abs(e)))"),
    "denominator_got": ("sr = float(np.sum(ref * ref))", "sr = float(np.sum(got * got))"),
    "abs_dropped": ("mx = float(np.max(np.abs(e)))", "mx = float(np.max(e))"),
    "per_unit_ignored": ("return w is None or within(w[1], OUT_REL_RMS)", "return True"),
    "state_planes_ignored": ("return w is None or within(w[1], STATE_REL_RMS)", "return True"),
    "merge_drops_units": ("        for key, (se, sr, mx, n) in other.units.items():",
                          "        for key, (se, sr, mx, n) in {}.items():"),
    "rel_rms_nan_to_zero": ("        return float(\"nan\")\n    if sr == 0.0:", "        return 0.0\n    if sr == 0.0:"),
}


def _mutant(name, patch):
    src = open(compare.__file__).read()
    old, new = patch
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType(f"compare_mutant_{name}")
    exec(compile(src.replace(old, new), f"<{name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_comparator_mistake_fails_a_pin(name):
    failed = _pins(_mutant(name, MUTANTS[name]))
    assert failed, f"mutant {name} passed every pin"


def test_unmodified_source_through_the_mutant_loader_passes():
    spec = importlib.util.spec_from_file_location("compare_copy", compare.__file__)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _pins(mod) == []

"""Planted mistakes in the oracle (CPU only): each mutant of oracle/la_oracle.c must fail at least one pin.

Every mutant is a plausible slip in the recurrence -- a dropped term, a wrong operand, a transposed state, a
decay applied at the wrong point, a wrong GVA head. The test builds the mutant from a copy of the source in a
temporary directory and runs a small pin battery against it: the closed form from the verify page, the
lambda = 1 and lambda = 0 special cases, the hand example and the GVA mapping. The unmodified source must
pass the same battery.
"""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from la_synth import bf16_bits, bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MUTANTS = {
    "decay_after_add": ("row[d] = lambda * row[d] + vt[e] * kt[d];", "row[d] = lambda * (row[d] + vt[e] * kt[d]);"),
    "output_uses_k": ("acc += row[d] * qt[d];", "acc += row[d] * kt[d];"),
    "scale_dropped": ("= scale * acc;", "= acc;"),
    "gva_modulo": ("const int32_t h = hv / G;", "const int32_t h = hv % H;"),
    "decay_by_qk_head": ("exp(-(double)slope[hv])", "exp(-(double)slope[h])"),
    "output_before_update": ("row[d] = lambda * row[d] + vt[e] * kt[d];\n                    acc += row[d] * qt[d];",
                             "acc += row[d] * qt[d];\n                    row[d] = lambda * row[d] + vt[e] * kt[d];"),
    "s0_transposed": ("memcpy(S, s0 + (size_t)u * DV * D, sizeof(double) * (size_t)DV * D);",
                      "for (int32_t a = 0; a < DV * D; ++a) S[a] = s0[(size_t)u * DV * D + (size_t)(a % D) * DV + a / D];"),
    "last_token_dropped": ("t < len[u]; ++t)", "t + 1 < len[u]; ++t)"),
    "decay_squared": ("const double lambda = exp(-(double)slope[hv]);",
                      "const double lambda = exp(-2.0 * (double)slope[hv]);"),
}


def _build(tmp_path, name, patch):
    src = open(oracle.SRC_PATH).read()
    if patch is not None:
        old, new = patch
        assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(c), "-o", str(so), "-lm"])
    return oracle.load(str(so))


def _f64(bits):
    return bits_to_f32(bits).astype(np.float64)


def _battery(L):
    """Return the list of failed pin names for oracle build L."""
    failed = []
    rng = np.random.default_rng(77)
    T, D, DV = 70, 12, 8
    q = bf16_bits(rng.standard_normal((T, 1, D)).astype(np.float32) * 0.3)
    k = bf16_bits(rng.standard_normal((T, 1, D)).astype(np.float32) * 0.3)
    v = bf16_bits(rng.standard_normal((T, 1, DV)).astype(np.float32))
    s0 = rng.standard_normal((DV, D))
    Q, K, V = _f64(q[:, 0]), _f64(k[:, 0]), _f64(v[:, 0])

    def run(slope, scale, s, qq=q, kk=k, vv=v, H=1, HV=1, units=None):
        units = units or [(0, qq.shape[0], 0)]
        return oracle.tokenwise(qq, kk, vv, H, HV, scale, np.asarray(slope, np.float32), units,
                                s0=None if s is None else np.stack([s] * len(units)), _with=L)

    def close(a, b, tol=1e-10):
        return np.allclose(a, b, rtol=tol, atol=tol * max(1.0, float(np.abs(b).max())))

    # closed form, two decays, scale != 1
    for slope in (0.05, 0.3):
        outs, sf = run([slope], 0.7, s0)
        lam = float(np.exp(-np.float64(np.float32(slope))))
        o_ref, s_ref = oracle.closed_form(Q, K, V, lam, 0.7, s0)
        if not (close(outs[0], o_ref) and close(sf[0], s_ref)):
            failed.append(f"closed_form[{slope}]")
    # lambda = 1
    outs, sf = run([0.0], 1.0, s0)
    if not (close(outs[0], np.tril(Q @ K.T) @ V + Q @ s0.T) and close(sf[0], s0 + V.T @ K)):
        failed.append("lambda_one")
    # lambda = 0
    outs, sf = run([np.inf], 1.0, s0)
    if not (close(outs[0], np.sum(Q * K, 1)[:, None] * V) and close(sf[0], np.outer(V[-1], K[-1]))):
        failed.append("lambda_zero")
    # hand example
    g = json.load(open(os.path.join(GOLDEN, "t1_hand.json")))
    gq = bf16_bits(np.array(g["q"], np.float32)[None, None])
    gk = bf16_bits(np.array(g["k"], np.float32)[None, None])
    gv = bf16_bits(np.array(g["v"], np.float32)[None, None])
    outs, sf = run([g["slope"]], g["scale"], np.array(g["S0"]), qq=gq, kk=gk, vv=gv)
    if not (np.allclose(outs[0][0], g["o"], atol=1e-6) and np.allclose(sf[0], g["S1"], atol=1e-6)):
        failed.append("hand_example")
    # GVA: each value head against its own single-head run with q/k head hv // G
    H, G = 2, 2
    q2 = bf16_bits(rng.standard_normal((20, H, D)).astype(np.float32) * 0.3)
    k2 = bf16_bits(rng.standard_normal((20, H, D)).astype(np.float32) * 0.3)
    v2 = bf16_bits(rng.standard_normal((20, H * G, DV)).astype(np.float32))
    sl = np.array([0.01, 0.1, 0.2, 0.4], np.float32)
    outs, _ = run(sl, 1.0, None, qq=q2, kk=k2, vv=v2, H=H, HV=H * G, units=[(0, 20, hv) for hv in range(4)])
    for hv in range(4):
        h = hv // G
        o_ref, _ = oracle.closed_form(_f64(q2[:, h]), _f64(k2[:, h]), _f64(v2[:, hv]),
                                      float(np.exp(-np.float64(sl[hv]))), 1.0, np.zeros((DV, D)))
        if not close(outs[hv], o_ref):
            failed.append(f"gva[{hv}]")
            break
    return failed


def test_unmodified_oracle_passes_battery(tmp_path):
    assert _battery(_build(tmp_path, "clean", None)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    failed = _battery(_build(tmp_path, name, MUTANTS[name]))
    assert failed, f"mutant {name} passed every pin"

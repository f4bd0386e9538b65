"""CPU oracle for the Lightning Attention forward (prefill) path.

TEST INFRASTRUCTURE ONLY: the plain, slow definition the HIP path is checked against. Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import this package. It shares no code with the HIP
library and never imports it.

Sources (the pages are cited by title):
  * "[LA] Lightning Attention MTP decode + KVBuffer parallel verify / commit" -- Description (the closed form
    o_t = a^{t+1} (h0 q_t scale) + sum_{i<=t} a^{t-i} (q_t . k_i scale) v_i of a draft output, and the commit by
    an accepted length) and Tests (the edge cases of the commit).
  * "[Lightning Attention] Add Hopper SM90 CuTe DSL prefill" -- Description (dtypes, head sizes, chunk length,
    state handling, head grouping, pool indices, packed input) and Reviewer notes (the state's precision and
    orientation, and the properties its tests cover).

Three independent evaluations live here:
  * ``tokenwise`` -- the recurrence S <- lambda S + v k^T, o = scale S q, token by token in FP64 (C/OpenMP,
    la_oracle.c). This is THE oracle.
  * ``closed_form`` -- the O(T^2) sum printed on the verify page, NumPy FP64. Used to pin ``tokenwise``.
  * ``chunked`` -- the 64-token chunked algorithm (intra-chunk decay-masked Q K^T V, inter-chunk Q S^T, state
    update lambda^Lc S + V^T diag(lambda^{Lc-1-i}) K), NumPy FP64. Pins the chunk algebra against
    ``tokenwise``.

On top of ``tokenwise``, ``prefill`` / ``commit`` give the boundary semantics: pool slots, negative or
out-of-range index = zero initial state and no write, READ/WRITE flags, accepted-length commit.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblaoracle.so")
SRC_PATH = os.path.join(HERE, "la_oracle.c")

STATE_READ = 1
STATE_WRITE = 2
DECAY_PER_QK_HEAD = 4

_lib = None


def build(force: bool = True) -> str:
    """Compile la_oracle.c with plain gcc -O2 and OpenMP (no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", SRC_PATH, "-o", tmp, "-lm"]
        )
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def load(path: str):
    """Load an oracle shared library (the default one, or a test-built variant) and declare its ABI."""
    L = ctypes.CDLL(path)
    p = ctypes.c_void_p
    L.la_oracle_fwd.restype = ctypes.c_int
    L.la_oracle_fwd.argtypes = [p, p, p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_double, p, ctypes.c_int32, p, p, p, p, p, p, p]
    L.la_oracle_threads.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load(LIB_PATH)
    return _lib


def threads() -> int:
    return int(lib().la_oracle_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------------------------------------
# bf16 helpers (inputs arrive as uint16 bit patterns; widening is exact)
# ---------------------------------------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------------------------
# THE oracle: tokenwise FP64 recurrence
# ---------------------------------------------------------------------------------------------------------
def tokenwise(q_bits, k_bits, v_bits, H, HV, scale, slope, units, s0=None, want_o=True, _with=None):
    """Evaluate units = [(row0, length, hv), ...] with the tokenwise FP64 recurrence.

    q_bits/k_bits: uint16 [rows, H, D]; v_bits: uint16 [rows, HV, DV]; slope: float32 [HV].
    s0: float64 [nunits, DV, D] or None (zero). Returns (list of float64 [length, DV] outputs or None,
    float64 [nunits, DV, D] final states). ``_with`` substitutes another build of la_oracle.c (tests only).
    """
    k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
    D = k_bits.shape[-1]
    DV = v_bits.shape[-1]
    n = len(units)
    row0 = np.ascontiguousarray([u[0] for u in units], dtype=np.int64)
    lens = np.ascontiguousarray([u[1] for u in units], dtype=np.int64)
    hvs = np.ascontiguousarray([u[2] for u in units], dtype=np.int32)
    off = np.zeros(n, dtype=np.int64)
    if n:
        off[1:] = np.cumsum(lens)[:-1]
    total = int(lens.sum())
    o = np.empty((max(total, 1), DV), dtype=np.float64) if want_o else None
    s_fin = np.empty((n, DV, D), dtype=np.float64)
    s0c = None if s0 is None else np.ascontiguousarray(s0, dtype=np.float64)
    qc = np.ascontiguousarray(q_bits, dtype=np.uint16) if want_o else None
    slope = np.ascontiguousarray(slope, dtype=np.float32)
    rc = (_with or lib()).la_oracle_fwd(_ptr(qc), _ptr(k_bits), _ptr(v_bits), H, HV, D, DV, float(scale), _ptr(slope), n,
                             _ptr(row0), _ptr(lens), _ptr(hvs), _ptr(s0c), _ptr(o), _ptr(off), _ptr(s_fin))
    if rc != 0:
        raise ValueError("la_oracle_fwd rejected its arguments")
    outs = None
    if want_o:
        outs = [o[off[i]:off[i] + lens[i]] for i in range(n)]
    return outs, s_fin


# ---------------------------------------------------------------------------------------------------------
# Independent evaluations used to pin the oracle
# ---------------------------------------------------------------------------------------------------------
def closed_form(q, k, v, lam, scale, s0):
    """O(T^2) closed form from the verify page, one unit, all FP64.

    q, k: [T, D]; v: [T, DV]; s0: [DV, D] ([V, K] orientation).
    o_t = scale * (lam^{t+1} S0 q_t + sum_{i<=t} lam^{t-i} (q_t . k_i) v_i)
    S_T = lam^T S0 + sum_{i<T} lam^{T-1-i} v_i k_i^T
    """
    T = q.shape[0]
    t = np.arange(T)
    diff = t[:, None] - t[None, :]
    w = np.where(diff >= 0, np.power(lam, np.maximum(diff, 0).astype(np.float64)), 0.0)
    scores = (q @ k.T) * w
    o = scale * (scores @ v + np.power(lam, (t + 1).astype(np.float64))[:, None] * (q @ s0.T))
    wk = np.power(lam, (T - 1 - t).astype(np.float64))
    s_T = np.power(lam, float(T)) * s0 + v.T @ (wk[:, None] * k)
    return o, s_T


def chunked(q, k, v, lam, scale, s0, C=64):
    """Chunked form of the same recurrence, one unit, all FP64.

    Per chunk of Lc <= C tokens with state S before the chunk (local positions j, i in [0, Lc)):
      O_c = scale * ( (Q K^T o M) V + diag(lam^{j+1}) Q S^T ),  M_ji = lam^{j-i} for i <= j else 0
      S   <- lam^{Lc} S + V^T diag(lam^{Lc-1-i}) K
    A short last chunk uses its own Lc in both exponents.
    """
    T = q.shape[0]
    S = s0.astype(np.float64).copy()
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        Lc = min(C, T - c0)
        Qc, Kc, Vc = q[c0:c0 + Lc], k[c0:c0 + Lc], v[c0:c0 + Lc]
        j = np.arange(Lc)
        diff = j[:, None] - j[None, :]
        M = np.where(diff >= 0, np.power(lam, np.maximum(diff, 0).astype(np.float64)), 0.0)
        inter = np.power(lam, (j + 1).astype(np.float64))[:, None] * (Qc @ S.T)
        o[c0:c0 + Lc] = scale * (((Qc @ Kc.T) * M) @ Vc + inter)
        kdec = np.power(lam, (Lc - 1 - j).astype(np.float64))[:, None] * Kc
        S = np.power(lam, float(Lc)) * S + Vc.T @ kdec
    return o, S


# ---------------------------------------------------------------------------------------------------------
# Boundary semantics on top of the tokenwise oracle
# ---------------------------------------------------------------------------------------------------------
def _slot_ok(idx, P):
    return 0 <= idx < P


def prefill(q_bits, k_bits, v_bits, seq_row0, seq_len, H, HV, scale, slope, pool=None, state_idx=None,
            flags=0, units=None, state_idx_out=None):
    """Prefill over sequences (fixed-length: row0 = b*T, len = T; packed: from cu_seqlens).

    pool: float32 [P, HV, DV, D] or None; state_idx: int [nseq] or None; flags: STATE_READ | STATE_WRITE
    (| DECAY_PER_QK_HEAD). units: list of (seq, hv) to evaluate (default: all). Returns (dict (seq, hv) ->
    float64 [len, DV] output, pool_after: float64 copy of the pool with the evaluated units' writes applied, or
    None). A slot index < 0 or >= P means zero initial state and no write. A zero-length sequence writes its
    initial state (S0, or zero without READ) when WRITE is set.

    state_idx_out (int [nseq], optional): the slot that receives sequence n's final state, in place of
    state_idx[n] (prefill page, comparison notes: indirect / shared state-pool ownership). Every read happens
    before any write, as when each sequence's reads and writes touch slots no other sequence writes.
    DECAY_PER_QK_HEAD: slope has H entries, one per q/k head, and value head hv decays with slope[hv // G]
    (prefill page, Performance: GVA rows with decay owned per q/k head, "_h"); this is the same recurrence as
    per-value-head slopes that repeat each q/k head's slope G times.
    """
    if flags & DECAY_PER_QK_HEAD:
        slope = np.repeat(np.asarray(slope, np.float32), HV // H)
    nseq = len(seq_len)
    if units is None:
        units = [(n, hv) for n in range(nseq) for hv in range(HV)]
    P = 0 if pool is None else pool.shape[0]
    D = k_bits.shape[-1]
    DV = v_bits.shape[-1]
    s0 = np.zeros((len(units), DV, D))
    for i, (n, hv) in enumerate(units):
        s = -1 if state_idx is None else int(state_idx[n])
        if (flags & STATE_READ) and pool is not None and _slot_ok(s, P):
            s0[i] = pool[s, hv].astype(np.float64)
    spec = [(int(seq_row0[n]), int(seq_len[n]), hv) for (n, hv) in units]
    outs, s_fin = tokenwise(q_bits, k_bits, v_bits, H, HV, scale, slope, spec, s0=s0, want_o=True)
    pool_after = None if pool is None else pool.astype(np.float64)
    dst = state_idx if state_idx_out is None else state_idx_out
    for i, (n, hv) in enumerate(units):
        s = -1 if dst is None else int(dst[n])
        if (flags & STATE_WRITE) and pool is not None and _slot_ok(s, P):
            pool_after[s, hv] = s_fin[i]
    return {u: outs[i] for i, u in enumerate(units)}, pool_after


def commit(k_bits, v_bits, B, T, H, HV, slope, pool, state_idx, accepted_len, units=None):
    """Advance pooled states by per-request accepted length L (verify page, state-update commit).

    S <- lambda^L S + sum_{i<L} lambda^{L-1-i} v_i k_i^T over request b's first L tokens (rows b*T ...).
    Slot < 0 or >= P: skipped. L = 0: no write at all (the slot stays bitwise as it was).
    Returns a float64 copy of the pool with the evaluated units' writes applied.
    """
    if units is None:
        units = [(b, hv) for b in range(B) for hv in range(HV)]
    P = pool.shape[0]
    pool_after = pool.astype(np.float64)
    todo = [(b, hv) for (b, hv) in units
            if _slot_ok(int(state_idx[b]), P) and int(accepted_len[b]) > 0]
    if not todo:
        return pool_after
    s0 = np.stack([pool[int(state_idx[b]), hv].astype(np.float64) for (b, hv) in todo])
    spec = [(b * T, int(accepted_len[b]), hv) for (b, hv) in todo]
    _, s_fin = tokenwise(None, k_bits, v_bits, H, HV, 1.0, slope, spec, s0=s0, want_o=False)
    for i, (b, hv) in enumerate(todo):
        pool_after[int(state_idx[b]), hv] = s_fin[i]
    return pool_after

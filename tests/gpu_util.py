"""Helpers for the GPU parity tests: move a synthetic workload to the device, run the HIP path through the
C-ABI binding, and evaluate the same units with the FP64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import linear_attention_decay_amd as la
import oracle
from oracle.compare import OUT_MAX_ABS, OUT_REL_RMS, STATE_REL_RMS, Accum, within

DEV = torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t if dtype is None else t.view(dtype)


class DevWorkload:
    """Device copies of a la_synth.Workload (q/k/v as bf16 tensors)."""

    def __init__(self, w):
        self.w = w
        self.q = to_dev(w.q, torch.bfloat16)
        self.k = to_dev(w.k, torch.bfloat16)
        self.v = to_dev(w.v, torch.bfloat16)
        self.slope = to_dev(w.slope)
        self.pool0 = None if w.pool is None else to_dev(w.pool)
        self.idx = None if w.state_idx is None else to_dev(w.state_idx)
        self.cu = None if w.cu_seqlens is None else to_dev(w.cu_seqlens)
        self.acc = None if w.accepted_len is None else to_dev(w.accepted_len)

    def fresh_pool(self):
        return None if self.pool0 is None else self.pool0.clone()

    def new_out(self, poison=True):
        o = torch.empty_like(self.v)
        if poison:
            o.fill_(float("nan"))
        return o

    def prefill(self, o=None, pool=None, flags=None, schedule=la.LA_SCHED_AUTO, stream=None, scale=None):
        w = self.w
        o = self.new_out() if o is None else o
        pool = self.fresh_pool() if pool is None else pool
        flags = w.flags if flags is None else flags
        scale = w.scale if scale is None else scale
        idx = self.idx if flags else self.idx
        if w.cu_seqlens is None:
            la.la_prefill_fwd(self.q, self.k, self.v, o, self.slope, scale=scale, state_pool=pool, state_idx=idx,
                              flags=flags, stream=stream)
        else:
            la.la_prefill_fwd_varlen(self.q, self.k, self.v, o, self.cu, self.slope, scale=scale, state_pool=pool,
                                     state_idx=idx, flags=flags, schedule=schedule, stream=stream)
        return o, pool

    def commit(self, pool):
        la.la_state_commit(self.k, self.v, self.slope, pool, self.idx, self.acc)
        return pool


def flat_rows(w, a):
    """View q/k/v/o-shaped arrays as [rows, heads, 128]."""
    return a.reshape(-1, a.shape[-2], a.shape[-1])


def oracle_prefill(w, units=None, flags=None, scale=None):
    rows = w.seq_rows()
    return oracle.prefill(flat_rows(w, w.q), flat_rows(w, w.k), flat_rows(w, w.v), [r for r, _ in rows],
                          [n for _, n in rows], w.H, w.HV, w.scale if scale is None else scale, w.slope,
                          pool=w.pool, state_idx=w.state_idx, flags=w.flags if flags is None else flags,
                          units=units)


def compare_prefill(w, o_dev, pool_dev, units=None, flags=None, scale=None):
    """Compare the GPU output/pool with the oracle on `units` (default all). Returns (out Accum, state Accum).

    Also checks that pool planes nobody selected are bitwise unchanged."""
    flags = w.flags if flags is None else flags
    ref_o, ref_pool = oracle_prefill(w, units=units, flags=flags, scale=scale)
    got = flat_rows(w, o_dev.float().cpu().numpy())
    rows = w.seq_rows()
    out = Accum()
    for (n, hv), ref in ref_o.items():
        r0, L = rows[n]
        out.add(got[r0:r0 + L, hv], ref, unit=(n, hv))
    st = Accum()
    if pool_dev is not None:
        pool_got = pool_dev.cpu().numpy()
        P = w.pool.shape[0]
        selected = set()
        if flags & la.LA_STATE_WRITE:
            for n in range(w.nseq):
                s = int(w.state_idx[n])
                if 0 <= s < P:
                    selected.add(s)
        for s in range(P):
            if s not in selected:
                assert np.array_equal(pool_got[s].view(np.uint32), w.pool[s].view(np.uint32)), f"slot {s} touched"
        checked = set()
        for (n, hv) in ref_o:
            s = int(w.state_idx[n]) if w.state_idx is not None else -1
            if (flags & la.LA_STATE_WRITE) and 0 <= s < P and (s, hv) not in checked:
                checked.add((s, hv))
                st.add(pool_got[s, hv], ref_pool[s, hv], unit=(s, hv))
    return out, st


def assert_parity(out, st=None, what=""):
    """Joint bars over the whole call, then the same relative-RMS bar for every unit the Accums name (a (sequence,
    value head) output unit, a (slot, value head) state plane). NaN fails every bar."""
    assert within(out.rel_rms, OUT_REL_RMS), f"{what} output rel RMS {out.rel_rms:.3e} > {OUT_REL_RMS}"
    assert within(out.max_abs, OUT_MAX_ABS), f"{what} output max abs {out.max_abs:.3e} > {OUT_MAX_ABS}"
    w = out.worst_unit()
    if w is not None:
        assert within(w[1], OUT_REL_RMS), f"{what} output unit {w[0]} rel RMS {w[1]:.3e} > {OUT_REL_RMS}"
    if st is not None and st.n:
        assert within(st.rel_rms, STATE_REL_RMS), f"{what} state rel RMS {st.rel_rms:.3e} > {STATE_REL_RMS}"
        w = st.worst_unit()
        if w is not None:
            assert within(w[1], STATE_REL_RMS), f"{what} state plane {w[0]} rel RMS {w[1]:.3e} > {STATE_REL_RMS}"


def add_state_slot(st, got, ref, slot):
    """Add the HV planes of one pool slot to a state Accum, one unit per (slot, value head) plane."""
    for hv in range(ref.shape[0]):
        st.add(got[hv], ref[hv], unit=(slot, hv))


def assert_state(st, what=""):
    """Final-state bar, jointly and per plane."""
    assert st.n, f"{what}: no state compared"
    assert within(st.rel_rms, STATE_REL_RMS), f"{what} state rel RMS {st.rel_rms:.3e} > {STATE_REL_RMS}"
    w = st.worst_unit()
    if w is not None:
        assert within(w[1], STATE_REL_RMS), f"{what} state plane {w[0]} rel RMS {w[1]:.3e} > {STATE_REL_RMS}"


def bitwise_equal(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))

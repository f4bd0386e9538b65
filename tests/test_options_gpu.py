"""GPU parity of the API variants: separate out slots (la_prefill_fwd_ex / la_prefill_fwd_varlen_ex) and decay owned
per q/k head (LA_DECAY_PER_QK_HEAD), on the chunked and the short-sequence kernels, against the FP64 oracle.

Tolerances as for the main path (output rel RMS <= 5e-3, max abs <= 2e-2, state rel RMS <= 1e-4); slots that no
sequence writes are checked bitwise, and per-q/k-head decay is also checked bitwise against the same call with
the slopes repeated per value head.
"""
import numpy as np
import pytest
import torch

import la_synth
import linear_attention_decay_amd as la
import oracle
from gpu_util import DevWorkload, add_state_slot, assert_parity, bitwise_equal, to_dev
from oracle.compare import Accum

pytestmark = pytest.mark.gpu


def _compare(w, o_dev, pool_dev, flags, idx_out, slope):
    rows = w.seq_rows()
    ref_o, ref_pool = oracle.prefill(w.q.reshape(-1, w.H, 128), w.k.reshape(-1, w.H, 128), w.v.reshape(-1, w.HV, 128),
                                     [r for r, _ in rows], [n for _, n in rows], w.H, w.HV, w.scale, slope,
                                     pool=w.pool, state_idx=w.state_idx, flags=flags, state_idx_out=idx_out)
    got = o_dev.float().cpu().numpy().reshape(-1, w.HV, 128)
    out = Accum()
    for (n, hv), ref in ref_o.items():
        r0, L = rows[n]
        out.add(got[r0:r0 + L, hv], ref, unit=(n, hv))
    st = Accum()
    pool_got = pool_dev.cpu().numpy()
    P = w.pool.shape[0]
    written = {int(s) for s in idx_out if 0 <= int(s) < P} if flags & la.LA_STATE_WRITE else set()
    for s in range(P):
        if s in written:
            add_state_slot(st, pool_got[s], ref_pool[s], s)
        else:
            assert np.array_equal(pool_got[s].view(np.uint32), w.pool[s].view(np.uint32)), f"slot {s} touched"
    return out, st


@pytest.mark.parametrize("T", [8, 200])
def test_out_slots_fixed(T):
    # sequences 1 and 2 share read slot 1; sequence 3 stores nothing; slots 0..3 are only read
    w = la_synth.fixed(500 + T, 4, T, 2, 4, pool_slots=8, state_idx=[0, 1, 1, 2], flags=3, scale=0.9)
    idx_out = np.array([4, 5, 6, -1], np.int32)
    d = DevWorkload(w)
    o, pool = d.new_out(), d.fresh_pool()
    la.la_prefill_fwd_ex(d.q, d.k, d.v, o, d.slope, scale=w.scale, state_pool=pool, state_idx=d.idx,
                         state_idx_out=to_dev(idx_out), flags=3)
    torch.cuda.synchronize()
    out, st = _compare(w, o, pool, 3, idx_out, w.slope)
    print(f"out slots T={T}: {out} {st}", flush=True)
    assert_parity(out, st, f"out slots T={T}")


def test_out_slots_varlen():
    w = la_synth.varlen(510, 6, 300, 2, 2, pool_slots=12, n_skip=1, flags=3)
    w.state_idx = np.array([0, 1, 2, 3, -1, 5], np.int32)     # read slots disjoint from the written ones
    idx_out = np.array([11, 10, 9, 8, 7, 6], np.int32)
    d = DevWorkload(w)
    o, pool = d.new_out(), d.fresh_pool()
    la.la_prefill_fwd_varlen_ex(d.q, d.k, d.v, o, d.cu, d.slope, scale=w.scale, state_pool=pool, state_idx=d.idx,
                                state_idx_out=to_dev(idx_out), flags=3)
    torch.cuda.synchronize()
    out, st = _compare(w, o, pool, 3, idx_out, w.slope)
    assert_parity(out, st, "varlen out slots")


@pytest.mark.parametrize("T", [8, 130])
def test_decay_per_qk_head(T):
    H, G = 2, 4
    w = la_synth.fixed(520 + T, 3, T, H, H * G, pool_slots=3, state_idx=[2, 0, 1], flags=3, scale=0.8)
    sl_h = np.array([0.02, 0.6], np.float32)
    d = DevWorkload(w)
    flags = la.LA_STATE_READ | la.LA_STATE_WRITE | la.LA_DECAY_PER_QK_HEAD
    o, pool = d.new_out(), d.fresh_pool()
    la.la_prefill_fwd(d.q, d.k, d.v, o, to_dev(sl_h), scale=w.scale, state_pool=pool, state_idx=d.idx, flags=flags)
    o2, pool2 = d.new_out(), d.fresh_pool()
    la.la_prefill_fwd(d.q, d.k, d.v, o2, to_dev(np.repeat(sl_h, G)), scale=w.scale, state_pool=pool2,
                      state_idx=d.idx, flags=3)
    torch.cuda.synchronize()
    assert bitwise_equal(o, o2) and bitwise_equal(pool, pool2), "per-q/k-head decay != repeated per-value-head slopes"
    out, st = _compare(w, o, pool, flags, w.state_idx, sl_h)
    assert_parity(out, st, f"per-q/k-head decay T={T}")


def test_unknown_flag_bit_is_rejected():
    w = la_synth.fixed(530, 1, 8, 2, 2)
    d = DevWorkload(w)
    with pytest.raises(la.LaError):
        la.la_prefill_fwd(d.q, d.k, d.v, d.new_out(), d.slope, flags=8)

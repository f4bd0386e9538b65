"""GPU parity of the HIP path against the FP64 oracle, through the C-ABI binding.

Tolerances (acceptance bar for this path): output relative RMS <= 5e-3 and max abs <= 2e-2, final-state
relative RMS <= 1e-4, against the unrounded FP64 oracle. Invariants that hold bitwise on the GPU (same kernel
arithmetic) are checked with exact equality: packed == fixed, persistent == non-persistent, continuation at a
64-token boundary, run-to-run determinism, concurrent streams, graph replay, untouched pool slots, commit at
L = T == prefill final state.
"""
import numpy as np
import pytest
import torch

import la_synth
import linear_attention_decay_amd as la
from gpu_util import DevWorkload, add_state_slot, assert_parity, assert_state, bitwise_equal, compare_prefill, to_dev

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------------------------------------ small sweeps
@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("T", [1, 7, 8, 31, 32, 33, 63, 64, 65, 97, 127, 129, 200])
def test_fixed_sweep(T, G):
    H = 2
    w = la_synth.fixed(100 + T * 7 + G, 2, T, H, H * G, pool_slots=3, state_idx=[2, 0], flags=3, scale=0.7)
    w.slope = np.array([0.0, 2.0 ** -8, 0.05, 0.25, 1.0, 3.0, 2.0 ** -3, 0.5][:H * G], np.float32)
    _log(f"fixed T={T} G={G}")
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    assert_parity(out, st, f"T={T} G={G}")


@pytest.mark.parametrize("B,H,G", [(1, 11, 2), (3, 3, 4), (2, 8, 3)])
def test_gva_groups_full_rows_and_tail(B, H, G):
    """Workgroups are dealt to (sequence, q/k head) groups in rows of 8 groups plus a last partial row: 11 and 9
    groups take both branches, 16 groups only full rows; every unit of every group is checked (o is NaN-poisoned,
    so a unit left out would show)."""
    w = la_synth.fixed(300 + 10 * H + G, B, 130, H, H * G, pool_slots=B + 1, state_idx=list(range(B)), flags=3)
    w.slope = (np.linspace(0.0, 0.5, H * G) ** 2).astype(np.float32)
    _log(f"gva groups B={B} H={H} G={G}")
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    assert_parity(out, st, f"B={B} H={H} G={G}")


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_state_flags(flags):
    w = la_synth.fixed(7, 3, 130, 2, 4, pool_slots=5, state_idx=[4, -1, 1], flags=flags)
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    assert_parity(out, st, f"flags={flags}")
    if not (flags & 2):
        assert bitwise_equal(pool, d.pool0), "pool written without LA_STATE_WRITE"


@pytest.mark.parametrize("scale", [0.0, 0.25, 1.0 / np.sqrt(128.0), 3.0])
def test_scale_multiplies_both_terms(scale):
    w = la_synth.fixed(8, 1, 100, 2, 2, pool_slots=1, state_idx=[0], flags=3, scale=float(scale))
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    if scale == 0.0:
        assert torch.count_nonzero(o.float()) == 0
        assert_state(st, "scale=0")
    else:
        assert_parity(out, st, f"scale={scale}")


def test_extreme_decay():
    """slope = 0 (lambda = 1), large slopes and slope = +inf (lambda = 0: only the same token survives)."""
    w = la_synth.fixed(9, 1, 150, 4, 4, pool_slots=1, state_idx=[0], flags=3)
    w.slope = np.array([0.0, 8.0, 80.0, np.inf], np.float32)
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    out, st = compare_prefill(w, o, pool)
    assert_parity(out, st, "extreme decay")


def test_varlen_small_with_edges():
    lengths = [0, 1, 64, 65, 7, 128, 200, 0, 63, 32, 33]
    w = la_synth.varlen(21, len(lengths), 0, 2, 4, pool_slots=12, n_skip=2, flags=3, lengths=lengths, scale=0.9)
    w.state_idx[3] = 40          # >= pool size: treated as "no state"
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any(), "some output row not written"
    out, st = compare_prefill(w, o, pool)
    assert_parity(out, st, "varlen edges")
    o2, pool2 = d.prefill(schedule=la.LA_SCHED_PERSISTENT)
    o3, pool3 = d.prefill(schedule=la.LA_SCHED_NONPERSISTENT)
    torch.cuda.synchronize()
    assert bitwise_equal(o2, o3) and bitwise_equal(pool2, pool3) and bitwise_equal(o, o3)


def test_varlen_equals_fixed_bitwise():
    B, T, H, HV = 3, 150, 2, 4
    wf = la_synth.fixed(31, B, T, H, HV, pool_slots=4, state_idx=[3, 0, 2], flags=3)
    df = DevWorkload(wf)
    of, pf = df.prefill()
    cu = to_dev(np.arange(B + 1, dtype=np.int32) * T)
    ov = torch.full((B * T, HV, 128), float("nan"), dtype=torch.bfloat16, device=cu.device)
    pv = df.fresh_pool()
    la.la_prefill_fwd_varlen(df.q.view(B * T, H, 128), df.k.view(B * T, H, 128), df.v.view(B * T, HV, 128), ov, cu,
                             df.slope, state_pool=pv, state_idx=df.idx, flags=3)
    torch.cuda.synchronize()
    assert bitwise_equal(of.view(B * T, HV, 128), ov)
    assert bitwise_equal(pf, pv)


def test_continuation_bitwise_at_chunk_boundary():
    """Running T1 = 128 tokens, then T2 = 100 more from the stored state == one run over T1 + T2."""
    T1, T2, H = 128, 100, 2
    w = la_synth.fixed(41, 1, T1 + T2, H, H, pool_slots=1, state_idx=[0], flags=3)
    d = DevWorkload(w)
    o_all, p_all = d.prefill()
    q, k, v = d.q, d.k, d.v
    p = d.fresh_pool()
    o1 = torch.empty_like(v[:, :T1])
    o2 = torch.empty_like(v[:, T1:])
    la.la_prefill_fwd(q[:, :T1].contiguous(), k[:, :T1].contiguous(), v[:, :T1].contiguous(), o1, d.slope,
                      state_pool=p, state_idx=d.idx, flags=3)
    la.la_prefill_fwd(q[:, T1:].contiguous(), k[:, T1:].contiguous(), v[:, T1:].contiguous(), o2, d.slope,
                      state_pool=p, state_idx=d.idx, flags=3)
    torch.cuda.synchronize()
    assert bitwise_equal(torch.cat([o1, o2], dim=1), o_all)
    assert bitwise_equal(p, p_all)


def test_determinism_and_two_streams():
    wa = la_synth.fixed(51, 2, 300, 4, 4, pool_slots=2, state_idx=[1, 0], flags=3)
    wb = la_synth.varlen(52, 5, 300, 2, 4, pool_slots=6, n_skip=1, flags=3)
    da, db = DevWorkload(wa), DevWorkload(wb)
    oa, pa = da.prefill()
    ob, pb = db.prefill()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(20):
        oa2, pa2 = da.new_out(), da.fresh_pool()
        ob2, pb2 = db.new_out(), db.fresh_pool()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            da.prefill(o=oa2, pool=pa2, stream=s1)
        with torch.cuda.stream(s2):
            db.prefill(o=ob2, pool=pb2, stream=s2, schedule=la.LA_SCHED_PERSISTENT)
        torch.cuda.current_stream().wait_stream(s1)
        torch.cuda.current_stream().wait_stream(s2)
        outs.append((oa2, pa2, ob2, pb2))
    torch.cuda.synchronize()
    for oa2, pa2, ob2, pb2 in outs:
        assert bitwise_equal(oa2, oa) and bitwise_equal(pa2, pa)
        assert bitwise_equal(ob2, ob) and bitwise_equal(pb2, pb)


def test_graph_replay_matches_eager():
    w = la_synth.fixed(61, 2, 256, 4, 4, pool_slots=2, state_idx=[0, 1], flags=2)   # WRITE only: idempotent
    d = DevWorkload(w)
    o_ref, p_ref = d.prefill()
    torch.cuda.synchronize()
    o, pool = d.new_out(), d.fresh_pool()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.prefill(o=o, pool=pool, stream=s)          # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.prefill(o=o, pool=pool, stream=torch.cuda.current_stream())
    for _ in range(5):
        o.fill_(float("nan"))
        pool.copy_(d.pool0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bitwise_equal(o, o_ref) and bitwise_equal(pool, p_ref)


# ------------------------------------------------------------------------------------------------ the 5 workloads
def test_config0_tiny_full():
    w = la_synth.config(0)
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    _log(f"config0: {out} {st}")
    assert_parity(out, st, "config 0")


def _all_units(w, o, pool, batch):
    """Compare every (sequence, value head) unit with the oracle, streaming batches of units."""
    from oracle.compare import Accum
    units = [(n, hv) for n in range(w.nseq) for hv in range(w.HV)]
    out, st = Accum(), Accum()
    for i in range(0, len(units), batch):
        a, b = compare_prefill(w, o, pool, units=units[i:i + batch])
        out.merge(a)
        st.merge(b)
    return units, out, st


@pytest.mark.slow
def test_config1_full_size_all_units():
    w = la_synth.config(1)
    d = DevWorkload(w)
    _log("config1: running")
    o, pool = d.prefill()
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    units, out, st = _all_units(w, o, pool, 32)
    _log(f"config1 all {len(units)} units: {out} {st}")
    assert_parity(out, st, "config 1")


@pytest.mark.slow
def test_config2_varlen_full_size_all_units():
    w = la_synth.config(2)
    d = DevWorkload(w)
    _log(f"config2: lengths {np.diff(w.cu_seqlens).tolist()} idx {w.state_idx.tolist()}")
    o, pool = d.prefill()
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    units, out, st = _all_units(w, o, pool, 64)
    _log(f"config2 all {len(units)} units: {out} {st}")
    assert_parity(out, st, "config 2")
    o2, p2 = d.prefill(schedule=la.LA_SCHED_PERSISTENT)
    torch.cuda.synchronize()
    assert bitwise_equal(o2, o) and bitwise_equal(p2, pool)


@pytest.mark.slow
def test_config3_gva_full_size_all_units():
    w = la_synth.config(3)
    d = DevWorkload(w)
    _log("config3: running")
    o, pool = d.prefill()
    torch.cuda.synchronize()
    units, out, st = _all_units(w, o, pool, 16)
    _log(f"config3 all {len(units)} units: {out} {st}")
    assert_parity(out, st, "config 3")


def test_config4_verify_and_commit_full():
    w = la_synth.config(4)
    d = DevWorkload(w)
    _log("config4: verify")
    pool = d.fresh_pool()
    o, _ = d.prefill(pool=pool, flags=la.LA_STATE_READ)
    torch.cuda.synchronize()
    assert bitwise_equal(pool, d.pool0), "verify must not write the pool"
    out, _ = compare_prefill(w, o, None, flags=la.LA_STATE_READ)
    _log(f"config4 verify: {out}")
    assert_parity(out, None, "config 4 verify")
    d.commit(pool)
    torch.cuda.synchronize()
    import oracle
    from oracle.compare import Accum
    ref = oracle.commit(w.k.reshape(-1, w.H, 128), w.v.reshape(-1, w.HV, 128), w.B, w.T, w.H, w.HV, w.slope,
                        w.pool, w.state_idx, w.accepted_len)
    got = pool.cpu().numpy()
    st = Accum()
    for b in range(w.B):
        s = int(w.state_idx[b])
        if w.accepted_len[b] == 0:
            assert np.array_equal(got[s].view(np.uint32), w.pool[s].view(np.uint32)), "L = 0 must not write"
        else:
            add_state_slot(st, got[s], ref[s], s)
    _log(f"config4 commit: {st}")
    assert_state(st, "config 4 commit")


def test_commit_full_length_equals_prefill_state():
    B, T, H = 4, 8, 2
    w = la_synth.verify(71, B, T, H, H, pool_slots=6)
    w.accepted_len[:] = T
    w.state_idx[1] = -1
    d = DevWorkload(w)
    p_commit = d.commit(d.fresh_pool())
    _, p_pref = d.prefill(flags=3)
    torch.cuda.synchronize()
    assert bitwise_equal(p_commit, p_pref)

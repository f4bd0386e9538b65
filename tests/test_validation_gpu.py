"""Validation beyond parity, on the GPU, through the C-ABI binding:

- guard bands: every buffer a call writes (o, the state pool, the KV buffer) sits between two bands of sentinel
  bytes; after fixed, packed (both schedules), short, decode, segmented, commit and KV-buffer calls with ragged
  sizes, the bands must be bitwise unchanged, so no store lands before or past the end of a buffer;
- the packed prefill captured in a HIP graph under each schedule and replayed, with eager work between replays;
- a long graph-replay run of the tiny workload, every element of o and of the final state compared with the
  eager result after every replay;
- a multi-chunk commit (T = 200 on the chunked kernel) with accepted lengths on both sides of chunk boundaries.
"""
import numpy as np
import pytest
import torch

import la_synth
import linear_attention_decay_amd as la
import oracle
from gpu_util import DevWorkload, add_state_slot, assert_parity, assert_state, bitwise_equal, compare_prefill, to_dev
from oracle.compare import Accum

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GUARD_BYTES = 64 << 10


def _log(msg):
    print(msg, flush=True)


class Guarded:
    """A tensor of `shape` placed between two guard bands of GUARD_BYTES filled with a sentinel byte pattern."""

    def __init__(self, shape, dtype, fill=None):
        esize = torch.tensor([], dtype=dtype).element_size()
        n = int(np.prod(shape))
        g = GUARD_BYTES // esize
        self.buf = torch.empty(g + n + g, dtype=dtype, device=DEV)
        raw = self.buf.view(torch.uint8)
        raw.fill_(0xA5)
        self.g, self.n = g, n
        self.t = self.buf[g:g + n].view(shape)
        if fill is not None:
            self.t.copy_(fill)
        self.pre = raw[:GUARD_BYTES].clone()
        self.post = raw[GUARD_BYTES + n * esize:].clone()

    def intact(self):
        raw = self.buf.view(torch.uint8)
        esize = self.buf.element_size()
        return (torch.equal(raw[:GUARD_BYTES], self.pre)
                and torch.equal(raw[GUARD_BYTES + self.n * esize:], self.post))


def _guarded_out(v):
    return Guarded(tuple(v.shape), torch.bfloat16, fill=torch.full_like(v, float("nan")))


def _guarded_pool(d):
    return Guarded(tuple(d.pool0.shape), torch.float32, fill=d.pool0)


def test_guard_bands_fixed_short_decode_and_commit():
    # chunked fixed-length (ragged tail), READ | WRITE with a skipped slot
    w = la_synth.fixed(1001, 3, 200, 2, 4, pool_slots=4, state_idx=[3, -1, 0], flags=3)
    d = DevWorkload(w)
    o, pool = _guarded_out(d.v), _guarded_pool(d)
    la.la_prefill_fwd(d.q, d.k, d.v, o.t, d.slope, scale=w.scale, state_pool=pool.t, state_idx=d.idx, flags=3)
    torch.cuda.synchronize()
    assert o.intact() and pool.intact(), "chunked fixed-length call wrote outside o or the pool"
    out, st = compare_prefill(w, o.t, pool.t)
    assert_parity(out, st, "guarded fixed")
    # out slot at the last plane of the pool
    pool2 = _guarded_pool(d)
    la.la_prefill_fwd_ex(d.q, d.k, d.v, o.t, d.slope, scale=w.scale, state_pool=pool2.t, state_idx=d.idx,
                         state_idx_out=to_dev(np.array([3, 2, 1], np.int32)), flags=3)
    torch.cuda.synchronize()
    assert o.intact() and pool2.intact(), "fixed call with out slots wrote outside o or the pool"
    # short path (T = 13) and decode
    ws = la_synth.fixed(1002, 5, 13, 2, 4, pool_slots=6, state_idx=[5, 0, -1, 2, 9], flags=3)
    ds = DevWorkload(ws)
    o, pool = _guarded_out(ds.v), _guarded_pool(ds)
    la.la_prefill_fwd(ds.q, ds.k, ds.v, o.t, ds.slope, scale=ws.scale, state_pool=pool.t, state_idx=ds.idx, flags=3)
    torch.cuda.synchronize()
    assert o.intact() and pool.intact(), "short-path call wrote outside o or the pool"
    out, st = compare_prefill(ws, o.t, pool.t)
    assert_parity(out, st, "guarded short")
    o, pool = _guarded_out(ds.v), _guarded_pool(ds)
    la.la_decode_mtp(ds.q, ds.k, ds.v, o.t, ds.slope, pool.t, ds.idx, scale=ws.scale)
    torch.cuda.synchronize()
    assert o.intact() and pool.intact(), "decode wrote outside o or the pool"
    # commit on the short kernel (T = 8) and on the chunked kernel (T = 130)
    for T in (8, 130):
        wc = la_synth.verify(1003 + T, 7, T, 2, 4, pool_slots=9)
        wc.state_idx[2] = -1
        wc.accepted_len[:] = np.array([T, 0, T // 2, 1, T, T - 1, 3], np.int32)
        dc = DevWorkload(wc)
        pool = _guarded_pool(dc)
        la.la_state_commit(dc.k, dc.v, dc.slope, pool.t, dc.idx, dc.acc)
        torch.cuda.synchronize()
        assert pool.intact(), f"commit T={T} wrote outside the pool"


@pytest.mark.parametrize("schedule", [la.LA_SCHED_PERSISTENT, la.LA_SCHED_NONPERSISTENT])
def test_guard_bands_varlen(schedule):
    w = la_synth.varlen(1010, 7, 300, 2, 4, pool_slots=8, n_skip=2, flags=3,
                        lengths=[1, 63, 0, 65, 200, 129, 17])
    d = DevWorkload(w)
    o, pool = _guarded_out(d.v), _guarded_pool(d)
    la.la_prefill_fwd_varlen(d.q, d.k, d.v, o.t, d.cu, d.slope, scale=w.scale, state_pool=pool.t, state_idx=d.idx,
                             flags=3, schedule=schedule)
    torch.cuda.synchronize()
    assert o.intact() and pool.intact(), "packed call wrote outside o or the pool"
    out, st = compare_prefill(w, o.t, pool.t)
    assert_parity(out, st, "guarded varlen")


def test_guard_bands_segmented_and_kvbuffer():
    w = la_synth.fixed(1020, 2, 1000, 2, 4, pool_slots=3, state_idx=[2, 0], flags=3)
    d = DevWorkload(w)
    o, pool = _guarded_out(d.v), _guarded_pool(d)
    nbytes = la.la_prefill_seg_workspace_bytes(2, 4, 5)
    ws = Guarded((nbytes // 4,), torch.float32)
    la.la_prefill_fwd_seg(d.q, d.k, d.v, o.t, d.slope, scale=w.scale, state_pool=pool.t, state_idx=d.idx, flags=3,
                          segments=5, workspace=ws.t)
    torch.cuda.synchronize()
    assert o.intact() and pool.intact() and ws.intact(), "segmented call wrote outside o, the pool or the workspace"
    out, st = compare_prefill(w, o.t, pool.t)
    assert_parity(out, st, "guarded segmented")
    # KV-buffer verify and commit (T = 11), skipped requests included
    wv = la_synth.verify(1021, 9, 11, 2, 4, pool_slots=12)
    wv.state_idx[1] = -1
    wv.state_idx[4] = 40
    dv = DevWorkload(wv)
    P = wv.pool.shape[0]
    kb = Guarded((P, 11, 2, 128), torch.bfloat16, fill=torch.zeros((P, 11, 2, 128), dtype=torch.bfloat16))
    vb = Guarded((P, 11, 4, 128), torch.bfloat16, fill=torch.zeros((P, 11, 4, 128), dtype=torch.bfloat16))
    o, pool = _guarded_out(dv.v), _guarded_pool(dv)
    la.la_verify_kvbuffer(dv.q, dv.k, dv.v, o.t, dv.slope, pool.t, dv.idx, k_buf=kb.t, v_buf=vb.t, scale=wv.scale)
    la.la_state_commit_kvbuffer(kb.t, vb.t, dv.slope, pool.t, dv.idx, dv.acc)
    torch.cuda.synchronize()
    assert o.intact() and pool.intact() and kb.intact() and vb.intact(), "KV-buffer chain wrote outside a buffer"


@pytest.mark.parametrize("schedule", [la.LA_SCHED_PERSISTENT, la.LA_SCHED_NONPERSISTENT])
def test_varlen_graph_replay_matches_eager(schedule):
    """The packed prefill captured in a HIP graph (nothing on its call path synchronises or allocates) and replayed
    5 times, with eager refills and synchronisations between replays; every replay equals the eager call."""
    w = la_synth.varlen(1030, 9, 400, 2, 4, pool_slots=12, n_skip=2, flags=3, lengths=[5, 64, 0, 333, 1, 129, 65,
                                                                                       400, 17])
    d = DevWorkload(w)
    o_ref, p_ref = d.prefill(schedule=schedule)
    torch.cuda.synchronize()
    o, pool = d.new_out(), d.fresh_pool()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.prefill(o=o, pool=pool, stream=s, schedule=schedule)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.prefill(o=o, pool=pool, stream=torch.cuda.current_stream(), schedule=schedule)
    for _ in range(5):
        o.fill_(float("nan"))
        pool.copy_(d.pool0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bitwise_equal(o, o_ref) and bitwise_equal(pool, p_ref)


def test_long_graph_replay_tiny_workload():
    """2,000 replays of the tiny workload's prefill (B=1, T=256, H=4) from one HIP graph; after every replay the
    output and the final state are compared element by element with the eager call, stopping at the first
    mismatch."""
    w = la_synth.config(0)
    d = DevWorkload(w)
    o_ref, p_ref = d.prefill()
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o_ref, p_ref)
    assert_parity(out, st, "config 0 eager")
    o, pool = d.new_out(), d.fresh_pool()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.prefill(o=o, pool=pool, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.prefill(o=o, pool=pool, stream=torch.cuda.current_stream())
    ref_o16, ref_p32 = o_ref.view(torch.int16), p_ref.view(torch.int32)
    n = 2000
    for r in range(n):
        o.fill_(float("nan"))
        pool.zero_()
        g.replay()
        ok = torch.equal(o.view(torch.int16), ref_o16) and torch.equal(pool.view(torch.int32), ref_p32)
        assert ok, f"replay {r} differs from the eager call"
    _log(f"{n} replays bitwise equal to eager")


def test_chunked_commit_accepted_lengths_across_chunks():
    """Commit over T = 200 draft tokens (the chunked kernel's commit mode): accepted lengths 0, 1, 63, 64, 65, 130,
    199, 200 -- zero, single token, both sides of the first chunk boundary, a later partial chunk and all tokens --
    against the oracle's commit; L = 0 and skipped slots stay bitwise unchanged."""
    T, H, G = 200, 2, 2
    lens = [0, 1, 63, 64, 65, 130, 199, 200]
    w = la_synth.verify(1040, len(lens) + 1, T, H, H * G, pool_slots=12)
    w.accepted_len[:] = np.array(lens + [77], np.int32)
    w.state_idx[-1] = -1                                  # skipped request
    d = DevWorkload(w)
    pool = d.fresh_pool()
    la.la_state_commit(d.k, d.v, d.slope, pool, d.idx, d.acc)
    torch.cuda.synchronize()
    ref = oracle.commit(w.k.reshape(-1, H, 128), w.v.reshape(-1, H * G, 128), w.B, T, H, H * G, w.slope, w.pool,
                        w.state_idx, w.accepted_len)
    got = pool.cpu().numpy()
    st = Accum()
    written = set()
    for b in range(w.B):
        s = int(w.state_idx[b])
        if 0 <= s < w.pool.shape[0] and w.accepted_len[b] > 0:
            written.add(s)
            add_state_slot(st, got[s], ref[s], s)
    for s in range(w.pool.shape[0]):
        if s not in written:
            assert np.array_equal(got[s].view(np.uint32), w.pool[s].view(np.uint32)), f"slot {s} written"
    _log(f"chunked commit T={T}: {st}")
    assert_state(st, "chunked commit")
    # L = T equals the READ | WRITE prefill's final state bit for bit
    full = int(w.state_idx[lens.index(T)])
    wp = la_synth.fixed(0, 1, T, H, H * G, pool_slots=w.pool.shape[0], state_idx=[full], flags=3)
    wp.q, wp.k, wp.v = w.q[lens.index(T):lens.index(T) + 1], w.k[lens.index(T):lens.index(T) + 1], \
        w.v[lens.index(T):lens.index(T) + 1]
    wp.pool, wp.slope = w.pool, w.slope
    dp = DevWorkload(wp)
    _, p_pre = dp.prefill()
    torch.cuda.synchronize()
    assert bitwise_equal(p_pre[full], pool[full]), "commit at L = T differs from the prefill's final state"

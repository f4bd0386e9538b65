"""GPU parity of the short-sequence path (1 <= T <= 16 draft tokens: verify, multi-token decode, commit, and the
KV-buffer variants) against the FP64 oracle, through the C-ABI binding.

Tolerances as for the chunked path: output relative RMS <= 5e-3 and max abs <= 2e-2, state relative RMS <= 1e-4
against the unrounded FP64 oracle. Buffer copies and untouched slots are checked bitwise, and so is the commit
from the KV buffer against the commit from the original k / v (same kernel arithmetic on the same rows).
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

SLOPES8 = np.array([0.0, 2.0 ** -8, 0.05, 0.25, 1.0, 3.0, 2.0 ** -3, 0.5], np.float32)


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("flags", [1, 3])
@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 13, 16])
def test_short_fixed_against_oracle(T, G, flags):
    H = 2
    w = la_synth.fixed(300 + 11 * T + G + flags, 3, T, H, H * G, pool_slots=5, state_idx=[4, -1, 1], flags=flags,
                       scale=0.8)
    w.slope = SLOPES8[:H * G].copy()
    _log(f"short T={T} G={G} flags={flags}")
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    assert_parity(out, st, f"T={T} G={G} flags={flags}")
    if not (flags & la.LA_STATE_WRITE):
        assert bitwise_equal(pool, d.pool0)


@pytest.mark.parametrize("flags", [0, 2])
def test_short_without_initial_state(flags):
    w = la_synth.fixed(77, 4, 8, 2, 2, pool_slots=3, state_idx=[2, 7, -3, 0], flags=flags)
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    assert_parity(out, st, f"flags={flags}")


def test_decode_mtp_matches_prefill_read_write():
    w = la_synth.fixed(91, 6, 8, 2, 8, pool_slots=9, state_idx=[3, 8, -1, 0, 5, 1], flags=3, scale=0.6)
    w.slope = SLOPES8.copy()
    d = DevWorkload(w)
    o = d.new_out()
    pool = d.fresh_pool()
    la.la_decode_mtp(d.q, d.k, d.v, o, d.slope, pool, d.idx, scale=w.scale)
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool, flags=3)
    _log(f"decode_mtp: {out} {st}")
    assert_parity(out, st, "decode_mtp")


@pytest.mark.parametrize("extra", [-1, 0])
def test_work_unit_forms_on_both_sides_of_the_cu_count(extra):
    """Fewer (request, head) units than CUs run as four one-wave workgroups per unit, otherwise as one four-wave
    workgroup per unit: decode with CUs - 1 and CUs units checks both forms, with every unit against the oracle,
    and the KV-buffer copy of verify (written by wave 0 of a unit) bitwise."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = cus + extra
    HV = 8 if units % 8 == 0 else 1
    B = units // HV
    w = la_synth.fixed(95 + extra, B, 8, HV, HV, pool_slots=B + 1, state_idx=list(range(B, 0, -1)), flags=3,
                       scale=0.7)
    _log(f"work units: {B} requests x {HV} heads = {B * HV} units, {cus} CUs")
    d = DevWorkload(w)
    o, pool = d.new_out(), d.fresh_pool()
    la.la_decode_mtp(d.q, d.k, d.v, o, d.slope, pool, d.idx, scale=w.scale)
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool, flags=3)
    assert_parity(out, st, f"{B * HV} units")
    kb = torch.zeros(B + 1, 8, HV, 128, dtype=torch.bfloat16, device=d.q.device)
    vb = torch.zeros_like(kb)
    o2 = d.new_out()
    la.la_verify_kvbuffer(d.q, d.k, d.v, o2, d.slope, d.fresh_pool(), d.idx, k_buf=kb, v_buf=vb, scale=w.scale)
    torch.cuda.synchronize()
    slots = torch.as_tensor(w.state_idx, device=d.q.device).long()
    assert bitwise_equal(kb[slots], d.k) and bitwise_equal(vb[slots], d.v)


def test_decode_mtp_two_steps_continue_the_recurrence():
    # decode 5 drafts, then 3 more from the updated pool == the 8-token recurrence
    w = la_synth.fixed(92, 3, 8, 2, 2, pool_slots=3, state_idx=[2, 0, 1], flags=3)
    d = DevWorkload(w)
    pool = d.fresh_pool()
    o = d.new_out()
    for t0, t1 in ((0, 5), (5, 8)):
        q, k, v = (x[:, t0:t1].contiguous() for x in (d.q, d.k, d.v))
        oo = torch.empty_like(v)
        la.la_decode_mtp(q, k, v, oo, d.slope, pool, d.idx, scale=w.scale)
        o[:, t0:t1] = oo
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool, flags=3)
    assert_parity(out, st, "two decode steps")


def _kv_buffers(w, dev_w, sentinel):
    P, T = w.pool.shape[0], w.T
    kb = torch.full((P, T, w.H, 128), sentinel, dtype=torch.bfloat16, device=dev_w.q.device)
    vb = torch.full((P, T, w.HV, 128), sentinel, dtype=torch.bfloat16, device=dev_w.q.device)
    return kb, vb


@pytest.mark.parametrize("T,G", [(8, 1), (5, 4), (16, 2)])
def test_verify_kvbuffer_outputs_and_buffer(T, G):
    w = la_synth.verify(120 + T + G, 10, T, 2, 2 * G, pool_slots=16)
    w.state_idx[3] = -1
    w.state_idx[6] = 99                                  # >= pool size: skipped
    d = DevWorkload(w)
    kb, vb = _kv_buffers(w, d, 3.0)
    pool = d.fresh_pool()
    o = d.new_out()
    la.la_verify_kvbuffer(d.q, d.k, d.v, o, d.slope, pool, d.idx, k_buf=kb, v_buf=vb, scale=w.scale)
    torch.cuda.synchronize()
    assert bitwise_equal(pool, d.pool0), "verify must not write the pool"
    out, _ = compare_prefill(w, o, None, flags=la.LA_STATE_READ)
    _log(f"verify_kvbuffer T={T} G={G}: {out}")
    assert_parity(out, None, "verify_kvbuffer")
    kb_h, vb_h = kb.view(torch.int16).cpu().numpy(), vb.view(torch.int16).cpu().numpy()
    k_h = d.k.view(torch.int16).cpu().numpy()
    v_h = d.v.view(torch.int16).cpu().numpy()
    sent = torch.tensor(3.0, dtype=torch.bfloat16).view(torch.int16).item()
    used = set()
    for b in range(w.B):
        s = int(w.state_idx[b])
        if 0 <= s < w.pool.shape[0]:
            used.add(s)
            assert np.array_equal(kb_h[s], k_h[b]) and np.array_equal(vb_h[s], v_h[b]), f"buffer slot {s}"
    for s in range(w.pool.shape[0]):
        if s not in used:
            assert (kb_h[s] == sent).all() and (vb_h[s] == sent).all(), f"slot {s} touched"


def test_verify_without_buffer_equals_prefill_read_bitwise():
    w = la_synth.verify(131, 6, 8, 2, 4, pool_slots=8)
    d = DevWorkload(w)
    o1 = d.new_out()
    la.la_verify_kvbuffer(d.q, d.k, d.v, o1, d.slope, d.fresh_pool(), d.idx, scale=w.scale)
    o2, _ = d.prefill(flags=la.LA_STATE_READ)
    torch.cuda.synchronize()
    assert bitwise_equal(o1, o2)


@pytest.mark.parametrize("T,G", [(8, 1), (16, 4)])
def test_commit_kvbuffer_against_oracle_and_direct_commit(T, G):
    w = la_synth.verify(140 + T + G, 12, T, 2, 2 * G, pool_slots=20)
    w.state_idx[2] = -1
    w.accepted_len[0] = 0
    w.accepted_len[1] = T
    d = DevWorkload(w)
    kb, vb = _kv_buffers(w, d, 0.0)
    la.la_verify_kvbuffer(d.q, d.k, d.v, d.new_out(), d.slope, d.fresh_pool(), d.idx, k_buf=kb, v_buf=vb,
                          scale=w.scale)
    pool_buf = d.fresh_pool()
    la.la_state_commit_kvbuffer(kb, vb, d.slope, pool_buf, d.idx, d.acc)
    pool_dir = d.commit(d.fresh_pool())
    torch.cuda.synchronize()
    assert bitwise_equal(pool_buf, pool_dir), "commit from the KV buffer differs from the direct commit"
    ref = oracle.commit(w.k.reshape(-1, w.H, 128), w.v.reshape(-1, w.HV, 128), w.B, w.T, w.H, w.HV, w.slope,
                        w.pool, w.state_idx, w.accepted_len)
    got = pool_buf.cpu().numpy()
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
    _log(f"commit_kvbuffer T={T} G={G}: {st}")
    assert_state(st, "commit")


def test_config4_kvbuffer_chain_full():
    w = la_synth.config(4)
    d = DevWorkload(w)
    kb, vb = _kv_buffers(w, d, 0.0)
    pool = d.fresh_pool()
    o = d.new_out()
    la.la_verify_kvbuffer(d.q, d.k, d.v, o, d.slope, pool, d.idx, k_buf=kb, v_buf=vb, scale=w.scale)
    la.la_state_commit_kvbuffer(kb, vb, d.slope, pool, d.idx, d.acc)
    torch.cuda.synchronize()
    out, _ = compare_prefill(w, o, None, flags=la.LA_STATE_READ)
    ref = oracle.commit(w.k.reshape(-1, w.H, 128), w.v.reshape(-1, w.HV, 128), w.B, w.T, w.H, w.HV, w.slope,
                        w.pool, w.state_idx, w.accepted_len)
    got = pool.cpu().numpy()
    st = Accum()
    for b in range(w.B):
        s = int(w.state_idx[b])
        if w.accepted_len[b] == 0:
            assert np.array_equal(got[s].view(np.uint32), w.pool[s].view(np.uint32))
        else:
            add_state_slot(st, got[s], ref[s], s)
    _log(f"config4 KV-buffer chain: verify {out} commit {st}")
    assert_parity(out, None, "config 4 verify (KV buffer)")
    assert_state(st, "commit")


def test_kvbuffer_chain_graph_replay_matches_eager():
    """verify + commit through the KV buffer captured in one HIP graph and replayed, with eager work between the
    replays, equals the eager chain bitwise every time."""
    w = la_synth.verify(170, 16, 8, 2, 4, pool_slots=20)
    d = DevWorkload(w)

    def chain(o, pool, kb, vb, stream):
        la.la_verify_kvbuffer(d.q, d.k, d.v, o, d.slope, pool, d.idx, k_buf=kb, v_buf=vb, scale=w.scale,
                              stream=stream)
        la.la_state_commit_kvbuffer(kb, vb, d.slope, pool, d.idx, d.acc, stream=stream)

    o_ref, p_ref = d.new_out(), d.fresh_pool()
    kb_ref, vb_ref = _kv_buffers(w, d, 0.0)
    chain(o_ref, p_ref, kb_ref, vb_ref, None)
    torch.cuda.synchronize()
    o, pool = d.new_out(), d.fresh_pool()
    kb, vb = _kv_buffers(w, d, 0.0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain(o, pool, kb, vb, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(o, pool, kb, vb, torch.cuda.current_stream())
    for _ in range(4):
        o.fill_(float("nan"))
        pool.copy_(d.pool0)
        kb.zero_()
        vb.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bitwise_equal(o, o_ref) and bitwise_equal(pool, p_ref)
        assert bitwise_equal(kb, kb_ref) and bitwise_equal(vb, vb_ref)

"""GPU parity of the segmented prefill (la_prefill_fwd_seg: local segment states, scan, full pass from every
segment's initial state) against the FP64 oracle. Tolerances as for the main path."""
import numpy as np
import pytest
import torch

import la_synth
import linear_attention_decay_amd as la
from gpu_util import DevWorkload, add_state_slot, assert_parity, bitwise_equal, compare_prefill, to_dev

pytestmark = pytest.mark.gpu

SLOPES8 = np.array([0.0, 2.0 ** -8, 0.05, 0.25, 1.0, 3.0, 2.0 ** -3, 0.5], np.float32)


def _ws(B, HV, segments, dev):
    n = la.la_prefill_seg_workspace_bytes(B, HV, segments)
    return torch.empty(max(n, 4) // 4, dtype=torch.float32, device=dev)


@pytest.mark.parametrize("B,T,H,G,segments,flags", [
    (1, 1000, 2, 1, 2, 3),
    (1, 1024, 2, 4, 4, 3),
    (2, 300, 1, 4, 3, 1),
    (1, 4096, 4, 1, 8, 2),
    (2, 777, 2, 2, 5, 0),
])
def test_segmented_against_oracle(B, T, H, G, segments, flags):
    w = la_synth.fixed(600 + T + segments, B, T, H, H * G, pool_slots=B + 1, state_idx=list(range(B, 0, -1)),
                       flags=flags, scale=0.75)
    if T <= 1024:
        # includes slope 0 (lambda = 1); over longer sequences its outputs grow past |o| = 16, where bf16 output
        # rounding alone exceeds the absolute tolerance, so long cases keep the decaying per-head slopes
        w.slope = SLOPES8[:H * G].copy()
    d = DevWorkload(w)
    o, pool = d.new_out(), d.fresh_pool()
    ws = _ws(B, H * G, segments, o.device)
    la.la_prefill_fwd_seg(d.q, d.k, d.v, o, d.slope, scale=w.scale, state_pool=pool, state_idx=d.idx, flags=flags,
                          segments=segments, workspace=ws)
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    print(f"segmented B={B} T={T} G={G} S={segments} flags={flags}: {out} {st}", flush=True)
    assert_parity(out, st, f"segmented S={segments}")


def test_segmented_auto_out_slots_and_qk_decay():
    B, T, H, G = 1, 2048, 2, 2
    w = la_synth.fixed(650, B, T, H, H * G, pool_slots=3, state_idx=[0], flags=3)
    d = DevWorkload(w)
    flags = la.LA_STATE_READ | la.LA_STATE_WRITE | la.LA_DECAY_PER_QK_HEAD
    sl_h = np.array([0.01, 0.3], np.float32)
    idx_out = np.array([2], np.int32)
    props = torch.cuda.get_device_properties(0)
    n_auto = max(1, props.multi_processor_count // (2 * B * H * G))
    ws = _ws(B, H * G, n_auto, d.q.device)
    o, pool = d.new_out(), d.fresh_pool()
    la.la_prefill_fwd_seg(d.q, d.k, d.v, o, to_dev(sl_h), scale=w.scale, state_pool=pool, state_idx=d.idx,
                          state_idx_out=to_dev(idx_out), flags=flags, segments=0, workspace=ws)
    torch.cuda.synchronize()
    import oracle
    from oracle.compare import Accum
    ref_o, ref_pool = oracle.prefill(w.q.reshape(-1, H, 128), w.k.reshape(-1, H, 128), w.v.reshape(-1, H * G, 128),
                                     [0], [T], H, H * G, w.scale, sl_h, pool=w.pool, state_idx=w.state_idx,
                                     flags=flags, state_idx_out=idx_out)
    got = o.float().cpu().numpy().reshape(-1, H * G, 128)
    out = Accum()
    for (n, hv), ref in ref_o.items():
        out.add(got[:, hv], ref, unit=(n, hv))
    st = Accum()
    pg = pool.cpu().numpy()
    add_state_slot(st, pg[2], ref_pool[2], 2)
    for s in (0, 1):
        assert np.array_equal(pg[s].view(np.uint32), w.pool[s].view(np.uint32))
    assert_parity(out, st, "segmented auto")


def test_segmented_rejects_small_workspace():
    w = la_synth.fixed(660, 1, 1024, 2, 2)
    d = DevWorkload(w)
    ws = torch.empty(16, dtype=torch.float32, device=d.q.device)
    with pytest.raises(la.LaError):
        la.la_prefill_fwd_seg(d.q, d.k, d.v, d.new_out(), d.slope, segments=4, workspace=ws)


def test_segmented_graph_replay_matches_eager():
    """The three launches of the segmented prefill captured in one HIP graph and replayed, with eager work between
    the replays, equal the eager call bitwise every time."""
    B, T, H = 1, 1024, 2
    w = la_synth.fixed(670, B, T, H, H, pool_slots=2, state_idx=[1], flags=3)
    d = DevWorkload(w)
    ws = _ws(B, H, 4, d.q.device)
    o_ref, p_ref = d.new_out(), d.fresh_pool()
    la.la_prefill_fwd_seg(d.q, d.k, d.v, o_ref, d.slope, state_pool=p_ref, state_idx=d.idx, flags=3, segments=4,
                          workspace=ws)
    torch.cuda.synchronize()
    o, pool = d.new_out(), d.fresh_pool()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        la.la_prefill_fwd_seg(d.q, d.k, d.v, o, d.slope, state_pool=pool, state_idx=d.idx, flags=3, segments=4,
                              workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        la.la_prefill_fwd_seg(d.q, d.k, d.v, o, d.slope, state_pool=pool, state_idx=d.idx, flags=3, segments=4,
                              workspace=ws, stream=torch.cuda.current_stream())
    for _ in range(4):
        o.fill_(float("nan"))
        pool.copy_(d.pool0)
        ws.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bitwise_equal(o, o_ref) and bitwise_equal(pool, p_ref)

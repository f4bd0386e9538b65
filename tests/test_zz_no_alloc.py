"""The allocation-free segmented prefill (la_prefill_fwd_seg_noalloc), called through the C ABI: its outputs and
states equal those of la_prefill_fwd_seg with a caller workspace, bit for bit, on two calls in a row (the second
smaller, so it runs on what the first left in the library's device array), and the first also meets the parity
bars against the FP64 oracle. A call needing more than the array holds is refused before any launch."""
import numpy as np
import pytest
import torch

import la_synth
import linear_attention_decay_amd as la
from gpu_util import DevWorkload, assert_parity, bitwise_equal, compare_prefill, to_dev

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _run_both(w, segments, idx_out=None):
    d = DevWorkload(w)
    out_idx = None if idx_out is None else to_dev(np.asarray(idx_out, np.int32))
    n = la.la_prefill_seg_workspace_bytes(w.B, w.HV, max(segments, 1))
    if segments == 0:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        n = la.la_prefill_seg_workspace_bytes(w.B, w.HV, max(1, cus // (2 * w.B * w.HV)))
    ws = torch.empty(max(n, 4) // 4, dtype=torch.float32, device=d.q.device)
    o_ref, pool_ref = d.new_out(), d.fresh_pool()
    la.la_prefill_fwd_seg(d.q, d.k, d.v, o_ref, d.slope, scale=w.scale, state_pool=pool_ref, state_idx=d.idx,
                          state_idx_out=out_idx, flags=w.flags, segments=segments, workspace=ws)
    o, pool = d.new_out(), d.fresh_pool()
    la.la_prefill_fwd_seg_noalloc(d.q, d.k, d.v, o, d.slope, scale=w.scale, state_pool=pool, state_idx=d.idx,
                                  state_idx_out=out_idx, flags=w.flags, segments=segments)
    torch.cuda.synchronize()
    return o_ref, pool_ref, o, pool


def test_noalloc_equals_workspace_call_twice_then_smaller():
    assert la.la_prefill_seg_noalloc_max_bytes() == 16 << 20
    # first call: ragged T, READ | WRITE, the segment count chosen from the CU count (128 state planes)
    w1 = la_synth.fixed(901, 1, 4096 + 37, 8, 8, pool_slots=3, state_idx=[1], flags=3, scale=0.8)
    _log("noalloc call 1: B=1 T=4133 H=HV=8 segments=auto")
    o_ref, pool_ref, o, pool = _run_both(w1, 0)
    assert bitwise_equal(o, o_ref), "call 1: output differs from la_prefill_fwd_seg"
    assert bitwise_equal(pool, pool_ref), "call 1: states differ from la_prefill_fwd_seg"
    out, st = compare_prefill(w1, o, pool)
    _log(f"noalloc call 1 vs oracle: {out} {st}")
    assert_parity(out, st, "noalloc call 1")
    # second call, smaller: GVA, 4 segments, out slot, the array still holding call 1's states
    w2 = la_synth.fixed(902, 2, 1000, 2, 4, pool_slots=4, state_idx=[3, 0], flags=3, scale=1.1)
    _log("noalloc call 2: B=2 T=1000 H=2 HV=4 segments=4")
    o_ref, pool_ref, o, pool = _run_both(w2, 4, idx_out=[1, 2])
    assert bitwise_equal(o, o_ref), "call 2: output differs from la_prefill_fwd_seg"
    assert bitwise_equal(pool, pool_ref), "call 2: states differ from la_prefill_fwd_seg"


def test_noalloc_refuses_more_than_its_array():
    # 1 x 8 segments x 64 heads = 512 planes > 256: refused on the host, nothing launched
    w = la_synth.fixed(903, 1, 1024, 64, 64, flags=0)
    d = DevWorkload(w)
    o = d.new_out()
    with pytest.raises(la.LaError) as e:
        la.la_prefill_fwd_seg_noalloc(d.q, d.k, d.v, o, d.slope, scale=w.scale, segments=8)
    assert e.value.status == la.LA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all(), "a refused call wrote output"

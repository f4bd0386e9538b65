"""Long sequences against the FP64 oracle: the config-5 workload (B=1, T=32768, H=HV=16) in full through both the
segmented and the plain chunked path, and one sequence of 131,072 tokens (2,048 chunks) carried in registers
from the first chunk to the last. Every (sequence, value head) unit is compared. Tolerances as for the main path."""
import pytest
import torch

import la_synth
import linear_attention_decay_amd as la
from gpu_util import DevWorkload, assert_parity, compare_prefill

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _log(msg):
    print(msg, flush=True)


def test_config5_full_size_segmented_and_plain():
    w = la_synth.config(5)
    d = DevWorkload(w)
    props = torch.cuda.get_device_properties(0)
    n_auto = max(1, props.multi_processor_count // (2 * w.B * w.HV))
    ws = torch.empty(max(la.la_prefill_seg_workspace_bytes(w.B, w.HV, n_auto), 4) // 4, dtype=torch.float32,
                     device=d.q.device)
    _log(f"config5: segmented, {n_auto} segments requested")
    o, pool = d.new_out(), d.fresh_pool()
    la.la_prefill_fwd_seg(d.q, d.k, d.v, o, d.slope, scale=w.scale, state_pool=pool, state_idx=d.idx,
                          flags=w.flags, segments=0, workspace=ws)
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    _log(f"config5 segmented: {out} {st}")
    assert_parity(out, st, "config 5 segmented")
    _log("config5: plain")
    o2, p2 = d.prefill()
    torch.cuda.synchronize()
    out2, st2 = compare_prefill(w, o2, p2)
    _log(f"config5 plain: {out2} {st2}")
    assert_parity(out2, st2, "config 5 plain")


def test_one_sequence_of_131072_tokens():
    T = 131072
    w = la_synth.fixed(710, 1, T, 2, 2, pool_slots=1, state_idx=[0], flags=3, scale=0.9)
    d = DevWorkload(w)
    _log(f"long sequence: T={T}, slopes {w.slope.tolist()}")
    o, pool = d.prefill()
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    out, st = compare_prefill(w, o, pool)
    _log(f"long sequence: {out} {st}")
    assert_parity(out, st, f"T={T}")

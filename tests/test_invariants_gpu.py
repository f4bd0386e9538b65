"""Exact invariants of the GPU path that hold at any size. Every stage is linear in v and S0 (jointly), in q, and in
scale, and every rounding step (bf16 splits, FP32 products and sums, the bf16 output) commutes with multiplication
by a power of two while no value leaves the normal range. So scaling v and S0 by 2^e must scale o and the final
state by exactly 2^e, and scaling q or scale must scale o alone: bit for bit, on both the one-pass short kernel
(T <= 16) and the chunked kernel. A step that depended on magnitude (a fixed threshold, an offset, a clamp)
would break it."""
import numpy as np
import pytest
import torch

import la_synth
import linear_attention_decay_amd as la
from gpu_util import DevWorkload, bitwise_equal

pytestmark = pytest.mark.gpu


def _run(d, q, v, pool, scale, flags=3):
    o = d.new_out()
    la.la_prefill_fwd(q, d.k, v, o, d.slope, scale=scale, state_pool=pool, state_idx=d.idx, flags=flags)
    return o


@pytest.mark.parametrize("T,G", [(8, 1), (16, 2), (200, 1), (131, 4)])
@pytest.mark.parametrize("e", [-40, 24])
def test_power_of_two_scaling_is_exact(T, G, e):
    H = 2
    w = la_synth.fixed(800 + T + G, 2, T, H, H * G, pool_slots=3, state_idx=[2, 0], flags=3, scale=0.8)
    w.slope = np.array([0.0, 2.0 ** -8, 0.05, 0.25, 1.0, 3.0, 2.0 ** -3, 0.5][:H * G], np.float32)
    d = DevWorkload(w)
    f = 2.0 ** e
    print(f"scaling T={T} G={G} e={e}", flush=True)

    pool = d.fresh_pool()
    o = _run(d, d.q, d.v, pool, w.scale)
    pool_v = d.fresh_pool() * f
    o_v = _run(d, d.q, d.v * f, pool_v, w.scale)                       # v and S0 scaled
    pool_q = d.fresh_pool()
    o_q = _run(d, d.q * f, d.v, pool_q, w.scale)                       # q scaled
    pool_s = d.fresh_pool()
    o_s = _run(d, d.q, d.v, pool_s, w.scale * f)                       # scale scaled
    torch.cuda.synchronize()

    assert not torch.isnan(o.float()).any()
    assert bitwise_equal(o_v, o * f) and bitwise_equal(pool_v, pool * f)
    assert bitwise_equal(o_q, o * f) and bitwise_equal(pool_q, pool)
    assert bitwise_equal(o_s, o * f) and bitwise_equal(pool_s, pool)


@pytest.mark.parametrize("T,G", [(8, 1), (130, 1), (130, 2), (70, 4)])
def test_sequence_and_head_permutation_is_exact(T, G):
    """Units are independent: reordering the sequences and the q/k heads (each with its G value heads, slopes and
    pool planes) must reorder the outputs and final states bit for bit. This pins the mapping from workgroups to
    (sequence, value head, half) and from value heads to q/k heads."""
    B, H = 3, 3
    HV = H * G
    w = la_synth.fixed(900 + T + G, B, T, H, HV, pool_slots=B + 1, state_idx=[3, 0, 2], flags=3, scale=0.6)
    w.slope = np.linspace(0.0, 0.4, HV).astype(np.float32) ** 2
    d = DevWorkload(w)
    rng = np.random.default_rng(T * 10 + G)
    pb = rng.permutation(B)                       # new sequence b' is old sequence pb[b']
    ph = rng.permutation(H)                       # new q/k head i is old head ph[i]
    pv = np.array([ph[i] * G + g for i in range(H) for g in range(G)])   # value heads follow their q/k head
    print(f"permutation T={T} G={G} seqs {pb.tolist()} heads {ph.tolist()}", flush=True)

    pool = d.fresh_pool()
    o = _run(d, d.q, d.v, pool, w.scale)
    tb, th, tv = (torch.as_tensor(x, device=d.q.device) for x in (pb, ph, pv))
    q2 = d.q[tb][:, :, th].contiguous()
    k2 = d.k[tb][:, :, th].contiguous()
    v2 = d.v[tb][:, :, tv].contiguous()
    slope2 = d.slope[tv].contiguous()
    pool2 = d.fresh_pool()[:, tv].contiguous()
    idx2 = d.idx[tb].contiguous()
    o2 = d.new_out()
    la.la_prefill_fwd(q2, k2, v2, o2, slope2, scale=w.scale, state_pool=pool2, state_idx=idx2, flags=3)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    assert bitwise_equal(o2, o[tb][:, :, tv].contiguous())
    assert bitwise_equal(pool2, pool[:, tv].contiguous())

"""Seeded random sweep of the GPU paths against the FP64 oracle: fixed-length prefill (short and chunked kernels,
with and without out slots and per-q/k-head decay), packed sequences, the segmented prefill and commit. Sizes,
head ratios, flags, scales, slopes and slot indices are drawn per case; every unit is compared. Tolerances as for
the main path."""
import numpy as np
import pytest
import torch

import la_synth
import linear_attention_decay_amd as la
import oracle
from gpu_util import DevWorkload, add_state_slot, assert_parity, assert_state, compare_prefill, to_dev
from oracle.compare import Accum

pytestmark = pytest.mark.gpu


def _draw(rng):
    H = int(rng.choice([1, 2, 3]))
    G = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 4))
    T = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 400))]))
    flags = int(rng.integers(0, 4))
    P = B + 2
    idx = rng.permutation(P)[:B].astype(np.int32)
    idx[rng.random(B) < 0.2] = -1
    return H, G, B, T, flags, P, idx


@pytest.mark.parametrize("case", range(12))
def test_random_fixed(case):
    rng = np.random.default_rng(900 + case)
    H, G, B, T, flags, P, idx = _draw(rng)
    w = la_synth.fixed(1000 + case, B, T, H, H * G, pool_slots=P, state_idx=idx.tolist(), flags=flags,
                       scale=float(rng.uniform(0.2, 1.5)))
    w.slope = (rng.uniform(0, 0.6, H * G) ** 2).astype(np.float32)
    print(f"case {case}: B={B} T={T} H={H} G={G} flags={flags} idx={idx.tolist()}", flush=True)
    d = DevWorkload(w)
    o, pool = d.prefill()
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    assert_parity(out, st, f"case {case}")


@pytest.mark.parametrize("case", range(6))
def test_random_segmented_with_options(case):
    rng = np.random.default_rng(950 + case)
    H, G, B, _, flags, P, idx = _draw(rng)
    T = int(rng.integers(130, 1500))
    segments = int(rng.integers(2, 7))
    w = la_synth.fixed(1100 + case, B, T, H, H * G, pool_slots=P + B, state_idx=idx.tolist(), flags=flags)
    idx_out = np.array([P + b if rng.random() < 0.8 else -1 for b in range(B)], np.int32)   # own slots
    qk = bool(rng.random() < 0.5)
    sl = (rng.uniform(0.001, 0.3, H if qk else H * G) ** 1.5).astype(np.float32)
    fl = flags | (la.LA_DECAY_PER_QK_HEAD if qk else 0)
    print(f"seg case {case}: B={B} T={T} H={H} G={G} S={segments} flags={fl} idx={idx.tolist()} out={idx_out.tolist()}",
          flush=True)
    d = DevWorkload(w)
    o, pool = d.new_out(), d.fresh_pool()
    nbytes = la.la_prefill_seg_workspace_bytes(B, H * G, segments)
    ws = torch.empty(max(nbytes, 4) // 4, dtype=torch.float32, device=o.device)
    la.la_prefill_fwd_seg(d.q, d.k, d.v, o, to_dev(sl), scale=w.scale, state_pool=pool, state_idx=d.idx,
                          state_idx_out=to_dev(idx_out), flags=fl, segments=segments, workspace=ws)
    torch.cuda.synchronize()
    rows = w.seq_rows()
    ref_o, ref_pool = oracle.prefill(w.q.reshape(-1, H, 128), w.k.reshape(-1, H, 128), w.v.reshape(-1, H * G, 128),
                                     [r for r, _ in rows], [n for _, n in rows], H, H * G, w.scale, sl, pool=w.pool,
                                     state_idx=w.state_idx, flags=fl, state_idx_out=idx_out)
    got = o.float().cpu().numpy().reshape(-1, H * G, 128)
    out = Accum()
    for (n, hv), ref in ref_o.items():
        r0, L = rows[n]
        out.add(got[r0:r0 + L, hv], ref, unit=(n, hv))
    st = Accum()
    pg = pool.cpu().numpy()
    written = {int(s) for s in idx_out if s >= 0} if fl & la.LA_STATE_WRITE else set()
    for s in range(pg.shape[0]):
        if s in written:
            add_state_slot(st, pg[s], ref_pool[s], s)
        else:
            assert np.array_equal(pg[s].view(np.uint32), w.pool[s].view(np.uint32)), f"slot {s} touched"
    assert_parity(out, st, f"seg case {case}")


@pytest.mark.parametrize("case", range(6))
def test_random_varlen_and_commit(case):
    rng = np.random.default_rng(980 + case)
    H = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 4]))
    N = int(rng.integers(1, 7))
    lengths = [int(x) for x in rng.choice([0, 1, 5, 16, 17, 63, 64, 65, 200], size=N)]
    w = la_synth.varlen(1200 + case, N, 0, H, H * G, pool_slots=N + 2, n_skip=int(rng.integers(0, 2)), flags=3,
                        lengths=lengths)
    d = DevWorkload(w)
    o, pool = d.prefill(schedule=int(rng.integers(0, 3)))
    torch.cuda.synchronize()
    out, st = compare_prefill(w, o, pool)
    assert_parity(out, st, f"varlen case {case} lengths {lengths}")
    # commit of T <= 16 drafts (short kernel) and of longer accepted runs (chunked kernel)
    T = int(rng.choice([8, 40]))
    v = la_synth.verify(1300 + case, 4, T, H, H * G, pool_slots=6)
    dv = DevWorkload(v)
    pool_c = dv.commit(dv.fresh_pool())
    torch.cuda.synchronize()
    ref = oracle.commit(v.k.reshape(-1, H, 128), v.v.reshape(-1, H * G, 128), v.B, v.T, H, H * G, v.slope, v.pool,
                        v.state_idx, v.accepted_len)
    got = pool_c.cpu().numpy()
    st = Accum()
    for b in range(v.B):
        s = int(v.state_idx[b])
        if v.accepted_len[b] > 0:
            add_state_slot(st, got[s], ref[s], s)
        else:
            assert np.array_equal(got[s].view(np.uint32), v.pool[s].view(np.uint32))
    assert_state(st, f"commit case {case}")

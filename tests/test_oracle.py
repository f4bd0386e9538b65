"""Pins for the CPU oracle (no GPU).

The tokenwise FP64 recurrence in oracle/la_oracle.c is checked against things other than itself:
  * the O(T^2) closed form printed on the verify page ("[LA] Lightning Attention MTP decode + KVBuffer
    parallel verify / commit", Description) -- a non-recursive sum;
  * the 64-token chunked algorithm (prefill page, Description) evaluated in FP64;
  * textbook special cases: lambda = 1 is plain causal linear attention, lambda = 0 keeps only the same token;
  * a hand-computed single-token example (tests/golden/t1_hand.json);
  * invariants the prefill page's Reviewer notes name: continuation, state-pool isolation, GVA mapping, packed
    equals per-sequence; and the commit invariants of the verify page (L = T equals the full run, L = 0 is a
    no-op, negative slots are skipped).
Non-square D != DV shapes are used where they expose a transposed state.
"""
import json
import os

import numpy as np
import pytest

import oracle
from la_synth import bf16_bits, bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_unit(rng, T, D, DV, H=1, HV=1):
    q = bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32) * 0.3)
    k = bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32) * 0.3)
    v = bf16_bits(rng.standard_normal((T, HV, DV)).astype(np.float32))
    return q, k, v


def _f64(bits):
    return bits_to_f32(bits).astype(np.float64)


def _run_one(q, k, v, slope, scale, s0, H=1, HV=1, hv=0):
    T = q.shape[0]
    outs, sf = oracle.tokenwise(q, k, v, H, HV, scale, np.asarray(slope, np.float32), [(0, T, hv)],
                                s0=None if s0 is None else s0[None])
    return outs[0], sf[0]


SLOPES = [0.0, 2.0 ** -8, 0.05, 0.25, 3.0]


@pytest.mark.parametrize("T", [1, 2, 7, 64, 65, 130, 300])
@pytest.mark.parametrize("slope", SLOPES)
def test_tokenwise_matches_closed_form(T, slope):
    """p1: recurrence == the verify page's closed form, with scale != 1, S0 != 0 and D != DV."""
    rng = np.random.default_rng(1000 + T)
    D, DV = 24, 16
    q, k, v = _rand_unit(rng, T, D, DV)
    s0 = rng.standard_normal((DV, D)) * 0.5
    scale = 0.37
    o, sT = _run_one(q, k, v, [slope], scale, s0)
    lam = float(np.exp(-np.float64(np.float32(slope))))
    o_ref, s_ref = oracle.closed_form(_f64(q[:, 0]), _f64(k[:, 0]), _f64(v[:, 0]), lam, scale, s0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-11 * np.abs(o_ref).max())
    np.testing.assert_allclose(sT, s_ref, rtol=1e-11, atol=1e-11 * np.abs(s_ref).max())


@pytest.mark.parametrize("C", [1, 7, 16, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_chunked_matches_tokenwise(C, T):
    """p2: the chunked algebra (intra mask, inter lambda^{j+1}, state lambda^{Lc}, ragged tail) == recurrence."""
    rng = np.random.default_rng(2000 + 7 * T + C)
    D, DV = 32, 16
    q, k, v = _rand_unit(rng, T, D, DV)
    s0 = rng.standard_normal((DV, D)) * 0.2
    for slope in (0.0, 0.02, 0.25):
        o, sT = _run_one(q, k, v, [slope], 1.3, s0)
        lam = float(np.exp(-np.float64(np.float32(slope))))
        oc, sc = oracle.chunked(_f64(q[:, 0]), _f64(k[:, 0]), _f64(v[:, 0]), lam, 1.3, s0, C=C)
        np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-11 * np.abs(o).max())
        np.testing.assert_allclose(sc, sT, rtol=1e-10, atol=1e-11 * np.abs(sT).max())


def test_lambda_one_is_causal_linear_attention():
    """p3: slope 0 (lambda = 1): o = scale (tril(Q K^T) V + Q S0^T), S_T = S0 + V^T K."""
    rng = np.random.default_rng(3)
    T, D, DV = 50, 20, 12
    q, k, v = _rand_unit(rng, T, D, DV)
    s0 = rng.standard_normal((DV, D))
    o, sT = _run_one(q, k, v, [0.0], 0.5, s0)
    Q, K, V = _f64(q[:, 0]), _f64(k[:, 0]), _f64(v[:, 0])
    np.testing.assert_allclose(o, 0.5 * (np.tril(Q @ K.T) @ V + Q @ s0.T), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(sT, s0 + V.T @ K, rtol=1e-11, atol=1e-11)


def test_lambda_zero_keeps_only_same_token():
    """p4: slope = +inf (lambda = 0): o_t = scale (q_t . k_t) v_t and S_T = v_{T-1} k_{T-1}^T (0^0 = 1)."""
    rng = np.random.default_rng(4)
    T, D, DV = 9, 16, 8
    q, k, v = _rand_unit(rng, T, D, DV)
    s0 = rng.standard_normal((DV, D))
    o, sT = _run_one(q, k, v, [np.inf], 2.0, s0)
    Q, K, V = _f64(q[:, 0]), _f64(k[:, 0]), _f64(v[:, 0])
    np.testing.assert_allclose(o, 2.0 * np.sum(Q * K, axis=1)[:, None] * V, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sT, np.outer(V[-1], K[-1]), rtol=1e-13, atol=1e-14)


def test_single_token_hand_example():
    """p5: T = 1 worked by hand (tests/golden/t1_hand.json)."""
    with open(os.path.join(GOLDEN, "t1_hand.json")) as f:
        g = json.load(f)
    q = bf16_bits(np.array(g["q"], np.float32)[None, None])
    k = bf16_bits(np.array(g["k"], np.float32)[None, None])
    v = bf16_bits(np.array(g["v"], np.float32)[None, None])
    s0 = np.array(g["S0"], np.float64)
    o, s1 = _run_one(q, k, v, [g["slope"]], g["scale"], s0)
    np.testing.assert_allclose(o[0], g["o"], rtol=0, atol=1e-6)
    np.testing.assert_allclose(s1, g["S1"], rtol=0, atol=1e-6)


def test_continuation():
    """p6: run(T1) -> state -> run(T2) == run(T1 + T2) (prefill page, Reviewer notes: continuation)."""
    rng = np.random.default_rng(6)
    T1, T2, D, DV = 37, 45, 16, 16
    q, k, v = _rand_unit(rng, T1 + T2, D, DV)
    s0 = rng.standard_normal((DV, D)) * 0.1
    o_all, s_all = _run_one(q, k, v, [0.03], 1.0, s0)
    o1, s1 = _run_one(q[:T1], k[:T1], v[:T1], [0.03], 1.0, s0)
    o2, s2 = _run_one(q[T1:], k[T1:], v[T1:], [0.03], 1.0, s1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_all, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s2, s_all, rtol=1e-12, atol=1e-12)


def test_linearity_in_v_and_s0():
    """p7: outputs and state are linear in (V, S0) jointly, and affine pieces add up."""
    rng = np.random.default_rng(7)
    T, D, DV = 40, 16, 8
    q, k, v = _rand_unit(rng, T, D, DV)
    s0 = rng.standard_normal((DV, D))
    o, sT = _run_one(q, k, v, [0.1], 0.9, s0)
    v2 = bf16_bits(bits_to_f32(v) * np.float32(2.0))            # exact doubling in bf16
    o2, sT2 = _run_one(q, k, v2, [0.1], 0.9, 2.0 * s0)
    np.testing.assert_allclose(o2, 2.0 * o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sT2, 2.0 * sT, rtol=1e-13, atol=1e-13)
    # additivity in S0 with V fixed: f(Sa + Sb) - f(Sa) - f(Sb) + f(0) == 0
    sa, sb = rng.standard_normal((DV, D)), rng.standard_normal((DV, D))
    oa, _ = _run_one(q, k, v, [0.1], 0.9, sa)
    ob, _ = _run_one(q, k, v, [0.1], 0.9, sb)
    oab, _ = _run_one(q, k, v, [0.1], 0.9, sa + sb)
    oz, _ = _run_one(q, k, v, [0.1], 0.9, np.zeros((DV, D)))
    np.testing.assert_allclose(oab - oa - ob + oz, 0.0, atol=1e-11)


def test_gva_mapping_equals_repeated_mha():
    """p11: G value heads share q/k head h = hv // G; equals MHA with each q/k head repeated G times."""
    rng = np.random.default_rng(11)
    T, D, DV, H, G = 33, 16, 8, 3, 2
    HV = H * G
    q, k, v = _rand_unit(rng, T, D, DV, H=H, HV=HV)
    sl = np.linspace(0.01, 0.4, HV).astype(np.float32)
    units = [(0, T, hv) for hv in range(HV)]
    o_gva, s_gva = oracle.tokenwise(q, k, v, H, HV, 1.0, sl, units)
    qr, kr = np.repeat(q, G, axis=1), np.repeat(k, G, axis=1)
    o_mha, s_mha = oracle.tokenwise(qr, kr, v, HV, HV, 1.0, sl, units)
    for a, b in zip(o_gva, o_mha):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(s_gva, s_mha)
    # and each value head really uses q/k head hv // G: compare against single-head runs
    for hv in range(HV):
        o1, s1 = _run_one(q[:, hv // G:hv // G + 1], k[:, hv // G:hv // G + 1], v[:, hv:hv + 1], [sl[hv]], 1.0,
                          None)
        np.testing.assert_array_equal(o1, o_gva[hv])


def _small_varlen(rng, lengths, H, HV, D=16, DV=8, P=6):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    tot = int(cu[-1])
    q = bf16_bits(rng.standard_normal((tot, H, D)).astype(np.float32) * 0.3)
    k = bf16_bits(rng.standard_normal((tot, H, D)).astype(np.float32) * 0.3)
    v = bf16_bits(rng.standard_normal((tot, HV, DV)).astype(np.float32))
    pool = (rng.standard_normal((P, HV, DV, D)) * 0.1).astype(np.float32)
    return cu, q, k, v, pool


def test_packed_equals_per_sequence_and_pool_isolation():
    """p8 + p9: packed varlen == per-sequence runs; slot -1 and slot >= P read zero and write nothing;
    slots nobody selects are untouched; a zero-length sequence writes its initial state."""
    rng = np.random.default_rng(8)
    H, HV = 2, 4
    lengths = [5, 0, 70, 1, 64]
    cu, q, k, v, pool = _small_varlen(rng, lengths, H, HV, P=7)
    idx = np.array([3, 5, -1, 1, 9], np.int32)           # 9 >= P: treated like -1
    sl = np.linspace(0.0, 0.3, HV).astype(np.float32)
    rows = list(zip(cu[:-1], np.diff(cu)))
    outs, pool_after = oracle.prefill(q, k, v, cu[:-1], np.diff(cu), H, HV, 0.8, sl, pool=pool,
                                      state_idx=idx, flags=oracle.STATE_READ | oracle.STATE_WRITE)
    for n, (r0, L) in enumerate(rows):
        s = idx[n]
        for hv in range(HV):
            s0 = pool[s, hv].astype(np.float64) if 0 <= s < 7 else np.zeros((8, 16))
            o1, sf = _run_one(q[r0:r0 + L, hv // 2:hv // 2 + 1], k[r0:r0 + L, hv // 2:hv // 2 + 1],
                              v[r0:r0 + L, hv:hv + 1], [sl[hv]], 0.8, s0)
            np.testing.assert_array_equal(outs[(n, hv)], o1)
            if 0 <= s < 7:
                np.testing.assert_array_equal(pool_after[s, hv], sf)
    untouched = [s for s in range(7) if s not in set(int(i) for i in idx)]
    for s in untouched:
        np.testing.assert_array_equal(pool_after[s], pool[s].astype(np.float64))
    # zero-length sequence 1 (slot 5): final state == its initial state
    np.testing.assert_array_equal(pool_after[5], pool[5].astype(np.float64))
    # write-only: initial state is zero even for a valid slot
    outs_w, pool_w = oracle.prefill(q, k, v, cu[:-1], np.diff(cu), H, HV, 0.8, sl, pool=pool, state_idx=idx,
                                    flags=oracle.STATE_WRITE)
    o1, sf = _run_one(q[0:5, 0:1], k[0:5, 0:1], v[0:5, 0:1], [sl[0]], 0.8, None)
    np.testing.assert_array_equal(outs_w[(0, 0)], o1)
    np.testing.assert_array_equal(pool_w[3, 0], sf)
    np.testing.assert_array_equal(pool_w[5], np.zeros_like(pool_w[5]))


def test_commit_invariants():
    """p10: commit at L = T equals the prefill's final state; L = 0 and slot -1 leave the pool bitwise as is;
    partial L equals a prefill over the first L tokens."""
    rng = np.random.default_rng(10)
    B, T, H, HV, D, DV, P = 5, 8, 2, 2, 16, 8, 6
    q = bf16_bits(rng.standard_normal((B, T, H, D)).astype(np.float32) * 0.3)
    k = bf16_bits(rng.standard_normal((B, T, H, D)).astype(np.float32) * 0.3)
    v = bf16_bits(rng.standard_normal((B, T, HV, DV)).astype(np.float32))
    pool = (rng.standard_normal((P, HV, DV, D)) * 0.1).astype(np.float32)
    pool[0, 0, 0, 0] = -0.0
    idx = np.array([2, 0, 4, -1, 1], np.int32)
    acc = np.array([T, 0, 3, 5, 1], np.int32)
    sl = np.array([0.02, 0.2], np.float32)
    qf, kf, vf = q.reshape(B * T, H, D), k.reshape(B * T, H, D), v.reshape(B * T, HV, DV)
    after = oracle.commit(kf, vf, B, T, H, HV, sl, pool, idx, acc)
    _, full = oracle.prefill(qf, kf, vf, np.arange(B) * T, [T] * B, H, HV, 1.0, sl, pool=pool, state_idx=idx,
                             flags=3)
    np.testing.assert_array_equal(after[2], full[2])                          # L = T
    assert np.signbit(after[0, 0, 0, 0]) and after[0, 0, 0, 0] == 0.0        # L = 0: bitwise untouched
    np.testing.assert_array_equal(after[0], pool[0].astype(np.float64))
    _, part = oracle.prefill(qf, kf, vf, np.arange(B) * T, acc, H, HV, 1.0, sl, pool=pool, state_idx=idx,
                             flags=3)
    np.testing.assert_array_equal(after[4], part[4])                          # partial L = 3
    np.testing.assert_array_equal(after[1], part[1])                          # L = 1
    for s in (3, 5):                                                          # unselected / skipped slots
        np.testing.assert_array_equal(after[s], pool[s].astype(np.float64))


def test_bf16_rounding_matches_torch():
    """The generator's float32 -> bf16 rounding is round-to-nearest-even (same as torch's .to(bfloat16))."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    x = rng.standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0e-39]                    # ties and a denormal
    mine = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)


def test_decay_per_qk_head_matches_closed_form():
    """With DECAY_PER_QK_HEAD the slope array has one entry per q/k head and every value head of the group decays
    with it (prefill page, Performance: GVA rows "_h"); checked against the O(T^2) closed form per value head."""
    rng = np.random.default_rng(23)
    T, D, DV, H, G = 21, 16, 8, 2, 3
    HV = H * G
    q, k, v = _rand_unit(rng, T, D, DV, H=H, HV=HV)
    pool = (rng.standard_normal((2, HV, DV, D)) * 0.1).astype(np.float32)
    sl_h = np.array([0.03, 0.7], np.float32)
    flags = oracle.STATE_READ | oracle.STATE_WRITE | oracle.DECAY_PER_QK_HEAD
    outs, pool_after = oracle.prefill(q, k, v, [0], [T], H, HV, 0.9, sl_h, pool=pool, state_idx=[1], flags=flags)
    qf, kf, vf = bits_to_f32(q).astype(np.float64), bits_to_f32(k).astype(np.float64), bits_to_f32(v).astype(np.float64)
    for hv in range(HV):
        lam = np.exp(-np.float64(sl_h[hv // G]))
        o_ref, s_ref = oracle.closed_form(qf[:, hv // G], kf[:, hv // G], vf[:, hv], lam, 0.9,
                                          pool[1, hv].astype(np.float64))
        np.testing.assert_allclose(outs[(0, hv)], o_ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(pool_after[1, hv], s_ref, rtol=1e-11, atol=1e-12)


def test_out_slot_relocates_the_state_and_continues():
    """state_idx_out: the final state lands in its own slot and the read slot is untouched; reading it back
    continues the recurrence (run(T1) -> slot 3, then run(T2) from slot 3 == run(T1 + T2) from slot 0)."""
    rng = np.random.default_rng(29)
    T1, T2, D, DV, H = 9, 14, 16, 8, 2
    q, k, v = _rand_unit(rng, T1 + T2, D, DV, H=H, HV=H)
    pool = (rng.standard_normal((5, H, DV, D)) * 0.1).astype(np.float32)
    rw = oracle.STATE_READ | oracle.STATE_WRITE
    sl = np.array([0.05, 0.4], np.float32)
    _, p1 = oracle.prefill(q[:T1], k[:T1], v[:T1], [0], [T1], H, H, 1.0, sl, pool=pool, state_idx=[0], flags=rw,
                           state_idx_out=[3])
    for s in (0, 1, 2, 4):
        np.testing.assert_array_equal(p1[s], pool[s].astype(np.float64))
    o2, p2 = oracle.prefill(q[T1:], k[T1:], v[T1:], [0], [T2], H, H, 1.0, sl, pool=p1.astype(np.float32),
                            state_idx=[3], flags=rw)
    o_all, p_all = oracle.prefill(q, k, v, [0], [T1 + T2], H, H, 1.0, sl, pool=pool, state_idx=[0], flags=rw)
    for hv in range(H):
        # the relocated state passed through float32 once; agreement is at float32 rounding of S
        np.testing.assert_allclose(o2[(0, hv)], o_all[(0, hv)][T1:], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(p2[3, hv], p_all[0, hv], rtol=1e-5, atol=1e-6)
    # an out slot outside the pool stores nothing
    _, p3 = oracle.prefill(q[:T1], k[:T1], v[:T1], [0], [T1], H, H, 1.0, sl, pool=pool, state_idx=[0], flags=rw,
                           state_idx_out=[-1])
    np.testing.assert_array_equal(p3, pool.astype(np.float64))


def test_segmented_scan_reproduces_the_recurrence():
    """Segments run from a zero state give local states L_g; the scan S_{g+1} = lambda^{Ls} S_g + L_g yields every
    segment's initial state, and each segment run from it reproduces the full recurrence (KDA sm90 page,
    Description: chunk-parallel PREP, sequential SCAN over the state -- here over whole segments)."""
    rng = np.random.default_rng(37)
    T, Ls, D, DV = 50, 12, 16, 8
    q, k, v = _rand_unit(rng, T, D, DV)
    s0 = rng.standard_normal((DV, D)) * 0.1
    sl = np.array([0.08], np.float32)
    lam = np.exp(-np.float64(sl[0]))
    bounds = [(a, min(a + Ls, T)) for a in range(0, T, Ls)]
    init = [s0]
    for a, b in bounds[:-1]:
        _, loc = oracle.tokenwise(q[a:b], k[a:b], v[a:b], 1, 1, 1.0, sl, [(0, b - a, 0)], s0=np.zeros((1, DV, D)),
                                  want_o=False)
        init.append(lam ** (b - a) * init[-1] + loc[0])
    o_full, s_full = oracle.tokenwise(q, k, v, 1, 1, 0.5, sl, [(0, T, 0)], s0=s0[None])
    for (a, b), si in zip(bounds, init):
        o_seg, s_seg = oracle.tokenwise(q[a:b], k[a:b], v[a:b], 1, 1, 0.5, sl, [(0, b - a, 0)], s0=si[None])
        np.testing.assert_allclose(o_seg[0], o_full[0][a:b], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s_seg[0], s_full[0], rtol=1e-11, atol=1e-13)

"""The Python binding rejects tensors whose shapes do not match what the kernels index: the library sees only
pointers, so a pool with the wrong head count or a short index tensor would be read or written out of bounds.
Every case here raises before anything is launched."""
import pytest
import torch

import linear_attention_decay_amd as la

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype, device=DEV)


def _prefill_args(B=2, T=70, H=2, HV=4, P=3):
    q, k = _t(B, T, H, 128), _t(B, T, H, 128)
    v, o = _t(B, T, HV, 128), _t(B, T, HV, 128)
    slope = _t(HV, dtype=torch.float32)
    pool = _t(P, HV, 128, 128, dtype=torch.float32)
    idx = torch.arange(B, dtype=torch.int32, device=DEV)
    return q, k, v, o, slope, pool, idx


def test_prefill_rejects_pool_with_wrong_head_count():
    q, k, v, o, slope, pool, idx = _prefill_args()
    bad = _t(3, 2, 128, 128, dtype=torch.float32)
    with pytest.raises(ValueError, match="state_pool"):
        la.la_prefill_fwd(q, k, v, o, slope, state_pool=bad, state_idx=idx, flags=3)
    with pytest.raises(ValueError, match="state_pool"):
        la.la_prefill_fwd(q, k, v, o, slope, state_pool=_t(3, 4, 128, dtype=torch.float32), state_idx=idx, flags=3)


def test_prefill_rejects_short_index_tensors():
    q, k, v, o, slope, pool, idx = _prefill_args()
    with pytest.raises(ValueError, match="state_idx"):
        la.la_prefill_fwd(q, k, v, o, slope, state_pool=pool, state_idx=idx[:1], flags=3)
    with pytest.raises(ValueError, match="state_idx_out"):
        la.la_prefill_fwd(q, k, v, o, slope, state_pool=pool, state_idx=idx, state_idx_out=idx[:1], flags=3)
    with pytest.raises(ValueError, match="state_idx"):
        la.la_prefill_fwd_seg(q, k, v, o, slope, state_pool=pool, state_idx=idx[:1], flags=3)


def test_varlen_rejects_bad_offsets_and_indices():
    q, k = _t(100, 2, 128), _t(100, 2, 128)
    v, o = _t(100, 4, 128), _t(100, 4, 128)
    slope = _t(4, dtype=torch.float32)
    pool = _t(3, 4, 128, 128, dtype=torch.float32)
    cu = torch.tensor([0, 40, 100], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="state_idx"):
        la.la_prefill_fwd_varlen(q, k, v, o, cu, slope, state_pool=pool,
                                 state_idx=torch.zeros(3, dtype=torch.int32, device=DEV), flags=3)
    with pytest.raises(ValueError, match="cu_seqlens"):
        la.la_prefill_fwd_varlen(q, k, v, o, cu.view(1, 3), slope)


def test_short_path_entry_points_reject_bad_shapes():
    q, k, v, o, slope, pool, idx = _prefill_args(T=8)
    acc = torch.zeros(2, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="accepted_len"):
        la.la_state_commit(k, v, slope, pool, idx, acc[:1])
    with pytest.raises(ValueError, match="slope"):
        la.la_state_commit(k, v, slope[:2], pool, idx, acc)
    with pytest.raises(ValueError, match="state_pool"):
        la.la_decode_mtp(q, k, v, o, slope, None, idx)
    with pytest.raises(ValueError, match="slope"):
        la.la_verify_kvbuffer(q, k, v, o, slope[:3], pool, idx)
    kb, vb = _t(3, 8, 2, 128), _t(3, 8, 4, 128)
    with pytest.raises(ValueError, match="accepted_len"):
        la.la_state_commit_kvbuffer(kb, vb, slope, pool, idx, acc[:1])
    with pytest.raises(ValueError, match="state_pool"):
        la.la_state_commit_kvbuffer(kb, vb, slope, _t(3, 2, 128, 128, dtype=torch.float32), idx, acc)

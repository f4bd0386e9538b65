"""Host-side checks of the C-ABI library (no GPU): it loads, exports every declared symbol, and each invalid call
returns an error status and enqueues no work (prefill page, Description)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la_prefill.h")

la = pytest.importorskip("linear_attention_decay_amd")
L = la.lib

FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below returns before any launch


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(la.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert L.la_abi_version() == 2
    assert L.la_status_string(0) == b"LA_OK"
    assert L.la_status_string(2) == b"LA_ERR_UNSUPPORTED"


def _fwd(B=1, T=64, H=2, HV=2, D=128, DV=128, slope=FAKE, pool=None, P=0, idx=None, flags=0, q=FAKE):
    return L.la_prefill_fwd(q, FAKE, FAKE, FAKE, B, T, H, HV, D, DV, 1.0, slope, pool, P, idx, flags, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), la.LA_ERR_UNSUPPORTED),
    (dict(DV=256), la.LA_ERR_UNSUPPORTED),
    (dict(H=3, HV=4), la.LA_ERR_UNSUPPORTED),
    (dict(H=4, HV=2), la.LA_ERR_UNSUPPORTED),
    (dict(H=0, HV=0), la.LA_ERR_UNSUPPORTED),
    (dict(H=1, HV=65537), la.LA_ERR_UNSUPPORTED),                # 32-bit row offsets
    (dict(B=-1), la.LA_ERR_INVALID_ARG),
    (dict(T=-5), la.LA_ERR_INVALID_ARG),
    (dict(slope=None), la.LA_ERR_INVALID_ARG),
    (dict(flags=1), la.LA_ERR_INVALID_ARG),                       # READ without pool / idx
    (dict(flags=2, pool=FAKE, P=1), la.LA_ERR_INVALID_ARG),       # WRITE without idx
    (dict(flags=8, pool=FAKE, P=1, idx=FAKE), la.LA_ERR_INVALID_ARG),
    (dict(q=None), la.LA_ERR_INVALID_ARG),
    (dict(flags=3, pool=FAKE, P=-1, idx=FAKE), la.LA_ERR_INVALID_ARG),
])
def test_fixed_rejects_before_launch(kw, status):
    assert _fwd(**kw) == status
    assert L.la_last_error() != b""


def test_empty_calls_are_noops():
    assert _fwd(B=0) == la.LA_OK
    assert _fwd(B=0, flags=4) == la.LA_OK                          # per-q/k-head decay needs no pool
    assert L.la_prefill_fwd_ex(FAKE, FAKE, FAKE, FAKE, 0, 64, 2, 2, 128, 128, 1.0, FAKE, FAKE, 1, FAKE, FAKE, 3,
                               None) == la.LA_OK
    assert _fwd(T=0) == la.LA_OK
    assert L.la_last_error() == b""
    assert L.la_prefill_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 2, 2, 128, 128, 1.0, FAKE, None, 0, None, 0,
                                   0, None) == la.LA_OK
    assert L.la_state_commit(FAKE, FAKE, 0, 8, 2, 2, 128, 128, FAKE, FAKE, 4, FAKE, FAKE, None) == la.LA_OK
    assert L.la_state_commit(FAKE, FAKE, 4, 0, 2, 2, 128, 128, FAKE, FAKE, 4, FAKE, FAKE, None) == la.LA_OK


def test_varlen_rejects_before_launch():
    f = L.la_prefill_fwd_varlen
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 10, 2, 2, 128, 128, 1.0, FAKE, None, 0, None, 0, 0, None) == \
        la.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, None, 3, 10, 2, 2, 128, 128, 1.0, FAKE, None, 0, None, 0, 0, None) == \
        la.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 10, 2, 2, 128, 128, 1.0, FAKE, None, 0, None, 0, 7, None) == \
        la.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 10, 2, 2, 96, 128, 1.0, FAKE, None, 0, None, 0, 0, None) == \
        la.LA_ERR_UNSUPPORTED


def test_commit_rejects_before_launch():
    f = L.la_state_commit
    assert f(FAKE, FAKE, 2, 8, 2, 2, 128, 128, FAKE, None, 4, FAKE, FAKE, None) == la.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 2, 8, 2, 2, 128, 128, FAKE, FAKE, 4, FAKE, None, None) == la.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 2, 8, 2, 3, 128, 128, FAKE, FAKE, 4, FAKE, FAKE, None) == la.LA_ERR_UNSUPPORTED


def test_short_path_entry_points_reject_before_launch():
    # decode: needs a pool and indices (it reads and writes the state)
    assert L.la_decode_mtp(FAKE, FAKE, FAKE, FAKE, 2, 4, 2, 2, 128, 128, 1.0, FAKE, None, 4, FAKE, None) == \
        la.LA_ERR_INVALID_ARG
    assert L.la_decode_mtp(FAKE, FAKE, FAKE, FAKE, 2, 4, 2, 2, 64, 128, 1.0, FAKE, FAKE, 4, FAKE, None) == \
        la.LA_ERR_UNSUPPORTED
    v = L.la_verify_kvbuffer
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 17, 2, 2, 128, 128, 1.0, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None) == \
        la.LA_ERR_UNSUPPORTED                                      # more than 16 draft tokens
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 2, 128, 128, 1.0, FAKE, FAKE, 4, FAKE, FAKE, None, None) == \
        la.LA_ERR_INVALID_ARG                                      # k_buf without v_buf
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 2, 128, 128, 1.0, FAKE, None, 4, FAKE, None, None, None) == \
        la.LA_ERR_INVALID_ARG                                      # verify reads the pool
    assert v(FAKE, FAKE, FAKE, FAKE, 0, 8, 2, 2, 128, 128, 1.0, FAKE, FAKE, 4, FAKE, None, None, None) == la.LA_OK
    c = L.la_state_commit_kvbuffer
    assert c(FAKE, FAKE, 2, 17, 2, 2, 128, 128, FAKE, FAKE, 4, FAKE, FAKE, None) == la.LA_ERR_UNSUPPORTED
    assert c(FAKE, None, 2, 8, 2, 2, 128, 128, FAKE, FAKE, 4, FAKE, FAKE, None) == la.LA_ERR_INVALID_ARG
    assert c(FAKE, FAKE, 2, 8, 2, 2, 128, 128, FAKE, FAKE, 4, FAKE, None, None) == la.LA_ERR_INVALID_ARG
    assert c(FAKE, FAKE, 2, 8, 3, 2, 128, 128, FAKE, FAKE, 4, FAKE, FAKE, None) == la.LA_ERR_UNSUPPORTED
    assert c(FAKE, FAKE, 2, 0, 2, 2, 128, 128, FAKE, FAKE, 4, FAKE, FAKE, None) == la.LA_OK


def test_seg_noalloc_refuses_beyond_its_array_before_launch():
    f = L.la_prefill_fwd_seg_noalloc
    assert L.la_prefill_seg_noalloc_max_bytes() == 16 << 20
    # 1 sequence x 8 segments x 64 heads = 512 state planes of 64 KiB > 16 MiB
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1024, 64, 64, 128, 128, 1.0, FAKE, None, 0, None, None, 0, 8, None) == \
        la.LA_ERR_UNSUPPORTED
    assert b"scratch" in L.la_last_error()
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1024, 2, 2, 128, 128, 1.0, FAKE, None, 0, None, None, 0, -1, None) == \
        la.LA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1024, 2, 2, 64, 128, 1.0, FAKE, None, 0, None, None, 0, 4, None) == \
        la.LA_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 1024, 2, 2, 128, 128, 1.0, FAKE, None, 0, None, None, 0, 4, None) == la.LA_OK


def test_python_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 64, 2, 128, dtype=torch.float16)
    with pytest.raises((TypeError, ValueError)):
        la.la_prefill_fwd(q, q, q, q, torch.zeros(2))

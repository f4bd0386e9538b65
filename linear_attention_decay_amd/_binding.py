"""Thin ctypes binding of liblaprefill.so (include/la_prefill.h). Argument marshalling only.

Device memory and streams come from torch; every step of the computation runs in the library's HIP kernels.
The functions have the same names as the C entry points and derive the sizes from the tensor shapes.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblaprefill.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP = 0, 1, 2, 3
LA_STATE_READ, LA_STATE_WRITE, LA_DECAY_PER_QK_HEAD = 1, 2, 4
LA_SCHED_AUTO, LA_SCHED_PERSISTENT, LA_SCHED_NONPERSISTENT = 0, 1, 2

EXPORTS = ("la_prefill_fwd", "la_prefill_fwd_ex", "la_prefill_fwd_seg", "la_prefill_seg_workspace_bytes",
           "la_prefill_fwd_seg_noalloc", "la_prefill_seg_noalloc_max_bytes",
           "la_prefill_fwd_varlen", "la_prefill_fwd_varlen_ex",
           "la_state_commit", "la_decode_mtp", "la_verify_kvbuffer", "la_state_commit_kvbuffer", "la_status_string",
           "la_last_error", "la_abi_version")


class LaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _load():
    # The library's HIP runtime dependency (soname libamdhip64.so.7) must resolve to the runtime the caller's
    # torch already loaded; loading the library first would bring in a second HIP runtime whose device
    # pointers and streams are not torch's. Import torch before dlopen so the soname is already satisfied.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing; build it with python linear_attention_decay_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    p, i32, u32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
    L.la_prefill_fwd.restype = ctypes.c_int
    L.la_prefill_fwd.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, p, i32, p, u32, p]
    L.la_prefill_fwd_ex.restype = ctypes.c_int
    L.la_prefill_fwd_ex.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, p, i32, p, p, u32, p]
    L.la_prefill_fwd_seg.restype = ctypes.c_int
    L.la_prefill_fwd_seg.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, p, i32, p, p, u32, i32, p,
                                     ctypes.c_size_t, p]
    L.la_prefill_fwd_seg_noalloc.restype = ctypes.c_int
    L.la_prefill_fwd_seg_noalloc.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, p, i32, p, p, u32, i32,
                                             p]
    L.la_prefill_seg_noalloc_max_bytes.restype = ctypes.c_size_t
    L.la_prefill_seg_noalloc_max_bytes.argtypes = []
    L.la_prefill_seg_workspace_bytes.restype = ctypes.c_size_t
    L.la_prefill_seg_workspace_bytes.argtypes = [i32, i32, i32]
    L.la_prefill_fwd_varlen_ex.restype = ctypes.c_int
    L.la_prefill_fwd_varlen_ex.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, p, i32, p, p, u32, i32,
                                           p]
    L.la_prefill_fwd_varlen.restype = ctypes.c_int
    L.la_prefill_fwd_varlen.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, p, i32, p, u32, i32, p]
    L.la_state_commit.restype = ctypes.c_int
    L.la_state_commit.argtypes = [p, p, i32, i32, i32, i32, i32, i32, p, p, i32, p, p, p]
    L.la_decode_mtp.restype = ctypes.c_int
    L.la_decode_mtp.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, p, i32, p, p]
    L.la_verify_kvbuffer.restype = ctypes.c_int
    L.la_verify_kvbuffer.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, p, i32, p, p, p, p]
    L.la_state_commit_kvbuffer.restype = ctypes.c_int
    L.la_state_commit_kvbuffer.argtypes = [p, p, i32, i32, i32, i32, i32, i32, p, p, i32, p, p, p]
    L.la_status_string.restype = ctypes.c_char_p
    L.la_status_string.argtypes = [ctypes.c_int]
    L.la_last_error.restype = ctypes.c_char_p
    L.la_last_error.argtypes = []
    L.la_abi_version.restype = i32
    L.la_abi_version.argtypes = []
    return L


lib = _load()


def _check(status):
    if status != LA_OK:
        raise LaError(status, f"{lib.la_status_string(status).decode()}: {lib.la_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, dev):
    import torch
    s = torch.cuda.current_stream(dev) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _req(t, name, dtype, dev):
    import torch
    if t is None:
        return
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must live on {dev}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _slope_len(slope, flags, H, HV):
    if slope is None:
        raise ValueError("slope is required")
    want = H if flags & LA_DECAY_PER_QK_HEAD else HV
    if slope.numel() != want:
        raise ValueError(f"slope must have {want} entries, got {slope.numel()}")


def _state_shapes(state_pool, HV, n, required=False, **idx):
    """The kernels index the pool as [P, HV, 128, 128] and read one entry of every index tensor per sequence: check
    the shapes here, since the library cannot see allocation sizes."""
    if state_pool is None:
        if required:
            raise ValueError("state_pool is required")
        return 0
    if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (HV, 128, 128):
        raise ValueError(f"state_pool must have shape [P, {HV}, 128, 128], got {tuple(state_pool.shape)}")
    for name, t in idx.items():
        if t is not None and t.numel() != n:
            raise ValueError(f"{name} must have {n} entries, got {t.numel()}")
    return state_pool.shape[0]


def la_prefill_fwd(q, k, v, o, slope, scale=1.0, state_pool=None, state_idx=None, flags=0, stream=None,
                   state_idx_out=None):
    """Fixed-length prefill. q, k: bf16 [B, T, H, 128]; v, o: bf16 [B, T, HV, 128]; slope: fp32 [HV] (or [H] with
    LA_DECAY_PER_QK_HEAD); state_pool: fp32 [P, HV, 128, 128]; state_idx: int32 [B]; flags: LA_STATE_READ |
    LA_STATE_WRITE | LA_DECAY_PER_QK_HEAD. state_idx_out (int32 [B]) selects la_prefill_fwd_ex."""
    if state_idx_out is not None:
        return la_prefill_fwd_ex(q, k, v, o, slope, scale, state_pool, state_idx, state_idx_out, flags, stream)
    import torch
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _req(t, n, torch.bfloat16, dev)
    _req(slope, "slope", torch.float32, dev)
    _req(state_pool, "state_pool", torch.float32, dev)
    _req(state_idx, "state_idx", torch.int32, dev)
    B, T, H, D = q.shape
    HV, DV = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or o.shape != v.shape:
        raise ValueError("shape mismatch between q, k, v, o")
    _slope_len(slope, flags, H, HV)
    P = _state_shapes(state_pool, HV, B, state_idx=state_idx)
    _check(lib.la_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, HV, D, DV, float(scale), _ptr(slope),
                              _ptr(state_pool), P, _ptr(state_idx), int(flags), _stream(stream, dev)))
    return o


def la_prefill_fwd_ex(q, k, v, o, slope, scale=1.0, state_pool=None, state_idx=None, state_idx_out=None, flags=0,
                      stream=None):
    """Fixed-length prefill whose final states go to state_idx_out (int32 [B]) instead of state_idx."""
    import torch
    dev = q.device
    B, T, H, HV, D, DV = _qkvo(q, k, v, o, dev)
    _req(slope, "slope", torch.float32, dev)
    _req(state_pool, "state_pool", torch.float32, dev)
    _req(state_idx, "state_idx", torch.int32, dev)
    _req(state_idx_out, "state_idx_out", torch.int32, dev)
    _slope_len(slope, flags, H, HV)
    P = _state_shapes(state_pool, HV, B, state_idx=state_idx, state_idx_out=state_idx_out)
    _check(lib.la_prefill_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, HV, D, DV, float(scale), _ptr(slope),
                                 _ptr(state_pool), P, _ptr(state_idx), _ptr(state_idx_out), int(flags),
                                 _stream(stream, dev)))
    return o


def la_prefill_fwd_varlen(q, k, v, o, cu_seqlens, slope, scale=1.0, state_pool=None, state_idx=None, flags=0,
                          schedule=LA_SCHED_AUTO, stream=None, state_idx_out=None):
    """Packed prefill. q, k: bf16 [total_T, H, 128]; v, o: bf16 [total_T, HV, 128]; cu_seqlens: int32 [N+1].
    state_idx_out (int32 [N]) selects la_prefill_fwd_varlen_ex."""
    import torch
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _req(t, n, torch.bfloat16, dev)
    _req(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _req(slope, "slope", torch.float32, dev)
    _req(state_pool, "state_pool", torch.float32, dev)
    _req(state_idx, "state_idx", torch.int32, dev)
    total_T, H, D = q.shape
    HV, DV = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != total_T or o.shape != v.shape:
        raise ValueError("shape mismatch between q, k, v, o")
    _req(state_idx_out, "state_idx_out", torch.int32, dev)
    _slope_len(slope, flags, H, HV)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
    N = cu_seqlens.shape[0] - 1
    P = _state_shapes(state_pool, HV, N, state_idx=state_idx, state_idx_out=state_idx_out)
    if state_idx_out is None:
        _check(lib.la_prefill_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(cu_seqlens), N, total_T, H, HV, D,
                                         DV, float(scale), _ptr(slope), _ptr(state_pool), P, _ptr(state_idx),
                                         int(flags), int(schedule), _stream(stream, dev)))
    else:
        _check(lib.la_prefill_fwd_varlen_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(cu_seqlens), N, total_T, H, HV,
                                            D, DV, float(scale), _ptr(slope), _ptr(state_pool), P, _ptr(state_idx),
                                            _ptr(state_idx_out), int(flags), int(schedule), _stream(stream, dev)))
    return o


def la_prefill_fwd_varlen_ex(q, k, v, o, cu_seqlens, slope, scale=1.0, state_pool=None, state_idx=None,
                             state_idx_out=None, flags=0, schedule=LA_SCHED_AUTO, stream=None):
    """Packed prefill whose final states go to state_idx_out (int32 [N]) instead of state_idx."""
    return la_prefill_fwd_varlen(q, k, v, o, cu_seqlens, slope, scale, state_pool, state_idx, flags, schedule, stream,
                                 state_idx_out=state_idx_out)


def la_state_commit(k, v, slope, state_pool, state_idx, accepted_len, stream=None):
    """Commit accepted draft tokens: k: bf16 [B, T, H, 128]; v: bf16 [B, T, HV, 128]; accepted_len: int32 [B]."""
    import torch
    dev = k.device
    _req(k, "k", torch.bfloat16, dev)
    _req(v, "v", torch.bfloat16, dev)
    _req(slope, "slope", torch.float32, dev)
    _req(state_pool, "state_pool", torch.float32, dev)
    _req(state_idx, "state_idx", torch.int32, dev)
    _req(accepted_len, "accepted_len", torch.int32, dev)
    B, T, H, D = k.shape
    HV, DV = v.shape[2], v.shape[3]
    if v.shape[:2] != (B, T):
        raise ValueError("shape mismatch between k and v")
    _slope_len(slope, 0, H, HV)
    P = _state_shapes(state_pool, HV, B, required=True, state_idx=state_idx, accepted_len=accepted_len)
    _check(lib.la_state_commit(_ptr(k), _ptr(v), B, T, H, HV, D, DV, _ptr(slope), _ptr(state_pool),
                               P, _ptr(state_idx), _ptr(accepted_len), _stream(stream, dev)))
    return state_pool


def _qkvo(q, k, v, o, dev):
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _req(t, n, torch.bfloat16, dev)
    B, T, H, D = q.shape
    HV, DV = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or o.shape != v.shape:
        raise ValueError("shape mismatch between q, k, v, o")
    return B, T, H, HV, D, DV


def la_decode_mtp(q, k, v, o, slope, state_pool, state_idx, scale=1.0, stream=None):
    """Multi-token decode: outputs of all T draft tokens, and each request's state advanced over them in place."""
    import torch
    dev = q.device
    B, T, H, HV, D, DV = _qkvo(q, k, v, o, dev)
    _req(slope, "slope", torch.float32, dev)
    _req(state_pool, "state_pool", torch.float32, dev)
    _req(state_idx, "state_idx", torch.int32, dev)
    _slope_len(slope, 0, H, HV)
    P = _state_shapes(state_pool, HV, B, required=True, state_idx=state_idx)
    _check(lib.la_decode_mtp(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, HV, D, DV, float(scale), _ptr(slope),
                             _ptr(state_pool), P, _ptr(state_idx), _stream(stream, dev)))
    return o


def la_verify_kvbuffer(q, k, v, o, slope, state_pool, state_idx, k_buf=None, v_buf=None, scale=1.0, stream=None):
    """Verify T draft tokens from each request's pooled state (read only); optionally copy their k/v rows into
    k_buf: bf16 [P, T, H, 128] and v_buf: bf16 [P, T, HV, 128] at the request's slot."""
    import torch
    dev = q.device
    B, T, H, HV, D, DV = _qkvo(q, k, v, o, dev)
    _req(slope, "slope", torch.float32, dev)
    _req(state_pool, "state_pool", torch.float32, dev)
    _req(state_idx, "state_idx", torch.int32, dev)
    _slope_len(slope, 0, H, HV)
    P = _state_shapes(state_pool, HV, B, required=True, state_idx=state_idx)
    for t, n, heads in ((k_buf, "k_buf", H), (v_buf, "v_buf", HV)):
        _req(t, n, torch.bfloat16, dev)
        if t is not None and tuple(t.shape) != (P, T, heads, 128):
            raise ValueError(f"{n} must have shape {(P, T, heads, 128)}, got {tuple(t.shape)}")
    _check(lib.la_verify_kvbuffer(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, HV, D, DV, float(scale), _ptr(slope),
                                  _ptr(state_pool), P, _ptr(state_idx), _ptr(k_buf), _ptr(v_buf),
                                  _stream(stream, dev)))
    return o


def la_state_commit_kvbuffer(k_buf, v_buf, slope, state_pool, state_idx, accepted_len, stream=None):
    """Commit accepted draft tokens read from the KV buffer: k_buf: bf16 [P, T, H, 128]; v_buf: bf16
    [P, T, HV, 128]; accepted_len: int32 [B]."""
    import torch
    dev = k_buf.device
    _req(k_buf, "k_buf", torch.bfloat16, dev)
    _req(v_buf, "v_buf", torch.bfloat16, dev)
    _req(slope, "slope", torch.float32, dev)
    _req(state_pool, "state_pool", torch.float32, dev)
    _req(state_idx, "state_idx", torch.int32, dev)
    _req(accepted_len, "accepted_len", torch.int32, dev)
    P, T, H, D = k_buf.shape
    HV, DV = v_buf.shape[2], v_buf.shape[3]
    if v_buf.shape[:2] != (P, T) or state_pool is None or state_pool.shape[0] != P:
        raise ValueError("k_buf, v_buf and state_pool must share the slot count and T")
    if state_idx is None or accepted_len is None:
        raise ValueError("state_idx and accepted_len are required")
    B = state_idx.numel()
    _slope_len(slope, 0, H, HV)
    _state_shapes(state_pool, HV, B, required=True, state_idx=state_idx, accepted_len=accepted_len)
    _check(lib.la_state_commit_kvbuffer(_ptr(k_buf), _ptr(v_buf), B, T, H, HV, D, DV, _ptr(slope),
                                        _ptr(state_pool), P, _ptr(state_idx), _ptr(accepted_len),
                                        _stream(stream, dev)))
    return state_pool


def la_prefill_seg_workspace_bytes(B, HV, segments):
    return int(lib.la_prefill_seg_workspace_bytes(int(B), int(HV), int(segments)))


def la_prefill_fwd_seg(q, k, v, o, slope, scale=1.0, state_pool=None, state_idx=None, state_idx_out=None, flags=0,
                       segments=0, workspace=None, stream=None):
    """Fixed-length prefill with every sequence split into segments run in parallel (segments = 0: chosen from the
    CU count). workspace: a contiguous device tensor of at least la_prefill_seg_workspace_bytes(B, HV, segments)
    bytes (for segments = 0, of the count la_prefill_fwd_seg may choose: use la_prefill_seg_workspace_bytes with
    max(1, CUs // (2 B HV)))."""
    import torch
    dev = q.device
    B, T, H, HV, D, DV = _qkvo(q, k, v, o, dev)
    _req(slope, "slope", torch.float32, dev)
    _req(state_pool, "state_pool", torch.float32, dev)
    _req(state_idx, "state_idx", torch.int32, dev)
    _req(state_idx_out, "state_idx_out", torch.int32, dev)
    _slope_len(slope, flags, H, HV)
    if workspace is not None and (not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    P = _state_shapes(state_pool, HV, B, state_idx=state_idx, state_idx_out=state_idx_out)
    _check(lib.la_prefill_fwd_seg(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, HV, D, DV, float(scale), _ptr(slope),
                                  _ptr(state_pool), P, _ptr(state_idx), _ptr(state_idx_out), int(flags),
                                  int(segments), _ptr(workspace), nbytes, _stream(stream, dev)))
    return o


def la_prefill_seg_noalloc_max_bytes():
    return int(lib.la_prefill_seg_noalloc_max_bytes())


def la_prefill_fwd_seg_noalloc(q, k, v, o, slope, scale=1.0, state_pool=None, state_idx=None, state_idx_out=None,
                               flags=0, segments=0, stream=None):
    """la_prefill_fwd_seg with the segment states in the library's fixed device array: no workspace and no
    allocation. Calls that overlap on one device race on that array."""
    import torch
    dev = q.device
    B, T, H, HV, D, DV = _qkvo(q, k, v, o, dev)
    _req(slope, "slope", torch.float32, dev)
    _req(state_pool, "state_pool", torch.float32, dev)
    _req(state_idx, "state_idx", torch.int32, dev)
    _req(state_idx_out, "state_idx_out", torch.int32, dev)
    _slope_len(slope, flags, H, HV)
    P = _state_shapes(state_pool, HV, B, state_idx=state_idx, state_idx_out=state_idx_out)
    _check(lib.la_prefill_fwd_seg_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, T, H, HV, D, DV, float(scale),
                                          _ptr(slope), _ptr(state_pool), P, _ptr(state_idx), _ptr(state_idx_out),
                                          int(flags), int(segments), _stream(stream, dev)))
    return o

"""Seeded synthetic inputs for the Lightning Attention prefill path.

Shared by the tests, the smoke check and the benchmark; feeds both the CPU oracle and the HIP path. It holds
random draws, bf16 rounding and workload shapes only -- none of the method's arithmetic.

Recipe (one numpy PCG64 generator per workload, ``numpy.random.default_rng(seed)``):
  * structure first when it decides shapes: packed sequence lengths ~ U{1..max_len};
  * then q, k ~ N(0, 1/128), v ~ N(0, 1) drawn as float32 (the second argument of N(.,.) is read as the
    variance), rounded to nearest-even bf16 (stored as uint16 bit patterns);
  * then the FP32 state pool ~ N(0, 0.01);
  * then slot indices (a permutation of the pool), skipped sequences (index -1), accepted lengths U{0..T}.
Slopes: slope_h = 2^(-8 (h+1) / n) for head h of n heads (per q/k head for MHA, per value head for GVA).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 128
DV = 128
Q_STD = 1.0 / np.sqrt(128.0)
V_STD = 1.0
S0_STD = 0.1


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bf16 with round-to-nearest-even; returns uint16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).reshape(-1)
    out = np.empty(u.shape, dtype=np.uint16)
    blk = 1 << 22                      # in cache-sized blocks: large inputs are tens of millions of elements
    r = np.empty(min(blk, u.size), dtype=np.uint32)
    for a in range(0, u.size, blk):
        ub = u[a:a + blk]
        rb = r[:ub.size]
        np.right_shift(ub, 16, out=rb)
        np.bitwise_and(rb, 1, out=rb)
        rb += np.uint32(0x7FFF)
        rb += ub
        rb >>= 16
        out[a:a + ub.size] = rb
    return out.reshape(np.shape(x))


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def slopes(n: int) -> np.ndarray:
    h = np.arange(n, dtype=np.float64)
    return np.power(2.0, -8.0 * (h + 1) / n).astype(np.float32)


def _normal_bf16(rng, shape, std):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(std)
    return bf16_bits(x)


@dataclass
class Workload:
    name: str
    mode: str                      # "fixed" | "varlen" | "verify"
    H: int
    HV: int
    q: np.ndarray                  # uint16 [..., H, D]
    k: np.ndarray
    v: np.ndarray                  # uint16 [..., HV, DV]
    slope: np.ndarray              # float32 [HV]
    scale: float = 1.0
    B: int = 0
    T: int = 0
    cu_seqlens: np.ndarray | None = None   # int32 [N+1] (varlen)
    pool: np.ndarray | None = None         # float32 [P, HV, DV, D]
    state_idx: np.ndarray | None = None    # int32 [B or N]
    flags: int = 0
    accepted_len: np.ndarray | None = None  # int32 [B] (verify/commit)
    meta: dict = field(default_factory=dict)

    @property
    def nseq(self):
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def seq_rows(self):
        """(row0, length) per sequence."""
        if self.cu_seqlens is None:
            return [(b * self.T, self.T) for b in range(self.B)]
        cu = self.cu_seqlens
        return [(int(cu[n]), int(cu[n + 1] - cu[n])) for n in range(len(cu) - 1)]

    @property
    def tokens(self):
        return sum(l for _, l in self.seq_rows())


def fixed(seed, B, T, H, HV, *, pool_slots=0, state_idx=None, flags=0, slope_per="h", scale=1.0,
          s0_std=S0_STD, name="fixed"):
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (B, T, H, D), Q_STD)
    k = _normal_bf16(rng, (B, T, H, D), Q_STD)
    v = _normal_bf16(rng, (B, T, HV, DV), V_STD)
    pool = None
    if pool_slots:
        pool = rng.standard_normal(size=(pool_slots, HV, DV, D), dtype=np.float32)
        pool *= np.float32(s0_std)
    if slope_per == "h":
        sl = np.repeat(slopes(H), HV // H)
    else:
        sl = slopes(HV)
    idx = None if state_idx is None else np.asarray(state_idx, dtype=np.int32)
    return Workload(name=name, mode="fixed", H=H, HV=HV, q=q, k=k, v=v, slope=sl, scale=scale, B=B, T=T,
                    pool=pool, state_idx=idx, flags=flags)


def varlen(seed, N, max_len, H, HV, *, pool_slots=32, n_skip=2, flags=3, scale=1.0, lengths=None,
           name="varlen"):
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(1, max_len + 1, size=N)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    tot = int(cu[-1])
    q = _normal_bf16(rng, (tot, H, D), Q_STD)
    k = _normal_bf16(rng, (tot, H, D), Q_STD)
    v = _normal_bf16(rng, (tot, HV, DV), V_STD)
    pool = None
    idx = None
    if pool_slots:
        pool = rng.standard_normal(size=(pool_slots, HV, DV, D), dtype=np.float32)
        pool *= np.float32(S0_STD)
        idx = rng.permutation(pool_slots)[:len(lengths)].astype(np.int32)
        if n_skip:
            skip = rng.choice(len(lengths), size=min(n_skip, len(lengths)), replace=False)
            idx[skip] = -1
    sl = np.repeat(slopes(H), HV // H)
    return Workload(name=name, mode="varlen", H=H, HV=HV, q=q, k=k, v=v, slope=sl, scale=scale,
                    cu_seqlens=cu, pool=pool, state_idx=idx, flags=flags)


def verify(seed, B, T, H, HV, *, pool_slots=128, name="verify"):
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (B, T, H, D), Q_STD)
    k = _normal_bf16(rng, (B, T, H, D), Q_STD)
    v = _normal_bf16(rng, (B, T, HV, DV), V_STD)
    pool = rng.standard_normal(size=(pool_slots, HV, DV, D), dtype=np.float32)
    pool *= np.float32(S0_STD)
    idx = rng.permutation(pool_slots)[:B].astype(np.int32)
    acc = rng.integers(0, T + 1, size=B).astype(np.int32)
    sl = np.repeat(slopes(H), HV // H)
    return Workload(name=name, mode="verify", H=H, HV=HV, q=q, k=k, v=v, slope=sl, B=B, T=T, pool=pool,
                    state_idx=idx, flags=1, accepted_len=acc)


# The five workloads the path is measured and checked on.
def config(i: int) -> Workload:
    if i == 0:
        # Tiny fixed-length prefill; zero initial state, final state returned.
        return fixed(0, 1, 256, 4, 4, pool_slots=1, state_idx=[0], flags=2, name="cfg0_tiny")
    if i == 1:
        # Fixed-length MHA prefill B=2, T=8192, H=HV=64; state read from and written back to a 2-slot pool.
        return fixed(1, 2, 8192, 64, 64, pool_slots=2, state_idx=[0, 1], flags=3, name="cfg1_b2_t8192_h64")
    if i == 2:
        # Packed varlen: 16 sequences, lengths U{1..4096}, 32-slot pool, two sequences skip state.
        return varlen(2, 16, 4096, 64, 64, pool_slots=32, n_skip=2, flags=3, name="cfg2_varlen_n16")
    if i == 3:
        # GVA: B=4, T=16384, 16 q/k heads shared by 4 value heads each (HV=64); per-value-head slopes.
        return fixed(3, 4, 16384, 16, 64, pool_slots=4, state_idx=[0, 1, 2, 3], flags=2, slope_per="hv",
                     name="cfg3_gva_b4_t16384")
    if i == 4:
        # Short-chunk verify: B=128 requests, T=8 drafts, 128-slot pool; then commit accepted lengths.
        return verify(4, 128, 8, 64, 64, pool_slots=128, name="cfg4_verify_b128_t8")
    if i == 5:
        # One long prompt with few heads (B=1, T=32768, H=HV=16): too few (sequence, head) units to fill the GPU,
        # the case the segmented prefill is for. State read from and written back to a 1-slot pool.
        return fixed(5, 1, 32768, 16, 16, pool_slots=1, state_idx=[0], flags=3, name="cfg5_long_b1_t32768_h16")
    raise ValueError(i)

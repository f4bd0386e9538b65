// la_prefill.hip -- Lightning Attention chunked prefill for AMD Instinct MI355X (gfx950, CDNA4), and the C ABI
// entry points of the prefill, commit and segmented calls.
//
// Computes, per (sequence, value head), the decayed linear-attention recurrence
//     S_t = lambda S_{t-1} + v_t k_t^T,   o_t = scale S_t q_t,   lambda = exp(-slope[hv])
// (page "[LA] Lightning Attention MTP decode + KVBuffer parallel verify / commit", Description, closed form
// used by verify) in 64-token chunks (page "[Lightning Attention] Add Hopper SM90 CuTe DSL prefill",
// Description: FP32 recurrent state resident across 64-token chunks). For a chunk of Lc tokens, local
// positions i, j in [0, Lc), and state S (before the chunk):
//     O_j = scale * ( sum_{i<=j} lambda^{j-i} (q_j . k_i) v_i  +  lambda^{j+1} S q_j )
//     S  <- lambda^{Lc} S + sum_i k_i (lambda^{Lc-1-i} v_i)^T      (kept as S^T[k][v] on chip)
//
// Work decomposition: one workgroup = (sequence, value head, half of the 128 value columns), 8 wave64s. The 4
// consumer waves each own value columns [16w, 16w+16) of the half: the state rows S[v][0..127] for those
// columns stay in that wave's registers as MFMA accumulators for the whole sequence. The 4 producer waves
// compute the decay-masked intra-chunk scores; two of them also stage Q, K, V tiles into LDS one chunk ahead
// and store the output tiles the consumers leave in LDS. The same kernel also runs the two chunked passes of a
// sequence split into segments (local segment states from zero; every segment from its initial state).
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, FP32 accumulate). Every operand fragment a lane holds is
// "row r = lane % 16, slot group g = lane / 16, 8 slots"; slots 0..3 carry contraction indices 4g..4g+3 of
// one 16-wide block and slots 4..7 carry 4g..4g+3 of the next block. The 16x16 accumulator of the same
// instruction holds, per lane, column lane % 16 and rows 4g..4g+3. Chaining works because an accumulator
// tile [m][n] is, lane for lane, a fragment with row n and contraction index m: scores computed as
// A^T[i][j] feed the P.V product as P[j][i] fragments; the state kept as S^T[k][v] feeds Q.S^T as S[v][k]
// fragments. K^T and V^T fragments come from transposing LDS reads (ds_read_b64_tr_b16).
//
// Precision: the state update multiplies the per-token decay into V (V_dec = lambda^{Lc-1-i} v_i) in FP32
// and feeds it as a bf16 hi + lo pair; the FP32 state enters Q S^T as a bf16 hi + lo pair; the decay-masked
// scores P enter P.V as a bf16 hi + lo pair (the state owners take the residuals of their two splits from an
// MFMA against minus the identity, the producers from v_dot2c). Q, K, V are exact in bf16. Every exponent
// handed to exp2 is <= 0, so powers of lambda can only underflow. O is rounded to bf16 once, round-to-nearest-even.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <stdio.h>
#include <stdarg.h>
#include <string.h>

#include "la_common.h"

using namespace la_detail;

namespace {

constexpr int kC = 64;                    // chunk length (tokens)
constexpr int kVSplit = 2;                // workgroups per (sequence, value head)
constexpr int kVW = kDV / kVSplit;        // value columns per workgroup
constexpr int kThreads = 512;             // 4 consumer waves (one 16-column value tile each) + 4 producer waves

// kSegStates / kSegFwd: the two chunked passes of a sequence split into segments of seg_len tokens (unit index
// seq = b * segments-per-sequence + g): local states of every segment but the last, from zero; then the full
// prefill of every segment from its true initial state
enum Mode { kFixed = 0, kVarlen = 1, kCommit = 2, kSegStates = 3, kSegFwd = 4 };

struct Params {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    uint16_t *o;
    const int32_t *cu_seqlens;
    const int32_t *accepted_len;
    const float *slope;
    float *pool;
    const int32_t *state_idx;
    const int32_t *state_idx_out;   // slot that receives the final state; NULL: the slot read from
    float *seg_states;              // segmented passes: [B * nseg, HV, 128, 128] segment initial / local states
    int32_t seg_len;                // segmented passes: tokens per segment (a multiple of 64)
    int32_t nseg;                   // segmented passes: segments per sequence
    int32_t nseq;
    int32_t T;          // fixed / commit: tokens per sequence
    int32_t total_T;    // varlen: rows in q/k/v
    int32_t H;
    int32_t HV;
    int32_t G;
    int32_t pool_size;
    int32_t npairs;     // nseq * HV
    int32_t nunits;     // npairs * kVSplit
    float scale;
    uint32_t flags;
};

struct Unit {
    int32_t seq, hv, vpart;
};

// Workgroup -> (sequence, value head, value half). The units that read the same Q/K rows -- the G value heads
// of one (sequence, q/k head) group, times the two value halves -- get indices 8 apart: workgroups are dealt
// round-robin over the 8 XCDs, so the whole group lands on one XCD, in consecutive dispatch slots, and shares
// that XCD's L2 for the Q/K tiles. Groups are dealt over the XCDs in rows of 8; a last partial row of m groups
// interleaves its units over all XCDs.
__device__ __forceinline__ Unit decode_unit(int u, const Params &p) {
    const int per = kVSplit * p.G;           // units per group
    const int ngroups = p.npairs / p.G;      // nseq * H
    const int full = ngroups >> 3;           // complete rows of 8 groups
    int group, j;
    if (u < full * 8 * per) {
        const int slot = u >> 3;             // dispatch slot on XCD u % 8
        const int row = slot / per;
        group = row * 8 + (u & 7);
        j = slot - row * per;
    } else {
        const int m = ngroups - full * 8;
        const int r = u - full * 8 * per;
        group = full * 8 + r % m;
        j = r / m;
    }
    const int half = j / p.G;
    const int seq = group / p.H;
    Unit t;
    t.seq = seq;
    t.hv = (group - seq * p.H) * p.G + (j - half * p.G);
    t.vpart = half;
    return t;
}

// ---------------------------------------------------------------------------------------------------------
// LDS layout (one workgroup per CU; 160 KiB).
//   Q, K tiles: 64 rows x 256 B; V tiles (one value half): 64 rows x 128 B. Row-major as in HBM, with the
//   16-byte segments of row r stored at segment index seg XOR (r % 16) for Q, seg XOR f(r % 16) for K
//   (f swaps the two 2-bit halves of its argument) and seg XOR 2((r/2) % 4) for V. LDS serves a 16-byte read
//   as pairs of 8-lane groups and an 8-byte read as pairs of 16-lane groups, each group within one 128-byte
//   bank half and the two groups in opposite halves: the Q pattern makes 16-row fragment reads conflict-free;
//   the K pattern spreads the transposing reads (4 rows x 4 segments per 16 lanes) to the two-way minimum
//   that a read of one 8-byte half of every segment allows; the V pattern makes the transposing reads of one
//   value tile (4 rows x 2 segments per 16 lanes) conflict-free. The tiles are filled
//   by buffer loads that write LDS directly; the XOR is applied on the source side (lane -> segment), and
//   rows past the end of a sequence fall outside the buffer range and arrive as zeros.
//   Q, K, V: 2 buffers each. In the iteration that handles chunk c, both roles read chunk c's tiles while
//   chunk c+1's loads, issued at the start of the iteration, land in the other buffers; the producers wait for
//   them before the iteration's barrier. (One iteration covers the load latency: a third buffer, with loads two
//   chunks ahead, measured no faster.)
//   P: 2 buffers of 6 lower-triangle (jt, token-pair) fragment blocks, hi and lo, 64 lanes x 16 B each:
//   written for chunk c by the producers while the consumers read chunk c-1's.
//   O: 2 buffers of one output tile (64 rows x 128 B, bf16, segments at seg XOR ((r/2) % 8), which spreads the
//   consumers' 8-byte row writes of 16 rows over the banks): the consumers write chunk c-1's
//   output in iteration c; the producers store it to HBM in iteration c+1 as whole 128-byte row halves.
// ---------------------------------------------------------------------------------------------------------
constexpr int kQKTileB = kC * kD * 2;        // 16384
constexpr int kVTileB = kC * kVW * 2;        // 8192
constexpr int kFragB = 64 * 16;              // one fragment block
constexpr int kPBufB = 6 * 2 * kFragB;       // 12288
constexpr int kOffQ = 0;
constexpr int kOffK = kOffQ + 2 * kQKTileB;
constexpr int kOffV = kOffK + 2 * kQKTileB;
constexpr int kOffP = kOffV + 2 * kVTileB;
constexpr int kOTileB = kC * kVW * 2;        // 8192
constexpr int kOffO = kOffP + 2 * kPBufB;
constexpr int kLdsBytes = kOffO + 2 * kOTileB;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int q_swz(int r) { return r & 15; }
__device__ __forceinline__ int k_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int q_seg_off(int r, int seg) { return r * 256 + ((seg ^ q_swz(r)) << 4); }
__device__ __forceinline__ int k_seg_off(int r, int seg) { return r * 256 + ((seg ^ k_swz(r)) << 4); }
// output tile
__device__ __forceinline__ int v_seg_off(int r, int seg) { return r * 128 + ((seg ^ ((r >> 1) & 7)) << 4); }
// V tile: rows 4g .. 4g+3 of a transposing read fall in alternate bank halves; the XOR 2((r/2) % 4) puts the
// 32 bytes that rows 4g and 4g+2 (and 4g+1, 4g+3) give one value tile into different banks
__device__ __forceinline__ int vt_swz(int r) { return ((r >> 1) & 3) << 1; }
__device__ __forceinline__ int vt_seg_off(int r, int seg) { return r * 128 + ((seg ^ vt_swz(r)) << 4); }

// 8 consecutive elements of a Q or K row: columns 8*seg .. 8*seg+7 (16-byte read)
__device__ __forceinline__ u32x4 ld16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
// transposing read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element i % 4 of the 8 bytes
// that lane 4e + i / 4 addresses, as its element e
__device__ __forceinline__ u32x2 ld_tr(const uint8_t *p) {
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
    return __builtin_bit_cast(u32x2, x);
}
__device__ __forceinline__ int p_blk(int jt, int ip) { return jt < 2 ? jt : 2 * jt - 2 + ip; }

// x = hi + lo for the 4 values a lane holds of a 16x16 accumulator tile, hi = bf16(x), lo = bf16(x - hi). The
// residual x - hi (exact in FP32) comes from one 16x16x16 MFMA: D = x + (-I) hi, with hi as the B operand,
// whose lane layout (lane (n, g) holds rows 4g .. 4g+3 of column n) is that of the accumulator. The state owners
// use this instead of v_dot2c residuals: beside MFMA work on the same SIMD a v_dot2c issues at less than half its
// rate alone, while the MFMA takes the matrix pipe for 16 cycles per 4 values.
__device__ __forceinline__ void split4_mfma(f32x4 x, s16x4 neg_ident, uint32_t &h0, uint32_t &h1, uint32_t &l0,
                                            uint32_t &l1) {
    h0 = pack_bf16x2(x[0], x[1]);
    h1 = pack_bf16x2(x[2], x[3]);
    const f32x4 r = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(neg_ident, __builtin_bit_cast(s16x4, u32x2{h0, h1}),
                                                              x, 0, 0, 0);
    l0 = pack_bf16x2(r[0], r[1]);
    l1 = pack_bf16x2(r[2], r[3]);
}

// ---------------------------------------------------------------------------------------------------------
// Producer: scores A^T[i][j] = K_i . Q_j for the lower-triangle 16x16 tiles of the block it in
// [IT0, IT0+NI), jt in [JT0, JT0+NJ), with the d-contraction taken over 8 consecutive columns per slot
// group; decay mask P = scale lambda^{j-i} A (i <= j) stored as bf16 hi + lo fragments; a strictly-upper
// tile inside a diagonal block pair is stored as zeros.
//   producer 0: (0..1, 2)   producer 1: (0..1, 3)   producer 2: (2..3, 2..3)   producer 3: (0..1, 0..1)
// ---------------------------------------------------------------------------------------------------------
template <int IT0, int NI, int JT0, int NJ>
__device__ __forceinline__ void score_factors(float (&pf)[16], float l2, float scale, int lr, int lg) {
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * (IT0 + ii) + 4 * lg + r, j = 16 * (JT0 + jj) + lr;
                pf[4 * (NJ * ii + jj) + r] = (IT0 + ii <= JT0 + jj && i <= j) ? scale * lam_pow(l2, j - i) : 0.f;
            }
}

template <int IT0, int NI, int JT0, int NJ>
__device__ __forceinline__ void produce_scores(const float (&pf)[16], const uint8_t *tq, const uint8_t *tk,
                                               uint8_t *pbuf, int lane, int lr, int lg) {
    f32x4 a[NI][NJ];
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) a[ii][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
        u32x4 kf[NI], qf[NJ];
#pragma unroll
        for (int x = 0; x < NI; ++x) kf[x] = ld16(tk + k_seg_off(16 * (IT0 + x) + lr, 4 * kp + lg));
#pragma unroll
        for (int x = 0; x < NJ; ++x) qf[x] = ld16(tq + q_seg_off(16 * (JT0 + x) + lr, 4 * kp + lg));
#pragma unroll
        for (int ii = 0; ii < NI; ++ii)
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
                if (IT0 + ii <= JT0 + jj) a[ii][jj] = mfma32(kf[ii], qf[jj], a[ii][jj]);
    }
    // every producer block covers whole (jt, token-pair) fragment blocks: NI = 2 with IT0 even, so tiles
    // (IT0, jt) and (IT0+1, jt) fill the two 8-byte halves of one block (a strictly-upper tile as zeros)
    static_assert(NI == 2 && (IT0 & 1) == 0, "producer blocks pair token tiles");
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
        const int jt = JT0 + jj;
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int it = IT0 + ii;
            if (it <= jt) {
                const float *f = &pf[4 * (NJ * ii + jj)];
                const u32x2 a01 = split_bf16x2(a[ii][jj][0] * f[0], a[ii][jj][1] * f[1]);
                const u32x2 a23 = split_bf16x2(a[ii][jj][2] * f[2], a[ii][jj][3] * f[3]);
                hi[2 * ii] = a01.x; hi[2 * ii + 1] = a23.x;
                lo[2 * ii] = a01.y; lo[2 * ii + 1] = a23.y;
            } else {
                hi[2 * ii] = hi[2 * ii + 1] = lo[2 * ii] = lo[2 * ii + 1] = 0u;
            }
        }
        uint8_t *dst = pbuf + (p_blk(jt, IT0 >> 1) * 2) * kFragB + lane * 16;
        *reinterpret_cast<u32x4 *>(dst) = u32x4{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<u32x4 *>(dst + kFragB) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
}

// ---------------------------------------------------------------------------------------------------------
// the kernel: 8 waves; waves 0..3 are consumers (state owners), waves 4..7 producers.
//
// Iteration c (one workgroup barrier at its end): the producers issue the staging loads of chunk c+1 and
// compute chunk c's decay-masked scores P; the consumers finish chunk c-1's output (P of chunk c-1 from the
// previous iteration, its history term from registers) and take chunk c's history term Q S^T and state
// update. The producers wait for chunk c+1's loads before the barrier, so each chunk's loads overlap one
// iteration of compute.
// ---------------------------------------------------------------------------------------------------------

// s_waitcnt with vmcnt(N), lgkmcnt(0) and no expcnt wait (gfx9 encoding: vmcnt bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8])
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Passes every field of the parameters through an empty asm, so that values derived from them count as
// computed anew wherever the copy is made.
__device__ __forceinline__ void opaque_params(Params &p) {
    asm volatile("" : "+s"(p.q), "+s"(p.k), "+s"(p.v), "+s"(p.o), "+s"(p.cu_seqlens), "+s"(p.accepted_len));
    asm volatile("" : "+s"(p.slope), "+s"(p.pool), "+s"(p.state_idx), "+s"(p.state_idx_out), "+s"(p.seg_states));
    asm volatile("" : "+s"(p.seg_len), "+s"(p.nseg), "+s"(p.nseq), "+s"(p.T), "+s"(p.total_T), "+s"(p.H), "+s"(p.HV),
                 "+s"(p.G), "+s"(p.pool_size), "+s"(p.npairs), "+s"(p.nunits), "+s"(p.scale), "+s"(p.flags));
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void la_chunk_kernel(Params params) {
    constexpr bool kOut = (MODE != kCommit && MODE != kSegStates);
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];

    const int tid = threadIdx.x;

    for (int u = blockIdx.x; u < params.nunits; u += gridDim.x) {
        // The parameters, lane and wave indices are re-derived through opaque copies in every unit iteration,
        // so that the compiler does not hoist set-up derived from them (decay exponents, masks, addresses, the
        // LDS destinations of the staging loads) out of this loop for both roles and keep it live in registers
        // for the whole kernel.
        Params p = params;
        opaque_params(p);
        int tid_u = tid;
        asm volatile("" : "+v"(tid_u));
        const int w = __builtin_amdgcn_readfirstlane(tid_u >> 6);   // wave index, uniform: role branches are scalar
        const bool consumer = w < 4;
        const int cw = w & 3;            // consumer: value tile; producer: producer index
        const int lane = tid_u & 63;
        const int lr = lane & 15;
        const int lg = lane >> 4;

        const Unit un = decode_unit(u, p);
        const int h = un.hv / p.G;
        const int v0 = un.vpart * kVW;

        int64_t row0;
        int len;
        // Values read from device memory (sequence bounds, accepted lengths, slots) are the same for every lane;
        // readfirstlane makes that visible to the compiler, so that the buffer descriptors built from them stay
        // in scalar registers instead of being wrapped in per-lane loops.
        if (MODE == kVarlen) {
            int a = __builtin_amdgcn_readfirstlane(p.cu_seqlens[un.seq]);
            int b = __builtin_amdgcn_readfirstlane(p.cu_seqlens[un.seq + 1]);
            a = min(max(a, 0), p.total_T);
            b = min(max(b, a), p.total_T);
            row0 = a;
            len = b - a;
        } else if (MODE == kCommit) {
            row0 = (int64_t)un.seq * p.T;
            len = min(max(__builtin_amdgcn_readfirstlane(p.accepted_len[un.seq]), 0), p.T);
        } else if (MODE == kSegStates || MODE == kSegFwd) {
            const int per = (MODE == kSegStates) ? p.nseg - 1 : p.nseg;
            const int b = un.seq / per, g = un.seq - b * per;
            row0 = (int64_t)b * p.T + (int64_t)g * p.seg_len;
            len = min(p.seg_len, p.T - g * p.seg_len);
        } else {
            row0 = (int64_t)un.seq * p.T;
            len = p.T;
        }
        // state source and destination planes of this unit (value head un.hv)
        const float *s_in = nullptr;
        float *s_out = nullptr;
        {
            constexpr int64_t kPlane = kDV * kD;
            if (MODE == kSegStates) {
                // local state of segment g from zero, stored as entry b * nseg + g + 1 of the segment buffer
                const int b = un.seq / (p.nseg - 1), g = un.seq - b * (p.nseg - 1);
                s_out = p.seg_states + ((int64_t)(b * p.nseg + g + 1) * p.HV + un.hv) * kPlane;
            } else {
                int bseq = un.seq, g = 0;
                if (MODE == kSegFwd) {
                    bseq = un.seq / p.nseg;
                    g = un.seq - bseq * p.nseg;
                    s_in = p.seg_states + ((int64_t)un.seq * p.HV + un.hv) * kPlane;
                }
                if (p.flags & (LA_STATE_READ | LA_STATE_WRITE)) {
                    int slot = -1;
                    const int s = __builtin_amdgcn_readfirstlane(p.state_idx[bseq]);
                    if (s >= 0 && s < p.pool_size) slot = s;
                    int slot_out = slot;
                    if (p.state_idx_out) {
                        const int so = __builtin_amdgcn_readfirstlane(p.state_idx_out[bseq]);
                        slot_out = (so >= 0 && so < p.pool_size) ? so : -1;
                    }
                    if (MODE == kCommit) {
                        // skipped request / L = 0: no write at all
                        if (slot < 0 || len == 0) continue;
                        s_in = s_out = p.pool + ((int64_t)slot * p.HV + un.hv) * kPlane;
                    } else {
                        if (MODE != kSegFwd && slot >= 0 && (p.flags & LA_STATE_READ))
                            s_in = p.pool + ((int64_t)slot * p.HV + un.hv) * kPlane;
                        if (slot_out >= 0 && (p.flags & LA_STATE_WRITE) && (MODE != kSegFwd || g == p.nseg - 1))
                            s_out = p.pool + ((int64_t)slot_out * p.HV + un.hv) * kPlane;
                    }
                } else if (MODE == kCommit) {
                    continue;
                }
            }
        }

        const float l2 = log2_lambda(p.slope[(p.flags & LA_DECAY_PER_QK_HEAD) ? h : un.hv]);
        const int nch = (len + kC - 1) / kC;
        const int qk_stride = p.H * kD * 2;                          // bytes between token rows
        const int v_stride = p.HV * kDV * 2;

        // The two roles run separate code with the same number of workgroup barriers (nch + 2 per unit), so
        // each role's loop-carried registers are allocated on their own.
        if (consumer) {
            // ======================================== consumer: owns the state rows of value tile cw
            // State tiles S[kt] (kt = 0..7), lane holds S[v][k] for v = v0 + 16cw + lr and the four keys
            // k = kappa(kt, 4lg + r) = 32(kt/2) + 8lg + 4(kt%2) + r, r = 0..3: the key order inside a tile is
            // chosen (through the transposing K reads that build the K^T fragments) so that tiles 2s and 2s+1
            // give each lane 8 consecutive keys -- the slot layout of a plain 16-byte Q row read.
            f32x4 S[8];
            float finter[4];            // scale lambda^{j+1} for j = 16jt+lr
            const float dec64 = lam_pow(l2, kC);
            const int vrow = v0 + 16 * cw + lr;
            if (s_in) {
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
                    S[kt] = *reinterpret_cast<const f32x4 *>(s_in + vrow * kD + 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1));
            } else {
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) S[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            float fvd64[16];            // V_dec factors of a full chunk, lambda^{63-i} for i = 16it+4lg+r
            s16x4 neg_ident;
            // per-lane LDS offsets reused by every chunk: Q fragment (row lr, segment 4s + lg; row tile jt adds
            // 4096 B); K^T source of key group s: lane (lg, lr) supplies token row 4lg + lr/4 (+ 32 per token
            // pair, + 16 for slots 4..7) and the 4 keys 32s + 8(lr%4) + 4kk .. +3; the transposing read hands
            // lane lr of each 16-lane group key kappa(2s + kk, lr) = 32s + 8(lr/4) + 4kk + lr%4 of the 4 rows of
            // its group. V^T source: lane (lg, lr) supplies token row 4lg + lr/4 and the value columns
            // 16cw + 4(lr%4) .. +3 of the value half (token tile it adds 2048 B); the transposing read hands lane
            // lr the 4 rows of column 16cw + lr. The output tile offset (row j, columns 16cw + 4lg .. +3 of the
            // value half) follows the output tile's swizzle.
            int q_off[4], tr_off[4], vt_off, o_off, clane, clg;
            // Every lane-dependent value of the consumer, from lane index ln. Called again after the steady-state
            // loop with a freshly derived lane index, so that nothing computed before the loop for use after it
            // has to stay in a register through the loop.
            auto lane_setup = [&](int ln) {
                const int llr = ln & 15, llg = ln >> 4;
                clane = ln;
                clg = llg;
#pragma unroll
                for (int x = 0; x < 16; ++x) fvd64[x] = lam_pow(l2, 63 - (16 * (x >> 2) + 4 * llg + (x & 3)));
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) finter[jt] = p.scale * lam_pow(l2, 16 * jt + llr + 1);
#pragma unroll
                for (int e = 0; e < 4; ++e) neg_ident[e] = (4 * llg + e == llr) ? (short)0xBF80 : (short)0;   // -1.0
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    q_off[s] = q_seg_off(llr, 4 * s + llg);
                    tr_off[s] = k_seg_off(4 * llg + (llr >> 2), 4 * s + (llr & 3));
                }
                vt_off = vt_seg_off(4 * llg + (llr >> 2), 2 * cw + ((llr & 3) >> 1)) + 8 * (llr & 1);
                o_off = v_seg_off(llr, 2 * cw + (llg >> 1)) + 8 * (llg & 1);
            };
            lane_setup(lane);

            // Carried from the iteration that takes chunk c's history term to the one that writes its output:
            // the history term (acc) and chunk c's V^T fragments (vf).
            f32x4 acc[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
            u32x4 vf[2];
            vf[0] = vf[1] = u32x4{0u, 0u, 0u, 0u};

            // V_dec factors lambda^{lc-1-i} of a chunk of lc tokens; the factors of missing rows are zero and
            // every exponent handed to exp2 stays >= 0
            auto tail_factors = [&](int lc, float (&fvd)[16]) {
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int r2 = 0; r2 < 4; ++r2) {
                        const int i = 16 * it + 4 * clg + r2;
                        fvd[4 * it + r2] = (i < lc) ? lam_pow(l2, lc - 1 - i) : 0.f;
                    }
            };
            // V fragments of token tile it from its V^T fragment `a` (bf16 rows 4lg .. 4lg+3 of column lr, as
            // the transposing read returns them): V^T for P.V as is, and V_dec = lambda^{lc-1-i} v_i as bf16 hi + lo
            // (tail: the factors of a short last chunk in fvd; else the full-chunk factors fvd64)
            auto prep_part = [&](u32x2 a, int it, bool tail, const float (&fvd)[16], u32x4 (&vdh)[2],
                                 u32x4 (&vdl)[2]) {
                // the 4 values widened exactly to FP32 (a bf16 is the upper half of its FP32 pattern)
                const uint32_t x0 = a.x, x1 = a.y;
                const f32x4 x = f32x4{__builtin_bit_cast(float, x0 << 16), __builtin_bit_cast(float, x0 & 0xFFFF0000u),
                                      __builtin_bit_cast(float, x1 << 16), __builtin_bit_cast(float, x1 & 0xFFFF0000u)};
                float f[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) f[r] = x[r] * (tail ? fvd[4 * it + r] : fvd64[4 * it + r]);
                uint32_t h0, h1, l0, l1;
                split4_mfma(f32x4{f[0], f[1], f[2], f[3]}, neg_ident, h0, h1, l0, l1);
                const u32x2 d01 = u32x2{h0, l0}, d23 = u32x2{h1, l1};
                if ((it & 1) == 0) {
                    vf[it >> 1].x = x0; vf[it >> 1].y = x1;
                    vdh[it >> 1].x = d01.x; vdh[it >> 1].y = d23.x;
                    vdl[it >> 1].x = d01.y; vdl[it >> 1].y = d23.y;
                } else {
                    vf[it >> 1].z = x0; vf[it >> 1].w = x1;
                    vdh[it >> 1].z = d01.x; vdh[it >> 1].w = d23.x;
                    vdl[it >> 1].z = d01.y; vdl[it >> 1].w = d23.y;
                }
            };
            auto load_v = [&](int c, u32x2 (&va)[4]) {
                const uint8_t *tv = smem + kOffV + (c & 1) * kVTileB + vt_off;
#pragma unroll
                for (int it = 0; it < 4; ++it) va[it] = ld_tr(tv + 2048 * it);
            };
            // the state before the chunk as bf16 hi + lo for the history term (key group s: keys 32s + 8lg .. +7
            // in tiles 2s, slots 0..3, and 2s+1, slots 4..7), then the decay of those two tiles
            auto split_dec = [&](int s, float dec, u32x4 &shi, u32x4 &slo) {
                // the decayed state goes to new registers first, so that the residuals of the split can be
                // accumulated in place into the (then dead) registers of the state before the chunk
                const f32x4 s0 = S[2 * s], s1 = S[2 * s + 1];
                S[2 * s] = s0 * dec;
                S[2 * s + 1] = s1 * dec;
                if (kOut) {
                    uint32_t h0, h1, l0, l1, h2, h3, l2, l3;
                    split4_mfma(s0, neg_ident, h0, h1, l0, l1);
                    split4_mfma(s1, neg_ident, h2, h3, l2, l3);
                    const u32x2 a = u32x2{h0, l0}, b2 = u32x2{h1, l1}, c2 = u32x2{h2, l2}, d2 = u32x2{h3, l3};
                    shi = u32x4{a.x, b2.x, c2.x, d2.x};
                    slo = u32x4{a.y, b2.y, c2.y, d2.y};
                }
            };
            // Q fragments (row tiles jt = 0..3) and K^T fragments (tiles 2s, 2s+1, token pairs 0, 1) of key
            // group s; the base addresses are opaque so that the per-read constants stay in the instruction
            // offsets instead of being hoisted as one address per read
            auto bases = [&](int c, int (&qb)[4], int (&kb)[4]) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    qb[s] = kOffQ + (c & 1) * kQKTileB + q_off[s];
                    kb[s] = kOffK + (c & 1) * kQKTileB + tr_off[s];
                    asm("" : "+v"(qb[s]), "+v"(kb[s]));
                }
            };
            auto load_qk = [&](const int (&qb)[4], const int (&kb)[4], int s, u32x4 (&qf)[4], u32x4 (&kf)[4]) {
                if (kOut) {
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) qf[jt] = ld16(smem + qb[s] + 4096 * jt);
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int ip = 0; ip < 2; ++ip) {
                        const uint8_t *src = smem + kb[s] + 8 * kk + (32 * ip) * 256;
                        const u32x2 lo = ld_tr(src);
                        const u32x2 hi = ld_tr(src + 16 * 256);
                        kf[2 * kk + ip] = u32x4{lo.x, lo.y, hi.x, hi.y};
                    }
            };
            // key group s: history term acc += S_s Q^T (hi + lo) and state update S <- S + K^T V_dec (hi + lo)
            auto group_mfma = [&](int s, const u32x4 &shi, const u32x4 &slo, const u32x4 (&qf)[4],
                                  const u32x4 (&kf)[4], const u32x4 (&vdh)[2], const u32x4 (&vdl)[2]) {
                if (kOut) {
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) {
                        acc[jt] = mfma32(shi, qf[jt], acc[jt]);
                        acc[jt] = mfma32(slo, qf[jt], acc[jt]);
                    }
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int ip = 0; ip < 2; ++ip) {
                        S[2 * s + kk] = mfma32(kf[2 * kk + ip], vdh[ip], S[2 * s + kk]);
                        S[2 * s + kk] = mfma32(kf[2 * kk + ip], vdl[ip], S[2 * s + kk]);
                    }
            };
            auto load_p = [&](int c, u32x4 (&pf)[12]) {
                const uint8_t *pbuf = smem + kOffP + (c & 1) * kPBufB + clane * 16;
#pragma unroll
                for (int x = 0; x < 12; ++x) pf[x] = ld16(pbuf + x * kFragB);
            };
            // chunk c's output: O = scale lambda^{j+1} history + P.V (P carries scale), rounded to bf16 into the
            // LDS output tile (row j, columns 16cw + 4lg .. +3 of the value half). Clears acc for the next chunk.
            auto output = [&](int c, const u32x4 (&pf)[12]) {
                uint8_t *ot = smem + kOffO + (c & 1) * kOTileB + o_off;
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    f32x4 a = acc[jt] * finter[jt];
#pragma unroll
                    for (int ip = 0; ip <= (jt >> 1); ++ip) {
                        a = mfma32(vf[ip], pf[2 * p_blk(jt, ip)], a);
                        a = mfma32(vf[ip], pf[2 * p_blk(jt, ip) + 1], a);
                    }
                    // row 16jt + lr: the swizzle term (row / 2) % 8 is the same for rows lr and 16jt + lr
                    *reinterpret_cast<u32x2 *>(ot + 2048 * jt) = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
                    acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            };

            // One iteration: [output of chunk c-1] + V fragments, history term and state update of chunk c.
            // The LDS reads of each stage are issued, into their own registers, one stage ahead of their use.
            //   kind: bit 0 = chunk c-1 has an output, bit 1 = chunk c is the short last chunk
            auto iteration = [&](int c, auto kind_tag) {
                constexpr int kind = decltype(kind_tag)::value;
                constexpr bool has_out = kOut && (kind & 1);
                constexpr bool tail = (kind & 2) != 0;
                float fvd[16];
                float dec = dec64;
                if (tail) {
                    const int lc = min(kC, len - c * kC);
                    tail_factors(lc, fvd);
                    dec = lam_pow(l2, lc);
                }
                int qb[4], kb[4];
                bases(c, qb, kb);
                u32x4 pf[12], qf[4], kf[4];
                u32x2 va[4];
                if (has_out) load_p(c - 1, pf);
                load_v(c, va);
                load_qk(qb, kb, 0, qf, kf);
                u32x4 shi, slo;
                split_dec(0, dec, shi, slo);
                if (has_out) output(c - 1, pf);
                u32x4 vdh[2], vdl[2];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4 qf2[4], kf2[4];
                    if (s < 3) load_qk(qb, kb, s + 1, qf2, kf2);
                    if (s == 0) {
#pragma unroll
                        for (int it = 0; it < 4; ++it) prep_part(va[it], it, tail, fvd, vdh, vdl);
                    }
                    group_mfma(s, shi, slo, qf, kf, vdh, vdl);
                    if (s < 3) {
                        split_dec(s + 1, dec, shi, slo);
#pragma unroll
                        for (int x = 0; x < 4; ++x) { qf[x] = qf2[x]; kf[x] = kf2[x]; }
                    }
                    }
            };
            using K_first_last = std::integral_constant<int, 2>;
            using K_first = std::integral_constant<int, 0>;
            using K_steady = std::integral_constant<int, 1>;
            using K_last = std::integral_constant<int, 3>;

            __syncthreads();
            if (nch == 0) {
                __syncthreads();
            } else {
                if (nch == 1)
                    iteration(0, K_first_last{});
                else
                    iteration(0, K_first{});
                __syncthreads();
                // steady state: full chunks, no branches in the body
                for (int c = 1; c < nch - 1; ++c) {
                    iteration(c, K_steady{});
                    __syncthreads();
                }
                {
                    int ln = tid;
                    asm volatile("" : "+v"(ln));
                    lane_setup(ln & 63);
                }
                if (nch >= 2) {
                    iteration(nch - 1, K_last{});
                    __syncthreads();
                }
                if (kOut) {
                    u32x4 pf[12];
                    load_p(nch - 1, pf);
                    output(nch - 1, pf);
                }
                __syncthreads();
            }

            if (s_out) {
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
                    *reinterpret_cast<f32x4 *>(s_out + (v0 + 16 * cw + (clane & 15)) * kD + 32 * (kt >> 1) + 8 * clg +
                                               4 * (kt & 1)) = S[kt];
            }
        } else {
            // ======================================== producer: staging and scores / P
            float pf[16];               // score decay factors (times scale) of this wave's tile block
            const uint8_t *qseq = reinterpret_cast<const uint8_t *>(p.q + (row0 * p.H + h) * kD);
            const uint8_t *kseq = reinterpret_cast<const uint8_t *>(p.k + (row0 * p.H + h) * kD);
            const uint8_t *vseq = reinterpret_cast<const uint8_t *>(p.v + (row0 * p.HV + un.hv) * kDV + v0);
            // Producers 2 and 3 compute 3 score tiles each, producers 0 and 1 two; each producer shares its SIMD
            // with one state owner. Producers 0 and 1 therefore take all of the staging loads and output
            // stores (rows 32cw .. 32cw+31 of every tile), so that the four SIMDs carry
            // about the same work per chunk.
            const bool io_wave = cw < 2;
            const int hw = cw & 1;
            // per-lane source offsets of the direct-to-LDS staging loads (the same for every chunk): Q/K
            // block b holds rows 4(8hw+b) .. +3, lane -> (row 4(8hw+b) + lane/16, physical segment lane%16);
            // V block b holds rows 8(4hw+b) .. +7, lane -> (row + lane/8, segment lane%8)
            int q_src[8], k_src[8], v_src[4];
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const int r = 4 * (8 * hw + b) + (lane >> 4);
                q_src[b] = r * qk_stride + (((lane & 15) ^ q_swz(r)) << 4);
                k_src[b] = r * qk_stride + (((lane & 15) ^ k_swz(r)) << 4);
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int r = 8 * (4 * hw + b) + (lane >> 3);
                v_src[b] = r * v_stride + (((lane & 7) ^ vt_swz(r)) << 4);
            }
            auto stage = [&](int c) {
                if (!io_wave) return;
                const int c0 = c * kC;
                const int lc = min(kC, len - c0);
                uint8_t *tq = smem + kOffQ + (c & 1) * kQKTileB;
                uint8_t *tk = smem + kOffK + (c & 1) * kQKTileB;
                uint8_t *tv = smem + kOffV + (c & 1) * kVTileB;
                // buffer ranges end with the last valid row of the chunk; rows beyond read as zeros
                const int qk_bytes = (lc - 1) * qk_stride + kD * 2;
                const int v_bytes = (lc - 1) * v_stride + kVW * 2;
                const __amdgpu_buffer_rsrc_t rk =
                    __builtin_amdgcn_make_buffer_rsrc((void *)(kseq + (int64_t)c0 * qk_stride), 0, qk_bytes, kBufDword3);
                const __amdgpu_buffer_rsrc_t rv =
                    __builtin_amdgcn_make_buffer_rsrc((void *)(vseq + (int64_t)c0 * v_stride), 0, v_bytes, kBufDword3);
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(tk + (8 * hw + b) * 1024), 16, k_src[b], 0, 0, 0);
                if (kOut) {
                    const __amdgpu_buffer_rsrc_t rq =
                        __builtin_amdgcn_make_buffer_rsrc((void *)(qseq + (int64_t)c0 * qk_stride), 0, qk_bytes, kBufDword3);
#pragma unroll
                    for (int b = 0; b < 8; ++b)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void *)(tq + (8 * hw + b) * 1024), 16, q_src[b], 0, 0, 0);
                }
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(tv + (4 * hw + b) * 1024), 16, v_src[b], 0, 0, 0);
            };

            if (kOut) {
                switch (cw) {
                case 0: score_factors<0, 2, 2, 1>(pf, l2, p.scale, lr, lg); break;
                case 1: score_factors<0, 2, 3, 1>(pf, l2, p.scale, lr, lg); break;
                case 2: score_factors<2, 2, 2, 2>(pf, l2, p.scale, lr, lg); break;
                default: score_factors<0, 2, 0, 2>(pf, l2, p.scale, lr, lg); break;
                }
            }
            // chunk c's output tile from LDS to HBM: producer cw < 2 stores rows 32cw .. 32cw+31 of the value
            // half, 8 lanes of 16 B per 128-byte row half; rows >= lc fall outside the buffer range and are dropped
            auto store_out = [&](int c) {
                if (!io_wave) return;
                const int c0 = c * kC;
                const int lc = min(kC, len - c0);
                const uint8_t *ot = smem + kOffO + (c & 1) * kOTileB;
                const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(p.o + ((row0 + c0) * p.HV + un.hv) * kDV + v0), 0, (lc - 1) * v_stride + kVW * 2,
                    kBufDword3);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 32 * hw + 8 * i + (lane >> 3);
                    const u32x4 x = ld16(ot + v_seg_off(r, lane & 7));
                    __builtin_amdgcn_raw_buffer_store_b128(x, ro, r * v_stride + 16 * (lane & 7), 0, 0);
                }
            };

            // Every iteration ends with all of this wave's loads and stores complete (vmcnt(0)), so the chunk
            // staged at its start has landed in LDS before the barrier.
            if (nch > 0) stage(0);
            wait_vmcnt_lgkm0<0>();
            __syncthreads();

            for (int t = 0; t <= nch; ++t) {
                if (t + 1 < nch) stage(t + 1);
                if (kOut && t >= 2) store_out(t - 2);   // completed by the consumers before the last barrier
                if (kOut && t < nch) {
                    const uint8_t *tq = smem + kOffQ + (t & 1) * kQKTileB;
                    const uint8_t *tk = smem + kOffK + (t & 1) * kQKTileB;
                    uint8_t *pbuf = smem + kOffP + (t & 1) * kPBufB;
                    switch (cw) {
                    case 0: produce_scores<0, 2, 2, 1>(pf, tq, tk, pbuf, lane, lr, lg); break;
                    case 1: produce_scores<0, 2, 3, 1>(pf, tq, tk, pbuf, lane, lr, lg); break;
                    case 2: produce_scores<2, 2, 2, 2>(pf, tq, tk, pbuf, lane, lr, lg); break;
                    default: produce_scores<0, 2, 0, 2>(pf, tq, tk, pbuf, lane, lr, lg); break;
                    }
                }
                wait_vmcnt_lgkm0<0>();                   // chunk t+1 has landed
                __syncthreads();
            }
            if (kOut && nch > 0) store_out(nch - 1);
        }
    }
}
// ---------------------------------------------------------------------------------------------------------
// Segmented sequences: the initial state of every segment (the segmented scan over segments of the affine
// maps S -> lambda^L S + L_g, page "linear_attention: add a Hopper (sm90) KDA prefill path", its chunk-parallel
// PREP and sequential SCAN over the state, applied here to whole segments). Entry b * nseg of the segment
// buffer receives sequence b's initial state (its pool slot with LA_STATE_READ, else zero); entry
// b * nseg + g (g >= 1), which holds segment g-1's local state (from zero), becomes
// lambda^{seg_len} * entry(g-1) + local state. One thread per 4 consecutive floats of one (sequence, head) plane.
// ---------------------------------------------------------------------------------------------------------
struct ScanParams {
    const float *pool;
    const int32_t *state_idx;
    const float *slope;
    float *seg_states;
    int32_t B, HV, G, pool_size, nseg, seg_len;
    uint32_t flags;
};

__global__ __launch_bounds__(256) void la_seg_scan_kernel(ScanParams p) {
    constexpr int kQuads = kDV * kD / 4;                          // float4 per plane
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t plane = gid / kQuads;
    const int e4 = (int)(gid - plane * kQuads);
    if (plane >= (int64_t)p.B * p.HV) return;
    const int b = (int)(plane / p.HV), hv = (int)(plane - (int64_t)b * p.HV);
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.flags & LA_STATE_READ) {
        const int slot = p.state_idx[b];
        if (slot >= 0 && slot < p.pool_size)
            st = reinterpret_cast<const f32x4 *>(p.pool + ((int64_t)slot * p.HV + hv) * (kDV * kD))[e4];
    }
    const float l2 = log2_lambda(p.slope[(p.flags & LA_DECAY_PER_QK_HEAD) ? hv / p.G : hv]);
    const float dec = __builtin_amdgcn_exp2f(l2 * (float)p.seg_len);
    f32x4 *w = reinterpret_cast<f32x4 *>(p.seg_states);
    const int64_t stride = (int64_t)p.HV * kQuads;                // one segment entry
    int64_t at = ((int64_t)b * p.nseg * p.HV + hv) * kQuads + e4;
    w[at] = st;
    for (int g = 1; g < p.nseg; ++g) {
        at += stride;
        st = st * dec + w[at];
        w[at] = st;
    }
}

}  // namespace

// ---------------------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------------------
namespace la_detail {

thread_local char g_err[512] = "";

void clear_error() { g_err[0] = 0; }

int cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

la_status fail(la_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

la_status check_common(int32_t H, int32_t HV, int32_t D, int32_t DV, uint32_t flags, const float *slope,
                       const float *pool, int32_t pool_size, const int32_t *state_idx) {
    if (D != kD || DV != kDV)
        return fail(LA_ERR_UNSUPPORTED, "only D = DV = 128 is supported (got D=%d, DV=%d)", D, DV);
    if (H <= 0 || HV <= 0)
        return fail(LA_ERR_UNSUPPORTED, "head counts must be positive (H=%d, HV=%d)", H, HV);
    if (HV % H != 0)
        return fail(LA_ERR_UNSUPPORTED, "HV (%d) must be a multiple of H (%d)", HV, H);
    // the kernels address a chunk's rows with 32-bit byte offsets: 63 rows of HV * 256 bytes must stay < 2^31
    if (HV > kMaxHeads)
        return fail(LA_ERR_UNSUPPORTED, "at most %d value heads are supported (got HV=%d)", kMaxHeads, HV);
    if (flags & ~(uint32_t)(LA_STATE_READ | LA_STATE_WRITE | LA_DECAY_PER_QK_HEAD))
        return fail(LA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
    if (!slope) return fail(LA_ERR_INVALID_ARG, "slope is NULL");
    if (pool_size < 0) return fail(LA_ERR_INVALID_ARG, "pool_size is negative");
    if ((flags & (LA_STATE_READ | LA_STATE_WRITE)) && (!pool || !state_idx))
        return fail(LA_ERR_INVALID_ARG, "state flags set but state_pool or state_idx is NULL");
    return LA_OK;
}

}  // namespace la_detail

namespace {

template <int MODE>
la_status launch(const Params &p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(la_chunk_kernel<MODE>, dim3(grid), dim3(kThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}


// Device scratch of la_prefill_fwd_seg_noalloc: the per-segment state buffer of the segmented prefill, in a fixed
// array of kScratchBytes that every device running the library holds until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for the symbol); it uses the device
// address that hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = (size_t)16 << 20;      // 256 state planes of 64 KiB
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

la_status scratch_address(hipStream_t stream, void **out) {
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> addr[kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return fail(LA_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(LA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p) {
        *out = p;
        return LA_OK;
    }
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
        // the symbol's address is per device: look it up with the stream's device current
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return fail(LA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(LA_ERR_HIP, "hipSetDevice(%d) failed: %s", dev, hipGetErrorString(e));
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = (cur != dev) ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess || !p)
            return fail(LA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
        if (e2 != hipSuccess) return fail(LA_ERR_HIP, "hipSetDevice(%d) failed: %s", cur, hipGetErrorString(e2));
        addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return LA_OK;
}

// The segmented prefill behind la_prefill_fwd_seg (caller's workspace) and la_prefill_fwd_seg_noalloc (the
// device scratch above). Every workspace entry a kernel reads was written earlier in the same call, so nothing
// has to be cleared first.
la_status seg_prefill(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                      int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                      int32_t pool_size, const int32_t *state_idx, const int32_t *state_idx_out, uint32_t flags,
                      int32_t segments, void *workspace, size_t workspace_bytes, bool use_scratch,
                      hipStream_t stream) {
    clear_error();
    la_status s = check_common(H, HV, D, DV, flags, slope, state_pool, pool_size, state_idx);
    if (s != LA_OK) return s;
    if (B < 0 || T < 0) return fail(LA_ERR_INVALID_ARG, "negative B or T (B=%d, T=%d)", B, T);
    if (segments < 0) return fail(LA_ERR_INVALID_ARG, "negative segment count %d", segments);
    const int nch = (T + kC - 1) / kC;
    int want = segments;
    if (want == 0) {
        // enough segments to give every CU a workgroup, each segment at least 4 chunks long
        const int cus = cu_count();
        const int64_t units = (int64_t)B * HV * kVSplit;
        want = (int)std::max<int64_t>(1, std::min<int64_t>(nch / 4, units > 0 ? cus / units : 1));
    }
    want = std::max(1, std::min(want, std::max(nch, 1)));
    const int seg_chunks = (nch + want - 1) / std::max(want, 1);
    const int seg_len = seg_chunks * kC;
    const int nseg = seg_len > 0 ? (T + seg_len - 1) / seg_len : 1;
    if (B == 0 || T <= kShortMax || nseg <= 1)
        return la_prefill_fwd_ex(q, k, v, o, B, T, H, HV, D, DV, scale, slope, state_pool, pool_size, state_idx,
                                 state_idx_out, flags, stream);
    if (!q || !k || !v || !o) return fail(LA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
    if ((int64_t)B * T > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "B * T exceeds 2^31 - 1 tokens");
    if ((int64_t)B * nseg * HV * kVSplit > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "too many segment units");
    const size_t need = la_prefill_seg_workspace_bytes(B, HV, nseg);
    if (use_scratch) {
        if (need > kScratchBytes)
            return fail(LA_ERR_UNSUPPORTED,
                        "%d segments of B=%d sequences and HV=%d heads need %zu bytes of scratch; the allocation-free "
                        "call holds at most %zu (B * segments * HV <= %zu state planes)",
                        nseg, B, HV, need, kScratchBytes, kScratchBytes / ((size_t)kDV * kD * sizeof(float)));
        s = scratch_address(stream, &workspace);
        if (s != LA_OK) return s;
    } else if (!workspace || workspace_bytes < need) {
        return fail(LA_ERR_INVALID_ARG, "workspace of %zu bytes needed for %d segments (got %zu)", need, nseg,
                    workspace ? workspace_bytes : (size_t)0);
    }

    // pass 1: local states of segments 0 .. nseg-2 from zero
    Params p{};
    p.k = (const uint16_t *)k; p.v = (const uint16_t *)v; p.slope = slope;
    p.seg_states = (float *)workspace; p.seg_len = seg_len; p.nseg = nseg;
    p.nseq = B * (nseg - 1); p.T = T; p.total_T = B * T; p.H = H; p.HV = HV; p.G = HV / H;
    p.npairs = p.nseq * HV; p.nunits = p.npairs * kVSplit; p.scale = scale;
    p.flags = flags & LA_DECAY_PER_QK_HEAD;
    s = launch<kSegStates>(p, p.nunits, stream);
    if (s != LA_OK) return s;

    // scan: every segment's initial state
    ScanParams sp{};
    sp.pool = state_pool; sp.state_idx = state_idx; sp.slope = slope; sp.seg_states = (float *)workspace;
    sp.B = B; sp.HV = HV; sp.G = HV / H; sp.pool_size = (flags & (LA_STATE_READ | LA_STATE_WRITE)) ? pool_size : 0;
    sp.nseg = nseg; sp.seg_len = seg_len; sp.flags = flags;
    const int64_t threads = (int64_t)B * HV * (kDV * kD / 4);
    hipLaunchKernelGGL(la_seg_scan_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, sp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));

    // pass 2: every segment from its initial state; the last one stores the final state
    Params f{};
    f.q = (const uint16_t *)q; f.k = (const uint16_t *)k; f.v = (const uint16_t *)v; f.o = (uint16_t *)o;
    f.slope = slope; f.pool = state_pool; f.state_idx = state_idx; f.state_idx_out = state_idx_out;
    f.seg_states = (float *)workspace; f.seg_len = seg_len; f.nseg = nseg;
    f.nseq = B * nseg; f.T = T; f.total_T = B * T; f.H = H; f.HV = HV; f.G = HV / H;
    f.pool_size = (flags & (LA_STATE_READ | LA_STATE_WRITE)) ? pool_size : 0;
    f.npairs = f.nseq * HV; f.nunits = f.npairs * kVSplit; f.scale = scale; f.flags = flags;
    return launch<kSegFwd>(f, f.nunits, stream);
}
}  // namespace

extern "C" {

la_status la_prefill_fwd_ex(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                            int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                            int32_t pool_size, const int32_t *state_idx, const int32_t *state_idx_out,
                            uint32_t flags, hipStream_t stream) {
    clear_error();
    la_status s = check_common(H, HV, D, DV, flags, slope, state_pool, pool_size, state_idx);
    if (s != LA_OK) return s;
    if (B < 0 || T < 0) return fail(LA_ERR_INVALID_ARG, "negative B or T (B=%d, T=%d)", B, T);
    if (B == 0) return LA_OK;
    if (T == 0 && !(flags & LA_STATE_WRITE)) return LA_OK;
    if (T > 0 && (!q || !k || !v || !o)) return fail(LA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
    if ((int64_t)B * HV * kVSplit > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "too many (sequence, head) units");
    if ((int64_t)B * T > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "B * T exceeds 2^31 - 1 tokens");
    if (T >= 1 && T <= kShortMax) {
        // a few tokens per sequence (verify / multi-token decode): one pass from the initial state
        ShortCall c{};
        c.q = q; c.k = k; c.v = v; c.o = o; c.slope = slope; c.pool = state_pool; c.state_idx = state_idx;
        c.state_idx_out = state_idx_out;
        c.B = B; c.T = T; c.H = H; c.HV = HV; c.pool_size = pool_size; c.scale = scale; c.flags = flags;
        return launch_short(c, stream);
    }
    Params p{};
    p.q = (const uint16_t *)q; p.k = (const uint16_t *)k; p.v = (const uint16_t *)v; p.o = (uint16_t *)o;
    p.slope = slope; p.pool = state_pool; p.state_idx = state_idx; p.state_idx_out = state_idx_out;
    p.nseq = B; p.T = T; p.total_T = B * T; p.H = H; p.HV = HV; p.G = HV / H;
    p.pool_size = (flags & (LA_STATE_READ | LA_STATE_WRITE)) ? pool_size : 0; p.npairs = B * HV; p.nunits = p.npairs * kVSplit;
    p.scale = scale; p.flags = flags;
    return launch<kFixed>(p, p.nunits, stream);
}

la_status la_prefill_fwd(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                         int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                         int32_t pool_size, const int32_t *state_idx, uint32_t flags, hipStream_t stream) {
    return la_prefill_fwd_ex(q, k, v, o, B, T, H, HV, D, DV, scale, slope, state_pool, pool_size, state_idx, nullptr,
                             flags, stream);
}

la_status la_prefill_fwd_varlen_ex(const void *q, const void *k, const void *v, void *o, const int32_t *cu_seqlens,
                                   int32_t N, int32_t total_T, int32_t H, int32_t HV, int32_t D, int32_t DV,
                                   float scale, const float *slope, float *state_pool, int32_t pool_size,
                                   const int32_t *state_idx, const int32_t *state_idx_out, uint32_t flags,
                                   int32_t schedule, hipStream_t stream) {
    clear_error();
    la_status s = check_common(H, HV, D, DV, flags, slope, state_pool, pool_size, state_idx);
    if (s != LA_OK) return s;
    if (N < 0 || total_T < 0) return fail(LA_ERR_INVALID_ARG, "negative N or total_T (N=%d, total_T=%d)", N, total_T);
    if (schedule < LA_SCHED_AUTO || schedule > LA_SCHED_NONPERSISTENT)
        return fail(LA_ERR_INVALID_ARG, "unknown schedule %d", schedule);
    if (N == 0) return LA_OK;
    if (!cu_seqlens) return fail(LA_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (total_T > 0 && (!q || !k || !v || !o)) return fail(LA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
    if ((int64_t)N * HV * kVSplit > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "too many (sequence, head) units");
    Params p{};
    p.q = (const uint16_t *)q; p.k = (const uint16_t *)k; p.v = (const uint16_t *)v; p.o = (uint16_t *)o;
    p.cu_seqlens = cu_seqlens; p.slope = slope; p.pool = state_pool; p.state_idx = state_idx;
    p.state_idx_out = state_idx_out;
    p.nseq = N; p.T = 0; p.total_T = total_T; p.H = H; p.HV = HV; p.G = HV / H;
    p.pool_size = (flags & (LA_STATE_READ | LA_STATE_WRITE)) ? pool_size : 0; p.npairs = N * HV; p.nunits = p.npairs * kVSplit;
    p.scale = scale; p.flags = flags;
    int grid = p.nunits;
    if (schedule == LA_SCHED_PERSISTENT) grid = std::min(grid, cu_count());
    return launch<kVarlen>(p, grid, stream);
}

la_status la_prefill_fwd_varlen(const void *q, const void *k, const void *v, void *o, const int32_t *cu_seqlens,
                                int32_t N, int32_t total_T, int32_t H, int32_t HV, int32_t D, int32_t DV,
                                float scale, const float *slope, float *state_pool, int32_t pool_size,
                                const int32_t *state_idx, uint32_t flags, int32_t schedule, hipStream_t stream) {
    return la_prefill_fwd_varlen_ex(q, k, v, o, cu_seqlens, N, total_T, H, HV, D, DV, scale, slope, state_pool,
                                    pool_size, state_idx, nullptr, flags, schedule, stream);
}

size_t la_prefill_seg_workspace_bytes(int32_t B, int32_t HV, int32_t segments) {
    if (B <= 0 || HV <= 0 || segments <= 1) return 0;
    return (size_t)B * (size_t)segments * (size_t)HV * (size_t)(kDV * kD) * sizeof(float);
}

la_status la_prefill_fwd_seg(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                             int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                             int32_t pool_size, const int32_t *state_idx, const int32_t *state_idx_out,
                             uint32_t flags, int32_t segments, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    return seg_prefill(q, k, v, o, B, T, H, HV, D, DV, scale, slope, state_pool, pool_size, state_idx, state_idx_out,
                       flags, segments, workspace, workspace_bytes, false, stream);
}

la_status la_prefill_fwd_seg_noalloc(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T,
                                     int32_t H, int32_t HV, int32_t D, int32_t DV, float scale, const float *slope,
                                     float *state_pool, int32_t pool_size, const int32_t *state_idx,
                                     const int32_t *state_idx_out, uint32_t flags, int32_t segments,
                                     hipStream_t stream) {
    return seg_prefill(q, k, v, o, B, T, H, HV, D, DV, scale, slope, state_pool, pool_size, state_idx, state_idx_out,
                       flags, segments, nullptr, 0, true, stream);
}

size_t la_prefill_seg_noalloc_max_bytes(void) { return kScratchBytes; }

la_status la_state_commit(const void *k, const void *v, int32_t B, int32_t T, int32_t H, int32_t HV, int32_t D,
                          int32_t DV, const float *slope, float *state_pool, int32_t pool_size,
                          const int32_t *state_idx, const int32_t *accepted_len, hipStream_t stream) {
    clear_error();
    la_status s = check_common(H, HV, D, DV, LA_STATE_READ | LA_STATE_WRITE, slope, state_pool, pool_size,
                               state_idx);
    if (s != LA_OK) return s;
    if (B < 0 || T < 0) return fail(LA_ERR_INVALID_ARG, "negative B or T (B=%d, T=%d)", B, T);
    if (B == 0 || T == 0) return LA_OK;
    if (!k || !v || !accepted_len) return fail(LA_ERR_INVALID_ARG, "k, v and accepted_len must be non-NULL");
    if ((int64_t)B * HV * kVSplit > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "too many (request, head) units");
    if ((int64_t)B * T > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "B * T exceeds 2^31 - 1 tokens");
    if (T <= kShortMax) {
        ShortCall c{};
        c.k = k; c.v = v; c.slope = slope; c.pool = state_pool; c.state_idx = state_idx;
        c.accepted_len = accepted_len; c.B = B; c.T = T; c.H = H; c.HV = HV; c.pool_size = pool_size;
        c.scale = 1.0f; c.flags = LA_STATE_READ | LA_STATE_WRITE; c.commit = true;
        return launch_short(c, stream);
    }
    Params p{};
    p.k = (const uint16_t *)k; p.v = (const uint16_t *)v;
    p.accepted_len = accepted_len; p.slope = slope; p.pool = state_pool; p.state_idx = state_idx;
    p.nseq = B; p.T = T; p.total_T = B * T; p.H = H; p.HV = HV; p.G = HV / H;
    p.pool_size = pool_size; p.npairs = B * HV; p.nunits = p.npairs * kVSplit;
    p.scale = 1.0f; p.flags = LA_STATE_READ | LA_STATE_WRITE;
    return launch<kCommit>(p, p.nunits, stream);
}

const char *la_status_string(la_status s) {
    switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_HIP: return "LA_ERR_HIP";
    }
    return "LA_ERR_UNKNOWN";
}

const char *la_last_error(void) { return la_detail::g_err; }

int32_t la_abi_version(void) { return LA_ABI_VERSION; }

}  // extern "C"

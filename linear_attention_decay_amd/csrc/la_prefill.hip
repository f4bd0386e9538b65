// la_prefill.hip -- Lightning Attention chunked prefill for AMD Instinct MI355X (gfx950, CDNA4).
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
// Work decomposition: one workgroup = (sequence, value head, half of the 128 value columns). 4 wave64s;
// wave w owns value columns [16w, 16w+16) of its half: the state rows S[v][0..127] for those columns stay in
// that wave's registers as MFMA accumulators for the whole sequence.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, FP32 accumulate). Every operand fragment a lane holds is
// "row r = lane % 16, slot group g = lane / 16, 8 slots"; slots 0..3 carry contraction indices 4g..4g+3 of
// one 16-wide block and slots 4..7 carry 4g..4g+3 of the next block. The 16x16 accumulator of the same
// instruction holds, per lane, column lane % 16 and rows 4g..4g+3. Chaining works because an accumulator
// tile [m][n] is, lane for lane, a fragment with row n and contraction index m: scores computed as
// A^T[i][j] feed the P.V product as P[j][i] fragments; the state kept as S^T[k][v] feeds Q.S^T as S[v][k]
// fragments; and K, V rows are turned into K^T, V^T fragments with one 16x16x16 MFMA against the identity
// (exact: a single nonzero product per output).
//
// Precision: the state update multiplies the per-token decay into V (V_dec = lambda^{Lc-1-i} v_i) in FP32
// and feeds it as a bf16 hi + lo pair; the FP32 state enters Q S^T as a bf16 hi + lo pair; the decay-masked
// scores P enter P.V as a bf16 hi + lo pair. Q, K, V are exact in bf16. Every exponent handed to exp2 is
// <= 0, so powers of lambda can only underflow. O is rounded to bf16 once, round-to-nearest-even.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <stdio.h>
#include <stdarg.h>
#include <string.h>

#include "la_prefill.h"

namespace {

constexpr int kC = 64;                    // chunk length (tokens)
constexpr int kD = 128;                   // key dim
constexpr int kDV = 128;                  // value dim
constexpr int kVSplit = 2;                // workgroups per (sequence, value head)
constexpr int kVW = kDV / kVSplit;        // value columns per workgroup
constexpr int kThreads = 512;             // 4 consumer waves (one 16-column value tile each) + 4 producer waves

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Mode { kFixed = 0, kVarlen = 1, kCommit = 2 };

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

// ---------------------------------------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 f = {a, b};
    bf16x2 h = __builtin_convertvector(f, bf16x2);   // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float lo_bf16_as_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16_as_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi); two values per call, returned as {hi pair, lo pair}.
__device__ __forceinline__ u32x2 split_bf16x2(float a, float b) {
    const uint32_t hi = pack_bf16x2(a, b);
    const uint32_t lo = pack_bf16x2(a - lo_bf16_as_f32(hi), b - hi_bf16_as_f32(hi));
    return u32x2{hi, lo};
}

__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(u32x2 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), b, c, 0, 0, 0);
}

// lambda^n for n >= 0 given l2 = log2(lambda) (finite, <= 0).
__device__ __forceinline__ float lam_pow(float l2, int n) { return __builtin_amdgcn_exp2f(l2 * (float)n); }

struct Unit {
    int32_t seq, hv, vpart;
};

// Workgroup -> (pair, value half). Pairs are handed out in groups of 8 so that the two halves of a pair
// sit 8 workgroups apart: workgroups are dealt round-robin over the 8 XCDs, so both halves of one
// (sequence, head) land on the same XCD and share its L2 for the Q/K rows they both read.
__device__ __forceinline__ Unit decode_unit(int u, const Params &p) {
    const int full = p.npairs >> 3;
    int pair, half;
    if ((u >> 4) < full) {
        pair = (u >> 4) * 8 + (u & 7);
        half = (u >> 3) & 1;
    } else {
        const int m = p.npairs - full * 8;
        const int r = u - full * 16;
        pair = full * 8 + r % m;
        half = r / m;
    }
    Unit t;
    t.seq = pair / p.HV;
    t.hv = pair - t.seq * p.HV;
    t.vpart = half;
    return t;
}

// ---------------------------------------------------------------------------------------------------------
// LDS layout. Q/K chunk tiles are 64 rows x 256 B, V tiles 64 rows x 128 B (one value half), stored with an
// XOR swizzle of 16-byte segments so that the fragment reads (16 rows x 8 B per lane group) hit distinct
// banks. P and K^T fragments are stored "fragment-native": 64 lanes x 16 B per block, read back by the same
// lane layout.
//   Q: 3 buffers (consumer reads chunk c-1, producer reads chunk c, chunk c+1 is being staged)
//   K: 2 buffers (producer reads chunk c, chunk c+1 is being staged)
//   V: 3 buffers (as Q)
//   P, K^T: 2 buffers (producer writes chunk c, consumer reads chunk c-1)
// ---------------------------------------------------------------------------------------------------------
constexpr int kQKTileB = kC * kD * 2;        // 16384
constexpr int kVTileB = kC * kVW * 2;        // 8192
constexpr int kFragB = 64 * 16;              // one fragment block
constexpr int kPBufB = 6 * 2 * kFragB;       // 6 lower-triangle (jt, i-pair) blocks, hi and lo
constexpr int kKTBufB = 8 * 2 * kFragB;      // 8 key tiles x 2 token pairs
constexpr int kOffQ = 0;
constexpr int kOffK = kOffQ + 3 * kQKTileB;
constexpr int kOffV = kOffK + 2 * kQKTileB;
constexpr int kOffP = kOffV + 3 * kVTileB;
constexpr int kOffKT = kOffP + 2 * kPBufB;
constexpr int kLdsBytes = kOffKT + 2 * kKTBufB;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

__device__ __forceinline__ int qk_off(int r, int c) {      // byte offset of element (r, c) in a Q/K tile
    return r * 256 + ((((c >> 3) ^ (r & 15))) << 4) + ((c & 7) << 1);
}
__device__ __forceinline__ int v_off(int r, int c) {       // byte offset of element (r, c) in a V tile
    return r * 128 + ((((c >> 3) ^ ((r >> 1) & 7))) << 4) + ((c & 7) << 1);
}
// fragment of a Q/K tile: slots 0..3 = row r, columns c..c+3; slots 4..7 = columns c+16..c+19
__device__ __forceinline__ u32x4 ld_frag_qk(const uint8_t *tile, int r, int c) {
    const u32x2 a = *reinterpret_cast<const u32x2 *>(tile + qk_off(r, c));
    const u32x2 b = *reinterpret_cast<const u32x2 *>(tile + qk_off(r, c + 16));
    return u32x4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ int p_blk(int jt, int ip) { return jt < 2 ? jt : 2 * jt - 2 + ip; }

// ---------------------------------------------------------------------------------------------------------
// Producer: scores A^T[i][j] = K_i . Q_j for the lower-triangle 16x16 tiles (it <= jt) a producer wave owns,
// decay mask P = lambda^{j-i} A (i <= j), written as bf16 hi + lo fragments.
//   wave 0: (0,3) (1,3) (2,3)   wave 1: (3,3) (0,2) (1,2)   wave 2: (2,2) (0,1)   wave 3: (1,1) (0,0)
// Waves 2 and 3 also zero the strictly-upper halves of the (2,2) and (0,0) block pairs.
// ---------------------------------------------------------------------------------------------------------
// tile t of producer PW: it = bits [4t, 4t+2), jt = bits [4t+2, 4t+4) of code
template <int PW> struct Tiles;
template <> struct Tiles<0> { static constexpr int n = 3, code = 0 | (3 << 2) | (1 << 4) | (3 << 6) | (2 << 8) | (3 << 10); };
template <> struct Tiles<1> { static constexpr int n = 3, code = 3 | (3 << 2) | (0 << 4) | (2 << 6) | (1 << 8) | (2 << 10); };
template <> struct Tiles<2> { static constexpr int n = 2, code = 2 | (2 << 2) | (0 << 4) | (1 << 6); };
template <> struct Tiles<3> { static constexpr int n = 2, code = 1 | (1 << 2) | (0 << 4) | (0 << 6); };
template <int PW> __device__ __forceinline__ constexpr int tile_it(int t) { return (Tiles<PW>::code >> (4 * t)) & 3; }
template <int PW> __device__ __forceinline__ constexpr int tile_jt(int t) { return (Tiles<PW>::code >> (4 * t + 2)) & 3; }

template <int PW>
__device__ __forceinline__ void score_factors(float (&pf)[12], float l2, int lr, int lg) {
#pragma unroll
    for (int t = 0; t < Tiles<PW>::n; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * tile_it<PW>(t) + 4 * lg + r, j = 16 * tile_jt<PW>(t) + lr;
            pf[4 * t + r] = (i <= j) ? lam_pow(l2, j - i) : 0.f;
        }
}

template <int PW>
__device__ __forceinline__ void produce_scores(const float (&pf)[12], const uint8_t *tq, const uint8_t *tk,
                                               uint8_t *pbuf, int lane, int lr, int lg) {
#pragma unroll
    for (int t = 0; t < Tiles<PW>::n; ++t) {
        const int it = tile_it<PW>(t), jt = tile_jt<PW>(t);
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < 4; ++kp)
            a = mfma32(ld_frag_qk(tk, 16 * it + lr, 32 * kp + 4 * lg), ld_frag_qk(tq, 16 * jt + lr, 32 * kp + 4 * lg), a);
        const u32x2 a01 = split_bf16x2(a[0] * pf[4 * t + 0], a[1] * pf[4 * t + 1]);
        const u32x2 a23 = split_bf16x2(a[2] * pf[4 * t + 2], a[3] * pf[4 * t + 3]);
        uint8_t *dst = pbuf + (p_blk(jt, it >> 1) * 2) * kFragB + lane * 16 + 8 * (it & 1);
        *reinterpret_cast<u32x2 *>(dst) = u32x2{a01.x, a23.x};
        *reinterpret_cast<u32x2 *>(dst + kFragB) = u32x2{a01.y, a23.y};
    }
    if (PW == 2 || PW == 3) {
        const int jt = PW == 3 ? 0 : 2;      // zero half (it = jt + 1) of the diagonal block pair
        uint8_t *dst = pbuf + (p_blk(jt, jt >> 1) * 2) * kFragB + lane * 16 + 8;
        *reinterpret_cast<u32x2 *>(dst) = u32x2{0, 0};
        *reinterpret_cast<u32x2 *>(dst + kFragB) = u32x2{0, 0};
    }
}

// ---------------------------------------------------------------------------------------------------------
// the kernel: 8 waves; waves 0..3 are consumers (state owners), waves 4..7 producers
// ---------------------------------------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(kThreads) void la_chunk_kernel(Params p) {
    constexpr bool kOut = (MODE != kCommit);
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform: role branches are scalar
    const bool consumer = w < 4;
    const int cw = w & 3;            // consumer: value tile; producer: producer index

    for (int u = blockIdx.x; u < p.nunits; u += gridDim.x) {
        // Lane indices are re-derived through an opaque copy in every unit iteration so that the compiler
        // does not hoist lane-dependent set-up (decay exponents, masks) of both roles out of this loop and
        // keep it live for the whole kernel.
        int tid_u = tid;
        asm volatile("" : "+v"(tid_u));
        const int lane = tid_u & 63;
        const int lr = lane & 15;
        const int lg = lane >> 4;
        const int ptid = tid_u - 256;      // producer thread index 0..255
        s16x4 ident;
#pragma unroll
        for (int e = 0; e < 4; ++e) ident[e] = (4 * lg + e == lr) ? (short)0x3F80 : (short)0;

        const Unit un = decode_unit(u, p);
        const int h = un.hv / p.G;
        const int v0 = un.vpart * kVW;

        int64_t row0;
        int len;
        if (MODE == kVarlen) {
            int a = p.cu_seqlens[un.seq];
            int b = p.cu_seqlens[un.seq + 1];
            a = min(max(a, 0), p.total_T);
            b = min(max(b, a), p.total_T);
            row0 = a;
            len = b - a;
        } else if (MODE == kCommit) {
            row0 = (int64_t)un.seq * p.T;
            len = min(max(p.accepted_len[un.seq], 0), p.T);
        } else {
            row0 = (int64_t)un.seq * p.T;
            len = p.T;
        }
        int slot = -1;
        if (p.flags != 0) {
            const int s = p.state_idx[un.seq];
            if (s >= 0 && s < p.pool_size) slot = s;
        }
        if (MODE == kCommit && (slot < 0 || len == 0)) continue;   // skipped request / L = 0: no write at all

        float l2 = -p.slope[un.hv] * 1.4426950408889634f;
        l2 = fmaxf(l2, -1.0e30f);                                    // slope = +inf -> lambda^0 = 1, lambda^n = 0
        const int nch = (len + kC - 1) / kC;
        const float dec64 = lam_pow(l2, kC);
        const int64_t qk_row_stride = (int64_t)p.H * kD;
        const int64_t v_row_stride = (int64_t)p.HV * kDV;

        float *plane = nullptr;
        if (slot >= 0) plane = p.pool + ((int64_t)slot * p.HV + un.hv) * (kDV * kD);

        // The two roles run separate loops with the same number of workgroup barriers (one before the chunk
        // loop, one per iteration), so each role's loop-carried registers are allocated on their own.
        if (consumer) {
            // ======================================== consumer: owns S^T for value tile cw
            // S^T tiles: lane holds S[v][k..k+3], v = v0 + 16cw + lr, k = 16kt + 4lg
            f32x4 S[8];
            float fvd[16];              // lambda^{63-i} for i = 16it+4lg+r (full chunk)
            float finter[4];            // lambda^{j+1} for j = 16jt+lr
            const int vrow = v0 + 16 * cw + lr;
            if (slot >= 0 && (p.flags & LA_STATE_READ)) {
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
                    S[kt] = *reinterpret_cast<const f32x4 *>(plane + vrow * kD + 16 * kt + 4 * lg);
            } else {
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) S[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r) fvd[4 * it + r] = lam_pow(l2, 63 - (16 * it + 4 * lg + r));
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) finter[jt] = lam_pow(l2, 16 * jt + lr + 1);
            __syncthreads();

            for (int t = 0; t <= nch; ++t) {
                if (t > 0) {
                    const int c = t - 1;
                    const int c0 = c * kC;
                    const int lc = min(kC, len - c0);
                    const uint8_t *tq = smem + kOffQ + (c % 3) * kQKTileB;
                    const uint8_t *tv = smem + kOffV + (c % 3) * kVTileB;
                    const uint8_t *pbuf = smem + kOffP + (c & 1) * kPBufB;
                    const uint8_t *ktbuf = smem + kOffKT + (c & 1) * kKTBufB;

                    // V^T fragments of this wave's value tile, and V_dec = lambda^{lc-1-i} v_i as hi + lo
                    u32x4 vf[2], vdh[2], vdl[2];
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const u32x2 a = *reinterpret_cast<const u32x2 *>(tv + v_off(16 * it + lr, 16 * cw + 4 * lg));
                        const f32x4 x = mfma16(a, ident, f32x4{0.f, 0.f, 0.f, 0.f});
                        float d[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float f = fvd[4 * it + r];
                            if (lc != kC) {
                                const int i = 16 * it + 4 * lg + r;
                                f = (i < lc) ? lam_pow(l2, lc - 1 - i) : 0.f;
                            }
                            d[r] = x[r] * f;
                        }
                        const uint32_t x0 = pack_bf16x2(x[0], x[1]), x1 = pack_bf16x2(x[2], x[3]);
                        const u32x2 d01 = split_bf16x2(d[0], d[1]);
                        const u32x2 d23 = split_bf16x2(d[2], d[3]);
                        if ((it & 1) == 0) {
                            vf[it >> 1].x = x0; vf[it >> 1].y = x1;
                            vdh[it >> 1].x = d01.x; vdh[it >> 1].y = d23.x;
                            vdl[it >> 1].x = d01.y; vdl[it >> 1].y = d23.y;
                        } else {
                            vf[it >> 1].z = x0; vf[it >> 1].w = x1;
                            vdh[it >> 1].z = d01.x; vdh[it >> 1].w = d23.x;
                            vdl[it >> 1].z = d01.y; vdl[it >> 1].w = d23.y;
                        }
                    }

                    if (kOut) {
                        // history term Q S^T with S = hi + lo (state before this chunk)
                        u32x4 shi[4], slo[4];
#pragma unroll
                        for (int kp = 0; kp < 4; ++kp) {
                            const u32x2 a = split_bf16x2(S[2 * kp][0], S[2 * kp][1]);
                            const u32x2 b2 = split_bf16x2(S[2 * kp][2], S[2 * kp][3]);
                            const u32x2 c2 = split_bf16x2(S[2 * kp + 1][0], S[2 * kp + 1][1]);
                            const u32x2 d2 = split_bf16x2(S[2 * kp + 1][2], S[2 * kp + 1][3]);
                            shi[kp] = u32x4{a.x, b2.x, c2.x, d2.x};
                            slo[kp] = u32x4{a.y, b2.y, c2.y, d2.y};
                        }
                        f32x4 acc[4];
#pragma unroll
                        for (int jt = 0; jt < 4; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kp = 0; kp < 4; ++kp)
#pragma unroll
                            for (int jt = 0; jt < 4; ++jt) {
                                const u32x4 qf = ld_frag_qk(tq, 16 * jt + lr, 32 * kp + 4 * lg);
                                acc[jt] = mfma32(shi[kp], qf, acc[jt]);
                                acc[jt] = mfma32(slo[kp], qf, acc[jt]);
                            }
                        // within-chunk term P.V, then O = scale (lambda^{j+1} history + within)
                        const float sc = p.scale;
                        uint16_t *obase = p.o + ((row0 + c0) * p.HV + un.hv) * kDV + v0 + 16 * cw + 4 * lg;
#pragma unroll
                        for (int jt = 0; jt < 4; ++jt) {
                            f32x4 a = acc[jt] * finter[jt];
#pragma unroll
                            for (int ip = 0; ip <= (jt >> 1); ++ip) {
                                const uint8_t *blk = pbuf + p_blk(jt, ip) * 2 * kFragB + lane * 16;
                                a = mfma32(vf[ip], *reinterpret_cast<const u32x4 *>(blk), a);
                                a = mfma32(vf[ip], *reinterpret_cast<const u32x4 *>(blk + kFragB), a);
                            }
                            const int j = 16 * jt + lr;
                            if (j < lc) {
                                const u32x2 ov = {pack_bf16x2(sc * a[0], sc * a[1]), pack_bf16x2(sc * a[2], sc * a[3])};
                                *reinterpret_cast<u32x2 *>(obase + (int64_t)j * v_row_stride) = ov;
                            }
                        }
                    }

                    // state update S <- lambda^{lc} S + K^T V_dec
                    const float dec = (lc == kC) ? dec64 : lam_pow(l2, lc);
#pragma unroll
                    for (int kt = 0; kt < 8; ++kt) S[kt] = S[kt] * dec;
#pragma unroll
                    for (int ip = 0; ip < 2; ++ip)
#pragma unroll
                        for (int kt = 0; kt < 8; ++kt) {
                            const u32x4 kf = *reinterpret_cast<const u32x4 *>(ktbuf + ((kt * 2 + ip) * 64 + lane) * 16);
                            S[kt] = mfma32(kf, vdh[ip], S[kt]);
                            S[kt] = mfma32(kf, vdl[ip], S[kt]);
                        }
                }
                __syncthreads();
            }

            if (slot >= 0 && (p.flags & LA_STATE_WRITE)) {
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
                    *reinterpret_cast<f32x4 *>(plane + vrow * kD + 16 * kt + 4 * lg) = S[kt];
            }
        } else {
            // ======================================== producer: staging, scores / P, K^T
            float pf[12];               // score decay factors of this wave's tiles
            u32x4 pq[4], pk[4], pv[2];  // one chunk of rows in flight
            const uint16_t *qbase = p.q + (row0 * p.H + h) * kD;
            const uint16_t *kbase = p.k + (row0 * p.H + h) * kD;
            const uint16_t *vbase = p.v + (row0 * p.HV + un.hv) * kDV + v0;
            auto prefetch = [&](int c) {
                const int c0 = c * kC;
                const int lc = min(kC, len - c0);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int seg = ptid + 256 * s;
                    const int r = seg >> 4, col = (seg & 15) * 8;
                    if (r < lc) {
                        if (kOut) pq[s] = *reinterpret_cast<const u32x4 *>(qbase + (c0 + r) * qk_row_stride + col);
                        pk[s] = *reinterpret_cast<const u32x4 *>(kbase + (c0 + r) * qk_row_stride + col);
                    } else {
                        pq[s] = u32x4{0, 0, 0, 0};
                        pk[s] = u32x4{0, 0, 0, 0};
                    }
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int seg = ptid + 256 * s;
                    const int r = seg >> 3, col = (seg & 7) * 8;
                    pv[s] = (r < lc) ? *reinterpret_cast<const u32x4 *>(vbase + (c0 + r) * v_row_stride + col)
                                     : u32x4{0, 0, 0, 0};
                }
            };
            auto stage = [&](int c) {
                uint8_t *tq = smem + kOffQ + (c % 3) * kQKTileB;
                uint8_t *tk = smem + kOffK + (c & 1) * kQKTileB;
                uint8_t *tv = smem + kOffV + (c % 3) * kVTileB;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int seg = ptid + 256 * s;
                    const int r = seg >> 4, col = (seg & 15) * 8;
                    if (kOut) *reinterpret_cast<u32x4 *>(tq + qk_off(r, col)) = pq[s];
                    *reinterpret_cast<u32x4 *>(tk + qk_off(r, col)) = pk[s];
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int seg = ptid + 256 * s;
                    const int r = seg >> 3, col = (seg & 7) * 8;
                    *reinterpret_cast<u32x4 *>(tv + v_off(r, col)) = pv[s];
                }
            };

            if (kOut) {
                switch (cw) {
                case 0: score_factors<0>(pf, l2, lr, lg); break;
                case 1: score_factors<1>(pf, l2, lr, lg); break;
                case 2: score_factors<2>(pf, l2, lr, lg); break;
                default: score_factors<3>(pf, l2, lr, lg); break;
                }
            }
            if (nch > 0) {
                prefetch(0);
                stage(0);
            }
            if (nch > 1) prefetch(1);
            __syncthreads();

            for (int t = 0; t <= nch; ++t) {
                if (t + 1 < nch) stage(t + 1);
                if (t + 2 < nch) prefetch(t + 2);
                if (t < nch) {
                    const uint8_t *tq = smem + kOffQ + (t % 3) * kQKTileB;
                    const uint8_t *tk = smem + kOffK + (t & 1) * kQKTileB;
                    if (kOut) {
                        uint8_t *pbuf = smem + kOffP + (t & 1) * kPBufB;
                        switch (cw) {
                        case 0: produce_scores<0>(pf, tq, tk, pbuf, lane, lr, lg); break;
                        case 1: produce_scores<1>(pf, tq, tk, pbuf, lane, lr, lg); break;
                        case 2: produce_scores<2>(pf, tq, tk, pbuf, lane, lr, lg); break;
                        default: produce_scores<3>(pf, tq, tk, pbuf, lane, lr, lg); break;
                        }
                    }
                    // K^T fragments (exact bf16) for key tiles 2cw, 2cw+1
                    uint8_t *ktbuf = smem + kOffKT + (t & 1) * kKTBufB;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const int kt = 2 * cw + kk;
#pragma unroll
                        for (int it = 0; it < 4; ++it) {
                            const u32x2 a = *reinterpret_cast<const u32x2 *>(tk + qk_off(16 * it + lr, 16 * kt + 4 * lg));
                            const f32x4 x = mfma16(a, ident, f32x4{0.f, 0.f, 0.f, 0.f});
                            *reinterpret_cast<u32x2 *>(ktbuf + ((kt * 2 + (it >> 1)) * 64 + lane) * 16 + 8 * (it & 1)) =
                                u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                        }
                    }
                }
                __syncthreads();
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------------------
thread_local char g_err[512] = "";

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
    if (flags & ~(uint32_t)(LA_STATE_READ | LA_STATE_WRITE))
        return fail(LA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
    if (!slope) return fail(LA_ERR_INVALID_ARG, "slope is NULL");
    if (pool_size < 0) return fail(LA_ERR_INVALID_ARG, "pool_size is negative");
    if (flags && (!pool || !state_idx))
        return fail(LA_ERR_INVALID_ARG, "state flags set but state_pool or state_idx is NULL");
    return LA_OK;
}

template <int MODE>
la_status launch(const Params &p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(la_chunk_kernel<MODE>, dim3(grid), dim3(kThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}

}  // namespace

extern "C" {

la_status la_prefill_fwd(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                         int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                         int32_t pool_size, const int32_t *state_idx, uint32_t flags, hipStream_t stream) {
    g_err[0] = 0;
    la_status s = check_common(H, HV, D, DV, flags, slope, state_pool, pool_size, state_idx);
    if (s != LA_OK) return s;
    if (B < 0 || T < 0) return fail(LA_ERR_INVALID_ARG, "negative B or T (B=%d, T=%d)", B, T);
    if (B == 0) return LA_OK;
    if (T == 0 && !(flags & LA_STATE_WRITE)) return LA_OK;
    if (T > 0 && (!q || !k || !v || !o)) return fail(LA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
    if ((int64_t)B * HV * kVSplit > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "too many (sequence, head) units");
    if ((int64_t)B * T > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "B * T exceeds 2^31 - 1 tokens");
    Params p{};
    p.q = (const uint16_t *)q; p.k = (const uint16_t *)k; p.v = (const uint16_t *)v; p.o = (uint16_t *)o;
    p.slope = slope; p.pool = state_pool; p.state_idx = state_idx;
    p.nseq = B; p.T = T; p.total_T = B * T; p.H = H; p.HV = HV; p.G = HV / H;
    p.pool_size = flags ? pool_size : 0; p.npairs = B * HV; p.nunits = p.npairs * kVSplit;
    p.scale = scale; p.flags = flags;
    return launch<kFixed>(p, p.nunits, stream);
}

la_status la_prefill_fwd_varlen(const void *q, const void *k, const void *v, void *o, const int32_t *cu_seqlens,
                                int32_t N, int32_t total_T, int32_t H, int32_t HV, int32_t D, int32_t DV,
                                float scale, const float *slope, float *state_pool, int32_t pool_size,
                                const int32_t *state_idx, uint32_t flags, int32_t schedule, hipStream_t stream) {
    g_err[0] = 0;
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
    p.nseq = N; p.T = 0; p.total_T = total_T; p.H = H; p.HV = HV; p.G = HV / H;
    p.pool_size = flags ? pool_size : 0; p.npairs = N * HV; p.nunits = p.npairs * kVSplit;
    p.scale = scale; p.flags = flags;
    int grid = p.nunits;
    if (schedule == LA_SCHED_PERSISTENT) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) {
            int v2 = 0;
            if (hipDeviceGetAttribute(&v2, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v2 > 0)
                cus = v2;
        }
        grid = std::min(grid, cus);
    }
    return launch<kVarlen>(p, grid, stream);
}

la_status la_state_commit(const void *k, const void *v, int32_t B, int32_t T, int32_t H, int32_t HV, int32_t D,
                          int32_t DV, const float *slope, float *state_pool, int32_t pool_size,
                          const int32_t *state_idx, const int32_t *accepted_len, hipStream_t stream) {
    g_err[0] = 0;
    la_status s = check_common(H, HV, D, DV, LA_STATE_READ | LA_STATE_WRITE, slope, state_pool, pool_size,
                               state_idx);
    if (s != LA_OK) return s;
    if (B < 0 || T < 0) return fail(LA_ERR_INVALID_ARG, "negative B or T (B=%d, T=%d)", B, T);
    if (B == 0 || T == 0) return LA_OK;
    if (!k || !v || !accepted_len) return fail(LA_ERR_INVALID_ARG, "k, v and accepted_len must be non-NULL");
    if ((int64_t)B * HV * kVSplit > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "too many (request, head) units");
    if ((int64_t)B * T > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "B * T exceeds 2^31 - 1 tokens");
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

const char *la_last_error(void) { return g_err; }

int32_t la_abi_version(void) { return LA_ABI_VERSION; }

}  // extern "C"

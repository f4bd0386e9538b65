// la_short.hip -- Lightning Attention over short sequences (T <= 16 tokens) for AMD Instinct MI355X (gfx950):
// speculative-decoding verify, multi-token decode and state commit.
//
// For a request with initial state S0 (FP32 [V][K]) and T draft tokens, every output has the closed form
//     o_t = scale ( lambda^{t+1} S0 q_t + sum_{i<=t} lambda^{t-i} (q_t . k_i) v_i )
// and the state after the first L tokens is
//     S_L = lambda^L S0 + sum_{i<L} lambda^{L-1-i} v_i k_i^T
// (page "[LA] Lightning Attention MTP decode + KVBuffer parallel verify / commit", Description: closed form
// used by verify, and the state-update / commit kernel). Both are computed straight from S0 in one pass, with
// no intermediate states.
//
// Work decomposition: wave w of a (request, value head) unit owns value rows [32w, 32w+32) of the state; value rows
// never interact, so the 4 waves of a unit are independent. They run as one 4-wave workgroup per unit, or, when
// there are fewer units than compute units (small-batch decode), as 4 one-wave workgroups per unit so that the
// state loads spread over 4 times as many CUs (the launch picks the form). Each wave holds its rows as 2 x 8 tiles
// of MFMA accumulators (tile kt: lane (lr, lg) holds
// S[v = 32w + 16vt + lr][k] for the keys k = kappa(kt, lg, r) = 32(kt/2) + 8lg + 4(kt%2) + r). The state is
// the dominant HBM traffic (64 KiB per request and head); each lane loads and stores it in 16-byte pieces.
//
// Matrix-core mapping (FP32 accumulate):
//   scores    A^T[i][t] = k_i . q_t                    16x16x32, K rows x Q rows, 4 steps over d
//   history   Y[v][t] = sum_k S0[v][k] q_t[k]           16x16x32, S0 as bf16 hi + lo, Q rows
//   intra     O^T[v][t] += sum_i V^T[v][i] P^T[i][t]     16x16x16, P^T = decay-masked scores as bf16 hi + lo
//   update    S^T[k][v] = lambda^L S^T + sum_i K^T[k][i] V_dec[i][v]   16x16x16, V_dec as bf16 hi + lo
// V^T and K^T fragments come from one 16x16x16 MFMA against the identity per 16x16 tile (exact).

#include <algorithm>

#include "la_common.h"

using namespace la_detail;

namespace {

constexpr int kShortThreads = 256;

struct ShortParams {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    uint16_t *kbuf, *vbuf;
    const float *slope;
    float *pool;
    const int32_t *state_idx, *accepted_len, *state_idx_out;
    int32_t B, T, H, HV, G, pool_size;
    float scale;
    uint32_t flags;
    int32_t rows_by_slot;
    int32_t wave_units;         // 1: one-wave workgroups, 4 per unit (blockIdx = 4 unit + wave)
};

template <bool kCommitMode>
__global__ __launch_bounds__(kShortThreads) void la_short_kernel(ShortParams p) {
    constexpr bool kOut = !kCommitMode;
    const int unit = p.wave_units ? (int)(blockIdx.x >> 2) : (int)blockIdx.x;
    const int b = unit / p.HV;
    const int hv = unit - b * p.HV;
    const int h = hv / p.G;
    const int w = p.wave_units ? (int)(blockIdx.x & 3) : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15, lg = lane >> 4;

    int slot = -1, slot_out = -1;
    if (p.flags & (LA_STATE_READ | LA_STATE_WRITE)) {
        const int s = p.state_idx[b];
        if (s >= 0 && s < p.pool_size) slot = s;
        slot_out = slot;
        if (p.state_idx_out) {
            const int so = p.state_idx_out[b];
            slot_out = (so >= 0 && so < p.pool_size) ? so : -1;
        }
    }
    int len;
    int64_t row0;
    if (kCommitMode) {
        len = min(max(p.accepted_len[b], 0), p.T);
        if (slot < 0 || len == 0) return;                 // skipped request / L = 0: no write at all
        row0 = (int64_t)(p.rows_by_slot ? slot : b) * p.T;
    } else {
        len = p.T;
        row0 = (int64_t)b * p.T;
    }
    const bool read = slot >= 0 && (p.flags & LA_STATE_READ);
    const bool write = slot_out >= 0 && (p.flags & LA_STATE_WRITE);
    const float l2 = log2_lambda(p.slope[(p.flags & LA_DECAY_PER_QK_HEAD) ? h : hv]);
    const int qk_stride = p.H * kD * 2;                   // bytes between token rows
    const int v_stride = p.HV * kDV * 2;
    const int v0 = 32 * w;                                // first value row of this wave

    // ---------------------------------------------------------------- loads: state, then token rows
    float *plane = slot >= 0 ? p.pool + ((int64_t)slot * p.HV + hv) * (kDV * kD) : nullptr;
    float *plane_out = slot_out >= 0 ? p.pool + ((int64_t)slot_out * p.HV + hv) * (kDV * kD) : nullptr;
    f32x4 S[2][8];
    if (read) {
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
                S[vt][kt] = *reinterpret_cast<const f32x4 *>(plane + (v0 + 16 * vt + lr) * kD + 32 * (kt >> 1) +
                                                               8 * lg + 4 * (kt & 1));
    } else {
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) S[vt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // rows >= len fall outside the buffer ranges and read as zeros
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.k + (row0 * p.H + h) * kD), 0, (len - 1) * qk_stride + kD * 2, kBufDword3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.v + (row0 * p.HV + hv) * kDV), 0, (len - 1) * v_stride + kDV * 2, kBufDword3);
    // K and Q rows as 16x16x32 fragments: lane (lr, lg) holds row lr, columns 32ks + 8lg .. +7
    u32x4 kq[4], qq[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        kq[ks] = __builtin_amdgcn_raw_buffer_load_b128(rk, lr * qk_stride + (32 * ks + 8 * lg) * 2, 0, 0);
    if (kOut) {
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.q + (row0 * p.H + h) * kD), 0, (len - 1) * qk_stride + kD * 2, kBufDword3);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qq[ks] = __builtin_amdgcn_raw_buffer_load_b128(rq, lr * qk_stride + (32 * ks + 8 * lg) * 2, 0, 0);
    }
    // V rows: lane (lr, lg) holds row lr, value columns v0 + 16vt + 4lg .. +3
    u32x2 vr[2];
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
        vr[vt] = __builtin_amdgcn_raw_buffer_load_b64(rv, lr * v_stride + (v0 + 16 * vt + 4 * lg) * 2, 0, 0);

    // the KV buffer keeps this request's T rows at its slot (k once per q/k head)
    if (kOut && p.vbuf && slot >= 0) {
        const __amdgpu_buffer_rsrc_t rvb = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.vbuf + ((int64_t)slot * p.T * p.HV + hv) * kDV), 0, (p.T - 1) * v_stride + kDV * 2,
            kBufDword3);
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
            __builtin_amdgcn_raw_buffer_store_b64(vr[vt], rvb, lr * v_stride + (v0 + 16 * vt + 4 * lg) * 2, 0, 0);
        if (w == 0 && hv % p.G == 0) {
            const __amdgpu_buffer_rsrc_t rkb = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(p.kbuf + ((int64_t)slot * p.T * p.H + h) * kD), 0, (p.T - 1) * qk_stride + kD * 2,
                kBufDword3);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                __builtin_amdgcn_raw_buffer_store_b128(kq[ks], rkb, lr * qk_stride + (32 * ks + 8 * lg) * 2, 0, 0);
        }
    }

    s16x4 ident;
#pragma unroll
    for (int e = 0; e < 4; ++e) ident[e] = (4 * lg + e == lr) ? (short)0x3F80 : (short)0;
    // V^T (exact): lane (lr, lg) receives V[i = 4lg + r][v0 + 16vt + lr]
    f32x4 xv[2];
    u32x2 vf[2];
#pragma unroll
    for (int vt = 0; vt < 2; ++vt) {
        xv[vt] = mfma16(vr[vt], ident, f32x4{0.f, 0.f, 0.f, 0.f});
        vf[vt] = u32x2{pack_bf16x2(xv[vt][0], xv[vt][1]), pack_bf16x2(xv[vt][2], xv[vt][3])};
    }

    if (kOut) {
        // ------------------------------------------------------------ outputs
        // scores A^T[i][t]: lane holds t = lr, i = 4lg + r; P^T = scale lambda^{t-i} A^T for i <= t
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a = mfma32(kq[ks], qq[ks], a);
        float pfac[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lg + r;
            pfac[r] = (i <= lr) ? p.scale * lam_pow(l2, lr - i) : 0.f;
        }
        const u32x2 p01 = split_bf16x2(a[0] * pfac[0], a[1] * pfac[1]);
        const u32x2 p23 = split_bf16x2(a[2] * pfac[2], a[3] * pfac[3]);
        const u32x2 phi = u32x2{p01.x, p23.x}, plo = u32x2{p01.y, p23.y};
        const float finter = p.scale * lam_pow(l2, lr + 1);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.o + (row0 * p.HV + hv) * kDV), 0, (len - 1) * v_stride + kDV * 2, kBufDword3);
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
            f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
            if (read) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x2 s0 = split_bf16x2(S[vt][2 * j][0], S[vt][2 * j][1]);
                    const u32x2 s1 = split_bf16x2(S[vt][2 * j][2], S[vt][2 * j][3]);
                    const u32x2 s2 = split_bf16x2(S[vt][2 * j + 1][0], S[vt][2 * j + 1][1]);
                    const u32x2 s3 = split_bf16x2(S[vt][2 * j + 1][2], S[vt][2 * j + 1][3]);
                    y = mfma32(u32x4{s0.x, s1.x, s2.x, s3.x}, qq[j], y);
                    y = mfma32(u32x4{s0.y, s1.y, s2.y, s3.y}, qq[j], y);
                }
            }
            y = y * finter;
            y = mfma16(vf[vt], phi, y);
            y = mfma16(vf[vt], plo, y);
            // lane holds O[t = lr][v0 + 16vt + 4lg .. +3]; rows t >= len are dropped by the buffer range
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])}, ro,
                                                  lr * v_stride + (v0 + 16 * vt + 4 * lg) * 2, 0, 0);
        }
    }

    if (write) {
        // ------------------------------------------------------------ state after len tokens
        // K^T tiles (exact): tile kt, lane (lr, lg) receives K[i = 4lg + r][kappa(kt, lr/4, lr%4)]
        u32x2 kT[8];
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            const u32x2 src = (kt & 1) ? u32x2{kq[kt >> 1].z, kq[kt >> 1].w} : u32x2{kq[kt >> 1].x, kq[kt >> 1].y};
            const f32x4 x = mfma16(src, ident, f32x4{0.f, 0.f, 0.f, 0.f});
            kT[kt] = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        }
        // V_dec[i][v] = lambda^{len-1-i} v_i as bf16 hi + lo; missing rows get a zero factor
        float fvd[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lg + r;
            fvd[r] = (i < len) ? lam_pow(l2, len - 1 - i) : 0.f;
        }
        const float dec = lam_pow(l2, len);
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
            const u32x2 d01 = split_bf16x2(xv[vt][0] * fvd[0], xv[vt][1] * fvd[1]);
            const u32x2 d23 = split_bf16x2(xv[vt][2] * fvd[2], xv[vt][3] * fvd[3]);
            const u32x2 vdh = u32x2{d01.x, d23.x}, vdl = u32x2{d01.y, d23.y};
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                f32x4 s = S[vt][kt] * dec;
                s = mfma16(kT[kt], vdh, s);
                s = mfma16(kT[kt], vdl, s);
                *reinterpret_cast<f32x4 *>(plane_out + (v0 + 16 * vt + lr) * kD + 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1)) = s;
            }
        }
    }
}

}  // namespace

namespace la_detail {

la_status launch_short(const ShortCall &c, hipStream_t stream) {
    if (c.T > kShortMax || c.T <= 0) return fail(LA_ERR_UNSUPPORTED, "short path takes 1 <= T <= %d (T=%d)", kShortMax, c.T);
    if ((int64_t)c.B * c.HV * 4 > INT32_MAX) return fail(LA_ERR_UNSUPPORTED, "too many (request, head) units");
    ShortParams p{};
    p.q = (const uint16_t *)c.q; p.k = (const uint16_t *)c.k; p.v = (const uint16_t *)c.v; p.o = (uint16_t *)c.o;
    p.kbuf = (uint16_t *)c.kbuf; p.vbuf = (uint16_t *)c.vbuf;
    p.slope = c.slope; p.pool = c.pool; p.state_idx = c.state_idx; p.accepted_len = c.accepted_len;
    p.state_idx_out = c.state_idx_out;
    p.B = c.B; p.T = c.T; p.H = c.H; p.HV = c.HV; p.G = c.HV / c.H;
    p.pool_size = (c.flags & (LA_STATE_READ | LA_STATE_WRITE)) ? c.pool_size : 0;
    p.scale = c.scale; p.flags = c.flags; p.rows_by_slot = c.rows_by_slot ? 1 : 0;
    // work units: with fewer (request, head) units than CUs, one-wave workgroups reach 4x as many CUs
    const int units = c.B * c.HV;
    p.wave_units = units < cu_count() ? 1 : 0;
    const dim3 grid(p.wave_units ? 4 * units : units), block(p.wave_units ? 64 : kShortThreads);
    if (c.commit)
        hipLaunchKernelGGL(la_short_kernel<true>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(la_short_kernel<false>, grid, block, 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}

}  // namespace la_detail

extern "C" {

la_status la_decode_mtp(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                        int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                        int32_t pool_size, const int32_t *state_idx, hipStream_t stream) {
    return la_prefill_fwd(q, k, v, o, B, T, H, HV, D, DV, scale, slope, state_pool, pool_size, state_idx,
                          LA_STATE_READ | LA_STATE_WRITE, stream);
}

la_status la_verify_kvbuffer(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                             int32_t HV, int32_t D, int32_t DV, float scale, const float *slope,
                             const float *state_pool, int32_t pool_size, const int32_t *state_idx, void *k_buf,
                             void *v_buf, hipStream_t stream) {
    clear_error();
    la_status s = check_common(H, HV, D, DV, LA_STATE_READ, slope, state_pool, pool_size, state_idx);
    if (s != LA_OK) return s;
    if (B < 0 || T < 0) return fail(LA_ERR_INVALID_ARG, "negative B or T (B=%d, T=%d)", B, T);
    if (T > kShortMax) return fail(LA_ERR_UNSUPPORTED, "verify takes at most %d draft tokens (T=%d)", kShortMax, T);
    if (B == 0 || T == 0) return LA_OK;
    if (!q || !k || !v || !o) return fail(LA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
    if ((k_buf == nullptr) != (v_buf == nullptr)) return fail(LA_ERR_INVALID_ARG, "k_buf and v_buf must both be given or both be NULL");
    ShortCall c{};
    c.q = q; c.k = k; c.v = v; c.o = o; c.kbuf = k_buf; c.vbuf = v_buf;
    c.slope = slope; c.pool = const_cast<float *>(state_pool); c.state_idx = state_idx;
    c.B = B; c.T = T; c.H = H; c.HV = HV; c.pool_size = pool_size; c.scale = scale; c.flags = LA_STATE_READ;
    return launch_short(c, stream);
}

la_status la_state_commit_kvbuffer(const void *k_buf, const void *v_buf, int32_t B, int32_t T, int32_t H, int32_t HV,
                                   int32_t D, int32_t DV, const float *slope, float *state_pool, int32_t pool_size,
                                   const int32_t *state_idx, const int32_t *accepted_len, hipStream_t stream) {
    clear_error();
    la_status s = check_common(H, HV, D, DV, LA_STATE_READ | LA_STATE_WRITE, slope, state_pool, pool_size,
                               state_idx);
    if (s != LA_OK) return s;
    if (B < 0 || T < 0) return fail(LA_ERR_INVALID_ARG, "negative B or T (B=%d, T=%d)", B, T);
    if (T > kShortMax) return fail(LA_ERR_UNSUPPORTED, "commit takes at most %d draft tokens (T=%d)", kShortMax, T);
    if (B == 0 || T == 0) return LA_OK;
    if (!k_buf || !v_buf || !accepted_len) return fail(LA_ERR_INVALID_ARG, "k_buf, v_buf and accepted_len must be non-NULL");
    ShortCall c{};
    c.k = k_buf; c.v = v_buf; c.slope = slope; c.pool = state_pool; c.state_idx = state_idx;
    c.accepted_len = accepted_len; c.B = B; c.T = T; c.H = H; c.HV = HV; c.pool_size = pool_size; c.scale = 1.0f;
    c.flags = LA_STATE_READ | LA_STATE_WRITE; c.commit = true; c.rows_by_slot = true;
    return launch_short(c, stream);
}

}  // extern "C"

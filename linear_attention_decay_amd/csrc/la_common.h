// la_common.h -- device helpers and host error handling shared by the prefill and short-sequence kernels of
// the Lightning Attention library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_prefill.h"

namespace la_detail {

constexpr int kD = 128;                      // key dim
constexpr int kDV = 128;                     // value dim
constexpr int kBufDword3 = 0x00020000;       // buffer resource word 3: raw 32-bit data format

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 f = {a, b};
    bf16x2 h = __builtin_convertvector(f, bf16x2);   // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, h);
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi); two values per call, returned as {hi pair, lo pair}.
// The residual x - hi is exact in FP32; it is formed by one bf16 dot product against (-1, 0) or (0, -1)
// accumulated onto x. The two masks are passed in registers: given the pair (-1, 0) as a constant, the
// compiler encodes it as the inline constant -1.0, which the hardware reads as the FP32 bit pattern
// 0xBF800000, i.e. the pair (0, -1).
__device__ __forceinline__ u32x2 split_bf16x2(float a, float b) {
    f32x2 f = {a, b};
    const bf16x2 hi = __builtin_convertvector(f, bf16x2);
    uint32_t m0 = 0x0000BF80u, m1 = 0xBF800000u;     // bf16 pairs (-1, 0) and (0, -1), element 0 low
    asm("" : "+v"(m0), "+v"(m1));
    const float ra = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2, m0), a, false);
    const float rb = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2, m1), b, false);
    return u32x2{__builtin_bit_cast(uint32_t, hi), pack_bf16x2(ra, rb)};
}

__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(u32x2 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                     c, 0, 0, 0);
}

// lambda^n for n >= 0 given l2 = log2(lambda) (finite, <= 0).
__device__ __forceinline__ float lam_pow(float l2, int n) { return __builtin_amdgcn_exp2f(l2 * (float)n); }

// log2(lambda) for lambda = exp(-slope); slope = +inf gives lambda^0 = 1, lambda^n = 0 for n > 0
__device__ __forceinline__ float log2_lambda(float slope) {
    return fmaxf(-slope * 1.4426950408889634f, -1.0e30f);
}

// host side: the thread-local error detail behind la_last_error(), and the argument checks every entry point
// makes before it enqueues anything
void clear_error();
la_status fail(la_status s, const char *fmt, ...);
// compute units of the current device (cached per device; 256 if the query fails)
int cu_count();

la_status check_common(int32_t H, int32_t HV, int32_t D, int32_t DV, uint32_t flags, const float *slope,
                       const float *pool, int32_t pool_size, const int32_t *state_idx);

// short-sequence path (T <= kShortMax), implemented next to its kernel
constexpr int kShortMax = 16;
// largest value-head count: a chunk's 64 token rows of HV * 256 bytes are addressed with 32-bit offsets
constexpr int kMaxHeads = 65536;
struct ShortCall {
    const void *q, *k, *v;       // token rows [B, T, H|HV, 128]; for a commit from a KV buffer, rows of slot s
    void *o;                     // output [B, T, HV, 128], or NULL when no output is produced
    void *kbuf, *vbuf;           // KV buffer to fill with the T rows of every request with a valid slot, or NULL
    const float *slope;
    float *pool;
    const int32_t *state_idx, *accepted_len;
    const int32_t *state_idx_out;  // slot that receives the final state; NULL: the slot read from
    int32_t B, T, H, HV, pool_size;
    float scale;
    uint32_t flags;
    bool commit;                 // state update over the first accepted_len[b] rows only, no output
    bool rows_by_slot;           // commit: token rows are indexed by the request's slot (KV buffer)
};
la_status launch_short(const ShortCall &c, hipStream_t stream);

}  // namespace la_detail

/*
 * la_prefill.h -- C ABI of the Lightning Attention chunked prefill library for AMD Instinct MI355X (gfx950).
 *
 * The operation (page "[LA] Lightning Attention MTP decode + KVBuffer parallel verify / commit", Description,
 * the closed form used by verify; page "[Lightning Attention] Add Hopper SM90 CuTe DSL prefill", Description
 * and Reviewer notes): for every sequence and value head hv, with q/k head h = hv / (HV / H) and
 * lambda = exp(-slope[hv]),
 *
 *     S_t = lambda * S_{t-1} + v_t k_t^T,     o_t = scale * S_t q_t,     S_{-1} = S0 (or 0),
 *
 * i.e. o_t = scale * (lambda^{t+1} S0 q_t + sum_{i<=t} lambda^{t-i} (q_t . k_i) v_i). S is FP32, DV x D = 128 x 128,
 * in [V, K] orientation (row = value index, column = key index). The library evaluates it in 64-token chunks on
 * bf16 matrix cores with FP32 accumulation; the FP32 state stays on chip across a sequence's chunks.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library never allocates, frees or
 *     synchronises, and never reads device memory from the host. All work is enqueued on `stream`, which is
 *     passed to the runtime verbatim (0 is the null stream).
 *   - Tensors are dense and row-major with the last dimension fastest:
 *       q, k  : bf16 [tokens, H, 128]        v, o : bf16 [tokens, HV, 128]
 *       state pool : fp32 [pool_size, HV, 128 (V), 128 (K)]      slope : fp32 [HV]
 *     Fixed-length calls index tokens as b * T + t. Pointers must be 16-byte aligned.
 *   - State pool: sequence n uses slot state_idx[n]. A slot < 0 or >= pool_size means "no state": the
 *     sequence starts from zero and its final state is not stored. With LA_STATE_READ the initial state is
 *     read from the slot; with LA_STATE_WRITE the final state is stored into the same slot (in place).
 *     Slots no sequence selects are never touched. Two sequences selecting the same slot with
 *     LA_STATE_WRITE is undefined. state_pool / state_idx may be NULL only when flags == 0.
 *   - o is written for every valid token (nothing relies on o being pre-initialised).
 *   - Device values (slot indices, cu_seqlens, accepted lengths) are not validated and cost no host sync;
 *     out-of-range values are clamped or skipped on the device as documented per call, never dereferenced
 *     out of bounds. Slopes must be >= 0 (+inf is allowed and means lambda = 0).
 *   - Host-checkable problems return an error before anything is enqueued:
 *       D != 128, DV != 128, H <= 0, HV % H != 0            -> LA_ERR_UNSUPPORTED
 *       HV > 65536 (row strides are 32-bit byte offsets)  -> LA_ERR_UNSUPPORTED
 *       negative sizes, NULL required pointer, bad flags     -> LA_ERR_INVALID_ARG
 *     A NULL state_pool / state_idx is allowed when flags holds neither LA_STATE_READ nor LA_STATE_WRITE.
 *     A call with no tokens and no sequences is a successful no-op. A launch failure returns LA_ERR_HIP.
 *     la_last_error() then describes the failure (thread-local).
 */
#ifndef LA_PREFILL_H
#define LA_PREFILL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 2

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = 1,
    LA_ERR_UNSUPPORTED = 2,
    LA_ERR_HIP = 3
} la_status;

/* flags bitmask. LA_DECAY_PER_QK_HEAD (prefill page, Performance: the GVA rows with decay owned per value head,
 * "_hv", and per q/k head, "_h"): slope has H entries and value head hv uses slope[hv / (HV / H)]; without it
 * slope has HV entries. */
enum { LA_STATE_READ = 1u, LA_STATE_WRITE = 2u, LA_DECAY_PER_QK_HEAD = 4u };

/* packed-sequence scheduling */
enum { LA_SCHED_AUTO = 0, LA_SCHED_PERSISTENT = 1, LA_SCHED_NONPERSISTENT = 2 };

/*
 * Fixed-length batched prefill (prefill page, Description: fixed-length BF16 prefill, optional initial/final
 * state, MHA and GVA, explicit state-pool indices).
 *   q, k        : bf16 [B, T, H, 128];  v, o : bf16 [B, T, HV, 128]
 *   scale       : multiplies both the history term and the within-sequence term
 *   state_idx   : int32 [B] (device)
 * B == 0 or T == 0 is a no-op except that, with T == 0 and LA_STATE_WRITE, each selected slot receives its
 * initial state (S0 with LA_STATE_READ, else zeros). Calls with 1 <= T <= 16 (draft-token verify and
 * multi-token decode) take a one-pass kernel that evaluates the closed form from the initial state; longer
 * ones take the 64-token chunked kernel.
 */
la_status la_prefill_fwd(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                         int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                         int32_t pool_size, const int32_t *state_idx, uint32_t flags, hipStream_t stream);

/*
 * As la_prefill_fwd, with the final state stored into a slot of its own (prefill page, comparison notes:
 * indirect / shared state-pool ownership). Sequence b reads its initial state from state_idx[b] (LA_STATE_READ)
 * and stores its final state into state_idx_out[b] (LA_STATE_WRITE); an out slot < 0 or >= pool_size stores
 * nothing. Several sequences may read the same slot. A slot that one sequence writes must not be read or
 * written by another sequence of the same call (undefined). state_idx_out == NULL means state_idx.
 *   state_idx_out : int32 [B] (device)
 */
la_status la_prefill_fwd_ex(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                            int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                            int32_t pool_size, const int32_t *state_idx, const int32_t *state_idx_out,
                            uint32_t flags, hipStream_t stream);

/*
 * Fixed-length prefill with every sequence split into segments processed in parallel, for calls whose
 * (sequence, head) units cannot fill the GPU (few long sequences, few heads). Results as la_prefill_fwd_ex.
 * The segments use the linear-attention form of the segmented scan (KDA sm90 page, Description: chunk-parallel
 * PREP, sequential SCAN over the state):
 *   1. each segment but the last runs from a zero state over its tokens and keeps its local state L_g;
 *   2. a scan forms every segment's initial state, S_{g+1} = lambda^{seg_len} S_g + L_g, with S_0 the pool
 *      state (LA_STATE_READ) or zero;
 *   3. every segment runs the full prefill from its initial state; the last one stores the final state.
 * segments : requested number of segments; 0 chooses one from the device's CU count (enough workgroups for
 *            every CU, segments of at least 4 chunks). Segments are whole 64-token chunks, so fewer may be used;
 *            with one segment, or T <= 16, the call is exactly la_prefill_fwd_ex.
 * workspace: device buffer of at least la_prefill_seg_workspace_bytes(B, HV, segments actually used) bytes,
 *            owned by the caller, not touched when one segment is used. la_prefill_seg_workspace_bytes(B, HV, n)
 *            for the requested n is always enough (segments = 0: n = CU count / (2 B HV), at least 1). Calls
 *            sharing a workspace must be ordered on one stream. Too small: LA_ERR_INVALID_ARG.
 * Extra HBM traffic: k and v of all but the last segment are read twice, plus 3 state planes per segment.
 */
la_status la_prefill_fwd_seg(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                             int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                             int32_t pool_size, const int32_t *state_idx, const int32_t *state_idx_out,
                             uint32_t flags, int32_t segments, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * la_prefill_fwd_seg without a workspace argument, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Arguments, results and errors as
 * la_prefill_fwd_seg. The per-segment states live in a fixed device array of the library instead of a caller
 * workspace:
 *   - its size is la_prefill_seg_noalloc_max_bytes() (16 MiB: B * segments * HV <= 256 state planes); a call
 *     whose segment count needs more returns LA_ERR_UNSUPPORTED before anything is enqueued (choose fewer
 *     segments, or use la_prefill_fwd_seg with a workspace). segments = 0 on a 256-CU device always fits;
 *   - every device that runs the library holds one copy until the process ends; its address is looked up once
 *     per device (the first call on a device), the only runtime call besides the launches;
 *   - this call allocates and frees nothing, and nothing in the array has to start at zero: each call writes
 *     every entry it reads before reading it;
 *   - all calls on one device share the array, so calls that overlap in time on one device (different streams
 *     without ordering between them) race and give undefined results; order them on one stream.
 * Calls that need one segment (or T <= 16) do not touch the array.
 */
la_status la_prefill_fwd_seg_noalloc(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T,
                                     int32_t H, int32_t HV, int32_t D, int32_t DV, float scale, const float *slope,
                                     float *state_pool, int32_t pool_size, const int32_t *state_idx,
                                     const int32_t *state_idx_out, uint32_t flags, int32_t segments,
                                     hipStream_t stream);

/* Bytes of the fixed device array la_prefill_fwd_seg_noalloc uses (its largest segment workspace). */
size_t la_prefill_seg_noalloc_max_bytes(void);

/* Workspace bytes la_prefill_fwd_seg needs for B sequences, HV value heads and the given segment count
 * (0 for segments <= 1). */
size_t la_prefill_seg_workspace_bytes(int32_t B, int32_t HV, int32_t segments);

/*
 * Packed variable-length prefill (prefill page, Description: packed variable-length BF16 prefill; persistent
 * or non-persistent packed scheduling). Sequence n occupies token rows [cu_seqlens[n], cu_seqlens[n+1]);
 * chunks never straddle sequences.
 *   q, k        : bf16 [total_T, H, 128];  v, o : bf16 [total_T, HV, 128]
 *   cu_seqlens  : int32 [N + 1] (device), cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] = total_T.
 *                 Values are clamped into [0, total_T] on the device.
 *   state_idx   : int32 [N] (device)
 *   schedule    : LA_SCHED_* ; every schedule produces bitwise identical o and states.
 * A zero-length sequence writes no output; with LA_STATE_WRITE its slot receives its initial state.
 */
la_status la_prefill_fwd_varlen(const void *q, const void *k, const void *v, void *o, const int32_t *cu_seqlens,
                                int32_t N, int32_t total_T, int32_t H, int32_t HV, int32_t D, int32_t DV,
                                float scale, const float *slope, float *state_pool, int32_t pool_size,
                                const int32_t *state_idx, uint32_t flags, int32_t schedule, hipStream_t stream);

/* As la_prefill_fwd_varlen, with a separate out slot per sequence (state_idx_out: int32 [N]; semantics as
 * la_prefill_fwd_ex). */
la_status la_prefill_fwd_varlen_ex(const void *q, const void *k, const void *v, void *o, const int32_t *cu_seqlens,
                                   int32_t N, int32_t total_T, int32_t H, int32_t HV, int32_t D, int32_t DV,
                                   float scale, const float *slope, float *state_pool, int32_t pool_size,
                                   const int32_t *state_idx, const int32_t *state_idx_out, uint32_t flags,
                                   int32_t schedule, hipStream_t stream);

/*
 * Commit after a short-chunk verify (verify page, Description and Tests). Once the caller knows how many of
 * request b's T draft tokens were accepted (L = accepted_len[b]), its pooled state moves past exactly those L:
 *     S <- lambda^L S + sum_{i<L} lambda^{L-1-i} v_i k_i^T
 *   k           : bf16 [B, T, H, 128];  v : bf16 [B, T, HV, 128]
 *   state_idx   : int32 [B] (device); slot < 0 or >= pool_size: request skipped
 *   accepted_len: int32 [B] (device), 0 <= L <= T (clamped into that range on the device)
 * L == 0 leaves the slot bitwise unchanged. The verify outputs themselves come from la_prefill_fwd with
 * flags = LA_STATE_READ on the same T draft tokens.
 */
la_status la_state_commit(const void *k, const void *v, int32_t B, int32_t T, int32_t H, int32_t HV, int32_t D,
                          int32_t DV, const float *slope, float *state_pool, int32_t pool_size,
                          const int32_t *state_idx, const int32_t *accepted_len, hipStream_t stream);

/*
 * Fused multi-token decode (verify page, Description). One launch runs every (request, head) through its T draft
 * tokens: it returns each token's output and stores the state reached after the last token back into the
 * request's slot, i.e. la_prefill_fwd with flags = LA_STATE_READ | LA_STATE_WRITE.
 *   q, k        : bf16 [B, T, H, 128];  v, o : bf16 [B, T, HV, 128];  state_idx : int32 [B] (device)
 *   state_pool, state_idx must be non-NULL. 1 <= T <= 16 runs in one pass; longer T are chunked.
 */
la_status la_decode_mtp(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                        int32_t HV, int32_t D, int32_t DV, float scale, const float *slope, float *state_pool,
                        int32_t pool_size, const int32_t *state_idx, hipStream_t stream);

/*
 * Parallel verify with a KV buffer (verify page, Description). Each draft token's output is evaluated from the
 * request's starting state by the closed-form sum over the draft prefix, so the state after an intermediate
 * token never exists; the draft k and v rows can be kept on the side for a later commit. Outputs as
 * la_prefill_fwd with flags = LA_STATE_READ (the pool is only read).
 * For every request b whose slot s = state_idx[b] is valid, the T draft rows of k and v are also copied to
 *   k_buf : bf16 [pool_size, T, H, 128]   rows k_buf[s, t]      v_buf : bf16 [pool_size, T, HV, 128]
 * so that la_state_commit_kvbuffer can advance the state later without the caller keeping k and v. Buffer
 * slots of skipped requests (slot < 0 or >= pool_size) are not touched. k_buf and v_buf are both NULL (no
 * buffer write) or both non-NULL. T <= 16, else LA_ERR_UNSUPPORTED.
 */
la_status la_verify_kvbuffer(const void *q, const void *k, const void *v, void *o, int32_t B, int32_t T, int32_t H,
                             int32_t HV, int32_t D, int32_t DV, float scale, const float *slope,
                             const float *state_pool, int32_t pool_size, const int32_t *state_idx, void *k_buf,
                             void *v_buf, hipStream_t stream);

/*
 * Commit from the KV buffer (verify page, Description and Tests): la_state_commit with the token rows read back
 * from the buffer la_verify_kvbuffer filled, so the caller need not keep k and v. Request b's rows are
 * k_buf[state_idx[b], 0 .. L-1] and v_buf[state_idx[b], 0 .. L-1] (layouts as written by la_verify_kvbuffer with
 * the same T). Out-of-range slots and L == 0 behave as in la_state_commit. T <= 16.
 */
la_status la_state_commit_kvbuffer(const void *k_buf, const void *v_buf, int32_t B, int32_t T, int32_t H, int32_t HV,
                                   int32_t D, int32_t DV, const float *slope, float *state_pool, int32_t pool_size,
                                   const int32_t *state_idx, const int32_t *accepted_len, hipStream_t stream);

/* Static name of a status code. */
const char *la_status_string(la_status s);

/* Thread-local description of the last non-OK status returned on this thread ("" if none). */
const char *la_last_error(void);

/* LA_ABI_VERSION of the built library. */
int32_t la_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_PREFILL_H */

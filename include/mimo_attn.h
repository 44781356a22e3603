/*
 * mimo_attn.h - C ABI of the MI355X (gfx950) sink-seeded sliding-window / global attention library.
 *
 * The operation (MiMo-V2-Flash Technical Report review (xllm-io), §3.1-§3.2; MiMo series notes
 * (plmsmile), MiMo-V2-Flash > local window and > Learnable Attention Sink > mechanism):
 * for batch b, query head h (KV head g = map(h)) and query position i,
 *
 *     s_ij  = scale * <q[b,i,h,:], k[b,j,g,:]>            for visible keys j
 *     o[b,i,h,:] = sum_j exp(s_ij) v[b,j,g,:] / (exp(sink[h]) + sum_j exp(s_ij))
 *     lse   = log(exp(sink[h]) + sum_j exp(s_ij))           (natural log, sink included)
 *
 * Key j is visible to query i iff 0 <= i - j < window (the window counts the query's own key);
 * window >= sequence length gives plain causal (global) attention. The sink is a per-query-head
 * logit that enters only the denominator: it is not multiplied by `scale` and carries no value, so
 * the weights of the real keys sum to less than one. A NULL sink pointer means "no sink".
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major, last dimension contiguous, and 16-byte aligned.
 *  - Every pointer except `kv_head_of_q` is a DEVICE pointer owned by the caller. The library
 *    allocates nothing, frees nothing and never synchronises: work is enqueued on `stream` and the
 *    call returns. Its only state is a thread-local error string and, for
 *    mimo_attn_decode_noalloc, a static device scratch array (and its address on each device).
 *  - All arguments are validated on the host before anything is launched. On a non-zero return
 *    nothing has been launched and no output has been written; mimo_attn_last_error() explains.
 *  - Device faults are asynchronous and surface at the caller's next synchronisation.
 *  - Results are deterministic: fixed reduction order, no atomics.
 *  - The library is reentrant; calls that write the same outputs or workspace race.
 *  - Sink entries may be finite or -inf; +inf or NaN sink entries give undefined results.
 *  - Supported head dims: d_qk = 192, d_v = 128 (the MiMo-V2-Flash shapes); anything else returns
 *    MIMO_EUNSUPPORTED.
 */
#ifndef MIMO_ATTN_H
#define MIMO_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtype shared by q, k, v, the caches and o. Softmax and accumulation are fp32 for both.
 * The two range markers are not dtypes (every entry point rejects them with MIMO_EUNSUPPORTED, as
 * any other value); they give the type the range of an int, so that the library can examine an
 * unknown value a caller passes without undefined behaviour. */
typedef enum {
  MIMO_F32 = 0,
  MIMO_BF16 = 1,
  MIMO_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  MIMO_DTYPE_RANGE_MAX_ = 2147483647
} mimo_dtype;

enum {
  MIMO_OK = 0,
  MIMO_EINVAL = -1,      /* a size, pointer, alignment, head map or window argument is invalid */
  MIMO_EUNSUPPORTED = -2, /* valid request that the library does not implement (dtype/dims)    */
  MIMO_EWORKSPACE = -3,  /* workspace missing or smaller than the size query returned            */
  MIMO_EHIP = -4         /* the HIP runtime refused a launch                                      */
};

/*
 * Prefill: every query position of every sequence attends to its window of keys.
 *
 *   q     [B, L, Hq,  d_qk]  dtype dt        k [B, L, Hkv, d_qk]   v [B, L, Hkv, d_v]
 *   o     [B, L, Hq,  d_v]   dtype dt        (written)
 *   lse   [B, Hq, L] fp32, nullable          (written when non-NULL)
 *   sink  [Hq] fp32 device, nullable (NULL = no sink, same as every entry -inf)
 *   kv_head_of_q [Hq] int32 HOST array, nullable. NULL means h / (Hq/Hkv). Otherwise every KV head
 *         must serve exactly Hq/Hkv query heads; query heads of one KV head are processed together.
 *   window >= 1; window >= L selects global causal attention. scale multiplies q.k only and must
 *   be finite and > 0 (the usual 1/sqrt(d_qk)).
 *
 * Errors: MIMO_EINVAL for B, L, Hq, Hkv < 1, Hq % Hkv != 0, a bad head map, window < 1, NULL or
 * misaligned q/k/v/o, misaligned sink/lse, a scale that is not finite and > 0, or tensors larger
 * than 2^62 bytes;
 * MIMO_EUNSUPPORTED for other head dims or dtypes; MIMO_EHIP if the launch fails.
 */
int mimo_attn_prefill(mimo_dtype dt, int B, int L, int Hq, int Hkv, int d_qk, int d_v,
                      const void* q, const void* k, const void* v, int window, const float* sink,
                      const int32_t* kv_head_of_q, float scale, void* o, float* lse,
                      hipStream_t stream);

/*
 * Bytes of device workspace that mimo_attn_decode needs for the same arguments (0 when the
 * single-pass path is used). num_splits follows mimo_attn_decode: 0 = automatic choice.
 * Returns 0 for arguments mimo_attn_decode would reject.
 */
size_t mimo_attn_decode_workspace_size(int B, int T, int Hq, int Hkv, int d_v, int max_cache_len,
                                       int window, int num_splits);

/*
 * Decode / MTP verification: T new tokens per sequence (the next token plus up to seven drafts:
 * three MTP drafts, MiMo series notes, MiMo-V2-Flash > lightweight MTP > inference, or a block
 * draft of 6 or 8 tokens, same notes, MiMo-V2.6 decoding ablation), attending to committed cache
 * entries and, causally, to each other.
 *
 *   q       [B, T, Hq,  d_qk]            k_new [B, T, Hkv, d_qk]   v_new [B, T, Hkv, d_v]
 *   k_cache [B, C, Hkv, d_qk]            v_cache [B, C, Hkv, d_v]
 *   cache_len    [B] int32 device: committed tokens P_b (new tokens excluded), 0 <= P_b <= max_cache_len.
 *   cache_offset [B] int32 device, nullable (NULL = 0): committed position p of sequence b is stored
 *                in slot (p + cache_offset[b]) mod C. A sliding-window layer uses a ring of
 *                C >= window - 1 slots; a global layer uses a linear cache with C >= max_cache_len.
 *   New token t sits at position P_b + t and sees committed positions >= P_b + t - window + 1 and new
 *   tokens 0..t. The caller appends accepted tokens to the cache afterwards.
 *   o   [B, T, Hq, d_v] dtype dt (written);  lse [B, T, Hq] fp32, nullable.
 *   num_splits: 0 = automatic; 1 = single pass per (sequence, KV head); > 1 = split the visible keys
 *   into that many parts (partials in `workspace`) followed by a combine that adds the sink once.
 *   A part is a contiguous stretch of keys, or, for bf16 calls with more than 32 query columns per
 *   KV head, every num_splits-th block of 32 keys; either way each key enters exactly one part.
 *   workspace / workspace_bytes: device scratch of at least mimo_attn_decode_workspace_size(...)
 *   bytes (may be NULL when that size is 0). Its contents are overwritten.
 *
 * Errors: MIMO_EINVAL for sizes < 1, T outside 1..8, Hq % Hkv != 0, a bad head map, window < 1,
 * max_cache_len < 0, a cache too small for the window (C < min(window - 1, max_cache_len)),
 * num_splits < 0, NULL or misaligned pointers; MIMO_EWORKSPACE when the workspace is too small;
 * MIMO_EUNSUPPORTED for other head dims or dtypes; MIMO_EHIP if a launch fails.
 * cache_len entries outside [0, max_cache_len] are clamped into that range on the device.
 */
int mimo_attn_decode(mimo_dtype dt, int B, int T, int Hq, int Hkv, int d_qk, int d_v,
                     const void* q, const void* k_new, const void* v_new, const void* k_cache,
                     const void* v_cache, int C, const int32_t* cache_len,
                     const int32_t* cache_offset, int max_cache_len, int window,
                     const float* sink, const int32_t* kv_head_of_q, float scale, int num_splits,
                     void* workspace, size_t workspace_bytes, void* o, float* lse,
                     hipStream_t stream);

/*
 * mimo_attn_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, meaning and errors as
 * mimo_attn_decode without the workspace: split-KV partial records go to a static device array of
 * 64 MiB (67108864 bytes) inside the library, which every GPU the library runs on holds until the
 * process ends. Nothing is allocated or freed by this call (its first call on a device looks up
 * that device's address of the array once).
 *  - Requests whose partials need more than 64 MiB (mimo_attn_decode_workspace_size() > 67108864)
 *    return MIMO_EWORKSPACE; a smaller num_splits needs less.
 *  - `stream` must belong to the current device (MIMO_EINVAL otherwise).
 *  - Every call on one GPU shares that GPU's array and leaves its partials there: calls that
 *    overlap in time on one GPU (other streams, other threads) race and give wrong results. Calls
 *    ordered on one stream are safe. Nothing in the array needs to start at zero: every record a
 *    call reads is written first by the same call.
 */
int mimo_attn_decode_noalloc(mimo_dtype dt, int B, int T, int Hq, int Hkv, int d_qk, int d_v,
                             const void* q, const void* k_new, const void* v_new,
                             const void* k_cache, const void* v_cache, int C,
                             const int32_t* cache_len, const int32_t* cache_offset,
                             int max_cache_len, int window, const float* sink,
                             const int32_t* kv_head_of_q, float scale, int num_splits, void* o,
                             float* lse, hipStream_t stream);

/*
 * Rotary position embedding of the leading Q/K dimensions (MiMo-V2-Flash Technical Report review
 * (xllm-io), §3.1: RoPE on the first 64 of the 192 Q/K dims; §4: base 10K for the sliding-window
 * layers, 5M for the global layers). The rot_dims leading dims of a head vector at position p form
 * pairs (i, i + rot_dims/2), i < rot_dims/2, rotated by a = p * base^(-2i / rot_dims):
 *     x' = x cos a - y sin a,   y' = y cos a + x sin a;
 * the other dims and V are not rotated. Only rot_dims = 64 is implemented.
 *
 * mimo_attn_rope_table fills `table` [n_pos][rot_dims/2][2] fp32 (device, caller-owned) with
 * (cos a, sin a) for positions 0 .. n_pos-1, evaluated in fp64 on the device and rounded to fp32.
 * Errors: MIMO_EINVAL for n_pos outside [1, 2^30], base not finite or <= 1, NULL or misaligned
 * table; MIMO_EUNSUPPORTED for rot_dims != 64; MIMO_EHIP if the launch fails.
 */
int mimo_attn_rope_table(int n_pos, int rot_dims, double base, float* table, hipStream_t stream);

/*
 * mimo_attn_prefill for q and k given BEFORE the rotary embedding: every Q and K head vector of row
 * i is rotated by position i with rope_table (rope_positions >= L rows from mimo_attn_rope_table)
 * before the dot products; in bf16 the rotated values are rounded to bf16 (nearest even) first.
 *
 * workspace (device, caller-owned, 16-byte aligned) is optional. With NULL, K is rotated as its
 * blocks are staged, by every workgroup that reads them. With at least
 * mimo_attn_prefill_rope_workspace_size() bytes, K is rotated once into the workspace (the same
 * arithmetic, so the same results) and the attention reads it from there; the size is 0 where
 * the chosen kernel rotates each key once anyway (bf16 sliding windows of at most 129 keys with
 * a multiple of 8 query heads per KV head), and B * L * Hkv * d_qk elements otherwise. The
 * workspace contents are scratch: nothing is expected in it and nothing is left for the caller.
 *
 * Other arguments and errors as mimo_attn_prefill; additionally MIMO_EINVAL for a NULL or
 * misaligned table, rope_positions < L or a misaligned workspace, MIMO_EWORKSPACE for a
 * non-NULL workspace smaller than the size query, MIMO_EUNSUPPORTED for rot_dims != 64.
 */
size_t mimo_attn_prefill_rope_workspace_size(mimo_dtype dt, int B, int L, int Hq, int Hkv,
                                             int window);
int mimo_attn_prefill_rope(mimo_dtype dt, int B, int L, int Hq, int Hkv, int d_qk, int d_v,
                           const void* q, const void* k, const void* v, int window,
                           const float* sink, const int32_t* kv_head_of_q, float scale,
                           const float* rope_table, int rope_positions, int rot_dims,
                           void* workspace, size_t workspace_bytes, void* o, float* lse,
                           hipStream_t stream);

/*
 * mimo_attn_decode for q and k_new given BEFORE the rotary embedding: new token t of sequence b is
 * rotated by position P_b + t (rope_positions >= max_cache_len + T); the cache is expected to hold
 * keys that were rotated when their tokens were processed. Other arguments and errors as
 * mimo_attn_decode (same workspace size), plus the table checks of mimo_attn_prefill_rope.
 */
int mimo_attn_decode_rope(mimo_dtype dt, int B, int T, int Hq, int Hkv, int d_qk, int d_v,
                          const void* q, const void* k_new, const void* v_new, const void* k_cache,
                          const void* v_cache, int C, const int32_t* cache_len,
                          const int32_t* cache_offset, int max_cache_len, int window,
                          const float* sink, const int32_t* kv_head_of_q, float scale,
                          const float* rope_table, int rope_positions, int rot_dims,
                          int num_splits, void* workspace, size_t workspace_bytes, void* o,
                          float* lse, hipStream_t stream);

/*
 * Commit after a verify step: for every sequence b, the first n_b of its T new tokens (the
 * accepted prefix, n_b = accept_len[b] clamped to [0, T], all T when accept_len is NULL) are
 * written to the cache at positions P_b .. P_b + n_b - 1, P_b = cache_len[b], i.e. to slots
 * (p + cache_offset[b]) mod C - the layout mimo_attn_decode reads - and cache_len[b] becomes
 * P_b + n_b (on the device, ordered on `stream` after any earlier decode). Rejected drafts are
 * rolled back by never being written: afterwards the cache is that of the accepted sequence.
 * (MiMo series notes (plmsmile), MiMo-V2-Flash > lightweight MTP > inference: only drafts the
 * main model accepts continue the sequence; jienda explainer §4.3: fixed-size cache for the
 * sliding-window layers.)
 *
 *   k_new [B, T, Hkv, d_qk], v_new [B, T, Hkv, d_v] dtype dt: the verify step's new K / V.
 *   k_cache [B, C, Hkv, d_qk], v_cache [B, C, Hkv, d_v]: updated in place.
 *   cache_len [B] int32 device: read and advanced. cache_offset [B] int32 device, nullable (0).
 *   accept_len [B] int32 device, nullable.
 *   max_cache_len: the cache never holds more positions: n_b is also clamped to
 *   max_cache_len - P_b. A linear (global-layer) cache holds positions < C, so pass
 *   max_cache_len <= C for it; a sliding-window ring of C >= window - 1 slots may take any
 *   max_cache_len, the oldest positions being overwritten.
 *
 * Errors: MIMO_EINVAL for B, Hkv, C < 1, T outside 1..8, max_cache_len outside [0, 2^30 - 8],
 * NULL or misaligned pointers; MIMO_EUNSUPPORTED for other head dims or dtypes; MIMO_EHIP if the
 * launch fails. cache_len entries outside [0, max_cache_len] are clamped into it first.
 */
int mimo_attn_cache_append(mimo_dtype dt, int B, int T, int Hkv, int d_qk, int d_v,
                           const void* k_new, const void* v_new, void* k_cache, void* v_cache, int C,
                           int32_t* cache_len, const int32_t* cache_offset,
                           const int32_t* accept_len, int max_cache_len, hipStream_t stream);

/*
 * Backward pass of mimo_attn_prefill: gradients of a scalar loss with respect to q, k, v and the
 * sink, given the loss gradient d_o of the output (the sink is a learned per-head logit,
 * MiMo-V2-Flash Technical Report review (xllm-io), §3.2; MiMo series notes (plmsmile),
 * MiMo-V2-Flash > Learnable Attention Sink). With p_ij = exp(s_ij - lse_i) and D_i = <d_o_i, o_i>:
 *
 *     ds_ij = p_ij (<d_o_i, v_j> - D_i)
 *     dq_i = scale sum_j ds_ij k_j       dk_j = scale sum_i ds_ij q_i       dv_j = sum_i p_ij d_o_i
 *     dsink_h = -sum_{b,i} exp(sink_h - lse_i) D_i
 *
 * where dk, dv also sum over the query heads that share the KV head.
 *
 *   q, k, v, window, sink, kv_head_of_q, scale: exactly as passed to mimo_attn_prefill.
 *   o   [B, L, Hq, d_v]  dtype dt, and lse [B, Hq, L] fp32: that call's outputs (lse required).
 *   d_o [B, L, Hq, d_v]  dtype dt: gradient of the loss with respect to o.
 *   dq  [B, L, Hq, d_qk], dk [B, L, Hkv, d_qk], dv [B, L, Hkv, d_v] dtype dt: written (overwritten,
 *       not accumulated); they must not overlap the inputs.
 *   dsink [Hq] fp32 device, nullable: written when non-NULL; must be NULL when sink is NULL.
 *   workspace / workspace_bytes: device scratch of at least
 *       mimo_attn_prefill_backward_workspace_size(B, L, Hq) bytes, 16-byte aligned; overwritten.
 *
 * Products run on bf16 operands for dt = MIMO_BF16 (p and ds are rounded to bf16 before their
 * products, as the forward does with p) and accumulate in fp32; dt = MIMO_F32 stays in fp32.
 * Errors: those of mimo_attn_prefill, plus MIMO_EINVAL for NULL or misaligned o, lse, d_o, dq,
 * dk, dv, workspace or dsink, or a dsink without a sink; MIMO_EWORKSPACE when the workspace is
 * too small.
 */
int mimo_attn_prefill_backward(mimo_dtype dt, int B, int L, int Hq, int Hkv, int d_qk, int d_v,
                               const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* d_o, int window, const float* sink,
                               const int32_t* kv_head_of_q, float scale, void* dq, void* dk,
                               void* dv, float* dsink, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Workspace bytes of mimo_attn_prefill_backward (0 for sizes < 1). */
size_t mimo_attn_prefill_backward_workspace_size(int B, int L, int Hq);

/* Thread-local description of the last non-zero return on this thread ("" if none). */
const char* mimo_attn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int mimo_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MIMO_ATTN_H */

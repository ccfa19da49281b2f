/*
 * grok_attn.h -- C ABI of the MI355X (gfx950) Grok-1 attention sub-layer core.
 *
 * Sources: the Grok-1 walkthrough pages
 *   [ch4] "model.py close reading, part 1: RMSNorm, RoPE, GQA Attention"
 *   [ch6] "model.py close reading, part 3: block assembly and sharding"
 *   [ch3] "Configuration and hyperparameters"
 *   [ch2] "Overall architecture"
 * Section numbers below are the pages' own.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers (HIP global memory), row-major and
 *   contiguous, owned by the caller. The library allocates nothing, keeps no
 *   state between calls (one exception: the per-GPU scratch array of
 *   grok_attn_decode_append_noalloc), and never synchronises: work is
 *   enqueued on `stream` (NULL = the default stream) and the call returns.
 * - Return value: GROK_OK (0) or a negative GROK_E* code. Arguments are
 *   validated on the host before anything is enqueued; on an error nothing is
 *   enqueued and grok_last_error() (thread-local) describes the problem.
 *   GROK_EHIP means a HIP launch failed after validation.
 * - dtype codes: GROK_BF16 (bfloat16 raw bits, 2 bytes) or GROK_F32.
 * - Head layout: query head h uses KV head h / (Hq/Hkv) ([ch4] §4.5.2: the
 *   queries are viewed as [B, T, Hkv, Hq/Hkv, D]); the attention output is
 *   [B, T, Hq*D] with head h in columns h*D .. h*D+D-1 ([ch4] §4.5.4).
 * - Device-resident integer arguments (step, kv_len) cannot be checked on the
 *   host. Kernels check them; a bad value skips that sequence's work and, if
 *   the optional device word `status` is non-NULL, stores GROK_ERANGE into it
 *   (the library never clears `status`; the caller zeroes it).
 */
#ifndef GROK_ATTN_H
#define GROK_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GROK_API __attribute__((visibility("default")))

#define GROK_ABI_VERSION 1

#define GROK_OK 0
#define GROK_EHIP (-5)     /* a HIP call failed (see grok_last_error) */
#define GROK_ENOMEM (-12)  /* caller-provided workspace too small */
#define GROK_EINVAL (-22)  /* bad shape, null pointer, unsupported dtype/size */
#define GROK_ERANGE (-34)  /* a cache position is outside [0, Tmax) */

#define GROK_BF16 0
#define GROK_F32 1

GROK_API int grok_abi_version(void);
GROK_API const char *grok_status_string(int status);
/* Description of the last error raised on the calling thread ("" if none). */
GROK_API const char *grok_last_error(void);

/*
 * RMSNorm over the last axis ([ch4] §4.2): for each of `rows` rows of `d`
 *   y = gamma * x / sqrt(mean(x^2) + eps)
 * computed in fp32 and rounded to `dtype`. No mean subtraction, no bias.
 *   x, y      [rows, d] of `dtype`; y may alias x.
 *   gamma     [d] fp32, or NULL for the unit scale (hk_rms_norm without scale).
 *   residual  [rows, d] of `dtype` or NULL. When given, the normalised row is
 *             rounded to `dtype` and then added to it, rounded again:
 *             y = residual + norm(x) -- the post-norm residual update of the
 *             sandwich norm ([ch6] §6.3.1). y may alias residual.
 * Errors: EINVAL if a required pointer is NULL, rows < 0, d < 1, eps < 0 or
 * dtype unknown. rows == 0 is a no-op.
 */
GROK_API int grok_rmsnorm(const void *x, const float *gamma, const void *residual, void *y,
                 int64_t rows, int d, float eps, int dtype, hipStream_t stream);

/*
 * int8-weight Linear ([ch4] §4.1, §4.1.1): y = x @ (w * scales), no bias.
 *   x       [M, K] bf16 activations.
 *   w       [K, N] int8 weights (input axis first, as the pages store them).
 *   scales  [N] fp32, one per output channel (broadcast along K).
 *   y       [M, N] bf16, must not overlap x.
 * The int8 values are used exactly (|w| <= 127 is exact in bf16), products are
 * accumulated in fp32, and the channel scale is applied to the fp32 sum before
 * rounding to bf16.
 * Errors: EINVAL for NULL pointers, M < 0, K < 1, N < 1, K or N not a
 * multiple of 8, misaligned pointers, or y overlapping x. M == 0 is a no-op.
 */
GROK_API int grok_linear_int8(const void *x, const int8_t *w, const float *scales, void *y,
                     int64_t M, int K, int N, hipStream_t stream);

/*
 * Packed form of an int8 weight matrix for grok_linear_int8_gemv (a pure
 * permutation of its bytes, padded with zeros): 1024-byte tiles of 64 rows x
 * 16 columns, KP = ceil(K/64) tiles per 16-column block, block j's tiles
 * contiguous and in K order; byte 16*l + 8*h + e (l < 64, h < 2, e < 8) of
 * tile (j, i), at offset (j*KP + i)*1024, holds
 *   w[64*i + 32*h + 8*(l/16) + e][16*j + l%16]   (0 past K or N).
 * grok_linear_int8_packed_bytes returns ceil(K/64) * ceil(N/16) * 1024, or 0
 * on bad sizes. grok_linear_int8_pack writes that many bytes.
 *   w         [K, N] int8 (device); w_packed device, 16-byte aligned, must not
 *             overlap w.
 * Errors: EINVAL for NULL pointers, K or N not a positive multiple of 8, a
 * misaligned w_packed, or overlapping buffers.
 */
GROK_API size_t grok_linear_int8_packed_bytes(int K, int N);
GROK_API int grok_linear_int8_pack(const int8_t *w, int8_t *w_packed, int K, int N,
                                   hipStream_t stream);

/*
 * int8-weight Linear for a few rows, as in decoding where every sequence
 * contributes one row ([ch4] §4.1, §4.1.1; the query, key and value
 * projections of one token, §4.5.1, share their input): for p < n_mats,
 *   y[p] = x @ (w[p] * scales[p])
 * with the numerics of grok_linear_int8 (exact int8, fp32 sums, channel scale
 * applied to the fp32 sum, bf16 result). The weights are read once per 32
 * rows of x, in the packed form above, so the call runs at the speed of HBM
 * for small M; for M in the hundreds or more, grok_linear_int8 is faster.
 *   x          [M, K] bf16 (device), 16-byte aligned.
 *   w_packed, scales, y, N   host arrays of n_mats (1..3) entries of device
 *              pointers: w_packed[p] the packed form of a [K, N[p]] int8
 *              matrix (16-byte aligned), scales[p] [N[p]] fp32, y[p]
 *              [M, N[p]] bf16 (must not overlap x or each other).
 * Errors: EINVAL for NULL pointers, n_mats outside [1, 3], M < 0, K or N[p]
 * not a positive multiple of 8, misaligned pointers, or a y[p] overlapping x.
 * M == 0 is a no-op.
 */
GROK_API int grok_linear_int8_gemv(const void *x, int n_mats, const int8_t *const *w_packed,
                                   const float *const *scales, void *const *y, const int *N,
                                   int64_t M, int K, hipStream_t stream);

/*
 * Front half of the attention sub-layer for one new token per sequence
 * ([ch6] §6.3.1 pre-norm, [ch4] §4.5.1 projections, §4.3.1 RoPE, §4.4
 * RoPE-then-cache), in one launch: with p = step[b],
 *   n        = prenorm ? rmsnorm(x; gamma, eps) rounded to bf16 : x
 *   q_out[b] = rope(bf16(n[b] @ Wq * sq), p)                       (bf16)
 *   k_cache[b, p] = rope(bf16(n[b] @ Wk * sk), p),  v_cache[b, p] = bf16(n[b] @ Wv * sv)
 *   new_step[b] = p + 1                                 (if new_step is not NULL)
 * with the same arithmetic (and, for a given n, the same bits) as
 * grok_linear_int8_gemv followed by grok_kv_append(q_inout = q_out); the
 * fused norm sums squares in another order than grok_rmsnorm, so n may
 * differ from it by one bf16 rounding.
 *   x        [B, d] bf16; gamma [d] fp32 or NULL (unit scale), used with prenorm.
 *   w*_packed  grok_linear_int8_pack of Wq [d, Hq*128], Wk, Wv [d, Hkv*128];
 *   s*       their fp32 channel scales; q_out [B, Hq*128] bf16 (must not overlap x).
 *   caches   [B, Tmax, Hkv, 128] bf16; step [B] int32 device, new_step [B]
 *            int32 device or NULL (must not alias step); status as for
 *            grok_kv_append: a sequence with step[b] outside [0, Tmax) gets
 *            no cache write, its unrotated q row, new_step[b] = step[b], and
 *            GROK_ERANGE is stored to *status.
 * Errors: EINVAL for NULL pointers, sizes < 1, d not a multiple of 8, D !=
 * 128, Hq % Hkv != 0, bad rope_base or eps, misaligned pointers, new_step ==
 * step, q_out overlapping x, or prenorm with B above what fits on chip (4
 * rows of width <= 8192).
 */
GROK_API int grok_decode_qkv(const void *x, const float *gamma, float eps, int prenorm,
                             const int8_t *wq_packed, const float *sq, const int8_t *wk_packed,
                             const float *sk, const int8_t *wv_packed, const float *sv,
                             void *q_out, void *k_cache, void *v_cache, const int32_t *step,
                             int32_t *new_step, int32_t *status, int B, int d, int Tmax, int Hq,
                             int Hkv, int D, float rope_base, hipStream_t stream);

/*
 * Back half of the attention sub-layer for one token per sequence ([ch4]
 * §4.1 int8 Linear, §4.5.4 output projection; [ch6] §6.3.1 sandwich norm
 * and residual): with o = bf16(attn[b] @ (Wo * so)),
 *   y[b] = bf16(residual[b] + bf16(gamma * o * rsqrt(mean(o^2) + eps)))
 * with the roundings (and, for a given o, the arithmetic) of
 * grok_linear_int8_gemv followed by grok_rmsnorm with the residual; the sum
 * of squares is taken in another order, so y may differ from those calls by
 * one bf16 rounding. Up to 4 rows (of d_in <= 8192) run as one launch: the
 * workgroups, 16 output channels each, meet through the workspace and the
 * last one to finish normalises and adds the residual. More rows run the
 * projection and the norm as two launches.
 *   attn     [B, d_in] bf16;  wo_packed  grok_linear_int8_pack of Wo [d_in, d_out];
 *   so       [d_out] fp32;    gamma [d_out] fp32 or NULL (unit scale);
 *   residual, y  [B, d_out] bf16 (y may alias residual, not attn).
 *   workspace    device, grok_decode_out_workspace_bytes(B, d_in, d_out)
 *                bytes, 16-byte aligned, ZEROED before its first use: it
 *                holds an arrival counter that every call leaves at zero.
 *                Calls that overlap in time must not share a workspace.
 * Errors: EINVAL for NULL pointers, B < 1, d_in or d_out not a positive
 * multiple of 8, a bad eps, misaligned pointers (16 bytes; so and gamma 4),
 * or overlaps with the workspace or of y with attn; ENOMEM if ws_bytes is too
 * small.
 */
GROK_API size_t grok_decode_out_workspace_bytes(int B, int d_in, int d_out);
GROK_API int grok_decode_out(const void *attn, const int8_t *wo_packed, const float *so,
                             const float *gamma, float eps, const void *residual, void *y,
                             void *workspace, size_t ws_bytes, int B, int d_in, int d_out,
                             hipStream_t stream);

/*
 * Rotary embedding, in place ([ch4] §4.3, §4.3.1): for x [B, T, H, D] and the
 * position p = offset[b] + t,
 *   inv_freq[i] = base^(-2i/D) (fp32),  theta_i = fp32(p * inv_freq[i]),
 *   x'_i       = x_i cos theta_i - x_{i+D/2} sin theta_i
 *   x'_{i+D/2} = x_i sin theta_i + x_{i+D/2} cos theta_i     (i < D/2)
 * i.e. x*cos + rotate_half(x)*sin with GPT-NeoX half-split pairing. Computed
 * in fp32, rounded to `dtype`.
 *   offset  [B] int32 device array, or NULL for offset 0.
 * Errors: EINVAL for NULL x, negative sizes, D odd or D > 512, base <= 0, or
 * unknown dtype. Empty tensors are a no-op.
 */
GROK_API int grok_rope(void *x, int B, int T, int H, int D, const int32_t *offset, float base,
              int dtype, hipStream_t stream);

/*
 * KV-cache append with RoPE applied first ([ch4] §4.4): for every sequence b
 * and new token t, position p = step[b] + t:
 *   k_cache[b, p] = rope(k_new[b, t], p)   (k_new itself is not modified)
 *   v_cache[b, p] = v_new[b, t]            (bit copy)
 *   q_inout[b, t] = rope(q_inout[b, t], p) (if q_inout is not NULL)
 *   new_step[b]   = step[b] + T            (if new_step is not NULL)
 * With rope_base <= 0 no rotation is applied (k is copied bit for bit).
 * No other cache slot is touched. All tensors bf16:
 *   caches [B, Tmax, Hkv, D]; k_new, v_new [B, T, Hkv, D]; q_inout [B, T, Hq, D].
 *   step   [B] int32 device array; new_step must not alias step (the
 *          workgroups of a sequence read step[b] while its new_step[b] is
 *          written).
 * A sequence with step[b] < 0 or step[b] + T > Tmax is skipped entirely (no
 * write, new_step[b] = step[b]) and GROK_ERANGE is stored to *status.
 * Errors: EINVAL for NULL required pointers, sizes < 1 (B, T, Tmax, Hkv, D),
 * Hq not a multiple of Hkv (when q_inout is given), D not a multiple of 16 or
 * D > 512, T > Tmax, a pointer not 16-byte aligned, or new_step == step.
 */
GROK_API int grok_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                   void *q_inout, const int32_t *step, int32_t *new_step, int32_t *status,
                   int B, int T, int Tmax, int Hq, int Hkv, int D, float rope_base,
                   hipStream_t stream);

/*
 * Causal grouped-query attention over a prompt ([ch4] §4.5.2-§4.5.4,
 * [ch6] §6.4.2). For query position i of sequence b and head h (KV head g):
 *   z_j  = attn_mult * <q[b,i,h], k[b,j,g]>                       (fp32)
 *   c_j  = softcap * tanh(z_j / softcap)
 *   l_j  = c_j if (j <= i and key_valid[b,j] != 0) else -1e30
 *   out[b,i,h*D:(h+1)*D] = sum_j softmax(l)_j * v[b,j,g]
 * Masked logits use the pages' finite -1e30 fill: a query that sees no valid
 * key averages all T value rows uniformly.
 *   q    [B, T, Hq, D]; k, v [B, kv_rows, Hkv, D] where kv_rows >= T is the
 *        per-sequence row stride (T for freshly projected K/V, Tmax when they
 *        are read in place from a cache); only rows 0..T-1 are read.
 *   key_valid [B, T] uint8 (1 = real token) or NULL (no padding).
 *   out  [B, T, Hq*D], same dtype as q/k/v.
 * dtype GROK_BF16: bf16 operands, fp32 logits/softmax/accumulation, bf16 out.
 * dtype GROK_F32: fp32 throughout.
 * Errors: EINVAL for NULL required pointers, sizes < 1, Hq % Hkv != 0,
 * kv_rows < T, D > 256 or D % 8 != 0, attn_mult not finite, softcap outside
 * (0, 40], unknown dtype, or (bf16 with D == 128) a pointer not 16-byte aligned.
 * The softcap bound comes from the kernels' softmax: every unmasked softcapped
 * logit lies in [-softcap, softcap], so exp(c - softcap) is used in place of
 * the max-subtracted exponent; for softcap <= 40 its smallest value,
 * exp(-2*softcap), stays a normal fp32/bf16 number.
 */
GROK_API int grok_attn_prefill(const void *q, const void *k, const void *v, int64_t kv_rows,
                      const uint8_t *key_valid, void *out, int B, int T, int Hq, int Hkv,
                      int D, float attn_mult, float softcap, int dtype, hipStream_t stream);

/*
 * Causal grouped-query attention of a chunk of T new tokens per sequence
 * after a cached prefix (continuation / chunked prefill; [ch4] §4.4, §4.5,
 * [ch6] §6.6.1). The pages' mask shapes do not cover this case; the causal
 * rule is applied on absolute positions: query row t of sequence b sits at
 * position p = offset[b] + t and attends cache slots [0, p]:
 *   out[b,t,h*D:(h+1)*D] = sum_{j <= p} softmax_j(softcap * tanh(attn_mult *
 *                           <q[b,t,h], k_cache[b,j,g]> / softcap)) * v_cache[b,j,g]
 *   q      [B, T, Hq, 128] bf16, already rotated at its positions;
 *   caches [B, Tmax, Hkv, 128] bf16 holding slots [0, offset[b] + T) (the
 *          chunk's own keys and values included, e.g. written by
 *          grok_kv_append with step = offset); only those slots are read;
 *   offset [B] int32 device; out [B, T, Hq*128] bf16.
 * A sequence with offset[b] < 0 or offset[b] + T > Tmax gets all-zero output
 * rows and GROK_ERANGE is stored to *status (if not NULL).
 * Errors: EINVAL for NULL pointers, sizes < 1, T > Tmax, Hq % Hkv != 0,
 * D != 128, bad attn_mult/softcap (as for prefill), or a pointer not 16-byte
 * aligned.
 */
GROK_API int grok_attn_prefill_chunk(const void *q, const void *k_cache, const void *v_cache,
                                     const int32_t *offset, void *out, int32_t *status, int B,
                                     int T, int Tmax, int Hq, int Hkv, int D, float attn_mult,
                                     float softcap, hipStream_t stream);

/*
 * grok_attn_prefill with the rotation of q folded in ([ch4] §4.3.1 RoPE,
 * §4.5.2-§4.5.4 attention): q arrives unrotated and every query row t is
 * rotated at position t while it is loaded, with the numerics (and the bits)
 * of grok_rope(q) followed by grok_attn_prefill; q itself is not modified.
 * k must already be rotated (grok_rope, or the cache written by
 * grok_kv_append / grok_prefill_qkv); mask, layout and the fully-masked-row
 * rule as for grok_attn_prefill. bf16 and D = 128 only.
 *   workspace  device, grok_attn_prefill_rope_workspace_bytes(T, 128) bytes
 *              (the cos/sin table of positions 0..T-1, rebuilt by each call;
 *              one launch before the attention kernel).
 * Errors: EINVAL as for grok_attn_prefill, D != 128, a bad rope_base, or out
 * or the workspace overlapping q (or each other); ENOMEM if ws_bytes is too
 * small.
 */
GROK_API size_t grok_attn_prefill_rope_workspace_bytes(int T, int D);
GROK_API int grok_attn_prefill_rope(const void *q, const void *k, const void *v, int64_t kv_rows,
                                    const uint8_t *key_valid, void *out, void *workspace,
                                    size_t ws_bytes, int B, int T, int Hq, int Hkv, int D,
                                    float attn_mult, float softcap, float rope_base,
                                    hipStream_t stream);

/*
 * Single-token decode attention against a KV cache ([ch4] §4.4, §4.5; the
 * causal mask of one query is all-ones and the memory mask keeps slots
 * j < kv_len[b]):
 *   out[b, 0, h*D:(h+1)*D] = sum_{j < kv_len[b]} softmax_j(softcap(attn_mult *
 *                             <q[b,0,h], k_cache[b,j,g]>)) * v_cache[b,j,g]
 * Slots j >= kv_len[b] never affect the output, whatever they hold (NaN and
 * Inf included). When the grid is small enough to be resident at once (at
 * most 768 workgroups: B*Hkv rounded up to a multiple of 8, times
 * ceil(Tmax/128)), the kernel may read them: it loads each 128-slot block
 * before its sequence's length arrives and discards what lies past it.
 *   q [B, 1, Hq, D]; caches [B, Tmax, Hkv, D]; kv_len [B] int32 device
 *   (= step + 1 after the new token was appended); out [B, 1, Hq*D]; bf16.
 *   workspace: device scratch of at least grok_attn_decode_workspace_bytes()
 *   bytes (per-split partial sums); its contents need no initialisation. Calls
 *   that overlap in time must not share a workspace.
 * A sequence with kv_len[b] outside [1, Tmax] gets an all-zero output row and
 * GROK_ERANGE is stored to *status.
 * Errors: EINVAL for NULL pointers, sizes < 1, Hq % Hkv != 0, Hq/Hkv > 16,
 * D != 128, bad attn_mult/softcap as for prefill; ENOMEM if ws_bytes is too
 * small.
 */
GROK_API int grok_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *kv_len, void *out, void *workspace, size_t ws_bytes,
                     int32_t *status, int B, int Tmax, int Hq, int Hkv, int D,
                     float attn_mult, float softcap, hipStream_t stream);

/*
 * One decode step of the attention core in one call ([ch4] §4.4 RoPE before
 * the cache write, §4.5 attention): for each sequence b with p = step[b],
 *   q_r = rope(q[b, 0], p),  k_cache[b, p] = rope(k_new[b, 0], p),
 *   v_cache[b, p] = v_new[b, 0],  out[b, 0] = attention of q_r over slots [0, p]
 * with the numerics (and the bits) of grok_kv_append followed by
 * grok_attn_decode with kv_len = step + 1. q is not modified; the rotated q
 * goes to q_out if it is not NULL. new_step[b] = p + 1 if new_step is not NULL.
 *   q [B, 1, Hq, 128]; k_new, v_new [B, 1, Hkv, 128]; caches [B, Tmax, Hkv, 128];
 *   step [B] int32 device (must not alias new_step); out [B, 1, Hq*128]; bf16;
 *   workspace as for grok_attn_decode (grok_attn_decode_workspace_bytes).
 * A sequence with step[b] outside [0, Tmax) gets no cache write, an all-zero
 * output row, new_step[b] = step[b], and GROK_ERANGE is stored to *status.
 * Errors: EINVAL for NULL pointers, sizes < 1, Hq % Hkv != 0, Hq/Hkv > 16,
 * D != 128, bad attn_mult/softcap (as for prefill) or rope_base, a misaligned
 * pointer (16 bytes), new_step == step, or q_out overlapping q (every split of
 * a sequence reads q while the first one writes q_out); ENOMEM if ws_bytes
 * is too small.
 */
GROK_API int grok_attn_decode_append(const void *q, const void *k_new, const void *v_new,
                                     void *k_cache, void *v_cache, const int32_t *step,
                                     int32_t *new_step, void *q_out, void *out, void *workspace,
                                     size_t ws_bytes, int32_t *status, int B, int Tmax, int Hq,
                                     int Hkv, int D, float attn_mult, float softcap,
                                     float rope_base, hipStream_t stream);

/*
 * grok_attn_decode_append without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * that must not call hipMalloc, harnesses that forbid it. Same arguments,
 * kernels, results (bit for bit) and errors as grok_attn_decode_append; the
 * split partial sums go to a device array inside the library instead, one
 * copy per GPU of grok_attn_decode_append_noalloc_max_bytes() (64 MiB) bytes,
 * held from the first call on that GPU until the process ends. Its address
 * is looked up on the first call on each GPU; no call allocates.
 * Limit: grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D) must not
 * exceed that maximum (at 48/8 heads: B * ceil(Tmax/128) <= 2709, e.g. 42
 * sequences of an 8192-slot cache), else ENOMEM and nothing is enqueued.
 * All calls on one GPU share the array and its contents persist between
 * calls (they need no initialisation): calls that may overlap in time on
 * one GPU (other streams, other host threads) race and must not be issued.
 */
GROK_API size_t grok_attn_decode_append_noalloc_max_bytes(void);
GROK_API int grok_attn_decode_append_noalloc(const void *q, const void *k_new, const void *v_new,
                                             void *k_cache, void *v_cache, const int32_t *step,
                                             int32_t *new_step, void *q_out, void *out,
                                             int32_t *status, int B, int Tmax, int Hq, int Hkv, int D,
                                             float attn_mult, float softcap, float rope_base,
                                             hipStream_t stream);

/* Workspace bytes grok_attn_decode needs for these sizes (0 on bad sizes). */
GROK_API size_t grok_attn_decode_workspace_bytes(int B, int Tmax, int Hq, int Hkv, int D);

/*
 * Front half of the attention sub-layer for T rows per sequence, in one launch
 * ([ch4] §4.1 int8 Linear, §4.5.1 projections, §4.3.1 RoPE, §4.4 RoPE before
 * the cache write): for each sequence b with s = step[b] (0 if step is NULL)
 * and row t,
 *   q_out[b, t]          = rope(x[b, t] @ (Wq * sq), s + t)
 *   k_cache[b, s + t]    = rope(x[b, t] @ (Wk * sk), s + t)
 *   v_cache[b, s + t]    = x[b, t] @ (Wv * sv)
 * with the numerics (and the bits) of three grok_linear_int8 calls followed
 * by grok_kv_append: each projection is rounded to bf16, then rotated. With
 * step NULL and Tmax == T the "cache" is simply the [B, T, Hkv, 128] K and V
 * of a prompt. new_step[b] = s + T if new_step is not NULL.
 *   x [B, T, d] bf16 (the normalised rows); wq [d, Hq*128], wk, wv
 *   [d, Hkv*128] int8; sq, sk, sv fp32 channel scales; q_out [B, T, Hq, 128];
 *   caches [B, Tmax, Hkv, 128] bf16; step [B] int32 device or NULL;
 *   q_out must not overlap x;
 *   workspace: device, grok_prefill_qkv_workspace_bytes(Tmax, 128) bytes (a
 *   cos/sin table of every cache position, rebuilt by each call).
 * A sequence with s < 0 or s + T > Tmax gets no writes at all (q_out rows
 * untouched), new_step[b] = s, and GROK_ERANGE is stored to *status.
 * Errors: EINVAL for NULL pointers, sizes < 1, D != 128, T > Tmax, d not a
 * multiple of 8, a bad rope_base, new_step == step, q_out overlapping x, or a
 * misaligned pointer (16 bytes; the weights 8); ENOMEM if ws_bytes is too
 * small.
 */
GROK_API size_t grok_prefill_qkv_workspace_bytes(int Tmax, int D);
GROK_API int grok_prefill_qkv(const void *x, const int8_t *wq, const float *sq, const int8_t *wk,
                              const float *sk, const int8_t *wv, const float *sv, void *q_out,
                              void *k_cache, void *v_cache, const int32_t *step, int32_t *new_step,
                              int32_t *status, void *workspace, size_t ws_bytes, int B, int T, int d,
                              int Tmax, int Hq, int Hkv, int D, float rope_base, hipStream_t stream);

/*
 * MoE FFN sub-layer: the FFN half of a decoder layer ([ch6] §6.3.1 sandwich
 * norm; [ch2] §2.2 data flow), for T token rows:
 *   n     = rmsnorm(x)                          (unit scale, bf16)
 *   p     = softmax(n @ w_router)               (fp32 logits and softmax, [ch3] §3.5)
 *   idx   = the k most probable experts of each row (equal probabilities:
 *           lower expert index first); gates = their probabilities, not
 *           renormalised ([ch2] §2.5.1)
 *   h_e   = bf16(gelu(bf16(n Wg_e)) * bf16(n Wv_e))   (tanh-form GELU, [ch6] §6.2)
 *   mix   = bf16(sum over the k chosen e of gate * bf16(h_e W1_e))  (fp32 sum)
 *   out   = bf16(x + bf16(rmsnorm(mix)))
 * Every row goes to its k experts (no capacity limit, nothing dropped). The
 * int8 Linears have the numerics of grok_linear_int8 (exact int8, fp32 sums,
 * per-channel scale on the fp32 sum).
 *
 * grok_moe_interleave writes the up-projection weights of one expert in the
 * form grok_moe_ffn reads: gate and value columns side by side in blocks of
 * four,
 *   wgv[r][8q + j] = wg[r][4q + j],  wgv[r][8q + 4 + j] = wv[r][4q + j]  (j < 4)
 * and the same for the scales (sgv [2F]).
 *   wg, wv [d, F] int8 (4-byte aligned); sg, sv [F] fp32 (16-byte aligned);
 *   wgv [d, 2F] int8 (8-byte aligned); sgv [2F] fp32 (16-byte aligned).
 *
 * grok_moe_route: the router alone, on already normalised rows.
 *   n [T, d] bf16 (16-byte aligned); w_router [d, E] fp32;
 *   idx [T, k] int32 and gates [T, k] fp32 (outputs).
 *
 * grok_moe_ffn: the whole sub-layer.
 *   x [T, d] bf16; w_router [d, E] fp32 (device);
 *   wgv, sgv, w1, s1: host arrays of E device pointers: wgv[e] [d, 2F] int8 and
 *     sgv[e] [2F] fp32 (grok_moe_interleave's output), w1[e] [F, d] int8,
 *     s1[e] [d] fp32;
 *   idx, gates: [T, k] int32 / fp32 device outputs, or NULL (then kept in
 *     the workspace only);
 *   workspace: device, 16-byte aligned, grok_moe_workspace_bytes(T, d, F, E, k)
 *     bytes (normalised rows, routing plan, [T*k, F] and [T*k, d] bf16
 *     intermediates); out [T, d] bf16, must not overlap x.
 * Limits: 1 <= k <= E <= 8, k <= 4; d and F multiples of 8; d <= 8192;
 * T*d*2 < 2^32. T == 0 is a no-op.
 * Errors: EINVAL for NULL pointers, sizes outside the limits, a bad eps or a
 * misaligned pointer (x, out, workspace, sgv[e], s1[e]: 16 bytes; wgv[e],
 * w1[e]: 8; w_router, idx, gates: 4); ENOMEM if ws_bytes is too small.
 */
GROK_API size_t grok_moe_workspace_bytes(int64_t T, int d, int F, int E, int k);
GROK_API int grok_moe_interleave(const int8_t *wg, const float *sg, const int8_t *wv, const float *sv,
                                 int8_t *wgv, float *sgv, int d, int F, hipStream_t stream);
GROK_API int grok_moe_route(const void *n, const float *w_router, int32_t *idx, float *gates,
                            int64_t T, int d, int E, int k, hipStream_t stream);
GROK_API int grok_moe_ffn(const void *x, const float *w_router, int E, int k,
                          const int8_t *const *wgv, const float *const *sgv,
                          const int8_t *const *w1, const float *const *s1, int64_t T, int d, int F,
                          float eps, int32_t *idx, float *gates, void *workspace, size_t ws_bytes,
                          void *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GROK_ATTN_H */

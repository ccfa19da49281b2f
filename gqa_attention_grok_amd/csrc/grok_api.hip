// C ABI entry points: host-side validation, then launch. See include/grok_attn.h
// for the contract of every function. Validation happens before any HIP call,
// so every error path can be exercised on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return GROK_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(GROK_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// True when the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool bad_softmax_params(float mult, float cap) {
  return !isfinite(mult) || !(cap > 0.f) || cap > 40.f;
}

}  // namespace

extern "C" {

int grok_abi_version(void) { return GROK_ABI_VERSION; }

const char *grok_status_string(int status) {
  switch (status) {
    case GROK_OK: return "ok";
    case GROK_EHIP: return "HIP error";
    case GROK_ENOMEM: return "workspace too small";
    case GROK_EINVAL: return "invalid argument";
    case GROK_ERANGE: return "cache position out of range";
    default: return "unknown status";
  }
}

const char *grok_last_error(void) { return g_err; }

int grok_rmsnorm(const void *x, const float *gamma, const void *residual, void *y, int64_t rows,
                 int d, float eps, int dtype, hipStream_t stream) {
  if (dtype != GROK_BF16 && dtype != GROK_F32) return fail(GROK_EINVAL, "rmsnorm: unknown dtype %d", dtype);
  if (rows < 0 || d < 1) return fail(GROK_EINVAL, "rmsnorm: bad shape rows=%lld d=%d", (long long)rows, d);
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(GROK_EINVAL, "rmsnorm: bad eps");
  if (rows == 0) return ok();
  if (!x || !y) return fail(GROK_EINVAL, "rmsnorm: null x or y");
  return hip_status(grok::launch_rmsnorm(x, gamma, residual, y, rows, d, eps, dtype, stream), "rmsnorm");
}

int grok_linear_int8(const void *x, const int8_t *w, const float *scales, void *y, int64_t M,
                     int K, int N, hipStream_t stream) {
  if (M < 0 || K < 1 || N < 1) return fail(GROK_EINVAL, "linear_int8: bad shape M=%lld K=%d N=%d", (long long)M, K, N);
  if (K % 8 || N % 8) return fail(GROK_EINVAL, "linear_int8: K and N must be multiples of 8 (K=%d N=%d)", K, N);
  if (M == 0) return ok();
  if ((M + 127) / 128 > 65535) return fail(GROK_EINVAL, "linear_int8: M=%lld too large", (long long)M);
  if (!x || !w || !scales || !y) return fail(GROK_EINVAL, "linear_int8: null pointer");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(scales)) % 16 ||
      (reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(y)) % 8)
    return fail(GROK_EINVAL, "linear_int8: misaligned pointer");
  if (overlaps(x, static_cast<size_t>(M) * K * 2, y, static_cast<size_t>(M) * N * 2))
    return fail(GROK_EINVAL, "linear_int8: y overlaps x");
  return hip_status(grok::launch_linear_int8(x, w, scales, y, M, K, N, stream), "linear_int8");
}

size_t grok_linear_int8_packed_bytes(int K, int N) {
  if (K < 1 || N < 1 || K % 8 || N % 8) return 0;
  return grok::gemv_packed_bytes(K, N);
}

int grok_linear_int8_pack(const int8_t *w, int8_t *w_packed, int K, int N, hipStream_t stream) {
  if (K < 1 || N < 1 || K % 8 || N % 8)
    return fail(GROK_EINVAL, "linear_int8_pack: K=%d and N=%d must be positive multiples of 8", K, N);
  if (!w || !w_packed) return fail(GROK_EINVAL, "linear_int8_pack: null pointer");
  if (reinterpret_cast<uintptr_t>(w_packed) % 16) return fail(GROK_EINVAL, "linear_int8_pack: misaligned w_packed");
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(w_packed);
  const size_t na = static_cast<size_t>(K) * N, nb = grok::gemv_packed_bytes(K, N);
  if (a < b + nb && b < a + na) return fail(GROK_EINVAL, "linear_int8_pack: w and w_packed overlap");
  return hip_status(grok::launch_linear_int8_pack(w, w_packed, K, N, stream), "linear_int8_pack");
}

int grok_linear_int8_gemv(const void *x, int n_mats, const int8_t *const *w_packed,
                          const float *const *scales, void *const *y, const int *N, int64_t M,
                          int K, hipStream_t stream) {
  if (n_mats < 1 || n_mats > 3) return fail(GROK_EINVAL, "linear_int8_gemv: n_mats=%d outside [1, 3]", n_mats);
  if (!N) return fail(GROK_EINVAL, "linear_int8_gemv: null N");
  if (M < 0 || K < 1 || K % 8)
    return fail(GROK_EINVAL, "linear_int8_gemv: bad shape M=%lld K=%d (K a positive multiple of 8)", (long long)M, K);
  int64_t blocks = 0;
  for (int p = 0; p < n_mats; ++p) {
    if (N[p] < 1 || N[p] % 8)
      return fail(GROK_EINVAL, "linear_int8_gemv: N[%d]=%d must be a positive multiple of 8", p, N[p]);
    blocks += (N[p] + 31) / 32;
  }
  if (blocks > 0x7fffffff) return fail(GROK_EINVAL, "linear_int8_gemv: too many output channels");
  if (M == 0) return ok();
  if (!x || !w_packed || !scales || !y) return fail(GROK_EINVAL, "linear_int8_gemv: null pointer");
  uintptr_t a16 = reinterpret_cast<uintptr_t>(x), a4 = 0, a2 = 0;
  for (int p = 0; p < n_mats; ++p) {
    if (!w_packed[p] || !scales[p] || !y[p]) return fail(GROK_EINVAL, "linear_int8_gemv: null pointer in matrix %d", p);
    a16 |= reinterpret_cast<uintptr_t>(w_packed[p]);
    a4 |= reinterpret_cast<uintptr_t>(scales[p]);
    a2 |= reinterpret_cast<uintptr_t>(y[p]);
  }
  if (a16 % 16 || a4 % 4 || a2 % 2) return fail(GROK_EINVAL, "linear_int8_gemv: misaligned pointer");
  for (int p = 0; p < n_mats; ++p)
    if (overlaps(x, static_cast<size_t>(M) * K * 2, y[p], static_cast<size_t>(M) * N[p] * 2))
      return fail(GROK_EINVAL, "linear_int8_gemv: y[%d] overlaps x", p);
  return hip_status(grok::launch_linear_int8_gemv(x, n_mats, w_packed, scales, y, N, M, K, stream),
                    "linear_int8_gemv");
}

int grok_decode_qkv(const void *x, const float *gamma, float eps, int prenorm,
                    const int8_t *wq_packed, const float *sq, const int8_t *wk_packed,
                    const float *sk, const int8_t *wv_packed, const float *sv, void *q_out,
                    void *k_cache, void *v_cache, const int32_t *step, int32_t *new_step,
                    int32_t *status, int B, int d, int Tmax, int Hq, int Hkv, int D,
                    float rope_base, hipStream_t stream) {
  if (B < 1 || d < 8 || d % 8 || Tmax < 1 || Hq < 1 || Hkv < 1)
    return fail(GROK_EINVAL, "decode_qkv: bad shape B=%d d=%d Tmax=%d Hq=%d Hkv=%d", B, d, Tmax, Hq, Hkv);
  if (D != 128) return fail(GROK_EINVAL, "decode_qkv: head size must be 128 (D=%d)", D);
  if (Hq % Hkv) return fail(GROK_EINVAL, "decode_qkv: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (static_cast<int64_t>(Hq) * D > (1 << 24)) return fail(GROK_EINVAL, "decode_qkv: too many heads");
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return fail(GROK_EINVAL, "decode_qkv: bad rope_base");
  if (prenorm && (!(eps >= 0.f) || !isfinite(eps))) return fail(GROK_EINVAL, "decode_qkv: bad eps");
  if (prenorm && B > grok::decode_qkv_max_prenorm_rows(d))
    return fail(GROK_EINVAL, "decode_qkv: the fused pre-norm takes at most %d rows of width %d (B=%d)",
                grok::decode_qkv_max_prenorm_rows(d), d, B);
  if (!x || !wq_packed || !sq || !wk_packed || !sk || !wv_packed || !sv || !q_out || !k_cache || !v_cache || !step)
    return fail(GROK_EINVAL, "decode_qkv: null pointer");
  if (new_step && new_step == step) return fail(GROK_EINVAL, "decode_qkv: new_step must not alias step");
  const uintptr_t a16 = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(wq_packed) |
                        reinterpret_cast<uintptr_t>(wk_packed) | reinterpret_cast<uintptr_t>(wv_packed);
  const uintptr_t a4 = reinterpret_cast<uintptr_t>(sq) | reinterpret_cast<uintptr_t>(sk) |
                       reinterpret_cast<uintptr_t>(sv) | reinterpret_cast<uintptr_t>(gamma);
  const uintptr_t a2 = reinterpret_cast<uintptr_t>(q_out) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache);
  if (a16 % 16 || a4 % 4 || a2 % 2) return fail(GROK_EINVAL, "decode_qkv: misaligned pointer");
  if (overlaps(x, static_cast<size_t>(B) * d * 2, q_out, static_cast<size_t>(B) * Hq * D * 2))
    return fail(GROK_EINVAL, "decode_qkv: q_out overlaps x");
  grok::RopeFreqs f;
  grok::rope_build_freqs(D, rope_base, &f);
  const int8_t *w[3] = {wq_packed, wk_packed, wv_packed};
  const float *sc[3] = {sq, sk, sv};
  return hip_status(grok::launch_decode_qkv(x, gamma, eps, prenorm != 0, w, sc, q_out, k_cache, v_cache,
                                            step, new_step, status, B, d, Tmax, Hq, Hkv, f, stream),
                    "decode_qkv");
}

size_t grok_decode_out_workspace_bytes(int B, int d_in, int d_out) {
  if (B < 1 || d_in < 8 || d_in % 8 || d_out < 8 || d_out % 8) return 0;
  return grok::out_norm_workspace_bytes(B, d_out);
}

int grok_decode_out(const void *attn, const int8_t *wo_packed, const float *so, const float *gamma, float eps,
                    const void *residual, void *y, void *workspace, size_t ws_bytes, int B, int d_in, int d_out,
                    hipStream_t stream) {
  if (B < 1 || d_in < 8 || d_in % 8 || d_out < 8 || d_out % 8)
    return fail(GROK_EINVAL, "decode_out: bad shape B=%d d_in=%d d_out=%d (positive multiples of 8)", B, d_in, d_out);
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(GROK_EINVAL, "decode_out: bad eps");
  if (!attn || !wo_packed || !so || !residual || !y || !workspace) return fail(GROK_EINVAL, "decode_out: null pointer");
  const uintptr_t a16 = reinterpret_cast<uintptr_t>(attn) | reinterpret_cast<uintptr_t>(wo_packed) |
                        reinterpret_cast<uintptr_t>(residual) | reinterpret_cast<uintptr_t>(y) |
                        reinterpret_cast<uintptr_t>(workspace);
  const uintptr_t a4 = reinterpret_cast<uintptr_t>(so) | reinterpret_cast<uintptr_t>(gamma);
  if (a16 % 16 || a4 % 4) return fail(GROK_EINVAL, "decode_out: misaligned pointer");
  const size_t need = grok::out_norm_workspace_bytes(B, d_out);
  if (ws_bytes < need) return fail(GROK_ENOMEM, "decode_out: workspace %zu bytes < %zu needed", ws_bytes, need);
  const size_t ny = static_cast<size_t>(B) * d_out * 2;
  if (overlaps(y, ny, attn, static_cast<size_t>(B) * d_in * 2) || overlaps(y, ny, workspace, need) ||
      overlaps(attn, static_cast<size_t>(B) * d_in * 2, workspace, need) ||
      overlaps(residual, ny, workspace, need))
    return fail(GROK_EINVAL, "decode_out: y, attn or residual overlaps the workspace, or y overlaps attn");
  return hip_status(grok::launch_out_norm(attn, wo_packed, so, gamma, eps, residual, y, workspace, B, d_in, d_out,
                                          stream),
                    "decode_out");
}

int grok_rope(void *x, int B, int T, int H, int D, const int32_t *offset, float base, int dtype,
              hipStream_t stream) {
  if (dtype != GROK_BF16 && dtype != GROK_F32) return fail(GROK_EINVAL, "rope: unknown dtype %d", dtype);
  if (B < 0 || T < 0 || H < 0 || D < 2) return fail(GROK_EINVAL, "rope: bad shape");
  if (D % 2 || D > 512) return fail(GROK_EINVAL, "rope: head size must be even and <= 512 (D=%d)", D);
  if (!(base > 0.f) || !isfinite(base)) return fail(GROK_EINVAL, "rope: bad base");
  if (static_cast<int64_t>(B) * T * H == 0) return ok();
  if (!x) return fail(GROK_EINVAL, "rope: null x");
  grok::RopeFreqs f;
  grok::rope_build_freqs(D, base, &f);
  return hip_status(grok::launch_rope(x, B, T, H, D, offset, f, dtype, stream), "rope");
}

int grok_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                   void *q_inout, const int32_t *step, int32_t *new_step, int32_t *status, int B,
                   int T, int Tmax, int Hq, int Hkv, int D, float rope_base, hipStream_t stream) {
  if (B < 1 || T < 1 || Tmax < 1 || Hkv < 1 || D < 2) return fail(GROK_EINVAL, "kv_append: bad shape");
  if (T > Tmax) return fail(GROK_EINVAL, "kv_append: T=%d exceeds Tmax=%d", T, Tmax);
  if (D % 16 || D > 512) return fail(GROK_EINVAL, "kv_append: head size must be a multiple of 16, <= 512 (D=%d)", D);
  if (q_inout && (Hq < 1 || Hq % Hkv)) return fail(GROK_EINVAL, "kv_append: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (!k_cache || !v_cache || !k_new || !v_new || !step) return fail(GROK_EINVAL, "kv_append: null pointer");
  if (!isfinite(rope_base)) return fail(GROK_EINVAL, "kv_append: bad rope_base");
  if (new_step && new_step == step) return fail(GROK_EINVAL, "kv_append: new_step must not alias step");
  const uintptr_t al = reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
                       reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
                       reinterpret_cast<uintptr_t>(q_inout);
  if (al % 16) return fail(GROK_EINVAL, "kv_append: misaligned pointer");
  if (static_cast<int64_t>(B) * T > 0x7fffffff) return fail(GROK_EINVAL, "kv_append: too many tokens");
  grok::RopeFreqs f;
  const bool do_rope = rope_base > 0.f;
  grok::rope_build_freqs(D, do_rope ? rope_base : 1.f, &f);
  return hip_status(grok::launch_kv_append(k_cache, v_cache, k_new, v_new, q_inout, step, new_step,
                                           status, B, T, Tmax, Hq, Hkv, D, do_rope, f, stream),
                    "kv_append");
}

int grok_attn_prefill(const void *q, const void *k, const void *v, int64_t kv_rows,
                      const uint8_t *key_valid, void *out, int B, int T, int Hq, int Hkv, int D,
                      float attn_mult, float softcap, int dtype, hipStream_t stream) {
  if (dtype != GROK_BF16 && dtype != GROK_F32) return fail(GROK_EINVAL, "attn_prefill: unknown dtype %d", dtype);
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1) return fail(GROK_EINVAL, "attn_prefill: bad shape");
  if (Hq % Hkv) return fail(GROK_EINVAL, "attn_prefill: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (kv_rows < T) return fail(GROK_EINVAL, "attn_prefill: kv_rows=%lld < T=%d", (long long)kv_rows, T);
  if (D % 8 || D > 256) return fail(GROK_EINVAL, "attn_prefill: head size must be a multiple of 8, <= 256 (D=%d)", D);
  if (bad_softmax_params(attn_mult, softcap))
    return fail(GROK_EINVAL, "attn_prefill: attn_mult must be finite and softcap in (0, 40]");
  if (!q || !k || !v || !out) return fail(GROK_EINVAL, "attn_prefill: null pointer");
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if (grok::prefill_mfma_supported(kv_rows, Hq, Hkv, D, dtype)) {
    if (al % 16) return fail(GROK_EINVAL, "attn_prefill: misaligned pointer");
    return hip_status(grok::launch_prefill_mfma(q, k, v, kv_rows, key_valid, out, B, T, Hq, Hkv,
                                                attn_mult, softcap, stream),
                      "attn_prefill");
  }
  return hip_status(grok::launch_prefill_generic(q, k, v, kv_rows, key_valid, out, B, T, Hq, Hkv, D,
                                                 attn_mult, softcap, dtype, stream),
                    "attn_prefill");
}

size_t grok_attn_prefill_rope_workspace_bytes(int T, int D) {
  if (T < 1 || D != 128) return 0;
  return static_cast<size_t>(T) * 128 * sizeof(float);
}

int grok_attn_prefill_rope(const void *q, const void *k, const void *v, int64_t kv_rows, const uint8_t *key_valid,
                           void *out, void *workspace, size_t ws_bytes, int B, int T, int Hq, int Hkv, int D,
                           float attn_mult, float softcap, float rope_base, hipStream_t stream) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1) return fail(GROK_EINVAL, "attn_prefill_rope: bad shape");
  if (Hq % Hkv) return fail(GROK_EINVAL, "attn_prefill_rope: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (D != 128) return fail(GROK_EINVAL, "attn_prefill_rope: head size must be 128 (D=%d)", D);
  if (kv_rows < T) return fail(GROK_EINVAL, "attn_prefill_rope: kv_rows=%lld < T=%d", (long long)kv_rows, T);
  if (bad_softmax_params(attn_mult, softcap))
    return fail(GROK_EINVAL, "attn_prefill_rope: attn_mult must be finite and softcap in (0, 40]");
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return fail(GROK_EINVAL, "attn_prefill_rope: bad rope_base");
  if (!q || !k || !v || !out || !workspace) return fail(GROK_EINVAL, "attn_prefill_rope: null pointer");
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out) |
                       reinterpret_cast<uintptr_t>(workspace);
  if (al % 16) return fail(GROK_EINVAL, "attn_prefill_rope: misaligned pointer");
  const size_t need = static_cast<size_t>(T) * 128 * sizeof(float);
  if (ws_bytes < need) return fail(GROK_ENOMEM, "attn_prefill_rope: workspace %zu bytes < %zu needed", ws_bytes, need);
  const size_t nq = static_cast<size_t>(B) * T * Hq * D * 2;
  if (overlaps(out, nq, q, nq) || overlaps(workspace, need, q, nq) || overlaps(workspace, need, out, nq))
    return fail(GROK_EINVAL, "attn_prefill_rope: out or the workspace overlaps q, or the workspace overlaps out");
  grok::RopeFreqs f;
  grok::rope_build_freqs(D, rope_base, &f);
  float *tab = static_cast<float *>(workspace);
  hipError_t e = grok::launch_rope_table(tab, T, f, stream);
  if (e != hipSuccess) return hip_status(e, "attn_prefill_rope: table");
  return hip_status(grok::launch_prefill_mfma(q, k, v, kv_rows, key_valid, out, B, T, Hq, Hkv, attn_mult, softcap,
                                              stream, nullptr, nullptr, tab),
                    "attn_prefill_rope");
}

size_t grok_attn_decode_workspace_bytes(int B, int Tmax, int Hq, int Hkv, int D) {
  if (B < 1 || Tmax < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D != 128) return 0;
  return grok::decode_workspace_bytes(B, Tmax, Hq, Hkv);
}

int grok_attn_decode(const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *kv_len, void *out, void *workspace, size_t ws_bytes,
                     int32_t *status, int B, int Tmax, int Hq, int Hkv, int D, float attn_mult,
                     float softcap, hipStream_t stream) {
  if (B < 1 || Tmax < 1 || Hq < 1 || Hkv < 1) return fail(GROK_EINVAL, "attn_decode: bad shape");
  if (Hq % Hkv) return fail(GROK_EINVAL, "attn_decode: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (Hq / Hkv > 16) return fail(GROK_EINVAL, "attn_decode: at most 16 query heads per KV head");
  if (D != 128) return fail(GROK_EINVAL, "attn_decode: head size must be 128 (D=%d)", D);
  if (bad_softmax_params(attn_mult, softcap))
    return fail(GROK_EINVAL, "attn_decode: attn_mult must be finite and softcap in (0, 40]");
  if (!q || !k_cache || !v_cache || !kv_len || !out || !workspace)
    return fail(GROK_EINVAL, "attn_decode: null pointer");
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(workspace);
  if (al % 16) return fail(GROK_EINVAL, "attn_decode: misaligned pointer");
  const size_t need = grok::decode_workspace_bytes(B, Tmax, Hq, Hkv);
  if (ws_bytes < need)
    return fail(GROK_ENOMEM, "attn_decode: workspace %zu bytes < %zu needed", ws_bytes, need);
  if (static_cast<int64_t>(B) * Hq > 0x7fffffff || B > 65535) return fail(GROK_EINVAL, "attn_decode: batch too large");
  return hip_status(grok::launch_decode(q, k_cache, v_cache, kv_len, out, workspace, status, B, Tmax,
                                        Hq, Hkv, attn_mult, softcap, stream),
                    "attn_decode");
}

namespace {

// Validation shared by the two decode-append entry points; 0 when fine.
int decode_append_check(const char *who, const void *q, const void *k_new, const void *v_new, const void *k_cache,
                        const void *v_cache, const int32_t *step, const int32_t *new_step, const void *q_out,
                        const void *out, int B, int Tmax, int Hq, int Hkv, int D, float attn_mult, float softcap,
                        float rope_base) {
  if (B < 1 || Tmax < 1 || Hq < 1 || Hkv < 1) return fail(GROK_EINVAL, "%s: bad shape", who);
  if (Hq % Hkv) return fail(GROK_EINVAL, "%s: Hq=%d not a multiple of Hkv=%d", who, Hq, Hkv);
  if (Hq / Hkv > 16) return fail(GROK_EINVAL, "%s: at most 16 query heads per KV head", who);
  if (D != 128) return fail(GROK_EINVAL, "%s: head size must be 128 (D=%d)", who, D);
  if (bad_softmax_params(attn_mult, softcap))
    return fail(GROK_EINVAL, "%s: attn_mult must be finite and softcap in (0, 40]", who);
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return fail(GROK_EINVAL, "%s: bad rope_base", who);
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !step || !out) return fail(GROK_EINVAL, "%s: null pointer", who);
  if (new_step && new_step == step) return fail(GROK_EINVAL, "%s: new_step must not alias step", who);
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_new) |
                       reinterpret_cast<uintptr_t>(v_new) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out) |
                       reinterpret_cast<uintptr_t>(q_out);
  if (al % 16) return fail(GROK_EINVAL, "%s: misaligned pointer", who);
  if (overlaps(q, static_cast<size_t>(B) * Hq * D * 2, q_out, static_cast<size_t>(B) * Hq * D * 2))
    return fail(GROK_EINVAL, "%s: q_out overlaps q", who);
  if (static_cast<int64_t>(B) * Hq > 0x7fffffff || B > 65535) return fail(GROK_EINVAL, "%s: batch too large", who);
  return 0;
}

}  // namespace

int grok_attn_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache,
                            void *v_cache, const int32_t *step, int32_t *new_step, void *q_out,
                            void *out, void *workspace, size_t ws_bytes, int32_t *status, int B,
                            int Tmax, int Hq, int Hkv, int D, float attn_mult, float softcap,
                            float rope_base, hipStream_t stream) {
  if (int r = decode_append_check("attn_decode_append", q, k_new, v_new, k_cache, v_cache, step, new_step, q_out,
                                  out, B, Tmax, Hq, Hkv, D, attn_mult, softcap, rope_base))
    return r;
  if (!workspace) return fail(GROK_EINVAL, "attn_decode_append: null workspace");
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return fail(GROK_EINVAL, "attn_decode_append: misaligned pointer");
  const size_t need = grok::decode_workspace_bytes(B, Tmax, Hq, Hkv);
  if (ws_bytes < need)
    return fail(GROK_ENOMEM, "attn_decode_append: workspace %zu bytes < %zu needed", ws_bytes, need);
  grok::RopeFreqs f;
  grok::rope_build_freqs(D, rope_base, &f);
  return hip_status(grok::launch_decode_append(q, k_new, v_new, k_cache, v_cache, step, new_step, q_out, out,
                                               workspace, status, B, Tmax, Hq, Hkv, attn_mult, softcap, f,
                                               stream),
                    "attn_decode_append");
}

size_t grok_attn_decode_append_noalloc_max_bytes(void) { return grok::kDecodeScratchBytes; }

int grok_attn_decode_append_noalloc(const void *q, const void *k_new, const void *v_new, void *k_cache,
                                    void *v_cache, const int32_t *step, int32_t *new_step, void *q_out,
                                    void *out, int32_t *status, int B, int Tmax, int Hq, int Hkv, int D,
                                    float attn_mult, float softcap, float rope_base, hipStream_t stream) {
  if (int r = decode_append_check("attn_decode_append_noalloc", q, k_new, v_new, k_cache, v_cache, step, new_step,
                                  q_out, out, B, Tmax, Hq, Hkv, D, attn_mult, softcap, rope_base))
    return r;
  const size_t need = grok::decode_workspace_bytes(B, Tmax, Hq, Hkv);
  if (need > grok::kDecodeScratchBytes)
    return fail(GROK_ENOMEM, "attn_decode_append_noalloc: these sizes need %zu bytes of scratch, above the "
                "%zu-byte maximum (use grok_attn_decode_append with a workspace)", need, grok::kDecodeScratchBytes);
  void *ws = nullptr;
  hipError_t e = grok::decode_static_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "attn_decode_append_noalloc: scratch lookup");
  grok::RopeFreqs f;
  grok::rope_build_freqs(D, rope_base, &f);
  return hip_status(grok::launch_decode_append(q, k_new, v_new, k_cache, v_cache, step, new_step, q_out, out, ws,
                                               status, B, Tmax, Hq, Hkv, attn_mult, softcap, f, stream),
                    "attn_decode_append_noalloc");
}

int grok_attn_prefill_chunk(const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *offset, void *out, int32_t *status, int B, int T, int Tmax,
                            int Hq, int Hkv, int D, float attn_mult, float softcap, hipStream_t stream) {
  if (B < 1 || T < 1 || Tmax < 1 || Hq < 1 || Hkv < 1) return fail(GROK_EINVAL, "attn_prefill_chunk: bad shape");
  if (T > Tmax) return fail(GROK_EINVAL, "attn_prefill_chunk: T=%d exceeds Tmax=%d", T, Tmax);
  if (Hq % Hkv) return fail(GROK_EINVAL, "attn_prefill_chunk: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (D != 128) return fail(GROK_EINVAL, "attn_prefill_chunk: head size must be 128 (D=%d)", D);
  if (bad_softmax_params(attn_mult, softcap))
    return fail(GROK_EINVAL, "attn_prefill_chunk: attn_mult must be finite and softcap in (0, 40]");
  if (!q || !k_cache || !v_cache || !offset || !out) return fail(GROK_EINVAL, "attn_prefill_chunk: null pointer");
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out);
  if (al % 16) return fail(GROK_EINVAL, "attn_prefill_chunk: misaligned pointer");
  if (!grok::prefill_mfma_supported(Tmax, Hq, Hkv, D, GROK_BF16))
    return fail(GROK_EINVAL, "attn_prefill_chunk: unsupported sizes");
  return hip_status(grok::launch_prefill_mfma(q, k_cache, v_cache, Tmax, nullptr, out, B, T, Hq, Hkv, attn_mult,
                                              softcap, stream, offset, status),
                    "attn_prefill_chunk");
}

namespace {

// Shared shape checks of the MoE entry points; 0 when fine.
int moe_shape_error(const char *who, int64_t T, int d, int F, int E, int k) {
  if (T < 0 || d < 8 || d % 8 || F < 8 || F % 8)
    return fail(GROK_EINVAL, "%s: bad shape T=%lld d=%d F=%d (d, F positive multiples of 8)", who,
                (long long)T, d, F);
  if (E < 1 || E > grok::moe_max_experts())
    return fail(GROK_EINVAL, "%s: E=%d outside [1, %d]", who, E, grok::moe_max_experts());
  if (k < 1 || k > E || k > grok::moe_max_k())
    return fail(GROK_EINVAL, "%s: k=%d outside [1, min(E, %d)]", who, k, grok::moe_max_k());
  if (d > grok::moe_max_width()) return fail(GROK_EINVAL, "%s: d=%d above %d", who, d, grok::moe_max_width());
  // gathered rows are addressed with 32-bit byte offsets; entries are int32
  if (T * d * 2 >= (int64_t(1) << 32) || T * k > 0x7fffffff)
    return fail(GROK_EINVAL, "%s: T=%lld too large", who, (long long)T);
  if ((T * k + 255) / 256 + E > 65535 || static_cast<int64_t>(d) * F * 2 >= (int64_t(1) << 32))
    return fail(GROK_EINVAL, "%s: T=%lld or F=%d too large", who, (long long)T, F);
  return 0;
}

}  // namespace

size_t grok_moe_workspace_bytes(int64_t T, int d, int F, int E, int k) {
  if (T < 0 || d < 1 || F < 1 || E < 1 || k < 1) return 0;
  return grok::moe_workspace(T, d, F, E, k).total;
}

int grok_moe_interleave(const int8_t *wg, const float *sg, const int8_t *wv, const float *sv, int8_t *wgv,
                        float *sgv, int d, int F, hipStream_t stream) {
  if (d < 1 || F < 8 || F % 8) return fail(GROK_EINVAL, "moe_interleave: bad shape d=%d F=%d", d, F);
  if (static_cast<int64_t>(d) * F * 2 >= (int64_t(1) << 32)) return fail(GROK_EINVAL, "moe_interleave: too large");
  if (!wg || !sg || !wv || !sv || !wgv || !sgv) return fail(GROK_EINVAL, "moe_interleave: null pointer");
  if ((reinterpret_cast<uintptr_t>(wg) | reinterpret_cast<uintptr_t>(wv)) % 4 ||
      reinterpret_cast<uintptr_t>(wgv) % 8 ||
      (reinterpret_cast<uintptr_t>(sg) | reinterpret_cast<uintptr_t>(sv) | reinterpret_cast<uintptr_t>(sgv)) % 16)
    return fail(GROK_EINVAL, "moe_interleave: misaligned pointer");
  return hip_status(grok::launch_moe_interleave(wg, wv, sg, sv, wgv, sgv, d, F, stream), "moe_interleave");
}

int grok_moe_route(const void *n, const float *w_router, int32_t *idx, float *gates, int64_t T, int d,
                   int E, int k, hipStream_t stream) {
  if (int r = moe_shape_error("moe_route", T, d, 8, E, k)) return r;
  if (T == 0) return ok();
  if (!n || !w_router || !idx || !gates) return fail(GROK_EINVAL, "moe_route: null pointer");
  if (reinterpret_cast<uintptr_t>(n) % 16 ||
      (reinterpret_cast<uintptr_t>(w_router) | reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(gates)) % 4)
    return fail(GROK_EINVAL, "moe_route: misaligned pointer");
  return hip_status(grok::launch_moe_route(n, w_router, idx, gates, T, d, E, k, stream), "moe_route");
}

int grok_moe_ffn(const void *x, const float *w_router, int E, int k, const int8_t *const *wgv,
                 const float *const *sgv, const int8_t *const *w1, const float *const *s1, int64_t T, int d,
                 int F, float eps, int32_t *idx, float *gates, void *workspace, size_t ws_bytes, void *out,
                 hipStream_t stream) {
  if (int r = moe_shape_error("moe_ffn", T, d, F, E, k)) return r;
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(GROK_EINVAL, "moe_ffn: bad eps");
  if (T == 0) return ok();
  if (!x || !w_router || !wgv || !sgv || !w1 || !s1 || !workspace || !out)
    return fail(GROK_EINVAL, "moe_ffn: null pointer");
  uintptr_t a16 = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out) |
                  reinterpret_cast<uintptr_t>(workspace);
  uintptr_t a8 = 0;
  for (int e = 0; e < E; ++e) {
    if (!wgv[e] || !sgv[e] || !w1[e] || !s1[e]) return fail(GROK_EINVAL, "moe_ffn: null pointer in expert %d", e);
    a16 |= reinterpret_cast<uintptr_t>(sgv[e]) | reinterpret_cast<uintptr_t>(s1[e]);
    a8 |= reinterpret_cast<uintptr_t>(wgv[e]) | reinterpret_cast<uintptr_t>(w1[e]);
  }
  const uintptr_t a4 = reinterpret_cast<uintptr_t>(w_router) | reinterpret_cast<uintptr_t>(idx) |
                       reinterpret_cast<uintptr_t>(gates);
  if (a16 % 16 || a8 % 8 || a4 % 4) return fail(GROK_EINVAL, "moe_ffn: misaligned pointer");
  const size_t need = grok::moe_workspace(T, d, F, E, k).total;
  if (ws_bytes < need) return fail(GROK_ENOMEM, "moe_ffn: workspace %zu bytes < %zu needed", ws_bytes, need);
  return hip_status(grok::launch_moe_ffn(x, w_router, E, k, wgv, sgv, w1, s1, T, d, F, eps, idx, gates, workspace,
                                         out, stream),
                    "moe_ffn");
}

size_t grok_prefill_qkv_workspace_bytes(int Tmax, int D) {
  if (Tmax < 1 || D != 128) return 0;
  return grok::prefill_qkv_workspace_bytes(Tmax);
}

int grok_prefill_qkv(const void *x, const int8_t *wq, const float *sq, const int8_t *wk, const float *sk,
                     const int8_t *wv, const float *sv, void *q_out, void *k_cache, void *v_cache,
                     const int32_t *step, int32_t *new_step, int32_t *status, void *workspace, size_t ws_bytes,
                     int B, int T, int d, int Tmax, int Hq, int Hkv, int D, float rope_base,
                     hipStream_t stream) {
  if (B < 1 || T < 1 || d < 8 || d % 8 || Tmax < 1 || Hq < 1 || Hkv < 1)
    return fail(GROK_EINVAL, "prefill_qkv: bad shape B=%d T=%d d=%d Tmax=%d Hq=%d Hkv=%d", B, T, d, Tmax, Hq, Hkv);
  if (D != 128) return fail(GROK_EINVAL, "prefill_qkv: head size must be 128 (D=%d)", D);
  if (T > Tmax) return fail(GROK_EINVAL, "prefill_qkv: T=%d exceeds Tmax=%d", T, Tmax);
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return fail(GROK_EINVAL, "prefill_qkv: bad rope_base");
  if ((static_cast<int64_t>(B) * T + 255) / 256 > 65535 || Hq + 2 * Hkv > 65535 ||
      static_cast<int64_t>(Tmax) * 128 > 0x7fffffff)
    return fail(GROK_EINVAL, "prefill_qkv: sizes too large");
  if (!x || !wq || !sq || !wk || !sk || !wv || !sv || !q_out || !k_cache || !v_cache || !workspace)
    return fail(GROK_EINVAL, "prefill_qkv: null pointer");
  if (new_step && new_step == step) return fail(GROK_EINVAL, "prefill_qkv: new_step must not alias step");
  const uintptr_t a16 = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(sq) |
                        reinterpret_cast<uintptr_t>(sk) | reinterpret_cast<uintptr_t>(sv) |
                        reinterpret_cast<uintptr_t>(q_out) | reinterpret_cast<uintptr_t>(k_cache) |
                        reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(workspace);
  const uintptr_t a8 = reinterpret_cast<uintptr_t>(wq) | reinterpret_cast<uintptr_t>(wk) |
                       reinterpret_cast<uintptr_t>(wv);
  if (a16 % 16 || a8 % 8) return fail(GROK_EINVAL, "prefill_qkv: misaligned pointer");
  if (overlaps(x, static_cast<size_t>(B) * T * d * 2, q_out, static_cast<size_t>(B) * T * Hq * D * 2))
    return fail(GROK_EINVAL, "prefill_qkv: q_out overlaps x");
  const size_t need = grok::prefill_qkv_workspace_bytes(Tmax);
  if (ws_bytes < need) return fail(GROK_ENOMEM, "prefill_qkv: workspace %zu bytes < %zu needed", ws_bytes, need);
  grok::PrefillQkvArgs qa = {};
  qa.out[0] = static_cast<grok::bf16_t *>(q_out);
  qa.out[1] = static_cast<grok::bf16_t *>(k_cache);
  qa.out[2] = static_cast<grok::bf16_t *>(v_cache);
  qa.w[0] = wq;
  qa.w[1] = wk;
  qa.w[2] = wv;
  qa.s[0] = sq;
  qa.s[1] = sk;
  qa.s[2] = sv;
  qa.step = step;
  qa.new_step = new_step;
  qa.status = status;
  qa.B = B;
  qa.T = T;
  qa.Tmax = Tmax;
  qa.Hq = Hq;
  qa.Hkv = Hkv;
  return hip_status(grok::launch_prefill_qkv(x, qa, workspace, d, rope_base, stream), "prefill_qkv");
}

}  // extern "C"

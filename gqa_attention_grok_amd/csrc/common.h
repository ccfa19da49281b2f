// Shared device helpers and internal launcher declarations of the gfx950 library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grok_attn.h"

namespace grok {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// RoPE of one pair at integer position `pos` (ch. 4 §4.3.1): the phase is the
// fp32 product pos * inv_freq, cos/sin are the accurate library functions, and
// every rounding step is pinned (no contraction), so that every kernel that
// rotates produces the same bits.
__device__ __forceinline__ void rope_phase(int pos, float inv, float &s, float &c) {
  const float theta = __fmul_rn(static_cast<float>(pos), inv);
  sincosf(theta, &s, &c);
}
__device__ __forceinline__ void rope_rotate(float x1, float x2, float c, float s, float &o1, float &o2) {
  o1 = __fmaf_rn(x1, c, -__fmul_rn(x2, s));
  o2 = __fmaf_rn(x2, c, __fmul_rn(x1, s));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---------------------------------------------------------------------------
// Host-side launchers (defined in the .hip files, called by api.cpp after
// validation). Each returns hipSuccess or the launch error.
// ---------------------------------------------------------------------------
struct RopeFreqs {
  float inv[256];  // inv_freq[i] = base^(-2i/D), i < D/2 (D <= 512)
};

// Correctly rounded fp32 of base^(-2i/D) for i < D/2 (computed in double).
void rope_build_freqs(int D, float base, RopeFreqs *f);

hipError_t launch_rmsnorm(const void *x, const float *gamma, const void *residual, void *y,
                          int64_t rows, int d, float eps, int dtype, hipStream_t s);
hipError_t launch_rope(void *x, int B, int T, int H, int D, const int32_t *offset,
                       const RopeFreqs &f, int dtype, hipStream_t s);
hipError_t launch_kv_append(void *kc, void *vc, const void *kn, const void *vn, void *q,
                            const int32_t *step, int32_t *new_step, int32_t *status, int B,
                            int T, int Tmax, int Hq, int Hkv, int D, bool do_rope,
                            const RopeFreqs &f, hipStream_t s);
hipError_t launch_linear_int8(const void *x, const int8_t *w, const float *scales, void *y,
                              int64_t M, int K, int N, hipStream_t s);
// Grouped (MoE) form of the tiled int8 GEMM: kMaxGroups groups at most.
constexpr int kMaxGroups = 8;
struct GroupArgs {
  const int32_t *offsets;  // [E + 1] device: group e owns rows [offsets[e], offsets[e+1])
  const int32_t *rows;     // [M] device: x row of each grouped row, or NULL
  const int8_t *w[kMaxGroups];
  const float *s[kMaxGroups];
  int E;
};
hipError_t launch_linear_int8_grouped(const void *x, const int32_t *rows, const int32_t *offsets, int E,
                                      const int8_t *const *w, const float *const *scales, void *y,
                                      int64_t M_total, int K, int N, bool geglu, hipStream_t s);
// MoE FFN sub-layer (moe.hip): workspace byte offsets of its intermediates.
struct MoeWorkspace {
  size_t n, idx, gates, offsets, rows, pos, h, y, total;
};
MoeWorkspace moe_workspace(int64_t T, int d, int F, int E, int k);
int moe_max_experts();
int moe_max_k();
int moe_max_width();
hipError_t launch_moe_route(const void *n, const float *wr, int32_t *idx, float *gates, int64_t T, int d, int E,
                            int k, hipStream_t s);
hipError_t launch_moe_interleave(const int8_t *wg, const int8_t *wv, const float *sg, const float *sv,
                                 int8_t *wgv, float *sgv, int K, int F, hipStream_t s);
hipError_t launch_moe_ffn(const void *x, const float *w_router, int E, int k, const int8_t *const *wgv,
                          const float *const *sgv, const int8_t *const *w1, const float *const *s1, int64_t T,
                          int d, int F, float eps, int32_t *idx, float *gates, void *workspace, void *out,
                          hipStream_t s);
// Fused Q/K/V projection of T rows per sequence (linear_int8.hip): one head
// (128 channels) per column tile, RoPE and the cache write in the epilogue.
struct PrefillQkvArgs {
  bf16_t *out[3];         // q_out [B,T,Hq,128], k_cache, v_cache [B,Tmax,Hkv,128]
  const int8_t *w[3];     // Wq [d, Hq*128], Wk, Wv [d, Hkv*128]
  const float *s[3];
  const int32_t *step;    // [B] first position of each sequence, or NULL (0)
  int32_t *new_step;      // [B] or NULL
  int32_t *status;        // or NULL
  const float *rtab;      // [Tmax][128]: cos of pairs 0..63, then sin
  int B, T, Tmax, Hq, Hkv;
};
size_t prefill_qkv_workspace_bytes(int Tmax);
hipError_t launch_prefill_qkv(const void *x, const PrefillQkvArgs &qa, void *workspace, int d, float rope_base,
                              hipStream_t s);
// Few-row int8 Linear on packed weights (layout in linear_int8_gemv.hip).
size_t gemv_packed_bytes(int K, int N);
hipError_t launch_linear_int8_pack(const int8_t *w, int8_t *wp, int K, int N, hipStream_t s);
hipError_t launch_linear_int8_gemv(const void *x, int n, const int8_t *const *w,
                                   const float *const *scales, void *const *y, const int *N,
                                   int64_t M, int K, hipStream_t s);
// Output projection + post-norm + residual for few rows (linear_int8_gemv.hip):
// one launch for up to out_norm_max_fused_rows(K) rows, else the projection
// and grok_rmsnorm's kernel. The workspace holds an arrival counter (zero
// between calls), per-workgroup sums of squares and the bf16 projection.
size_t out_norm_workspace_bytes(int64_t M, int N);
int out_norm_max_fused_rows(int K);
hipError_t launch_out_norm(const void *x, const int8_t *w, const float *scale, const float *gamma, float eps,
                           const void *res, void *y, void *ws, int64_t M, int K, int N, hipStream_t stream);
// Decode front half: [norm] -> Q|K|V (packed weights) -> RoPE -> cache slot.
hipError_t launch_decode_qkv(const void *x, const float *gamma, float eps, bool prenorm,
                             const int8_t *const *w, const float *const *scales, void *q_out,
                             void *kc, void *vc, const int32_t *step, int32_t *new_step,
                             int32_t *status, int B, int d, int Tmax, int Hq, int Hkv,
                             const RopeFreqs &f, hipStream_t s);
// Largest B for which the fused pre-norm is available at model width d.
int decode_qkv_max_prenorm_rows(int d);
hipError_t launch_prefill_generic(const void *q, const void *k, const void *v, int64_t kv_rows,
                                  const uint8_t *key_valid, void *out, int B, int T, int Hq,
                                  int Hkv, int D, float mult, float cap, int dtype,
                                  hipStream_t s);
hipError_t launch_prefill_mfma(const void *q, const void *k, const void *v, int64_t kv_rows,
                               const uint8_t *key_valid, void *out, int B, int T, int Hq,
                               int Hkv, float mult, float cap, hipStream_t s,
                               const int32_t *offset = nullptr, int32_t *status = nullptr,
                               const float *rtab = nullptr);
// cos/sin of rope_phase for positions 0..npos-1 and the D/2 = 64 pairs:
// tab[p][i] = cos, tab[p][64 + i] = sin (linear_int8.hip).
hipError_t launch_rope_table(float *tab, int npos, const RopeFreqs &f, hipStream_t s);
bool prefill_mfma_supported(int64_t kv_rows, int Hq, int Hkv, int D, int dtype);
hipError_t launch_decode(const void *q, const void *kc, const void *vc, const int32_t *kv_len,
                         void *out, void *ws, int32_t *status, int B, int Tmax, int Hq, int Hkv,
                         float mult, float cap, hipStream_t s);
size_t decode_workspace_bytes(int B, int Tmax, int Hq, int Hkv);
// Device scratch of the allocation-free decode entry point (decode.hip): its
// size, and its device address on the current GPU (looked up once per GPU).
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t decode_static_scratch(void **ptr);
hipError_t launch_decode_append(const void *q, const void *kn, const void *vn, void *kc, void *vc,
                                const int32_t *step, int32_t *new_step, void *q_out, void *out,
                                void *ws, int32_t *status, int B, int Tmax, int Hq, int Hkv,
                                float mult, float cap, const RopeFreqs &f, hipStream_t st);

}  // namespace grok

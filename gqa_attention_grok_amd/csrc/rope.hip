// Rotary position embedding and the RoPE-then-append KV-cache write.
//
// RoPE (Grok-1 walkthrough, ch. 4 "model.py close reading, part 1", §4.3 and
// §4.3.1): x' = x*cos(phase) + rotate_half(x)*sin(phase), with
// rotate_half([x1, x2]) = [-x2, x1] (GPT-NeoX half split, §4.3.1.1), the phase
// the fp32 product position * inv_freq[i] and inv_freq[i] = base^(-2i/D).
//
// KV append (same page, §4.4): K and Q are rotated at their absolute position
// step[b] + t first, then K/V are written into the cache at that slot.
//
// Both kernels are HBM-bound elementwise passes. cos/sin depend only on
// (position, pair), so they are computed once per token into LDS and shared by
// every head of that token.
#include <math.h>

#include "common.h"

namespace grok {

void rope_build_freqs(int D, float base, RopeFreqs *f) {
  for (int i = 0; i < 256; ++i) f->inv[i] = 0.f;
  for (int i = 0; i < D / 2; ++i)
    f->inv[i] = static_cast<float>(pow(static_cast<double>(base), -2.0 * i / D));
}

namespace {

constexpr int kThreads = 256;

// One rotated pair (rope_rotate / rope_phase of common.h: every rounding step
// pinned, so that grok_rope and the fused appends produce identical bits).
__device__ __forceinline__ void rotate_pair(float x1, float x2, float c, float s, float &o1,
                                            float &o2) {
  rope_rotate(x1, x2, c, s, o1, o2);
}

__device__ __forceinline__ void phase_sincos(int pos, float inv, float &s, float &c) {
  rope_phase(pos, inv, s, c);
}

// Vector of V consecutive elements of type T.
template <typename T, int V>
struct Vec {
  T v[V];
};

template <typename T>
__device__ __forceinline__ float ld(T x);
template <>
__device__ __forceinline__ float ld<bf16_t>(bf16_t x) { return bf16_to_f32(x); }
template <>
__device__ __forceinline__ float ld<float>(float x) { return x; }
template <typename T>
__device__ __forceinline__ T st(float x);
template <>
__device__ __forceinline__ bf16_t st<bf16_t>(float x) { return f32_to_bf16(x); }
template <>
__device__ __forceinline__ float st<float>(float x) { return x; }

// Rotate V pairs (i0..i0+V-1, i0+P..) of one head from src into dst (may alias).
template <typename T, int V>
__device__ __forceinline__ void rope_head_chunk(const T *src, T *dst, int i0, int P,
                                                const float *cs, const float *sn) {
  const Vec<T, V> a = *reinterpret_cast<const Vec<T, V> *>(src + i0);
  const Vec<T, V> b = *reinterpret_cast<const Vec<T, V> *>(src + P + i0);
  Vec<T, V> oa, ob;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    float o1, o2;
    rotate_pair(ld<T>(a.v[j]), ld<T>(b.v[j]), cs[j], sn[j], o1, o2);
    oa.v[j] = st<T>(o1);
    ob.v[j] = st<T>(o2);
  }
  *reinterpret_cast<Vec<T, V> *>(dst + i0) = oa;
  *reinterpret_cast<Vec<T, V> *>(dst + P + i0) = ob;
}

// grid.x = B*T tokens (grid-stride). Per token, the D/2 (cos, sin) pairs are
// computed once into LDS, then the threads rotate (head, pair-chunk) items.
template <typename T, int V>
__global__ __launch_bounds__(kThreads) void rope_kernel(T *x, int64_t ntok, int T_, int H, int D,
                                                        const int32_t *offset, RopeFreqs f) {
  __shared__ float cs_s[256], sn_s[256];
  const int P = D / 2;
  const int nchunk = P / V;
  for (int64_t tok = blockIdx.x; tok < ntok; tok += gridDim.x) {
    const int b = static_cast<int>(tok / T_);
    const int t = static_cast<int>(tok % T_);
    const int pos = (offset ? offset[b] : 0) + t;
    if (threadIdx.x < P) phase_sincos(pos, f.inv[threadIdx.x], sn_s[threadIdx.x], cs_s[threadIdx.x]);
    __syncthreads();
    T *row = x + tok * static_cast<int64_t>(H) * D;
    for (int w = threadIdx.x; w < H * nchunk; w += kThreads) {
      const int h = w / nchunk, c = w % nchunk;
      rope_head_chunk<T, V>(row + static_cast<int64_t>(h) * D, row + static_cast<int64_t>(h) * D,
                            c * V, P, cs_s + c * V, sn_s + c * V);
    }
    __syncthreads();  // LDS reused by the next token
  }
}

// grid.x = B*T (one block per new token). Work items of a token:
// (cos, sin) of the token's position are computed once into LDS.
//   [0, Hq*nchunk)                     rotate q head chunks in place
//   [.., + Hkv*nchunk)                 rotate k_new chunks into the cache
//   [.., + Hkv*(D/8))                  copy v_new 16-byte chunks into the cache
template <int V>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    bf16_t *kc, bf16_t *vc, const bf16_t *kn, const bf16_t *vn, bf16_t *q, const int32_t *step,
    int32_t *new_step, int32_t *status, int T_, int Tmax, int Hq, int Hkv, int D, int do_rope,
    RopeFreqs f) {
  const int b = blockIdx.x / T_;
  const int t = blockIdx.x % T_;
  const int s0 = step[b];
  const bool ok = s0 >= 0 && s0 <= Tmax - T_;
  if (t == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    if (new_step) new_step[b] = ok ? s0 + T_ : s0;
    if (!ok && status) *status = GROK_ERANGE;
  }
  if (!ok) return;
  const int pos = s0 + t;
  const int P = D / 2;
  __shared__ float cs_s[256], sn_s[256];
  if (do_rope && threadIdx.x < P) phase_sincos(pos, f.inv[threadIdx.x], sn_s[threadIdx.x], cs_s[threadIdx.x]);
  __syncthreads();
  const int nchunk = P / V;
  const int nq = q ? Hq * nchunk : 0;
  const int nk = Hkv * nchunk;
  const int nv = Hkv * (D / 8);
  const int64_t tok = static_cast<int64_t>(b) * T_ + t;
  const int64_t slot = static_cast<int64_t>(b) * Tmax + pos;
  // One work item (a q or k chunk pair to rotate, or a 16-byte piece of v)
  // per thread: the token's items are spread over gridDim.y workgroups so that
  // all loads are in flight at once.
  for (int w = blockIdx.y * kThreads + threadIdx.x; w < nq + nk + nv; w += kThreads * gridDim.y) {
    if (w < nq + nk) {
      const int ww = w < nq ? w : w - nq;
      const int h = ww / nchunk, c = ww % nchunk;
      const bf16_t *src;
      bf16_t *dst;
      if (w < nq) {
        src = dst = q + (tok * Hq + h) * D;
      } else {
        src = kn + (tok * Hkv + h) * D;
        dst = kc + (slot * Hkv + h) * D;
      }
      if (do_rope) {
        rope_head_chunk<bf16_t, V>(src, dst, c * V, P, cs_s + c * V, sn_s + c * V);
      } else if (src != dst) {
        *reinterpret_cast<Vec<bf16_t, V> *>(dst + c * V) =
            *reinterpret_cast<const Vec<bf16_t, V> *>(src + c * V);
        *reinterpret_cast<Vec<bf16_t, V> *>(dst + P + c * V) =
            *reinterpret_cast<const Vec<bf16_t, V> *>(src + P + c * V);
      }
    } else {
      const int ww = w - nq - nk;
      const int h = ww / (D / 8), c = ww % (D / 8);
      *reinterpret_cast<u32x4 *>(vc + (slot * Hkv + h) * D + c * 8) =
          *reinterpret_cast<const u32x4 *>(vn + (tok * Hkv + h) * D + c * 8);
    }
  }
}

template <typename T>
hipError_t rope_dispatch(void *x, int B, int T_, int H, int D, const int32_t *offset,
                         const RopeFreqs &f, hipStream_t s) {
  const int64_t ntok = static_cast<int64_t>(B) * T_;
  const int grid = static_cast<int>(ntok < (1 << 20) ? ntok : (1 << 20));
  const int P = D / 2;
  constexpr int VB = sizeof(T) == 2 ? 8 : 4;
  const bool vec = (P % VB == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  if (vec)
    hipLaunchKernelGGL((rope_kernel<T, VB>), dim3(grid), dim3(kThreads), 0, s,
                       static_cast<T *>(x), ntok, T_, H, D, offset, f);
  else
    hipLaunchKernelGGL((rope_kernel<T, 1>), dim3(grid), dim3(kThreads), 0, s,
                       static_cast<T *>(x), ntok, T_, H, D, offset, f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(void *x, int B, int T, int H, int D, const int32_t *offset,
                       const RopeFreqs &f, int dtype, hipStream_t s) {
  if (dtype == GROK_BF16) return rope_dispatch<bf16_t>(x, B, T, H, D, offset, f, s);
  return rope_dispatch<float>(x, B, T, H, D, offset, f, s);
}

hipError_t launch_kv_append(void *kc, void *vc, const void *kn, const void *vn, void *q,
                            const int32_t *step, int32_t *new_step, int32_t *status, int B,
                            int T, int Tmax, int Hq, int Hkv, int D, bool do_rope,
                            const RopeFreqs &f, hipStream_t s) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(kc) | reinterpret_cast<uintptr_t>(vc) |
                      reinterpret_cast<uintptr_t>(kn) | reinterpret_cast<uintptr_t>(vn) |
                      reinterpret_cast<uintptr_t>(q);
  if (a % 16 != 0 || D % 16 != 0) return hipErrorInvalidValue;  // validated by the caller
  const int items = (q ? Hq * (D / 2 / 8) : 0) + Hkv * (D / 2 / 8) + Hkv * (D / 8);
  const int wgs_per_token = (items + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((kv_append_kernel<8>), dim3(B * T, wgs_per_token), dim3(kThreads), 0, s,
                     static_cast<bf16_t *>(kc), static_cast<bf16_t *>(vc),
                     static_cast<const bf16_t *>(kn), static_cast<const bf16_t *>(vn),
                     static_cast<bf16_t *>(q), step, new_step, status, T, Tmax, Hq, Hkv, D,
                     do_rope ? 1 : 0, f);
  return hipGetLastError();
}

}  // namespace grok

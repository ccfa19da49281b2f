// RMSNorm over the last axis (Grok-1 walkthrough, ch. 4 "model.py close reading,
// part 1", §4.2): y = gamma * x * rsqrt(mean(x^2) + eps), fp32 inside.
// Optional fused residual add of the sandwich norm (ch. 6 "model.py close reading,
// part 3", §6.3.1): y = residual + round(norm(x)).
//
// One 256-thread workgroup per row. HBM-bound: a row is read once (twice in
// the fallback for very wide or unaligned rows) and written once.
#include "common.h"

namespace grok {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 4;  // 16-byte chunks per thread kept in registers

template <typename T>
struct Io;
template <>
struct Io<bf16_t> {
  static constexpr int kVec = 8;
  static __device__ __forceinline__ void unpack(const u32x4 &w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = lo_bf16(w[i]);
      f[2 * i + 1] = hi_bf16(w[i]);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float *f) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return w;
  }
  static __device__ __forceinline__ float round(float f) { return bf16_to_f32(f32_to_bf16(f)); }
  static __device__ __forceinline__ float load1(const bf16_t *p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store1(bf16_t *p, float f) { *p = f32_to_bf16(f); }
};
template <>
struct Io<float> {
  static constexpr int kVec = 4;
  static __device__ __forceinline__ void unpack(const u32x4 &w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
  static __device__ __forceinline__ u32x4 pack(const float *f) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(f[i]);
    return w;
  }
  static __device__ __forceinline__ float round(float f) { return f; }
  static __device__ __forceinline__ float load1(const float *p) { return *p; }
  static __device__ __forceinline__ void store1(float *p, float f) { *p = f; }
};

__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();  // previous use of red[] finished
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) s += red[i];
  return s;
}

// Vector path: every row fits in kMaxChunks 16-byte chunks per thread.
template <typename T, bool kGamma, bool kRes>
__global__ __launch_bounds__(kThreads) void rmsnorm_vec(const T *x,
                                                        const float *__restrict__ gamma,
                                                        const T *residual, T *y,
                                                        int64_t rows, int d, float eps) {
  constexpr int V = Io<T>::kVec;
  __shared__ float red[kThreads / kWave];
  const int nchunk = d / V;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + row * d);
    u32x4 raw[kMaxChunks];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int ci = threadIdx.x + c * kThreads;
      if (ci < nchunk) {
        raw[c] = xr[ci];
        float f[V];
        Io<T>::unpack(raw[c], f);
#pragma unroll
        for (int i = 0; i < V; ++i) ss += f[i] * f[i];
      }
    }
    const float r = rsqrtf(block_sum(ss, red) / static_cast<float>(d) + eps);
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int ci = threadIdx.x + c * kThreads;
      if (ci < nchunk) {
        float f[V];
        Io<T>::unpack(raw[c], f);
        if constexpr (kGamma) {
          const f32x4 *g4 = reinterpret_cast<const f32x4 *>(gamma + ci * V);
#pragma unroll
          for (int j = 0; j < V / 4; ++j) {
            const f32x4 g = g4[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) f[4 * j + i] = g[i] * (f[4 * j + i] * r);
          }
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i) f[i] = f[i] * r;
        }
        if constexpr (kRes) {
          float rf[V];
          Io<T>::unpack(reinterpret_cast<const u32x4 *>(residual + row * d)[ci], rf);
#pragma unroll
          for (int i = 0; i < V; ++i) f[i] = rf[i] + Io<T>::round(f[i]);
        }
        reinterpret_cast<u32x4 *>(y + row * d)[ci] = Io<T>::pack(f);
      }
    }
  }
}

// Fallback: any d, two passes over the row.
template <typename T, bool kGamma, bool kRes>
__global__ __launch_bounds__(kThreads) void rmsnorm_any(const T *x, const float *gamma,
                                                        const T *residual, T *y, int64_t rows,
                                                        int d, float eps) {
  __shared__ float red[kThreads / kWave];
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const T *xr = x + row * d;
    float ss = 0.f;
    for (int i = threadIdx.x; i < d; i += kThreads) {
      const float f = Io<T>::load1(xr + i);
      ss += f * f;
    }
    const float r = rsqrtf(block_sum(ss, red) / static_cast<float>(d) + eps);
    // y may alias x: every thread reads element i before writing element i,
    // and the sum above completed before the first write.
    for (int i = threadIdx.x; i < d; i += kThreads) {
      float f = Io<T>::load1(xr + i) * r;
      if constexpr (kGamma) f = gamma[i] * f;
      if constexpr (kRes) f = Io<T>::load1(residual + row * d + i) + Io<T>::round(f);
      Io<T>::store1(y + row * d + i, f);
    }
  }
}

template <typename T>
hipError_t dispatch(const void *x, const float *gamma, const void *res, void *y, int64_t rows,
                    int d, float eps, hipStream_t s) {
  constexpr int V = Io<T>::kVec;
  const uintptr_t align = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y) |
                          reinterpret_cast<uintptr_t>(res) | reinterpret_cast<uintptr_t>(gamma);
  const bool vec = (d % V == 0) && (d / V <= kThreads * kMaxChunks) && (align % 16 == 0);
  const int grid = static_cast<int>(rows < (1 << 20) ? rows : (1 << 20));
  const T *xt = static_cast<const T *>(x);
  const T *rt = static_cast<const T *>(res);
  T *yt = static_cast<T *>(y);
#define GROK_RMS_LAUNCH(KERNEL, G, R) \
  hipLaunchKernelGGL((KERNEL<T, G, R>), dim3(grid), dim3(kThreads), 0, s, xt, gamma, rt, yt, rows, d, eps)
  if (vec) {
    if (gamma && res) GROK_RMS_LAUNCH(rmsnorm_vec, true, true);
    else if (gamma) GROK_RMS_LAUNCH(rmsnorm_vec, true, false);
    else if (res) GROK_RMS_LAUNCH(rmsnorm_vec, false, true);
    else GROK_RMS_LAUNCH(rmsnorm_vec, false, false);
  } else {
    if (gamma && res) GROK_RMS_LAUNCH(rmsnorm_any, true, true);
    else if (gamma) GROK_RMS_LAUNCH(rmsnorm_any, true, false);
    else if (res) GROK_RMS_LAUNCH(rmsnorm_any, false, true);
    else GROK_RMS_LAUNCH(rmsnorm_any, false, false);
  }
#undef GROK_RMS_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const void *x, const float *gamma, const void *residual, void *y,
                          int64_t rows, int d, float eps, int dtype, hipStream_t s) {
  if (dtype == GROK_BF16) return dispatch<bf16_t>(x, gamma, residual, y, rows, d, eps, s);
  return dispatch<float>(x, gamma, residual, y, rows, d, eps, s);
}

}  // namespace grok

// Causal GQA prefill, generic path: any head size D <= 256 (D % 8 == 0), fp32
// or bf16 I/O. One wavefront per (sequence, position, query head); simple and
// latency-bound, used for fp32 and for head sizes the MFMA kernel does not
// cover. The method (Grok-1 walkthrough, ch. 4 "model.py close reading, part 1",
// §4.5.2-§4.5.4; causal x padding mask from ch. 6 "model.py close reading,
// part 3", §6.4.2):
//   c_j = cap * tanh(mult * <q, k_j> / cap);  masked c_j -> -1e30;
//   out = softmax(c) . V
//
// Softmax shift: every unmasked c_j lies in [-cap, cap], so exp(c_j - cap)
// never overflows and, for cap <= 40, never underflows below fp32's normal
// range: the row maximum is not needed. Masked entries contribute exactly 0.
// A row with no unmasked key gets the pages' -1e30 semantics: equal weights
// on all T keys.
#include "common.h"

namespace grok {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxR = 4;  // D <= 64 * kMaxR

template <typename T>
__device__ __forceinline__ float ldf(const T *p);
template <>
__device__ __forceinline__ float ldf<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float ldf<bf16_t>(const bf16_t *p) { return bf16_to_f32(*p); }
template <typename T>
__device__ __forceinline__ void stf(T *p, float v);
template <>
__device__ __forceinline__ void stf<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void stf<bf16_t>(bf16_t *p, float v) { *p = f32_to_bf16(v); }

template <typename T>
__global__ __launch_bounds__(kThreads) void prefill_generic_kernel(
    const T *q, const T *k, const T *v, int64_t kv_rows, const uint8_t *key_valid, T *out, int B,
    int T_, int Hq, int Hkv, int D, float mult, float cap) {
  const int64_t nrows = static_cast<int64_t>(B) * T_ * Hq;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
  if (row >= nrows) return;
  const int lane = threadIdx.x % kWave;
  const int h = static_cast<int>(row % Hq);
  const int i = static_cast<int>((row / Hq) % T_);
  const int b = static_cast<int>(row / (static_cast<int64_t>(Hq) * T_));
  const int g = h / (Hq / Hkv);
  const T *qr = q + row * D;
  const T *kb = k + (static_cast<int64_t>(b) * kv_rows * Hkv + g) * D;
  const T *vb = v + (static_cast<int64_t>(b) * kv_rows * Hkv + g) * D;
  const int64_t kstride = static_cast<int64_t>(Hkv) * D;
  const uint8_t *kv = key_valid ? key_valid + static_cast<int64_t>(b) * T_ : nullptr;

  float qv[kMaxR], o[kMaxR];
#pragma unroll
  for (int r = 0; r < kMaxR; ++r) {
    const int d = lane + kWave * r;
    qv[r] = d < D ? ldf<T>(qr + d) : 0.f;
    o[r] = 0.f;
  }
  float l = 0.f;
  for (int j = 0; j <= i; ++j) {
    if (kv && kv[j] == 0) continue;
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxR; ++r) {
      const int d = lane + kWave * r;
      if (d < D) part += qv[r] * ldf<T>(kb + j * kstride + d);
    }
    const float z = wave_sum(part) * mult;
    const float c = cap * tanhf(z / cap);
    const float p = expf(c - cap);
    l += p;
#pragma unroll
    for (int r = 0; r < kMaxR; ++r) {
      const int d = lane + kWave * r;
      if (d < D) o[r] += p * ldf<T>(vb + j * kstride + d);
    }
  }
  float inv;
  if (l > 0.f) {
    inv = 1.f / l;
  } else {  // no valid key: uniform weights over all T keys
#pragma unroll
    for (int r = 0; r < kMaxR; ++r) o[r] = 0.f;
    for (int j = 0; j < T_; ++j) {
#pragma unroll
      for (int r = 0; r < kMaxR; ++r) {
        const int d = lane + kWave * r;
        if (d < D) o[r] += ldf<T>(vb + j * kstride + d);
      }
    }
    inv = 1.f / static_cast<float>(T_);
  }
  T *orow = out + row * D;  // [B, T, Hq*D] == [B*T*Hq, D]
#pragma unroll
  for (int r = 0; r < kMaxR; ++r) {
    const int d = lane + kWave * r;
    if (d < D) stf<T>(orow + d, o[r] * inv);
  }
}

}  // namespace

hipError_t launch_prefill_generic(const void *q, const void *k, const void *v, int64_t kv_rows,
                                  const uint8_t *key_valid, void *out, int B, int T, int Hq,
                                  int Hkv, int D, float mult, float cap, int dtype,
                                  hipStream_t s) {
  const int64_t nrows = static_cast<int64_t>(B) * T * Hq;
  const int64_t grid = (nrows + (kThreads / kWave) - 1) / (kThreads / kWave);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (dtype == GROK_F32)
    hipLaunchKernelGGL((prefill_generic_kernel<float>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, s, static_cast<const float *>(q),
                       static_cast<const float *>(k), static_cast<const float *>(v), kv_rows,
                       key_valid, static_cast<float *>(out), B, T, Hq, Hkv, D, mult, cap);
  else
    hipLaunchKernelGGL((prefill_generic_kernel<bf16_t>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, s, static_cast<const bf16_t *>(q),
                       static_cast<const bf16_t *>(k), static_cast<const bf16_t *>(v), kv_rows,
                       key_valid, static_cast<bf16_t *>(out), B, T, Hq, Hkv, D, mult, cap);
  return hipGetLastError();
}

}  // namespace grok

// int8-weight Linear with per-output-channel scales (Grok-1 walkthrough, ch. 4
// "model.py close reading, part 1", §4.1 and §4.1.1): y = x @ (w * s),
// x [M,K] bf16, w [K,N] int8, s [N] fp32, y [M,N] bf16, no bias.
//
// W8A16 MFMA GEMM for gfx950. The weights stay int8 in HBM (half the bytes of
// bf16) and are widened once per workgroup tile, while being staged into LDS:
// |w| <= 127 is exact in bf16, so the MFMA sees the exact integers and the
// channel scale is applied to the fp32 sum in the epilogue.
//
// Formulation (v_mfma_f32_16x16x32_bf16), computed transposed so that the
// epilogue writes runs of 4 consecutive output channels:
//   Y^T[n, m] = sum_k W^T[n, k] X^T[k, m]     A = W^T (LDS, k-contiguous)
//                                             B = X   (LDS, k-contiguous)
// Workgroup tile 128 (n) x 128 (m), K step 64, 4 waves in 2 x 2, each wave
// 64 x 64 = 4 x 4 MFMA tiles; LDS double-buffered.
#include "common.h"

namespace grok {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 128;  // output channels per workgroup
constexpr int kBM = 128;  // rows per workgroup
constexpr int kBK = 64;
constexpr int kRow = kBK + 8;  // padded LDS row (bf16 elements)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float i8_to_f32(uint32_t word, int byte) {
  return static_cast<float>(static_cast<int8_t>((word >> (8 * byte)) & 0xffu));
}

__global__ __launch_bounds__(kThreads, 2) void linear_int8_kernel(
    const bf16_t *__restrict__ x, const int8_t *__restrict__ w, const float *__restrict__ scales,
    bf16_t *__restrict__ y, int64_t M, int K, int N) {
  __shared__ __attribute__((aligned(16))) bf16_t Xs[2][kBM][kRow];
  __shared__ __attribute__((aligned(16))) bf16_t Wt[2][kBN][kRow];

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int wn = wave % 2, wm = wave / 2;
  const int n0 = blockIdx.x * kBN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;

  // X staging: 4 chunks of 16 B per thread: row = c/8, k chunk = c%8.
  // W staging: 4 rows (k) x 8 channels (n) int8 per thread.
  const int wnc = tid % 16, wkq = tid / 16;  // channels 8*wnc.., k rows 4*wkq..
  u32x4 xr[4];
  u32x2 wr[4];

  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + kThreads * r;
      const int64_t m = m0 + c / 8;
      const int k = k0 + (c % 8) * 8;
      xr[r] = (m < M && k < K) ? *reinterpret_cast<const u32x4 *>(x + m * K + k) : u32x4{0, 0, 0, 0};
    }
    const int n = n0 + 8 * wnc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = k0 + 4 * wkq + r;
      wr[r] = (k < K && n < N) ? *reinterpret_cast<const u32x2 *>(w + static_cast<int64_t>(k) * N + n) : u32x2{0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = tid + kThreads * r;
      *reinterpret_cast<u32x4 *>(&Xs[buf][c / 8][(c % 8) * 8]) = xr[r];
    }
    // Transpose the 4x8 int8 block: for each channel j, the 4 k values become 4
    // consecutive bf16 of row W^T[n = 8*wnc + j].
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int wd = j / 4, by = j % 4;
      const float f0 = i8_to_f32(wr[0][wd], by), f1 = i8_to_f32(wr[1][wd], by);
      const float f2 = i8_to_f32(wr[2][wd], by), f3 = i8_to_f32(wr[3][wd], by);
      const u32x2 pk = {cvt_pk_bf16(f0, f1), cvt_pk_bf16(f2, f3)};
      *reinterpret_cast<u32x2 *>(&Wt[buf][8 * wnc + j][4 * wkq]) = pk;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + kBK - 1) / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const int buf = t & 1;
    if (t + 1 < nk) gload((t + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      bf16x8 bx[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        bx[mb] = *reinterpret_cast<const bf16x8 *>(&Xs[buf][64 * wm + 16 * mb + lr][32 * kk + 8 * lg]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 aw = *reinterpret_cast<const bf16x8 *>(&Wt[buf][64 * wn + 16 * nb + lr][32 * kk + 8 * lg]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bx[mb], acc[nb][mb], 0, 0, 0);
      }
    }
    if (t + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds Y^T[n = nbase + 4*lg + v, m = mbase + lr], v = 0..3.
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + 64 * wn + 16 * nb + 4 * lg;
    if (n >= N) continue;
    const f32x4 sc = *reinterpret_cast<const f32x4 *>(scales + n);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int64_t m = m0 + 64 * wm + 16 * mb + lr;
      if (m >= M) continue;
      const f32x4 v = acc[nb][mb];
      const u32x2 o = {cvt_pk_bf16(v[0] * sc[0], v[1] * sc[1]), cvt_pk_bf16(v[2] * sc[2], v[3] * sc[3])};
      *reinterpret_cast<u32x2 *>(y + m * N + n) = o;
    }
  }
}

}  // namespace

hipError_t launch_linear_int8(const void *x, const int8_t *w, const float *scales, void *y,
                              int64_t M, int K, int N, hipStream_t s) {
  const int64_t gm = (M + kBM - 1) / kBM;
  if (gm > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((N + kBN - 1) / kBN, static_cast<unsigned>(gm));
  hipLaunchKernelGGL(linear_int8_kernel, grid, dim3(kThreads), 0, s,
                     static_cast<const bf16_t *>(x), w, scales, static_cast<bf16_t *>(y), M, K, N);
  return hipGetLastError();
}

}  // namespace grok

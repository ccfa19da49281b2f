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
constexpr int kRowB = kBK * 2;  // one LDS row: 64 bf16 = 128 bytes, unpadded
constexpr int kTileB = 128 * kRowB;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float i8_to_f32(uint32_t word, int byte) {
  return static_cast<float>(static_cast<int8_t>((word >> (8 * byte)) & 0xffu));
}

// LDS layout of both tiles (X rows m, W^T rows n; 64 k values = 128 bytes per
// row): 16-byte chunk c of row r sits at chunk c ^ sw(r). Two rows share one
// 256-byte line of the 64 four-byte banks; the swizzle spreads the 16 rows of a
// fragment read over all 16 chunk positions of a line pair and keeps the
// transposed W^T stores at two lanes per position.
__device__ __forceinline__ int sw(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * kRowB + ((c ^ sw(r)) << 4); }

__global__ __launch_bounds__(kThreads, 2) void linear_int8_kernel(
    const bf16_t *__restrict__ x, const int8_t *__restrict__ w, const float *__restrict__ scales,
    bf16_t *__restrict__ y, int64_t M, int K, int N) {
  __shared__ __attribute__((aligned(1024))) unsigned char Xs[2][kTileB];
  __shared__ __attribute__((aligned(1024))) unsigned char Wt[2][kTileB];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane % 16, lg = lane / 16;
  const int wn = wave % 2, wm = wave / 2;
  const int n0 = blockIdx.x * kBN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;

  // X tile: HBM -> LDS directly (global_load_lds, 16 bytes per lane). Wave
  // `wave`, instruction i fills rows 32*wave + 8*i .. +7; lane L writes chunk
  // position L%8 of row 32*wave + 8*i + L/8, fetching logical chunk
  // (L%8) ^ sw(row). Rows past M read row M-1 and columns past K read the last
  // 8 columns (finite values; the matching W^T entries are zero).
  const int xl_row = lane / 8, xl_pos = lane % 8;
  auto issue_x = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wave + 8 * i + xl_row;
      const int64_t m = min(m0 + r, M - 1);
      const int k = min(k0 + 8 * (xl_pos ^ sw(r)), K - 8);
      __builtin_amdgcn_global_load_lds(x + m * K + k, (lds_void *)(&Xs[buf][(32 * wave + 8 * i) * kRowB]), 16,
                                       0, 0);
    }
  };

  // W staging: 4 rows (k) x 8 channels (n) int8 per thread, widened to bf16 and
  // stored transposed (8 rows of W^T, 4 k values = 8 bytes each).
  const int wnc = tid % 16, wkq = tid / 16;  // channels 8*wnc.., k rows 4*wkq..
  u32x2 wr[4];
  auto gload_w = [&](int k0) {
    const int n = n0 + 8 * wnc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = k0 + 4 * wkq + r;
      wr[r] = (k < K && n < N) ? *reinterpret_cast<const u32x2 *>(w + static_cast<int64_t>(k) * N + n) : u32x2{0, 0};
    }
  };
  auto lstore_w = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int wd = j / 4, by = j % 4;
      const float f0 = i8_to_f32(wr[0][wd], by), f1 = i8_to_f32(wr[1][wd], by);
      const float f2 = i8_to_f32(wr[2][wd], by), f3 = i8_to_f32(wr[3][wd], by);
      const u32x2 pk = {cvt_pk_bf16(f0, f1), cvt_pk_bf16(f2, f3)};
      const int n = 8 * wnc + j;
      *reinterpret_cast<u32x2 *>(&Wt[buf][lds_off(n, wkq >> 1) + 8 * (wkq & 1)]) = pk;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + kBK - 1) / kBK;
  issue_x(0, 0);
  gload_w(0);
  lstore_w(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < nk;
    if (more) {
      issue_x((t + 1) * kBK, buf ^ 1);
      gload_w((t + 1) * kBK);
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      bf16x8 bx[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        bx[mb] = *reinterpret_cast<const bf16x8 *>(&Xs[buf][lds_off(64 * wm + 16 * mb + lr, 4 * kk + lg)]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 aw = *reinterpret_cast<const bf16x8 *>(&Wt[buf][lds_off(64 * wn + 16 * nb + lr, 4 * kk + lg)]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bx[mb], acc[nb][mb], 0, 0, 0);
      }
    }
    if (more) lstore_w(buf ^ 1);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's X loads for the next step have landed
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

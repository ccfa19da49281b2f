// int8-weight Linear for a few rows at a time (Grok-1 walkthrough, ch. 4
// "model.py close reading, part 1", §4.1 and §4.1.1): y = x @ (w * s) with
// x [M,K] bf16, w [K,N] int8, s [N] fp32, y [M,N] bf16, at most 32 rows per
// launch. In decoding each sequence contributes one row, so the product is a
// matrix-vector one and its time is the time to stream the int8 weights from
// HBM once (88 MB per layer for Grok-1's four attention projections).
//
// Up to three matrices that share x (the query, key and value projections of
// §4.5.1) are computed in one launch: their column blocks are numbered one
// after another and each workgroup picks its matrix from its block number.
//
// Two kernels, chosen by the number of rows of the launch:
//
// * up to 4 rows (gemv_rows_kernel): each workgroup owns 32 output channels
//   and the whole K axis, so no partial sums ever leave it. Its 8 waves take
//   interleaved 16-row steps; in a step, 4 lanes read one row's 32 channels
//   (8 bytes each) and 16 rows are read per instruction, 16 steps ahead.
//   Each weight is widened to fp32 once and used in one fma per row of x.
//   The four workgroups of a 128-channel line group are given ids that the
//   dispatcher sends to the same XCD one after another, so each 128-byte line
//   of W comes from HBM once and is shared through that XCD's L2.
//
// * 5 to 32 rows (gemv_int8_kernel): the products go to the matrix cores. A
//   workgroup owns 128 output channels and one of S slices of the K axis; its
//   4 waves take interleaved 32-row steps of that slice. Per step a lane loads
//   8 bytes (8 channels) from each of 8 consecutive rows: lanes 0-15 cover one
//   row's 128 channels, lanes 16-31 the row 8 further on, and so on. The 8
//   rows x 8 channels a lane holds are exactly the B operands of 8
//   v_mfma_f32_16x16x32_bf16 (one per channel: B[k][n] with k the lane's 8
//   rows and n = lane % 16), after each int8 is widened to an exact bf16; the
//   A operand is 16 rows of x (row m = lane % 16, zero beyond M).
//   The 4 waves' sums meet in LDS. With S > 1 each workgroup then writes its
//   slice's sums to the workspace, and the last of the S workgroups of a
//   column block to finish (an atomic ticket per block) adds the S slices in
//   a fixed order, applies the channel scale and writes bf16, then resets the
//   ticket for the next call; the result does not depend on which workgroup
//   finishes last. The slice sums are stored and loaded with device-scope
//   (sc1) accesses, which go to the device's coherence point rather than to a
//   per-XCD L2, and every wave waits for its stores to be acknowledged before
//   the workgroup takes its ticket; no cache write-back or invalidation is
//   needed (a device-scope fence costs a whole L2 write-back per workgroup).
#include "common.h"

namespace grok {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBN = 128;     // output channels per workgroup
constexpr int kStepK = 32;   // rows per MFMA step
constexpr int kBatch = 4;    // steps whose loads are issued together
constexpr int kMaxRows = 32; // rows of x per launch
constexpr int kMaxJ = 8;     // steps per wave per slice

constexpr int kRThreads = 512;  // few-row kernel: 8 waves
constexpr int kRWaves = kRThreads / kWave;
constexpr int kRBN = 32;        // output channels per workgroup (4 lanes x 8)
constexpr int kRRows = 16;      // rows per wave step (one per 4 lanes)
constexpr int kRDepth = 16;     // steps in flight per wave
constexpr int kRMaxRows = 4;    // rows of x the few-row kernel takes

struct GemvMat {
  const int8_t *w;
  const float *s;
  bf16_t *y;
  int N;
  int cb0;  // number of the matrix's first column block
};

struct GemvArgs {
  const bf16_t *x;
  GemvMat mat[3];
  int nmat;
  int M;      // rows of this launch, 1..32
  int K;
  int S;      // slices of K
  int xcd;    // 1: the S workgroups of a column block share an XCD
  float *part;    // [ncb][S][M][128] fp32 slice sums
  uint32_t *cnt;  // [ncb] tickets, zero between calls
};

// Bits of the bf16 that equals int8 byte `b` of `word` (exact: |v| <= 127).
__device__ __forceinline__ float i8_at(uint32_t word, int b) {
  return static_cast<float>(static_cast<int8_t>((word >> (8 * b)) & 0xffu));
}

// High halves of two floats whose values are exact in bf16: (hi << 16) | lo.
__device__ __forceinline__ uint32_t pack_hi(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

template <int MT, int J>
__global__ __launch_bounds__(kThreads) void gemv_int8_kernel(GemvArgs a) {
  extern __shared__ f32x4 red4[];  // [kWaves][M][kBN] floats, 16-byte aligned
  __shared__ int is_last;
  float *red = reinterpret_cast<float *>(red4);
  const int tid = threadIdx.x;
  const int wv = tid / kWave, l = tid % kWave, g = l / 16, i = l % 16;
  const int M = a.M, K = a.K, S = a.S;

  int cb, s;
  if (a.xcd) {  // workgroup b runs on XCD b % 8
    const int q = blockIdx.x >> 3;
    cb = (blockIdx.x & 7) + 8 * (q / S);
    s = q % S;
  } else {
    cb = blockIdx.x / S;
    s = blockIdx.x % S;
  }
  const bool m1 = a.nmat > 1 && cb >= a.mat[1].cb0;
  const bool m2 = a.nmat > 2 && cb >= a.mat[2].cb0;
  const int8_t *w = m2 ? a.mat[2].w : (m1 ? a.mat[1].w : a.mat[0].w);
  const float *sc = m2 ? a.mat[2].s : (m1 ? a.mat[1].s : a.mat[0].s);
  bf16_t *y = m2 ? a.mat[2].y : (m1 ? a.mat[1].y : a.mat[0].y);
  const int N = m2 ? a.mat[2].N : (m1 ? a.mat[1].N : a.mat[0].N);
  const int c0 = (cb - (m2 ? a.mat[2].cb0 : (m1 ? a.mat[1].cb0 : a.mat[0].cb0))) * kBN;

  // This lane's 8 channels; a block's channels past N load the last valid 8
  // (in bounds) and are never stored.
  const int col = c0 + 8 * i;
  const int8_t *wl = w + (col < N ? col : N - 8);
  const int k0 = s * (J * kWaves * kStepK);

  f32x4 acc[MT][8];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j0 = 0; j0 < J; j0 += kBatch) {
    constexpr int kB0 = J < kBatch ? J : kBatch;
    u32x2 wr[kB0][8];
    bf16x8 xa[kB0][MT];
#pragma unroll
    for (int u = 0; u < kB0; ++u) {
      if (j0 + u >= J) break;
      // rows rb .. rb+7 (all valid or all past K: K is a multiple of 8)
      const int rb = k0 + ((j0 + u) * kWaves + wv) * kStepK + 8 * g;
      const bool ok = rb < K;
      const int8_t *src = wl + static_cast<int64_t>(ok ? rb : 0) * N;
#pragma unroll
      for (int r = 0; r < 8; ++r) wr[u][r] = *reinterpret_cast<const u32x2 *>(src + static_cast<int64_t>(r) * N);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = 16 * t + i;
        bf16x8 v = {};
        if (ok && m < M) v = *reinterpret_cast<const bf16x8 *>(a.x + static_cast<int64_t>(m) * K + rb);
        xa[u][t] = v;
      }
    }
#pragma unroll
    for (int u = 0; u < kB0; ++u) {
      if (j0 + u >= J) break;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x4 bw;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bw[e] = pack_hi(i8_at(wr[u][2 * e][j >> 2], j & 3), i8_at(wr[u][2 * e + 1][j >> 2], j & 3));
        const bf16x8 b = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[u][t], b, acc[t][j], 0, 0, 0);
      }
    }
  }

  // acc[t][j][v] = y row 16t + 4g + v, channel c0 + 8i + j (this wave's rows).
  float *mine = red + wv * M * kBN;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * t + 4 * g + v;
      if (m < M) {
        f32x4 *dst = reinterpret_cast<f32x4 *>(mine + m * kBN + 8 * i);
        dst[0] = f32x4{acc[t][0][v], acc[t][1][v], acc[t][2][v], acc[t][3][v]};
        dst[1] = f32x4{acc[t][4][v], acc[t][5][v], acc[t][6][v], acc[t][7][v]};
      }
    }
  __syncthreads();

  const int nq = M * (kBN / 4);  // float4 groups of the block's [M][128] sums
  if (S == 1) {
    for (int q = tid; q < nq; q += kThreads) {
      const int m = q / (kBN / 4), c = (q % (kBN / 4)) * 4;
      if (c0 + c >= N) continue;
      f32x4 sum = *reinterpret_cast<const f32x4 *>(red + m * kBN + c);
#pragma unroll
      for (int u = 1; u < kWaves; ++u) sum += *reinterpret_cast<const f32x4 *>(red + (u * M + m) * kBN + c);
      const f32x4 k4 = *reinterpret_cast<const f32x4 *>(sc + c0 + c);
      const u32x2 o = {pack_bf16x2(sum[0] * k4[0], sum[1] * k4[1]), pack_bf16x2(sum[2] * k4[2], sum[3] * k4[3])};
      *reinterpret_cast<u32x2 *>(y + static_cast<int64_t>(m) * N + c0 + c) = o;
    }
    return;
  }

  float *blk = a.part + static_cast<int64_t>(cb) * S * M * kBN;
  for (int q = tid; q < nq; q += kThreads) {
    const int m = q / (kBN / 4), c = (q % (kBN / 4)) * 4;
    f32x4 sum = *reinterpret_cast<const f32x4 *>(red + m * kBN + c);
#pragma unroll
    for (int u = 1; u < kWaves; ++u) sum += *reinterpret_cast<const f32x4 *>(red + (u * M + m) * kBN + c);
    float *dst = blk + (static_cast<int64_t>(s) * M + m) * kBN + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) __hip_atomic_store(dst + e, sum[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // This wave's slice sums are acknowledged by the coherence point once its
  // memory counter drains; then the workgroup takes its ticket.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.cnt + cb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == static_cast<uint32_t>(S - 1);
    if (last) __hip_atomic_store(a.cnt + cb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = last;
  }
  __syncthreads();
  if (!is_last) return;
  for (int q = tid; q < nq; q += kThreads) {
    const int m = q / (kBN / 4), c = (q % (kBN / 4)) * 4;
    if (c0 + c >= N) continue;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int u = 0; u < S; ++u) {
      const float *src = blk + (static_cast<int64_t>(u) * M + m) * kBN + c;
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += __hip_atomic_load(src + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const f32x4 k4 = *reinterpret_cast<const f32x4 *>(sc + c0 + c);
    const u32x2 o = {pack_bf16x2(sum[0] * k4[0], sum[1] * k4[1]), pack_bf16x2(sum[2] * k4[2], sum[3] * k4[3])};
    *reinterpret_cast<u32x2 *>(y + static_cast<int64_t>(m) * N + c0 + c) = o;
  }
}

// Plain loads as inline assembly (see the few-row kernel's main loop).
__device__ __forceinline__ u32x2 load_w8(const int8_t *p) {
  u32x2 v;
  asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t load_x2(const bf16_t *p) {
  uint32_t v;
  asm volatile("global_load_ushort %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// Lane m of each quad holds the bf16 bits of x row m: broadcast them to the
// whole quad (DPP quad_perm m,m,m,m) as fp32.
template <int m>
__device__ __forceinline__ float quad_lane(uint32_t v) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x55 * m, 0xf, 0xf, false)) << 16);
}
template <int MR>
__device__ __forceinline__ void quad_rows(uint32_t v, float (&xm)[MR]) {
  xm[0] = quad_lane<0>(v);
  if constexpr (MR > 1) xm[1] = quad_lane<1>(v);
  if constexpr (MR > 2) xm[2] = quad_lane<2>(v);
  if constexpr (MR > 3) xm[3] = quad_lane<3>(v);
}

// Few-row kernel (M <= 4): whole K per workgroup, fp32 fma on the vector units.
template <int MR>
__global__ __launch_bounds__(kRThreads) void gemv_rows_kernel(GemvArgs a) {
  __shared__ float red[kRWaves][kRMaxRows][kRBN];
  const int tid = threadIdx.x;
  const int wv = tid / kWave, l = tid % kWave, q4 = l & 3, rl = l >> 2;
  const int M = a.M, K = a.K;

  int cb;
  if (a.xcd) {  // workgroup b runs on XCD b % 8; 4 blocks = one 128-channel line group
    const int q = blockIdx.x >> 3;
    cb = 4 * ((blockIdx.x & 7) + 8 * (q >> 2)) + (q & 3);
  } else {
    cb = blockIdx.x;
  }
  const bool m1 = a.nmat > 1 && cb >= a.mat[1].cb0;
  const bool m2 = a.nmat > 2 && cb >= a.mat[2].cb0;
  const int8_t *w = m2 ? a.mat[2].w : (m1 ? a.mat[1].w : a.mat[0].w);
  const float *sc = m2 ? a.mat[2].s : (m1 ? a.mat[1].s : a.mat[0].s);
  bf16_t *y = m2 ? a.mat[2].y : (m1 ? a.mat[1].y : a.mat[0].y);
  const int N = m2 ? a.mat[2].N : (m1 ? a.mat[1].N : a.mat[0].N);
  const int c0 = (cb - (m2 ? a.mat[2].cb0 : (m1 ? a.mat[1].cb0 : a.mat[0].cb0))) * kRBN;

  // This lane's 8 channels (past N: the last valid 8, never stored) and the
  // row of x this lane fetches for the whole quad (lane q4 of a quad loads
  // row m = q4 of x; the quad shares them through DPP).
  const int col = c0 + 8 * q4;
  const int8_t *wl = w + (col < N ? col : N - 8);
  const bf16_t *xl = a.x + static_cast<int64_t>(q4 < M ? q4 : 0) * K;
  const int nsteps = (K + kRWaves * kRRows - 1) / (kRWaves * kRRows);

  float acc[MR][8];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;

  u32x2 wr[kRDepth];
  uint32_t xr[kRDepth];
  // Step t covers rows (t * 8 + wave) * 16 .. +15; rows past K (including
  // the prefetches past the last step) read row 0 and count with x = 0.
  // Every step issues exactly two loads (8 bytes of W, then the lane's x),
  // in order, 16 steps ahead, as inline assembly with an explicit wait: when
  // a step is consumed the 30 loads of the 15 later steps may still be in
  // flight (loads return in issue order), a count the compiler's own waits
  // get wrong at the loop head.
#pragma unroll
  for (int u = 0; u < kRDepth; ++u) {
    const int row = (u * kRWaves + wv) * kRRows + rl;
    const int rc = row < K ? row : 0;
    wr[u] = load_w8(wl + static_cast<int64_t>(rc) * N);
    xr[u] = load_x2(xl + rc);
  }
  for (int t0 = 0; t0 < nsteps; t0 += kRDepth) {
#pragma unroll
    for (int u = 0; u < kRDepth; ++u) {
      asm volatile("s_waitcnt vmcnt(30)" : "+v"(wr[u]), "+v"(xr[u]) : : "memory");
      const u32x2 wv2 = wr[u];
      float xm[MR];
      quad_rows<MR>(xr[u], xm);
      if (((t0 + u) * kRWaves + wv) * kRRows + rl >= K) {
#pragma unroll
        for (int m = 0; m < MR; ++m) xm[m] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float wf = i8_at(wv2[j >> 2], j & 3);
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m][j] = fmaf(xm[m], wf, acc[m][j]);
      }
      const int row = ((t0 + u + kRDepth) * kRWaves + wv) * kRRows + rl;
      const int rc = row < K ? row : 0;
      wr[u] = load_w8(wl + static_cast<int64_t>(rc) * N);
      xr[u] = load_x2(xl + rc);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the unused prefetches

  // Sum over the wave's 16 row lanes (lanes with equal q4), then over waves.
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = acc[m][j];
      v += __shfl_xor(v, 4, kWave);
      v += __shfl_xor(v, 8, kWave);
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[m][j] = v;
    }
  if (l < 4) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wv][m][8 * q4 + j] = acc[m][j];
  }
  __syncthreads();
  if (tid < MR * kRBN) {
    const int m = tid / kRBN, c = tid % kRBN;
    if (m < M && c0 + c < N) {
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < kRWaves; ++u) sum += red[u][m][c];
      y[static_cast<int64_t>(m) * N + c0 + c] = f32_to_bf16(sum * sc[c0 + c]);
    }
  }
}

typedef void (*GemvKernel)(GemvArgs);

template <int MT>
GemvKernel pick_j(int J) {
  switch (J) {
    case 1: return gemv_int8_kernel<MT, 1>;
    case 2: return gemv_int8_kernel<MT, 2>;
    case 3: return gemv_int8_kernel<MT, 3>;
    case 4: return gemv_int8_kernel<MT, 4>;
    case 5: return gemv_int8_kernel<MT, 5>;
    case 6: return gemv_int8_kernel<MT, 6>;
    case 7: return gemv_int8_kernel<MT, 7>;
    default: return gemv_int8_kernel<MT, 8>;
  }
}

}  // namespace

GemvPlan gemv_plan(int64_t M, int K, int ncb) {
  GemvPlan p;
  p.rows = static_cast<int>(M < kMaxRows ? M : kMaxRows);
  p.mt = p.rows <= 16 ? 1 : 2;
  p.ncb = ncb;
  const size_t tickets = (static_cast<size_t>(ncb) * 4 + 255) / 256 * 256;
  if (p.rows <= kRMaxRows) {  // only the few-row kernel runs: no slices
    p.s = p.j = 1;
    p.ws_bytes = tickets;
    return p;
  }
  // Aim for about four (one row tile) or two (two tiles) workgroups per CU.
  const int target = p.mt == 1 ? 1024 : 512;
  int s_want = target / ncb;
  if (s_want < 1) s_want = 1;
  const int per = kWaves * kStepK;  // rows per slice per step of every wave
  int J = (K + per * s_want - 1) / (per * s_want);
  if (J < 1) J = 1;
  if (J > kMaxJ) J = kMaxJ;
  p.j = J;
  p.s = (K + per * J - 1) / (per * J);
  p.ws_bytes = tickets + (p.s > 1 ? static_cast<size_t>(ncb) * p.s * p.rows * kBN * 4 : 0);
  return p;
}

int gemv_column_blocks(int n, const int *N) {
  int ncb = 0;
  for (int p = 0; p < n; ++p) ncb += (N[p] + kBN - 1) / kBN;
  return ncb;
}

hipError_t launch_linear_int8_gemv(const void *x, int n, const int8_t *const *w,
                                   const float *const *scales, void *const *y, const int *N,
                                   int64_t M, int K, void *ws, hipStream_t stream) {
  const int ncb = gemv_column_blocks(n, N);
  const GemvPlan p = gemv_plan(M, K, ncb);
  const size_t tickets = (static_cast<size_t>(ncb) * 4 + 255) / 256 * 256;
  for (int64_t r0 = 0; r0 < M; r0 += kMaxRows) {
    GemvArgs a = {};
    const int rows = static_cast<int>(M - r0 < kMaxRows ? M - r0 : kMaxRows);
    const int bn = rows <= kRMaxRows ? kRBN : kBN;  // channels per workgroup
    a.x = static_cast<const bf16_t *>(x) + r0 * K;
    int nb = 0;
    for (int q = 0; q < n; ++q) {
      a.mat[q] = GemvMat{w[q], scales[q], static_cast<bf16_t *>(y[q]) + r0 * N[q], N[q], nb};
      nb += (N[q] + bn - 1) / bn;
    }
    a.nmat = n;
    a.M = rows;
    a.K = K;
    if (rows <= kRMaxRows) {
      a.S = 1;
      a.xcd = nb % 32 == 0;
      GemvKernel k = rows == 1 ? gemv_rows_kernel<1>
                   : rows == 2 ? gemv_rows_kernel<2>
                   : rows == 3 ? gemv_rows_kernel<3> : gemv_rows_kernel<4>;
      hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(nb)), dim3(kRThreads), 0, stream, a);
    } else {
      a.S = p.s;
      a.xcd = ncb % 8 == 0;
      a.cnt = static_cast<uint32_t *>(ws);
      a.part = reinterpret_cast<float *>(static_cast<char *>(ws) + tickets);
      const GemvKernel k = rows <= 16 ? pick_j<1>(p.j) : pick_j<2>(p.j);
      hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(ncb) * p.s), dim3(kThreads),
                         kWaves * rows * kBN * sizeof(float), stream, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace grok

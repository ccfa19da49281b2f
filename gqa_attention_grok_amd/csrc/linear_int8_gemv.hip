// int8-weight Linear for a few rows at a time (Grok-1 walkthrough, ch. 4
// "model.py close reading, part 1", §4.1 and §4.1.1): y = x @ (w * s) with
// x [M,K] bf16, w [K,N] int8, s [N] fp32, y [M,N] bf16, at most 32 rows per
// launch. In decoding each sequence contributes one row, so the product is a
// matrix-vector one and its time is the time to stream the int8 weights from
// HBM once (88 MB per layer for Grok-1's four attention projections).
//
// Packed weights. Read in their [K, N] order, a workgroup that owns a few
// output channels takes a short piece of every 6 KB row, and the DRAM pages
// are opened many times each: measured, that halves the achieved bandwidth.
// The weights are therefore repacked once (grok_linear_int8_pack, a pure
// permutation of the bytes) into 1 KB tiles of 64 rows x 16 channels, each
// tile already in the lane order of the B operand of v_mfma_f32_16x16x32_bf16
// for two 32-row steps: byte 16*l + 8*h + e of tile (j, i) is
//   W[64*i + 32*h + 8*(l / 16) + e][16*j + l % 16]     (zero past K or N),
// and the tiles of one 16-channel block j follow each other along K. A wave
// then reads 1 KB of contiguous memory per load instruction, and the 16 bytes
// a lane receives are its two B operands after widening (int8 is exact in
// bf16).
//
// Work split. A workgroup owns NB blocks of 16 channels and the whole K axis,
// so no partial sums leave it; its 8 waves take contiguous ranges of tiles,
// each with a ring of loads 6 to 16 steps deep. The A operand is 16 rows of x
// (row m = lane % 16, zero beyond M), read from LDS for up to 4 rows (x is
// copied there once per workgroup) and loaded with the weights otherwise.
// The 8 waves' sums meet in LDS, where the channel scale is applied and bf16
// written.
//
// Up to three matrices that share x (the query, key and value projections of
// §4.5.1) are computed in one launch: their workgroups are numbered one after
// another and each picks its matrix from its number.
#include "common.h"

namespace grok {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kTileRows = 64;   // rows of one packed tile
constexpr int kTileCols = 16;   // channels of one packed tile
constexpr int kTileBytes = kTileRows * kTileCols;
constexpr int kMaxRows = 32;    // rows of x per launch

struct GemvMat {
  const int8_t *w;  // packed
  const float *s;
  bf16_t *y;
  int N;
  int wg0;  // number of the matrix's first workgroup
};

struct GemvArgs {
  const bf16_t *x;
  GemvMat mat[3];
  int nmat;
  int M;   // rows of this launch, 1..32
  int K;
  int KP;  // tiles along K
};

__device__ __forceinline__ u32x4 load16(const void *p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

// The 8 int8 weights of one B operand (bytes of `lo`, `hi`) as exact bf16.
__device__ __forceinline__ float i8_at(uint32_t word, int b) {
  return static_cast<float>(static_cast<int8_t>((word >> (8 * b)) & 0xffu));
}
__device__ __forceinline__ uint32_t pack_hi(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = pack_hi(i8_at(lo, 0), i8_at(lo, 1));
  r[1] = pack_hi(i8_at(lo, 2), i8_at(lo, 3));
  r[2] = pack_hi(i8_at(hi, 0), i8_at(hi, 1));
  r[3] = pack_hi(i8_at(hi, 2), i8_at(hi, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// Pass registers filled by inline-assembly loads through empty asm statements
// placed right after a wait: their uses cannot move above it (volatile asm
// statements keep their order).
template <int NW, int NX>
__device__ __forceinline__ void tie_after_wait(u32x4 *w, u32x4 *x) {
#pragma unroll
  for (int v = 1; v < NW; ++v) asm volatile("" : "+v"(w[v]));
#pragma unroll
  for (int v = 0; v < NX; ++v) asm volatile("" : "+v"(x[v]));
}

// MT row tiles of 16 (M <= 16*MT), NB 16-channel blocks per workgroup, W
// waves, a ring of D steps (one step = one 64-row tile of each block, plus
// its x unless XL). With XL the M (<= 4) rows of x are first copied to LDS and
// the A operands read from there.
template <int MT, int NB, int W, int D, bool XL>
__global__ __launch_bounds__(W * kWave) void gemv_packed_kernel(GemvArgs a) {
  constexpr int kLoads = XL ? NB : NB + 2 * MT;  // ring loads per step
  static_assert((D - 1) * kLoads <= 63, "the wait count must fit vmcnt");
  static_assert(!XL || MT == 1, "x in LDS is for at most 4 rows");
  extern __shared__ f32x4 xs4[];  // XL: x rows [M][K] bf16
  __shared__ float red[W][XL ? 4 : kMaxRows][NB * kTileCols];
  const int tid = threadIdx.x;
  const int wv = tid / kWave, l = tid % kWave, g = l / 16, i16 = l % 16;
  const int M = a.M, K = a.K, KP = a.KP;

  const int b = blockIdx.x;
  const bool m1 = a.nmat > 1 && b >= a.mat[1].wg0;
  const bool m2 = a.nmat > 2 && b >= a.mat[2].wg0;
  const int8_t *w = m2 ? a.mat[2].w : (m1 ? a.mat[1].w : a.mat[0].w);
  const float *sc = m2 ? a.mat[2].s : (m1 ? a.mat[1].s : a.mat[0].s);
  bf16_t *y = m2 ? a.mat[2].y : (m1 ? a.mat[1].y : a.mat[0].y);
  const int N = m2 ? a.mat[2].N : (m1 ? a.mat[1].N : a.mat[0].N);
  const int j0 = (b - (m2 ? a.mat[2].wg0 : (m1 ? a.mat[1].wg0 : a.mat[0].wg0))) * NB;
  const int NP = (N + kTileCols - 1) / kTileCols;

  // This wave's tiles: [i0, i1) of every block; blocks past NP re-read block j0.
  const int i0 = static_cast<int>(static_cast<int64_t>(KP) * wv / W);
  const int i1 = static_cast<int>(static_cast<int64_t>(KP) * (wv + 1) / W);
  const int8_t *wb[NB];
#pragma unroll
  for (int v = 0; v < NB; ++v)
    wb[v] = w + (static_cast<int64_t>(j0 + v < NP ? j0 + v : j0) * KP) * kTileBytes + 16 * l;
  // x rows of this lane (clamped into x; rows >= M are zeroed when consumed)
  const bf16_t *xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xr[t] = a.x + static_cast<int64_t>(16 * t + i16 < M ? 16 * t + i16 : 0) * K;

  f32x4 acc[NB][MT];
#pragma unroll
  for (int v = 0; v < NB; ++v)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[v][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // With XL: x is copied to LDS with loads issued ahead of the ring's, so the
  // wait below the ring's prologue covers them.
  constexpr int kStage = XL ? 4 : 1;  // 16-byte x pieces per thread (M*K <= 4*W*64*8)
  u32x4 st[kStage];
  const int nst = XL ? M * K / 8 : 0;
  if constexpr (XL) {
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      const int c = tid + r * W * kWave;
      st[r] = load16(a.x + 8 * static_cast<int64_t>(c < nst ? c : 0));
    }
  }

  // Ring of D steps, loads as inline assembly with an explicit wait: when a
  // step is consumed, the (D-1) * kLoads loads of the later steps may still be
  // in flight (loads return in issue order). Steps past the wave's range
  // re-read its last tile (a cache hit) and are not consumed.
  u32x4 wr[D][NB];
  u32x4 xa[XL ? 1 : D][MT][2];
  auto issue = [&](int slot, int i) {
    const int ic = i < i1 ? i : i1 - 1;
#pragma unroll
    for (int v = 0; v < NB; ++v) wr[slot][v] = load16(wb[v] + static_cast<int64_t>(ic) * kTileBytes);
    if constexpr (!XL) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k = kTileRows * ic + 32 * h + 8 * g;
          xa[slot][t][h] = load16(xr[t] + (k < K ? k : 0));
        }
    }
  };
  const bool busy = i1 > i0;
  if (busy) {
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u, i0 + u);
  }
  if constexpr (XL) {
    if (busy) {
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(D * kLoads) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
#pragma unroll
    for (int r = 0; r < kStage; ++r) asm volatile("" : "+v"(st[r]));  // uses stay below the wait
    bf16_t *xs = reinterpret_cast<bf16_t *>(xs4);
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      const int c = tid + r * W * kWave;
      if (c < nst) *reinterpret_cast<u32x4 *>(xs + 8 * c) = st[r];
    }
    __syncthreads();
  }
  if (busy) {
    for (int c0 = i0; c0 < i1; c0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        asm volatile("s_waitcnt vmcnt(%1)" : "+v"(wr[u][0]) : "n"((D - 1) * kLoads) : "memory");
        tie_after_wait<NB, XL ? 0 : 2 * MT>(&wr[u][0], &xa[XL ? 0 : u][0][0]);
        __builtin_amdgcn_sched_barrier(0);
        const int i = c0 + u;
        if (i < i1) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int k = kTileRows * i + 32 * h + 8 * g;
            const bool kok = k < K;
            bf16x8 A[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
              const bool ok = kok && 16 * t + i16 < M;
              u32x4 xv;
              if constexpr (XL) {
                const bf16_t *xs = reinterpret_cast<const bf16_t *>(xs4);
                xv = *reinterpret_cast<const u32x4 *>(xs + static_cast<int64_t>(i16 < M ? i16 : 0) * K +
                                                      (kok ? k : 0));
              } else {
                xv = xa[u][t][h];
              }
              A[t] = __builtin_bit_cast(bf16x8, ok ? xv : u32x4{0u, 0u, 0u, 0u});
            }
#pragma unroll
            for (int v = 0; v < NB; ++v) {
              const bf16x8 B = widen8(wr[u][v][2 * h], wr[u][v][2 * h + 1]);
#pragma unroll
              for (int t = 0; t < MT; ++t)
                acc[v][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[t], B, acc[v][t], 0, 0, 0);
            }
          }
        }
        issue(u, c0 + u + D);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the unused prefetches
  }

  // acc[v][t][e] = sum for x row 16t + 4g + e, channel 16*(j0+v) + i16.
#pragma unroll
  for (int v = 0; v < NB; ++v)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 16 * t + 4 * g + e;
        if (m < M) red[wv][m][kTileCols * v + i16] = acc[v][t][e];
      }
  __syncthreads();
  for (int q = tid; q < M * NB * kTileCols; q += W * kWave) {
    const int m = q / (NB * kTileCols), c = q % (NB * kTileCols);
    const int n = kTileCols * j0 + c;
    if (n >= N) continue;
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < W; ++u) sum += red[u][m][c];
    y[static_cast<int64_t>(m) * N + n] = f32_to_bf16(sum * sc[n]);
  }
}

// Packing: one thread per 16-byte lane chunk of a tile.
__global__ __launch_bounds__(256) void pack_kernel(const int8_t *w, int8_t *wp, int K, int N, int KP,
                                                   int64_t chunks) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int l = static_cast<int>(c % 64);
  const int64_t tile = c / 64;
  const int i = static_cast<int>(tile % KP);
  const int j = static_cast<int>(tile / KP);
  const int n = kTileCols * j + l % 16;
  uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = kTileRows * i + 32 * h + 8 * (l / 16) + e;
      const uint32_t v = (k < K && n < N) ? static_cast<uint8_t>(w[static_cast<int64_t>(k) * N + n]) : 0u;
      word[2 * h + e / 4] |= v << (8 * (e % 4));
    }
  *reinterpret_cast<u32x4 *>(wp + c * 16) = u32x4{word[0], word[1], word[2], word[3]};
}

typedef void (*GemvKernel)(GemvArgs);

}  // namespace

size_t gemv_packed_bytes(int K, int N) {
  return static_cast<size_t>((K + kTileRows - 1) / kTileRows) * ((N + kTileCols - 1) / kTileCols) * kTileBytes;
}

hipError_t launch_linear_int8_pack(const int8_t *w, int8_t *wp, int K, int N, hipStream_t stream) {
  const int KP = (K + kTileRows - 1) / kTileRows;
  const int64_t chunks = static_cast<int64_t>(gemv_packed_bytes(K, N)) / 16;
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, w, wp, K, N, KP,
                     chunks);
  return hipGetLastError();
}

hipError_t launch_linear_int8_gemv(const void *x, int n, const int8_t *const *w,
                                   const float *const *scales, void *const *y, const int *N,
                                   int64_t M, int K, hipStream_t stream) {
  for (int64_t r0 = 0; r0 < M; r0 += kMaxRows) {
    const int rows = static_cast<int>(M - r0 < kMaxRows ? M - r0 : kMaxRows);
    // Up to 4 rows: 16 channels per workgroup, x staged in LDS (when it fits
    // the staging registers, 4 x 16 bytes per thread), 16 steps in flight;
    // up to 16 rows: 32 channels, x from the ring; more: two row tiles.
    int NB = 2;
    bool xl = false;
    GemvKernel k = gemv_packed_kernel<1, 2, kWaves, 8, false>;
    if (rows > 16) {
      k = gemv_packed_kernel<2, 2, kWaves, 6, false>;
    } else if (rows <= 4 && static_cast<int64_t>(rows) * K <= 4 * kThreads * 8) {
      xl = true;
      NB = 1;
      k = gemv_packed_kernel<1, 1, kWaves, 16, true>;
    }
    GemvArgs a = {};
    a.x = static_cast<const bf16_t *>(x) + r0 * K;
    int wg = 0;
    for (int q = 0; q < n; ++q) {
      a.mat[q] = GemvMat{w[q], scales[q], static_cast<bf16_t *>(y[q]) + r0 * N[q], N[q], wg};
      const int np = (N[q] + kTileCols - 1) / kTileCols;
      wg += (np + NB - 1) / NB;
    }
    a.nmat = n;
    a.M = rows;
    a.K = K;
    a.KP = (K + kTileRows - 1) / kTileRows;
    const size_t lds = xl ? static_cast<size_t>(rows) * K * 2 : 0;
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(wg)), dim3(kThreads), lds, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace grok

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

// The product of one wave: tiles [i0, i1) of NB 16-channel blocks (wb[v]
// points at this lane's 16 bytes of the block's first tile) against MT row
// tiles of x, accumulated into acc[v][t] (lane: x row 16t + 4g + e, channel
// i16 of block v). With XL the A operands come from the copy of x in LDS,
// otherwise they are loaded with the weights.
//
// The loads form a ring of D steps, as inline assembly with an explicit wait:
// when a step is consumed, the (D-1) * kLoads loads of the later steps may
// still be in flight (loads return in issue order; the compiler's own waits
// get this count wrong at the loop head). Steps past the range re-read its
// last tile (a cache hit) and are not consumed.
template <int MT, int NB, int D, bool XL>
struct TileRing {
  static constexpr int kLoads = XL ? NB : NB + 2 * MT;  // load instructions per step
  static_assert((D - 1) * kLoads <= 63, "the wait count must fit vmcnt");
  u32x4 wr[D][NB];
  u32x4 xa[XL ? 1 : D][MT][2];
  const int8_t *wb[NB];
  const bf16_t *xr[MT];  // this lane's x rows (clamped into x; zeroed past M when used)
  int i0, i1, K, M, g, i16;

  __device__ __forceinline__ bool busy() const { return i1 > i0; }

  __device__ __forceinline__ void issue(int slot, int i) {
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
  }

  __device__ __forceinline__ void prologue() {
    if (busy()) {
#pragma unroll
      for (int u = 0; u < D; ++u) issue(u, i0 + u);
    }
  }

  __device__ __forceinline__ void run(const bf16_t *xs, f32x4 (&acc)[NB][MT]) {
#pragma unroll
    for (int v = 0; v < NB; ++v)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[v][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!busy()) return;
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
              if constexpr (XL)
                xv = *reinterpret_cast<const u32x4 *>(xs + static_cast<int64_t>(i16 < M ? i16 : 0) * K + (kok ? k : 0));
              else
                xv = xa[u][t][h];
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
    // Their registers pass through empty statements after the wait: the last
    // D prefetches are never read, and without a use the compiler could hand
    // their registers to other values while the loads are still in flight.
#pragma unroll
    for (int u = 0; u < D; ++u) {
#pragma unroll
      for (int v = 0; v < NB; ++v) asm volatile("" : "+v"(wr[u][v]));
      if constexpr (!XL) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(xa[u][t][h]));
      }
    }
  }
};

// Copy of the M rows of x ([M][K] bf16, M*K <= kStageElems) into LDS, loaded
// ahead of the ring's prologue and written once the prologue is issued. With
// kNorm the rows are first normalised as the RMSNorm entry point does
// (n = bf16(gamma * (x * r)), r = rsqrt(mean(x^2) + eps), fp32 inside).
constexpr int kStage = 8;  // 16-byte pieces of x per thread
constexpr int kStageElems = kStage * kThreads * 8;

struct XStage {
  u32x4 st[kStage];
  __device__ __forceinline__ void load(const bf16_t *x, int n8) {
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      const int c = threadIdx.x + r * kThreads;
      st[r] = load16(x + 8 * static_cast<int64_t>(c < n8 ? c : 0));
    }
  }
  // `left` ring loads issued after these may stay in flight.
  template <int kLeftBusy, bool kNorm>
  __device__ __forceinline__ void store(bf16_t *xs, bool busy, int M, int K, const float *gamma,
                                        float eps, float *red /* [kWaves][4] */) {
    if (busy) {
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(kLeftBusy) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
#pragma unroll
    for (int r = 0; r < kStage; ++r) asm volatile("" : "+v"(st[r]));  // uses stay below the wait
    const int n8 = M * K / 8;
    if constexpr (kNorm) {
      // per-row sums of squares (a piece lies in one row: K % 8 == 0)
      float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < kStage; ++r) {
        const int c = threadIdx.x + r * kThreads;
        if (c < n8) {
          const int m = 8 * c / K;
          float part = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float lo = lo_bf16(st[r][q]), hi = hi_bf16(st[r][q]);
            part += lo * lo;
            part += hi * hi;
          }
#pragma unroll
          for (int mm = 0; mm < 4; ++mm)
            if (m == mm) ss[mm] += part;
        }
      }
      const int wv = threadIdx.x / kWave;
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const float v = wave_sum(ss[mm]);
        if ((threadIdx.x & (kWave - 1)) == 0) red[wv * 4 + mm] = v;
      }
      __syncthreads();
      float rr[4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        float t = 0.f;
#pragma unroll
        for (int u = 0; u < kWaves; ++u) t += red[u * 4 + mm];
        rr[mm] = rsqrtf(t / static_cast<float>(K) + eps);
      }
#pragma unroll
      for (int r = 0; r < kStage; ++r) {
        const int c = threadIdx.x + r * kThreads;
        if (c < n8) {
          const int m = 8 * c / K;
          const int k0 = 8 * c - m * K;
          const float rm = m == 0 ? rr[0] : m == 1 ? rr[1] : m == 2 ? rr[2] : rr[3];
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float lo = lo_bf16(st[r][q]) * rm, hi = hi_bf16(st[r][q]) * rm;
            if (gamma) {
              lo = gamma[k0 + 2 * q] * lo;
              hi = gamma[k0 + 2 * q + 1] * hi;
            }
            o[q] = pack_bf16x2(lo, hi);
          }
          *reinterpret_cast<u32x4 *>(xs + 8 * c) = o;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < kStage; ++r) {
        const int c = threadIdx.x + r * kThreads;
        if (c < n8) *reinterpret_cast<u32x4 *>(xs + 8 * c) = st[r];
      }
    }
    __syncthreads();
  }
};

// Matrix of workgroup b (matrices' workgroups are numbered one after another).
struct MatSel {
  const int8_t *w;
  const float *s;
  bf16_t *y;
  int N, lw, p;
  __device__ __forceinline__ MatSel(const GemvArgs &a, int b) {
    const bool m1 = a.nmat > 1 && b >= a.mat[1].wg0;
    const bool m2 = a.nmat > 2 && b >= a.mat[2].wg0;
    p = m2 ? 2 : (m1 ? 1 : 0);
    w = m2 ? a.mat[2].w : (m1 ? a.mat[1].w : a.mat[0].w);
    s = m2 ? a.mat[2].s : (m1 ? a.mat[1].s : a.mat[0].s);
    y = m2 ? a.mat[2].y : (m1 ? a.mat[1].y : a.mat[0].y);
    N = m2 ? a.mat[2].N : (m1 ? a.mat[1].N : a.mat[0].N);
    lw = b - (m2 ? a.mat[2].wg0 : (m1 ? a.mat[1].wg0 : a.mat[0].wg0));
  }
};

// MT row tiles of 16 (M <= 16*MT), NB consecutive 16-channel blocks per
// workgroup, a ring of D steps; XL: x (at most 4 rows) copied to LDS first.
template <int MT, int NB, int D, bool XL>
__global__ __launch_bounds__(kThreads) void gemv_packed_kernel(GemvArgs a) {
  static_assert(!XL || MT == 1, "x in LDS is for at most 4 rows");
  extern __shared__ f32x4 xs4[];  // XL: x rows [M][K] bf16
  __shared__ float red[kWaves][XL ? 4 : kMaxRows][NB * kTileCols];
  const int tid = threadIdx.x;
  const int wv = tid / kWave, l = tid % kWave, g = l / 16, i16 = l % 16;
  const int M = a.M, K = a.K, KP = a.KP;
  const MatSel ms(a, blockIdx.x);
  const int j0 = ms.lw * NB;
  const int NP = (ms.N + kTileCols - 1) / kTileCols;

  TileRing<MT, NB, D, XL> ring;
  ring.i0 = static_cast<int>(static_cast<int64_t>(KP) * wv / kWaves);
  ring.i1 = static_cast<int>(static_cast<int64_t>(KP) * (wv + 1) / kWaves);
  ring.K = K;
  ring.M = M;
  ring.g = g;
  ring.i16 = i16;
#pragma unroll
  for (int v = 0; v < NB; ++v)  // blocks past NP re-read block j0
    ring.wb[v] = ms.w + (static_cast<int64_t>(j0 + v < NP ? j0 + v : j0) * KP) * kTileBytes + 16 * l;
#pragma unroll
  for (int t = 0; t < MT; ++t) ring.xr[t] = a.x + static_cast<int64_t>(16 * t + i16 < M ? 16 * t + i16 : 0) * K;

  XStage xst;
  if constexpr (XL) xst.load(a.x, M * K / 8);
  ring.prologue();
  bf16_t *xs = reinterpret_cast<bf16_t *>(xs4);
  if constexpr (XL)
    xst.template store<D * TileRing<MT, NB, D, XL>::kLoads, false>(xs, ring.busy(), M, K, nullptr, 0.f,
                                                                    &red[0][0][0]);
  f32x4 acc[NB][MT];
  ring.run(xs, acc);

  __syncthreads();  // red[] may have held the staging sums
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
  for (int q = tid; q < M * NB * kTileCols; q += kThreads) {
    const int m = q / (NB * kTileCols), c = q % (NB * kTileCols);
    const int n = kTileCols * j0 + c;
    if (n >= ms.N) continue;
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) sum += red[u][m][c];
    ms.y[static_cast<int64_t>(m) * ms.N + n] = f32_to_bf16(sum * ms.s[n]);
  }
}

// Decode front half: Q|K|V projections of one token per sequence (head size
// 128), with RoPE of q and k at position step[b] and the k, v rows written to
// cache slot step[b] (ch. 4 §4.4, §4.5.1), optionally normalising x first
// (kNorm; x then in LDS, at most 4 rows). A workgroup owns the two blocks of
// 16 channels that RoPE pairs (channels c and c + 64 of a head), so that the
// rotation happens in its epilogue. The arithmetic after the fp32 sums is the
// one of the unfused calls: the projection is rounded to bf16, rotated in fp32
// with the same phase and pinned operations, and rounded again.
struct QkvArgs {
  GemvArgs g;    // mat[0] = q (y = q_out), mat[1] = k, mat[2] = v (y unused)
  bf16_t *kc, *vc;
  const int32_t *step;
  int32_t *new_step, *status;
  const float *gamma;
  float eps;
  int Tmax, Hkv;
  RopeFreqs f;
};

__device__ __forceinline__ void rope_pair_at(int pos, float inv, float x1, float x2, float &o1, float &o2) {
  float s, c;
  rope_phase(pos, inv, s, c);
  rope_rotate(x1, x2, c, s, o1, o2);
}

template <int MT, int D, bool XL, bool kNorm>
__global__ __launch_bounds__(kThreads) void decode_qkv_kernel(QkvArgs qa) {
  constexpr int NB = 2;
  static_assert(!XL || MT == 1, "x in LDS is for at most 4 rows");
  static_assert(XL || !kNorm, "the norm needs x in LDS");
  extern __shared__ f32x4 xs4[];
  __shared__ float red[kWaves][XL ? 4 : kMaxRows][NB * kTileCols];
  const GemvArgs &a = qa.g;
  const int tid = threadIdx.x;
  const int wv = tid / kWave, l = tid % kWave, g = l / 16, i16 = l % 16;
  const int M = a.M, K = a.K, KP = a.KP;
  const MatSel ms(a, blockIdx.x);
  // blocks (jA, jA + 4) with jA % 8 < 4: channels c and c + 64 of one head
  const int jA = 8 * (ms.lw / 4) + ms.lw % 4;

  TileRing<MT, NB, D, XL> ring;
  ring.i0 = static_cast<int>(static_cast<int64_t>(KP) * wv / kWaves);
  ring.i1 = static_cast<int>(static_cast<int64_t>(KP) * (wv + 1) / kWaves);
  ring.K = K;
  ring.M = M;
  ring.g = g;
  ring.i16 = i16;
  ring.wb[0] = ms.w + (static_cast<int64_t>(jA) * KP) * kTileBytes + 16 * l;
  ring.wb[1] = ms.w + (static_cast<int64_t>(jA + 4) * KP) * kTileBytes + 16 * l;
#pragma unroll
  for (int t = 0; t < MT; ++t) ring.xr[t] = a.x + static_cast<int64_t>(16 * t + i16 < M ? 16 * t + i16 : 0) * K;

  XStage xst;
  if constexpr (XL) xst.load(a.x, M * K / 8);
  ring.prologue();
  bf16_t *xs = reinterpret_cast<bf16_t *>(xs4);
  if constexpr (XL)
    xst.template store<D * TileRing<MT, NB, D, XL>::kLoads, kNorm>(xs, ring.busy(), M, K, qa.gamma, qa.eps,
                                                                     &red[0][0][0]);
  f32x4 acc[NB][MT];
  ring.run(xs, acc);

  __syncthreads();  // red[] may have held the staging sums
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
  for (int q = tid; q < M * kTileCols; q += kThreads) {
    const int m = q / kTileCols, c = q % kTileCols;
    const int nA = kTileCols * jA + c, nB = nA + 64;
    float sA = 0.f, sB = 0.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      sA += red[u][m][c];
      sB += red[u][m][kTileCols + c];
    }
    // the projection as the unfused call hands it on (bf16)
    const float yA = bf16_to_f32(f32_to_bf16(sA * ms.s[nA]));
    const float yB = bf16_to_f32(f32_to_bf16(sB * ms.s[nB]));
    const int pos = qa.step[m];
    const bool ok = pos >= 0 && pos < qa.Tmax;
    const int h = nA / 128, i = nA % 128;  // i < 64: nB is its RoPE partner
    if (ms.p == 0) {  // q: rotated in place of the unfused append, unrotated if skipped
      float oA = yA, oB = yB;
      if (ok) rope_pair_at(pos, qa.f.inv[i], yA, yB, oA, oB);
      ms.y[static_cast<int64_t>(m) * ms.N + nA] = f32_to_bf16(oA);
      ms.y[static_cast<int64_t>(m) * ms.N + nB] = f32_to_bf16(oB);
    } else if (ok) {
      bf16_t *dst = (ms.p == 1 ? qa.kc : qa.vc) + ((static_cast<int64_t>(m) * qa.Tmax + pos) * qa.Hkv + h) * 128;
      float oA = yA, oB = yB;
      if (ms.p == 1) rope_pair_at(pos, qa.f.inv[i], yA, yB, oA, oB);
      dst[i] = f32_to_bf16(oA);
      dst[i + 64] = f32_to_bf16(oB);
    }
  }
  if (blockIdx.x == 0 && tid < M) {
    const int pos = qa.step[tid];
    const bool ok = pos >= 0 && pos < qa.Tmax;
    if (qa.new_step) qa.new_step[tid] = ok ? pos + 1 : pos;
    if (!ok && qa.status) *qa.status = GROK_ERANGE;
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
    // the staging registers, 8 x 16 bytes per thread), 16 steps in flight;
    // up to 16 rows: 32 channels, x from the ring; more: two row tiles.
    int NB = 2;
    bool xl = false;
    GemvKernel k = gemv_packed_kernel<1, 2, 8, false>;
    if (rows > 16) {
      k = gemv_packed_kernel<2, 2, 6, false>;
    } else if (rows <= 4 && static_cast<int64_t>(rows) * K <= kStageElems) {
      xl = true;
      NB = 1;
      k = gemv_packed_kernel<1, 1, 16, true>;
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

hipError_t launch_decode_qkv(const void *x, const float *gamma, float eps, bool prenorm,
                             const int8_t *const *w, const float *const *scales, void *q_out,
                             void *kc, void *vc, const int32_t *step, int32_t *new_step,
                             int32_t *status, int B, int d, int Tmax, int Hq, int Hkv,
                             const RopeFreqs &f, hipStream_t stream) {
  for (int r0 = 0; r0 < B; r0 += kMaxRows) {
    const int rows = B - r0 < kMaxRows ? B - r0 : kMaxRows;
    QkvArgs qa = {};
    GemvArgs &a = qa.g;
    a.x = static_cast<const bf16_t *>(x) + static_cast<int64_t>(r0) * d;
    const int Ns[3] = {Hq * 128, Hkv * 128, Hkv * 128};
    int wg = 0;
    for (int q = 0; q < 3; ++q) {
      bf16_t *yq = q == 0 ? static_cast<bf16_t *>(q_out) + static_cast<int64_t>(r0) * Ns[0] : nullptr;
      a.mat[q] = GemvMat{w[q], scales[q], yq, Ns[q], wg};
      wg += Ns[q] / 32;  // pairs of 16-channel blocks
    }
    a.nmat = 3;
    a.M = rows;
    a.K = d;
    a.KP = (d + kTileRows - 1) / kTileRows;
    const int64_t slot0 = static_cast<int64_t>(r0) * Tmax * Hkv * 128;
    qa.kc = static_cast<bf16_t *>(kc) + slot0;
    qa.vc = static_cast<bf16_t *>(vc) + slot0;
    qa.step = step + r0;
    qa.new_step = new_step ? new_step + r0 : nullptr;
    qa.status = status;
    qa.gamma = gamma;
    qa.eps = eps;
    qa.Tmax = Tmax;
    qa.Hkv = Hkv;
    qa.f = f;
    const bool xl = rows <= 4 && static_cast<int64_t>(rows) * d <= kStageElems;
    if (prenorm && !xl) return hipErrorInvalidValue;  // validated by the caller
    void (*k)(QkvArgs);
    if (xl)
      k = prenorm ? decode_qkv_kernel<1, 16, true, true> : decode_qkv_kernel<1, 16, true, false>;
    else if (rows <= 16)
      k = decode_qkv_kernel<1, 8, false, false>;
    else
      k = decode_qkv_kernel<2, 6, false, false>;
    const size_t lds = xl ? static_cast<size_t>(rows) * d * 2 : 0;
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(wg)), dim3(kThreads), lds, stream, qa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int decode_qkv_max_prenorm_rows(int d) { return d > 0 ? (kStageElems / d < 4 ? kStageElems / d : 4) : 0; }

}  // namespace grok

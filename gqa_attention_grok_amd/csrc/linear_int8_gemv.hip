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
// last tile (a cache hit) and are not consumed. A wave with no tiles (fewer
// tiles than waves) issues and waits for its loads all the same, on tile 0:
// no load or wait depends on a branch, so the compiler cannot give the
// registers of a load still in flight to another value on some path.
template <int MT, int NB, int D, bool XL>
struct TileRing {
  static constexpr int kLoads = XL ? NB : NB + 2 * MT;  // load instructions per step
  static_assert((D - 1) * kLoads <= 63, "the wait count must fit vmcnt");
  u32x4 wr[D][NB];
  u32x4 xa[XL ? 1 : D][MT][2];
  const int8_t *wb[NB];
  const bf16_t *xr[MT];  // this lane's x rows (clamped into x; zeroed past M when used)
  int i0, i1, K, M, g, i16;

  __device__ __forceinline__ void issue(int slot, int i) {
    const int il = i < i1 ? i : i1 - 1;
    const int ic = il > 0 ? il : 0;
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
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u, i0 + u);
  }

  __device__ __forceinline__ void run(const bf16_t *xs, f32x4 (&acc)[NB][MT]) {
#pragma unroll
    for (int v = 0; v < NB; ++v)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[v][t] = f32x4{0.f, 0.f, 0.f, 0.f};
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
  // The kLeft ring loads issued after these may stay in flight.
  template <int kLeft, bool kNorm>
  __device__ __forceinline__ void store(bf16_t *xs, int M, int K, const float *gamma, float eps,
                                        float *red /* [kWaves][4] */) {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(kLeft) : "memory");
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
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid % kWave, g = l / 16, i16 = l % 16;
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
    xst.template store<D * TileRing<MT, NB, D, XL>::kLoads, false>(xs, M, K, nullptr, 0.f,
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
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid % kWave, g = l / 16, i16 = l % 16;
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
    xst.template store<D * TileRing<MT, NB, D, XL>::kLoads, kNorm>(xs, M, K, qa.gamma, qa.eps,
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

// Output projection with the sandwich post-norm and the residual add in one
// launch (ch. 6 "model.py close reading, part 3", §6.3.1: h = x + norm(o),
// o = attn @ (Wo * s), ch. 4 §4.1), for at most 4 rows held in LDS:
//   o = bf16(attn @ (w * s)),  r_m = rsqrt(mean_n(o_mn^2) + eps),
//   y = bf16(res + bf16(gamma * (o * r_m)))
// with the roundings of grok_linear_int8_gemv followed by grok_rmsnorm. The
// norm needs every channel of a row, and each workgroup owns 16 channels, so
// the workgroups meet through memory: each writes its bf16 o values and its
// rows' sums of squares with device-coherent stores, waits until they are
// written, and counts itself in with a device-scope atomic add; the last one
// to arrive reads everything back with device-coherent loads, sums the
// squares in workgroup order (so the result does not depend on the arrival
// order), normalises, adds the residual and writes y. It also puts the
// counter back to zero, so each call leaves it as it found it.
struct OutNormArgs {
  GemvArgs g;          // mat[0]: the packed Wo, y = the o buffer of the workspace
  const bf16_t *res;   // [M][N]
  bf16_t *out;         // [M][N]
  const float *gamma;  // [N] or NULL (unit scale)
  float eps;
  float *ss;           // [workgroups][4] sums of squares of o
  uint32_t *count;     // arrivals; zero between calls
};

__device__ __forceinline__ uint32_t coherent_load(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kOutPieces = 6;  // 16-byte pieces of o per thread held in registers (4 rows of 6144)

__global__ __launch_bounds__(kThreads) void gemv_out_norm_kernel(OutNormArgs na) {
  constexpr int MT = 1, NB = 1, D = 16;
  extern __shared__ f32x4 xs4[];  // attn rows [M][K] bf16
  __shared__ float red[kWaves][4][kTileCols];
  __shared__ float rsum[kWaves][4];
  __shared__ int last;
  const GemvArgs &a = na.g;
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid % kWave, g = l / 16, i16 = l % 16;
  const int M = a.M, K = a.K, KP = a.KP, N = a.mat[0].N;
  const int j0 = blockIdx.x;

  TileRing<MT, NB, D, true> ring;
  ring.i0 = static_cast<int>(static_cast<int64_t>(KP) * wv / kWaves);
  ring.i1 = static_cast<int>(static_cast<int64_t>(KP) * (wv + 1) / kWaves);
  ring.K = K;
  ring.M = M;
  ring.g = g;
  ring.i16 = i16;
  ring.wb[0] = a.mat[0].w + (static_cast<int64_t>(j0) * KP) * kTileBytes + 16 * l;
  ring.xr[0] = a.x;
  XStage xst;
  xst.load(a.x, M * K / 8);
  ring.prologue();
  bf16_t *xs = reinterpret_cast<bf16_t *>(xs4);
  xst.template store<D * TileRing<MT, NB, D, true>::kLoads, false>(xs, M, K, nullptr, 0.f,
                                                                    &red[0][0][0]);
  f32x4 acc[NB][MT];
  ring.run(xs, acc);

  __syncthreads();  // red[] may have held the staging sums
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (4 * g + e < M) red[wv][4 * g + e][i16] = acc[0][0][e];
  __syncthreads();
  // wave 0, lane 16m + c: channel 16*j0 + c of row m
  if (wv == 0) {
    const int m = g, n = kTileCols * j0 + i16;
    float sq = 0.f;
    if (m < M && n < N) {
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < kWaves; ++u) sum += red[u][m][i16];
      const bf16_t o = f32_to_bf16(sum * a.mat[0].s[n]);
      __hip_atomic_store(a.mat[0].y + static_cast<int64_t>(m) * N + n, o, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      const float of = bf16_to_f32(o);
      sq = of * of;
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, kWave);
    if (i16 == 0 && m < M)
      __hip_atomic_store(na.ss + 4 * j0 + m, sq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are written
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(na.count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!last) return;

  // The last workgroup: every o value and sum of squares has been written.
  // Its loads all go out before the first use (one memory round trip): the
  // thread's pieces of o, the residual and gamma, then the sums of squares.
  if (tid == 0) __hip_atomic_store(na.count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int n8 = M * N / 8;  // 8 values (16 bytes) per piece; a piece lies in one row (N % 8 == 0)
  u32x4 ow[kOutPieces], xw[kOutPieces];
#pragma unroll
  for (int u = 0; u < kOutPieces; ++u) {
    const int c = tid + u * kThreads;
    if (c < n8) {
      const uint32_t *op = reinterpret_cast<const uint32_t *>(a.mat[0].y + 8 * static_cast<int64_t>(c));
      ow[u] = u32x4{coherent_load(op), coherent_load(op + 1), coherent_load(op + 2), coherent_load(op + 3)};
      xw[u] = *reinterpret_cast<const u32x4 *>(na.res + 8 * static_cast<int64_t>(c));
    }
  }
  float part[4] = {0.f, 0.f, 0.f, 0.f};
  for (int w = tid; w < static_cast<int>(gridDim.x); w += kThreads)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (m < M) part[m] += __uint_as_float(coherent_load(reinterpret_cast<const uint32_t *>(na.ss + 4 * w + m)));
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float v = wave_sum(part[m]);
    if (l == 0) rsum[wv][m] = v;
  }
  __syncthreads();
  float r[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) t += rsum[u][m];
    r[m] = rsqrtf(t / static_cast<float>(N) + na.eps);
  }
  auto finish = [&](int c, const u32x4 &o4, const u32x4 &x4) {
    const int m = 8 * c / N, n0 = 8 * c - m * N;
    const float rm = m == 0 ? r[0] : m == 1 ? r[1] : m == 2 ? r[2] : r[3];
    u32x4 yw;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f0 = lo_bf16(o4[q]) * rm, f1 = hi_bf16(o4[q]) * rm;
      if (na.gamma) {
        f0 = na.gamma[n0 + 2 * q] * f0;
        f1 = na.gamma[n0 + 2 * q + 1] * f1;
      }
      f0 = lo_bf16(x4[q]) + bf16_to_f32(f32_to_bf16(f0));
      f1 = hi_bf16(x4[q]) + bf16_to_f32(f32_to_bf16(f1));
      yw[q] = pack_bf16x2(f0, f1);
    }
    *reinterpret_cast<u32x4 *>(na.out + 8 * static_cast<int64_t>(c)) = yw;
  };
#pragma unroll
  for (int u = 0; u < kOutPieces; ++u) {
    const int c = tid + u * kThreads;
    if (c < n8) finish(c, ow[u], xw[u]);
  }
  for (int c = tid + kOutPieces * kThreads; c < n8; c += kThreads) {  // rows wider than the registers hold
    const uint32_t *op = reinterpret_cast<const uint32_t *>(a.mat[0].y + 8 * static_cast<int64_t>(c));
    finish(c, u32x4{coherent_load(op), coherent_load(op + 1), coherent_load(op + 2), coherent_load(op + 3)},
           *reinterpret_cast<const u32x4 *>(na.res + 8 * static_cast<int64_t>(c)));
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

size_t out_norm_workspace_bytes(int64_t M, int N) {
  const size_t nwg = static_cast<size_t>((N + kTileCols - 1) / kTileCols);
  const size_t ss = (nwg * 4 * sizeof(float) + 255) / 256 * 256;
  return 256 + ss + static_cast<size_t>(M) * N * 2;
}

int out_norm_max_fused_rows(int K) { return K > 0 ? (kStageElems / K < 4 ? kStageElems / K : 4) : 0; }

hipError_t launch_out_norm(const void *x, const int8_t *w, const float *scale, const float *gamma, float eps,
                           const void *res, void *y, void *ws, int64_t M, int K, int N, hipStream_t stream) {
  unsigned char *wsb = static_cast<unsigned char *>(ws);
  const size_t nwg = static_cast<size_t>((N + kTileCols - 1) / kTileCols);
  uint32_t *count = reinterpret_cast<uint32_t *>(wsb);
  float *ss = reinterpret_cast<float *>(wsb + 256);
  bf16_t *o = reinterpret_cast<bf16_t *>(wsb + 256 + (nwg * 4 * sizeof(float) + 255) / 256 * 256);
  if (M > out_norm_max_fused_rows(K)) {
    // more rows than the fused form keeps on chip: the projection, then the norm
    const int8_t *wp[1] = {w};
    const float *sp[1] = {scale};
    void *yp[1] = {o};
    const int Np[1] = {N};
    hipError_t e = launch_linear_int8_gemv(x, 1, wp, sp, yp, Np, M, K, stream);
    if (e != hipSuccess) return e;
    return launch_rmsnorm(o, gamma, res, y, M, N, eps, GROK_BF16, stream);
  }
  OutNormArgs na = {};
  GemvArgs &a = na.g;
  a.x = static_cast<const bf16_t *>(x);
  a.mat[0] = GemvMat{w, scale, o, N, 0};
  a.nmat = 1;
  a.M = static_cast<int>(M);
  a.K = K;
  a.KP = (K + kTileRows - 1) / kTileRows;
  na.res = static_cast<const bf16_t *>(res);
  na.out = static_cast<bf16_t *>(y);
  na.gamma = gamma;
  na.eps = eps;
  na.ss = ss;
  na.count = count;
  const size_t lds = static_cast<size_t>(M) * K * 2;
  hipLaunchKernelGGL(gemv_out_norm_kernel, dim3(static_cast<unsigned>(nwg)), dim3(kThreads), lds, stream, na);
  return hipGetLastError();
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

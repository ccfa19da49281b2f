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
// Workgroup tile 128 (n) x 256 (m), K step 64, 8 waves in 4 (m) x 2 (n), each
// wave 64 x 64 = 4 x 4 MFMA tiles; one workgroup per CU (128 KB of LDS). X
// tiles triple-buffered in LDS (requested two steps ahead), W^T tiles
// double-buffered (one step ahead, via registers; staged by waves 0-3, so the
// int8 widening is paid once per 256 rows).
#include "common.h"

namespace grok {
namespace {

constexpr int kThreads = 512;
constexpr int kStageThreads = 256;  // threads that stage the W tile
constexpr int kBN = 128;  // output channels per workgroup
constexpr int kBM = 256;  // rows per workgroup
constexpr int kBK = 64;
constexpr int kRowB = kBK * 2;  // one LDS row: 64 bf16 = 128 bytes, unpadded
constexpr int kTileB = 128 * kRowB;       // W^T tile: 128 rows
constexpr int kXTileB = kBM * kRowB;      // X tile: 256 rows

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
// row): 16-byte chunk c of row r sits at chunk c ^ sw(r). This swizzle was
// chosen by measurement (SQ_LDS_BANK_CONFLICT on isolated access patterns):
// it is conflict-free both for the fragment reads (16 consecutive rows, one
// chunk) and for the transposed W^T stores (rows 4*g + j over 32 lanes g).
__device__ __forceinline__ int sw(int r) { return (r ^ (r >> 2)) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * kRowB + ((c ^ sw(r)) << 4); }

// Fragment reads as inline assembly: the compiler cannot tell them apart from
// the X tiles still streaming into other LDS buffers and would wait for those
// loads first. LDS operations complete in order; results are used only after
// lds_wait, which passes them through.
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
  return r;
}
template <int kOff>
__device__ __forceinline__ bf16x8 lds_read_b128_at(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff) : "memory");
  return r;
}
// The 8 fragment reads of k-step kk: blocks b = 0..3 of 16 rows at byte
// 16*b*128 from the base for q = kk ^ (b % 2).
template <int kKK>
__device__ __forceinline__ void read_frags(bf16x8 (&bx)[4], bf16x8 (&aw)[4], const uint32_t (&xq)[2],
                                           const uint32_t (&wq)[2]) {
  bx[0] = lds_read_b128_at<0 * 2048>(xq[kKK ^ 0]);
  bx[1] = lds_read_b128_at<1 * 2048>(xq[kKK ^ 1]);
  bx[2] = lds_read_b128_at<2 * 2048>(xq[kKK ^ 0]);
  bx[3] = lds_read_b128_at<3 * 2048>(xq[kKK ^ 1]);
  aw[0] = lds_read_b128_at<0 * 2048>(wq[kKK ^ 0]);
  aw[1] = lds_read_b128_at<1 * 2048>(wq[kKK ^ 1]);
  aw[2] = lds_read_b128_at<2 * 2048>(wq[kKK ^ 0]);
  aw[3] = lds_read_b128_at<3 * 2048>(wq[kKK ^ 1]);
}

template <int kLeft>
__device__ __forceinline__ void lds_wait(bf16x8 (&a)[4], bf16x8 (&b)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3])
               : "i"(kLeft));
}

// tanh form of GELU in fp32: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3),
// tanh(u) = 1 - 2 / (1 + exp(2u)) (saturates correctly at both ends).
__device__ __forceinline__ float gelu_tanh(float x) {
  const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x);
  const float t = 1.f - 2.f / (1.f + __expf(2.f * u));
  return 0.5f * x * (1.f + t);
}

// kGrouped: the rows of y are grouped by expert (MoE, grouped GEMM): group e
// owns rows [ga.offsets[e], ga.offsets[e+1]) and is multiplied by its own
// weights ga.w[e], scales ga.s[e]; blockIdx.y enumerates the row tiles of the
// groups in order (tiles past the last group exit). kGather: row m of x is
// row ga.rows[m] of the x buffer (the token a grouped row stands for).
// kGeGLU: the weight columns hold gate and value channels interleaved by four
// (columns 8q..8q+3 = gate channels 4q..4q+3, 8q+4..8q+7 = value channels),
// and the epilogue writes h = gelu(gate) * value into y [M, N/2].
// kQkv: the fused Q/K/V projection (PrefillQkvArgs): column tile c is head c of Q,
// then the heads of K, then of V (128 channels each, D = 128 = kBN); the
// epilogue rounds the projection to bf16 as a separate projection would, then
// rotates Q and K at their positions (the two halves of a head sit in waves w
// and w ^ 1 at the same register and lane: one exchange through LDS) and
// writes q to its buffer and k, v to their cache slots.
template <bool kGrouped, bool kGather, bool kGeGLU, bool kQkv = false>
__global__ __launch_bounds__(kThreads, 1) void linear_int8_kernel(
    const bf16_t *__restrict__ x, const int8_t *__restrict__ w_in, const float *__restrict__ scales_in,
    bf16_t *__restrict__ y, int64_t M, int K, int N, GroupArgs ga, PrefillQkvArgs qa = {}) {
  __shared__ __attribute__((aligned(1024))) unsigned char Xs[3][kXTileB];
  __shared__ __attribute__((aligned(1024))) unsigned char Wt[2][kTileB];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane % 16, lg = lane / 16;
  const int wn = wave % 2, wm = wave / 2;
  int n0 = blockIdx.x * kBN;
  int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int8_t *w = w_in;
  const float *scales = scales_in;
  int mat = 0, head = 0;
  if constexpr (kQkv) {
    const int c = blockIdx.x;
    mat = c < qa.Hq ? 0 : (c < qa.Hq + qa.Hkv ? 1 : 2);
    head = c - (mat == 0 ? 0 : (mat == 1 ? qa.Hq : qa.Hq + qa.Hkv));
    w = qa.w[mat];
    scales = qa.s[mat];
    N = (mat == 0 ? qa.Hq : qa.Hkv) * kBN;
    n0 = head * kBN;
  }
  if constexpr (kGrouped) {
    // this tile's group: walk the groups' tile counts (uniform, scalar loads)
    int ty = blockIdx.y, e = -1;
    int64_t lo = 0;
    for (int q = 0; q < ga.E; ++q) {
      const int o0 = ga.offsets[q], o1 = ga.offsets[q + 1];
      const int nt = (o1 - o0 + kBM - 1) / kBM;
      if (e < 0 && ty < nt) {
        e = q;
        m0 = o0 + static_cast<int64_t>(ty) * kBM;
        lo = o1;
      }
      if (e < 0) ty -= nt;
    }
    if (e < 0) return;  // whole workgroup: past the last group's tiles
    M = lo;             // the group's end row
    w = ga.w[e];
    scales = ga.s[e];
  }

  // X tile: HBM -> LDS directly (global_load_lds, 16 bytes per lane). Wave
  // `wave`, instruction i fills rows 32*wave + 8*i .. +7; lane L writes chunk
  // position L%8 of row 32*wave + 8*i + L/8, fetching logical chunk
  // (L%8) ^ sw(row). Rows past M read row M-1 and columns past K read the last
  // 8 columns (finite values; the matching W^T entries are zero).
  const int xl_row = lane / 8, xl_pos = lane % 8;
  // Fast path: byte offsets from the tile's first element, fixed per lane
  // (rows already clamped to M-1); slow path only for a K tail.
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + xl_row;
    if constexpr (kGather)
      xoff[i] = static_cast<uint32_t>(static_cast<int64_t>(ga.rows[min(m0 + r, M - 1)]) * K * 2) +
                16 * (xl_pos ^ sw(r));
    else
      xoff[i] = static_cast<uint32_t>((min(m0 + r, M - 1) - m0) * K * 2) + 16 * (xl_pos ^ sw(r));
  }
  const char *xtile = reinterpret_cast<const char *>(kGather ? x : x + m0 * K);
  auto issue_x = [&](int k0, int buf) {
    if (k0 + kBK <= K) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(xtile + 2 * k0 + xoff[i],
                                         (lds_void *)(&Xs[buf][(32 * wave + 8 * i) * kRowB]), 16, 0, 0);
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wave + 8 * i + xl_row;
      const int64_t mr = min(m0 + r, M - 1);
      const int64_t m = kGather ? static_cast<int64_t>(ga.rows[mr]) : mr;
      const int k = min(k0 + 8 * (xl_pos ^ sw(r)), K - 8);
      __builtin_amdgcn_global_load_lds(x + m * K + k, (lds_void *)(&Xs[buf][(32 * wave + 8 * i) * kRowB]), 16,
                                       0, 0);
    }
  };

  // W staging: 8 rows (k) x 4 channels (n) int8 per thread (one 4-byte load
  // per k row; 32 lanes cover 128 contiguous channels), widened to bf16 and
  // stored transposed: channel j's 8 k values are one 16-byte chunk of W^T row
  // 4*wg + j. The loads are inline assembly so that the compiler does not add
  // its own wait for them (it cannot count them against the X tile loads); the
  // loop waits explicitly. Entries past K or N read a clamped address and are
  // zeroed after the wait (wvalid).
  const int wg = tid % 32, wkc = tid / 32;  // channels 4*wg.., k rows 8*wkc..
  uint32_t wr[8];
  uint32_t wvalid = 0;
  const uint32_t woff = static_cast<uint32_t>(8 * wkc) * N + 4 * wg;  // byte offset in a k-step tile
  const bool w_full_n = n0 + kBN <= N;
  auto gload_w = [&](int k0) {
    if (w_full_n && k0 + kBK <= K) {
      wvalid = 0xffu;
      const int8_t *wt = w + static_cast<int64_t>(k0) * N + n0;  // wave-uniform
#pragma unroll
      for (int r = 0; r < 8; ++r)
        asm volatile("global_load_dword %0, %1, %2" : "=v"(wr[r]) : "v"(woff + r * N), "s"(wt) : "memory");
      return;
    }
    const int n = n0 + 4 * wg;
    wvalid = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int k = k0 + 8 * wkc + r;
      const bool ok = k < K && n < N;
      wvalid |= ok ? (1u << r) : 0u;
      const int8_t *src = w + static_cast<int64_t>(ok ? k : 0) * N + (ok ? n : 0);
      asm volatile("global_load_dword %0, %1, off" : "=v"(wr[r]) : "v"(src) : "memory");
    }
  };
  auto lstore_w = [&](int buf) {
    if (wvalid != 0xffu) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (!(wvalid & (1u << r))) wr[r] = 0;
    }
    const uint32_t wt0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)(&Wt[buf][0])));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 pk;
#pragma unroll
      for (int q = 0; q < 4; ++q) pk[q] = cvt_pk_bf16(i8_to_f32(wr[2 * q], j), i8_to_f32(wr[2 * q + 1], j));
      const uint32_t a = wt0 + lds_off(4 * wg + j, wkc);
      asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(pk) : "memory");
    }
  };

  // Fragment read addresses. For row R0 + lr (R0 = 16 * block, a multiple of
  // 16) and chunk 4*kk + lg, lds_off = R0*128 + lr*128 + 16*((lg ^ s) ^ 4*q)
  // with s = (lr % 8) ^ (lr / 4) and q = kk ^ (block % 2): two per-lane bases
  // (q = 0, 1) plus immediates cover every fragment read of a step.
  uint32_t xrd[2], wrd[2];
  {
    const int sl = (lr & 7) ^ (lr >> 2);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t a = lr * kRowB + 16 * ((lg ^ sl) ^ (4 * q));
      xrd[q] = 64 * wm * kRowB + a;
      wrd[q] = 64 * wn * kRowB + a;
    }
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Pipeline: the X tile of step t+2 is requested while step t computes (three
  // X buffers), the W tile of step t+1 one step ahead (two W buffers). The
  // loads of a step are issued W first, then X, so the wait at the end of step
  // t (W of t+1 and X of t+1 complete) leaves the four X(t+2) loads in flight.
  const int nk = (K + kBK - 1) / kBK;
  const bool stager = wave < kStageThreads / kWave;  // wave-uniform
  if (stager) gload_w(0);
  issue_x(0, 0);
  issue_x(min(1, nk - 1) * kBK, 1);
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(wr[0]), "+v"(wr[1]), "+v"(wr[2]), "+v"(wr[3]), "+v"(wr[4]),
               "+v"(wr[5]), "+v"(wr[6]), "+v"(wr[7]) : : "memory");
  if (stager) lstore_w(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const int buf = t & 1;
    const int xbuf = t % 3;
    const bool more = t + 1 < nk;
    // Issued unconditionally (clamped at the end) so that every step has the
    // same number of loads in flight: W(t+1), then X(t+2).
    if (stager) gload_w(min(t + 1, nk - 1) * kBK);
    issue_x(min(t + 2, nk - 1) * kBK, (t + 2) % 3);
    const uint32_t xb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)(&Xs[xbuf][0])));
    const uint32_t wb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)(&Wt[buf][0])));
    const uint32_t xq[2] = {xb + xrd[0], xb + xrd[1]};
    const uint32_t wq[2] = {wb + wrd[0], wb + wrd[1]};
    bf16x8 bx[2][4], aw[2][4];
    read_frags<0>(bx[0], aw[0], xq, wq);
    read_frags<1>(bx[1], aw[1], xq, wq);
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      if (kk == 0) {
        lds_wait<8>(bx[0], aw[0]);
      } else {
        __builtin_amdgcn_sched_barrier(0);
        lds_wait<0>(bx[1], aw[1]);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[kk][nb], bx[kk][mb], acc[nb][mb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // the waits below stay after this step's MFMAs
    // W(t+1) and X(t+1) have landed once at most the 4 X(t+2) loads remain.
    asm volatile("s_waitcnt vmcnt(4)" : "+v"(wr[0]), "+v"(wr[1]), "+v"(wr[2]), "+v"(wr[3]), "+v"(wr[4]),
                 "+v"(wr[5]), "+v"(wr[6]), "+v"(wr[7]) : : "memory");
    if (stager && more) lstore_w(buf ^ 1);
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");  // LDS stores done
    // Workgroup barrier without a memory fence (a fence would wait for the X
    // loads still in flight); the asm memory clobber keeps LDS accesses on
    // their side of it.
    asm volatile("s_barrier" ::: "memory");
  }

  // The last steps re-requested tiles they do not use: let those LDS-bound
  // loads land before the workgroup can exit and release its LDS.
  __builtin_amdgcn_s_waitcnt(0);

  // Epilogue: lane holds Y^T[n = nbase + 4*lg + v, m = mbase + lr], v = 0..3.
  if constexpr (kQkv) {
    if (blockIdx.x == 0 && blockIdx.y == 0) {  // per sequence: new_step, status
      for (int bb = tid; bb < qa.B; bb += kThreads) {
        const int s0 = qa.step ? qa.step[bb] : 0;
        const bool ok = s0 >= 0 && s0 <= qa.Tmax - qa.T;
        if (qa.new_step) qa.new_step[bb] = ok ? s0 + qa.T : s0;
        if (!ok && qa.status) *qa.status = GROK_ERANGE;
      }
    }
    // the projection handed on in bf16, packed in pairs: r[nb][mb][h] holds v = 2h, 2h+1
    uint32_t r[4][4][2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const f32x4 sc = *reinterpret_cast<const f32x4 *>(scales + n0 + 64 * wn + 16 * nb + 4 * lg);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const f32x4 v = acc[nb][mb];
        r[nb][mb][0] = cvt_pk_bf16(v[0] * sc[0], v[1] * sc[1]);
        r[nb][mb][1] = cvt_pk_bf16(v[2] * sc[2], v[3] * sc[3]);
      }
    }
    uint32_t pr[4][4][2];  // the partner half of the head (channel d +- 64)
    if (mat < 2) {
      // every wave is past its last LDS read (loop barrier) and its own tile
      // loads (wait above); after this barrier no load still targets Xs
      __syncthreads();
      uint32_t *xch = reinterpret_cast<uint32_t *>(&Xs[0][0]);  // [8 waves][32][64 lanes]
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int h = 0; h < 2; ++h) xch[(wave * 32 + (nb * 4 + mb) * 2 + h) * kWave + lane] = r[nb][mb][h];
      __syncthreads();
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int h = 0; h < 2; ++h) pr[nb][mb][h] = xch[((wave ^ 1) * 32 + (nb * 4 + mb) * 2 + h) * kWave + lane];
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int64_t m = m0 + 64 * wm + 16 * mb + lr;
      if (m >= M) continue;
      const int bq = static_cast<int>(m / qa.T), t = static_cast<int>(m % qa.T);
      const int s0 = qa.step ? qa.step[bq] : 0;
      if (s0 < 0 || s0 > qa.Tmax - qa.T) continue;  // sequence outside the cache: nothing is written
      const int pos = s0 + t;
      bf16_t *dst = mat == 0 ? qa.out[0] + (m * qa.Hq + head) * kBN
                             : qa.out[mat] + ((static_cast<int64_t>(bq) * qa.Tmax + pos) * qa.Hkv + head) * kBN;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int d = 64 * wn + 16 * nb + 4 * lg;
        u32x2 o = {r[nb][mb][0], r[nb][mb][1]};
        if (mat < 2) {
          const int i = 16 * nb + 4 * lg;  // pair index of v = 0
          const f32x4 cs = *reinterpret_cast<const f32x4 *>(qa.rtab + pos * 128 + i);
          const f32x4 sn = *reinterpret_cast<const f32x4 *>(qa.rtab + pos * 128 + 64 + i);
          float ov[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t mine = r[nb][mb][v >> 1], other = pr[nb][mb][v >> 1];
            const float xm = (v & 1) ? hi_bf16(mine) : lo_bf16(mine);
            const float xo = (v & 1) ? hi_bf16(other) : lo_bf16(other);
            float o1, o2;
            if (wn == 0)
              rope_rotate(xm, xo, cs[v], sn[v], o1, o2), ov[v] = o1;
            else
              rope_rotate(xo, xm, cs[v], sn[v], o1, o2), ov[v] = o2;
          }
          o = u32x2{cvt_pk_bf16(ov[0], ov[1]), cvt_pk_bf16(ov[2], ov[3])};
        }
        *reinterpret_cast<u32x2 *>(dst + d) = o;
      }
    }
    return;
  }
  if constexpr (kGeGLU) {
    // lanes lg and lg ^ 1 hold the gate and the value columns of the same 4
    // channels: the even one combines and stores them. Both projections are
    // rounded to bf16 (as a separate projection would hand them on), then
    // gelu(gate) * value is rounded once.
    const int Nh = N / 2;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + 64 * wn + 16 * nb + 4 * lg;  // lg even: gate columns, n % 8 == 0
      const bool ok_n = n < N;
      const f32x4 sc = ok_n ? *reinterpret_cast<const f32x4 *>(scales + n) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const f32x4 v = acc[nb][mb];
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = bf16_to_f32(f32_to_bf16(v[e] * sc[e]));
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __shfl_xor(r[e], 16, kWave);
        const int64_t m = m0 + 64 * wm + 16 * mb + lr;
        if ((lg & 1) || !ok_n || m >= M) continue;
        const u32x2 hw = {cvt_pk_bf16(gelu_tanh(r[0]) * o[0], gelu_tanh(r[1]) * o[1]),
                          cvt_pk_bf16(gelu_tanh(r[2]) * o[2], gelu_tanh(r[3]) * o[3])};
        *reinterpret_cast<u32x2 *>(y + m * Nh + n / 2) = hw;
      }
    }
    return;
  }
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
  hipLaunchKernelGGL((linear_int8_kernel<false, false, false>), grid, dim3(kThreads), 0, s,
                     static_cast<const bf16_t *>(x), w, scales, static_cast<bf16_t *>(y), M, K, N, GroupArgs{});
  return hipGetLastError();
}

hipError_t launch_linear_int8_grouped(const void *x, const int32_t *rows, const int32_t *offsets, int E,
                                      const int8_t *const *w, const float *const *scales, void *y,
                                      int64_t M_total, int K, int N, bool geglu, hipStream_t s) {
  GroupArgs ga = {};
  ga.offsets = offsets;
  ga.rows = rows;
  ga.E = E;
  for (int e = 0; e < E; ++e) {
    ga.w[e] = w[e];
    ga.s[e] = scales[e];
  }
  // row tiles: at most one partial tile per group beyond the full ones
  const int64_t gm = (M_total + kBM - 1) / kBM + E;
  if (gm > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((N + kBN - 1) / kBN, static_cast<unsigned>(gm));
  const bf16_t *xb = static_cast<const bf16_t *>(x);
  bf16_t *yb = static_cast<bf16_t *>(y);
  if (rows && geglu)
    hipLaunchKernelGGL((linear_int8_kernel<true, true, true>), grid, dim3(kThreads), 0, s, xb, w[0], scales[0], yb,
                       M_total, K, N, ga);
  else if (rows)
    hipLaunchKernelGGL((linear_int8_kernel<true, true, false>), grid, dim3(kThreads), 0, s, xb, w[0], scales[0], yb,
                       M_total, K, N, ga);
  else if (geglu)
    hipLaunchKernelGGL((linear_int8_kernel<true, false, true>), grid, dim3(kThreads), 0, s, xb, w[0], scales[0], yb,
                       M_total, K, N, ga);
  else
    hipLaunchKernelGGL((linear_int8_kernel<true, false, false>), grid, dim3(kThreads), 0, s, xb, w[0], scales[0],
                       yb, M_total, K, N, ga);
  return hipGetLastError();
}

namespace {

// cos / sin of every (position, pair) of a head of 128, from the pinned RoPE
// helpers, so that the fused epilogue rotates with the bits of the RoPE kernels.
__global__ __launch_bounds__(64) void rope_table_kernel(float *tab, RopeFreqs f) {
  const int pos = blockIdx.x, i = threadIdx.x;
  float sn, cs;
  rope_phase(pos, f.inv[i], sn, cs);
  tab[pos * 128 + i] = cs;
  tab[pos * 128 + 64 + i] = sn;
}

}  // namespace

size_t prefill_qkv_workspace_bytes(int Tmax) { return static_cast<size_t>(Tmax) * 128 * sizeof(float); }

hipError_t launch_rope_table(float *tab, int npos, const RopeFreqs &f, hipStream_t s) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(npos), dim3(64), 0, s, tab, f);
  return hipGetLastError();
}

hipError_t launch_prefill_qkv(const void *x, const PrefillQkvArgs &qa_in, void *workspace, int d, float rope_base,
                              hipStream_t s) {
  RopeFreqs f;
  rope_build_freqs(kBN, rope_base, &f);
  PrefillQkvArgs qa = qa_in;
  qa.rtab = static_cast<const float *>(workspace);
  hipError_t e = launch_rope_table(static_cast<float *>(workspace), qa.Tmax, f, s);
  if (e != hipSuccess) return e;
  const int64_t M = static_cast<int64_t>(qa.B) * qa.T;
  const int64_t gm = (M + kBM - 1) / kBM;
  if (gm > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid(qa.Hq + 2 * qa.Hkv, static_cast<unsigned>(gm));
  hipLaunchKernelGGL((linear_int8_kernel<false, false, false, true>), grid, dim3(kThreads), 0, s,
                     static_cast<const bf16_t *>(x), qa.w[0], qa.s[0], qa.out[0], M, d, qa.Hq * kBN, GroupArgs{}, qa);
  return hipGetLastError();
}

}  // namespace grok

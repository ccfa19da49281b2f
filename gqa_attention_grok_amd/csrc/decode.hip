// Single-token GQA decode against the KV cache, split over the cache length.
//
// Method (Grok-1 walkthrough, ch. 4 "model.py close reading, part 1", §4.4 and
// §4.5): one query per sequence attends cache slots j < kv_len[b] (the memory
// mask; the causal mask of one query is all-ones); logits are scaled, soft-capped
// and soft-maxed in fp32; P.V in bf16 MFMA with fp32 accumulation.
//
// HBM-bound: every valid K/V row (256 B each) is read exactly once and slots at
// or beyond kv_len are never touched.
//
// Kernel 1 (decode_split_kernel), one workgroup per (sequence, KV head, split of
// kChunk keys): each of its 4 waves takes 32 keys. Rows of the MFMA tiles are
// the G <= 16 query heads of the KV head (unused rows are zero):
//   S^T[key, head] = K . Q^T   (K fragments loaded straight from HBM)
//   O^T[d, head]  += V^T . P^T (V transposed through LDS)
// The softmax uses the fixed shift exp(c - cap) (unmasked softcapped logits lie
// in [-cap, cap]), so split partials are plain sums: (sum p*v, sum p).
// Kernel 2 (decode_combine_kernel) adds the partials of each (sequence, head)
// and writes bf16 out = sum(p*v) / sum(p).
#include "common.h"

namespace grok {
namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTile = 32;
constexpr int kChunk = kWaves * kTile;  // keys per split
constexpr int kVRow = kTile + 8;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

struct DecodeArgs {
  const bf16_t *q, *kc, *vc;
  const int32_t *kv_len;
  bf16_t *out;
  float *part_o;  // [B, Hkv, S, G, D]
  float *part_l;  // [B, Hkv, S, G]
  int32_t *status;
  int B, Tmax, Hq, Hkv, G, S;
  float k1, k2;
};

__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kWaves * kD * kVRow * 2];
  bf16_t(*Vt)[kD][kVRow] = reinterpret_cast<bf16_t(*)[kD][kVRow]>(smem);
  float(*red)[16][kD] = reinterpret_cast<float(*)[16][kD]>(smem);  // reused after P.V
  __shared__ float redl[kWaves][16];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int len = a.kv_len[b];
  if (len < 1 || len > a.Tmax) return;  // reported by the combine kernel
  const int kbeg = s * kChunk;
  if (kbeg >= len) return;

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int kw0 = kbeg + wave * kTile;
  const bool active = kw0 < len;
  const int64_t rstride = static_cast<int64_t>(a.Hkv) * kD;
  const bf16_t *kbase = a.kc + (static_cast<int64_t>(b) * a.Tmax * a.Hkv + g) * kD;
  const bf16_t *vbase = a.vc + (static_cast<int64_t>(b) * a.Tmax * a.Hkv + g) * kD;

  // K fragments (A operand of S^T), straight from HBM: rows permuted so that
  // accumulator slot v of lane l is key 8*lg + 4*kb + v.
  u32x4 kf[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int j = kw0 + 8 * (lr / 4) + 4 * kb + (lr % 4);
    const bool ok = active && j < len;
    const bf16_t *kp = kbase + (ok ? j : 0) * rstride + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      kf[kb][kk] = ok ? *reinterpret_cast<const u32x4 *>(kp + 32 * kk) : u32x4{0, 0, 0, 0};
  }

  // Q fragment: head row lr (zero beyond G), dims 32*kk + 8*lg.
  bf16x8 qf[4];
  {
    const bool ok = lr < a.G;
    const bf16_t *qp = a.q + (static_cast<int64_t>(b) * a.Hq + g * a.G + (ok ? lr : 0)) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 w = ok ? *reinterpret_cast<const u32x4 *>(qp + 32 * kk + 8 * lg) : u32x4{0, 0, 0, 0};
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // V rows of this wave's 32 keys, transposed into LDS: 4 (key pair, 8-dim chunk)
  // items per lane.
  if (active) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int item = lane + kWave * r;
      const int m = item / 16, c = item % 16;
      const int j0 = kw0 + 2 * m, j1 = j0 + 1;
      const u32x4 w0 = j0 < len ? *reinterpret_cast<const u32x4 *>(vbase + j0 * rstride + 8 * c) : u32x4{0, 0, 0, 0};
      const u32x4 w1 = j1 < len ? *reinterpret_cast<const u32x4 *>(vbase + j1 * rstride + 8 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint32_t *>(&Vt[wave][8 * c + 2 * e][2 * m]) = (w0[e] & 0xffffu) | (w1[e] << 16);
        *reinterpret_cast<uint32_t *>(&Vt[wave][8 * c + 2 * e + 1][2 * m]) = (w0[e] >> 16) | (w1[e] & 0xffff0000u);
      }
    }
  }
  __syncthreads();

  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;

  if (active) {
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kb][kk]), qf[kk], sacc[kb], 0, 0, 0);
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = sacc[e >> 2][e & 3];
      const float ex = __builtin_amdgcn_exp2f(sv * a.k1);
      const float r = __builtin_amdgcn_rcpf(1.f + ex);
      const float pv = __builtin_amdgcn_exp2f(a.k2 * r);
      p[e] = (kw0 + 8 * lg + e < len) ? pv : 0.f;
    }
    const u32x4 pw = {cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]), cvt_pk_bf16(p[4], p[5]),
                      cvt_pk_bf16(p[6], p[7])};
    // Row sum of the bf16-rounded weights that P.V uses.
#pragma unroll
    for (int e = 0; e < 4; ++e) lsum += lo_bf16(pw[e]) + hi_bf16(pw[e]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&Vt[wave][16 * db + lr][8 * lg]);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[db], 0, 0, 0);
    }
  }
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);

  // Reduce the 4 waves through LDS (reusing the V^T space).
  __syncthreads();
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][lr][16 * db + 4 * lg + v] = oacc[db][v];
  if (lg == 0) redl[wave][lr] = lsum;
  __syncthreads();

  const int64_t pbase = ((static_cast<int64_t>(b) * a.Hkv + g) * a.S + s) * a.G;
  for (int i = tid; i < a.G * kD; i += kThreads) {
    const int hh = i / kD, d = i % kD;
    a.part_o[(pbase + hh) * kD + d] = red[0][hh][d] + red[1][hh][d] + red[2][hh][d] + red[3][hh][d];
  }
  if (tid < a.G) a.part_l[pbase + tid] = redl[0][tid] + redl[1][tid] + redl[2][tid] + redl[3][tid];
}

__global__ __launch_bounds__(kD) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int g = h / a.G, hh = h % a.G;
  const int d = threadIdx.x;
  bf16_t *o = a.out + static_cast<int64_t>(bh) * kD + d;
  const int len = a.kv_len[b];
  if (len < 1 || len > a.Tmax) {
    *o = 0;
    if (d == 0 && a.status) *a.status = GROK_ERANGE;
    return;
  }
  const int ns = (len + kChunk - 1) / kChunk;
  const int64_t base = (static_cast<int64_t>(b) * a.Hkv + g) * a.S;
  float acc = 0.f, l = 0.f;
  for (int s = 0; s < ns; ++s) {
    acc += a.part_o[((base + s) * a.G + hh) * kD + d];
    l += a.part_l[(base + s) * a.G + hh];
  }
  *o = f32_to_bf16(acc / l);
}

}  // namespace

size_t decode_workspace_bytes(int B, int Tmax, int Hq, int Hkv) {
  const size_t S = (static_cast<size_t>(Tmax) + kChunk - 1) / kChunk;
  const size_t G = static_cast<size_t>(Hq / Hkv);
  const size_t n = static_cast<size_t>(B) * Hkv * S * G;
  const size_t o_bytes = n * kD * sizeof(float);
  return o_bytes + n * sizeof(float);
}

hipError_t launch_decode(const void *q, const void *kc, const void *vc, const int32_t *kv_len,
                         void *out, void *ws, int32_t *status, int B, int Tmax, int Hq, int Hkv,
                         float mult, float cap, hipStream_t st) {
  DecodeArgs a;
  a.q = static_cast<const bf16_t *>(q);
  a.kc = static_cast<const bf16_t *>(kc);
  a.vc = static_cast<const bf16_t *>(vc);
  a.kv_len = kv_len;
  a.out = static_cast<bf16_t *>(out);
  a.B = B;
  a.Tmax = Tmax;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.S = (Tmax + kChunk - 1) / kChunk;
  const size_t n = static_cast<size_t>(B) * Hkv * a.S * a.G;
  a.part_o = static_cast<float *>(ws);
  a.part_l = a.part_o + n * kD;
  a.status = status;
  a.k1 = 2.f * mult * kLog2e / cap;
  a.k2 = -2.f * cap * kLog2e;
  hipLaunchKernelGGL(decode_split_kernel, dim3(a.S, Hkv, B), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(B * Hq), dim3(kD), 0, st, a);
  return hipGetLastError();
}

}  // namespace grok

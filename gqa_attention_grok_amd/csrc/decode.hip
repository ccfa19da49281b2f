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
// Kernel 1 (decode_split_kernel): one workgroup per (sequence, split of
// `split_keys` cache slots, group of up to 8 KV heads), one wave per KV head.
// The cache stores the 8 KV heads of a slot side by side (2 KB), so the waves
// of a workgroup together stream whole contiguous slot rows. Each wave walks
// its split in tiles of 32 keys, loading tile t+1 while it computes tile t.
// MFMA rows are the G <= 16 query heads of the wave's KV head (unused rows are
// zero):
//   S^T[key, head] = K . Q^T   (K fragments loaded straight from HBM)
//   O^T[d, head]  += V^T . P^T (V transposed through the wave's own LDS slice)
// The softmax uses the fixed shift exp(c - cap): unmasked softcapped logits lie
// in [-cap, cap], so a split's partial result is a plain pair of sums
// (sum p*v, sum p) with no running maximum to reconcile.
// Kernel 2 (decode_combine_kernel): one workgroup per (sequence, query head)
// adds the partials of the splits and writes bf16 sum(p*v) / sum(p).
#include "common.h"

namespace grok {
namespace {

constexpr int kD = 128;
constexpr int kWavesMax = 8;  // KV heads per workgroup
constexpr int kTile = 32;
// V^T slice of a wave: 128 rows (dims) of 32 keys (64 B, four 16-byte groups of
// 8 keys). The group of key k in row d is stored at (k/8) ^ ((d/2) % 4), which
// spreads the 16-byte fragment reads of 8 consecutive rows over all banks.
__device__ __forceinline__ int vt_index(int d, int k) {
  return d * kTile + ((((k >> 3) ^ (d >> 1)) & 3) << 3) + (k & 7);
}
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
  int B, Tmax, Hq, Hkv, G, S, split_keys;
  float k1, k2;
};

// One tile's operands in registers: K fragments (A operand of S^T, rows
// permuted so that accumulator slot v of lane l is key 8*lg + 4*kb + v) and two
// (4-key quad, 8-dim chunk) slices of V.
struct TileRegs {
  u32x4 k[2][4];
  u32x4 v[2][4];
};

__device__ __forceinline__ void load_tile(TileRegs &r, const bf16_t *kbase, const bf16_t *vbase,
                                          int64_t rstride, int key0, int len, int lane) {
  const int lr = lane % 16, lg = lane / 16;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int j = key0 + 8 * (lr / 4) + 4 * kb + (lr % 4);
    const bool ok = j < len;
    const bf16_t *kp = kbase + (ok ? j : 0) * rstride + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      r.k[kb][kk] = ok ? *reinterpret_cast<const u32x4 *>(kp + 32 * kk) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int item = lane + kWave * it;
    const int kq = item % 8, vc = item / 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = key0 + 4 * kq + i;
      r.v[it][i] = j < len ? *reinterpret_cast<const u32x4 *>(vbase + j * rstride + 8 * vc) : u32x4{0, 0, 0, 0};
    }
  }
}

__global__ __launch_bounds__(kWavesMax * kWave) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t Vt[kWavesMax][kD * kTile];

  const int b = blockIdx.z, s = blockIdx.x;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int g = blockIdx.y * kWavesMax + wave;
  const int len = a.kv_len[b];
  if (len < 1 || len > a.Tmax) return;  // reported by the combine kernel
  const int sbase = s * a.split_keys;
  if (sbase >= len || g >= a.Hkv) return;  // no barrier below: waves may leave

  const int lr = lane % 16, lg = lane / 16;
  const int64_t rstride = static_cast<int64_t>(a.Hkv) * kD;
  const bf16_t *kbase = a.kc + (static_cast<int64_t>(b) * a.Tmax * a.Hkv + g) * kD;
  const bf16_t *vbase = a.vc + (static_cast<int64_t>(b) * a.Tmax * a.Hkv + g) * kD;
  const int send = min(len, sbase + a.split_keys);

  TileRegs cur, nxt;
  load_tile(cur, kbase, vbase, rstride, sbase, send, lane);

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

  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;

  for (int key0 = sbase; key0 < send; key0 += kTile) {
    const int next0 = key0 + kTile;
    if (next0 < send) load_tile(nxt, kbase, vbase, rstride, next0, send, lane);

    // V^T of this tile into the wave's own LDS slice: 4 keys per 8-byte write.
    // LDS operations of one wave complete in order, so the fragment reads below
    // see these writes and the next tile's writes follow this tile's reads.
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = lane + kWave * it;
      const int kq = item % 8, vc = item / 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        uint32_t x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (e & 1) ? (cur.v[it][i][wd] >> 16) : (cur.v[it][i][wd] & 0xffffu);
        const u32x2 w = {x[0] | (x[1] << 16), x[2] | (x[3] << 16)};
        *reinterpret_cast<u32x2 *>(&Vt[wave][vt_index(8 * vc + e, 4 * kq)]) = w;
      }
    }
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[kb][kk]), qf[kk],
                                                           sacc[kb], 0, 0, 0);
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sv = sacc[e >> 2][e & 3];
      const float ex = __builtin_amdgcn_exp2f(sv * a.k1);
      const float r = __builtin_amdgcn_rcpf(1.f + ex);
      const float pv = __builtin_amdgcn_exp2f(a.k2 * r);
      p[e] = (key0 + 8 * lg + e < send) ? pv : 0.f;
    }
    const u32x4 pw = {cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]), cvt_pk_bf16(p[4], p[5]),
                      cvt_pk_bf16(p[6], p[7])};
    // Row sum of the bf16-rounded weights that P.V uses.
#pragma unroll
    for (int e = 0; e < 4; ++e) lsum += lo_bf16(pw[e]) + hi_bf16(pw[e]);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&Vt[wave][vt_index(16 * db + lr, 8 * lg)]);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[db], 0, 0, 0);
    }
    cur = nxt;
  }
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);

  // This wave's partial: O^T lane l holds head row lr, dims 16*db + 4*lg + v.
  const int64_t pbase = ((static_cast<int64_t>(b) * a.Hkv + g) * a.S + s) * a.G;
  if (lr < a.G) {
    float *po = a.part_o + (pbase + lr) * kD;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4 *>(po + 16 * db + 4 * lg) = oacc[db];
    if (lg == 0) a.part_l[pbase + lr] = lsum;
  }
}

constexpr int kCombineThreads = 256;
constexpr int kSplitGroups = kCombineThreads / (kD / 4);  // 8 groups of 32 float4 lanes

// One workgroup per (sequence, query head): 32 lanes x float4 cover the head's
// 128 outputs; 8 groups take every 8th split; the groups are added in LDS.
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeArgs a) {
  __shared__ f32x4 red_o[kSplitGroups][kD / 4];
  __shared__ float red_l[kSplitGroups];
  const int b = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int g = h / a.G, hh = h % a.G;
  const int len = a.kv_len[b];
  bf16_t *orow = a.out + (static_cast<int64_t>(b) * a.Hq + h) * kD;
  if (len < 1 || len > a.Tmax) {  // outside the contract: zero row, flag it
    if (threadIdx.x < kD) orow[threadIdx.x] = 0;
    if (threadIdx.x == 0 && a.status) *a.status = GROK_ERANGE;
    return;
  }
  const int ns = (len + a.split_keys - 1) / a.split_keys;
  const int c = threadIdx.x % (kD / 4), sg = threadIdx.x / (kD / 4);
  const int64_t base = (static_cast<int64_t>(b) * a.Hkv + g) * a.S;
  // 4 independent partial sums per thread keep 4 loads in flight.
  f32x4 acc[4];
  float l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    l[u] = 0.f;
  }
  int sp = sg;
  for (; sp + 3 * kSplitGroups < ns; sp += 4 * kSplitGroups) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t row = (base + sp + u * kSplitGroups) * a.G + hh;
      acc[u] += *reinterpret_cast<const f32x4 *>(a.part_o + row * kD + 4 * c);
      l[u] += a.part_l[row];
    }
  }
  for (; sp < ns; sp += kSplitGroups) {
    const int64_t row = (base + sp) * a.G + hh;
    acc[0] += *reinterpret_cast<const f32x4 *>(a.part_o + row * kD + 4 * c);
    l[0] += a.part_l[row];
  }
  acc[0] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  l[0] = (l[0] + l[1]) + (l[2] + l[3]);
  red_o[sg][c] = acc[0];
  if (c == 0) red_l[sg] = l[0];
  __syncthreads();
  if (sg == 0) {
    f32x4 o = red_o[0][c];
    float lt = red_l[0];
#pragma unroll
    for (int k = 1; k < kSplitGroups; ++k) {
      o += red_o[k][c];
      lt += red_l[k];
    }
    const u32x2 w = {pack_bf16x2(o[0] / lt, o[1] / lt), pack_bf16x2(o[2] / lt, o[3] / lt)};
    *reinterpret_cast<u32x2 *>(orow + 4 * c) = w;
  }
}

// Keys per split: long splits amortise the partial sums, short ones give a
// small batch enough workgroups to cover the 256 compute units.
int split_keys_for(int B, int Tmax, int Hkv) {
  const int groups = (Hkv + kWavesMax - 1) / kWavesMax;
  const int64_t wgs_long = static_cast<int64_t>(B) * groups * ((Tmax + 127) / 128);
  return wgs_long >= 1024 ? 128 : 32;
}

}  // namespace

size_t decode_workspace_bytes(int B, int Tmax, int Hq, int Hkv) {
  const int sk = split_keys_for(B, Tmax, Hkv);
  const size_t S = (static_cast<size_t>(Tmax) + sk - 1) / sk;
  const size_t G = static_cast<size_t>(Hq / Hkv);
  const size_t n = static_cast<size_t>(B) * Hkv * S * G;
  return n * kD * sizeof(float) + n * sizeof(float);
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
  a.split_keys = split_keys_for(B, Tmax, Hkv);
  a.S = (Tmax + a.split_keys - 1) / a.split_keys;
  const size_t n = static_cast<size_t>(B) * Hkv * a.S * a.G;
  a.part_o = static_cast<float *>(ws);
  a.part_l = a.part_o + n * kD;
  a.status = status;
  a.k1 = 2.f * mult * kLog2e / cap;
  a.k2 = -2.f * cap * kLog2e;
  const int groups = (Hkv + kWavesMax - 1) / kWavesMax;
  const int waves = Hkv < kWavesMax ? Hkv : kWavesMax;
  hipLaunchKernelGGL(decode_split_kernel, dim3(a.S, groups, B), dim3(waves * kWave), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(B * Hq), dim3(kCombineThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace grok

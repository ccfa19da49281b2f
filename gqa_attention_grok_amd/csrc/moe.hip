// MoE FFN sub-layer pieces (Grok-1 walkthrough: ch. 3 "Configuration and
// hyperparameters" §3.5 router; ch. 6 "model.py close reading, part 3" §6.2
// gated FFN and §6.3.1 sandwich norm; ch. 2 "Overall architecture" §2.2 data
// flow and §2.5.1 unnormalised gates). The expert products themselves run on
// the grouped form of the tiled int8 GEMM (linear_int8.hip).
//
//  moe_route_kernel    router logits n @ W_r in fp32 (W_r [d, E] fp32), fp32
//                      softmax, the k most probable experts (ties: lower
//                      index first) and their probabilities as gates.
//  moe_plan_kernel     a stable counting sort of the (token, slot) entries by
//                      expert: group offsets, the token of every grouped row,
//                      and the grouped row of every entry. One workgroup; the
//                      order inside a group is entry order, so the plan (and
//                      everything after it) is deterministic.
//  moe_interleave_kernel  gate and value weights of an expert side by side in
//                      blocks of four columns, for the GeGLU epilogue.
//  moe_combine_kernel  per token: the gate-weighted sum of its k expert rows
//                      (fp32, rounded once), RMSNorm, and the residual add.
#include "common.h"

namespace grok {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteTokens = 8;  // tokens per workgroup
constexpr int kMaxE = 8;
constexpr int kMaxK = 4;

// One workgroup per 8 tokens; thread c8 owns columns 8*c8 .. 8*c8+7 of n and
// rows 8*c8 .. 8*c8+7 of W_r (E floats each), reused for all 8 tokens.
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const bf16_t *n, const float *wr,
                                                                  int32_t *idx, float *gates, int64_t T,
                                                                  int d, int E, int k) {
  __shared__ float red[kRouteThreads / kWave][kRouteTokens][kMaxE];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouteTokens;
  const int tid = threadIdx.x;
  float acc[kRouteTokens][kMaxE];
#pragma unroll
  for (int j = 0; j < kRouteTokens; ++j)
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) acc[j][e] = 0.f;
  for (int c8 = tid; c8 < d / 8; c8 += kRouteThreads) {
    float wv[8][kMaxE];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int e = 0; e < kMaxE; ++e) wv[r][e] = e < E ? wr[static_cast<int64_t>(8 * c8 + r) * E + e] : 0.f;
#pragma unroll
    for (int j = 0; j < kRouteTokens; ++j) {
      const int64_t t = t0 + j < T ? t0 + j : T - 1;
      const u32x4 xv = *reinterpret_cast<const u32x4 *>(n + t * d + 8 * c8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = lo_bf16(xv[q]), b = hi_bf16(xv[q]);
#pragma unroll
        for (int e = 0; e < kMaxE; ++e) acc[j][e] = fmaf(b, wv[2 * q + 1][e], fmaf(a, wv[2 * q][e], acc[j][e]));
      }
    }
  }
  const int wave = tid / kWave;
#pragma unroll
  for (int j = 0; j < kRouteTokens; ++j)
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      const float v = wave_sum(acc[j][e]);
      if ((tid & (kWave - 1)) == 0) red[wave][j][e] = v;
    }
  __syncthreads();
  if (tid < kRouteTokens && t0 + tid < T) {
    const int64_t t = t0 + tid;
    float p[kMaxE];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      float l = 0.f;
#pragma unroll
      for (int u = 0; u < kRouteThreads / kWave; ++u) l += red[u][tid][e];
      p[e] = l;
      if (e < E) mx = fmaxf(mx, l);
    }
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      p[e] = e < E ? expf(p[e] - mx) : 0.f;
      sum += p[e];
    }
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) p[e] = p[e] / sum;
    // k most probable, strictly greater wins: equal probabilities keep the lower index
    unsigned taken = 0;
    for (int s = 0; s < k; ++s) {
      int best = -1;
      float bp = -1.f;
      for (int e = 0; e < E; ++e)
        if (!(taken & (1u << e)) && p[e] > bp) {
          bp = p[e];
          best = e;
        }
      if (best >= 0) taken |= 1u << best;  // best < 0 only for non-finite logits
      idx[t * k + s] = best;
      gates[t * k + s] = best >= 0 ? bp : 0.f;
    }
  }
}

constexpr int kPlanThreads = 1024;

// Stable counting sort of n_ent entries (expert idx[i]) in one workgroup:
// thread q owns the contiguous entries [q*per, (q+1)*per), so the running
// per-expert counts of the threads before it place its entries.
__global__ __launch_bounds__(kPlanThreads) void moe_plan_kernel(const int32_t *idx, int n_ent, int k, int E,
                                                                int32_t *offsets, int32_t *rows,
                                                                int32_t *pos) {
  __shared__ int cnt[kPlanThreads][kMaxE];
  __shared__ int base[kMaxE + 1];
  const int tid = threadIdx.x;
  const int per = (n_ent + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(n_ent, tid * per), i1 = min(n_ent, i0 + per);
  int c[kMaxE];
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) c[e] = 0;
  for (int i = i0; i < i1; ++i) {
    const int e = idx[i];
#pragma unroll
    for (int q = 0; q < kMaxE; ++q) c[q] += (e == q) ? 1 : 0;
  }
  // inclusive scan over the threads (Hillis-Steele: read, barrier, add, barrier)
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) cnt[tid][e] = c[e];
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    int v[kMaxE];
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) v[e] = tid >= off ? cnt[tid - off][e] : 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) cnt[tid][e] += v[e];
    __syncthreads();
  }
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < kMaxE; ++e) {
      base[e] = acc;
      acc += e < E ? cnt[kPlanThreads - 1][e] : 0;
    }
    base[kMaxE] = acc;
    for (int e = 0; e <= E; ++e) offsets[e] = e < E ? base[e] : acc;
  }
  __syncthreads();
  int run[kMaxE];
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) run[e] = base[e] + cnt[tid][e] - c[e];  // this thread's first slot
  for (int i = i0; i < i1; ++i) {
    const int e = idx[i];
    int p = -1;
#pragma unroll
    for (int q = 0; q < kMaxE; ++q)
      if (e == q && q < E) p = run[q]++;
    pos[i] = p;  // -1: expert index out of range, the entry is dropped
    if (p >= 0) rows[p] = i / k;
  }
}

// wgv[kk][8q + j] = wg[kk][4q + j], wgv[kk][8q + 4 + j] = wv[kk][4q + j]; same for scales.
__global__ __launch_bounds__(256) void moe_interleave_kernel(const int8_t *wg, const int8_t *wv, const float *sg,
                                                             const float *sv, int8_t *wgv, float *sgv, int K,
                                                             int F) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // one 4-byte group
  const int64_t ngroups = static_cast<int64_t>(K) * (F / 4);
  if (i < ngroups) {
    const int64_t kk = i / (F / 4);
    const int q = static_cast<int>(i % (F / 4));
    const uint32_t g = *reinterpret_cast<const uint32_t *>(wg + kk * F + 4 * q);
    const uint32_t v = *reinterpret_cast<const uint32_t *>(wv + kk * F + 4 * q);
    *reinterpret_cast<u32x2 *>(wgv + kk * 2 * F + 8 * q) = u32x2{g, v};
  }
  if (i < F / 4) {
    const int q = static_cast<int>(i);
    *reinterpret_cast<f32x4 *>(sgv + 8 * q) = *reinterpret_cast<const f32x4 *>(sg + 4 * q);
    *reinterpret_cast<f32x4 *>(sgv + 8 * q + 4) = *reinterpret_cast<const f32x4 *>(sv + 4 * q);
  }
}

constexpr int kCombThreads = 256;
constexpr int kCombChunks = 4;  // 8-element chunks per thread: d <= 8192

// One workgroup per token: mix = bf16(sum_s gate_s * y[pos_s]) (fp32 sum),
// out = x + bf16(mix * rsqrt(mean(mix^2) + eps)) (unit scale).
__global__ __launch_bounds__(kCombThreads) void moe_combine_kernel(const bf16_t *ys, const int32_t *pos,
                                                                   const float *gates, const bf16_t *x,
                                                                   bf16_t *out, int d, int k, float eps) {
  __shared__ float red[kCombThreads / kWave];
  const int64_t t = blockIdx.x;
  const int nch = d / 8;
  float mix[kCombChunks][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kCombChunks; ++c) {
    const int ci = threadIdx.x + c * kCombThreads;
#pragma unroll
    for (int j = 0; j < 8; ++j) mix[c][j] = 0.f;
    if (ci >= nch) continue;
    for (int s = 0; s < k; ++s) {
      const int p = pos[t * k + s];
      if (p < 0) continue;
      const float gsc = gates[t * k + s];
      const u32x4 w = *reinterpret_cast<const u32x4 *>(ys + static_cast<int64_t>(p) * d + 8 * ci);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mix[c][2 * q] = fmaf(gsc, lo_bf16(w[q]), mix[c][2 * q]);
        mix[c][2 * q + 1] = fmaf(gsc, hi_bf16(w[q]), mix[c][2 * q + 1]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mix[c][j] = bf16_to_f32(f32_to_bf16(mix[c][j]));  // the sum handed on in bf16
      ss += mix[c][j] * mix[c][j];
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int u = 0; u < kCombThreads / kWave; ++u) tot += red[u];
  const float r = rsqrtf(tot / static_cast<float>(d) + eps);
#pragma unroll
  for (int c = 0; c < kCombChunks; ++c) {
    const int ci = threadIdx.x + c * kCombThreads;
    if (ci >= nch) continue;
    const u32x4 xr = *reinterpret_cast<const u32x4 *>(x + t * d + 8 * ci);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = lo_bf16(xr[q]) + bf16_to_f32(f32_to_bf16(mix[c][2 * q] * r));
      const float b = hi_bf16(xr[q]) + bf16_to_f32(f32_to_bf16(mix[c][2 * q + 1] * r));
      o[q] = pack_bf16x2(a, b);
    }
    *reinterpret_cast<u32x4 *>(out + t * d + 8 * ci) = o;
  }
}

}  // namespace

int moe_max_experts() { return kMaxE; }
int moe_max_k() { return kMaxK; }
int moe_max_width() { return kCombChunks * kCombThreads * 8; }

namespace {
size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }
}  // namespace

MoeWorkspace moe_workspace(int64_t T, int d, int F, int E, int k) {
  const size_t ent = static_cast<size_t>(T) * k;
  MoeWorkspace w = {};
  size_t o = 0;
  w.n = o;       o += align256(static_cast<size_t>(T) * d * 2);
  w.idx = o;     o += align256(ent * 4);
  w.gates = o;   o += align256(ent * 4);
  w.offsets = o; o += align256(static_cast<size_t>(E + 1) * 4);
  w.rows = o;    o += align256(ent * 4);
  w.pos = o;     o += align256(ent * 4);
  w.h = o;       o += align256(ent * F * 2);
  w.y = o;       o += align256(ent * d * 2);
  w.total = o;
  return w;
}

hipError_t launch_moe_route(const void *n, const float *wr, int32_t *idx, float *gates, int64_t T, int d, int E,
                            int k, hipStream_t s) {
  const int64_t blocks = (T + kRouteTokens - 1) / kRouteTokens;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(moe_route_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kRouteThreads), 0, s,
                     static_cast<const bf16_t *>(n), wr, idx, gates, T, d, E, k);
  return hipGetLastError();
}

hipError_t launch_moe_plan(const int32_t *idx, int n_ent, int k, int E, int32_t *offsets, int32_t *rows,
                           int32_t *pos, hipStream_t s) {
  hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, idx, n_ent, k, E, offsets, rows, pos);
  return hipGetLastError();
}

hipError_t launch_moe_interleave(const int8_t *wg, const int8_t *wv, const float *sg, const float *sv,
                                 int8_t *wgv, float *sgv, int K, int F, hipStream_t s) {
  const int64_t ngroups = static_cast<int64_t>(K) * (F / 4);
  const int64_t blocks = (ngroups + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(moe_interleave_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, wg, wv, sg, sv,
                     wgv, sgv, K, F);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void *ys, const int32_t *pos, const float *gates, const void *x, void *out,
                              int64_t T, int d, int k, float eps, hipStream_t s) {
  if (T > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(static_cast<unsigned>(T)), dim3(kCombThreads), 0, s,
                     static_cast<const bf16_t *>(ys), pos, gates, static_cast<const bf16_t *>(x),
                     static_cast<bf16_t *>(out), d, k, eps);
  return hipGetLastError();
}

// norm -> route -> plan -> grouped GeGLU up projection (rows gathered by
// token) -> grouped down projection -> gate-weighted combine, norm, residual.
hipError_t launch_moe_ffn(const void *x, const float *w_router, int E, int k, const int8_t *const *wgv,
                          const float *const *sgv, const int8_t *const *w1, const float *const *s1, int64_t T,
                          int d, int F, float eps, int32_t *idx, float *gates, void *workspace, void *out,
                          hipStream_t s) {
  const MoeWorkspace L = moe_workspace(T, d, F, E, k);
  char *ws = static_cast<char *>(workspace);
  void *n = ws + L.n;
  int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
  int32_t *rows = reinterpret_cast<int32_t *>(ws + L.rows);
  int32_t *pos = reinterpret_cast<int32_t *>(ws + L.pos);
  void *h = ws + L.h;
  void *y = ws + L.y;
  if (!idx) idx = reinterpret_cast<int32_t *>(ws + L.idx);
  if (!gates) gates = reinterpret_cast<float *>(ws + L.gates);
  const int64_t ent = T * k;
  hipError_t e = launch_rmsnorm(x, nullptr, nullptr, n, T, d, eps, GROK_BF16, s);
  if (e == hipSuccess) e = launch_moe_route(n, w_router, idx, gates, T, d, E, k, s);
  if (e == hipSuccess) e = launch_moe_plan(idx, static_cast<int>(ent), k, E, offsets, rows, pos, s);
  if (e == hipSuccess) e = launch_linear_int8_grouped(n, rows, offsets, E, wgv, sgv, h, ent, d, 2 * F, true, s);
  if (e == hipSuccess) e = launch_linear_int8_grouped(h, nullptr, offsets, E, w1, s1, y, ent, F, d, false, s);
  if (e == hipSuccess) e = launch_moe_combine(y, pos, gates, x, out, T, d, k, eps, s);
  return e;
}

}  // namespace grok

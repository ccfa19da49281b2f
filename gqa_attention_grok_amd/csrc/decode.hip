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
// Kernel 1 (decode_split_kernel): one workgroup of 4 waves per (sequence, KV
// head, split of 128 cache slots). The whole split -- 128 K rows and 128 V
// rows of the head, 64 KB -- is requested up front: K straight into the
// registers that feed the MFMA (each lane loads its own fragments), V HBM ->
// LDS (global_load_lds) for the transpose reads. With 33 KB of LDS per
// workgroup, four workgroups per CU keep up to 256 KB in flight and overlap
// one's loads with another's compute. Wave w owns slots 32w .. 32w+31 of the
// split: it loads them itself (no barrier before the compute) and runs, with
// the G <= 16 query heads of the KV head as MFMA rows (unused rows zero),
//   S^T[slot, head] = K . Q^T    (slot rows permuted as in the prefill K tile)
//   O^T[d, head]  += V^T . P^T   (V^T from LDS transpose reads)
// using the tile layouts of the prefill kernel. The softmax uses the fixed shift
// exp(c - cap): unmasked softcapped logits lie in [-cap, cap], so partial
// results are plain sums (sum p*v, sum p) with no running maximum to
// reconcile. The four waves' partials are added in LDS and one partial per
// split is written.
// Kernel 2 (decode_combine_kernel): one workgroup per (sequence, query head)
// adds the partials of the splits and writes bf16 sum(p*v) / sum(p).
//
// With the append fused (decode_split_kernel<true>, §4.4: RoPE before the
// cache write), the new token's position is step[b] and the cache holds slots
// [0, step[b]) only: every workgroup rotates its query heads in registers
// (the rotation pairs dims i and i + 64, which one lane holds together), the
// workgroup whose split contains slot step[b] takes that slot's K row from
// the new k (rotated the same way) and its V row from the new v, and writes
// both into the cache. The rotation is rope_rotate of common.h at the phases
// of rope_phase, rounded to bf16 as the unfused append rounds it, so the
// results are those of the separate append + decode calls.
#include <mutex>

#include "attn_tile.h"

namespace grok {

// Split-partial buffer of the allocation-free decode entry point: one copy per
// GPU, held from the library's load on that GPU until the process ends. Host
// code must not pass this name to a kernel (on the host it is a stand-in, not
// a device address): decode_static_scratch() returns the device address.
__device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];

namespace {

using namespace attn;

constexpr int kD = 128;
constexpr int kSplit = 128;  // cache slots per workgroup
constexpr int kSplitWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;  // dies of the device: workgroup i is dispatched to die i % 8

struct DecodeArgs {
  const bf16_t *q, *kc, *vc;
  const int32_t *kv_len;
  bf16_t *out;
  float *part_o;  // [B, Hkv, S, G, D]
  float *part_l;  // [B, Hkv, S, G]
  int32_t *status;
  int B, Tmax, Hq, Hkv, G, S, split_keys;
  int by_die;  // workgroup layout: by die (several sequences) or splits fastest
  float k1, k2inv;
  // fused append: q is unrotated, len = step[b] + 1
  const bf16_t *kn, *vn;  // [B, Hkv, D] new k (unrotated), v
  bf16_t *kcw, *vcw;      // the caches, written at slot step[b]
  const int32_t *step;
  int32_t *new_step;      // or NULL
  bf16_t *q_out;          // rotated q, or NULL
  float inv[kD / 2];      // RoPE inv_freq
};

// kSpec (small grids, every workgroup resident at once): the loads are issued
// before the sequence length is known. They cover the split's slots clamped to
// the cache (every address stays inside [B, Tmax]); slots past the sequence
// are masked out of the weights, and in LDS their V rows are replaced by zeros
// (or, with the append, by the new v row) before the P.V product, so the
// unread contents of the cache cannot reach the output. The new k / v rows
// are loaded by every workgroup and used by the one holding the new slot.
// This takes the length load off the path to the first K/V bytes; the
// workgroups past the sequence load a split they do not use, so it is chosen
// only where the grid fits the device in one go.
template <bool kAppend, bool kSpec>
__global__ __launch_bounds__(kSplitWaves * kWave, 3) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char Vs[kSplit * kRowBytes];
  __shared__ float red_l[kSplitWaves][16];
  __shared__ __attribute__((aligned(16))) float rcs[kAppend ? kD / 2 : 1], rsn[kAppend ? kD / 2 : 1];

  // Workgroup -> (split s, KV head g, sequence b). Die x = blockIdx.x % 8
  // takes, sequence by sequence with splits fastest, the KV heads g with
  // (b + g) % 8 == x: each die gets one head of every sequence (the same work
  // per die for any length mix) and the head it reads rotates with b. With a
  // KV head count that is not a multiple of 8, die x takes the pairs
  // b * Hkv + g = x (mod 8). A single sequence runs with splits fastest, heads
  // next (measured faster for it). Only speed depends on the dispatch order:
  // every (split, KV head, sequence) has exactly one workgroup either way.
  const int xi = blockIdx.x % kXcds, xj = blockIdx.x / kXcds;
  const int pl = xj / a.S;
  int s = xj % a.S, b, g;
  if (!a.by_die) {
    s = blockIdx.x % a.S;
    g = (blockIdx.x / a.S) % a.Hkv;
    b = blockIdx.x / (a.S * a.Hkv);
  } else if (a.Hkv % kXcds == 0) {
    const int hk = a.Hkv / kXcds;
    b = pl / hk;
    g = (xi - b % kXcds + kXcds) % kXcds + kXcds * (pl % hk);
  } else {
    const int pair = xi + kXcds * pl;
    b = pair / a.Hkv;
    g = pair % a.Hkv;
  }
  if (b >= a.B) return;
  const int sbase = s * kSplit;
  int len = 0;
  if constexpr (!kSpec) {
    len = kAppend ? a.step[b] + 1 : a.kv_len[b];
    if (kAppend && s == 0 && g == 0 && threadIdx.x == 0 && a.new_step)
      a.new_step[b] = (len >= 1 && len <= a.Tmax) ? len : len - 1;
    if (len < 1 || len > a.Tmax) return;  // reported by the combine kernel
    if (sbase >= len) return;  // whole workgroup: no barrier is skipped
  }

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lr = lane % 16, lg = lane / 16;
  // highest slot the loads read: the sequence's last one, or (kSpec) the cache's
  const int lim = kSpec ? a.Tmax - 1 : len - 1;

  // Q fragment: head row lr (zero beyond G), dims 32*kk + 8*lg; then this
  // wave's 32 K slots: the S^T A operand of key block kb is, for lane
  // (lr, lg), slot 32*wave + k_row_key(16*kb + lr) of the split, dims
  // 32*kk + 8*lg .. +8. Both go straight into registers; then the V slots,
  // HBM -> LDS: instruction j (0..7) fills LDS rows R = 32*wave + 4*j + L/16
  // (slot R), lane L writing physical chunk L%16. Slots past the sequence read
  // its last slot (masked below). The register loads are inline assembly and
  // issued first, so one explicit wait (vmcnt(8)) makes Q and K usable while
  // the eight V loads stay in flight. With the append fused, slot `last`
  // (and the clamped slots past it) reads the new k / v rows instead.
  const int64_t rstride = static_cast<int64_t>(a.Hkv) * kD;
  const bf16_t *kbase = a.kc + (static_cast<int64_t>(b) * a.Tmax * a.Hkv + g) * kD;
  const bf16_t *vbase = a.vc + (static_cast<int64_t>(b) * a.Tmax * a.Hkv + g) * kD;
  const int64_t nrow = (static_cast<int64_t>(b) * a.Hkv + g) * kD;  // new k / v row
  const bool qok = lr < a.G;
  // kSpec: the length is the first of the loads below (a vector load, waited
  // for on its own by count while the others fly)
  uint32_t lenv = 0;
  if constexpr (kSpec)
    asm volatile("global_load_dword %0, %1, off" : "=v"(lenv) : "v"(kAppend ? a.step + b : a.kv_len + b) : "memory");
  u32x4 qw[4], kf[2][4];
  {
    const bf16_t *qp = a.q + (static_cast<int64_t>(b) * a.Hq + g * a.G + (qok ? lr : 0)) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(qw[kk]) : "v"(qp + 32 * kk + 8 * lg) : "memory");
  }
  bool knew[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kj = min(sbase + 32 * wave + k_row_key(16 * kb + lr), lim);
    knew[kb] = kAppend && !kSpec && kj == lim;
    const bf16_t *kp = (knew[kb] ? a.kn + nrow : kbase + kj * rstride) + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(kf[kb][kk]) : "v"(kp + 32 * kk) : "memory");
  }
  // kSpec + append: the new k row (this lane's dims of it) and chunk lane % 16
  // of the new v row, for the workgroup that holds the new slot
  u32x4 nk[kAppend && kSpec ? 4 : 1], nv;
  if constexpr (kAppend && kSpec) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(nk[kk]) : "v"(a.kn + nrow + 32 * kk + 8 * lg) : "memory");
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(nv) : "v"(a.vn + nrow + 8 * (lane % 16)) : "memory");
  }
  {
    const int lrow = lane / 16, lchunk = lane % 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int R = 32 * wave + 4 * j + lrow;
      const int vj = min(sbase + R, lim);
      const bf16_t *vrow = (kAppend && !kSpec && vj == lim) ? a.vn + nrow : vbase + vj * rstride;
      __builtin_amdgcn_global_load_lds(vrow + 8 * (lchunk ^ v_swz(R)),
                                       (lds_void *)(&Vs[(32 * wave + 4 * j) * kRowBytes]), 16, 0, 0);
    }
  }
  if constexpr (kSpec) {
    // loads issued after the length: q 4, K 8, new k / v rows 5 (append), V 8
    if constexpr (kAppend)
      asm volatile("s_waitcnt vmcnt(25)" : "+v"(lenv) : : "memory");
    else
      asm volatile("s_waitcnt vmcnt(20)" : "+v"(lenv) : : "memory");
    len = __builtin_amdgcn_readfirstlane(static_cast<int>(lenv)) + (kAppend ? 1 : 0);
    if (kAppend && s == 0 && g == 0 && threadIdx.x == 0 && a.new_step)
      a.new_step[b] = (len >= 1 && len <= a.Tmax) ? len : len - 1;
  }
  const int last = len - 1;
  if constexpr (kAppend) {
    // cos/sin of the new position, once per workgroup, while the loads fly
    // (the table is read with uniform indices: scalar loads, which do not
    // count against the vector-memory wait below)
    float inv = 0.f;
#pragma unroll
    for (int i = 0; i < kD / 2; ++i) inv = threadIdx.x == i ? a.inv[i] : inv;
    if (threadIdx.x < kD / 2) rope_phase(last, inv, rsn[threadIdx.x], rcs[threadIdx.x]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // Workgroup barrier without a memory fence (a fence would wait for the
    // loads in flight); the memory clobber keeps the table reads below it.
    asm volatile("s_barrier" ::: "memory");
  }

  asm volatile("s_waitcnt vmcnt(8)"
               : "+v"(qw[0]), "+v"(qw[1]), "+v"(qw[2]), "+v"(qw[3]), "+v"(kf[0][0]), "+v"(kf[0][1]), "+v"(kf[0][2]),
                 "+v"(kf[0][3]), "+v"(kf[1][0]), "+v"(kf[1][1]), "+v"(kf[1][2]), "+v"(kf[1][3])
               :
               : "memory");
  if constexpr (kSpec) {
    if constexpr (kAppend)  // landed with the wait above (issued before the V loads)
      asm volatile("" : "+v"(nk[0]), "+v"(nk[1]), "+v"(nk[2]), "+v"(nk[3]), "+v"(nv));
    if (len < 1 || len > a.Tmax || sbase >= len) {  // whole workgroup
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the V loads write this workgroup's LDS
      return;
    }
    if constexpr (kAppend) {
      // slots at or past the new one take the new k row (as the clamped rows
      // of the other form do)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        knew[kb] = sbase + 32 * wave + k_row_key(16 * kb + lr) >= last;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kf[kb][kk] = knew[kb] ? nk[kk] : kf[kb][kk];
      }
    }
  }
  if constexpr (kAppend) {
    // lane (lr, lg) holds dims 32*kk + 8*lg + e of its rows: kk = 0, 1 pair
    // with kk = 2, 3 (dim + 64)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float cs[8], sn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cs[e] = rcs[32 * kk + 8 * lg + e];
        sn[e] = rsn[32 * kk + 8 * lg + e];
      }
      rope8(qw[kk], qw[kk + 2], cs, sn);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (knew[kb]) rope8(kf[kb][kk], kf[kb][kk + 2], cs, sn);
    }
    // the rotated q (split 0) and the rotated new k row (its own slot) out
    if (s == 0 && qok && a.q_out) {
      bf16_t *qo = a.q_out + (static_cast<int64_t>(b) * a.Hq + g * a.G + lr) * kD + 8 * lg;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) *reinterpret_cast<u32x4 *>(qo + 32 * kk) = qw[kk];
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (knew[kb] && sbase + 32 * wave + k_row_key(16 * kb + lr) == last) {
        bf16_t *ko = a.kcw + (static_cast<int64_t>(b) * a.Tmax + last) * rstride + g * kD + 8 * lg;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) *reinterpret_cast<u32x4 *>(ko + 32 * kk) = kf[kb][kk];
      }
  }
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, qok ? qw[kk] : u32x4{0, 0, 0, 0});

  // S^T for the wave's 32 slots; accumulator slot v of lane l is slot
  // 32*wave + 8*lg + 4*kb + v of the split.
  f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kb][kk]), qf[kk], sacc[kb],
                                                         0, 0, 0);
  // p = exp2(k2 / (1 + exp2(k1*s))), masked past the sequence; bf16 for P.V.
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float ex = __builtin_amdgcn_exp2f(sacc[e >> 2][e & 3] * a.k1);
    const float pv = __builtin_amdgcn_exp2f(__builtin_amdgcn_rcpf(__builtin_fmaf(ex, a.k2inv, a.k2inv)));
    p[e] = (sbase + 32 * wave + 8 * lg + e <= last) ? pv : 0.f;
  }
  const u32x4 pw = {cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]), cvt_pk_bf16(p[4], p[5]),
                    cvt_pk_bf16(p[6], p[7])};
  // Row sum of the bf16-rounded weights that P.V uses.
  float lsum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) lsum = add_bf16_pair(lsum, pw[e]);
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);

  // This wave's V slots have landed (it reads only those). The softmax results
  // pass through the wait so that it is not hoisted above the softmax.
  u32x4 pw2 = pw;
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(pw2), "+v"(lsum) : : "memory");
  const bf16x8 pf = __builtin_bit_cast(bf16x8, pw2);
  if constexpr (kSpec) {
    // this wave's V rows past the sequence: zeros, or the new v row from the
    // new slot on (what the clamped loads of the other form put there)
    const int first = kAppend ? last : last + 1;
    if (sbase + 32 * wave + 31 >= first) {  // wave-uniform
      const u32x4 fill = kAppend ? nv : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int R = 32 * wave + 4 * j + lane / 16;
        if (sbase + R >= first)
          *reinterpret_cast<u32x4 *>(&Vs[R * kRowBytes + 16 * ((lane % 16) ^ v_swz(R))]) = fill;
      }
    }
  }
  if constexpr (kAppend) {
    // the new v row landed in LDS row last - sbase of this wave: copy it to
    // its cache slot (16 lanes x 16 bytes, undoing the chunk swizzle)
    const int R = last - sbase;
    if (R >= 32 * wave && R < 32 * wave + 32 && lane < 16) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(&Vs[R * kRowBytes + 16 * (lane ^ v_swz(R))]);
      *reinterpret_cast<u32x4 *>(a.vcw + (static_cast<int64_t>(b) * a.Tmax + last) * rstride + g * kD + 8 * lane) = v;
    }
  }

  // O^T += V^T . P^T: lane l's V^T fragment (dim 16*db + lr, slots 8*lg .. +7
  // of the wave's 32) from two transpose reads of 4 slots.
  f32x4 oacc[8];
  {
    const int vrow0 = 32 * wave + 8 * lg + lr / 4;
    const int gs = v_swz(vrow0) >> 1;
    const uint32_t vb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)(&Vs[0]))) +
                        vrow0 * kRowBytes + 16 * ((lr & 3) >> 1) + 8 * (lr & 1);
    u32x2 lo[8], hi[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint32_t ad = vb + 32 * (db ^ gs);
      lo[db] = lds_read_tr16<0>(ad);
      hi[db] = lds_read_tr16<4 * kRowBytes>(ad);
    }
    lds_wait<8>(lo, hi);
    lds_wait<0>(lo + 4, hi + 4);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[db][0], lo[db][1], hi[db][0], hi[db][1]});
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
  }

  // Add the four waves' partials (lane l: head row lr, dims 16*db + 4*lg + v)
  // in LDS, reusing the V tile, and write this split's partial.
  __syncthreads();  // every wave is done with Vs
  float *red_o = reinterpret_cast<float *>(Vs);  // [4][16][128]
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *reinterpret_cast<f32x4 *>(&red_o[(wave * 16 + lr) * kD + 16 * db + 4 * lg]) = oacc[db];
  if (lg == 0) red_l[wave][lr] = lsum;
  __syncthreads();
  const int64_t pbase = ((static_cast<int64_t>(b) * a.Hkv + g) * a.S + s) * a.G;
  for (int it = threadIdx.x; it < a.G * (kD / 4); it += kSplitWaves * kWave) {
    const int row = it / (kD / 4), c4 = it % (kD / 4);
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) o += *reinterpret_cast<const f32x4 *>(&red_o[(w * 16 + row) * kD + 4 * c4]);
    *reinterpret_cast<f32x4 *>(a.part_o + (pbase + row) * kD + 4 * c4) = o;
  }
  if (threadIdx.x < a.G) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) l += red_l[w][threadIdx.x];
    a.part_l[pbase + threadIdx.x] = l;
  }
}

constexpr int kCombineThreads = 256;
constexpr int kSplitGroups = kCombineThreads / (kD / 4);  // 8 groups of 32 float4 lanes

// One workgroup per (sequence, query head): 32 lanes x float4 cover the head's
// 128 outputs; 8 groups take every 8th split; the groups are added in LDS.
// kSpec: the first round of partial loads goes out before the length is known
// (splits past the sequence hold stale values and are not added).
template <bool kSpec>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeArgs a) {
  __shared__ f32x4 red_o[kSplitGroups][kD / 4];
  __shared__ float red_l[kSplitGroups];
  const int b = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int g = h / a.G, hh = h % a.G;
  const int c = threadIdx.x % (kD / 4), sg = threadIdx.x / (kD / 4);
  const int64_t base = (static_cast<int64_t>(b) * a.Hkv + g) * a.S;
  // Up to 8 partials per thread per round, all loads issued before any sum, so
  // a round costs one memory latency (one round covers 64 splits = 8192 slots).
  constexpr int kU = 8;
  f32x4 vo[kU];
  float vl[kU];
  auto load_round = [&](int sp0, int ns) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int sp = sp0 + u * kSplitGroups;
      const int64_t row = (base + (sp < ns ? sp : 0)) * a.G + hh;
      vo[u] = *reinterpret_cast<const f32x4 *>(a.part_o + row * kD + 4 * c);
      vl[u] = a.part_l[row];
    }
  };
  if constexpr (kSpec) load_round(sg, a.S);
  const int len = a.step ? a.step[b] + 1 : a.kv_len[b];
  bf16_t *orow = a.out + (static_cast<int64_t>(b) * a.Hq + h) * kD;
  if (len < 1 || len > a.Tmax) {  // outside the contract: zero row, flag it
    if (threadIdx.x < kD) orow[threadIdx.x] = 0;
    if (threadIdx.x == 0 && a.status) *a.status = GROK_ERANGE;
    return;
  }
  const int ns = (len + a.split_keys - 1) / a.split_keys;
  f32x4 acc[4];
  float l[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    l[u] = 0.f;
  }
  for (int sp0 = sg; sp0 < ns; sp0 += kU * kSplitGroups) {
    if (!kSpec || sp0 != sg) load_round(sp0, ns);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (sp0 + u * kSplitGroups < ns) {
        acc[u % 4] += vo[u];
        l[u % 4] += vl[u];
      }
    }
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

}  // namespace

hipError_t decode_static_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *dev_ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!dev_ptr[dev]) {
    // once per device, with that device current: its own copy's address
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

namespace {
// One workgroup per (split, pair) slot, the pairs rounded up to a multiple of
// the die count; 0 when that does not fit a grid dimension.
int64_t split_blocks(const DecodeArgs &a) {
  const int64_t pairs = static_cast<int64_t>(a.B) * a.Hkv;
  const int64_t n = kXcds * ((pairs + kXcds - 1) / kXcds) * a.S;
  return n > 0x7fffffff ? 0 : n;
}

// Grids up to this many split workgroups are resident at once (256 CUs, three
// workgroups each by the kernel's launch bounds): they take the speculative
// loads.
constexpr int64_t kSpecMaxBlocks = 256 * 3;

template <bool kAppend>
hipError_t launch_split_combine(const DecodeArgs &a, hipStream_t st) {
  const int64_t nblk = split_blocks(a);
  if (nblk == 0) return hipErrorInvalidConfiguration;
  const bool spec = nblk <= kSpecMaxBlocks;
  const dim3 grid(static_cast<unsigned>(nblk)), block(kSplitWaves * kWave);
  if (spec)
    hipLaunchKernelGGL((decode_split_kernel<kAppend, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<kAppend, false>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid(static_cast<unsigned>(a.B * a.Hq));
  if (spec)
    hipLaunchKernelGGL(decode_combine_kernel<true>, cgrid, dim3(kCombineThreads), 0, st, a);
  else
    hipLaunchKernelGGL(decode_combine_kernel<false>, cgrid, dim3(kCombineThreads), 0, st, a);
  return hipGetLastError();
}
}  // namespace

size_t decode_workspace_bytes(int B, int Tmax, int Hq, int Hkv) {
  const size_t S = (static_cast<size_t>(Tmax) + kSplit - 1) / kSplit;
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
  a.split_keys = kSplit;
  a.S = (Tmax + kSplit - 1) / kSplit;
  a.by_die = B > 1;
  const size_t n = static_cast<size_t>(B) * Hkv * a.S * a.G;
  a.part_o = static_cast<float *>(ws);
  a.part_l = a.part_o + n * kD;
  a.status = status;
  a.k1 = 2.f * mult * kLog2e / cap;
  a.k2inv = 1.f / (-2.f * cap * kLog2e);
  a.kn = a.vn = nullptr;
  a.kcw = a.vcw = nullptr;
  a.step = nullptr;
  a.new_step = nullptr;
  a.q_out = nullptr;
  return launch_split_combine<false>(a, st);
}

hipError_t launch_decode_append(const void *q, const void *kn, const void *vn, void *kc, void *vc,
                                const int32_t *step, int32_t *new_step, void *q_out, void *out,
                                void *ws, int32_t *status, int B, int Tmax, int Hq, int Hkv,
                                float mult, float cap, const RopeFreqs &f, hipStream_t st) {
  DecodeArgs a;
  a.q = static_cast<const bf16_t *>(q);
  a.kc = static_cast<const bf16_t *>(kc);
  a.vc = static_cast<const bf16_t *>(vc);
  a.kv_len = nullptr;
  a.out = static_cast<bf16_t *>(out);
  a.B = B;
  a.Tmax = Tmax;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.split_keys = kSplit;
  a.S = (Tmax + kSplit - 1) / kSplit;
  a.by_die = B > 1;
  const size_t n = static_cast<size_t>(B) * Hkv * a.S * a.G;
  a.part_o = static_cast<float *>(ws);
  a.part_l = a.part_o + n * kD;
  a.status = status;
  a.k1 = 2.f * mult * kLog2e / cap;
  a.k2inv = 1.f / (-2.f * cap * kLog2e);
  a.kn = static_cast<const bf16_t *>(kn);
  a.vn = static_cast<const bf16_t *>(vn);
  a.kcw = static_cast<bf16_t *>(kc);
  a.vcw = static_cast<bf16_t *>(vc);
  a.step = step;
  a.new_step = new_step;
  a.q_out = static_cast<bf16_t *>(q_out);
  for (int i = 0; i < kD / 2; ++i) a.inv[i] = f.inv[i];
  return launch_split_combine<true>(a, st);
}

}  // namespace grok

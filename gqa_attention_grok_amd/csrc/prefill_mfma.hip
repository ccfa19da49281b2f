// Causal grouped-query flash attention for prefill on gfx950 bf16 MFMA, D = 128.
//
// Method (Grok-1 walkthrough, ch. 4 "model.py close reading, part 1", §4.5.2 to
// §4.5.4; mask from ch. 6 "model.py close reading, part 3", §6.4.2):
//   z = mult * <q_i, k_j>, c = cap*tanh(z/cap), masked -> -1e30, softmax, P.V.
//
// Work decomposition
//   A workgroup (4 waves) owns 12 "row blocks" of 16 query rows. A row block is
//   16 consecutive positions of one query head. The 12 blocks are Gc heads of
//   one KV group x (12/Gc) position blocks, so every K/V tile staged in LDS is
//   used by all those heads (for Grok-1's 6:1 grouping: 6 heads x 32 positions).
//   Each wave owns 3 row blocks and walks the causal key range in tiles of 64
//   keys, double-buffered in LDS (one barrier per tile).
//
// Data movement
//   K and V tiles go from HBM straight into LDS (global_load_lds, 16 bytes per
//   lane, no staging registers): while a tile is computed the next one is in
//   flight. Rows are 256 bytes with the 16-byte chunks XOR-swizzled by row, so
//   the fragment reads below are free of bank conflicts.
//
// MFMA formulation (v_mfma_f32_16x16x32_bf16), transposed so that each lane
// always holds data of query row (lane % 16):
//   S^T[key, row]  = K[key, :] . Q[row, :]^T          A = K (LDS), B = Q (regs)
//   O^T[d, row]   += V^T[d, key] . P^T[key, row]      A = V^T (LDS), B = P (regs)
//   K rows are stored in the order the S^T A operand reads them (a permutation
//   of each 32-key half) so that the S^T accumulator of lane l holds keys
//   8*(l/16) .. 8*(l/16)+7 of the half for its row -- exactly the B-operand
//   layout P needs for the P.V product, so P never leaves registers. The V^T
//   A operand is read from row-major V with the LDS transpose read
//   (ds_read_b64_tr_b16): in each group of 16 lanes, output lane 4a+j receives
//   element j of the 4 elements addressed by source lanes a, a+4, a+8, a+12.
//
// Softmax without a running max: after the softcap every unmasked logit lies in
// [-cap, cap], so p = exp(c - cap) is in [exp(-2cap), 1] -- no overflow, and no
// underflow below fp32/bf16 normals for cap <= 40. Softmax is shift-invariant,
// so this is the same distribution as the max-subtracted form, without the
// per-tile max reduction and rescaling of O. With r = 1/(1+exp(2z/cap)):
//   c - cap = -2*cap*r,   p = exp2(-2*cap*log2(e) * r).
// Masked logits give p = 0 exactly. A row with no unmasked key (only possible
// with key padding) takes the -1e30 semantics of the pages: the uniform mean
// of all T value rows, computed in the epilogue for such rows only.
#include "attn_tile.h"

namespace grok {
namespace {

using namespace attn;

constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRB = 3;             // row blocks per wave
constexpr int kRowBlocks = kWaves * kRB;
constexpr int kBN = 64;            // keys per tile (two halves of 32 per MFMA step)
constexpr int kTileBytes = kBN * kRowBytes;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSortMaxB = 64;      // chunked prefill: batches ordered by cached length up to this size

struct PrefillArgs {
  const bf16_t *q, *k, *v;
  const uint8_t *key_valid;
  const int32_t *offset;  // kOffset: position of each sequence's first query row
  int32_t *status;
  bf16_t *out;
  int64_t kv_rows;
  int B, T, Hq, Hkv, G, Gc, npb, nhc, nqt;
  float k1, k2inv;  // exp2 scale inside the softcap; 1 / (outer exp2 scale)
  const float *rtab;  // kRopeQ: [T][128] cos of pairs 0..63, then sin, per position
};

// kOffset: the T query rows of sequence b sit at positions offset[b] + t (a
// chunk after a cached prefix) and attend keys [0, offset[b] + t] of K/V
// read in place from the cache (kv_rows = its capacity); without it the
// offset is 0 and the code is the plain causal prefill.
// kRopeQ: q arrives unrotated and each query row is rotated at its position
// while its fragments are loaded (ch. 4 §4.3.1), from the table rtab of
// rope_phase values: the bits of grok_rope followed by the plain prefill.
template <bool kHasValid, bool kOffset, bool kRopeQ = false>
__global__ __launch_bounds__(kThreads, 2) void prefill_mfma_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char Ks[2][kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kvs[2][kBN];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform, in an SGPR
  const int lr = lane % 16;  // this lane's row inside a row block
  const int lg = lane / 16;  // this lane's k/key group

  // blockIdx -> (g, head chunk, sequence, query tile); g fastest so that, with
  // 8 KV heads, all tiles of one KV head land on one XCD's L2; the query tile
  // slowest, longest first, so that the causally longest tiles of every
  // sequence start before any shorter one (the grid runs in several rounds of
  // resident workgroups, and the shortest tiles fill the last round).
  int id = blockIdx.x;
  const int g = id % a.Hkv;
  id /= a.Hkv;
  const int hc = id % a.nhc;
  id /= a.nhc;
  int qt = a.nqt - 1 - id / a.B;
  int b = id % a.B;
  if constexpr (kOffset) {
    // Chunks after cached prefixes of different lengths: the work of a query
    // tile grows with its sequence's offset. Items (sequence, query tile) are
    // ranked by work -- sequences by offset, longest first, then query tiles
    // longest first -- and the first half of the grid takes them from the
    // longest end, the second half from the shortest, so that the workgroups
    // resident together on a CU pair long items with short ones.
    __shared__ int seq_by_len[kSortMaxB];
    if (a.B <= kSortMaxB) {  // uniform
      if (tid < a.B) {
        const int ot = a.offset[tid];
        int rank = 0;
        for (int j = 0; j < a.B; ++j) {
          const int oj = a.offset[j];
          rank += (oj > ot || (oj == ot && j < tid)) ? 1 : 0;
        }
        seq_by_len[rank] = tid;
      }
      __syncthreads();
      const int V = a.B * a.nqt, h = (V + 1) / 2;
      const int u = id < h ? id : V - 1 - (id - h);
      b = seq_by_len[u / a.nqt];
      qt = a.nqt - 1 - (u % a.nqt);
    }
  }
  const int span = 16 * a.npb;
  // o: position of row 0; klen: keys [0, klen) exist (prefix + this chunk)
  const int o = kOffset ? a.offset[b] : 0;
  const int klen = o + a.T;
  const int p0 = qt * span;  // first row of the workgroup (row index)
  const int kend = min(a.T, p0 + span);
  const int ntiles = (o + kend + kBN - 1) / kBN;

  // This wave's row blocks; pos[] are positions (row index + o).
  int head[kRB], pos[kRB];
  int wmin = 1 << 30, wmax = -1;
#pragma unroll
  for (int i = 0; i < kRB; ++i) {
    const int r = wave * kRB + i;
    head[i] = g * a.G + hc * a.Gc + (r % a.Gc);
    const int pb = r / a.Gc;
    pos[i] = o + p0 + 16 * pb + lr;
    wmin = min(wmin, o + p0 + 16 * pb);
    wmax = max(wmax, o + p0 + 16 * pb + 15);
  }
  wmax = min(wmax, klen - 1);
  if constexpr (kOffset) {
    if (o < 0 || static_cast<int64_t>(klen) > a.kv_rows) {  // outside the cache: zero rows, flag it
#pragma unroll
      for (int i = 0; i < kRB; ++i) {
        const int row = pos[i] - o;
        if (row >= a.T) continue;
        bf16_t *orow = a.out + ((static_cast<int64_t>(b) * a.T + row) * a.Hq + head[i]) * kD;
#pragma unroll
        for (int db = 0; db < 8; ++db) *reinterpret_cast<u32x2 *>(orow + 16 * db + 4 * lg) = u32x2{0u, 0u};
      }
      if (tid == 0 && a.status) *a.status = GROK_ERANGE;
      return;
    }
  }

  // Tile loads, HBM -> LDS. Each wave moves 4 KB of K and 4 KB of V per tile:
  // instruction j (0..3) fills 1 KB = LDS rows 16*wave + 4*j .. +3, lane L
  // writing physical chunk L%16 of row 16*wave + 4*j + L/16. Row R of the K tile
  // holds key k_row_key(R), which for these rows is key_l + 8*j; its chunk
  // swizzle (R % 8 = 4*(j%2) + L/16) alternates with the parity of j. Row R of
  // the V tile holds key R, with swizzle 2*(L/16) for every j. So one per-lane
  // byte offset per K parity and one for V, plus a wave-uniform base, address
  // all eight loads. Keys at or past klen (ragged last tile) read row klen-1
  // instead: they are masked out below.
  const bf16_t *kbase = a.k + (static_cast<int64_t>(b) * a.kv_rows * a.Hkv + g) * kD;
  const bf16_t *vbase = a.v + (static_cast<int64_t>(b) * a.kv_rows * a.Hkv + g) * kD;
  const int64_t rstride = static_cast<int64_t>(a.Hkv) * kD;
  const uint32_t rs2 = static_cast<uint32_t>(rstride) * 2;  // bytes between key rows
  const int lrow = lane / 16, lchunk = lane % 16;
  const int key_l = 32 * (wave >> 1) + 4 * (wave & 1) + lrow;
  const uint32_t koff = key_l * rs2;
  const uint32_t voff = lrow * rs2;
  auto issue_tile = [&](int key0, int buf) {
    if (key0 + kBN <= klen) {
      const char *kt = reinterpret_cast<const char *>(kbase) + static_cast<int64_t>(key0) * rs2;
      const char *vt = reinterpret_cast<const char *>(vbase) + static_cast<int64_t>(key0 + 16 * wave) * rs2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // R % 16 = 4*j + L/16; v_swz(R) = 2*(L/16) + 8*(j/2)
        __builtin_amdgcn_global_load_lds(kt + 8 * j * rs2 + (koff + 16 * (lchunk ^ (4 * j + lrow))),
                                         (lds_void *)(&Ks[buf][(16 * wave + 4 * j) * kRowBytes]), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + 4 * j * rs2 + (voff + 16 * (lchunk ^ ((lrow << 1) | ((j >> 1) << 3)))),
                                         (lds_void *)(&Vs[buf][(16 * wave + 4 * j) * kRowBytes]), 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int R = 16 * wave + 4 * j + lrow;
      const int kj = min(key0 + k_row_key(R), klen - 1);
      const int kc = lchunk ^ (R & 15);
      __builtin_amdgcn_global_load_lds(kbase + kj * rstride + 8 * kc,
                                       (lds_void *)(&Ks[buf][(16 * wave + 4 * j) * kRowBytes]),
                                       16, 0, 0);
      const int vj = min(key0 + R, klen - 1);
      const int vc = lchunk ^ v_swz(R);
      __builtin_amdgcn_global_load_lds(vbase + vj * rstride + 8 * vc,
                                       (lds_void *)(&Vs[buf][(16 * wave + 4 * j) * kRowBytes]),
                                       16, 0, 0);
    }
  };
  uint8_t kvr = 0;
  // the sequence's key-valid row (wave-uniform base; the lane offset is 32-bit)
  const uint8_t *kvrow = kHasValid ? a.key_valid + static_cast<int64_t>(b) * a.T : nullptr;
  auto load_valid = [&](int key0) {
    if constexpr (kHasValid) {
      const int j = key0 + tid;
      if (tid < kBN) kvr = j < a.T ? kvrow[j] : 0;
    }
  };
  auto store_valid = [&](int buf) {
    if constexpr (kHasValid) {
      if (tid < kBN) kvs[buf][tid] = kvr;
    }
  };

  issue_tile(0, 0);
  load_valid(0);

  // Q fragments (B operand of S^T): row lr, dims 32*kk + 8*lg .. +8.
  bf16x8 qf[kRB][4];
#pragma unroll
  for (int i = 0; i < kRB; ++i) {
    const int row = pos[i] - o;
    const bool ok = row < a.T;
    const bf16_t *qp = a.q + ((static_cast<int64_t>(b) * a.T + (ok ? row : 0)) * a.Hq + head[i]) * kD;
    u32x4 w[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) w[kk] = ok ? *reinterpret_cast<const u32x4 *>(qp + 32 * kk + 8 * lg) : u32x4{0, 0, 0, 0};
    if constexpr (kRopeQ) {
      // dims d (kk = 0, 1) pair with d + 64 (kk + 2) in the same lane
      const float *tp = a.rtab + static_cast<int64_t>(ok ? row : 0) * kD + 8 * lg;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float cs[8], sn[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          cs[e] = tp[32 * kk + e];
          sn[e] = tp[64 + 32 * kk + e];
        }
        rope8(w[kk], w[kk + 2], cs, sn);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[i][kk] = __builtin_bit_cast(bf16x8, w[kk]);
  }

  f32x4 oacc[kRB][8];
  float lsum[kRB];  // this lane's part of each row's weight sum
#pragma unroll
  for (int i = 0; i < kRB; ++i) {
    lsum[i] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[i][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  store_valid(0);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's LDS-bound loads have landed
  __syncthreads();                // ... and everyone else's

  // Per-lane V^T transpose-read addresses: source lane s = lr of group lg points
  // at key 8*lg + s/4 of the half (+4 for hi), dims 16*db + 4*(s%4); am[db] is
  // that address for dims block db in the first half of Vs[0] (v_byte with the
  // swizzle folded in; g is the same for the row 4 further down).
  uint32_t am[8];
  {
    const int vrow0 = 8 * lg + lr / 4;
    const int gs = v_swz(vrow0) >> 1;
    const uint32_t vbase0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)(&Vs[0][0])));
#pragma unroll
    for (int db = 0; db < 8; ++db)
      am[db] = vbase0 + vrow0 * kRowBytes + 32 * (db ^ gs) + 16 * ((lr & 3) >> 1) + 8 * (lr & 1);
  }

  // One tile of 64 keys. kMask: apply the causal (and key-valid) mask; tiles
  // wholly below the workgroup's first query row need none and run without it,
  // as one branch-free block the scheduler can interleave freely.
  auto tile = [&](int t, auto mask_c) {
    constexpr bool kMask = decltype(mask_c)::value;
    const int buf = t & 1;
    const int key0 = t * kBN;
    const bool more = !kMask || t + 1 < ntiles;  // unmasked tiles always have a successor
    if (more) {
      // (the key-valid byte first: whatever the compiler waits for to issue
      // it is then not behind the tile loads)
      load_valid(key0 + kBN);
      issue_tile(key0 + kBN, buf ^ 1);
    }
    uint32_t amb[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) amb[db] = am[db] + buf * kTileBytes;

    auto half = [&](auto hconst) {
      constexpr int h = decltype(hconst)::value;
      const int hk0 = key0 + 32 * h;  // first key of this half
      if (kMask && hk0 > wmax) return;  // wave-uniform: causally empty for this wave
      // S^T for the 3 row blocks; accumulator slot v of lane l is key
      // hk0 + 8*lg + 4*kb + v.
      f32x4 sacc[kRB][2];
#pragma unroll
      for (int i = 0; i < kRB; ++i) sacc[i][0] = sacc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      u32x2 kv8 = {0u, 0u};  // kHasValid: this lane's 8 key-valid bytes of the half
      if constexpr (kOffset || kHasValid) {
        // K fragments (and the key-valid bytes) as inline-assembly LDS reads:
        // in these instantiations the compiler otherwise waits for the next
        // tile's loads (all of them) before the first read, which serialises
        // the prefetch with the tile. The reads go out, then each key block
        // is waited for by count.
        if constexpr (kHasValid)
          asm volatile("ds_read_b64 %0, %1" : "=v"(kv8)
                       : "v"(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)(&kvs[buf][32 * h + 8 * lg]))))
                       : "memory");
        u32x4 kr[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            kr[kb][kk] = lds_read_b128(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                (lds_void *)(&Ks[buf][k_byte(32 * h + 16 * kb + lr, 4 * kk + lg)]))));
        lds_wait4<4>(kr[0]);
        if constexpr (kHasValid) asm volatile("" : "+v"(kv8));  // issued before kr[0]: landed
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb == 1) lds_wait4<0>(kr[1]);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < kRB; ++i)
              sacc[i][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kb][kk]),
                                                                   qf[i][kk], sacc[i][kb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int R = 32 * h + 16 * kb + lr;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 af = *reinterpret_cast<const bf16x8 *>(&Ks[buf][k_byte(R, 4 * kk + lg)]);
#pragma unroll
            for (int i = 0; i < kRB; ++i)
              sacc[i][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[i][kk], sacc[i][kb], 0, 0, 0);
          }
        }
      }
      // softcap + shifted exp -> P (bf16) in the B-operand layout of P.V:
      // p = exp2(k2 / (1 + exp2(k1*s))) = exp2(rcp((1 + e) * (1/k2))).
      const bool diag = kMask && hk0 + 31 > wmin;
      auto softmax_rows = [&](int i) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sv = sacc[i][e >> 2][e & 3];
          const float ex = __builtin_amdgcn_exp2f(sv * a.k1);
          p[e] = __builtin_amdgcn_exp2f(__builtin_amdgcn_rcpf(__builtin_fmaf(ex, a.k2inv, a.k2inv)));
        }
        if (diag || (kMask && kHasValid)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = hk0 + 8 * lg + e;
            bool ok = key <= pos[i];
            if constexpr (kHasValid) ok = ok && ((kv8[e >> 2] >> (8 * (e & 3))) & 0xffu) != 0;
            p[e] = ok ? p[e] : 0.f;
          }
        }
        const u32x4 w = {cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]), cvt_pk_bf16(p[4], p[5]),
                         cvt_pk_bf16(p[6], p[7])};
        // Row sum of the bf16-rounded weights that the P.V product uses (so the
        // normalised weights of a row sum to one): bf16 pair dot (1, 1).
#pragma unroll
        for (int e = 0; e < 4; ++e) lsum[i] = add_bf16_pair(lsum[i], w[e]);
        return __builtin_bit_cast(bf16x8, w);
      };
      // O^T += V^T . P^T; the V^T fragment of lane l (dim 16*db + lr, keys
      // 8*lg .. 8*lg+7 of the half) comes from two transpose reads of 4 keys.
      u32x2 lo[8], hi[8];
      if constexpr (!kHasValid && !kOffset) {
        // Plain prefill: the V^T reads go out first and land during the first
        // softmax; then row block by row block, so that the P.V MFMAs of one
        // block execute while the next block's softmax is issued.
        read_vt_half<h * 32 * kRowBytes>(lo, hi, amb, std::make_integer_sequence<int, 8>{});
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
          const bf16x8 pfi = softmax_rows(i);
          if (i == 0) lds_wait<0>(lo, hi), lds_wait<0>(lo + 4, hi + 4);
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[db][0], lo[db][1], hi[db][0], hi[db][1]});
            oacc[i][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfi, oacc[i][db], 0, 0, 0);
          }
        }
      } else {
        // With padding masks or a cache offset the register budget is tighter:
        // all softmaxes first, then the V^T reads and the P.V product.
        bf16x8 pf[kRB];
#pragma unroll
        for (int i = 0; i < kRB; ++i) pf[i] = softmax_rows(i);
        read_vt_half<h * 32 * kRowBytes>(lo, hi, amb, std::make_integer_sequence<int, 8>{});
        lds_wait<8>(lo, hi);
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          if (db == 4) lds_wait<0>(lo + 4, hi + 4);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[db][0], lo[db][1], hi[db][0], hi[db][1]});
#pragma unroll
          for (int i = 0; i < kRB; ++i)
            oacc[i][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[i], oacc[i][db], 0, 0, 0);
        }
      }
    };
    half(std::integral_constant<int, 0>{});
    half(std::integral_constant<int, 1>{});

    if (more) store_valid(buf ^ 1);
    __builtin_amdgcn_s_waitcnt(0);  // next tile's LDS-bound loads have landed
    __syncthreads();
  };

  // Tiles [0, tfull) end below the workgroup's first query position o + p0.
  const int tfull = kHasValid ? 0 : (o + p0) / kBN;
  int t = 0;
  for (; t < tfull; ++t) tile(t, std::false_type{});
  for (; t < ntiles; ++t) tile(t, std::true_type{});

  // Epilogue: normalise by the row sum and store bf16.
#pragma unroll
  for (int i = 0; i < kRB; ++i) {
    float l = lsum[i];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const int row = pos[i] - o;
    if (row >= a.T) continue;
    bf16_t *orow = a.out + ((static_cast<int64_t>(b) * a.T + row) * a.Hq + head[i]) * kD;
    if (kHasValid && l == 0.f) {
      // No valid key for this row: equal weights on all T value rows.
      f32x4 acc[8];
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < a.T; ++j) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const u32x2 w = *reinterpret_cast<const u32x2 *>(vbase + j * rstride + 16 * db + 4 * lg);
          acc[db][0] += lo_bf16(w[0]);
          acc[db][1] += hi_bf16(w[0]);
          acc[db][2] += lo_bf16(w[1]);
          acc[db][3] += hi_bf16(w[1]);
        }
      }
      const float invt = 1.f / static_cast<float>(a.T);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = 16 * db + 4 * lg;
        u32x2 w = {cvt_pk_bf16(acc[db][0] * invt, acc[db][1] * invt),
                   cvt_pk_bf16(acc[db][2] * invt, acc[db][3] * invt)};
        *reinterpret_cast<u32x2 *>(orow + d) = w;
      }
      continue;
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = 16 * db + 4 * lg;
      const f32x4 o = oacc[i][db];
      u32x2 w = {cvt_pk_bf16(o[0] / l, o[1] / l), cvt_pk_bf16(o[2] / l, o[3] / l)};
      *reinterpret_cast<u32x2 *>(orow + d) = w;
    }
  }
}

int pick_gc(int G) {
  for (int c = kRowBlocks; c >= 1; --c)
    if (G % c == 0 && kRowBlocks % c == 0) return c;
  return 1;
}

}  // namespace

bool prefill_mfma_supported(int64_t kv_rows, int Hq, int Hkv, int D, int dtype) {
  return dtype == GROK_BF16 && D == kD && Hkv > 0 && Hq % Hkv == 0;
}

hipError_t launch_prefill_mfma(const void *q, const void *k, const void *v, int64_t kv_rows,
                               const uint8_t *key_valid, void *out, int B, int T, int Hq,
                               int Hkv, float mult, float cap, hipStream_t s,
                               const int32_t *offset, int32_t *status, const float *rtab) {
  PrefillArgs a;
  a.rtab = rtab;
  a.offset = offset;
  a.status = status;
  a.q = static_cast<const bf16_t *>(q);
  a.k = static_cast<const bf16_t *>(k);
  a.v = static_cast<const bf16_t *>(v);
  a.key_valid = key_valid;
  a.out = static_cast<bf16_t *>(out);
  a.kv_rows = kv_rows;
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.Gc = pick_gc(a.G);
  a.npb = kRowBlocks / a.Gc;
  a.nhc = a.G / a.Gc;
  a.nqt = (T + 16 * a.npb - 1) / (16 * a.npb);
  a.k1 = 2.f * mult * kLog2e / cap;
  a.k2inv = 1.f / (-2.f * cap * kLog2e);
  const int64_t nblk = static_cast<int64_t>(B) * Hkv * a.nhc * a.nqt;
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (offset && key_valid) return hipErrorInvalidValue;  // validated by the caller
  if (rtab && offset) return hipErrorInvalidValue;
  if (rtab && key_valid)
    hipLaunchKernelGGL((prefill_mfma_kernel<true, false, true>), dim3(static_cast<unsigned>(nblk)), dim3(kThreads), 0,
                       s, a);
  else if (rtab)
    hipLaunchKernelGGL((prefill_mfma_kernel<false, false, true>), dim3(static_cast<unsigned>(nblk)), dim3(kThreads),
                       0, s, a);
  else if (offset)
    hipLaunchKernelGGL((prefill_mfma_kernel<false, true>), dim3(static_cast<unsigned>(nblk)), dim3(kThreads), 0,
                       s, a);
  else if (key_valid)
    hipLaunchKernelGGL((prefill_mfma_kernel<true, false>), dim3(static_cast<unsigned>(nblk)), dim3(kThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<false, false>), dim3(static_cast<unsigned>(nblk)), dim3(kThreads), 0,
                       s, a);
  return hipGetLastError();
}

}  // namespace grok

// LDS tile layouts and fragment helpers shared by the attention kernels
// (prefill and decode) for head size 128 on gfx950 bf16 MFMA.
//
// Tiles hold 256-byte rows (one key's 128 bf16 values of one KV head). The
// S^T = K.Q^T product reads K fragments from a permuted, XOR-swizzled K tile so
// that its accumulator comes out in the B-operand layout of the P.V product;
// the V^T operand of P.V is read from row-major V with LDS transpose reads.
#pragma once

#include <utility>

#include "common.h"

namespace grok {
namespace attn {

constexpr int kRowBytes = 256;  // one K or V row in LDS (unpadded)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

// acc + lo + hi of a packed bf16 pair in one instruction (v_dot2c_f32_bf16
// against the pair (1.0, 1.0)). Inline assembly: this compiler's
// __builtin_amdgcn_fdot2_f32_bf16 passes the same 32-bit source for every
// element of a vector it is given.
__device__ __forceinline__ float add_bf16_pair(float acc, uint32_t pair) {
  asm("v_dot2c_f32_bf16 %0, 0x3f803f80, %1" : "+v"(acc) : "v"(pair));
  return acc;
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// LDS bank layout. A 256-byte row spans all 64 four-byte banks of the LDS, so
// which banks an access hits depends only on the 16-byte chunk position within
// the row; chunks are XOR-swizzled by row so that the lanes served together by
// one fragment read hit distinct banks (16 lanes for a 16-byte read, 32 for an
// 8-byte read; the same holds for a 32-bank, 128-byte-per-cycle organisation).
//
// K tile layout: LDS row R holds key perm(R) (within each 32-key half, the
// S^T A operand of key block kb reads keys 8*(r/4) + 4*kb + r%4 in lane order
// r = lane%16; they sit at rows 16*kb + r). Chunk c (16 bytes) of row R is
// stored at chunk c ^ (R % 16): the 16 rows of one read land on 16 chunks.
__device__ __forceinline__ int k_row_key(int R) {  // key held by LDS row R
  const int h = R >> 5, r = R & 31;
  const int kb = r >> 4, a = (r >> 2) & 3, cc = r & 3;
  return 32 * h + 8 * a + 4 * kb + cc;
}
__device__ __forceinline__ int k_byte(int R, int c) { return R * kRowBytes + ((c ^ (R & 15)) << 4); }
// V tile layout: row r holds key r; chunk c is stored at chunk c ^ (2 * g(r)),
// g(r) = (r % 4) + 4 * ((r / 8) % 2). The even XOR keeps the two chunks of each
// 32-byte transpose-read span adjacent; one 32-lane pass of a transpose read
// covers rows {0..3, 8..11} (+4, +16, +32 ...), whose g are all distinct, so
// its eight 32-byte spans fill the 64 banks. For the P.V operand
// (c = 2*db + (0|1), rows r and r + 4 with the same g) dims block db sits at
// byte 32*(db ^ g(r)) + 16*(c & 1) of the row.
__device__ __forceinline__ int v_swz(int r) { return ((r & 3) << 1) | (((r >> 3) & 1) << 3); }
__device__ __forceinline__ int v_byte(int r, int c) { return r * kRowBytes + ((c ^ v_swz(r)) << 4); }

// LDS transpose read (ds_read_b64_tr_b16) at addr + kOff. Written as inline
// assembly because the compiler treats the builtin form as possibly aliasing
// the in-flight global_load_lds of the next tile and waits for those loads
// before the first read, which would serialise the prefetch with the P.V
// product. The asm is invisible to the compiler's LDS counter tracking, so its
// results are only used after an explicit wait (lds_wait) that takes them as
// operands. LDS operations complete in issue order, so the compiler's own
// waits stay correct with these reads in flight.
template <int kOff>
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff) : "memory");
  return r;
}

// The 16 reads of one 32-key half: lo/hi[db] for dims 16*db .. 16*db + 15,
// keys 8*(lane/16) + 0..3 (lo) and + 4..7 (hi, 4 rows = 1024 bytes further);
// am[db] is this lane's address of dims block db in the tile's first half.
template <int kHalfOff, int... kDb>
__device__ __forceinline__ void read_vt_half(u32x2 *lo, u32x2 *hi, const uint32_t *am,
                                             std::integer_sequence<int, kDb...>) {
  ((lo[kDb] = lds_read_tr16<kHalfOff>(am[kDb]), hi[kDb] = lds_read_tr16<kHalfOff + 1024>(am[kDb])),
   ...);
}

// 16-byte LDS read as inline assembly (same reason as above); its result is
// used only after lds_wait4.
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
  return r;
}

// Waits until at most kLeft LDS operations are outstanding, with four 16-byte
// fragments passing through.
template <int kLeft>
__device__ __forceinline__ void lds_wait4(u32x4 *r) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]) : "i"(kLeft));
}

// Waits until at most kLeft LDS operations are outstanding; the four fragment
// pairs pass through so that no use of them is scheduled above the wait.
template <int kLeft>
__device__ __forceinline__ void lds_wait(u32x2 *lo, u32x2 *hi) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(lo[0]), "+v"(lo[1]), "+v"(lo[2]), "+v"(lo[3]), "+v"(hi[0]), "+v"(hi[1]),
                 "+v"(hi[2]), "+v"(hi[3])
               : "i"(kLeft));
}

// RoPE of 8 bf16 pairs held by one lane: element e of w1 is dim i0 + e, element
// e of w2 dim i0 + e + 64 (the half-split partner), with the cos/sin of those
// pairs; rope_rotate of common.h, rounded to bf16 as grok_rope rounds.
__device__ __forceinline__ void rope8(u32x4 &w1, u32x4 &w2, const float *cs, const float *sn) {
  u32x4 o1, o2;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float a0, a1, b0, b1;
    rope_rotate(lo_bf16(w1[q]), lo_bf16(w2[q]), cs[2 * q], sn[2 * q], a0, b0);
    rope_rotate(hi_bf16(w1[q]), hi_bf16(w2[q]), cs[2 * q + 1], sn[2 * q + 1], a1, b1);
    o1[q] = pack_bf16x2(a0, a1);
    o2[q] = pack_bf16x2(b0, b1);
  }
  w1 = o1;
  w2 = o2;
}

}  // namespace attn
}  // namespace grok

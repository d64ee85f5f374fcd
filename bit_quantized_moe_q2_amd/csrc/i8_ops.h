// Q2_K block loads shared by the matrix-core kernels that stream Q2_K weight
// rows (the expert-grouped decode, decode_grouped.hip, and the fp16 prefill
// GEMMs, prefill_f16.hip), and the int8 B operands of the grouped decode.
//
// Arithmetic (block layout of "【#2】ds4.c 해독하기", Q2_K table): one
// 256-value block of a weight row dotted with an activation row a is
//   d * sum_v (sc*q)_v a_v  -  dmin * sum_s mn_s A_s,
// A_s the sums of a over the 16 sub-blocks.
#pragma once
#include "common.h"

namespace ds4q {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));


// 24-bit unsigned multiply (full-rate v_mul_u32_u24; both operands < 2^24).
__device__ __forceinline__ uint32_t mul_u24(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_mul_u32_u24 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// The bytes of one Q2_K block that lane group g uses: code quarter g
// (16 bytes), the scale/min bytes of sub-blocks 8(g>>1)..8(g>>1)+7, d|dmin.
// Two requests per lane: the codes, and 8 bytes that are the scale/min bytes
// of the pair (g even: bytes 8(g>>1)..+7) or end with d|dmin (g odd: bytes
// 76..83); finish() hands each 16-lane group its partner's part
// (v_permlane16_swap pairs groups 0/1 and 2/3).
struct Q2KPart {
  u32x4 q;
  uint32_t s0, s1, dd;
  uint32_t p0, p1;  // the 8 bytes as loaded, until finish()
  __device__ __forceinline__ void load(const uint8_t *__restrict__ blk, int g) {
    q = *reinterpret_cast<const u32x4a *>(blk + 16 + 16 * g);
    typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));
    const u32x2a p = *reinterpret_cast<const u32x2a *>(blk + ((g & 1) ? 76 : 8 * (g >> 1)));
    p0 = p.x;
    p1 = p.y;
  }
  __device__ __forceinline__ void finish() {
    s0 = __builtin_amdgcn_permlane16_swap(p0, p0, false, false)[0];  // the even group's bytes
    const auto sw = __builtin_amdgcn_permlane16_swap(p1, p1, false, false);
    s1 = sw[0];  // the even group's bytes 4..7 of its pair
    dd = sw[1];  // the odd group's bytes 80..83
  }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));

// Raw bytes of one block for lane group g, as Q2KPart::load requests them
// (the 16 code bytes of quarter g; 8 bytes that are scale/min bytes or end
// with d|dmin), kept as two vectors so that a loop can reload them in place.
struct RawBlk {
  u32x4 q;
  u32x2 p;
  __device__ __forceinline__ void load(const uint8_t *__restrict__ blk, int g) {
    q = *reinterpret_cast<const u32x4a *>(blk + 16 + 16 * g);
    p = *reinterpret_cast<const u32x2a *>(blk + ((g & 1) ? 76 : 8 * (g >> 1)));
  }
};

// The operand bytes of a raw block, as Q2KPart::finish makes them, with one
// exchange per result: the raw registers are only read (an exchange rewrites
// both of its operands), so they can take the next block in place.
__device__ __forceinline__ Q2KPart take_block(const RawBlk &r) {
  Q2KPart o;
  o.q = r.q;
  o.p0 = o.p1 = 0;
  o.s0 = __builtin_amdgcn_permlane16_swap(r.p.x, r.p.x, false, false)[0];  // the even group's bytes
  o.s1 = __builtin_amdgcn_permlane16_swap(r.p.y, r.p.y, false, false)[0];  // its bytes 4..7
  o.dd = __builtin_amdgcn_permlane16_swap(r.p.y, r.p.y, true, false)[1];   // the odd group's d|dmin
  return o;
}

// Weight operands of one block for one 16-row n-subtile.  Code byte c of
// dword j of quarter g holds, in bit pair k, value
// 128(g>>1) + 32k + 16(g&1) + 4j + c, of sub-block 8(g>>1) + 2k + (g&1);
// K-tile j, dword k of the B fragment is that bit pair looked up in the
// sub-block's table [0, sc, 2sc, 3sc].

// The four sub-block tables of the lane (bit pair k -> table k).
struct WTab {
  uint32_t tab[4];
  __device__ __forceinline__ void build(const Q2KPart &r, int g) {
    const int p = g & 1;
    const uint32_t a0 = r.s0 >> (8 * p), a1 = r.s1 >> (8 * p);
    tab[0] = mul_u24(a0 & 15u, 0x03020100u >> 8) << 8;
    tab[1] = mul_u24((a0 >> 16) & 15u, 0x03020100u >> 8) << 8;
    tab[2] = mul_u24(a1 & 15u, 0x03020100u >> 8) << 8;
    tab[3] = mul_u24((a1 >> 16) & 15u, 0x03020100u >> 8) << 8;
  }
  // integer B fragment of K-tile j
  __device__ __forceinline__ i32x4 bfrag(const Q2KPart &r, int j) const {
    const uint32_t w = r.q[j];
    i32x4 b;
    b.x = (int)__builtin_amdgcn_perm(0u, tab[0], w & 0x03030303u);
    b.y = (int)__builtin_amdgcn_perm(0u, tab[1], (w >> 2) & 0x03030303u);
    b.z = (int)__builtin_amdgcn_perm(0u, tab[2], (w >> 4) & 0x03030303u);
    b.w = (int)__builtin_amdgcn_perm(0u, tab[3], (w >> 6) & 0x03030303u);
    return b;
  }
};

// sched_barrier mask: ALU, MFMA and LDS instructions may be scheduled
// across, global memory instructions may not.
constexpr int SCHED_NOVMEM = 0x1 | 0x2 | 0x4 | 0x8 | 0x80 | 0x100 | 0x200;

}  // namespace
}  // namespace ds4q

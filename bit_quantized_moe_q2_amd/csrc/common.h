// Shared device helpers and block-format constants for the gfx950 kernels.
//
// Block formats:
//  Q2_K ("【#2】ds4.c 해독하기", Q2_K block-layout table and packing expression):
//    84 B per 256 values; bytes 0..15 one byte per 16-value sub-block (scale in
//    the low nibble, min in the high nibble), bytes 16..79 the 2-bit codes
//    (code of value v sits in byte 16 + 32*(v>>7) + (v&31) at bit 2*((v>>5)&3)),
//    fp16 d at 80, fp16 dmin at 82; value = d*scale*code - dmin*min.
//  Q4_1 (ThakiCloud "...GGUF Q4_1 재부호화", Q4_1 block section):
//    20 B per 32 values; fp16 d at 0, fp16 m at 2, qs[16] at 4; value j < 16 is
//    the low nibble of qs[j], value j+16 its high nibble; value = d*code + m.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4q {

constexpr int QK_Q2K = 256, BB_Q2K = 84;
constexpr int QK_Q41 = 32, BB_Q41 = 20;
constexpr int TYPE_Q4_1 = 3, TYPE_Q2_K = 10;

__host__ __device__ constexpr int64_t row_bytes(int type, int64_t cols) {
  return type == TYPE_Q2_K ? cols / QK_Q2K * BB_Q2K : cols / QK_Q41 * BB_Q41;
}

__device__ __forceinline__ float f16lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Byte n of a dword as float (v_cvt_f32_ubyteN).
__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xFFu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }

// 4-byte-aligned dword loads of block fields (blocks are only 4-byte aligned).
__device__ __forceinline__ uint32_t ld32(const uint8_t *p) {
  return *reinterpret_cast<const uint32_t *>(p);
}

// bf16 round-to-nearest-even of an fp32 value (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32, one instruction and no branch.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two values rounded as by bf16_rne_bits, packed a (low half), b (high half).
__device__ __forceinline__ uint32_t bf16_rne_pair(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, b2));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Sum over groups of W consecutive lanes of a wave64 (W power of two <= 64);
// every lane of the group gets the group total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Matrix-core issue fence.  On gfx950, a vector instruction that overwrites
// the accumulator input (SrcC) registers of an integer MFMA a few wait states
// after the MFMA issues was measured to corrupt that MFMA's result (wrong
// int32 sums in one of two otherwise identical chains), although the
// compiler's hazard model allowed it (it leaves 3 wait states).  Kernels
// therefore issue independent MFMAs in groups and follow each group with this
// fence: no instruction moves across it and 8 wait states pass before the next
// one, so the accumulator inputs are read before anything can reuse their
// registers.  A CPU test scans the built assembly for such writes closer than
// 8 wait states.  mfma_group_begin() before a group keeps earlier
// instructions out of it, so one fence covers all the group's MFMAs.
__device__ __forceinline__ void mfma_group_begin() { __builtin_amdgcn_sched_barrier(0); }
__device__ __forceinline__ void mfma_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}

// Direct global-to-LDS copy of 16 bytes per lane (lane i's bytes land at
// lds + 16 i, lds wave-uniform) from base + soff + voff, soff wave-uniform,
// as buffer_load_dwordx4 ... lds.  global_load_lds copies the same way, but
// the compiler counts a pending global_load_lds as an access that may
// complete LDS operations out of order, so every later wait for an LDS read
// becomes a wait for all of them and LDS reads issued ahead of their use no
// longer overlap anything; with the buffer form those waits stay exact.  No
// range limit is set: callers keep offsets in bounds (and below 2^32).
struct DmaSrc {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ explicit DmaSrc(const void *base)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, -1, 0x00020000)) {}
  __device__ __forceinline__ void copy16(uint32_t voff, uint32_t soff, uint8_t *lds) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff,
                                             soff, 0, 0);
  }
};

// Grouped-GEMM work item -> (m-tile, n-tile).  The live m-tiles, largest
// first (the grouping's size-ordered list; their count is known on the
// device only), are dealt to the 8 XCDs in turn: m-tile t to XCD t % 8, and
// workgroup i runs on XCD i % 8 as slot i / 8, which is n-tile
// slot % n_ntiles of that XCD's (slot / n_ntiles)-th m-tile.  So every XCD
// gets about the same work, the n-tiles of an m-tile share one XCD's L2, and
// each XCD runs its largest items first.  The grid is 8 * ceil(max m-tiles /
// 8) * n_ntiles (xcd_grid); returns false for a workgroup without work.
__device__ __forceinline__ bool xcd_tile_of(int n_live_m, int n_ntiles, int *mtile, int *ntile) {
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int t = x + 8 * (slot / n_ntiles);
  if (t >= n_live_m) return false;
  *mtile = t;
  *ntile = slot % n_ntiles;
  return true;
}
inline unsigned xcd_grid(int max_tiles, int n_ntiles) {
  return (unsigned)(8 * ((max_tiles + 7) / 8) * n_ntiles);
}

// ---------------------------------------------------------------- routing

// Order-preserving uint32 of an fp32 value, with -0.0 folded onto +0.0 so
// that equal logits tie exactly as floating-point comparison says.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64), hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

constexpr int ROUTE_MAX_E = 1024;

// DPP (data-parallel primitives) lane exchanges: results stay in VALU
// registers, no LDS round trip.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within 16

__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// bf16 store of a lane's two output rows r0 = base + n and r1 = base + 16 + n
// (n = lane & 15; `p` points at row r0 of the token) as one 4-byte store per
// lane instead of two 2-byte ones: lanes n and n ^ 1 swap one fp32 value,
// then the even lane writes rows (r0, r0 + 1) and the odd lane rows
// (r1 - 1, r1).  base must be even, and lanes n and n ^ 1 both active.
__device__ __forceinline__ void store_bf16_row_pair(uint16_t *p, int n, float v0, float v1) {
  const bool odd = n & 1;
  const float got = __builtin_bit_cast(float, dpp<DPP_XOR1>(__builtin_bit_cast(uint32_t, odd ? v0 : v1)));
  const uint32_t word = odd ? bf16_rne_pair(got, v1) : bf16_rne_pair(v0, got);
  *reinterpret_cast<uint32_t *>(p + (odd ? 15 : 0)) = word;
}

// Wave-wide unsigned max; the result is uniform.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp<DPP_XOR1>(v));
  v = max(v, dpp<DPP_XOR2>(v));
  v = max(v, dpp<DPP_HALF_MIRROR>(v));
  v = max(v, dpp<DPP_MIRROR>(v));
  return max(max(readlane(v, 0), readlane(v, 16)), max(readlane(v, 32), readlane(v, 48)));
}

__device__ __forceinline__ float float_from_ordered(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __builtin_bit_cast(float, u);
}

// Top-k for E <= 256 logits (four per lane: expert lane + 64i): each round
// takes the wave max of the order-preserving keys, then the smallest expert
// index holding it (ties -> lower index) from ballots.  Lane j < k returns slot j's expert
// and softmax weight.  load() only issues the reads, so that a caller can
// queue other loads behind them before select() waits.
struct TopK256 {
  float v[4];
  __device__ __forceinline__ void load(const float *__restrict__ lg, int E, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? lg[e] : 0.f;
    }
  }
  // The first k_need slots (k_need <= k); with weights, the softmax over the
  // k selected (then k_need must equal k).
  __device__ __forceinline__ void select(int E, int k, int k_need, bool weights, int lane, int *id,
                                         float *w) const {
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = lane + 64 * i < E ? ordered_bits(v[i]) : 0u;
    uint32_t my_id = 0, my_key = 0;
    for (int j = 0; j < k_need; ++j) {
      const uint32_t gm = wave_umax(max(max(key[0], key[1]), max(key[2], key[3])));
      // The smallest expert index holding gm: experts lane + 64i are in
      // index order i-major, so the first non-empty ballot in i and its
      // lowest set lane give it (scalar bit scans, no second reduction).
      const uint64_t m0 = __builtin_amdgcn_ballot_w64(key[0] == gm);
      const uint64_t m1 = __builtin_amdgcn_ballot_w64(key[1] == gm);
      const uint64_t m2 = __builtin_amdgcn_ballot_w64(key[2] == gm);
      const uint64_t m3 = __builtin_amdgcn_ballot_w64(key[3] == gm);
      const uint32_t c0 = m0 ? (uint32_t)__builtin_ctzll(m0) : 256u;
      const uint32_t c1 = m1 ? 64u + (uint32_t)__builtin_ctzll(m1) : 256u;
      const uint32_t c2 = m2 ? 128u + (uint32_t)__builtin_ctzll(m2) : 256u;
      const uint32_t c3 = m3 ? 192u + (uint32_t)__builtin_ctzll(m3) : 256u;
      const uint32_t ew = min(min(c0, c1), min(c2, c3));
#pragma unroll
      for (int i = 0; i < 4; ++i) key[i] = (uint32_t)(lane + 64 * i) == ew ? 0u : key[i];
      if (lane == j) { my_id = ew; my_key = gm; }
    }
    *id = (int)my_id;
    *w = 0.f;
    if (weights) {
      const float top = float_from_ordered(readlane(my_key, 0));
      const float ex = lane < k ? expf(float_from_ordered(my_key) - top) : 0.f;
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += __builtin_bit_cast(float, readlane(__builtin_bit_cast(uint32_t, ex), j));
      *w = ex / den;
    }
  }
};

__device__ __forceinline__ void wave_topk256(const float *__restrict__ lg, int E, int k, int lane,
                                             int *id, float *w) {
  TopK256 t;
  t.load(lg, E, lane);
  t.select(E, k, k, true, lane, id, w);
}

// Top-k of E logits by (logit desc, index asc) for one token, computed by a
// whole wave64; softmax weights over the k selected (max-subtracted).  Lane
// j < k returns slot j's expert in *id and weight in *w; every lane returns
// the same values for the slot it asks for through the arrays.
template <int MAXE>
__device__ __forceinline__ void wave_topk(const float *__restrict__ lg, int E, int k, int lane,
                                          int *id, float *w) {
  uint64_t key[MAXE / 64];
#pragma unroll
  for (int i = 0; i < MAXE / 64; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? ((uint64_t)ordered_bits(lg[e]) << 32) | (0xFFFFFFFFu - (uint32_t)e) : 0ull;
  }
  int my_id = 0;
  float my_val = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < MAXE / 64; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
#pragma unroll
    for (int i = 0; i < MAXE / 64; ++i)
      if (lane + 64 * i == e) key[i] = 0ull;
    if (lane == j) { my_id = e; my_val = lg[e]; }
  }
  const float top = __shfl(my_val, 0, 64);
  const float ex = lane < k ? expf(my_val - top) : 0.f;
  float den = ex;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o, 64);
  *id = my_id;
  *w = ex / den;
}

}  // namespace ds4q

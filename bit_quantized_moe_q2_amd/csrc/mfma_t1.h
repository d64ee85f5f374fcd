// Shared parts of the one-token decode kernels on int8 matrix cores (Q2_K in
// decode_mfma.hip, Q4_1 in decode_q41.hip):
// operand types, the quantisation of an activation vector into three int8
// limbs per value in a wave's LDS area (in the fragment order of either block
// format), the routing of one token by a wave, and the weight operands and
// per-block arithmetic of both formats.
//
// Limbs: per 256-value chunk sigma = max|x| / 127 and
// N = trunc(x * 127 * 65536 / max|x| + 32896), whose balanced base-256 digits
// a0 = byte 2, a1 = byte 1 - 128, a2 = byte 0 - 128 give
// x ~= sigma * (a0 + a1/256 + a2/65536), residual below 2^-23 of the chunk's
// largest value.  The fragment of a chunk is 3 limbs x 64 dwords.
#pragma once
#include "common.h"

namespace ds4q {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float INV256 = 1.0f / 256.0f;
constexpr float INV65536 = 1.0f / 65536.0f;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One thread quantises the 16 activations of one sub-block s (values
// 16s..16s+15 of a block) with the block scale inv = 127 / max|x| and writes
// its 3 limbs x 4 dwords into the block's fragments frag[limb][j][g][k]: the
// digits of N (see above) are gathered byte-wise with v_perm.
__device__ __forceinline__ void quantize_subblock(const float v[16], float inv, int s,
                                                  uint32_t *__restrict__ frag_blk) {
  const int h = s >> 3, k = (s >> 1) & 3, p = s & 1, g = 2 * h + p;
  const float scale = inv * 65536.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) n[i] = (uint32_t)(int)fmaf(v[4 * j + i], scale, 32896.0f);
    // bytes 0 and 1 of values 0..3, and byte 2
    const uint32_t p01 = __builtin_amdgcn_perm(n[1], n[0], 0x05010400u);
    const uint32_t p23 = __builtin_amdgcn_perm(n[3], n[2], 0x05010400u);
    const uint32_t q01 = __builtin_amdgcn_perm(n[1], n[0], 0x0C0C0602u);
    const uint32_t q23 = __builtin_amdgcn_perm(n[3], n[2], 0x0C0C0602u);
    const int off = (j * 4 + g) * 4 + k;
    frag_blk[0 * 64 + off] = __builtin_amdgcn_perm(q23, q01, 0x05040100u);
    frag_blk[1 * 64 + off] = __builtin_amdgcn_perm(p23, p01, 0x07060302u) ^ 0x80808080u;
    frag_blk[2 * 64 + off] = __builtin_amdgcn_perm(p23, p01, 0x05040100u) ^ 0x80808080u;
  }
}

// The same for the Q4_1 fragment order.  A 256-value chunk holds eight
// 32-value blocks; K tile j (64 K slots) carries blocks 2j and 2j+1, lane
// group g = 2*(block & 1) + p of the tile taking half p of its block: K slot
// i < 8 is value 8p + i of the block, slot 8 + i value 16 + 8p + i (the low
// and the high nibbles of code bytes 8p..8p+7).  Sub-block s (values
// 16s..16s+15) is half s & 1 of block s >> 1: its values 0..7 go to half p = 0
// and 8..15 to p = 1, at dwords 2*(s & 1) and 2*(s & 1) + 1 of each.
__device__ __forceinline__ void quantize_subblock_q41(const float v[16], float inv, int s,
                                                      uint32_t *__restrict__ frag_blk) {
  const int bb = s >> 1, tile = bb >> 1;
  const float scale = inv * 65536.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) n[i] = (uint32_t)(int)fmaf(v[4 * j + i], scale, 32896.0f);
    const uint32_t p01 = __builtin_amdgcn_perm(n[1], n[0], 0x05010400u);
    const uint32_t p23 = __builtin_amdgcn_perm(n[3], n[2], 0x05010400u);
    const uint32_t q01 = __builtin_amdgcn_perm(n[1], n[0], 0x0C0C0602u);
    const uint32_t q23 = __builtin_amdgcn_perm(n[3], n[2], 0x0C0C0602u);
    const int g = 2 * (bb & 1) + (j >> 1);
    const int off = (tile * 4 + g) * 4 + 2 * (s & 1) + (j & 1);
    frag_blk[0 * 64 + off] = __builtin_amdgcn_perm(q23, q01, 0x05040100u);
    frag_blk[1 * 64 + off] = __builtin_amdgcn_perm(p23, p01, 0x07060302u) ^ 0x80808080u;
    frag_blk[2 * 64 + off] = __builtin_amdgcn_perm(p23, p01, 0x05040100u) ^ 0x80808080u;
  }
}

__device__ __forceinline__ float max16(float m) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// One lane's share of quantising NB blocks of a vector (global) into a wave's
// LDS area: sub-blocks lane, lane+64, ...  load() reads the values, quantise()
// writes the limbs, sums and scales.
template <int NB, bool Q41 = false>
struct QuantStage {
  static constexpr int IT = (NB * 16 + 63) / 64;
  float x[IT][16];
  __device__ __forceinline__ void load(const float *__restrict__ v, int lane) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int t = lane + 64 * it;
      if (t < NB * 16) {
        const float4 *src = reinterpret_cast<const float4 *>(v + t * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 f = src[i];
          x[it][4 * i] = f.x; x[it][4 * i + 1] = f.y; x[it][4 * i + 2] = f.z; x[it][4 * i + 3] = f.w;
        }
      }
    }
  }
  // Sum of squares of the lane's values (0 for lanes without a sub-block).
  __device__ __forceinline__ float sumsq(int lane) const {
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < IT; ++it)
      if (lane + 64 * it < NB * 16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) ss = fmaf(x[it][i], x[it][i], ss);
      }
    return ss;
  }
  __device__ __forceinline__ void quantise(int lane, uint32_t *__restrict__ frag, float *__restrict__ sum,
                                           float *__restrict__ sig) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int t = lane + 64 * it;
      if (t < NB * 16) {
        const int b = t >> 4, sb = t & 15;
        float m = 0.f, acc = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          m = fmaxf(m, fabsf(x[it][i]));
          acc += x[it][i];
        }
        m = max16(m);
        const float inv = m > 0.f ? 127.0f / m : 0.0f;
        if constexpr (Q41) quantize_subblock_q41(x[it], inv, sb, frag + b * 192);
        else quantize_subblock(x[it], inv, sb, frag + b * 192);
        sum[b * 16 + sb] = acc;
        if (sb == 0) sig[b] = m / 127.0f;
      }
    }
    wave_lds_sync();
  }
};

// Routing of the one token by a whole wave: lane j < k gets slot j's expert
// and weight.  The logit loads are issued by load(); select() waits for them.
template <int MAXE>
struct TokenRoute {
  TopK256 t;
  const float *lg;
  __device__ __forceinline__ void load(const float *__restrict__ logits, int E, int lane) {
    lg = logits;
    if constexpr (MAXE == 256) t.load(logits, E, lane);
  }
  // The first k_need slots; the softmax weights only when asked for (then
  // all k slots are selected).
  __device__ __forceinline__ void select(int E, int k, int k_need, bool weights, int lane, int *id,
                                         float *w) const {
    if constexpr (MAXE == 256) t.select(E, k, weights ? k : k_need, weights, lane, id, w);
    else wave_topk<MAXE>(lg, E, k, lane, id, w);
  }
};

// ---------------------------------------------------------------- Q2_K operands

// Raw bytes of one 256-value Q2_K block that lane group g uses: code
// quarter g, the scale/min bytes of sub-blocks 8(g>>1)..+7, d|dmin.  Two
// requests per lane: the 16 code bytes, and 8 bytes that are the scale/min
// bytes of the pair (g even) or end with d|dmin (g odd: bytes 76..83);
// finish() hands each 16-lane group its partner's part (v_permlane16_swap
// pairs groups 0/1 and 2/3).
typedef uint32_t u32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2u __attribute__((ext_vector_type(2), aligned(4)));
struct Q2KRaw {
  uint32_t q[4], s0, s1, dd;
  uint32_t p0, p1;  // the 8 bytes as loaded, until finish()
  __device__ __forceinline__ void load(const uint8_t *__restrict__ blk, int g) {
    const u32x4u v = *reinterpret_cast<const u32x4u *>(blk + 16 + 16 * g);
    q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
    const u32x2u p = *reinterpret_cast<const u32x2u *>(blk + ((g & 1) ? 76 : 8 * (g >> 1)));
    p0 = p.x;
    p1 = p.y;
  }
  __device__ __forceinline__ void finish() {
    s0 = __builtin_amdgcn_permlane16_swap(p0, p0, false, false)[0];  // the even group's bytes
    const auto sw = __builtin_amdgcn_permlane16_swap(p1, p1, false, false);
    s1 = sw[0];
    dd = sw[1];  // the odd group's bytes 80..83
  }
};

// Scale/min bytes of the lane's four sub-blocks (k = 0..3).
__device__ __forceinline__ void sub_bytes(const Q2KRaw &r, int p, uint32_t sb[4]) {
  const uint32_t a0 = r.s0 >> (8 * p), a1 = r.s1 >> (8 * p);
  sb[0] = a0 & 0xFFu; sb[1] = (a0 >> 16) & 0xFFu; sb[2] = a1 & 0xFFu; sb[3] = (a1 >> 16) & 0xFFu;
}

// Byte table [0, sc, 2sc, 3sc] of a sub-block's integer weights: sc * 0x030201
// puts sc, 2sc, 3sc (at most 45) in bytes 0..2 without carries.
__device__ __forceinline__ uint32_t qsc_table(uint32_t sb) {
  return ((sb & 15u) * 0x030201u) << 8;
}

// B operand of K tile j: dword k = the sub-block's table looked up with the
// four 2-bit codes of bit pair k as byte selectors (v_perm_b32).
__device__ __forceinline__ i32x4 b_frag(const Q2KRaw &r, int j, const uint32_t tab[4]) {
  const uint32_t w = r.q[j];
  i32x4 b;
  b.x = (int)__builtin_amdgcn_perm(tab[0], tab[0], w & 0x03030303u);
  b.y = (int)__builtin_amdgcn_perm(tab[1], tab[1], (w >> 2) & 0x03030303u);
  b.z = (int)__builtin_amdgcn_perm(tab[2], tab[2], (w >> 4) & 0x03030303u);
  b.w = (int)__builtin_amdgcn_perm(tab[3], tab[3], (w >> 6) & 0x03030303u);
  return b;
}


// A operand of one block: row r < 3 of A is limb r of the activations, rows
// 3..15 are zero, so one MFMA yields the three limb dot products of 16 weight
// rows at once (C[limb][row]).  Lane (n, g) holds row n's 16 int8 of K group
// g for each of the 4 K tiles j.
struct AFrag {
  i32x4 a[4];
  __device__ __forceinline__ void load(const uint32_t *__restrict__ frag_blk, int n, int g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = (i32x4){0, 0, 0, 0};
    if (n < 3) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[j] = *reinterpret_cast<const i32x4 *>(frag_blk + n * 64 + (j * 4 + g) * 4);
    }
  }
};

// Block epilogue: the main term (C rows 0..2 = limbs, held by lane group 0;
// zero in the other groups) and the lane group's quarter of the min term.
__device__ __forceinline__ void block_post(const Q2KRaw &r, const uint32_t sb[4], const i32x4 c,
                                           const float *__restrict__ xsum_blk, float sigma, int g,
                                           float &main_acc, float &min_acc) {
  const int p = g & 1, h = g >> 1;
  const float f = fmaf((float)c.z, INV65536, fmaf((float)c.y, INV256, (float)c.x));
  main_acc = fmaf(f16lo(r.dd) * sigma, f, main_acc);
  float mn = (float)(sb[0] >> 4) * xsum_blk[8 * h + p];
  mn = fmaf((float)(sb[1] >> 4), xsum_blk[8 * h + 2 + p], mn);
  mn = fmaf((float)(sb[2] >> 4), xsum_blk[8 * h + 4 + p], mn);
  mn = fmaf((float)(sb[3] >> 4), xsum_blk[8 * h + 6 + p], mn);
  min_acc = fmaf(f16hi(r.dd), mn, min_acc);
}

// One block of NM weight rows (gate and up share the activations): the four
// A fragments are read from LDS once, then 4*NM MFMAs.
template <int NM, int KG>
__device__ __forceinline__ void block_dot(const Q2KRaw *const r[NM], const uint32_t *__restrict__ frag_blk,
                                          const float *__restrict__ xsum_blk, float sigma, int n, int g,
                                          float *main_acc, float *min_acc) {
  AFrag af;
  af.load(frag_blk, n, g);
  uint32_t sb[NM][4], tab[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    sub_bytes(*r[m], g & 1, sb[m]);
#pragma unroll
    for (int q = 0; q < 4; ++q) tab[m][q] = qsc_table(sb[m][q]);
  }
  i32x4 c[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) c[m] = (i32x4){0, 0, 0, 0};
  // Fenced MFMA groups of KG K tiles (1, 2 or 4).  Larger groups fence less
  // often but hold the B fragments of the whole group, which costs the
  // gate/up kernel registers and a resident workgroup per CU, so it uses
  // KG = 1 and the down kernel (one workgroup per CU) KG = 4.
#pragma unroll
  for (int j0 = 0; j0 < 4; j0 += KG) {
    i32x4 bj[KG][NM];
#pragma unroll
    for (int j = 0; j < KG; ++j)
#pragma unroll
      for (int m = 0; m < NM; ++m) bj[j][m] = b_frag(*r[m], j0 + j, tab[m]);
    mfma_group_begin();
#pragma unroll
    for (int j = 0; j < KG; ++j)
#pragma unroll
      for (int m = 0; m < NM; ++m) c[m] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af.a[j0 + j], bj[j][m], c[m], 0, 0, 0);
    mfma_fence();
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) block_post(*r[m], sb[m], c[m], xsum_blk, sigma, g, main_acc[m], min_acc[m]);
}

// ---------------------------------------------------------------- Q4_1 operands

typedef uint32_t u32x3a __attribute__((ext_vector_type(3), aligned(4)));

constexpr int CHUNK_BYTES = 8 * BB_Q41;  // 256 values

// The 12 bytes lane (n, g) reads of K tile j of a chunk: block 2j + (g >> 1)
// from offset 8 * (g & 1) (dm is the block's (d, m) in the lanes of half 0).
struct Q41Raw {
  uint32_t q0, q1, dm;
  __device__ __forceinline__ void load(const uint8_t *__restrict__ chunk, int j, int g) {
    const u32x3a v = *reinterpret_cast<const u32x3a *>(chunk + (2 * j + (g >> 1)) * BB_Q41 + 8 * (g & 1));
    dm = v.x;
    q0 = v.y;
    q1 = v.z;
  }
};

// One chunk (four K tiles, eight blocks) of 16 weight rows.
__device__ __forceinline__ void chunk_dot_q41(const Q41Raw r[4], const uint32_t *__restrict__ frag_blk,
                                              const float *__restrict__ xsum_blk, float sigma, int n, int g,
                                              float &acc) {
  const int limb = g < 2 ? n : n - 8;
  const bool arow = limb >= 0 && limb < 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    i32x4 a = (i32x4){0, 0, 0, 0};
    if (arow) a = *reinterpret_cast<const i32x4 *>(frag_blk + limb * 64 + (j * 4 + g) * 4);
    i32x4 b;
    b.x = (int)(r[j].q0 & 0x0F0F0F0Fu);
    b.y = (int)(r[j].q1 & 0x0F0F0F0Fu);
    b.z = (int)((r[j].q0 >> 4) & 0x0F0F0F0Fu);
    b.w = (int)((r[j].q1 >> 4) & 0x0F0F0F0Fu);
    const i32x4 c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, (i32x4){0, 0, 0, 0}, 0, 0, 0);
    if ((g & 1) == 0) {
      const int blk = 2 * j + (g >> 1);
      const float f = fmaf((float)c.z, INV65536, fmaf((float)c.y, INV256, (float)c.x));
      const float X = xsum_blk[2 * blk] + xsum_blk[2 * blk + 1];
      acc = fmaf(f16lo(r[j].dm) * sigma, f, acc);
      acc = fmaf(f16hi(r[j].dm), X, acc);
    }
  }
}

}  // namespace
}  // namespace ds4q

// Shared parts of the single-token decode kernels on int8 matrix cores
// (Q2_K in decode_mfma.hip, Q4_1 in decode_q41.hip): operand types, the
// quantisation of an activation vector into three int8 limbs per value in a
// wave's LDS area (in the fragment order of either block format), and the
// routing of the one token by a wave.
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

}  // namespace
}  // namespace ds4q

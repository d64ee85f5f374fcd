// Single-token decode on Q2_K weights with int8 matrix cores.
//
// Arithmetic.  For one 256-value block of a weight row ("【#2】ds4.c
// 해독하기", Q2_K block-layout table) the dot with activations x is
//   sum_v (d*sc_s(v)*q_v - dmin*mn_s(v)) * x_v
//     = d * sum_v (sc_s(v)*q_v) * x_v  -  dmin * sum_s mn_s * X_s,
// X_s being the sum of x over sub-block s.  The integer weights sc*q lie in
// 0..45 and are fed to v_mfma_i32_16x16x64_i8 as they are; the block's
// activations are split into three int8 limbs with a per-block scale
// sigma = max|x| / 127:
//   x ~= sigma * (a0 + a1/254 + a2/254^2),  |a_i| <= 127,
// (residual below sigma/2/254^2, about 2^-22 of the block's largest value),
// so each limb's product with the weights is accumulated exactly in int32 and
// the block result is d*sigma*(C0 + C1/254 + C2/254^2) in fp32.  The min term
// uses X_s summed in fp32 from the unquantised activations.
//
// MFMA operand layout (v_mfma_i32_16x16x64_i8): lane l holds 16 int8 of A
// row l%16 and 16 int8 of B column l%16 for the same 16 K slots (K group
// l/16); C lane l holds C[4*(l/16) + i][l%16].  The K order inside a block is
// free as long as A and B agree: lane group g takes quarter g of the block
// (code bytes 16+16g..16+16g+15), K tile j of the block its code dword j, and
// byte k*4 + i of the 16-byte operand is value 128(g>>1) + 32k + 16(g&1) + 4j
// + i, whose code sits in byte i of dword j at bit pair k and whose sub-block
// 8(g>>1) + 2k + (g&1) is the same for all four i.  With a single token the
// A rows are all the same vector, so every C row holds the result.
//
// A step is three kernels: a one-workgroup prologue (routing + quantised
// activations into the workspace), gate/up + SwiGLU, and down + weighted
// combine (each of its waves quantises its slot's SwiGLU row into LDS).  The
// gate/up waves do no routing or activation arithmetic of their own: each
// reads its expert id, issues its weight loads, copies its quantised
// activation fragments into LDS and runs the MFMA loop.
#include "common.h"
#include "launch.h"

namespace ds4q {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float INV254 = 1.0f / 254.0f;
constexpr float INV254SQ = 1.0f / (254.0f * 254.0f);

// Raw bytes of one 256-value Q2_K block that lane group g uses.
struct Q2KRaw {
  uint32_t q[4], s0, s1, dd;
  __device__ __forceinline__ void load(const uint8_t *__restrict__ blk, int g) {
    const uint8_t *qs = blk + 16 + 16 * g;
    q[0] = ld32(qs); q[1] = ld32(qs + 4); q[2] = ld32(qs + 8); q[3] = ld32(qs + 12);
    s0 = ld32(blk + 8 * (g >> 1));
    s1 = ld32(blk + 8 * (g >> 1) + 4);
    dd = ld32(blk + 80);
  }
};

// Scale/min bytes of the lane's four sub-blocks (k = 0..3).
__device__ __forceinline__ void sub_bytes(const Q2KRaw &r, int p, uint32_t sb[4]) {
  const uint32_t a0 = r.s0 >> (8 * p), a1 = r.s1 >> (8 * p);
  sb[0] = a0 & 0xFFu; sb[1] = (a0 >> 16) & 0xFFu; sb[2] = a1 & 0xFFu; sb[3] = (a1 >> 16) & 0xFFu;
}

// Byte table [0, sc, 2sc, 3sc] of a sub-block's integer weights.
__device__ __forceinline__ uint32_t qsc_table(uint32_t sb) {
  const uint32_t sc = sb & 15u;
  return __umul24(sc, 0x00020100u) + (__umul24(sc, 3u) << 24);
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

__device__ __forceinline__ uint32_t pack_i8(float a, float b, float c, float d) {
  return ((uint32_t)(int)a & 0xFFu) | (((uint32_t)(int)b & 0xFFu) << 8) |
         (((uint32_t)(int)c & 0xFFu) << 16) | (((uint32_t)(int)d & 0xFFu) << 24);
}

// Quantised activations of one vector of NBV blocks (global workspace):
// frag [NBV][3 limbs][4 j][4 g][4 k] dwords, sum [NBV][16] (sub-block sums),
// sig [NBV] (block scales).
struct QAct {
  uint32_t *frag;
  float *sum;
  float *sig;
};

// One thread quantises the 16 activations of one sub-block s (values
// 16s..16s+15 of a block) with the block scale inv = 127 / max|x| and writes
// its 3 limbs x 4 dwords into the block's fragments frag[limb][j][g][k].
__device__ __forceinline__ void quantize_subblock(const float v[16], float inv, int s,
                                                  uint32_t *__restrict__ frag_blk) {
  const int h = s >> 3, k = (s >> 1) & 3, p = s & 1, g = 2 * h + p;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a0[4], a1[4], a2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = v[4 * j + i] * inv;
      a0[i] = rintf(u);
      const float r1 = (u - a0[i]) * 254.0f;
      a1[i] = rintf(r1);
      a2[i] = rintf((r1 - a1[i]) * 254.0f);
    }
    const int off = (j * 4 + g) * 4 + k;
    frag_blk[0 * 64 + off] = pack_i8(a0[0], a0[1], a0[2], a0[3]);
    frag_blk[1 * 64 + off] = pack_i8(a1[0], a1[1], a1[2], a1[3]);
    frag_blk[2 * 64 + off] = pack_i8(a2[0], a2[1], a2[2], a2[3]);
  }
}

__device__ __forceinline__ float max16(float m) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// Thread `t` (of at least 16*NBV, groups of 16 consecutive threads inside one
// wave per block) quantises sub-block t&15 of block t>>4 of `v` (global); the
// block's sigma and sub-block sums are multiplied by `scale` (a positive
// per-vector factor: limbs do not change with it).  `ld` selects coherent
// loads for data written by other workgroups of the same kernel.
template <bool COHERENT>
__device__ __forceinline__ void quantize_one(const float *__restrict__ v, int t, float scale,
                                             QAct q) {
  const int b = t >> 4, s = t & 15;
  float x[16];
  const float *src = v + b * 256 + 16 * s;
  if constexpr (COHERENT) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = reinterpret_cast<const float4 *>(src)[i];
      x[4 * i] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
    }
  }
  float m = 0.f, sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m = fmaxf(m, fabsf(x[i]));
    sum += x[i];
  }
  m = max16(m);
  const float inv = m > 0.f ? 127.0f / m : 0.0f;
  quantize_subblock(x, inv, s, q.frag + b * 192);
  q.sum[b * 16 + s] = sum * scale;
  if (s == 0) q.sig[b] = (m / 127.0f) * scale;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Quantised activations of NBW blocks (from block b0) held in registers on
// their way from the workspace into a wave's LDS area.  Loaded before the
// weight loads are issued and stored after, so that waiting for them does not
// wait for the (in-order) weight loads.
template <int NBW>
struct QActStage {
  static constexpr int NF = (NBW * 48 + 63) / 64, NS = (NBW * 16 + 63) / 64;
  u32x4 f[NF];
  float sm[NS];
  float sg;
  __device__ __forceinline__ void load(const QAct &q, int b0, int lane) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(q.frag + b0 * 192);
#pragma unroll
    for (int i = 0; i < NF; ++i)
      if (lane + 64 * i < NBW * 48) f[i] = src[lane + 64 * i];
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (lane + 64 * i < NBW * 16) sm[i] = q.sum[b0 * 16 + lane + 64 * i];
    if (lane < NBW) sg = q.sig[b0 + lane];
  }
  __device__ __forceinline__ void store(int lane, uint32_t *__restrict__ frag, float *__restrict__ sum,
                                        float *__restrict__ sig) const {
    u32x4 *dst = reinterpret_cast<u32x4 *>(frag);
#pragma unroll
    for (int i = 0; i < NF; ++i)
      if (lane + 64 * i < NBW * 48) dst[lane + 64 * i] = f[i];
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (lane + 64 * i < NBW * 16) sum[lane + 64 * i] = sm[i];
    if (lane < NBW) sig[lane] = sg;
    wave_lds_sync();
  }
};

// The 12 A fragments (3 limbs x 4 K tiles) of one block for lane group g.
struct AFrag {
  i32x4 a[3][4];
  __device__ __forceinline__ void load(const uint32_t *__restrict__ frag_blk, int g) {
#pragma unroll
    for (int l = 0; l < 3; ++l)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[l][j] = *reinterpret_cast<const i32x4 *>(frag_blk + l * 64 + (j * 4 + g) * 4);
  }
};

// Block epilogue: main (replicated over the four lane groups) and the lane
// group's quarter of the min term.
__device__ __forceinline__ void block_post(const Q2KRaw &r, const uint32_t sb[4], const i32x4 c[3],
                                           const float *__restrict__ xsum_blk, float sigma, int g,
                                           float &main_acc, float &min_acc) {
  const int p = g & 1, h = g >> 1;
  const float f = fmaf((float)c[2].x, INV254SQ, fmaf((float)c[1].x, INV254, (float)c[0].x));
  main_acc = fmaf(f16lo(r.dd) * sigma, f, main_acc);
  float mn = (float)(sb[0] >> 4) * xsum_blk[8 * h + p];
  mn = fmaf((float)(sb[1] >> 4), xsum_blk[8 * h + 2 + p], mn);
  mn = fmaf((float)(sb[2] >> 4), xsum_blk[8 * h + 4 + p], mn);
  mn = fmaf((float)(sb[3] >> 4), xsum_blk[8 * h + 6 + p], mn);
  min_acc = fmaf(f16hi(r.dd), mn, min_acc);
}

// One block of NM weight rows (gate and up share the activations): all
// twelve A fragments are read from LDS once, then 12*NM MFMAs.
template <int NM>
__device__ __forceinline__ void block_dot(const Q2KRaw *const r[NM], const uint32_t *__restrict__ frag_blk,
                                          const float *__restrict__ xsum_blk, float sigma, int g,
                                          float *main_acc, float *min_acc) {
  AFrag af;
  af.load(frag_blk, g);
  uint32_t sb[NM][4], tab[NM][4];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    sub_bytes(*r[m], g & 1, sb[m]);
#pragma unroll
    for (int q = 0; q < 4; ++q) tab[m][q] = qsc_table(sb[m][q]);
  }
  i32x4 c[NM][3];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int l = 0; l < 3; ++l) c[m][l] = (i32x4){0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const i32x4 b = b_frag(*r[m], j, tab[m]);
#pragma unroll
      for (int l = 0; l < 3; ++l) c[m][l] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af.a[l][j], b, c[m][l], 0, 0, 0);
    }
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) block_post(*r[m], sb[m], c[m], xsum_blk, sigma, g, main_acc[m], min_acc[m]);
}

template <int MAXE>
__device__ __forceinline__ void route_token(const float *__restrict__ lg, int E, int k, int lane,
                                            int *id, float *w) {
  if constexpr (MAXE == 256) wave_topk256(lg, E, k, lane, id, w);
  else wave_topk<MAXE>(lg, E, k, lane, id, w);
}

// Prologue, one workgroup of 256 threads: routing of the token (wave 0:
// ids, weights) and the
// quantised activations of x (optionally RMS-normalised: only the block
// scales and sub-block sums carry the factor).
template <int D, int MAXE>
__global__ __launch_bounds__(256) void prologue_t1_kernel(const float *__restrict__ x,
                                                          const float *__restrict__ logits, int E,
                                                          int k, int rmsnorm, float eps, QAct xq,
                                                          int32_t *__restrict__ ids,
                                                          float *__restrict__ wts) {
  constexpr int NB = D / 256;
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (w == 0) {
    int id;
    float wt;
    route_token<MAXE>(logits, E, k, lane, &id, &wt);
    if (lane < k) {
      ids[lane] = id;
      wts[lane] = wt;
    }
  }
  float scale = 1.0f;
  if (rmsnorm) {
    float ss = 0.f;
    for (int i = 4 * tid; i < D; i += 1024) {
      const float4 t = *reinterpret_cast<const float4 *>(x + i);
      ss = fmaf(t.x, t.x, ss); ss = fmaf(t.y, t.y, ss);
      ss = fmaf(t.z, t.z, ss); ss = fmaf(t.w, t.w, ss);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) red[w] = ss;
    __syncthreads();
    scale = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)D + eps);
  }
  if (tid < NB * 16) quantize_one<false>(x, tid, scale, xq);
}

// Gate/up + SwiGLU for one token.  Grid (F/16, k): 16 rows of one routed
// expert per workgroup; its four waves split each row's NB blocks into
// quarters and meet in LDS.
template <int D>
__global__ __launch_bounds__(256) void gateup_q2k_t1_kernel(
    const uint8_t *__restrict__ gate, const uint8_t *__restrict__ up, int F, QAct xq,
    const int32_t *__restrict__ ids, float *__restrict__ h) {
  constexpr int NB = D / 256;
  constexpr int BPW = NB >= 4 ? NB / 4 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t frag[4][BPW][192];
  __shared__ float xsum[4][BPW][16];
  __shared__ float sig[4][BPW];
  __shared__ float part[4][2][16];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int slot = blockIdx.y;
  const int row = blockIdx.x * 16 + n;
  const int b0 = w * BPW;
  const bool has = b0 < NB;
  const int64_t rb = (int64_t)NB * BB_Q2K;
  Q2KRaw rg[BPW], ru[BPW];
  float main_g = 0.f, main_u = 0.f, min_g = 0.f, min_u = 0.f;
  if (has) {
    QActStage<BPW> st;
    st.load(xq, b0, lane);
    const int e = ids[slot];
    const int64_t off = ((int64_t)e * F + row) * rb;
#pragma unroll
    for (int bl = 0; bl < BPW; ++bl) {
      rg[bl].load(gate + off + (b0 + bl) * BB_Q2K, g);
      ru[bl].load(up + off + (b0 + bl) * BB_Q2K, g);
      __builtin_amdgcn_sched_barrier(0);
    }
    st.store(lane, &frag[w][0][0], &xsum[w][0][0], &sig[w][0]);
    float mains[2] = {0.f, 0.f}, mins[2] = {0.f, 0.f};
#pragma unroll
    for (int bl = 0; bl < BPW; ++bl) {
      const Q2KRaw *rr[2] = {&rg[bl], &ru[bl]};
      block_dot<2>(rr, frag[w][bl], xsum[w][bl], sig[w][bl], g, mains, mins);
      __builtin_amdgcn_sched_barrier(0);
    }
    main_g = mains[0]; main_u = mains[1];
    min_g = mins[0] + __shfl_xor(mins[0], 16, 64);
    min_g += __shfl_xor(min_g, 32, 64);
    min_u = mins[1] + __shfl_xor(mins[1], 16, 64);
    min_u += __shfl_xor(min_u, 32, 64);
  }
  if (g == 0) {
    part[w][0][n] = main_g - min_g;
    part[w][1][n] = main_u - min_u;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const float gs = (part[0][0][n] + part[1][0][n]) + (part[2][0][n] + part[3][0][n]);
    const float us = (part[0][1][n] + part[1][1][n]) + (part[2][1][n] + part[3][1][n]);
    h[(int64_t)slot * F + row] = silu(gs) * us;
  }
}

// One lane's share of quantising NB blocks of a vector (global) into a wave's
// LDS area: sub-blocks lane, lane+64, ...  load() reads the values, quantise()
// writes the limbs, sums and scales.
template <int NB>
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
        quantize_subblock(x[it], inv, sb, frag + b * 192);
        sum[b * 16 + sb] = acc;
        if (sb == 0) sig[b] = m / 127.0f;
      }
    }
    wave_lds_sync();
  }
};

// Down projection + weighted combine for one token.  Grid D/16, one wave per
// routing slot (blockDim = 64k): each wave quantises its slot's SwiGLU row
// into LDS, streams its expert's 16 down rows, and the slots meet in LDS:
// y (+)= sum_j w_j * (W2[e_j] h_j), summed in slot order.
template <int F>
__global__ __launch_bounds__(512) void down_q2k_t1_kernel(
    const uint8_t *__restrict__ down, int D, int k, const int32_t *__restrict__ ids,
    const float *__restrict__ wts, const float *__restrict__ h, float *__restrict__ y,
    int accumulate) {
  constexpr int NB = F / 256;
  __shared__ __attribute__((aligned(16))) uint32_t frag[8][NB][192];
  __shared__ float xsum[8][NB][16];
  __shared__ float sig[8][NB];
  __shared__ float part[8][16];

  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = blockIdx.x * 16 + n;
  QuantStage<NB> qs;
  qs.load(h + (int64_t)j * F, lane);
  const int e = ids[j];

  const int64_t rb = (int64_t)NB * BB_Q2K;
  Q2KRaw rw[NB];
  const uint8_t *rowp = down + ((int64_t)e * D + row) * rb;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    rw[b].load(rowp + b * BB_Q2K, g);
    __builtin_amdgcn_sched_barrier(0);
  }
  qs.quantise(lane, &frag[j][0][0], &xsum[j][0][0], &sig[j][0]);
  float main_acc = 0.f, min_acc = 0.f;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const Q2KRaw *rr[1] = {&rw[b]};
    block_dot<1>(rr, frag[j][b], xsum[j][b], sig[j][b], g, &main_acc, &min_acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  min_acc += __shfl_xor(min_acc, 16, 64);
  min_acc += __shfl_xor(min_acc, 32, 64);
  if (g == 0) part[j][n] = main_acc - min_acc;
  __syncthreads();
  if (threadIdx.x < 16) {
    float acc = 0.f;
    for (int s = 0; s < k; ++s) acc = fmaf(wts[s], part[s][n], acc);
    y[row] = accumulate ? y[row] + acc : acc;
  }
}

}  // namespace

size_t qact_bytes(int n_vec, int len) {
  const size_t nb = (size_t)len / 256;
  return ((size_t)n_vec * nb * (192 * 4 + 16 * 4 + 4) + 255) & ~(size_t)255;
}

static QAct qact_view(void *base, int n_vec, int len) {
  const size_t nb = (size_t)n_vec * (len / 256);
  QAct q;
  q.frag = static_cast<uint32_t *>(base);
  q.sum = reinterpret_cast<float *>(q.frag + nb * 192);
  q.sig = q.sum + nb * 16;
  return q;
}

hipError_t launch_decode_q2k_t1(const MoeDims &m, const float *x, const float *logits,
                                bool rmsnorm, float eps, const RouteBufs &rb, float *h, void *qbuf,
                                float *y, bool accumulate, int phase, hipStream_t s) {
  const QAct xq = qact_view(qbuf, 1, m.D);
  if (phase == 0) {
#define DS4Q_PRO(DD)                                                                            \
  if (m.E <= 256)                                                                               \
    hipLaunchKernelGGL((prologue_t1_kernel<DD, 256>), dim3(1), dim3(256), 0, s, x, logits, m.E,  \
                       m.k, rmsnorm ? 1 : 0, eps, xq, rb.ids, rb.w);                             \
  else                                                                                          \
    hipLaunchKernelGGL((prologue_t1_kernel<DD, ROUTE_MAX_E>), dim3(1), dim3(256), 0, s, x,       \
                       logits, m.E, m.k, rmsnorm ? 1 : 0, eps, xq, rb.ids, rb.w)
    switch (m.D) {
      case 256: DS4Q_PRO(256); break;
      case 512: DS4Q_PRO(512); break;
      case 1024: DS4Q_PRO(1024); break;
      case 2048: DS4Q_PRO(2048); break;
      case 4096: DS4Q_PRO(4096); break;
      default: return hipErrorInvalidValue;
    }
#undef DS4Q_PRO
  } else if (phase == 1) {
    const dim3 grid(m.F / 16, m.k);
#define DS4Q_GU(DD)                                                                             \
  hipLaunchKernelGGL((gateup_q2k_t1_kernel<DD>), grid, dim3(256), 0, s, m.gate, m.up, m.F, xq,   \
                     rb.ids, h)
    switch (m.D) {
      case 256: DS4Q_GU(256); break;
      case 512: DS4Q_GU(512); break;
      case 1024: DS4Q_GU(1024); break;
      case 2048: DS4Q_GU(2048); break;
      case 4096: DS4Q_GU(4096); break;
      default: return hipErrorInvalidValue;
    }
#undef DS4Q_GU
  } else {
    const dim3 block(64 * m.k);
#define DS4Q_DN(FF)                                                                             \
  hipLaunchKernelGGL((down_q2k_t1_kernel<FF>), dim3(m.D / 16), block, 0, s, m.down, m.D, m.k,    \
                     rb.ids, rb.w, h, y, accumulate ? 1 : 0)
    switch (m.F) {
      case 256: DS4Q_DN(256); break;
      case 512: DS4Q_DN(512); break;
      case 1024: DS4Q_DN(1024); break;
      case 2048: DS4Q_DN(2048); break;
      case 4096: DS4Q_DN(4096); break;
      default: return hipErrorInvalidValue;
    }
#undef DS4Q_DN
  }
  return hipGetLastError();
}

}  // namespace ds4q

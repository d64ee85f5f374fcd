// Decode of 2..64 tokens on int8 matrix cores, either block format, grouped
// by expert.
//
// The arithmetic is that of the one-token kernels (mfma_t1.h): activations as
// three int8 limbs per value with one scale per 256 values, weights as exact
// integers (sc*q for Q2_K, q for Q4_1) on v_mfma_i32_16x16x64_i8, the min /
// offset term in fp32.  What changes is the work split: a workgroup owns 16
// weight rows of one active expert ("【#2】ds4.c 해독하기": routed experts,
// w1 = gate, w3 = up, w2 = down) and every token routed to it.  Its waves
// issue all their weight loads first and build the weight operands once
// (Q2_K: the B fragments of every K tile), then loop over the expert's pairs
// in sorted order: the next token's activations are quantised into the other
// of two LDS buffers while the current one runs through the MFMAs.  Each
// weight byte is read once per call, with as many requests in flight as the
// one-token kernels.
//
// Gate/up + SwiGLU: grid (F/16, active experts), eight waves (four K
// quarters of the gate rows, four of the up rows); the gate waves quantise
// the shared activations.  h is written per pair (pair index t*k + slot).
// Down: grid (D/16, active experts), eight waves splitting K; each wave
// quantises its own slice of the pair's SwiGLU row; the unweighted product is
// written per pair to o, and the combine kernel sums a token's slots with the
// routing weights in slot order (deterministic, no atomics).
#include "common.h"
#include "launch.h"
#include "mfma_t1.h"

namespace ds4q {
namespace {

// The weight operands of one Q2_K block for the lane: the B fragments of the
// four K tiles, the four min nibbles of its sub-blocks and (d, dmin).
struct Q2KOps {
  i32x4 b[4];
  uint32_t mn, dd;
  __device__ __forceinline__ void build(const Q2KRaw &r, int g) {
    uint32_t sb[4], tab[4];
    sub_bytes(r, g & 1, sb);
#pragma unroll
    for (int q = 0; q < 4; ++q) tab[q] = qsc_table(sb[q]);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = b_frag(r, j, tab);
    mn = (sb[0] >> 4) | ((sb[1] >> 4) << 8) | ((sb[2] >> 4) << 16) | ((sb[3] >> 4) << 24);
    dd = r.dd;
  }
  // one token's block: main term (lane group 0) and the lane group's quarter
  // of the min term, as block_post
  __device__ __forceinline__ void dot(const uint32_t *__restrict__ frag_blk, const float *__restrict__ xsum_blk,
                                      float sigma, int n, int g, float &main_acc, float &min_acc) const {
    AFrag af;
    af.load(frag_blk, n, g);
    i32x4 c = (i32x4){0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j == 0) mfma_group_begin();
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(af.a[j], b[j], c, 0, 0, 0);
    }
    mfma_fence();
    const int p = g & 1, h = g >> 1;
    const float f = fmaf((float)c.z, INV65536, fmaf((float)c.y, INV256, (float)c.x));
    main_acc = fmaf(f16lo(dd) * sigma, f, main_acc);
    float m = (float)(mn & 0xFFu) * xsum_blk[8 * h + p];
    m = fmaf((float)((mn >> 8) & 0xFFu), xsum_blk[8 * h + 2 + p], m);
    m = fmaf((float)((mn >> 16) & 0xFFu), xsum_blk[8 * h + 4 + p], m);
    m = fmaf((float)(mn >> 24), xsum_blk[8 * h + 6 + p], m);
    min_acc = fmaf(f16hi(dd), m, min_acc);
  }
};

// A wave's weights of NB256 256-value chunks of one row (lane's share), for
// either format, and its dot with one token's quantised chunks.
template <bool Q41, int NC>
struct WaveRows {
  Q2KRaw raw2[Q41 ? 1 : NC];
  Q2KOps ops2[Q41 ? 1 : NC];
  Q41Raw raw4[Q41 ? NC : 1][4];
  __device__ __forceinline__ void load(const uint8_t *__restrict__ rowp, int g) {
    if constexpr (Q41) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) raw4[c][j].load(rowp + c * 8 * BB_Q41, j, g);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) raw2[c].load(rowp + c * BB_Q2K, g);
    }
  }
  __device__ __forceinline__ void build(int g) {
    if constexpr (!Q41) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        raw2[c].finish();
        ops2[c].build(raw2[c], g);
      }
    }
  }
  // sum over the chunks of the 16 rows x this token; lane group 0 returns it
  __device__ __forceinline__ float dot(const uint32_t *__restrict__ frag, const float *__restrict__ xsum,
                                       const float *__restrict__ sig, int n, int g) const {
    float acc = 0.f;
    if constexpr (Q41) {
#pragma unroll
      for (int c = 0; c < NC; ++c) chunk_dot_q41(raw4[c], frag + c * 192, xsum + c * 16, sig[c], n, g, acc);
      acc += __shfl_xor(acc, 32, 64);
    } else {
      float mn = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) ops2[c].dot(frag + c * 192, xsum + c * 16, sig[c], n, g, acc, mn);
      mn += __shfl_xor(mn, 16, 64);
      mn += __shfl_xor(mn, 32, 64);
      acc -= mn;
    }
    return acc;
  }
};

template <int D, bool Q41>
__global__ __launch_bounds__(512) void gateup_tn_kernel(const uint8_t *__restrict__ gate,
                                                        const uint8_t *__restrict__ up, int F, int k,
                                                        const float *__restrict__ x,
                                                        const float *__restrict__ inv_rms, RouteBufs rb,
                                                        float *__restrict__ h) {
  constexpr int NB = D / 256;
  constexpr int BPW = NB >= 4 ? NB / 4 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t frag[2][4][BPW][192];
  __shared__ float xsum[2][4][BPW][16];
  __shared__ float sig[2][4][BPW];
  __shared__ float part[8][16];

  const int j = blockIdx.y;
  if (j >= *rb.n_active) return;
  const int e = rb.act_expert[j], pb = rb.act_begin[j], np = rb.act_begin[j + 1] - pb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = blockIdx.x * 16 + n;
  const int quarter = w & 3, b0 = quarter * BPW;
  const bool has = b0 < NB;
  const bool quantiser = w < 4 && has;  // the gate waves quantise the shared activations
  const uint8_t *__restrict__ mat = w < 4 ? gate : up;

  // the first token's activations are requested before the weights, so that
  // quantising them waits only for them (requests complete in order)
  QuantStage<BPW, Q41> xs;
  if (quantiser) xs.load(x + (int64_t)(rb.pairs[pb] / k) * D + b0 * 256, lane);
  WaveRows<Q41, BPW> wr;
  if (has) {
    const int64_t rb_bytes = row_bytes(Q41 ? TYPE_Q4_1 : TYPE_Q2_K, D);
    wr.load(mat + ((int64_t)e * F + row) * rb_bytes + (int64_t)b0 * (Q41 ? 8 * BB_Q41 : BB_Q2K), g);
  }
  if (quantiser) xs.quantise(lane, &frag[0][quarter][0][0], &xsum[0][quarter][0][0], &sig[0][quarter][0]);
  if (has) wr.build(g);
  __syncthreads();
  for (int i = 0; i < np; ++i) {
    const int buf = i & 1;
    const bool next = quantiser && i + 1 < np;
    if (next) xs.load(x + (int64_t)(rb.pairs[pb + i + 1] / k) * D + b0 * 256, lane);
    float acc = 0.f;
    if (has) acc = wr.dot(&frag[buf][quarter][0][0], &xsum[buf][quarter][0][0], &sig[buf][quarter][0], n, g);
    if (g == 0) part[w][n] = acc;
    if (next) xs.quantise(lane, &frag[buf ^ 1][quarter][0][0], &xsum[buf ^ 1][quarter][0][0], &sig[buf ^ 1][quarter][0]);
    __syncthreads();  // this token's parts and the next token's fragments are visible
    if (threadIdx.x < 16) {
      const int p = rb.pairs[pb + i];
      const float scale = inv_rms ? inv_rms[p / k] : 1.0f;
      const float gs = ((part[0][n] + part[1][n]) + (part[2][n] + part[3][n])) * scale;
      const float us = ((part[4][n] + part[5][n]) + (part[6][n] + part[7][n])) * scale;
      h[(int64_t)p * F + row] = silu(gs) * us;
    }
    __syncthreads();  // parts read; buffer buf free for token i+2
  }
}

template <int F, bool Q41>
__global__ __launch_bounds__(512) void down_tn_kernel(const uint8_t *__restrict__ down, int D,
                                                      const float *__restrict__ h, RouteBufs rb,
                                                      float *__restrict__ o) {
  constexpr int NB = F / 256;
  constexpr int BPW = NB >= 8 ? NB / 8 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t frag[2][8][BPW][192];
  __shared__ float xsum[2][8][BPW][16];
  __shared__ float sig[2][8][BPW];
  __shared__ float part[8][16];

  const int j = blockIdx.y;
  if (j >= *rb.n_active) return;
  const int e = rb.act_expert[j], pb = rb.act_begin[j], np = rb.act_begin[j + 1] - pb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = blockIdx.x * 16 + n;
  const int b0 = w * BPW;
  const bool has = b0 < NB;

  WaveRows<Q41, BPW> wr;
  QuantStage<BPW, Q41> hs;
  if (has) {
    const int64_t rb_bytes = row_bytes(Q41 ? TYPE_Q4_1 : TYPE_Q2_K, F);
    hs.load(h + (int64_t)rb.pairs[pb] * F + b0 * 256, lane);  // before the weights (see above)
    wr.load(down + ((int64_t)e * D + row) * rb_bytes + (int64_t)b0 * (Q41 ? 8 * BB_Q41 : BB_Q2K), g);
    hs.quantise(lane, &frag[0][w][0][0], &xsum[0][w][0][0], &sig[0][w][0]);
    wr.build(g);
  }
  for (int i = 0; i < np; ++i) {
    const int buf = i & 1;
    const bool next = has && i + 1 < np;
    if (next) hs.load(h + (int64_t)rb.pairs[pb + i + 1] * F + b0 * 256, lane);
    float acc = 0.f;
    if (has) acc = wr.dot(&frag[buf][w][0][0], &xsum[buf][w][0][0], &sig[buf][w][0], n, g);
    if (g == 0) part[w][n] = acc;
    if (next) hs.quantise(lane, &frag[buf ^ 1][w][0][0], &xsum[buf ^ 1][w][0][0], &sig[buf ^ 1][w][0]);
    __syncthreads();
    if (threadIdx.x < 16) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) s += part[q][n];
      o[(int64_t)rb.pairs[pb + i] * D + row] = s;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_decode_tn(const MoeDims &m, const float *x, const float *inv_rms, int T,
                            const RouteBufs &rb, float *h, float *o, int phase, hipStream_t s) {
  const int max_active = T * m.k < m.E ? T * m.k : m.E;
  if (T == 0 || max_active == 0) return hipSuccess;
  if (phase == 1) {
    const dim3 grid(m.F / 16, max_active);
    const bool q41 = m.tg == TYPE_Q4_1;
#define DS4Q_GU(DD)                                                                                   \
  if (q41) hipLaunchKernelGGL((gateup_tn_kernel<DD, true>), grid, dim3(512), 0, s, m.gate, m.up, m.F, m.k, \
                              x, inv_rms, rb, h);                                                       \
  else hipLaunchKernelGGL((gateup_tn_kernel<DD, false>), grid, dim3(512), 0, s, m.gate, m.up, m.F, m.k,    \
                          x, inv_rms, rb, h)
    switch (m.D) {
      case 256: DS4Q_GU(256); break;
      case 512: DS4Q_GU(512); break;
      case 1024: DS4Q_GU(1024); break;
      case 2048: DS4Q_GU(2048); break;
      case 4096: DS4Q_GU(4096); break;
      default: return hipErrorInvalidValue;
    }
#undef DS4Q_GU
  } else if (phase == 2) {
    const dim3 grid(m.D / 16, max_active);
    const bool q41 = m.td == TYPE_Q4_1;
#define DS4Q_DN(FF)                                                                                  \
  if (q41) hipLaunchKernelGGL((down_tn_kernel<FF, true>), grid, dim3(512), 0, s, m.down, m.D, h, rb, o); \
  else hipLaunchKernelGGL((down_tn_kernel<FF, false>), grid, dim3(512), 0, s, m.down, m.D, h, rb, o)
    switch (m.F) {
      case 256: DS4Q_DN(256); break;
      case 512: DS4Q_DN(512); break;
      case 1024: DS4Q_DN(1024); break;
      case 2048: DS4Q_DN(2048); break;
      case 4096: DS4Q_DN(4096); break;
      default: return hipErrorInvalidValue;
    }
#undef DS4Q_DN
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ds4q

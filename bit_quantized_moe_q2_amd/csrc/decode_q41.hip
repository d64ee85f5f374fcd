// Single-token decode on Q4_1 weights with int8 matrix cores.
//
// Arithmetic.  A 32-value Q4_1 block (ThakiCloud "...GGUF Q4_1 재부호화",
// Q4_1 block section: fp16 d, fp16 m, 16 code bytes, value = d*q + m) dotted
// with activations x is d * sum_v q_v x_v + m * X, X the sum of x over the
// block.  The codes q (0..15) are the B operand of v_mfma_i32_16x16x64_i8 as
// they are; the activations enter as three int8 limbs per value with one
// scale per 256 values (mfma_t1.h), so each block's integer sums are exact
// and the block result is d*sigma*(C0 + C1/256 + C2/65536) + m*X in fp32.
//
// Operand layout.  One MFMA covers K tile j of a 256-value chunk: blocks 2j
// and 2j+1.  Lane (n, g) holds B column n (weight row n) for K slots
// 16g..16g+15: half p = g & 1 of block 2j + (g >> 1), i.e. the low nibbles
// (values 8p..8p+7) and the high nibbles (values 16+8p..16+8p+7) of its code
// bytes 8p..8p+7.  Every lane reads 12 bytes at block offset 8p: half 0
// gets (d, m) and code bytes 0..7, half 1 code bytes 4..15, so the codes are
// dwords 1 and 2 for both and the lanes of half 0 hold their block's d and m.
// A rows 0..2 are the limbs of block 2j in K slots 0..31 (zero elsewhere),
// rows 8..10 those of block 2j+1 in K slots 32..63, so C rows 0..2 (lanes
// 0..15, g = 0) hold block 2j's three limb sums and C rows 8..10 (lanes
// 32..47, g = 2) block 2j+1's: exactly the lanes of half 0 of each block,
// which scale it with their own d and add m*X.  The other lanes carry zero
// rows and skip the epilogue (their fp16 fields are never used, so no NaN can
// enter).
//
// Kernels and launches as for Q2_K (decode_mfma.hip): gate/up + SwiGLU with
// the routing inside, then down + weighted combine.
#include "common.h"
#include "launch.h"
#include "mfma_t1.h"

namespace ds4q {
namespace {

// Gate/up + SwiGLU for one token on Q4_1 (same grid, waves, routing and
// epilogue as gateup_q2k_t1_kernel).
template <int D, int MAXE>
__global__ __launch_bounds__(512) void gateup_q41_t1_kernel(
    const uint8_t *__restrict__ gate, const uint8_t *__restrict__ up, int F, int E, int k,
    const float *__restrict__ x, const float *__restrict__ logits, int rmsnorm, float eps,
    int32_t *__restrict__ ids_out, float *__restrict__ w_out, float *__restrict__ h) {
  constexpr int NB = D / 256;
  constexpr int BPW = NB >= 4 ? NB / 4 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t frag[4][BPW][192];
  __shared__ float xsum[4][BPW][16];
  __shared__ float sig[4][BPW];
  __shared__ float part[8][16];
  __shared__ float ssq[4];
  __shared__ int expert;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int slot = blockIdx.y;
  const int row = blockIdx.x * 16 + n;
  const int quarter = w & 3;
  const int b0 = quarter * BPW;
  const bool has = b0 < NB;
  const uint8_t *__restrict__ mat = w < 4 ? gate : up;
  const int router_w = (blockIdx.x + blockIdx.y) & 7;
  const bool router = w == router_w;
  const bool quantiser = w == (quarter == (router_w & 3) ? (router_w ^ 4) : quarter);
  TokenRoute<MAXE> rt;
  if (router) rt.load(logits, E, lane);
  QuantStage<BPW, true> xs;
  float ss = 0.f;
  if (quantiser && has) xs.load(x + b0 * 256, lane);
  if (router) {
    int my_id;
    float my_w;
    const bool store = blockIdx.x == 0 && slot == 0;
    __builtin_amdgcn_s_setprio(3);
    rt.select(E, k, slot + 1, store, lane, &my_id, &my_w);
    __builtin_amdgcn_s_setprio(0);
    if (store && lane < k) {
      ids_out[lane] = my_id;
      w_out[lane] = my_w;
    }
    if (lane == slot) expert = my_id;
  } else if (quantiser && has) {
    xs.quantise(lane, &frag[quarter][0][0], &xsum[quarter][0][0], &sig[quarter][0]);
    if (rmsnorm) ss = xs.sumsq(lane);
  }
  if (quantiser && rmsnorm) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) ssq[quarter] = ss;
  }
  __syncthreads();
  const int e = expert;
  const int64_t rb = (int64_t)(D / 32) * BB_Q41;
  float acc = 0.f;
  if (has) {
    Q41Raw rw[BPW][4];
    const uint8_t *rowp = mat + ((int64_t)e * F + row) * rb + b0 * CHUNK_BYTES;
#pragma unroll
    for (int bl = 0; bl < BPW; ++bl) {
#pragma unroll
      for (int j = 0; j < 4; ++j) rw[bl][j].load(rowp + bl * CHUNK_BYTES, j, g);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int bl = 0; bl < BPW; ++bl) {
      chunk_dot_q41(rw[bl], frag[quarter][bl], xsum[quarter][bl], sig[quarter][bl], n, g, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    acc += __shfl_xor(acc, 32, 64);
  }
  if (g == 0) part[w][n] = acc;
  __syncthreads();
  if (threadIdx.x < 16) {
    const float scale = rmsnorm ? 1.0f / sqrtf(((ssq[0] + ssq[1]) + (ssq[2] + ssq[3])) / (float)D + eps) : 1.0f;
    const float gs = ((part[0][n] + part[1][n]) + (part[2][n] + part[3][n])) * scale;
    const float us = ((part[4][n] + part[5][n]) + (part[6][n] + part[7][n])) * scale;
    h[(int64_t)slot * F + row] = silu(gs) * us;
  }
}

// Down projection + weighted combine for one token on Q4_1 (grid D/16, WPS
// waves per routing slot, as down_q2k_t1_kernel).
template <int F>
__global__ __launch_bounds__(1024) void down_q41_t1_kernel(
    const uint8_t *__restrict__ down, int D, int k, const int32_t *__restrict__ ids,
    const float *__restrict__ wts, const float *__restrict__ h, float *__restrict__ y,
    int accumulate, float *__restrict__ stage) {
  constexpr int NB = F / 256;
  constexpr int WPS = NB >= 2 ? 2 : 1;
  constexpr int BPW = NB / WPS;
  __shared__ __attribute__((aligned(16))) uint32_t frag[8 * WPS][BPW][192];
  __shared__ float xsum[8 * WPS][BPW][16];
  __shared__ float sig[8 * WPS][BPW];
  __shared__ float part[8 * WPS][16];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int j = wv / WPS, b0 = (wv % WPS) * BPW;
  const int n = lane & 15, g = lane >> 4;
  const int row = blockIdx.x * 16 + n;
  // the output row to accumulate into, requested first (the result is
  // stored last, so waiting for this load there would add its latency)
  const float y_old = accumulate && !stage && threadIdx.x < 16 ? y[row] : 0.f;
  QuantStage<BPW, true> qs;
  qs.load(h + (int64_t)j * F + b0 * 256, lane);
  const int e = ids[j];
  // weight loads first, the quantisation of the SwiGLU row runs under them;
  // at n_ff = 4096 the row and 8 blocks of weights do not fit in registers
  // together, so there the row is quantised first
  constexpr bool QFIRST = F >= 4096;
  if constexpr (QFIRST) qs.quantise(lane, &frag[wv][0][0], &xsum[wv][0][0], &sig[wv][0]);
  const int64_t rb = (int64_t)(F / 32) * BB_Q41;
  Q41Raw rw[BPW][4];
  const uint8_t *rowp = down + ((int64_t)e * D + row) * rb + b0 * CHUNK_BYTES;
#pragma unroll
  for (int bl = 0; bl < BPW; ++bl) {
#pragma unroll
    for (int t = 0; t < 4; ++t) rw[bl][t].load(rowp + bl * CHUNK_BYTES, t, g);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!QFIRST) qs.quantise(lane, &frag[wv][0][0], &xsum[wv][0][0], &sig[wv][0]);
  float acc = 0.f;
#pragma unroll
  for (int bl = 0; bl < BPW; ++bl) {
    chunk_dot_q41(rw[bl], frag[wv][bl], xsum[wv][bl], sig[wv][bl], n, g, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  acc += __shfl_xor(acc, 32, 64);
  if (g == 0) part[wv][n] = acc;
  __syncthreads();
  if (threadIdx.x < 16) {
    float out = 0.f;
    for (int s = 0; s < k; ++s) {
      float ps = part[s * WPS][n];
#pragma unroll
      for (int q = 1; q < WPS; ++q) ps += part[s * WPS + q][n];
      out = fmaf(wts[s], ps, out);
    }
    if (stage) stage[row] = out;  // steered by the launch that follows
    else y[row] = accumulate ? y_old + out : out;
  }
}

}  // namespace

hipError_t launch_decode_q41_t1(const MoeDims &m, const float *x, const float *logits,
                                bool rmsnorm, float eps, const RouteBufs &rb, float *h, float *y,
                                bool accumulate, int phase, const SteerArgs &st, hipStream_t s) {
  if (phase == 1) {
    const dim3 grid(m.F / 16, m.k);
#define DS4Q_GU(DD, ME)                                                                          \
  hipLaunchKernelGGL((gateup_q41_t1_kernel<DD, ME>), grid, dim3(512), 0, s, m.gate, m.up, m.F,     \
                     m.E, m.k, x, logits, rmsnorm ? 1 : 0, eps, rb.ids, rb.w, h)
#define DS4Q_GU_E(DD)                            \
  if (m.E <= 256) DS4Q_GU(DD, 256);              \
  else DS4Q_GU(DD, ROUTE_MAX_E)
    switch (m.D) {
      case 256: DS4Q_GU_E(256); break;
      case 512: DS4Q_GU_E(512); break;
      case 1024: DS4Q_GU_E(1024); break;
      case 2048: DS4Q_GU_E(2048); break;
      case 4096: DS4Q_GU_E(4096); break;
      default: return hipErrorInvalidValue;
    }
#undef DS4Q_GU_E
#undef DS4Q_GU
  } else if (phase == 2) {
    const int wps = m.F >= 512 ? 2 : 1;
    const dim3 block(64 * m.k * wps);
#define DS4Q_DN(FF)                                                                             \
  hipLaunchKernelGGL((down_q41_t1_kernel<FF>), dim3(m.D / 16), block, 0, s, m.down, m.D, m.k,    \
                     rb.ids, rb.w, h, y, accumulate ? 1 : 0, st.dir ? st.stage : nullptr)
    switch (m.F) {
      case 256: DS4Q_DN(256); break;
      case 512: DS4Q_DN(512); break;
      case 1024: DS4Q_DN(1024); break;
      case 2048: DS4Q_DN(2048); break;
      case 4096: DS4Q_DN(4096); break;
      default: return hipErrorInvalidValue;
    }
#undef DS4Q_DN
    if (st.dir) {
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      return launch_steer(st.dir, st.scale, st.stage, 1, m.D, y, accumulate, s);
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ds4q

// Single-token decode on Q2_K weights with int8 matrix cores.
//
// Arithmetic.  For one 256-value block of a weight row ("【#2】ds4.c
// 해독하기", Q2_K block-layout table) the dot with activations x is
//   sum_v (d*sc_s(v)*q_v - dmin*mn_s(v)) * x_v
//     = d * sum_v (sc_s(v)*q_v) * x_v  -  dmin * sum_s mn_s * X_s,
// X_s being the sum of x over sub-block s.  The integer weights sc*q lie in
// 0..45 and are fed to v_mfma_i32_16x16x64_i8 as they are; the block's
// activations are split into three int8 limbs with a per-block scale
// sigma = max|x| / 127: N = trunc(x * 127 * 65536 / max|x| + 32896) has the
// balanced base-256 digits a0 = byte 2, a1 = byte 1 - 128, a2 = byte 0 - 128
// (all within [-127, 127]), so that
//   x ~= sigma * (a0 + a1/256 + a2/65536)
// with a residual below 1.3 * sigma / 65536 (about 2^-23 of the block's
// largest value).  Each limb's product with the weights is accumulated
// exactly in int32 and the block result is d*sigma*(C0 + C1/256 + C2/65536)
// in fp32.  The min term uses X_s summed in fp32 from the unquantised
// activations.
//
// MFMA operand layout (v_mfma_i32_16x16x64_i8): lane l holds 16 int8 of A
// row l%16 and 16 int8 of B column l%16 for the same 16 K slots (K group
// l/16); C lane l holds C[4*(l/16) + i][l%16].  The K order inside a block is
// free as long as A and B agree: lane group g takes quarter g of the block
// (code bytes 16+16g..16+16g+15), K tile j of the block its code dword j, and
// byte k*4 + i of the 16-byte operand is value 128(g>>1) + 32k + 16(g&1) + 4j
// + i, whose code sits in byte i of dword j at bit pair k and whose sub-block
// 8(g>>1) + 2k + (g&1) is the same for all four i.  With a single token the
// three limbs take A rows 0..2 (rows 3..15 are zero), so one MFMA per K tile
// gives all three limb products of 16 weight rows: C[limb][row], held by
// lanes 0..15.
//
// A step is two kernels.  Gate/up + SwiGLU: each workgroup routes the token
// itself (top-k of the logits in one wave, a few hundred VALU instructions,
// cheaper than a launch and a round trip through memory); every wave then
// issues its expert's weight loads, quantises its own quarter of x into LDS
// meanwhile and runs the MFMA loop; workgroup (0, 0) also stores the routing
// for the second kernel.  Down +
// weighted combine: each wave quantises its share of its slot's SwiGLU row
// into LDS while its weight loads are in flight.  The RMS norm of the input
// is a per-token factor, applied to the gate and up sums in the epilogue.
#include "common.h"
#include "launch.h"
#include "mfma_t1.h"

namespace ds4q {
namespace {

// Gate/up + SwiGLU for one token.  Grid (F/16, k): 16 rows of one routed
// expert per workgroup of eight waves; waves 0..3 take the four quarters of
// each gate row's NB blocks, waves 4..7 those of the up rows (one matrix per
// wave streams faster than interleaving both), and the waves meet in LDS.
// One wave routes the token ("ds4.c 해독하기 1/8", DS4_SHAPE_FLASH passage: 6
// of 256 routed experts); the other wave of its quarter pair quantises that
// quarter of x, gate and up waves share the fragments; workgroup (0, 0)
// stores the routing for the down kernel.  With rmsnorm, the sums are
// multiplied by 1/sqrt(mean(x^2) + eps): the quantised limbs do not depend on
// that factor.
template <int D, int MAXE>
__global__ __launch_bounds__(512) void gateup_q2k_t1_kernel(
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
  // One wave per workgroup routes (which one rotates with the workgroup, so
  // that the routing work spreads over the SIMDs); the other wave of its
  // quarter pair quantises, and so does the gate wave of each other pair.
  const int router_w = (blockIdx.x + blockIdx.y) & 7;
  const bool router = w == router_w;
  const bool quantiser = w == (quarter == (router_w & 3) ? (router_w ^ 4) : quarter);
  TokenRoute<MAXE> rt;
  if (router) rt.load(logits, E, lane);
  QuantStage<BPW> xs;
  float ss = 0.f;
  if (quantiser && has) xs.load(x + b0 * 256, lane);
  if (router) {
    int my_id;
    float my_w;
    // only workgroup (0, 0) stores the routing; the others need their slot.
    // Every wave of the workgroup waits for this, so it is issued ahead of
    // the quantising waves that share its SIMD.
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
  const int64_t rb = (int64_t)NB * BB_Q2K;
  float main_acc = 0.f, min_acc = 0.f;
  if (has) {
    Q2KRaw rw[BPW];
    const uint8_t *rowp = mat + ((int64_t)e * F + row) * rb + b0 * BB_Q2K;
#pragma unroll
    for (int bl = 0; bl < BPW; ++bl) {
      rw[bl].load(rowp + bl * BB_Q2K, g);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int bl = 0; bl < BPW; ++bl) {
      rw[bl].finish();
      const Q2KRaw *rr[1] = {&rw[bl]};
      block_dot<1, 1>(rr, frag[quarter][bl], xsum[quarter][bl], sig[quarter][bl], n, g, &main_acc, &min_acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    min_acc += __shfl_xor(min_acc, 16, 64);
    min_acc += __shfl_xor(min_acc, 32, 64);
  }
  if (g == 0) part[w][n] = main_acc - min_acc;
  __syncthreads();
  if (threadIdx.x < 16) {
    const float scale = rmsnorm ? 1.0f / sqrtf(((ssq[0] + ssq[1]) + (ssq[2] + ssq[3])) / (float)D + eps) : 1.0f;
    const float gs = ((part[0][n] + part[1][n]) + (part[2][n] + part[3][n])) * scale;
    const float us = ((part[4][n] + part[5][n]) + (part[6][n] + part[7][n])) * scale;
    h[(int64_t)slot * F + row] = silu(gs) * us;
  }
}

// Down projection + weighted combine for one token.  Grid D/16; WPS waves per
// routing slot (blockDim = 64 * k * WPS), each taking NB/WPS blocks of the
// slot's rows: a wave requests its expert's 16 down rows, quantises its part
// of the slot's SwiGLU row into LDS meanwhile, and the waves meet in LDS:
// y (+)= sum_j w_j * (W2[e_j] h_j), summed in slot order.
template <int F>
__global__ __launch_bounds__(1024) void down_q2k_t1_kernel(
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
  QuantStage<BPW> qs;
  qs.load(h + (int64_t)j * F + b0 * 256, lane);
  const int e = ids[j];
  // The weight loads go out as soon as the expert id is in, before the
  // quantisation of the SwiGLU row (which waits for that row only), so the
  // quantisation runs under the weights' latency.
  const int64_t rb = (int64_t)NB * BB_Q2K;
  Q2KRaw rw[BPW];
  const uint8_t *rowp = down + ((int64_t)e * D + row) * rb + b0 * BB_Q2K;
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
    rw[b].load(rowp + b * BB_Q2K, g);
    __builtin_amdgcn_sched_barrier(0);
  }
  qs.quantise(lane, &frag[wv][0][0], &xsum[wv][0][0], &sig[wv][0]);
  float main_acc = 0.f, min_acc = 0.f;
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
    rw[b].finish();
    const Q2KRaw *rr[1] = {&rw[b]};
    block_dot<1, 4>(rr, frag[wv][b], xsum[wv][b], sig[wv][b], n, g, &main_acc, &min_acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  min_acc += __shfl_xor(min_acc, 16, 64);
  min_acc += __shfl_xor(min_acc, 32, 64);
  if (g == 0) part[wv][n] = main_acc - min_acc;
  __syncthreads();
  if (threadIdx.x < 16) {
    float acc = 0.f;
    for (int s = 0; s < k; ++s) {
      float ps = part[s * WPS][n];
#pragma unroll
      for (int q = 1; q < WPS; ++q) ps += part[s * WPS + q][n];
      acc = fmaf(wts[s], ps, acc);
    }
    if (stage) stage[row] = acc;  // steered by the launch that follows
    else y[row] = accumulate ? y_old + acc : acc;
  }
}

}  // namespace

hipError_t launch_decode_q2k_t1(const MoeDims &m, const float *x, const float *logits,
                                bool rmsnorm, float eps, const RouteBufs &rb, float *h, float *y,
                                bool accumulate, int phase, const SteerArgs &st, hipStream_t s) {
  if (phase == 1) {
    const dim3 grid(m.F / 16, m.k);
#define DS4Q_GU(DD, ME)                                                                          \
  hipLaunchKernelGGL((gateup_q2k_t1_kernel<DD, ME>), grid, dim3(512), 0, s, m.gate, m.up, m.F,     \
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
  hipLaunchKernelGGL((down_q2k_t1_kernel<FF>), dim3(m.D / 16), block, 0, s, m.down, m.D, m.k,    \
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

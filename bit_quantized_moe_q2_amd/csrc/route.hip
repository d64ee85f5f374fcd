// Routing: top-k of n_expert router logits per token with softmax weights over
// the selected k ("ds4.c 해독하기 1/8", DS4_SHAPE_FLASH passage: 6 of 256
// routed experts per token), and the token->expert grouping (counting sort of
// the T*k (token, slot) pairs by expert, stable in pair index).
//
// Selection order is (logit desc, index asc): each candidate is packed into a
// 64-bit key (order-preserving fp32 bits << 32 | ~index) and the wave takes
// k rounds of a 64-bit max; -0.0 is folded onto +0.0 so that equal logits
// tie exactly as floating-point comparison says.
#include "common.h"
#include "launch.h"

namespace ds4q {
namespace {

constexpr int MAX_E = ROUTE_MAX_E;

// One wave per token.
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k, const float *__restrict__ x, int D,
                                                   float eps, RouteBufs rb) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *lg = logits + (int64_t)t * E;
  int my_id;
  float my_w;
  wave_topk<MAX_E>(lg, E, k, lane, &my_id, &my_w);
  if (lane < k) {
    rb.ids[t * k + lane] = my_id;
    rb.w[t * k + lane] = my_w;
  }
  if (x) {
    const float *xr = x + (int64_t)t * D;
    float ss = 0.f;
    for (int i = lane; i < D; i += 64) ss = fmaf(xr[i], xr[i], ss);
    ss = group_sum<64>(ss);
    if (lane == 0) rb.inv_rms[t] = 1.0f / sqrtf(ss / (float)D + eps);
  }
}

// One workgroup per expert: histogram of all pair experts (for its offset),
// then a stable, order-preserving compaction of its own pairs.  Workgroup 0
// also writes counts, offsets, the active-expert list and the m-tile list.
__global__ __launch_bounds__(1024) void group_kernel(int T, int E, int k, int tile_m, RouteBufs rb) {
  __shared__ int hist[MAX_E];
  __shared__ int wave_tot[16];
  __shared__ int s_off;
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int P = T * k;
  for (int i = tid; i < E; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += 1024) atomicAdd(&hist[rb.ids[p]], 1);
  __syncthreads();
  if (tid == 0) {
    int off = 0;
    for (int i = 0; i < e; ++i) off += hist[i];
    s_off = off;
    if (e == 0) {
      int acc = 0, na = 0, nt = 0;
      for (int i = 0; i < E; ++i) {
        rb.counts[i] = hist[i];
        rb.offsets[i] = acc;
        if (hist[i] > 0) {
          rb.act_expert[na] = i;
          rb.act_begin[na] = acc;
          ++na;
          if (tile_m > 0)
            for (int m0 = 0; m0 < hist[i]; m0 += tile_m) {
              rb.tiles[2 * nt] = i;
              rb.tiles[2 * nt + 1] = acc + m0;
              ++nt;
            }
        }
        acc += hist[i];
      }
      rb.offsets[E] = acc;
      rb.act_begin[na] = acc;
      *rb.n_active = na;
      if (tile_m > 0) *rb.n_tiles = nt;
    }
  }
  __syncthreads();
  int running = s_off;
  for (int base = 0; base < P; base += 1024) {
    const int p = base + tid;
    const bool mine = p < P && rb.ids[p] == e;
    const uint64_t bal = __ballot(mine);
    const int rank = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wv] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
    for (int i = 0; i < 16; ++i) {
      before += i < wv ? wave_tot[i] : 0;
      total += wave_tot[i];
    }
    if (mine) {
      const int pos = running + before + rank;
      rb.pairs[pos] = p;
      rb.pair_pos[p] = pos;
    }
    running += total;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_topk(const float *logits, int T, int E, int k, const float *x, int D, float eps,
                       const RouteBufs &rb, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, x, D, eps,
                     rb);
  return hipGetLastError();
}

hipError_t launch_group(int T, int E, int k, int tile_m, const RouteBufs &rb, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(group_kernel, dim3(E), dim3(1024), 0, s, T, E, k, tile_m, rb);
  return hipGetLastError();
}

}  // namespace ds4q

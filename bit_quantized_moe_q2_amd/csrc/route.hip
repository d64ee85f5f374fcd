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
  if (E <= 256) {  // four logits per lane, DPP reductions (the one-token path's selection)
    TopK256 tk;
    tk.load(lg, E, lane);
    tk.select(E, k, k, true, lane, &my_id, &my_w);
  } else {
    wave_topk<MAX_E>(lg, E, k, lane, &my_id, &my_w);
  }
  if (lane < k) {
    rb.ids[t * k + lane] = my_id;
    rb.w[t * k + lane] = my_w;
  }
  if (x) {  // D is a multiple of 256 (path sizes)
    const float4 *xr = reinterpret_cast<const float4 *>(x + (int64_t)t * D);
    float ss = 0.f;
    for (int i = lane; i < D / 4; i += 64) {
      const float4 v = xr[i];
      ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss); ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
    }
    ss = group_sum<64>(ss);
    if (lane == 0) rb.inv_rms[t] = 1.0f / sqrtf(ss / (float)D + eps);
  }
}

// Exclusive prefix sum over a 1024-thread workgroup (every thread calls it);
// scratch holds 16 ints.  Returns the sum of v over threads < threadIdx.x and
// sets *total to the sum over all threads.
__device__ __forceinline__ int block_excl_scan(int v, int *scratch, int *total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) scratch[wv] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = scratch[i];
    before += i < wv ? c : 0;
    all += c;
  }
  __syncthreads();  // scratch may be reused by the next scan
  *total = all;
  return before + incl - v;
}

// Pairs per thread and round of the grouping: 24 consecutive pair indices,
// so that a round covers 24,576 pairs (4096 tokens x 6 slots) and each thread
// requests its ids as six 16-byte loads.
constexpr int GROUP_CH = 24;

// The expert ids of pairs p .. p + GROUP_CH - 1 (-1 past the last pair).  p is
// a multiple of 4 and the ids array 16-byte aligned.
__device__ __forceinline__ void load_pair_ids(const int32_t *__restrict__ ids, int p, int P,
                                              int v[GROUP_CH]) {
#pragma unroll
  for (int i = 0; i < GROUP_CH; i += 4) {
    if (p + i + 3 < P) {
      const int4 q = *reinterpret_cast<const int4 *>(ids + p + i);
      v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[i + j] = p + i + j < P ? ids[p + i + j] : -1;
    }
  }
}

// One workgroup per expert: histogram of all pair experts (for its offset),
// then a stable, order-preserving compaction of its own pairs.  Workgroup 0
// also writes counts, offsets, the active-expert list and the m-tile list;
// by_size, workgroup 1 writes the size-ordered copy.  Thread t takes pairs
// base + 24t .. base + 24t + 23 of each round of 24,576; the first round's ids
// stay in registers from the histogram to the compaction.
__global__ __launch_bounds__(1024) void group_kernel(int T, int E, int k, int tile_m, int by_size, RouteBufs rb) {
  __shared__ int hist[MAX_E];
  __shared__ int wave_tot[16];
  __shared__ int s_off;
  const int e = blockIdx.x, tid = threadIdx.x;
  const int P = T * k;
  constexpr int ROUND = 1024 * GROUP_CH;
  const int pt = GROUP_CH * tid;
  int v0[GROUP_CH];
  load_pair_ids(rb.ids, pt, P, v0);
  for (int i = tid; i < E; i += 1024) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < GROUP_CH; ++i)
    if ((unsigned)v0[i] < (unsigned)E) atomicAdd(&hist[v0[i]], 1);
  for (int base = ROUND; base < P; base += ROUND) {
    int v[GROUP_CH];
    load_pair_ids(rb.ids, base + pt, P, v);
#pragma unroll
    for (int i = 0; i < GROUP_CH; ++i)
      if ((unsigned)v[i] < (unsigned)E) atomicAdd(&hist[v[i]], 1);
  }
  __syncthreads();
  // thread i < E takes expert i: its offset, its place among the active
  // experts and its first m-tile, by exclusive scans over the workgroup
  const int c = tid < E ? hist[tid] : 0;
  int n_pairs;
  const int off = block_excl_scan(c, wave_tot, &n_pairs);
  if (tid == e) s_off = off;
  if (e == 0) {
    int n_act, n_til;
    const int apos = block_excl_scan(c > 0 ? 1 : 0, wave_tot, &n_act);
    const int ntile_mine = tile_m > 0 ? (c + tile_m - 1) / tile_m : 0;
    const int tpos = block_excl_scan(ntile_mine, wave_tot, &n_til);
    if (tid < E) {
      rb.counts[tid] = c;
      rb.offsets[tid] = off;
      if (c > 0) {
        rb.act_expert[apos] = tid;
        rb.act_begin[apos] = off;
      }
      for (int j = 0; j < ntile_mine; ++j) {
        rb.tiles[2 * (tpos + j)] = tid;
        rb.tiles[2 * (tpos + j) + 1] = off + j * tile_m;
      }
    }
    if (tid == 0) {
      rb.offsets[E] = n_pairs;
      rb.act_begin[n_act] = n_pairs;
      *rb.n_active = n_act;
      if (tile_m > 0) *rb.n_tiles = n_til;
    }
  }
  // The size-ordered m-tile list, written by workgroup 1 (0 with a single
  // expert) while workgroup 0 writes the others.
  if (by_size && tile_m > 0 && e == (E > 1 ? 1 : 0)) {
    // The same tiles, the full ones first (expert order), then the
    // partial ones by falling count of 16-pair groups, each class in
    // expert order: ranks by ballots per wave, class bases from the
    // per-wave counts.  (Prefill GEMMs deal this list to the XCDs in turn,
    // largest work first.)
    __shared__ int cls_cnt[16][17];
    const int lane = tid & 63, wv = tid >> 6;
    const int full = c / tile_m, rem = c - full * tile_m;
    const int ncls = (tile_m + 15) >> 4;  // <= 16
    const int cls = rem > 0 ? (rem + 15) >> 4 : 0;
    int n_full;
    const int fpos = block_excl_scan(full, wave_tot, &n_full);
    for (int j = 0; j < full; ++j) {
      rb.tiles_sz[2 * (fpos + j)] = tid;
      rb.tiles_sz[2 * (fpos + j) + 1] = off + j * tile_m;
    }
    int rank_w = 0;
    for (int q = 1; q <= ncls; ++q) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(cls == q);
      if (lane == 0) cls_cnt[wv][q] = __builtin_popcountll(m);
      if (cls == q) rank_w = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    }
    __syncthreads();
    if (cls > 0) {
      int pos = n_full;
      for (int q = ncls; q > cls; --q)
        for (int v = 0; v < 16; ++v) pos += cls_cnt[v][q];
      for (int v = 0; v < wv; ++v) pos += cls_cnt[v][cls];
      pos += rank_w;
      rb.tiles_sz[2 * pos] = tid;
      rb.tiles_sz[2 * pos + 1] = off + full * tile_m;
    }
  }
  __syncthreads();
  // stable compaction of the expert's pairs, one scan per round
  int running = s_off;
  for (int base = 0; base < P; base += ROUND) {
    int v[GROUP_CH];
    if (base == 0) {
#pragma unroll
      for (int i = 0; i < GROUP_CH; ++i) v[i] = v0[i];
    } else {
      load_pair_ids(rb.ids, base + pt, P, v);
    }
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < GROUP_CH; ++i) cnt += v[i] == e ? 1 : 0;
    int total;
    int pos = running + block_excl_scan(cnt, wave_tot, &total);
#pragma unroll
    for (int i = 0; i < GROUP_CH; ++i) {
      if (v[i] == e) {
        rb.pairs[pos] = base + pt + i;
        rb.pair_pos[base + pt + i] = pos;
        ++pos;
      }
    }
    running += total;
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

hipError_t launch_group(int T, int E, int k, int tile_m, bool by_size, const RouteBufs &rb, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (by_size && !rb.tiles_sz) return hipErrorInvalidValue;
  hipLaunchKernelGGL(group_kernel, dim3(E), dim3(1024), 0, s, T, E, k, tile_m, by_size ? 1 : 0, rb);
  return hipGetLastError();
}

}  // namespace ds4q

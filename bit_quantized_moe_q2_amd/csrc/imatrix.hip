// Activation statistics of the routed experts ("【#2】ds4.c 해독하기", imatrix
// passage): per expert and input column, the sum of squares of the values the
// expert's gate/up projections read (the MoE input row) and of the values its
// down projection reads (the routed SwiGLU row after the routing weight),
// accumulated into expert-major [n_expert][n_cols] f32 arrays.
//
// The pairs of one expert are visited in segments: the k routing slots (one
// token), the active experts (2..64 tokens on the vector kernels), or the
// m-tiles of at most PREFILL_TILE_M sorted pairs (prefill, and 2..64 tokens on
// the int8 kernels).  A workgroup owns one segment and 1024 columns and sums
// its pairs in order in registers.  A segment that is its expert's only one
// adds straight into the statistics; m-tiles write partial rows that a second
// launch adds up per expert in tile order.  No atomics: the result does not
// depend on scheduling.
#include "common.h"
#include "launch.h"

namespace ds4q {
namespace {

struct Seg {
  int e, b, n;  // expert, first position (slot or sorted position), pair count
};

template <int MODE>
__device__ __forceinline__ bool segment(int i, const RouteBufs &rb, int k, Seg &s) {
  if constexpr (MODE == IMAT_SEG_SLOTS) {
    if (i >= k) return false;
    s.e = rb.ids[i];
    s.b = i;
    s.n = 1;
  } else if constexpr (MODE == IMAT_SEG_ACTIVE) {
    if (i >= *rb.n_active) return false;
    s.e = rb.act_expert[i];
    s.b = rb.act_begin[i];
    s.n = rb.act_begin[i + 1] - s.b;
  } else {
    if (i >= *rb.n_tiles) return false;
    s.e = rb.tiles[2 * i];
    s.b = rb.tiles[2 * i + 1];
    s.n = min(PREFILL_TILE_M, rb.offsets[s.e + 1] - s.b);
  }
  return true;
}

__device__ __forceinline__ float4 load4(const void *rows, bool bf16, int64_t off) {
  if (bf16) {
    const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(rows) + off);
    return make_float4(bf16_to_f32(u.x & 0xFFFFu), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xFFFFu),
                       bf16_to_f32(u.y >> 16));
  }
  return *reinterpret_cast<const float4 *>(static_cast<const float *>(rows) + off);
}

__device__ __forceinline__ float rnd_bf16(float v) { return bf16_to_f32(bf16_rne_bits(v)); }

// grid (column chunks of 1024, segments), 256 threads.  IN: the statistic of
// the MoE input (rows of x by token, scaled by the inverse RMS and rounded to
// bf16 as the path feeds them to the gate/up GEMMs); else of the SwiGLU rows
// times the pair's routing weight.
template <int MODE, bool IN>
__global__ __launch_bounds__(256) void imat_kernel(ImatRows a, RouteBufs rb, int k, int ncols,
                                                   float *__restrict__ dst) {
  __shared__ float red[4];
  __shared__ int row_s[PREFILL_TILE_M];    // the segment's row indices,
  __shared__ float scale_s[PREFILL_TILE_M];  // and the factor of each row
  Seg sg;
  if (!segment<MODE>(blockIdx.y, rb, k, sg)) return;  // uniform over the workgroup
  const int c = 4 * (blockIdx.x * 256 + threadIdx.x);
  float inv_self = 1.0f;
  if (IN && a.norm_self) {
    // one token without a stored inverse RMS: the workgroup computes it
    const float *xr = static_cast<const float *>(a.rows);
    float ss = 0.f;
    for (int i = 4 * threadIdx.x; i < ncols; i += 1024) {
      const float4 v = *reinterpret_cast<const float4 *>(xr + i);
      ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = (red[0] + red[1]) + (red[2] + red[3]);
    inv_self = 1.0f / sqrtf(ss / (float)ncols + a.eps);
  }
  // a segment holds at most PREFILL_TILE_M pairs (an m-tile, or the <= 64
  // pairs of one expert at <= 64 tokens, or one slot)
  if ((int)threadIdx.x < sg.n) {
    const int s = sg.b + threadIdx.x;
    const int p = MODE == IMAT_SEG_SLOTS ? s : rb.pairs[s];
    if constexpr (IN) {
      const int t = p / k;
      row_s[threadIdx.x] = t;
      scale_s[threadIdx.x] = a.inv_rms ? a.inv_rms[t] : inv_self;
    } else {
      row_s[threadIdx.x] = a.by_sorted ? s : p;
      scale_s[threadIdx.x] = rb.w[p];
    }
  }
  __syncthreads();
  if (c >= ncols) return;
  const bool scaled = !IN || a.inv_rms || a.norm_self;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
  for (int j = 0; j < sg.n; ++j) {
    float4 v = load4(a.rows, a.bf16, (int64_t)row_s[j] * ncols + c);
    if (scaled) {
      const float sc = scale_s[j];
      v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
    }
    if (IN && a.round_bf16) {
      v.x = rnd_bf16(v.x); v.y = rnd_bf16(v.y); v.z = rnd_bf16(v.z); v.w = rnd_bf16(v.w);
    }
    acc.x = fmaf(v.x, v.x, acc.x); acc.y = fmaf(v.y, v.y, acc.y);
    acc.z = fmaf(v.z, v.z, acc.z); acc.w = fmaf(v.w, v.w, acc.w);
  }
  if constexpr (MODE == IMAT_SEG_TILES) {
    *reinterpret_cast<float4 *>(dst + (int64_t)blockIdx.y * ncols + c) = acc;
  } else {
    float4 *o = reinterpret_cast<float4 *>(dst + (int64_t)sg.e * ncols + c);
    const float4 old = *o;
    *o = make_float4(old.x + acc.x, old.y + acc.y, old.z + acc.z, old.w + acc.w);
  }
}

// grid (column chunks, tiles): the first tile of each expert's run adds the
// run's partial rows in tile order into the statistics.
__global__ __launch_bounds__(256) void imat_reduce_kernel(const float *__restrict__ partial,
                                                          RouteBufs rb, int ncols,
                                                          float *__restrict__ dst) {
  const int i = blockIdx.y;
  const int nt = *rb.n_tiles;
  if (i >= nt) return;
  const int e = rb.tiles[2 * i];
  if (i > 0 && rb.tiles[2 * (i - 1)] == e) return;
  const int c = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (c >= ncols) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = i; j < nt && rb.tiles[2 * j] == e; ++j) {
    const float4 v = *reinterpret_cast<const float4 *>(partial + (int64_t)j * ncols + c);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  float4 *o = reinterpret_cast<float4 *>(dst + (int64_t)e * ncols + c);
  const float4 old = *o;
  *o = make_float4(old.x + acc.x, old.y + acc.y, old.z + acc.z, old.w + acc.w);
}

template <bool IN>
hipError_t launch_one(int mode, int max_seg, const ImatRows &a, const RouteBufs &rb, int k,
                      int ncols, float *stat, float *partial, hipStream_t s) {
  const dim3 grid((unsigned)((ncols + 1023) / 1024), (unsigned)max_seg);
  if (mode == IMAT_SEG_SLOTS) {
    hipLaunchKernelGGL((imat_kernel<IMAT_SEG_SLOTS, IN>), grid, dim3(256), 0, s, a, rb, k, ncols, stat);
  } else if (mode == IMAT_SEG_ACTIVE) {
    hipLaunchKernelGGL((imat_kernel<IMAT_SEG_ACTIVE, IN>), grid, dim3(256), 0, s, a, rb, k, ncols, stat);
  } else {
    hipLaunchKernelGGL((imat_kernel<IMAT_SEG_TILES, IN>), grid, dim3(256), 0, s, a, rb, k, ncols,
                       partial);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(imat_reduce_kernel, grid, dim3(256), 0, s, partial, rb, ncols, stat);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_imatrix(const MoeDims &m, const RouteBufs &rb, int seg_mode, int max_seg,
                          const ImatRows &in, float *stat_in, const ImatRows &h, float *stat_down,
                          float *partial, hipStream_t s) {
  if (max_seg <= 0) return hipSuccess;
  if (stat_in) {
    const hipError_t err = launch_one<true>(seg_mode, max_seg, in, rb, m.k, m.D, stat_in, partial, s);
    if (err != hipSuccess) return err;
  }
  if (stat_down) return launch_one<false>(seg_mode, max_seg, h, rb, m.k, m.F, stat_down, partial, s);
  return hipSuccess;
}

}  // namespace ds4q

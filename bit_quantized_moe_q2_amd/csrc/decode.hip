// The single quantised matvec on fp32 vector arithmetic, and the
// routing-weighted combine of the experts' outputs (with the steering
// epilogue) shared by the decode and prefill paths.
//
// Work layout.  A row of C = 64*L values is split into L "chunks" of 64 values,
// one per lane; L consecutive lanes of a wave64 share a row, so a wave covers
// 64/L rows per row slot.  A Q2_K chunk is one quarter of a 256-value block
// (16 code bytes + its 4 scale bytes + d/dmin), a Q4_1 chunk is two 32-value
// blocks (40 contiguous bytes).  Each lane keeps the 64 activations its chunk
// multiplies in registers for the whole row loop and streams only weights.
//
// Arithmetic per chunk (Q2_K): sum_k d*sc_k*(sum_i q_i x_i) - dmin*mn_k*(sum_i x_i)
// over its four 16-value sub-blocks, with sum_i x_i precomputed once per token
// (the min term hoisted out of the row loop); Q4_1: d*(sum q x) + m*(sum x).
// Partial sums are combined with an xor-butterfly over the row's L lanes.
//
// Combine ("【#2】ds4.c 해독하기": the routing weight multiplies the routed
// SwiGLU row; the down projection is linear, so it is applied to each
// expert's output instead): y_t (+)= sum_j p_j * o_j.
#include "common.h"
#include "launch.h"

namespace ds4q {
namespace {

constexpr int WAVES = 4;

// Block fields are 4-byte aligned only: wide loads of 4-byte-aligned data.
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(4)));

// ---------------------------------------------------------------- x slices

template <int TYPE>
struct XSlice {
  float v[64];
  float s[TYPE == TYPE_Q2_K ? 4 : 2];

  // Activations multiplied by chunk c of a row, scaled by `scale`.
  __device__ __forceinline__ void load(const float *__restrict__ X, int c, float scale) {
    if constexpr (TYPE == TYPE_Q2_K) {
      // quarter g = c&3 of block c>>2: values 128h + 32k + 16p + l'
      const int b = c >> 2, g = c & 3, h = g >> 1, p = g & 1;
      const float *base = X + 256 * b + 128 * h + 16 * p;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 t = *reinterpret_cast<const float4 *>(base + 32 * k + 4 * j);
          v[16 * k + 4 * j + 0] = t.x * scale;
          v[16 * k + 4 * j + 1] = t.y * scale;
          v[16 * k + 4 * j + 2] = t.z * scale;
          v[16 * k + 4 * j + 3] = t.w * scale;
        }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a += v[16 * k + i];
        s[k] = a;
      }
    } else {
      const float *base = X + 64 * c;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float4 t = *reinterpret_cast<const float4 *>(base + 4 * j);
        v[4 * j + 0] = t.x * scale;
        v[4 * j + 1] = t.y * scale;
        v[4 * j + 2] = t.z * scale;
        v[4 * j + 3] = t.w * scale;
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) a += v[32 * b + i];
        s[b] = a;
      }
    }
  }
};

// ---------------------------------------------------------------- weight chunks

template <int TYPE>
struct Chunk;

template <>
struct Chunk<TYPE_Q2_K> {
  uint32_t q[4], s0, s1, dd;
  int p;
  // row: first byte of the row; c: chunk index within the row
  __device__ __forceinline__ void load(const uint8_t *__restrict__ row, int c) {
    const uint8_t *blk = row + (c >> 2) * BB_Q2K;
    const int g = c & 3, h = g >> 1;
    p = g & 1;
    const u32x4a qv = *reinterpret_cast<const u32x4a *>(blk + 16 + 16 * g);
    q[0] = qv.x; q[1] = qv.y; q[2] = qv.z; q[3] = qv.w;
    const u32x2a sv = *reinterpret_cast<const u32x2a *>(blk + 8 * h);
    s0 = sv.x;
    s1 = sv.y;
    dd = ld32(blk + 80);
  }
  __device__ __forceinline__ float dot(const XSlice<TYPE_Q2_K> &x) const {
    float acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t t = (q[j] >> (2 * k)) & 0x03030303u;
        a = fmaf(ub0(t), x.v[16 * k + 4 * j + 0], a);
        a = fmaf(ub1(t), x.v[16 * k + 4 * j + 1], a);
        a = fmaf(ub2(t), x.v[16 * k + 4 * j + 2], a);
        a = fmaf(ub3(t), x.v[16 * k + 4 * j + 3], a);
      }
      acc[k] = a;
    }
    // sub-block 8h + 2k + p: bytes p, 2+p of s0 (k = 0, 1), of s1 (k = 2, 3)
    const uint32_t a0 = s0 >> (8 * p), a1 = s1 >> (8 * p);
    float sc = (float)(a0 & 15u) * acc[0];
    sc = fmaf((float)((a0 >> 16) & 15u), acc[1], sc);
    sc = fmaf((float)(a1 & 15u), acc[2], sc);
    sc = fmaf((float)((a1 >> 16) & 15u), acc[3], sc);
    float mn = (float)((a0 >> 4) & 15u) * x.s[0];
    mn = fmaf((float)((a0 >> 20) & 15u), x.s[1], mn);
    mn = fmaf((float)((a1 >> 4) & 15u), x.s[2], mn);
    mn = fmaf((float)((a1 >> 20) & 15u), x.s[3], mn);
    return f16lo(dd) * sc - f16hi(dd) * mn;
  }
};

template <>
struct Chunk<TYPE_Q4_1> {
  uint32_t w[10];
  __device__ __forceinline__ void load(const uint8_t *__restrict__ row, int c) {
    // the chunk's 40 bytes (two blocks, 8-byte aligned) in three loads
    const uint8_t *p = row + c * (2 * BB_Q41);
    const u32x4a a = *reinterpret_cast<const u32x4a *>(p);
    const u32x4a b = *reinterpret_cast<const u32x4a *>(p + 16);
    const u32x2a e = *reinterpret_cast<const u32x2a *>(p + 32);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    w[8] = e.x; w[9] = e.y;
  }
  __device__ __forceinline__ float dot(const XSlice<TYPE_Q4_1> &x) const {
    float r = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t qw = w[5 * b + 1 + j];
        const uint32_t lo = qw & 0x0F0F0F0Fu, hi = (qw >> 4) & 0x0F0F0F0Fu;
        const float *xl = x.v + 32 * b + 4 * j, *xh = x.v + 32 * b + 16 + 4 * j;
        a = fmaf(ub0(lo), xl[0], a); a = fmaf(ub1(lo), xl[1], a);
        a = fmaf(ub2(lo), xl[2], a); a = fmaf(ub3(lo), xl[3], a);
        a = fmaf(ub0(hi), xh[0], a); a = fmaf(ub1(hi), xh[1], a);
        a = fmaf(ub2(hi), xh[2], a); a = fmaf(ub3(hi), xh[3], a);
      }
      r = fmaf(f16lo(w[5 * b]), a, r);
      r = fmaf(f16hi(w[5 * b]), x.s[b], r);
    }
    return r;
  }
};

// ---------------------------------------------------------------- matvec

// y[t][r] = sum_c W[r][c] x[t][c].  L lanes per row, RS row slots per wave.
template <int TYPE, int L, int RS>
__global__ __launch_bounds__(256) void matvec_kernel(const uint8_t *__restrict__ W, int64_t rows,
                                                     const float *__restrict__ x, int n_tok,
                                                     float *__restrict__ y) {
  constexpr int RPW = 64 / L;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane % L, rs = lane / L;
  const int64_t rbytes = row_bytes(TYPE, 64 * L);
  const int64_t row0 = ((int64_t)blockIdx.x * WAVES + wv) * RS * RPW;
  for (int t = 0; t < n_tok; ++t) {
    XSlice<TYPE> xs;
    xs.load(x + (int64_t)t * 64 * L, c, 1.0f);
    Chunk<TYPE> ch[RS];
#pragma unroll
    for (int i = 0; i < RS; ++i) {
      const int64_t r = row0 + i * RPW + rs;
      if (r < rows) ch[i].load(W + r * rbytes, c);
    }
#pragma unroll
    for (int i = 0; i < RS; ++i) {
      const int64_t r = row0 + i * RPW + rs;
      float v = r < rows ? ch[i].dot(xs) : 0.f;
      v = group_sum<L>(v);
      if (c == 0 && r < rows) y[(int64_t)t * rows + r] = v;
    }
  }
}

// ---------------------------------------------------------------- combine

// Four consecutive values of a row of o: fp32, or bf16 (prefill).
__device__ __forceinline__ float4 load4(const float *o, int64_t off) {
  return *reinterpret_cast<const float4 *>(o + off);
}
__device__ __forceinline__ float4 load4(const uint16_t *o, int64_t off) {
  const uint2 u = *reinterpret_cast<const uint2 *>(o + off);
  return make_float4(bf16_to_f32(u.x & 0xFFFFu), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xFFFFu),
                     bf16_to_f32(u.y >> 16));
}
// V consecutive values from offset off (a multiple of V): f32 rows four at a
// time, bf16 rows four or eight (one 16-byte request).
template <int V>
__device__ __forceinline__ void loadv(const float *o, int64_t off, float v[V]) {
  static_assert(V == 4, "f32 rows: four values per request");
  const float4 f = load4(o, off);
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}
template <int V>
__device__ __forceinline__ void loadv(const uint16_t *o, int64_t off, float v[V]) {
  if constexpr (V == 4) {
    const float4 f = load4(o, off);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    static_assert(V == 8, "bf16 rows: four or eight values per request");
    const uint4 u = *reinterpret_cast<const uint4 *>(o + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
}

// y[t] (+)= sum_j w[t][j] * o[row(t, j)] in slot order; each thread takes V
// consecutive values of one token row (D a multiple of V).
template <typename OT, bool BY_POS, int KC, int V>
__global__ __launch_bounds__(256) void combine_kernel(const OT *__restrict__ o, RouteBufs rb,
                                                      int T, int k_rt, int D,
                                                      float *__restrict__ y, int accumulate) {
  const int64_t iv = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int DV = D / V;
  if (iv >= (int64_t)T * DV) return;
  const int t = (int)(iv / DV), c = (int)(iv % DV);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  float4 *yp = reinterpret_cast<float4 *>(y + (int64_t)t * D + V * c);
  float old[V];
  if constexpr (KC > 0) {
    // the slot count known at compile time: straight-line code requests every
    // slot's position, then every slot's row (and the old y row), before the
    // sum in slot order
    if (accumulate) {
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        const float4 f = yp[q];
        old[4 * q] = f.x; old[4 * q + 1] = f.y; old[4 * q + 2] = f.z; old[4 * q + 3] = f.w;
      }
    }
    int64_t row[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) row[j] = BY_POS ? rb.pair_pos[t * KC + j] : t * KC + j;
    float v[KC][V];
    float w[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      loadv<V>(o, row[j] * D + V * c, v[j]);
      w[j] = rb.w[t * KC + j];
    }
#pragma unroll
    for (int j = 0; j < KC; ++j)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(w[j], v[j][i], acc[i]);
  } else {
    for (int j = 0; j < k_rt; ++j) {
      const int p = t * k_rt + j;
      const int64_t row = BY_POS ? rb.pair_pos[p] : p;
      float v[V];
      loadv<V>(o, row * D + V * c, v);
      const float w = rb.w[p];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(w, v[i], acc[i]);
    }
    if (accumulate) {
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        const float4 f = yp[q];
        old[4 * q] = f.x; old[4 * q + 1] = f.y; old[4 * q + 2] = f.z; old[4 * q + 3] = f.w;
      }
    }
  }
  if (accumulate) {
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += old[i];
  }
#pragma unroll
  for (int q = 0; q < V / 4; ++q) yp[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
}

// Combine with directional steering: one workgroup per token row (D <= 4096,
// four float4 per thread), the row's weighted sum kept in registers while its
// dot product with the direction is reduced, then y (+)= v - scale*dir*(dir.v).
// KC > 0 (the slot count, with D = 4096 so that every thread owns all four
// float4): straight-line code requests every slot's position, then all rows,
// before any arithmetic; the sums keep the same order.
template <typename OT, bool BY_POS, int KC>
__global__ __launch_bounds__(256) void combine_steer_kernel(const OT *__restrict__ o, RouteBufs rb,
                                                            int k, int D,
                                                            const float *__restrict__ dir, float scale,
                                                            float *__restrict__ y, int accumulate) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  float4 v[4];
  float p = 0.f;
  if constexpr (KC > 0) {
    int64_t row[KC];
    float w[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      row[j] = BY_POS ? rb.pair_pos[t * KC + j] : t * KC + j;
      w[j] = rb.w[t * KC + j];
    }
    float4 a[4][KC];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < KC; ++j) a[c][j] = load4(o, row[j] * D + 4 * (threadIdx.x + 256 * c));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[c] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        v[c].x = fmaf(w[j], a[c][j].x, v[c].x); v[c].y = fmaf(w[j], a[c][j].y, v[c].y);
        v[c].z = fmaf(w[j], a[c][j].z, v[c].z); v[c].w = fmaf(w[j], a[c][j].w, v[c].w);
      }
      const float4 d = *reinterpret_cast<const float4 *>(dir + 4 * (threadIdx.x + 256 * c));
      p = fmaf(d.x, v[c].x, p); p = fmaf(d.y, v[c].y, p);
      p = fmaf(d.z, v[c].z, p); p = fmaf(d.w, v[c].w, p);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = 4 * (threadIdx.x + 256 * c);
      v[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < D) {
        for (int j = 0; j < k; ++j) {
          const int pp = t * k + j;
          const int64_t row = BY_POS ? rb.pair_pos[pp] : pp;
          const float4 a = load4(o, row * D + i);
          const float w = rb.w[pp];
          v[c].x = fmaf(w, a.x, v[c].x); v[c].y = fmaf(w, a.y, v[c].y);
          v[c].z = fmaf(w, a.z, v[c].z); v[c].w = fmaf(w, a.w, v[c].w);
        }
        const float4 d = *reinterpret_cast<const float4 *>(dir + i);
        p = fmaf(d.x, v[c].x, p); p = fmaf(d.y, v[c].y, p);
        p = fmaf(d.z, v[c].z, p); p = fmaf(d.w, v[c].w, p);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) p += __shfl_xor(p, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = p;
  __syncthreads();
  const float sd = -scale * ((red[0] + red[1]) + (red[2] + red[3]));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = 4 * (threadIdx.x + 256 * c);
    if (i < D) {
      const float4 d = *reinterpret_cast<const float4 *>(dir + i);
      float4 r = make_float4(fmaf(sd, d.x, v[c].x), fmaf(sd, d.y, v[c].y), fmaf(sd, d.z, v[c].z),
                             fmaf(sd, d.w, v[c].w));
      float4 *yp = reinterpret_cast<float4 *>(y + (int64_t)t * D + i);
      if (accumulate) {
        const float4 old = *yp;
        r.x += old.x; r.y += old.y; r.z += old.z; r.w += old.w;
      }
      *yp = r;
    }
  }
}

// ---------------------------------------------------------------- dispatch

#define DS4Q_DISPATCH_L(L_VAL, ...)                     \
  switch (L_VAL) {                                      \
    case 4: { constexpr int LL = 4; __VA_ARGS__; break; }   \
    case 8: { constexpr int LL = 8; __VA_ARGS__; break; }   \
    case 16: { constexpr int LL = 16; __VA_ARGS__; break; } \
    case 32: { constexpr int LL = 32; __VA_ARGS__; break; } \
    case 64: { constexpr int LL = 64; __VA_ARGS__; break; } \
    default: return hipErrorInvalidValue;               \
  }

// Row slots per wave: enough rows in flight per wave, while keeping >= 8
// waves per CU on the largest grids.
template <int L>
constexpr int row_slots() { return L == 64 ? 2 : 1; }

}  // namespace

hipError_t launch_matvec(int w_type, const void *w, int64_t rows, int64_t cols, const float *x,
                         int n_tok, float *y, hipStream_t s) {
  if (rows == 0 || n_tok == 0) return hipSuccess;
  const uint8_t *W = static_cast<const uint8_t *>(w);
  const int L = (int)(cols / 64);
  DS4Q_DISPATCH_L(L, {
    constexpr int RS = 1;
    const int64_t per_wg = (int64_t)WAVES * RS * (64 / LL);
    const unsigned grid = (unsigned)((rows + per_wg - 1) / per_wg);
    if (w_type == TYPE_Q2_K)
      hipLaunchKernelGGL((matvec_kernel<TYPE_Q2_K, LL, RS>), dim3(grid), dim3(256), 0, s, W, rows, x, n_tok, y);
    else
      hipLaunchKernelGGL((matvec_kernel<TYPE_Q4_1, LL, RS>), dim3(grid), dim3(256), 0, s, W, rows, x, n_tok, y);
  });
  return hipGetLastError();
}

namespace {
template <typename OT>
hipError_t combine_any(const OT *o, const RouteBufs &rb, int T, int k, int D, bool by_pos, float *y,
                       bool accumulate, const SteerArgs &st, hipStream_t s) {
  const int64_t n4 = (int64_t)T * (D / 4);
  if (n4 == 0) return hipSuccess;
  if (st.dir) {
    const int kc = D == 4096 ? k : 0;
#define DS4Q_STEER(KC)                                                                             \
  do {                                                                                             \
    if (by_pos)                                                                                    \
      hipLaunchKernelGGL((combine_steer_kernel<OT, true, KC>), dim3((unsigned)T), dim3(256), 0, s, o, rb, k, \
                         D, st.dir, st.scale, y, accumulate ? 1 : 0);                              \
    else                                                                                           \
      hipLaunchKernelGGL((combine_steer_kernel<OT, false, KC>), dim3((unsigned)T), dim3(256), 0, s, o, rb, k, \
                         D, st.dir, st.scale, y, accumulate ? 1 : 0);                              \
  } while (0)
    switch (kc) {
      case 6: DS4Q_STEER(6); break;
      case 8: DS4Q_STEER(8); break;
      default: DS4Q_STEER(0); break;
    }
#undef DS4Q_STEER
    return hipGetLastError();
  }
  // bf16 rows: eight values per thread (one 16-byte request per slot)
  constexpr int V = sizeof(OT) == 2 ? 8 : 4;
  if (D % V) return hipErrorInvalidValue;
  const int64_t nv = (int64_t)T * (D / V);
  const dim3 grid((unsigned)((nv + 255) / 256));
  const int acc = accumulate ? 1 : 0;
#define DS4Q_COMBINE(KC)                                                                           \
  do {                                                                                             \
    if (by_pos)                                                                                    \
      hipLaunchKernelGGL((combine_kernel<OT, true, KC, V>), grid, dim3(256), 0, s, o, rb, T, k, D, y, acc); \
    else                                                                                           \
      hipLaunchKernelGGL((combine_kernel<OT, false, KC, V>), grid, dim3(256), 0, s, o, rb, T, k, D, y, acc); \
  } while (0)
  switch (k) {
    case 6: DS4Q_COMBINE(6); break;
    case 8: DS4Q_COMBINE(8); break;
    default: DS4Q_COMBINE(0); break;
  }
#undef DS4Q_COMBINE
  return hipGetLastError();
}
}  // namespace

hipError_t launch_combine(const float *o, const RouteBufs &rb, int T, int k, int D, bool by_pos,
                          float *y, bool accumulate, const SteerArgs &st, hipStream_t s) {
  return combine_any(o, rb, T, k, D, by_pos, y, accumulate, st, s);
}

hipError_t launch_combine(const uint16_t *o, const RouteBufs &rb, int T, int k, int D, bool by_pos,
                          float *y, bool accumulate, const SteerArgs &st, hipStream_t s) {
  return combine_any(o, rb, T, k, D, by_pos, y, accumulate, st, s);
}

}  // namespace ds4q

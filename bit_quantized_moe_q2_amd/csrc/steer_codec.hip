// Two small HBM-bound operations around the MoE layer:
//
// Directional steering ("【#8】ds4.c 해독하기", directional-steering section):
// per row, out (+)= y - scale * dir * (dir . y), the layer's direction
// projected out of its FFN output.  One workgroup per row: a block reduction
// of dir . y in fp32, then one fma per value.  The one-token decode path runs
// this on the row the down kernel staged.
//
// Activation wire formats ("【#6】ds4.c 분석하기", distributed-transport
// passage): the activations between pipeline stages travel as 32-bit floats
// or packed to 16 bits (f16) or 8 bits (E4M3) and are decoded back to float.
// f16 is IEEE binary16 (round to nearest even, overflow to infinity, NaN to
// the quiet NaN sign|0x7E00); E4M3 is the OCP 8-bit E4M3 encoding (bias 7,
// subnormals, largest finite 448, NaN sign|0x7F, no infinities), rounded to
// nearest even, with magnitudes beyond 448 (and infinities) saturated.
#include "common.h"
#include "launch.h"

namespace ds4q {
namespace {

// ---------------------------------------------------------------- steering

// One workgroup per row.  Up to 4096 values the row stays in registers (CH
// float4 per thread, all loads issued before the first use): one memory round
// trip, the block reduction, then the writes.  Longer rows loop twice.
template <int CH>
__global__ __launch_bounds__(256) void steer_kernel(const float *__restrict__ dir, float scale,
                                                    const float *y, int n, float *out, int accumulate) {
  const int64_t row = blockIdx.x;
  const float *yr = y + row * n;
  float *orow = out + row * n;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  __shared__ float red[4];
  float p = 0.f;
  float4 a[CH > 0 ? CH : 1], b[CH > 0 ? CH : 1];
  if constexpr (CH > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = 4 * (t + 256 * c);
      if (i < n) {
        a[c] = *reinterpret_cast<const float4 *>(dir + i);
        b[c] = *reinterpret_cast<const float4 *>(yr + i);
      } else {
        a[c] = b[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      p = fmaf(a[c].x, b[c].x, p);
      p = fmaf(a[c].y, b[c].y, p);
      p = fmaf(a[c].z, b[c].z, p);
      p = fmaf(a[c].w, b[c].w, p);
    }
  } else {
    for (int i = 4 * t; i < n; i += 1024) {
      const float4 u = *reinterpret_cast<const float4 *>(dir + i);
      const float4 v = *reinterpret_cast<const float4 *>(yr + i);
      p = fmaf(u.x, v.x, p);
      p = fmaf(u.y, v.y, p);
      p = fmaf(u.z, v.z, p);
      p = fmaf(u.w, v.w, p);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) p += __shfl_xor(p, o, 64);
  if (lane == 0) red[w] = p;
  __syncthreads();  // also orders every read of the row before any write (out may be y)
  const float sd = -scale * ((red[0] + red[1]) + (red[2] + red[3]));
  auto emit = [&](int i, float4 u, float4 v) {
    float4 r = make_float4(fmaf(sd, u.x, v.x), fmaf(sd, u.y, v.y), fmaf(sd, u.z, v.z), fmaf(sd, u.w, v.w));
    if (accumulate) {
      const float4 o = *reinterpret_cast<const float4 *>(orow + i);
      r = make_float4(o.x + r.x, o.y + r.y, o.z + r.z, o.w + r.w);
    }
    *reinterpret_cast<float4 *>(orow + i) = r;
  };
  if constexpr (CH > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = 4 * (t + 256 * c);
      if (i < n) emit(i, a[c], b[c]);
    }
  } else {
    for (int i = 4 * t; i < n; i += 1024)
      emit(i, *reinterpret_cast<const float4 *>(dir + i), *reinterpret_cast<const float4 *>(yr + i));
  }
}

// ---------------------------------------------------------------- codec

__device__ __forceinline__ uint32_t enc_f16(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7E00u;
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32: round to nearest even
}

__device__ __forceinline__ uint32_t enc_e4m3(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a >= 0x43E80000u) return sign | 0x7Eu;  // >= 464 (and inf): 448, the midpoint's even side, or saturated
  if (a < 0x3C800000u) {                      // below 2^-6: the subnormal grid m * 2^-9, m = 0..8
    const float m = __builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);  // exact scaling, RNE
    return sign | (uint32_t)m;                // m = 8 is the code of 2^-6
  }
  // normal: keep 3 mantissa bits, round to nearest even (a carry moves the
  // exponent); the f32 biased exponent E maps to the E4M3 field E - 120
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));
}

__device__ __forceinline__ float dec_f16(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float dec_e4m3(uint32_t b) {
  const uint32_t s = (b & 0x80u) << 24, e = (b >> 3) & 15u, m = b & 7u;
  if (e == 15u && m == 7u) return __builtin_bit_cast(float, s | 0x7FC00000u);
  if (e == 0u) return __builtin_bit_cast(float, s | __builtin_bit_cast(uint32_t, (float)m * (1.0f / 512.0f)));
  return __builtin_bit_cast(float, s | ((e + 120u) << 23) | (m << 20));
}

// Each thread converts G groups of 4 consecutive values; group q of thread
// t in a workgroup lies at (workgroup base) + 1024q + 4t, so every load and
// store instruction of a wave covers one contiguous span.  Groups past a
// ragged end fall back to single values.
template <int G>
__device__ __forceinline__ int64_t group_base(int q) {
  return ((int64_t)blockIdx.x * G + q) * 1024 + 4 * threadIdx.x;
}

__global__ __launch_bounds__(256) void encode16_kernel(const float *__restrict__ src, int64_t n,
                                                       uint16_t *__restrict__ dst) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t i = group_base<2>(q);
    if (i + 4 <= n) {
      const float4 a = *reinterpret_cast<const float4 *>(src + i);
      *reinterpret_cast<uint2 *>(dst + i) =
          make_uint2(enc_f16(a.x) | (enc_f16(a.y) << 16), enc_f16(a.z) | (enc_f16(a.w) << 16));
    } else {
      for (int64_t j = i; j < n && j < i + 4; ++j) dst[j] = (uint16_t)enc_f16(src[j]);
    }
  }
}

__global__ __launch_bounds__(256) void encode8_kernel(const float *__restrict__ src, int64_t n,
                                                      uint8_t *__restrict__ dst) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = group_base<4>(q);
    if (i + 4 <= n) {
      const float4 a = *reinterpret_cast<const float4 *>(src + i);
      *reinterpret_cast<uint32_t *>(dst + i) =
          enc_e4m3(a.x) | (enc_e4m3(a.y) << 8) | (enc_e4m3(a.z) << 16) | (enc_e4m3(a.w) << 24);
    } else {
      for (int64_t j = i; j < n && j < i + 4; ++j) dst[j] = (uint8_t)enc_e4m3(src[j]);
    }
  }
}

__global__ __launch_bounds__(256) void decode16_kernel(const uint16_t *__restrict__ src, int64_t n,
                                                       float *__restrict__ dst) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t i = group_base<2>(q);
    if (i + 4 <= n) {
      const uint2 h = *reinterpret_cast<const uint2 *>(src + i);
      *reinterpret_cast<float4 *>(dst + i) =
          make_float4(dec_f16(h.x & 0xFFFFu), dec_f16(h.x >> 16), dec_f16(h.y & 0xFFFFu), dec_f16(h.y >> 16));
    } else {
      for (int64_t j = i; j < n && j < i + 4; ++j) dst[j] = dec_f16(src[j]);
    }
  }
}

__global__ __launch_bounds__(256) void decode8_kernel(const uint8_t *__restrict__ src, int64_t n,
                                                      float *__restrict__ dst) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = group_base<4>(q);
    if (i + 4 <= n) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(src + i);
      *reinterpret_cast<float4 *>(dst + i) =
          make_float4(dec_e4m3(w & 0xFFu), dec_e4m3((w >> 8) & 0xFFu), dec_e4m3((w >> 16) & 0xFFu),
                      dec_e4m3(w >> 24));
    } else {
      for (int64_t j = i; j < n && j < i + 4; ++j) dst[j] = dec_e4m3(src[j]);
    }
  }
}

// workgroups of 256 threads x G groups of 4 values
unsigned blocks_of(int64_t n, int groups) {
  return (unsigned)((n + 1024LL * groups - 1) / (1024LL * groups));
}

}  // namespace

hipError_t launch_steer(const float *dir, float scale, const float *y, int64_t n_rows, int n,
                        float *out, bool accumulate, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)n_rows);
  const int acc = accumulate ? 1 : 0;
  if (n <= 1024)
    hipLaunchKernelGGL(steer_kernel<1>, grid, dim3(256), 0, s, dir, scale, y, n, out, acc);
  else if (n <= 2048)
    hipLaunchKernelGGL(steer_kernel<2>, grid, dim3(256), 0, s, dir, scale, y, n, out, acc);
  else if (n <= 4096)
    hipLaunchKernelGGL(steer_kernel<4>, grid, dim3(256), 0, s, dir, scale, y, n, out, acc);
  else
    hipLaunchKernelGGL(steer_kernel<0>, grid, dim3(256), 0, s, dir, scale, y, n, out, acc);
  return hipGetLastError();
}

hipError_t launch_act_encode(const float *src, int64_t n, int bits, void *dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (bits == 32) return hipMemcpyAsync(dst, src, (size_t)n * 4, hipMemcpyDeviceToDevice, s);
  if (bits == 16)
    hipLaunchKernelGGL(encode16_kernel, dim3(blocks_of(n, 2)), dim3(256), 0, s, src, n,
                       static_cast<uint16_t *>(dst));
  else
    hipLaunchKernelGGL(encode8_kernel, dim3(blocks_of(n, 4)), dim3(256), 0, s, src, n,
                       static_cast<uint8_t *>(dst));
  return hipGetLastError();
}

hipError_t launch_act_decode(const void *src, int64_t n, int bits, float *dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (bits == 32) return hipMemcpyAsync(dst, src, (size_t)n * 4, hipMemcpyDeviceToDevice, s);
  if (bits == 16)
    hipLaunchKernelGGL(decode16_kernel, dim3(blocks_of(n, 2)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(src), n, dst);
  else
    hipLaunchKernelGGL(decode8_kernel, dim3(blocks_of(n, 4)), dim3(256), 0, s,
                       static_cast<const uint8_t *>(src), n, dst);
  return hipGetLastError();
}

}  // namespace ds4q

// Standalone block dequantisation: Q2_K / Q4_1 -> f32 or bf16.
//
// Each thread produces 4 consecutive output values with one dword of codes,
// so a wave writes one contiguous 1 KB (f32) / 512 B (bf16) run: the kernel is
// bound by HBM writes.  Value arithmetic: d*scale (exact in fp32: 11 x 4
// bits) times the code (exact) plus -(dmin*min) (exact) in one fma, so the
// fp32 result is rounded exactly once; bf16 is its round-to-nearest-even.
#include "common.h"
#include "launch.h"

namespace ds4q {
namespace {

template <bool BF16>
__device__ __forceinline__ void store4(void *dst, int64_t idx, float a, float b, float c, float d) {
  if constexpr (BF16) {
    uint2 v;
    v.x = bf16_rne_bits(a) | (bf16_rne_bits(b) << 16);
    v.y = bf16_rne_bits(c) | (bf16_rne_bits(d) << 16);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(dst) + idx) = v;
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(dst) + idx) = make_float4(a, b, c, d);
  }
}

// Q2_K: 64 threads per block; thread i covers values 4i..4i+3, which share
// one sub-block (i>>2) and one code dword (bit pair (i>>3)&3).
template <bool BF16>
__global__ __launch_bounds__(256) void dequant_q2k_kernel(const uint8_t *__restrict__ src,
                                                          void *__restrict__ dst, int64_t n_thr) {
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < n_thr;
       g += (int64_t)gridDim.x * 256) {
    const int64_t b = g >> 6;
    const int i = (int)(g & 63);
    const uint8_t *blk = src + b * BB_Q2K;
    const int e0 = 4 * i;
    const int h = e0 >> 7, k = (e0 >> 5) & 3, l0 = e0 & 31;
    const uint32_t qw = (ld32(blk + 16 + 32 * h + l0) >> (2 * k)) & 0x03030303u;
    const uint32_t sb = blk[i >> 2];
    const uint32_t dd = ld32(blk + 80);
    const float ds = f16lo(dd) * (float)(sb & 15u);
    const float dm = f16hi(dd) * (float)(sb >> 4);
    store4<BF16>(dst, b * 256 + e0, fmaf(ds, ub0(qw), -dm), fmaf(ds, ub1(qw), -dm),
                 fmaf(ds, ub2(qw), -dm), fmaf(ds, ub3(qw), -dm));
  }
}

// Q4_1: 8 threads per block; thread i covers values 4i..4i+3: low nibbles of
// qs[4i..4i+3] for i < 4, high nibbles of qs[4(i-4)..] for i >= 4.
template <bool BF16>
__global__ __launch_bounds__(256) void dequant_q41_kernel(const uint8_t *__restrict__ src,
                                                          void *__restrict__ dst, int64_t n_thr) {
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < n_thr;
       g += (int64_t)gridDim.x * 256) {
    const int64_t b = g >> 3;
    const int i = (int)(g & 7);
    const uint8_t *blk = src + b * BB_Q41;
    const uint32_t qw = (ld32(blk + 4 + 4 * (i & 3)) >> (4 * (i >> 2))) & 0x0F0F0F0Fu;
    const uint32_t dm = ld32(blk);
    const float d = f16lo(dm), m = f16hi(dm);
    store4<BF16>(dst, b * 32 + 4 * i, fmaf(d, ub0(qw), m), fmaf(d, ub1(qw), m),
                 fmaf(d, ub2(qw), m), fmaf(d, ub3(qw), m));
  }
}

}  // namespace

hipError_t launch_dequant(int src_type, const void *src, int64_t rows, int64_t cols, bool bf16,
                          void *dst, hipStream_t s) {
  const int64_t n_thr = rows * cols / 4;
  if (n_thr <= 0) return hipSuccess;
  const int64_t want = (n_thr + 255) / 256;
  const unsigned grid = (unsigned)(want < (1 << 20) ? want : (1 << 20));
  const uint8_t *p = static_cast<const uint8_t *>(src);
  if (src_type == TYPE_Q2_K) {
    if (bf16) hipLaunchKernelGGL(dequant_q2k_kernel<true>, dim3(grid), dim3(256), 0, s, p, dst, n_thr);
    else hipLaunchKernelGGL(dequant_q2k_kernel<false>, dim3(grid), dim3(256), 0, s, p, dst, n_thr);
  } else {
    if (bf16) hipLaunchKernelGGL(dequant_q41_kernel<true>, dim3(grid), dim3(256), 0, s, p, dst, n_thr);
    else hipLaunchKernelGGL(dequant_q41_kernel<false>, dim3(grid), dim3(256), 0, s, p, dst, n_thr);
  }
  return hipGetLastError();
}

}  // namespace ds4q

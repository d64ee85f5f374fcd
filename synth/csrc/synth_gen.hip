// Device twin of the synth module's seeded block generators.
//
// Draws exactly the bytes that synth.q2k_blocks / synth.q41_blocks draw on the
// host (SplitMix64 used counter-style; Steele, Lea & Flood, OOPSLA 2014), so
// that multi-GB expert stacks can be generated in place on the GPU.  It holds
// no arithmetic of the quantised-MoE method: it writes random bytes and picks
// fp16 bit patterns out of caller-supplied quantile tables.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t sm64(uint64_t key, uint64_t idx) {
  uint64_t z = key + (idx + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// One thread per Q2_K block: words 11b..11b+10 of the stream.
__global__ void synth_q2k_kernel(uint32_t *__restrict__ dst, const uint64_t *__restrict__ keys,
                                 int64_t blocks_per_tensor, int64_t n_total,
                                 const uint16_t *__restrict__ half_tab) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_total) return;
  int64_t t = g / blocks_per_tensor;
  int64_t b = g - t * blocks_per_tensor;
  uint64_t key = keys[t];
  uint32_t *o = dst + g * 21;
  uint64_t base = (uint64_t)b * 11ull;
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    uint64_t w = sm64(key, base + j);
    o[2 * j] = (uint32_t)w;
    o[2 * j + 1] = (uint32_t)(w >> 32);
  }
  uint64_t w10 = sm64(key, base + 10);
  uint32_t d = half_tab[(uint32_t)w10 & 0xFFFFu];
  uint32_t dmin = half_tab[((uint32_t)w10 >> 16) & 0xFFFFu];
  o[20] = d | (dmin << 16);
}

// One thread per Q4_1 block: words 3b..3b+2 of the stream.
__global__ void synth_q41_kernel(uint32_t *__restrict__ dst, const uint64_t *__restrict__ keys,
                                 int64_t blocks_per_tensor, int64_t n_total,
                                 const uint16_t *__restrict__ half_tab,
                                 const uint16_t *__restrict__ m_tab) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_total) return;
  int64_t t = g / blocks_per_tensor;
  int64_t b = g - t * blocks_per_tensor;
  uint64_t key = keys[t];
  uint32_t *o = dst + g * 5;
  uint64_t base = (uint64_t)b * 3ull;
  uint64_t w0 = sm64(key, base), w1 = sm64(key, base + 1), w2 = sm64(key, base + 2);
  uint32_t d = half_tab[(uint32_t)w0 & 0xFFFFu];
  uint32_t m = m_tab[((uint32_t)w0 >> 16) & 0xFFFFu];
  o[0] = d | (m << 16);
  o[1] = (uint32_t)(w0 >> 32);
  o[2] = (uint32_t)w1;
  o[3] = (uint32_t)(w1 >> 32);
  o[4] = (uint32_t)w2;
}

}  // namespace

// Fill n_tensors consecutive tensors of blocks_per_tensor blocks each; tensor i
// uses stream keys[i] (device array).  dst must be 4-byte aligned.  Returns 0 or
// a hipError_t value.
extern "C" int synth_q2k_fill(void *dst, const uint64_t *keys, int64_t n_tensors,
                              int64_t blocks_per_tensor, const uint16_t *half_tab, void *stream) {
  int64_t n = n_tensors * blocks_per_tensor;
  if (n <= 0) return 0;
  int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(synth_q2k_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t *)dst, keys, blocks_per_tensor, n, half_tab);
  return (int)hipGetLastError();
}

extern "C" int synth_q41_fill(void *dst, const uint64_t *keys, int64_t n_tensors,
                              int64_t blocks_per_tensor, const uint16_t *half_tab,
                              const uint16_t *m_tab, void *stream) {
  int64_t n = n_tensors * blocks_per_tensor;
  if (n <= 0) return 0;
  int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(synth_q41_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t *)dst, keys, blocks_per_tensor, n, half_tab, m_tab);
  return (int)hipGetLastError();
}

// Shared device helpers and block-format constants for the gfx950 kernels.
//
// Block formats:
//  Q2_K ("【#2】ds4.c 해독하기", Q2_K block-layout table and packing expression):
//    84 B per 256 values; bytes 0..15 one byte per 16-value sub-block (scale in
//    the low nibble, min in the high nibble), bytes 16..79 the 2-bit codes
//    (code of value v sits in byte 16 + 32*(v>>7) + (v&31) at bit 2*((v>>5)&3)),
//    fp16 d at 80, fp16 dmin at 82; value = d*scale*code - dmin*min.
//  Q4_1 (ThakiCloud "...GGUF Q4_1 재부호화", Q4_1 block section):
//    20 B per 32 values; fp16 d at 0, fp16 m at 2, qs[16] at 4; value j < 16 is
//    the low nibble of qs[j], value j+16 its high nibble; value = d*code + m.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4q {

constexpr int QK_Q2K = 256, BB_Q2K = 84;
constexpr int QK_Q41 = 32, BB_Q41 = 20;
constexpr int TYPE_Q4_1 = 3, TYPE_Q2_K = 10;

__host__ __device__ constexpr int64_t row_bytes(int type, int64_t cols) {
  return type == TYPE_Q2_K ? cols / QK_Q2K * BB_Q2K : cols / QK_Q41 * BB_Q41;
}

__device__ __forceinline__ float f16lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Byte n of a dword as float (v_cvt_f32_ubyteN).
__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xFFu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }

// 4-byte-aligned dword loads of block fields (blocks are only 4-byte aligned).
__device__ __forceinline__ uint32_t ld32(const uint8_t *p) {
  return *reinterpret_cast<const uint32_t *>(p);
}

// bf16 round-to-nearest-even of an fp32 value, NaN kept quiet.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Sum over groups of W consecutive lanes of a wave64 (W power of two <= 64);
// every lane of the group gets the group total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace ds4q

// Standalone block dequantisation: Q2_K / Q4_1 -> f32 or bf16.
//
// Data movement.  Each wave converts groups of whole blocks: the group's
// bytes come in as 16-byte loads of consecutive chunks (4 Q2_K blocks = 336 B
// = 21 chunks; 32 Q4_1 blocks = 640 B = 40 chunks; both multiples of 16 from
// a 16-byte aligned tensor), are parked in the wave's own LDS area, and each
// lane then produces 4 consecutive values per block row it covers, so every
// store instruction of a wave writes one contiguous 1 KB (f32) / 512 B (bf16)
// run.  The next group's chunks are requested before the current group is
// converted.  Outputs are streamed with non-temporal stores (they are not
// read again by this kernel).  The last, partial group is read dword by
// dword, so no byte past the tensor is touched.
//
// Value arithmetic ("【#2】ds4.c 해독하기", Q2_K block-layout table; ThakiCloud
// Q4_1 block section): d*scale (exact in fp32: 11 x 4 bits) times the code
// (exact) plus -(dmin*min) (exact) in one fma, so the fp32 result is rounded
// exactly once; bf16 is its round-to-nearest-even.  Q4_1: fma(d, code, m).
#include "common.h"
#include "launch.h"

namespace ds4q {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
__device__ __forceinline__ void store4(void *dst, int64_t idx, float a, float b, float c, float d) {
  if constexpr (BF16) {
    const u32x2 v = {bf16_rne_pair(a, b), bf16_rne_pair(c, d)};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(dst) + idx));
  } else {
    const f32x4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(static_cast<float *>(dst) + idx));
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One group of GB blocks of BB bytes (GB * BB a multiple of 16): the lane's
// 16-byte chunk (lanes < GB * BB / 16), or nothing past the group's nb blocks.
template <int GB, int BB>
struct GroupLoad {
  static constexpr int CHUNKS = GB * BB / 16;
  static_assert(GB * BB % 16 == 0 && CHUNKS <= 64, "group must be whole 16-byte chunks");
  u32x4 v;
  __device__ __forceinline__ void load(const uint8_t *__restrict__ src, int64_t b0, int lane) {
    if (lane < CHUNKS) v = *reinterpret_cast<const u32x4 *>(src + b0 * BB + 16 * lane);
  }
  __device__ __forceinline__ void park(uint32_t *__restrict__ st, int lane) const {
    if (lane < CHUNKS) *reinterpret_cast<u32x4 *>(st + 4 * lane) = v;
  }
};

// The partial last group (nb < GB blocks): dword loads straight into LDS.
template <int BB>
__device__ __forceinline__ void park_tail(const uint8_t *__restrict__ src, int64_t b0, int nb,
                                          uint32_t *__restrict__ st, int lane) {
  for (int dw = lane; dw < nb * (BB / 4); dw += 64) st[dw] = ld32(src + b0 * BB + 4 * dw);
}

// Q2_K: groups of 4 blocks; lane i covers values 4i..4i+3 of each block,
// which share one sub-block (i>>2) and one code dword (bit pair (i>>3)&3).
template <bool BF16>
__global__ __launch_bounds__(256) void dequant_q2k_kernel(const uint8_t *__restrict__ src,
                                                          void *__restrict__ dst, int64_t nblk) {
  constexpr int GB = 4, DW = BB_Q2K / 4;  // 21 dwords per block
  __shared__ __attribute__((aligned(16))) uint32_t stage[4][GB * DW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t *st = stage[w];
  const int64_t ngroups = (nblk + GB - 1) / GB;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  int64_t grp = (int64_t)blockIdx.x * 4 + w;
  const int e0 = 4 * lane;
  const int h = e0 >> 7, k = (e0 >> 5) & 3, l0 = e0 & 31;
  const int code_dw = (16 + 32 * h + l0) >> 2;
  GroupLoad<GB, BB_Q2K> cur, nxt;
  if (grp < ngroups && (grp + 1) * GB <= nblk) cur.load(src, grp * GB, lane);
  for (; grp < ngroups; grp += nwaves) {
    const int64_t b0 = grp * GB;
    const int nb = nblk - b0 < GB ? (int)(nblk - b0) : GB;
    if (nb == GB) cur.park(st, lane);
    else park_tail<BB_Q2K>(src, b0, nb, st, lane);
    wave_sync();
    const int64_t gn = grp + nwaves;
    if (gn < ngroups && (gn + 1) * GB <= nblk) nxt.load(src, gn * GB, lane);
    for (int j = 0; j < nb; ++j) {
      const uint32_t *blk = st + j * DW;
      const uint32_t qw = (blk[code_dw] >> (2 * k)) & 0x03030303u;
      const uint32_t sb = (blk[lane >> 4] >> (8 * ((lane >> 2) & 3))) & 0xFFu;
      const uint32_t dd = blk[20];
      const float ds = f16lo(dd) * (float)(sb & 15u);
      const float dm = f16hi(dd) * (float)(sb >> 4);
      store4<BF16>(dst, (b0 + j) * 256 + e0, fmaf(ds, ub0(qw), -dm), fmaf(ds, ub1(qw), -dm),
                   fmaf(ds, ub2(qw), -dm), fmaf(ds, ub3(qw), -dm));
    }
    wave_sync();  // the LDS area is rewritten by the next group
    cur = nxt;
  }
}

// Q4_1: groups of 32 blocks; per step of 8 blocks, lane i covers values
// 4(i&7)..+3 of block i>>3: low nibbles of qs[4(i&3)..] for (i&7) < 4, high
// nibbles for (i&7) >= 4.
template <bool BF16>
__global__ __launch_bounds__(256) void dequant_q41_kernel(const uint8_t *__restrict__ src,
                                                          void *__restrict__ dst, int64_t nblk) {
  constexpr int GB = 32, DW = BB_Q41 / 4;  // 5 dwords per block
  __shared__ __attribute__((aligned(16))) uint32_t stage[4][GB * DW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t *st = stage[w];
  const int64_t ngroups = (nblk + GB - 1) / GB;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  int64_t grp = (int64_t)blockIdx.x * 4 + w;
  const int bi = lane >> 3, i = lane & 7;
  GroupLoad<GB, BB_Q41> cur, nxt;
  if (grp < ngroups && (grp + 1) * GB <= nblk) cur.load(src, grp * GB, lane);
  for (; grp < ngroups; grp += nwaves) {
    const int64_t b0 = grp * GB;
    const int nb = nblk - b0 < GB ? (int)(nblk - b0) : GB;
    if (nb == GB) cur.park(st, lane);
    else park_tail<BB_Q41>(src, b0, nb, st, lane);
    wave_sync();
    const int64_t gn = grp + nwaves;
    if (gn < ngroups && (gn + 1) * GB <= nblk) nxt.load(src, gn * GB, lane);
    for (int s = 0; s < GB / 8; ++s) {
      const int j = 8 * s + bi;
      if (j < nb) {
        const uint32_t *blk = st + j * DW;
        const uint32_t qw = (blk[1 + (i & 3)] >> (4 * (i >> 2))) & 0x0F0F0F0Fu;
        const uint32_t dm = blk[0];
        const float d = f16lo(dm), m = f16hi(dm);
        store4<BF16>(dst, (b0 + j) * 32 + 4 * i, fmaf(d, ub0(qw), m), fmaf(d, ub1(qw), m),
                     fmaf(d, ub2(qw), m), fmaf(d, ub3(qw), m));
      }
    }
    wave_sync();
    cur = nxt;
  }
}

}  // namespace

hipError_t launch_dequant(int src_type, const void *src, int64_t rows, int64_t cols, bool bf16,
                          void *dst, hipStream_t s) {
  const int qk = src_type == TYPE_Q2_K ? QK_Q2K : QK_Q41;
  const int64_t nblk = rows * (cols / qk);
  if (nblk <= 0) return hipSuccess;
  const int gb = src_type == TYPE_Q2_K ? 4 : 32;
  const int64_t ngroups = (nblk + gb - 1) / gb;
  // about two groups per wave (the next group's loads overlap the current
  // group's stores), at most 4096 workgroups
  const int64_t want = (ngroups + 7) / 8;
  const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
  const uint8_t *p = static_cast<const uint8_t *>(src);
  if (src_type == TYPE_Q2_K) {
    if (bf16) hipLaunchKernelGGL(dequant_q2k_kernel<true>, dim3(grid), dim3(256), 0, s, p, dst, nblk);
    else hipLaunchKernelGGL(dequant_q2k_kernel<false>, dim3(grid), dim3(256), 0, s, p, dst, nblk);
  } else {
    if (bf16) hipLaunchKernelGGL(dequant_q41_kernel<true>, dim3(grid), dim3(256), 0, s, p, dst, nblk);
    else hipLaunchKernelGGL(dequant_q41_kernel<false>, dim3(grid), dim3(256), 0, s, p, dst, nblk);
  }
  return hipGetLastError();
}

}  // namespace ds4q

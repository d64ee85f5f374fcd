// Prefill path on Q4_1 weights: grouped GEMMs over experts on gfx950 bf16
// matrix cores.  (Q2_K weights take the int8 path in prefill_i8.hip.)
//
// The pairs (token, slot) are grouped by expert (route.hip); the m-tile list
// holds up to PREFILL_TILE_M consecutive sorted pairs of one expert.  For one
// work item (m-tile, n-tile):
//   GEMM-1: A = the tile's token rows of x (bf16, gathered), B = gate and up
//           rows of the expert, C = A * B^T in fp32; epilogue h = silu(g) * u
//           rounded to bf16, stored per sorted pair position.
//   GEMM-2: A = the tile's rows of h (contiguous in sorted order), B = down
//           rows; C stored as fp32 per sorted pair position, summed over the
//           token's slots with the routing weights by the combine kernel.
// ("【#2】ds4.c 해독하기": w1 = gate, w3 = up, w2 = down, SwiGLU, and the
// routing weight multiplies the routed SwiGLU row before the down projection.)
//
// Data movement.  The A tile (m-tile rows x 256 K, bf16) is staged in LDS once
// per K step and read by all four waves.  B never touches LDS: each lane
// dequantises exactly the 8 weights its MFMA B operand holds — 8 nibbles of
// one half of a Q4_1 block — straight from global memory into registers (fp32
// fma, one rounding, then round-to-nearest-even bf16).  Each weight of the
// expert's n-tile is dequantised once per m-tile.
//
// MFMA v_mfma_f32_16x16x32_bf16: A lane l holds A[l%16][8*(l/16) .. +7],
// B lane l holds B[8*(l/16) .. +7][l%16] (the same K slots as A),
// C lane l holds C[4*(l/16) + i][l%16], i = 0..3.
#include "common.h"
#include "launch.h"

namespace ds4q {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int TM = PREFILL_TILE_M;  // pairs per m-tile
constexpr int KS = 256;             // K per LDS stage
constexpr int LDA = KS + 8;         // padded LDS row (bf16 elements)
constexpr int MT = TM / 16;         // 16-row MFMA tiles along M

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 to_frag(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, (u32x4){a, b, c, d});
}

// Raw bytes of one weight row's K step (eight Q4_1 blocks) that lane group g
// needs: MFMA step j = Q4_1 block j of the K step, values 8g + i, i.e.
// nibbles of qs[8(g&1) + i], low for g < 2, high for g >= 2.
struct Q41Step {
  const uint8_t *base;
  __device__ __forceinline__ void load(const uint8_t *__restrict__ blk) { base = blk; }
  template <int J>
  __device__ __forceinline__ bf16x8 frag(int g) const {
    const uint8_t *blk = base + J * BB_Q41;
    const uint32_t dm = ld32(blk);
    const int sh = 4 * (g >> 1);
    const uint32_t t0 = (ld32(blk + 4 + 8 * (g & 1)) >> sh) & 0x0F0F0F0Fu;
    const uint32_t t1 = (ld32(blk + 8 + 8 * (g & 1)) >> sh) & 0x0F0F0F0Fu;
    const float d = f16lo(dm), m = f16hi(dm);
    return to_frag(pack_bf16(fmaf(d, ub0(t0), m), fmaf(d, ub1(t0), m)),
                   pack_bf16(fmaf(d, ub2(t0), m), fmaf(d, ub3(t0), m)),
                   pack_bf16(fmaf(d, ub0(t1), m), fmaf(d, ub1(t1), m)),
                   pack_bf16(fmaf(d, ub2(t1), m), fmaf(d, ub3(t1), m)));
  }
};

// SWIGLU: n-tile = 128 rows of F for gate and up (wave w: rows 32w..32w+31 of
// both); otherwise n-tile = 256 down rows (wave w: rows 64w..64w+63).
template <bool SWIGLU>
__global__ __launch_bounds__(256, 2) void prefill_gemm_kernel(
    const uint8_t *__restrict__ W0, const uint8_t *__restrict__ W1, int K, int rows_per_expert,
    const uint16_t *__restrict__ A, int gather_tokens, int kslots, RouteBufs rb, int n_ntiles,
    uint16_t *__restrict__ hb, float *__restrict__ o) {
  __shared__ __attribute__((aligned(16))) uint16_t As[TM * LDA];
  __shared__ int arow[TM];

  int mtile, ntile;
  if (!xcd_tile_of(*rb.n_tiles, n_ntiles, &mtile, &ntile)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int e = rb.tiles[2 * mtile], start = rb.tiles[2 * mtile + 1];
  const int end = rb.offsets[e + 1];
  const int valid = end - start < TM ? end - start : TM;
  const int n_mt = (valid + 15) >> 4;

  if (tid < TM) {
    int src = -1;
    if (tid < valid) src = gather_tokens ? rb.pairs[start + tid] / kslots : start + tid;
    arow[tid] = src;
  }

  const int64_t rbytes = row_bytes(TYPE_Q4_1, K);
  const uint8_t *brow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    int r;
    const uint8_t *Wt;
    if constexpr (SWIGLU) {
      r = ntile * 128 + 32 * w + 16 * (t & 1) + n;
      Wt = (t < 2) ? W0 : W1;
    } else {
      r = ntile * 256 + 64 * w + 16 * t + n;
      Wt = W0;
    }
    brow[t] = Wt + ((int64_t)e * rows_per_expert + r) * rbytes;
  }

  f32x4 acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int step_bytes = (int)row_bytes(TYPE_Q4_1, KS);
  for (int kb = 0; kb < K / KS; ++kb) {
    __syncthreads();
    // stage A: 128 rows x 256 bf16 = 32 chunks of 16 B per row, four chunks
    // per thread at a time (bounds the registers in flight)
#pragma unroll
    for (int i0 = 0; i0 < TM * (KS / 8) / 256; i0 += 4) {
      uint4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // rows of absent pairs read row 0 and store zeros (no branch)
        const int c = tid + 256 * (i0 + i);
        const int src = arow[c >> 5];
        const uint4 t = *reinterpret_cast<const uint4 *>(A + (int64_t)(src < 0 ? 0 : src) * K + kb * KS + (c & 31) * 8);
        v[i] = src < 0 ? make_uint4(0u, 0u, 0u, 0u) : t;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * (i0 + i);
        *reinterpret_cast<uint4 *>(&As[(c >> 5) * LDA + (c & 31) * 8]) = v[i];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    Q41Step rs[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) rs[t].load(brow[t] + (int64_t)kb * step_bytes);

    // K order inside the step: MFMA step J, lane group g takes the step's
    // values 32J + 8g .. +7 (the same for A and B).
#define DS4Q_STEP(J)                                                                   \
  {                                                                                    \
    /* A fragments first (rows of absent pairs hold zeros), so that their    */ \
    /* LDS latency hides behind the weight dequantisation                    */ \
    const int koff = 32 * (J) + 8 * g;                                                 \
    bf16x8 a[MT];                                                                      \
    _Pragma("unroll") for (int i = 0; i < MT; ++i)                                     \
        a[i] = *reinterpret_cast<const bf16x8 *>(&As[(16 * i + n) * LDA + koff]);      \
    bf16x8 b[4];                                                                       \
    _Pragma("unroll") for (int t = 0; t < 4; ++t) b[t] = rs[t].template frag<J>(g);    \
    _Pragma("unroll") for (int i = 0; i < MT; ++i) {                                   \
      if (i < n_mt) {                                                                  \
        _Pragma("unroll") for (int t = 0; t < 4; ++t)                                  \
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[t], acc[i][t], 0, 0, 0); \
      }                                                                                \
    }                                                                                  \
  }
    DS4Q_STEP(0) DS4Q_STEP(1) DS4Q_STEP(2) DS4Q_STEP(3)
    DS4Q_STEP(4) DS4Q_STEP(5) DS4Q_STEP(6) DS4Q_STEP(7)
#undef DS4Q_STEP
  }

  // epilogue
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    if (i >= n_mt) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 16 * i + 4 * g + q;
      if (m >= valid) continue;
      const int64_t pos = start + m;
      if constexpr (SWIGLU) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r = ntile * 128 + 32 * w + 16 * t + n;
          const float hv = silu(acc[i][t][q]) * acc[i][t + 2][q];
          hb[pos * rows_per_expert + r] = (uint16_t)bf16_rne_bits(hv);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = ntile * 256 + 64 * w + 16 * t + n;
          o[pos * rows_per_expert + r] = acc[i][t][q];
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void prep_bf16_kernel(const float *__restrict__ x,
                                                        const float *__restrict__ inv_rms, int D,
                                                        int64_t n4, uint16_t *__restrict__ xb) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float s = inv_rms ? inv_rms[(4 * i) / D] : 1.0f;
  const float4 v = *reinterpret_cast<const float4 *>(x + 4 * i);
  uint2 out;
  out.x = bf16_rne_bits(v.x * s) | (bf16_rne_bits(v.y * s) << 16);
  out.y = bf16_rne_bits(v.z * s) | (bf16_rne_bits(v.w * s) << 16);
  *reinterpret_cast<uint2 *>(xb + 4 * i) = out;
}

unsigned grid_for(int max_tiles, int n_ntiles) {
  const int64_t total = (int64_t)max_tiles * n_ntiles;
  return (unsigned)((total + 7) / 8 * 8);
}

}  // namespace

hipError_t launch_prep_bf16(const float *x, const float *inv_rms, int T, int D, uint16_t *xb,
                            hipStream_t s) {
  const int64_t n4 = (int64_t)T * D / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(prep_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, x,
                     inv_rms, D, n4, xb);
  return hipGetLastError();
}

hipError_t launch_prefill_gateup(const MoeDims &m, const uint16_t *xb, int T, const RouteBufs &rb,
                                 int max_tiles, uint16_t *hb, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nn = m.F / 128;
  const dim3 grid(grid_for(max_tiles, nn));
  hipLaunchKernelGGL((prefill_gemm_kernel<true>), grid, dim3(256), 0, s, m.gate, m.up, m.D, m.F, xb,
                     1, m.k, rb, nn, hb, nullptr);
  return hipGetLastError();
}

hipError_t launch_prefill_down(const MoeDims &m, const uint16_t *hb, int T, const RouteBufs &rb,
                               int max_tiles, float *o, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nn = m.D / 256;
  const dim3 grid(grid_for(max_tiles, nn));
  hipLaunchKernelGGL((prefill_gemm_kernel<false>), grid, dim3(256), 0, s, m.down, nullptr, m.F, m.D,
                     hb, 0, m.k, rb, nn, nullptr, o);
  return hipGetLastError();
}

}  // namespace ds4q

// Prefill path on Q4_1 weights: grouped GEMMs over experts on gfx950 bf16
// matrix cores.  (Q2_K weights take the fp16 path in prefill_f16.hip.)
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
// Data movement (eight waves; wave w owns 16 gate + 16 up rows, or 32 down
// rows, and all the tile's rows of A).  K advances in steps of 256 values
// (eight Q4_1 blocks).  The next step's A tile (128 rows x 512 B of bf16) goes
// to the other of two LDS buffers by direct buffer loads to LDS (one 1-KiB
// instruction = 2 rows x 32 chunks; chunk c of row r is stored at chunk
// position c ^ (r & 15), so the 16 lanes reading one chunk column touch 16
// distinct bank groups), and the raw bytes of the next step's weights go to
// registers, while the current step computes.  One wait and one barrier per
// step.  B never touches LDS: each lane dequantises exactly the 8 weights its
// MFMA B operand holds -- 8 nibbles of one half of a Q4_1 block -- from those
// registers (fp32 fma, one rounding, then round-to-nearest-even bf16); each
// weight of the n-tile is dequantised once per m-tile.  The step loop is
// instantiated per count of live 16-row subtiles, so it has no branches;
// rows of absent pairs repeat row 0 and are never stored.
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

constexpr int TM = PREFILL_TILE_M;        // pairs per m-tile
constexpr int MT = TM / 16;               // 16-row MFMA subtiles along M
constexpr int KS = 256;                   // K per step (eight Q4_1 blocks)
constexpr int NJ = KS / 64;               // Q4_1 block pairs per step (two MFMAs each)
constexpr int AROWB = KS * 2;             // bytes of one A row per step
constexpr int ASTAGE = TM * AROWB;        // one LDS buffer (64 KiB)
static_assert(MT >= 4 && MT <= 8, "m-tiles of 64..128 rows (the step-loop instances below)");
constexpr int STEP_BYTES = KS / 32 * BB_Q41;  // bytes of one weight row per step


__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 to_frag(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, (u32x4){a, b, c, d});
}

// Raw bytes of a pair of Q4_1 blocks (2jp, 2jp+1) for lane group g: block
// b = 2jp + (g >> 1), half p = g & 1 -- 12 bytes from offset 8p, i.e. (d, m)
// and code bytes 0..7 for p = 0, code bytes 4..15 for p = 1; the lane's code
// bytes 8p..8p+7 are dwords 1 and 2 either way.  Their low nibbles are values
// 8p..8p+7 of block b (the lane's B operand of the pair's "low" MFMA), their
// high nibbles values 16+8p..16+8p+7 (of the "high" MFMA); so the pair's two
// MFMAs cover its 64 values with one load per lane.  Lanes of half 1 take
// (d, m) from their half-0 partner 16 lanes below (v_permlane16_swap).
typedef uint32_t u32x3a __attribute__((ext_vector_type(3), aligned(4)));
struct Q41Raw {
  uint32_t x, c0, c1;
  __device__ __forceinline__ void load(const uint8_t *__restrict__ pair, int g) {
    const u32x3a v = *reinterpret_cast<const u32x3a *>(pair + (g >> 1) * BB_Q41 + 8 * (g & 1));
    x = v.x;
    c0 = v.y;
    c1 = v.z;
  }
  // B operands of the low and the high MFMA
  __device__ __forceinline__ void frags(bf16x8 &lo, bf16x8 &hi) const {
    // the even 16-lane row of each pair (p = 0) holds (d, m); both rows get it
    const uint32_t dm = __builtin_amdgcn_permlane16_swap(x, x, false, false)[0];
    uint32_t l0 = c0 & 0x0F0F0F0Fu, l1 = c1 & 0x0F0F0F0Fu;
    uint32_t h0 = (c0 >> 4) & 0x0F0F0F0Fu, h1 = (c1 >> 4) & 0x0F0F0F0Fu;
    // opaque to the combiner, so that each byte converts with one
    // v_cvt_f32_ubyteN instead of a bit-field extract and a convert
    asm("" : "+v"(l0), "+v"(l1), "+v"(h0), "+v"(h1));
    const float d = f16lo(dm), m = f16hi(dm);
    lo = to_frag(pack_bf16(fmaf(d, ub0(l0), m), fmaf(d, ub1(l0), m)),
                 pack_bf16(fmaf(d, ub2(l0), m), fmaf(d, ub3(l0), m)),
                 pack_bf16(fmaf(d, ub0(l1), m), fmaf(d, ub1(l1), m)),
                 pack_bf16(fmaf(d, ub2(l1), m), fmaf(d, ub3(l1), m)));
    hi = to_frag(pack_bf16(fmaf(d, ub0(h0), m), fmaf(d, ub1(h0), m)),
                 pack_bf16(fmaf(d, ub2(h0), m), fmaf(d, ub3(h0), m)),
                 pack_bf16(fmaf(d, ub0(h1), m), fmaf(d, ub1(h1), m)),
                 pack_bf16(fmaf(d, ub2(h1), m), fmaf(d, ub3(h1), m)));
  }
};

struct StepCtx {
  const uint8_t *abase;     // A rows (bytes) from row rbase
  uint32_t aoff[MT];        // byte offsets of the lane's DMA chunks from abase (row part + chunk)
  int aoffj[2 * NJ];        // LDS offsets of the lane's A chunks, low and high MFMA of pair jp
  const uint8_t *brow[2];   // the lane's two weight rows
  int w, g;
};

// Wait for every request of this wave, then a bare workgroup barrier (a
// workgroup fence would add nothing: the wait already covers the DMA).
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The step loop for NMT live subtiles: acc[i][t] += A(subtile i) * B(t)^T.
// Every wave issues the same requests every step (the A rows of NU DMA
// loads, rows >= 16*NMT repeating row 0 and never read, and its weights);
// the step past the end requests the last step again, so the loop has no
// branches and the only wait is the one at the step's end.
template <int NMT>
__device__ __forceinline__ void q41_loop(const StepCtx &cx, int ns, uint8_t *As0, uint8_t *As1,
                                         f32x4 (&acc)[MT][2]) {
  constexpr int NU = NMT;  // DMA loads per wave (2 rows each): rows 0 .. 16*NU-1
  const int w = cx.w, g = cx.g;
  const DmaSrc asrc(cx.abase);
  auto issue_a = [&](int s, uint8_t *As) {
#pragma unroll
    for (int u = 0; u < NU; ++u) asrc.copy16(cx.aoff[u], (uint32_t)s * AROWB, As + (8 * u + w) * 1024);
  };
  auto issue_w = [&](int s, Q41Raw (&r)[2][NJ]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < NJ; ++j) r[t][j].load(cx.brow[t] + (int64_t)s * STEP_BYTES + 2 * j * BB_Q41, g);
  };
  auto compute = [&](const uint8_t *As, const Q41Raw (&r)[2][NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      bf16x8 b[2][2];  // [t][low/high]
      r[0][j].frags(b[0][0], b[0][1]);
      r[1][j].frags(b[1][0], b[1][1]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 a[NMT];
#pragma unroll
        for (int i = 0; i < NMT; ++i)
          a[i] = *reinterpret_cast<const bf16x8 *>(As + i * (16 * AROWB) + cx.aoffj[2 * j + h]);
        // one fenced MFMA group (no later instruction within 8 wait states of
        // any of them)
        mfma_group_begin();
#pragma unroll
        for (int i = 0; i < NMT; ++i) {
          acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[0][h], acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[1][h], acc[i][1], 0, 0, 0);
        }
        mfma_fence();
      }
    }
  };
  Q41Raw rw0[2][NJ], rw1[2][NJ];
  issue_a(0, As0);
  issue_w(0, rw0);
  step_barrier();
  for (int s = 0; s + 1 < ns; s += 2) {
    // nothing is outstanding here (the last step ended with a full wait);
    // saying so at the loop head keeps the compiler from adding a wait for
    // the loads issued below before this step's computation
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_sched_barrier(0);
    issue_a(s + 1, As1);
    issue_w(s + 1, rw1);
    __builtin_amdgcn_sched_barrier(0);
    compute(As0, rw0);
    __builtin_amdgcn_sched_barrier(0);
    step_barrier();  // step s+1 landed; every wave is done with As0
    const int s2 = s + 2 < ns ? s + 2 : ns - 1;
    issue_a(s2, As0);
    issue_w(s2, rw0);
    __builtin_amdgcn_sched_barrier(0);
    compute(As1, rw1);
    __builtin_amdgcn_sched_barrier(0);
    step_barrier();
  }
  if (ns & 1) compute(As0, rw0);  // a single step (K = 256)
}

// SWIGLU: n-tile = 128 rows of F for gate and up (wave w: row 16w + n of
// both); otherwise n-tile = 256 down rows (wave w: rows 32w + 16t + n).
template <bool SWIGLU>
__global__ __launch_bounds__(512) void prefill_q41_kernel(
    const uint8_t *__restrict__ W0, const uint8_t *__restrict__ W1, int K, int rows_per_expert,
    const uint16_t *__restrict__ A, int gather_tokens, int kslots, RouteBufs rb, int n_ntiles,
    uint16_t *__restrict__ hb, uint16_t *__restrict__ o) {
  __shared__ __attribute__((aligned(1024))) uint8_t As0[ASTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[ASTAGE];
  __shared__ int arow[TM];

  int mtile, ntile;
  if (!xcd_tile_of(*rb.n_tiles, n_ntiles, &mtile, &ntile)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int e = rb.tiles_sz[2 * mtile], start = rb.tiles_sz[2 * mtile + 1];
  const int end = rb.offsets[e + 1];
  const int valid = end - start < TM ? end - start : TM;
  const int nmt = (valid + 15) >> 4;

  if (tid < TM) {
    const int m = tid < valid ? tid : 0;  // absent rows repeat row 0; never stored
    arow[tid] = gather_tokens ? rb.pairs[start + m] / kslots : start + m;
  }
  __syncthreads();

  StepCtx cx;
  cx.w = w;
  cx.g = g;
  // offsets from the tile's first row (gathered token rows: from row 0;
  // T * K * 2 < 2^29 bytes), so they fit the 32-bit buffer offsets
  const int rbase = gather_tokens ? 0 : start;
  cx.abase = reinterpret_cast<const uint8_t *>(A) + (int64_t)rbase * (2 * K);
  // DMA load I = 8u + w covers rows 2I, 2I+1: lane l takes row 2I + l/32 and
  // stores it at chunk position l%32, which holds data chunk (l%32) ^ (row%16)
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int r = 2 * (8 * u + w) + (lane >> 5);
    const int c = (lane & 31) ^ (r & 15);
    cx.aoff[u] = (uint32_t)(arow[r] - rbase) * (2 * K) + c * 16;
  }
  // pair jp: block b = 2jp + (g >> 1); the low MFMA reads chunk 4b + (g & 1)
  // (values 8p..8p+7), the high one chunk 4b + 2 + (g & 1)
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = 4 * (2 * j + (g >> 1)) + (g & 1);
    cx.aoffj[2 * j] = n * AROWB + ((c ^ n) * 16);
    cx.aoffj[2 * j + 1] = n * AROWB + (((c + 2) ^ n) * 16);
  }
  const int64_t rbytes = row_bytes(TYPE_Q4_1, K);
  int wrow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if constexpr (SWIGLU) {
      wrow[t] = ntile * 128 + 16 * w + n;
      cx.brow[t] = (t == 0 ? W0 : W1) + ((int64_t)e * rows_per_expert + wrow[t]) * rbytes;
    } else {
      wrow[t] = ntile * 256 + 32 * w + 16 * t + n;
      cx.brow[t] = W0 + ((int64_t)e * rows_per_expert + wrow[t]) * rbytes;
    }
  }

  f32x4 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i][0] = acc[i][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int ns = K / KS;
  switch (nmt) {
    case 1: q41_loop<1>(cx, ns, As0, As1, acc); break;
    case 2: q41_loop<2>(cx, ns, As0, As1, acc); break;
    case 3: q41_loop<3>(cx, ns, As0, As1, acc); break;
    case 4: q41_loop<4>(cx, ns, As0, As1, acc); break;
    case 5: if constexpr (MT >= 5) q41_loop<5>(cx, ns, As0, As1, acc); break;
    case 6: if constexpr (MT >= 6) q41_loop<6>(cx, ns, As0, As1, acc); break;
    case 7: if constexpr (MT >= 7) q41_loop<7>(cx, ns, As0, As1, acc); break;
    default: if constexpr (MT >= 8) q41_loop<8>(cx, ns, As0, As1, acc); break;
  }

  // epilogue: rows of live pairs only
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 16 * i + 4 * g + q;
      if (m >= valid) continue;
      const int64_t pos = start + m;
      if constexpr (SWIGLU) {
        const float hv = silu(acc[i][0][q]) * acc[i][1][q];
        hb[pos * rows_per_expert + wrow[0]] = (uint16_t)bf16_rne_bits(hv);
      } else {
        // wrow[1] = wrow[0] + 16; lanes n, n ^ 1 share g, hence m and validity
        store_bf16_row_pair(o + pos * rows_per_expert + wrow[0], n, acc[i][0][q], acc[i][1][q]);
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
  const dim3 grid(xcd_grid(max_tiles, nn));
  hipLaunchKernelGGL((prefill_q41_kernel<true>), grid, dim3(512), 0, s, m.gate, m.up, m.D, m.F, xb,
                     1, m.k, rb, nn, hb, nullptr);
  return hipGetLastError();
}

hipError_t launch_prefill_down(const MoeDims &m, const uint16_t *hb, int T, const RouteBufs &rb,
                               int max_tiles, uint16_t *o, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nn = m.D / 256;
  const dim3 grid(xcd_grid(max_tiles, nn));
  hipLaunchKernelGGL((prefill_q41_kernel<false>), grid, dim3(512), 0, s, m.down, nullptr, m.F, m.D,
                     hb, 0, m.k, rb, nn, nullptr, o);
  return hipGetLastError();
}

}  // namespace ds4q

// Decode of 2..64 tokens on Q2_K weights: expert-grouped, streaming.
//
// At decode sizes an expert holds a few of the call's token-expert pairs,
// so the work is the weight stream of the routed experts ("【#2】ds4.c
// 해독하기": only the routed experts' bytes move per token).  A work item is an
// m-tile of at most DECODE_TILE_M sorted pairs of one expert and an n-tile of
// weight rows.  Each of the eight waves owns 32 weight rows (two 16-row
// subtiles) and a quarter or half of K (four blocks), and requests all of its
// raw weight bytes as soon as the expert is known; the tile's prepared
// activation rows (i8_ops.h) for the whole K then go to LDS by direct
// global->LDS loads, only for the pairs that are present.  One wait and one
// barrier later each wave runs its blocks on the matrix cores, the K parts
// meet in LDS, and the epilogue writes SwiGLU rows (gate/up) or the down rows,
// in sorted-pair order.
//
// Arithmetic as in the prefill GEMMs (prefill_i8.hip), with the bf16 residues
// of -dmin*mn applied as well (min term to about 16 bits): the integer MFMA's
// 16 A rows are the 8 pairs x 2 digits (row 2*pair + digit); the min-term
// MFMA's A row i is pair 2(i>>2) + (i&1), so that accumulator rows 0 and 1 of
// a lane with group g are pairs 2g and 2g+1 in both (rows 2 and 3 repeat them
// and are not used).
//
// LDS: digit rows [pair][block][digit][16 chunks] with data chunk c of row
// r = 2*pair + digit stored at chunk c ^ r (the 16 lanes reading one chunk
// column of the 16 A rows hit 16 different bank groups), then the sums
// [block][pair][64 bytes].
#include "common.h"
#include "i8_ops.h"
#include "launch.h"

namespace ds4q {
namespace {

constexpr int GT = DECODE_TILE_M;
static_assert(GT == 8, "the A operand holds 8 pairs x 2 digits");

template <int NB>
struct GLayout {
  static constexpr int BPW = NB < 4 ? NB : 4;  // blocks per wave
  static constexpr int KS = NB / BPW;          // K parts
  static constexpr int DIG = GT * NB * QROW;   // digit rows
  static constexpr int SUM = GT * NB * XROW < 1024 ? 1024 : GT * NB * XROW;
  static constexpr int NDMA_S = SUM / 1024;    // 1-KiB direct loads of the sums
  static constexpr int PART = 8 * GT * 32 * 4;  // K parts of the eight waves
  static constexpr int BYTES = DIG + SUM > PART ? DIG + SUM : PART;
};

// Weight rows of one work item: 32 per wave over the waves that share a K part.
constexpr int rows_per_item(bool swiglu, int nb) { return 32 * 8 / ((swiglu ? 2 : 1) * (nb < 4 ? 1 : nb / 4)); }

// SWIGLU: W0 = gate, W1 = up, rows = n_ff, the A rows are the pairs' token
// rows (gathered through the sorted pair list); out = SwiGLU rows [pos][n_ff].
// Otherwise W0 = down, rows = n_embd, the A rows are the sorted positions;
// out = down rows [pos][n_embd].  Waves: w = (mat * RG + rg) * KS + kq.
template <bool SWIGLU, int NB>
__global__ __launch_bounds__(512, 4) void decode_grouped_kernel(
    const uint8_t *__restrict__ W0, const uint8_t *__restrict__ W1, int rows_per_expert,
    const uint8_t *__restrict__ aq, const uint8_t *__restrict__ ax, const float *__restrict__ asig,
    int kslots, int n_pairs, RouteBufs rb, int n_ntiles, float *__restrict__ out) {
  using L = GLayout<NB>;
  constexpr int BPW = L::BPW, KS = L::KS, NMAT = SWIGLU ? 2 : 1, RG = 8 / (NMAT * KS);
  constexpr int ROWS = RG * 32;  // weight rows per work item
  static_assert(NMAT * KS * RG == 8 && ROWS == rows_per_item(SWIGLU, NB), "eight waves");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::BYTES];
  __shared__ float sig_s[GT];

  // Work item: m-tile blockIdx.x / n_ntiles, n-tile blockIdx.x % n_ntiles
  // (a tile's activation rows are small, so keeping its n-tiles on one XCD
  // buys little; this mapping lets the tile and the live tile count be read
  // together).  Items past the live m-tiles exit at once.
  const int mtile = blockIdx.x / n_ntiles, ntile = blockIdx.x % n_ntiles;
  const int n_live = *rb.n_tiles;
  const int e = rb.tiles[2 * mtile], start = rb.tiles[2 * mtile + 1];  // in the array (grid bound)
  if (mtile >= n_live || e < 0) return;  // uniform; testing e keeps both loads ahead of the branch
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int kq = w % KS, rg = (w / KS) % RG, mat = w / (KS * RG);

  // the pair list entries of the tile (clamped into the list; entries past
  // the tile's end are never used)
  int pr = 0;
  if constexpr (SWIGLU) pr = rb.pairs[min(start + (lane & (GT - 1)), n_pairs - 1)];
  const int end = rb.offsets[e + 1];
  __builtin_amdgcn_sched_barrier(0);

  // all raw weight bytes of the wave: blocks kq*BPW .. +BPW-1 of rows
  // ntile*ROWS + rg*32 + 16t + n
  const int64_t rbytes = (int64_t)NB * BB_Q2K;
  const uint8_t *wm = mat ? W1 : W0;
  Q2KPart raw[BPW][2];
#pragma unroll
  for (int b = 0; b < BPW; ++b)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = ntile * ROWS + rg * 32 + 16 * t + n;
      raw[b][t].load(wm + ((int64_t)e * rows_per_expert + row) * rbytes + (int64_t)(kq * BPW + b) * BB_Q2K, g);
    }
  __builtin_amdgcn_sched_barrier(0);

  const int valid = min(end - start, GT);  // >= 1
  // source row of pair m (m < GT; pairs past the end repeat the last one)
  auto arow = [&](int m) {
    const int mm = min(m, valid - 1);
    if constexpr (SWIGLU) return __shfl(pr, mm, 64) / kslots;
    else return start + mm;
  };
  // Activation rows to LDS, every load 1 KiB (64 lanes x 16 bytes).  Digit
  // rows: wave w loads those of pair w (NB/2 loads), or with one block per
  // row waves 0..3 load pairs 2w and 2w+1; pairs that are absent are not
  // loaded.  Sums: wave w loads bytes [1024 w, 1024 w + 1024) of the sum
  // area (blocks 2w, 2w+1 of all pairs).  Each lane's source rows are found
  // before the first load, so the loads are straight-line code.
  const int lane_pair = NB >= 2 ? w : 2 * w + (lane >> 5);
  const int row_dig = arow(lane_pair);
  const int row_sum = arow((lane >> 2) & (GT - 1));
  // the row scales of the tile's pairs, requested with the activation rows
  // and kept in registers until the K parts meet
  const float sig_r = tid < GT ? asig[arow(tid)] : 0.f;
  {
    const int d = (lane >> 4) & 1, c = (lane & 15) ^ ((2 * lane_pair + d) & 15);
    const uint8_t *src = aq + (int64_t)row_dig * NB * QROW + (NB >= 2 ? (lane >> 5) * QROW : 0) + d * 256 + c * 16;
    if (NB >= 2 ? w < valid : (w < 4 && 2 * w < valid)) {
      uint8_t *dst = lds + (NB >= 2 ? w * NB * QROW : 1024 * w);
#pragma unroll
      for (int u = 0; u < (NB >= 2 ? NB / 2 : 1); ++u) dma16(src + u * 2 * QROW, dst + 1024 * u);
    }
    if (w < L::NDMA_S) {
      const int b = min(2 * w + (lane >> 5), NB - 1);
      dma16(ax + ((int64_t)row_sum * NB + b) * XROW + (lane & 3) * 16, lds + L::DIG + 1024 * w);
    }
  }
  // the wave's loads (weights and LDS) landed; the barrier publishes LDS
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  f32x4 acc[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
  const int aoff = (n >> 1) * NB * QROW + (n & 1) * 256;
  const int soff = L::DIG + (2 * (n >> 2) + (n & 1)) * XROW;
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
    const int kb = kq * BPW + b;
    i32x4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[j] = *reinterpret_cast<const i32x4 *>(lds + aoff + kb * QROW + (((4 * j + g) ^ n) << 4));
    const uint8_t *sp = lds + soff + kb * (GT * XROW);
    const bf16x8 xa = *reinterpret_cast<const bf16x8 *>(sp + (g & 1) * 32 + (g >> 1) * 16);
    const s16x4 xh = *reinterpret_cast<const s16x4 *>(sp + 8 * g);
    // the two subtiles' chains are independent: they are issued in pairs per
    // K tile (B fragments built just before), each pair a fenced MFMA group
    WTab tb[2];
    WMin<true> wm[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      raw[b][t].finish();
      tb[t].build(raw[b][t], g);
    }
    i32x4 c[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      i32x4 bj[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) bj[t] = tb[t].bfrag(raw[b][t], j);
      mfma_group_begin();
#pragma unroll
      for (int t = 0; t < 2; ++t)
        c[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], bj[t], j ? c[t] : (i32x4){0, 0, 0, 0}, 0, 0, 0);
      mfma_fence();
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) wm[t].build(raw[b][t], g);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[t][0] = fmaf(wm[t].dsc, (float)((c[t].x << 8) + c[t].y), acc[t][0]);
      acc[t][1] = fmaf(wm[t].dsc, (float)((c[t].z << 8) + c[t].w), acc[t][1]);
    }
    // the min-term MFMAs one at a time (their accumulators are assembled by
    // vector moves, which must not fall between two of them)
    mfma_fence();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wm[t].bmin, acc[t], 0, 0, 0);
      mfma_fence();
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xh, wm[t].bminlo, acc[t], 0, 0, 0);
      mfma_fence();
    }
  }

  // K parts: part[w][pair][32 rows] over the (no longer needed) digit rows
  __syncthreads();
  float *part = reinterpret_cast<float *>(lds);
  if (tid < GT) sig_s[tid] = sig_r;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    part[(w * GT + 2 * g) * 32 + 16 * t + n] = acc[t][0];
    part[(w * GT + 2 * g + 1) * 32 + 16 * t + n] = acc[t][1];
  }
  __syncthreads();
  for (int i = tid; i < GT * ROWS; i += 512) {
    const int m = i / ROWS, r = i % ROWS;
    if (m >= valid) break;  // i grows with m
    const int rgi = r / 32, rr = r % 32;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      v0 += part[(((0 * RG + rgi) * KS + q) * GT + m) * 32 + rr];
      if constexpr (SWIGLU) v1 += part[(((1 * RG + rgi) * KS + q) * GT + m) * 32 + rr];
    }
    const float sg = sig_s[m];
    const int64_t pos = start + m;
    const int row = ntile * ROWS + r;
    if constexpr (SWIGLU) out[pos * rows_per_expert + row] = silu(v0 * sg) * (v1 * sg);
    else out[pos * rows_per_expert + row] = v0 * sg;
  }
}


template <bool SWIGLU>
hipError_t launch_nb(int nb, const uint8_t *W0, const uint8_t *W1, int rows, const PrepI8 &a, int k,
                     int P, const RouteBufs &rb, int max_tiles, float *out, hipStream_t s) {
  const int nn = rows / rows_per_item(SWIGLU, nb);
  const dim3 grid((unsigned)max_tiles * nn);  // exactly: every item's m-tile is in the tile array
  const uint8_t *ax = reinterpret_cast<const uint8_t *>(a.x);
#define DS4Q_DG(NBV)                                                                                 \
  hipLaunchKernelGGL((decode_grouped_kernel<SWIGLU, NBV>), grid, dim3(512), 0, s, W0, W1, rows, a.q, \
                     ax, a.sig, k, P, rb, nn, out)
  switch (nb) {
    case 1: DS4Q_DG(1); break;
    case 2: DS4Q_DG(2); break;
    case 4: DS4Q_DG(4); break;
    case 8: DS4Q_DG(8); break;
    case 16: DS4Q_DG(16); break;
    default: return hipErrorInvalidValue;
  }
#undef DS4Q_DG
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_grouped(const MoeDims &m, const PrepI8 &a, int T, const RouteBufs &rb,
                                 int max_tiles, float *out, int phase, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T > 64) return hipErrorInvalidValue;
  const int P = T * m.k;
  if (phase == 1) return launch_nb<true>(m.D / 256, m.gate, m.up, m.F, a, m.k, P, rb, max_tiles, out, s);
  if (phase == 2) return launch_nb<false>(m.F / 256, m.down, nullptr, m.D, a, m.k, P, rb, max_tiles, out, s);
  return hipErrorInvalidValue;
}

}  // namespace ds4q

// Prefill path on Q2_K weights with int8 matrix cores.
//
// Arithmetic.  For one 256-value block of a weight row ("【#2】ds4.c 해독하기",
// Q2_K block-layout table) and an activation row a,
//   sum_v w_v a_v = d * sum_v (sc*q)_v a_v  -  dmin * sum_s mn_s A_s,
// A_s the sums of a over the 16 sub-blocks.  prep_i8_kernel prepares each
// activation row once per call (layer-input token rows, or the bf16 SwiGLU
// rows of the down projection): sigma = max|a| / 127 over the row,
// N = round(a / sigma * 256) split into balanced base-256 digits a0 (high)
// and a1 (low), both int8, so a = sigma * (a0 + a1/256) up to sigma/512;
// the sub-block sums A_s / sigma (of the unquantised row) are kept as two
// bf16 halves, hi + lo.
//
// prefill_i8_kernel: the integer part runs on v_mfma_i32_16x16x64_i8 with
// the 16 A rows = 8 tokens x 2 digits (row 2*token + digit) and B = the
// integer weights sc*q in 0..45 (v_perm of the byte table [0, sc, 2sc, 3sc]
// with the 2-bit codes); per block the two digit rows of a token combine
// exactly as 256*C0 + C1 and enter fp32 as d/256 * (256*C0 + C1).  The min
// term runs on v_mfma_f32_16x16x32_bf16 over K = 16 sub-blocks x {hi, lo}
// with B = bf16(-dmin * mn), accumulating straight into the same fp32
// registers; its 16 A rows are 16 tokens ordered so that each lane's four
// accumulator rows are the tokens of its integer results.  The epilogue
// scales by sigma (then SwiGLU, or the plain store of the down rows).
//
// Data movement: the activation tiles reach LDS by direct global->LDS loads
// (buffer_load_dwordx4 ... lds), double-buffered one 256-column block ahead;
// each 256-byte digit row is stored with its 16-byte chunks XOR-swizzled by
// the row index, so the 16 lanes that read one chunk column hit 16
// different bank groups.  Weights go straight to registers, also one block
// ahead.
#include "common.h"
#include "i8_ops.h"
#include "launch.h"

namespace ds4q {
namespace {

constexpr int TMI = PREFILL_TILE_M;  // tokens (sorted pairs) per m-tile
constexpr int SUBT = TMI / 8;        // integer MFMA row groups of 8 tokens
constexpr int NPAIR = SUBT / 2;      // min-term MFMA row groups of 16 tokens
constexpr int ASTAGE = TMI * QROW;   // LDS bytes of one stage of digit rows
constexpr int XSTAGE = 8 * 1024;       // one 1-KiB sum-row load per wave (16 tokens)
static_assert(TMI % 16 == 0 && TMI <= 128, "m-tile must be a multiple of 16, at most 128");

// One workgroup per activation row, one thread per 16-value sub-block.
// F32IN: the row is x * inv_rms (or x), rounded to bf16 first when ROUND
// (the prefill input contract), else taken as it is (decode: fp32 rows);
// otherwise the row is bf16 bits.  Output per (row, block):
// digits [digit][chunk c = 4j + g][dword k][byte] with byte i of dword k of
// chunk 4j+g the value 128(g>>1) + 32k + 16(g&1) + 4j + i (the B order
// above), hi/lo sums [2][16] bf16, and sigma per row.
template <bool F32IN, bool ROUND>
__global__ __launch_bounds__(256) void prep_i8_kernel(const void *__restrict__ src,
                                                      const float *__restrict__ inv_rms, int K,
                                                      uint8_t *__restrict__ aq,
                                                      uint16_t *__restrict__ ax,
                                                      float *__restrict__ asig) {
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nsub = K >> 4, nb = K >> 8;
  __shared__ float red[4];
  float v[16];
  float m = 0.f;
  const bool act = t < nsub;
  if (act) {
    if constexpr (F32IN) {
      const float s = inv_rms ? inv_rms[row] : 1.0f;
      const float4 *x = reinterpret_cast<const float4 *>(static_cast<const float *>(src) + row * K + 16 * t);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f = x[i];
        v[4 * i] = ROUND ? bf16_to_f32(bf16_rne_bits(f.x * s)) : f.x * s;
        v[4 * i + 1] = ROUND ? bf16_to_f32(bf16_rne_bits(f.y * s)) : f.y * s;
        v[4 * i + 2] = ROUND ? bf16_to_f32(bf16_rne_bits(f.z * s)) : f.z * s;
        v[4 * i + 3] = ROUND ? bf16_to_f32(bf16_rne_bits(f.w * s)) : f.w * s;
      }
    } else {
      const u32x4 *x = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(src) + row * K + 16 * t);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4 u = x[i];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v[8 * i + 2 * c] = bf16_to_f32(u[c] & 0xFFFFu);
          v[8 * i + 2 * c + 1] = bf16_to_f32(u[c] >> 16);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) red[w] = m;
  __syncthreads();
  const float mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = mx > 0.f ? 127.0f / mx : 0.0f;
  if (t == 0) asig[row] = mx * (1.0f / 127.0f);
  if (!act) return;
  const int b = t >> 4, s = t & 15;
  const int g = 2 * (s >> 3) + (s & 1), k = (s >> 1) & 3;
  uint32_t *qb = reinterpret_cast<uint32_t *>(aq + (row * nb + b) * QROW);
  const float scale = inv * 256.0f;
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // N + 32896 = 256 * (a0 + 128) + (a1 + 128), positive for |N| <= 32512
    uint32_t n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sum += v[4 * j + i];
      n[i] = (uint32_t)(int)fmaf(v[4 * j + i], scale, 32896.5f);
    }
    const uint32_t p01 = __builtin_amdgcn_perm(n[1], n[0], 0x05010400u);
    const uint32_t p23 = __builtin_amdgcn_perm(n[3], n[2], 0x05010400u);
    const int off = (4 * j + g) * 4 + k;
    qb[off] = __builtin_amdgcn_perm(p23, p01, 0x07060302u) ^ 0x80808080u;       // a0
    qb[64 + off] = __builtin_amdgcn_perm(p23, p01, 0x05040100u) ^ 0x80808080u;  // a1
  }
  const float xs = sum * inv;
  const uint32_t hi = bf16_rne_bits(xs);
  const uint32_t lo = bf16_rne_bits(xs - bf16_to_f32(hi));
  uint16_t *xr = ax + (row * nb + b) * (XROW / 2);
  xr[s] = (uint16_t)hi;
  xr[16 + s] = (uint16_t)lo;
}

// Per-wave state of one work item (set up once, shared by every block).
struct ItemCtx {
  const uint8_t *abase;         // uniform: digit rows of row rbase
  const uint8_t *xbase;         // uniform: sub-block sums of row rbase
  const int *arow;              // LDS: source row of each of the tile's TMI tokens
  int rbase;                    // 0 (gathered token rows) or the tile's first sorted row
  const uint8_t *brow[2];       // weight rows of the two n-subtiles (lane's row)
  int aoff[4];                  // LDS offsets of the lane's A chunks, K-tiles 0..3
  int xoff;                     // LDS offset of the lane's min-term chunk
  int nb, w, g, lane;           // w wave-uniform
};

// The block loop for NP live 16-token groups (tokens >= 16*NP are absent):
// acc[ip][t] += the products of blocks 0..nb-1.
template <int NP, int NPMAX>
__device__ __forceinline__ void block_loop(const ItemCtx &cx, uint8_t *As0, uint8_t *As1, uint8_t *Xs0,
                                           uint8_t *Xs1, f32x4 (&acc)[NPMAX][2]) {
  const int w = cx.w, g = cx.g, nb = cx.nb, lane = cx.lane;
  // Requests per block: waves 0..3 issue the 2*NP digit-row loads (load
  // I = 4u + w covers digit rows 4I..4I+3 = tokens 2I, 2I+1; lane -> row
  // 4I + lane/16, stored chunk lane%16 = data chunk (lane%16) ^ (row%16)),
  // so that the MFMAs of waves 4..7 on the same SIMDs run while they issue
  // (measured 3 % faster than eight waves issuing NP each); every wave
  // issues one sum-row load (tokens
  // 16(w % NP) + lane/4 into the wave's 1-KiB slot, so slot t/16 holds token
  // t at byte 64t; slots >= NP hold copies nobody reads), and the raw weight
  // bytes of its two n-subtiles.  Every wave's last requests of a block are
  // its four weight loads, so the block-end wait count is exact for both
  // kinds of wave.  Request offsets are relative to row rbase (gathered token
  // rows: < 2^29 bytes).  Blocks past the end are requested again as the
  // last block, so the loop has no branches.
  const int64_t rowq = (int64_t)nb * QROW, rowx = (int64_t)nb * XROW;
  uint32_t aoffs[2 * NP];
#pragma unroll
  for (int u = 0; u < 2 * NP; ++u) {
    const int I = 4 * u + (w & 3);
    const int r = 4 * I + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    aoffs[u] = (uint32_t)((cx.arow[r >> 1] - cx.rbase) * rowq) + (r & 1) * 256 + c * 16;
  }
  const int xtok = 16 * (w % NP) + (lane >> 2);
  const uint32_t xoffs = (uint32_t)((cx.arow[xtok] - cx.rbase) * rowx) + (lane & 3) * 16;

  const DmaSrc asrc(cx.abase), xsrc(cx.xbase);
  auto issue_a = [&](int u, int kb, uint8_t *As) {
    if (w < 4) asrc.copy16(aoffs[u], (uint32_t)kb * QROW, As + (4 * u + w) * 1024);
  };
  auto issue_x = [&](int kb, uint8_t *Xs) { xsrc.copy16(xoffs, (uint32_t)kb * XROW, Xs + w * 1024); };
  auto issue_tile = [&](int kb, uint8_t *As, uint8_t *Xs) {
    issue_x(kb, Xs);
#pragma unroll
    for (int u = 0; u < 2 * NP; ++u) issue_a(u, kb, As);
  };
  auto issue_w = [&](int kb, Q2KPart (&r)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) r[t].load(cx.brow[t] + (int64_t)kb * BB_Q2K, g);
  };

  // Weights run two blocks ahead (raw bytes of blocks kb+1 and kb+2 in
  // flight or landed during block kb, alternating between rw[0] and rw[1]);
  // the tile of kb+1 is requested before the weights of kb+2, so waiting
  // until only the last NWLD requests are outstanding means the tile landed.
  constexpr int NWLD = 4;  // weight load instructions per block: 2 x (16 + 8 bytes)
  Q2KPart rw[2][2];
  issue_tile(0, As0, Xs0);
  issue_w(0, rw[0]);
  issue_w(nb > 1 ? 1 : 0, rw[1]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  auto step = [&](int kb, Q2KPart (&r)[2], const uint8_t *As, const uint8_t *Xs, uint8_t *An,
                  uint8_t *Xn) {
    // the integer operands first; the min-term operand is built once the
    // first row group's integer MFMAs are issued (r is reloaded before then
    // when NP = 1, so its scale/min bytes and d|dmin are kept apart)
    WOps<false> wo[2];
    Q2KPart mp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      r[t].finish();
      wo[t].build_int(r[t], g);
      mp[t].s0 = r[t].s0;
      mp[t].s1 = r[t].s1;
      mp[t].dd = r[t].dd;
      asm volatile("" : "+v"(mp[t].s0), "+v"(mp[t].s1), "+v"(mp[t].dd));
    }
    // requests for later blocks, in this order: the sum rows and digit-row
    // load 0 before row group 0, digit-row load u before group u, and the
    // weights right after the last one.  SCHED_NOVMEM lets computation and
    // LDS accesses move across these points but no global request.
    const int kn = kb + 1 < nb ? kb + 1 : nb - 1, kw = kb + 2 < nb ? kb + 2 : nb - 1;
    issue_x(kn, Xn);
    // A fragments of row group i come from As + i*4096 + aoff[j]; the
    // next group's reads are issued before this group's MFMAs
    const uint8_t *ap[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ap[j] = As + cx.aoff[j];
    const uint8_t *xp = Xs + cx.xoff;
    i32x4 a[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[0][j] = *reinterpret_cast<const i32x4 *>(ap[j]);
#pragma unroll
    for (int ip = 0; ip < NP; ++ip) {
      __builtin_amdgcn_sched_barrier(SCHED_NOVMEM);
      issue_a(2 * ip, kn, An);
      issue_a(2 * ip + 1, kn, An);
      if (ip == NP - 1) {
        __builtin_amdgcn_sched_barrier(SCHED_NOVMEM);
        issue_w(kw, r);
      }
      __builtin_amdgcn_sched_barrier(SCHED_NOVMEM);
      const bf16x8 xa = *reinterpret_cast<const bf16x8 *>(xp + ip * 16 * XROW);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = 2 * ip + h;
        if (i + 1 < 2 * NP) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            a[(i + 1) & 1][j] = *reinterpret_cast<const i32x4 *>(ap[j] + (i + 1) * 4096);
        }
        // the two n-subtiles' chains, interleaved, as one fenced MFMA group
        i32x4 c[2];
        mfma_group_begin();
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            c[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i & 1][j], wo[t].b[j], j ? c[t] : (i32x4){0, 0, 0, 0}, 0, 0, 0);
        mfma_fence();
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc[ip][t][2 * h] = fmaf(wo[t].dsc, (float)((c[t].x << 8) + c[t].y), acc[ip][t][2 * h]);
          acc[ip][t][2 * h + 1] = fmaf(wo[t].dsc, (float)((c[t].z << 8) + c[t].w), acc[ip][t][2 * h + 1]);
        }
      }
      if (ip == 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) wo[t].build_min(mp[t], g);
      }
      mfma_group_begin();
#pragma unroll
      for (int t = 0; t < 2; ++t)
        acc[ip][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wo[t].bmin, acc[ip][t], 0, 0, 0);
      mfma_fence();
    }
    // Each wave waits for its own tile requests and LDS reads; then the
    // barrier alone publishes the tile (a workgroup fence would also wait
    // for the weight requests still in flight).  The scheduling barriers
    // keep the next block's operand build (which needs those weights) below
    // this point; the empty asm statements keep memory accesses in place.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0070 | NWLD);  // vmcnt(NWLD) lgkmcnt(0): tile of kb+1 landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // nb is a power of two; the loop body is exactly two blocks, so every path
  // into a block leaves the same requests outstanding
  if (nb == 1) {
    step(0, rw[0], As0, Xs0, As1, Xs1);
  } else {
    for (int kb = 0; kb < nb; kb += 2) {
      step(kb, rw[0], As0, Xs0, As1, Xs1);
      step(kb + 1, rw[1], As1, Xs1, As0, Xs0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no request outlives the loop
}

// SWIGLU: an n-tile is 128 rows of F; wave w owns rows 16w..16w+15 of both
// gate (t = 0) and up (t = 1).  Otherwise an n-tile is 256 down rows, wave w
// owning rows 32w + 16t .. +15.  Eight waves; m-tile = up to TMI sorted pairs
// of one expert, of which at most 16*NPMAX are present (the caller's bound).
// SwiGLU rows are written as bf16 (hb), down rows as fp32 (o).
template <bool SWIGLU, int NPMAX>
__global__ __launch_bounds__(512, 1) void prefill_i8_kernel(
    const uint8_t *__restrict__ W0, const uint8_t *__restrict__ W1, int K, int rows_per_expert,
    const uint8_t *__restrict__ aq, const uint16_t *__restrict__ ax, const float *__restrict__ asig,
    int gather_tokens, int kslots, RouteBufs rb, int n_ntiles, uint16_t *__restrict__ hb,
    uint16_t *__restrict__ o) {
  __shared__ __attribute__((aligned(1024))) uint8_t As0[ASTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[ASTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t Xs0[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t Xs1[XSTAGE];
  __shared__ int arow[TMI];

  int mtile, ntile;
  if (!xcd_tile_of(*rb.n_tiles, n_ntiles, &mtile, &ntile)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int e = rb.tiles_sz[2 * mtile], start = rb.tiles_sz[2 * mtile + 1];
  const int end = rb.offsets[e + 1];
  const int cap = 16 * NPMAX < TMI ? 16 * NPMAX : TMI;
  const int valid = end - start < cap ? end - start : cap;
  const int np = (valid + 15) >> 4;  // live 16-token groups

  if (tid < TMI) {
    const int m = tid < valid ? tid : 0;  // absent rows repeat row 0; never stored
    arow[tid] = gather_tokens ? rb.pairs[start + m] / kslots : start + m;
  }
  __syncthreads();

  ItemCtx cx;
  cx.nb = K >> 8;
  cx.w = __builtin_amdgcn_readfirstlane(w);
  cx.g = g;
  cx.lane = lane;
  cx.arow = arow;
  cx.rbase = gather_tokens ? 0 : start;
  cx.abase = aq + (int64_t)cx.rbase * cx.nb * QROW;
  cx.xbase = reinterpret_cast<const uint8_t *>(ax) + (int64_t)cx.rbase * cx.nb * XROW;
  const int64_t rbytes = (int64_t)cx.nb * BB_Q2K;
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
  // LDS read offsets: digit row 16i + n, data chunk 4j + g (stored at
  // (4j + g) ^ n); min-term row n of group ip = token
  // 16ip + 8((n&3)>>1) + 2(n>>2) + (n&1), chunk g = (half g&1, sub-blocks
  // 8(g>>1)..+7)
#pragma unroll
  for (int j = 0; j < 4; ++j) cx.aoff[j] = n * 256 + (((4 * j + g) ^ n) << 4);
  cx.xoff = (8 * ((n & 3) >> 1) + 2 * (n >> 2) + (n & 1)) * XROW + (g & 1) * 32 + (g >> 1) * 16;

  f32x4 acc[NPMAX][2];
#pragma unroll
  for (int ip = 0; ip < NPMAX; ++ip)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[ip][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  static_assert(NPMAX >= 1 && NPMAX <= NPAIR && NPAIR <= 8, "1..8 groups of 16 tokens");
  // np <= NPMAX: the number of live groups picks the instance (each case
  // exists when NPMAX allows it)
  switch (np) {
    case 1: block_loop<1, NPMAX>(cx, As0, As1, Xs0, Xs1, acc); break;
    case 2: if constexpr (NPMAX >= 2) block_loop<2, NPMAX>(cx, As0, As1, Xs0, Xs1, acc); break;
    case 3: if constexpr (NPMAX >= 3) block_loop<3, NPMAX>(cx, As0, As1, Xs0, Xs1, acc); break;
    case 4: if constexpr (NPMAX >= 4) block_loop<4, NPMAX>(cx, As0, As1, Xs0, Xs1, acc); break;
    case 5: if constexpr (NPMAX >= 5) block_loop<5, NPMAX>(cx, As0, As1, Xs0, Xs1, acc); break;
    case 6: if constexpr (NPMAX >= 6) block_loop<6, NPMAX>(cx, As0, As1, Xs0, Xs1, acc); break;
    case 7: if constexpr (NPMAX >= 7) block_loop<7, NPMAX>(cx, As0, As1, Xs0, Xs1, acc); break;
    default: if constexpr (NPMAX >= 8) block_loop<8, NPMAX>(cx, As0, As1, Xs0, Xs1, acc); break;
  }

  // epilogue: lane (g, n) holds, for group ip, rows q = 0..3 = tokens
  // 16ip + 8(q>>1) + 2g + (q&1) of weight row n of each n-subtile t
#pragma unroll
  for (int ip = 0; ip < NPMAX; ++ip) {
    if (ip >= np) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 16 * ip + 8 * (q >> 1) + 2 * g + (q & 1);
      if (m >= valid) continue;
      const float sg = asig[arow[m]];
      const int64_t pos = start + m;
      const float v0 = acc[ip][0][q] * sg, v1 = acc[ip][1][q] * sg;
      if constexpr (SWIGLU) {
        hb[pos * rows_per_expert + wrow[0]] = (uint16_t)bf16_rne_bits(silu(v0) * v1);
      } else {
        // wrow[1] = wrow[0] + 16; lanes n, n ^ 1 share g, hence m and validity
        store_bf16_row_pair(o + pos * rows_per_expert + wrow[0], n, v0, v1);
      }
    }
  }
}

}  // namespace

size_t prep_i8_bytes(int64_t rows, int K) {
  const size_t nb = (size_t)K / 256;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return up((size_t)rows * nb * QROW) + up((size_t)rows * nb * XROW) + up((size_t)rows * 4);
}

PrepI8 prep_i8_view(void *base, int64_t rows, int K) {
  const size_t nb = (size_t)K / 256;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  PrepI8 p;
  uint8_t *b = static_cast<uint8_t *>(base);
  p.q = b;
  p.x = reinterpret_cast<uint16_t *>(b + up((size_t)rows * nb * QROW));
  p.sig = reinterpret_cast<float *>(b + up((size_t)rows * nb * QROW) + up((size_t)rows * nb * XROW));
  return p;
}

hipError_t launch_prep_i8(const void *src, bool f32in, bool round_bf16, const float *inv_rms,
                          int64_t rows, int K, const PrepI8 &p, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (f32in && round_bf16)
    hipLaunchKernelGGL((prep_i8_kernel<true, true>), dim3((unsigned)rows), dim3(256), 0, s, src, inv_rms,
                       K, p.q, p.x, p.sig);
  else if (f32in)
    hipLaunchKernelGGL((prep_i8_kernel<true, false>), dim3((unsigned)rows), dim3(256), 0, s, src, inv_rms,
                       K, p.q, p.x, p.sig);
  else
    hipLaunchKernelGGL((prep_i8_kernel<false, false>), dim3((unsigned)rows), dim3(256), 0, s, src,
                       nullptr, K, p.q, p.x, p.sig);
  return hipGetLastError();
}

hipError_t launch_prefill_i8_gateup(const MoeDims &m, const PrepI8 &a, int T, const RouteBufs &rb,
                                    int max_tiles, uint16_t *hb, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nn = m.F / 128;
  hipLaunchKernelGGL((prefill_i8_kernel<true, NPAIR>), dim3(xcd_grid(max_tiles, nn)), dim3(512), 0, s, m.gate,
                     m.up, m.D, m.F, a.q, a.x, a.sig, 1, m.k, rb, nn, hb, nullptr);
  return hipGetLastError();
}

hipError_t launch_prefill_i8_down(const MoeDims &m, const PrepI8 &a, int T, const RouteBufs &rb,
                                  int max_tiles, uint16_t *o, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nn = m.D / 256;
  hipLaunchKernelGGL((prefill_i8_kernel<false, NPAIR>), dim3(xcd_grid(max_tiles, nn)), dim3(512), 0, s, m.down,
                     nullptr, m.F, m.D, a.q, a.x, a.sig, 0, m.k, rb, nn, nullptr, o);
  return hipGetLastError();
}

}  // namespace ds4q

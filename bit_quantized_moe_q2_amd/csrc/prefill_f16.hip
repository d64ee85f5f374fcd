// Prefill path (grouped GEMMs over expert-sorted token-expert pairs) with
// fp16 matrix cores, on Q2_K or Q4_1 weights per tensor.
//
// Arithmetic.  A weight of a 256-value Q2_K block ("【#2】ds4.c 해독하기",
// Q2_K block-layout table and code-packing expression) is
//   w = d * sc * q - dmin * mn,
// q the 2-bit code, sc / mn the 4-bit scale and min of its 16-value
// sub-block, d / dmin the block's fp16 fields.  For each sub-block the four
// possible weights (q = 0..3) are evaluated in fp32 (d*sc*q and dmin*mn are
// exact there, the difference rounds once) and rounded to fp16; each
// weight of the B operand is then one table lookup (v_perm_b32 on the lane's
// 2-bit codes).  A Q4_1 weight is d*q + m, one packed fp16 fma (OpsQ41).
// The activation rows are prepared once per call (prep_f16_kernel): each row
// is scaled by the power of two 2^k that puts its largest magnitude in
// [2^14, 2^15) and stored as fp16 (exact for bf16 input: 8 significant bits
// fit fp16's 11 down to 2^-17 of the scaled maximum, below which values round
// to fp16's subnormal grid), with 2^-k kept per row.  The products run on
// v_mfma_f32_16x16x32_f16 and accumulate over the whole K range in the
// matrix core's fp32 registers; the epilogue scales by 2^-k (then SwiGLU, or
// the plain store of the down rows).
//
// K order (Q2_K; Q4_1 at OpsQ41).  Any permutation of K serves as long as
// both operands use it.  Lane group g (lanes 16g..16g+15) of K-tile
// j = 2p + h of a block takes the 8 values 128(g>>1) + 32p + 16(g&1) + 8h + i,
// i = 0..7: code bytes 16g + 8h + i of the block's code area, bit pair p, all
// of sub-block 8(g>>1) + 2p + (g&1).  So a lane's 16 code bytes (one 16-byte
// load) cover K-tiles 0..7 of its weight row, and each of its four
// sub-blocks feeds exactly two K-tiles.  The prepared activation row holds,
// per block, 32 chunks of 16 bytes, chunk 4j + g = those 8 values of K-tile j
// as fp16.
//
// Data movement: activation tiles reach LDS by direct global->LDS loads
// (buffer_load_dwordx4 ... lds), double-buffered one block ahead, each
// 512-byte row with its 16-byte chunks XOR-swizzled by the row index within
// its 16-row group; raw weight bytes go to registers one block ahead.
#include <type_traits>

#include "common.h"
#include "i8_ops.h"
#include "launch.h"

namespace ds4q {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int TMF = PREFILL_TILE_M;  // tokens (sorted pairs) per m-tile
constexpr int NGF = TMF / 16;        // MFMA row groups of 16 tokens
constexpr int HROW = 512;            // fp16 bytes of one row's 256-value block
constexpr int HSTAGE = TMF * HROW;   // LDS bytes of one activation stage
// consecutive n-tiles of one m-tile per work item (fewer when the matrix has
// fewer): the next n-tile's first blocks are requested during the current
// one's last, so only an item's first n-tile waits for its start-up
constexpr int NTILES_PER_ITEM = 2;
static_assert(TMF % 16 == 0 && TMF <= 128, "m-tile must be a multiple of 16, at most 128");

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}

// One workgroup per activation row, one thread per 16 values.
// F32IN: the row is x * inv_rms (or x), rounded to bf16 first when ROUND
// (the prefill input contract); otherwise the row is bf16 bits.  Output per
// (row, 256-value block): 32 chunks [4j + g][8 fp16] in the K order of the
// weight format the row meets (Q41: the Q4_1 order, else the Q2_K one), and
// per row the factor 2^-k that undoes the scaling.
template <bool F32IN, bool ROUND, bool Q41>
__global__ __launch_bounds__(256) void prep_f16_kernel(const void *__restrict__ src,
                                                       const float *__restrict__ inv_rms, int K,
                                                       uint16_t *__restrict__ aq,
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
  // mx = f * 2^e with f in [0.5, 1): mx * 2^(15 - e) lies in [2^14, 2^15)
  int k = 0;
  if (mx > 0.f && mx <= 3.402823466e38f) k = 15 - __builtin_amdgcn_frexp_expf(mx);
  if (t == 0) asig[row] = ldexpf(1.0f, -k);
  if (!act) return;
  const int b = t >> 4, s = t & 15;
  if constexpr (Q41) {
    // values 16s..16s+15: the low (s even) or high nibbles of Q4_1 block
    // jb = s/2, code bytes 0..15; code dword cd goes to chunk
    // 4(4(jb&1) + cd) + jb/2, half s&1, in the order bytes 0, 2, 1, 3
    const int jb = s >> 1;
    u32x2 *out = reinterpret_cast<u32x2 *>(aq + (row * nb + b) * (HROW / 2));
#pragma unroll
    for (int cd = 0; cd < 4; ++cd) {
      const float *q = v + 4 * cd;
      out[2 * (4 * (4 * (jb & 1) + cd) + (jb >> 1)) + (s & 1)] =
          (u32x2){pack_f16x2(ldexpf(q[0], k), ldexpf(q[2], k)), pack_f16x2(ldexpf(q[1], k), ldexpf(q[3], k))};
    }
  } else {
    const int g = 2 * (s >> 3) + (s & 1), p = (s >> 1) & 3;
    u32x4 *out = reinterpret_cast<u32x4 *>(aq + (row * nb + b) * (HROW / 2));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 o;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        o[c] = pack_f16x2(ldexpf(v[8 * h + 2 * c], k), ldexpf(v[8 * h + 2 * c + 1], k));
      out[4 * (2 * p + h) + g] = o;
    }
  }
}

// The fp16 weight tables of one weight row's four sub-blocks in lane group
// g: sub-block p (bit pair p of the lane's code bytes) is
// 8(g>>1) + 2p + (g&1); lo[p] / hi[p] hold the low / high bytes of its
// weights for codes 0..3 (byte q = code q).
struct HTab {
  uint32_t lo[4], hi[4];
  // Tables of sub-block P from the block's scale/min bytes and d|dmin
  // (bytes 0 and 2 of a0 = sub-blocks 0 and 1, of a1 = 2 and 3).
  template <int P>
  __device__ __forceinline__ void build(uint32_t a0, uint32_t a1, float d, float dm) {
    const uint32_t byte = ((P < 2 ? a0 : a1) >> (16 * (P & 1))) & 0xFFu;
    const float ds = d * (float)(byte & 15u), mn = dm * (float)(byte >> 4);
    const uint32_t e01 = pack_f16x2(-mn, ds - mn);
    const uint32_t e23 = pack_f16x2(fmaf(2.0f, ds, -mn), fmaf(3.0f, ds, -mn));
    lo[P] = __builtin_amdgcn_perm(e23, e01, 0x06040200u);
    hi[P] = __builtin_amdgcn_perm(e23, e01, 0x07050301u);
  }
  // B fragment of K-tile j = 2p + h: the codes of bytes 8h..8h+7 (dwords
  // 2h, 2h+1 of q), bit pair p, looked up and interleaved into fp16 pairs.
  template <int J>
  __device__ __forceinline__ f16x8 bfrag(const u32x4 &q) const {
    constexpr int P = J >> 1, H = J & 1;
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t sel = (q[2 * H + c] >> (2 * P)) & 0x03030303u;
      const uint32_t l = __builtin_amdgcn_perm(0u, lo[P], sel), h = __builtin_amdgcn_perm(0u, hi[P], sel);
      o[2 * c] = __builtin_amdgcn_perm(h, l, 0x05010400u);
      o[2 * c + 1] = __builtin_amdgcn_perm(h, l, 0x07030602u);
    }
    return __builtin_bit_cast(f16x8, o);
  }
};

// Weight operands of one block of one weight row for lane group g, per
// format.  BYTES: the row bytes of one 256-value block; KEEP_RAW: the B
// fragments read the raw registers during the whole block (then the next
// block goes to a second set of raw registers).

// Q2_K: the code bytes are copied out and the scale/min bytes exchanged at
// the block's start (take), the raw registers are free after that.
struct OpsQ2K {
  using Raw = RawBlk;
  static constexpr int BYTES = BB_Q2K;
  static constexpr bool KEEP_RAW = false;
  u32x4 q;
  uint32_t sa0, sa1;
  float sd, sm;
  HTab tb;
  __device__ __forceinline__ void take(const Raw &r, int g) {
    const Q2KPart o = take_block(r);
    q = o.q;
    sa0 = o.s0 >> (8 * (g & 1));
    sa1 = o.s1 >> (8 * (g & 1));
    sd = f16lo(o.dd);
    sm = f16hi(o.dd);
    tb.template build<0>(sa0, sa1, sd, sm);
  }
  // before K-tile J's lookups: the tables of its sub-block when it is new
  template <int J>
  __device__ __forceinline__ void ahead() {
    if constexpr (J > 0 && (J & 1) == 0) tb.template build<(J >> 1)>(sa0, sa1, sd, sm);
  }
  template <int J>
  __device__ __forceinline__ f16x8 bfrag(const Raw &) const { return tb.template bfrag<J>(q); }
};

// Q4_1 ("자체 저비트 포맷을 llama.cpp로 옮기기", Q4_1 block section: fp16 d at
// byte 0, fp16 m at 2, code bytes 4..19 with value j the low nibble of byte
// j and value j + 16 its high nibble; value = d*code + m).  A 256-value block
// is 8 Q4_1 blocks, 160 bytes; lane group g loads its two whole Q4_1 blocks
// 2g and 2g + 1 (40 bytes at 40g: dwords 0 and 5 are their d|m, 1..4 and
// 6..9 their codes).  K order: K-tile j takes, in lane group g, code dword
// j & 3 of Q4_1 block 2g + (j >> 2): the low nibbles of its bytes 0, 2, 1, 3,
// then the high ones.  Each weight is q*d + m by one packed fp16 fma on the
// exact fp16 q (1024 + q - 1024): one rounding.
struct RawQ41 {
  u32x4 a, b;
  u32x2 c;
  __device__ __forceinline__ void load(const uint8_t *__restrict__ blk, int g) {
    const uint8_t *p = blk + 40 * g;
    a = *reinterpret_cast<const u32x4a *>(p);
    b = *reinterpret_cast<const u32x4a *>(p + 16);
    c = *reinterpret_cast<const u32x2a *>(p + 32);
  }
};
struct OpsQ41 {
  using Raw = RawQ41;
  static constexpr int BYTES = 8 * BB_Q41;
  static constexpr bool KEEP_RAW = true;
  h2 d2[2], m2[2];  // d and m of the lane's two Q4_1 blocks, in both halves
  __device__ __forceinline__ void take(const Raw &r, int) {
    d2[0] = __builtin_bit_cast(h2, __builtin_amdgcn_perm(r.a[0], r.a[0], 0x01000100u));
    m2[0] = __builtin_bit_cast(h2, __builtin_amdgcn_perm(r.a[0], r.a[0], 0x03020302u));
    d2[1] = __builtin_bit_cast(h2, __builtin_amdgcn_perm(r.b[1], r.b[1], 0x01000100u));
    m2[1] = __builtin_bit_cast(h2, __builtin_amdgcn_perm(r.b[1], r.b[1], 0x03020302u));
  }
  template <int J>
  __device__ __forceinline__ void ahead() {}
  // the nibble mask and the fp16 exponent bits of 1024 in registers (a
  // vector instruction cannot encode two literals), so that each code pair
  // is one v_and_or_b32
  uint32_t nib, magic;
  __device__ __forceinline__ OpsQ41() {
    asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(nib));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
  }
  template <int J>
  __device__ __forceinline__ f16x8 bfrag(const Raw &r) const {
    constexpr int JB = J >> 2, CD = J & 3;
    const uint32_t w = JB == 0 ? (CD == 0 ? r.a[1] : CD == 1 ? r.a[2] : CD == 2 ? r.a[3] : r.b[0])
                               : (CD == 0 ? r.b[2] : CD == 1 ? r.b[3] : CD == 2 ? r.c[0] : r.c[1]);
    const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // i = 0: low nibbles of bytes 0, 2; 1: of bytes 1, 3; 2, 3: the high nibbles
      const uint32_t sh = (i & 1) * 8 + (i >> 1) * 4;
      const h2 qv = __builtin_bit_cast(h2, ((w >> sh) & nib) | magic) - k1024;
      o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(qv, d2[JB], m2[JB]));
    }
    return __builtin_bit_cast(f16x8, o);
  }
};

// Per-wave state of one work item (set up once, shared by every block).
struct FCtx {
  const uint8_t *abase;    // uniform: prepared rows of row rbase
  const int *arow;         // LDS: source row of each of the tile's TMF tokens
  int rbase;               // 0 (gathered token rows) or the tile's first sorted row
  const uint8_t *brow[2];  // weight rows of the two n-subtiles (lane's row)
  int64_t nstride;         // bytes from a weight row to the same row of the next n-tile
  uint32_t aoff[4];        // LDS offsets of the lane's A chunks, K-tiles 0..3 (+256 for 4..7)
  int nb, nvt, w, g, lane; // nvt = blocks of all the item's n-tiles; w wave-uniform
};

// The block loop for NP live 16-token groups (tokens >= 16*NP are absent)
// over the item's n-tiles one after the other: nvt = n-tiles * nb blocks in
// one stream, v = nt * nb + kb; after the last block of n-tile nt, epi(nt)
// stores acc and acc restarts at zero.  The requests run one block ahead
// across n-tile boundaries (the activation rows are the same, the weight
// rows move by nstride), so only the item's first n-tile waits for its first
// blocks.  Each K-tile j has a vector
// phase (the A fragments of K-tile j + 1 from LDS, the lookups that build its
// B fragments) and a matrix phase (K-tile j's MFMAs as one fenced group).
// MFIRST (waves 4..7) runs the matrix phase first, the other waves the vector
// phase first: waves w and w + 4 share a SIMD, and after every block barrier
// they would otherwise be in the same phase, competing for the vector unit
// and then for the matrix core, instead of one using each.
template <class OPS, int NP, int NPMAX, bool MFIRST, class EPI>
__device__ __forceinline__ void block_loop_f16(const FCtx &cx, uint8_t *As0, uint8_t *As1,
                                               f32x4 (&acc)[NPMAX][2], const EPI &epi) {
  using Raw = typename OPS::Raw;
  constexpr int KR = OPS::KEEP_RAW ? 1 : 0;  // index of the second raw register set
  const int w = cx.w, g = cx.g, nb = cx.nb, nvt = cx.nvt, lane = cx.lane;
  // Activation requests per block: waves 0..3 issue the 2*NP row-pair loads
  // (load I = 4u + w covers token rows 2I, 2I+1; lane -> row 2I + lane/32,
  // stored chunk lane%32 = data chunk (lane%32) ^ (row%16)), so the MFMAs of
  // waves 4..7 on the same SIMDs run while they issue; every wave requests
  // the raw weight bytes of its two n-subtiles for the next block at the
  // start of a block, and the block ends waiting for all of its requests.
  // Offsets are relative to row rbase
  // (gathered token rows: < 2^29 bytes).  Blocks past the end are requested
  // again as the last block, so the loop has no branches.  Requests name
  // virtual blocks v.
  const int64_t rowq = (int64_t)nb * HROW;
  uint32_t aoffs[2 * NP];
#pragma unroll
  for (int u = 0; u < 2 * NP; ++u) {
    const int I = 4 * u + (w & 3);
    const int r = 2 * I + (lane >> 5);
    const int c = (lane & 31) ^ (r & 15);
    aoffs[u] = (uint32_t)((cx.arow[r] - cx.rbase) * rowq) + c * 16;
  }
  const DmaSrc asrc(cx.abase);
  auto issue_a = [&](int u, int v, uint8_t *As) {
    if (w < 4) asrc.copy16(aoffs[u], (uint32_t)(v % nb) * HROW, As + (4 * u + w) * 1024);
  };
  auto issue_w = [&](int v, Raw (&r)[2]) {
    const int64_t off = (int64_t)(v / nb) * cx.nstride + (int64_t)(v % nb) * OPS::BYTES;
#pragma unroll
    for (int t = 0; t < 2; ++t) r[t].load(cx.brow[t] + off, g);
  };

  // Raw weight registers: a block's bytes are taken apart at its start and
  // the next block's requested right after, a whole block ahead of their use,
  // into the same registers (Q2_K) or, when the lookups read them during the
  // block (Q4_1), into a second set.
  Raw rw[KR + 1][2];
#pragma unroll
  for (int u = 0; u < 2 * NP; ++u) issue_a(u, 0, As0);
  issue_w(0, rw[0]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  auto step = [&](int kb, Raw (&r)[2], Raw (&rn)[2], const uint8_t *As, uint8_t *An) {
    // this block's operands, then the next block's request (rn is r when the
    // raw registers are free after take)
    OPS op[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) op[t].take(r[t], g);
    const int kn = kb + 1 < nvt ? kb + 1 : nvt - 1;
    __builtin_amdgcn_sched_barrier(0);
    issue_w(kn, rn);
    __builtin_amdgcn_sched_barrier(0);
    // Per K-tile j: the requests of this step, then the two phases in the
    // wave's order; a sub-block's tables are built just before its first
    // K-tile's lookups.
    f16x8 a[2][NP], b[2][2];
#pragma unroll
    for (int i = 0; i < NP; ++i) a[0][i] = *reinterpret_cast<const f16x8 *>(As + cx.aoff[0] + i * 16 * HROW);
    b[0][0] = op[0].template bfrag<0>(r[0]);
    b[0][1] = op[1].template bfrag<0>(r[1]);
#define VPART(J)                                                                                  \
      if ((J) < 7) {                                                                              \
        constexpr int JN = ((J) + 1) & 7;                                                         \
        _Pragma("unroll") for (int i = 0; i < NP; ++i) a[((J) & 1) ^ 1][i] =                      \
            *reinterpret_cast<const f16x8 *>(As + cx.aoff[JN & 3] + (JN >> 2) * 256 + i * 16 * HROW); \
        op[0].template ahead<JN>();                                                               \
        op[1].template ahead<JN>();                                                               \
        b[((J) & 1) ^ 1][0] = op[0].template bfrag<JN>(r[0]);                                     \
        b[((J) & 1) ^ 1][1] = op[1].template bfrag<JN>(r[1]);                                     \
      }
#define MPART(J)                                                                                  \
      mfma_group_begin();                                                                         \
      _Pragma("unroll") for (int i = 0; i < NP; ++i) {                                            \
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[(J) & 1][i], b[(J) & 1][0], acc[i][0], 0, 0, 0); \
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[(J) & 1][i], b[(J) & 1][1], acc[i][1], 0, 0, 0); \
      }                                                                                           \
      mfma_fence();
#define DS4Q_F16_KTILE(J)                                                                         \
    {                                                                                             \
      constexpr int U0 = (2 * NP * (J)) / 8, U1 = (2 * NP * ((J) + 1)) / 8;                        \
      __builtin_amdgcn_sched_barrier(SCHED_NOVMEM);                                               \
      _Pragma("unroll") for (int u = U0; u < U1; ++u) issue_a(u, kn, An);                         \
      __builtin_amdgcn_sched_barrier(SCHED_NOVMEM);                                               \
      if constexpr (MFIRST) { MPART(J) VPART(J) } else { VPART(J) MPART(J) }                      \
    }
    DS4Q_F16_KTILE(0)
    DS4Q_F16_KTILE(1)
    DS4Q_F16_KTILE(2)
    DS4Q_F16_KTILE(3)
    DS4Q_F16_KTILE(4)
    DS4Q_F16_KTILE(5)
    DS4Q_F16_KTILE(6)
    DS4Q_F16_KTILE(7)
#undef DS4Q_F16_KTILE
#undef VPART
#undef MPART
    // Each wave waits for its own tile requests and LDS reads; then the
    // barrier alone publishes the tile (a workgroup fence would also wait
    // for the weight requests still in flight).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): tile and weights of kb+1 landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // after the last block of an n-tile: its results out, the sums restarted
  auto ntile_end = [&](int v) {
    if ((v + 1) % nb == 0) {
      mfma_fence();
      epi(v / nb);
#pragma unroll
      for (int i = 0; i < NP; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[i][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  };
  // nb is a power of two and nvt is 1 or even; the loop body is exactly two
  // blocks, so every path into a block leaves the same requests outstanding,
  // and with nb >= 2 an n-tile ends after the second of them
  if (nb == 1) {
    step(0, rw[0], rw[KR], As0, As1);
    ntile_end(0);
    if (nvt == 2) {
      step(1, rw[KR], rw[0], As1, As0);
      ntile_end(1);
    }
  } else {
    for (int v = 0; v < nvt; v += 2) {
      step(v, rw[0], rw[KR], As0, As1);
      step(v + 1, rw[KR], rw[0], As1, As0);
      ntile_end(v + 1);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no request outlives the loop
}

// SWIGLU: an n-tile is 128 rows of F; wave w owns rows 16w..16w+15 of both
// gate (t = 0) and up (t = 1).  Otherwise an n-tile is 256 down rows, wave w
// owning rows 32w + 16t .. +15.  Eight waves; a work item is an m-tile (up to
// TMF sorted pairs of one expert) and ntper consecutive n-tiles, run as one
// block stream.  SwiGLU rows are written as bf16 (hb), down rows as bf16 (o).
template <bool SWIGLU, bool Q41>
__global__ __launch_bounds__(512, 1) void prefill_f16_kernel(
    const uint8_t *__restrict__ W0, const uint8_t *__restrict__ W1, int K, int rows_per_expert,
    const uint16_t *__restrict__ aq, const float *__restrict__ asig, int gather_tokens, int kslots,
    RouteBufs rb, int n_groups, int ntper, uint16_t *__restrict__ hb, uint16_t *__restrict__ o) {
  using OPS = typename std::conditional<Q41, OpsQ41, OpsQ2K>::type;
  constexpr int NTROWS = SWIGLU ? 128 : 256;  // weight rows of one matrix per n-tile
  __shared__ __attribute__((aligned(1024))) uint8_t As0[HSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[HSTAGE];
  __shared__ int arow[TMF];
  __shared__ float asg[TMF];

  int mtile, ngrp;
  if (!xcd_tile_of(*rb.n_tiles, n_groups, &mtile, &ngrp)) return;
  const int ntile0 = ngrp * ntper;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int e = rb.tiles_sz[2 * mtile], start = rb.tiles_sz[2 * mtile + 1];
  const int end = rb.offsets[e + 1];
  const int valid = end - start < TMF ? end - start : TMF;
  const int np = (valid + 15) >> 4;  // live 16-token groups

  if (tid < TMF) {
    const int m = tid < valid ? tid : 0;  // absent rows repeat row 0; never stored
    const int r = gather_tokens ? rb.pairs[start + m] / kslots : start + m;
    arow[tid] = r;
    asg[tid] = asig[r];
  }
  __syncthreads();

  FCtx cx;
  cx.nb = K >> 8;
  cx.nvt = ntper * cx.nb;
  cx.w = __builtin_amdgcn_readfirstlane(w);
  cx.g = g;
  cx.lane = lane;
  cx.arow = arow;
  cx.rbase = gather_tokens ? 0 : start;
  cx.abase = reinterpret_cast<const uint8_t *>(aq) + (int64_t)cx.rbase * cx.nb * HROW;
  const int64_t rbytes = (int64_t)cx.nb * OPS::BYTES;
  cx.nstride = NTROWS * rbytes;
  int wrow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if constexpr (SWIGLU) {
      wrow[t] = ntile0 * 128 + 16 * w + n;
      cx.brow[t] = (t == 0 ? W0 : W1) + ((int64_t)e * rows_per_expert + wrow[t]) * rbytes;
    } else {
      wrow[t] = ntile0 * 256 + 32 * w + 16 * t + n;
      cx.brow[t] = W0 + ((int64_t)e * rows_per_expert + wrow[t]) * rbytes;
    }
  }
  // LDS read offsets: token row n of a 16-row group, data chunk 4j + g
  // stored at (4j + g) ^ n, i.e. byte (j << 6) ^ ((g ^ n) << 4) of the row;
  // K-tiles 4..7 add 256 to those of 0..3
#pragma unroll
  for (int j = 0; j < 4; ++j) cx.aoff[j] = n * HROW + (uint32_t)((j << 6) ^ ((g ^ n) << 4));

  f32x4 acc[NGF][2];
#pragma unroll
  for (int i = 0; i < NGF; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[i][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // n-tile nt of the item done: lane (g, n) holds, for group i, rows
  // q = 0..3 = tokens 16i + 4g + q of weight row n of each n-subtile t
  // (the caller has fenced the last MFMAs)
  // Stores go through the uniform row base of the tile and 32-bit per-lane
  // offsets (fewer live registers inside the block loop).
  uint16_t *const obase = (SWIGLU ? hb : o) + (int64_t)start * rows_per_expert;
  auto epi = [&](int nt) {
    const uint32_t r0 = (uint32_t)(wrow[0] + nt * NTROWS);
#pragma unroll
    for (int i = 0; i < NGF; ++i) {
      if (i >= np) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = 16 * i + 4 * g + q;
        if (m >= valid) continue;
        const float sg = asg[m];
        const uint32_t off = (uint32_t)m * (uint32_t)rows_per_expert + r0;
        const float v0 = acc[i][0][q] * sg, v1 = acc[i][1][q] * sg;
        if constexpr (SWIGLU) {
          // silu(v0) * v1 with a hardware reciprocal: the result is rounded to bf16
          const float sl = v0 * __builtin_amdgcn_rcpf(1.0f + __expf(-v0));
          obase[off] = (uint16_t)bf16_rne_bits(sl * v1);
        } else {
          // the second subtile's row is r0 + 16; lanes n, n ^ 1 share g, hence m and validity
          store_bf16_row_pair(obase + off, n, v0, v1);
        }
      }
    }
  };

  if (cx.w >= 4) {
    switch (np) {
      case 1: block_loop_f16<OPS, 1, NGF, true>(cx, As0, As1, acc, epi); break;
      case 2: block_loop_f16<OPS, 2, NGF, true>(cx, As0, As1, acc, epi); break;
      case 3: block_loop_f16<OPS, 3, NGF, true>(cx, As0, As1, acc, epi); break;
      case 4: block_loop_f16<OPS, 4, NGF, true>(cx, As0, As1, acc, epi); break;
      case 5: block_loop_f16<OPS, 5, NGF, true>(cx, As0, As1, acc, epi); break;
      case 6: block_loop_f16<OPS, 6, NGF, true>(cx, As0, As1, acc, epi); break;
      case 7: block_loop_f16<OPS, 7, NGF, true>(cx, As0, As1, acc, epi); break;
      default: block_loop_f16<OPS, 8, NGF, true>(cx, As0, As1, acc, epi); break;
    }
  } else {
    switch (np) {
      case 1: block_loop_f16<OPS, 1, NGF, false>(cx, As0, As1, acc, epi); break;
      case 2: block_loop_f16<OPS, 2, NGF, false>(cx, As0, As1, acc, epi); break;
      case 3: block_loop_f16<OPS, 3, NGF, false>(cx, As0, As1, acc, epi); break;
      case 4: block_loop_f16<OPS, 4, NGF, false>(cx, As0, As1, acc, epi); break;
      case 5: block_loop_f16<OPS, 5, NGF, false>(cx, As0, As1, acc, epi); break;
      case 6: block_loop_f16<OPS, 6, NGF, false>(cx, As0, As1, acc, epi); break;
      case 7: block_loop_f16<OPS, 7, NGF, false>(cx, As0, As1, acc, epi); break;
      default: block_loop_f16<OPS, 8, NGF, false>(cx, As0, As1, acc, epi); break;
    }
  }
}

}  // namespace

size_t prep_f16_bytes(int64_t rows, int K) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return up((size_t)rows * K * 2) + up((size_t)rows * 4);
}

PrepF16 prep_f16_view(void *base, int64_t rows, int K) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  PrepF16 p;
  uint8_t *b = static_cast<uint8_t *>(base);
  p.q = reinterpret_cast<uint16_t *>(b);
  p.sig = reinterpret_cast<float *>(b + up((size_t)rows * K * 2));
  return p;
}

hipError_t launch_prep_f16(const void *src, bool f32in, bool round_bf16, const float *inv_rms,
                           int64_t rows, int K, int wtype, const PrepF16 &p, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const bool q41 = wtype == TYPE_Q4_1;
  const dim3 grid((unsigned)rows), block(256);
  if (f32in && round_bf16) {
    if (q41) hipLaunchKernelGGL((prep_f16_kernel<true, true, true>), grid, block, 0, s, src, inv_rms, K, p.q, p.sig);
    else hipLaunchKernelGGL((prep_f16_kernel<true, true, false>), grid, block, 0, s, src, inv_rms, K, p.q, p.sig);
  } else if (f32in) {
    if (q41) hipLaunchKernelGGL((prep_f16_kernel<true, false, true>), grid, block, 0, s, src, inv_rms, K, p.q, p.sig);
    else hipLaunchKernelGGL((prep_f16_kernel<true, false, false>), grid, block, 0, s, src, inv_rms, K, p.q, p.sig);
  } else {
    if (q41) hipLaunchKernelGGL((prep_f16_kernel<false, false, true>), grid, block, 0, s, src, nullptr, K, p.q, p.sig);
    else hipLaunchKernelGGL((prep_f16_kernel<false, false, false>), grid, block, 0, s, src, nullptr, K, p.q, p.sig);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_f16_gateup(const MoeDims &m, const PrepF16 &a, int T, const RouteBufs &rb,
                                     int max_tiles, uint16_t *hb, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nn = m.F / 128, per = nn >= NTILES_PER_ITEM ? NTILES_PER_ITEM : nn;
  const dim3 grid(xcd_grid(max_tiles, nn / per)), block(512);
  if (m.tg == TYPE_Q4_1)
    hipLaunchKernelGGL((prefill_f16_kernel<true, true>), grid, block, 0, s, m.gate, m.up, m.D, m.F, a.q, a.sig,
                       1, m.k, rb, nn / per, per, hb, nullptr);
  else
    hipLaunchKernelGGL((prefill_f16_kernel<true, false>), grid, block, 0, s, m.gate, m.up, m.D, m.F, a.q, a.sig,
                       1, m.k, rb, nn / per, per, hb, nullptr);
  return hipGetLastError();
}

hipError_t launch_prefill_f16_down(const MoeDims &m, const PrepF16 &a, int T, const RouteBufs &rb,
                                   int max_tiles, uint16_t *o, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nn = m.D / 256, per = nn >= NTILES_PER_ITEM ? NTILES_PER_ITEM : nn;
  const dim3 grid(xcd_grid(max_tiles, nn / per)), block(512);
  if (m.td == TYPE_Q4_1)
    hipLaunchKernelGGL((prefill_f16_kernel<false, true>), grid, block, 0, s, m.down, nullptr, m.F, m.D, a.q,
                       a.sig, 0, m.k, rb, nn / per, per, nullptr, o);
  else
    hipLaunchKernelGGL((prefill_f16_kernel<false, false>), grid, block, 0, s, m.down, nullptr, m.F, m.D, a.q,
                       a.sig, 0, m.k, rb, nn / per, per, nullptr, o);
  return hipGetLastError();
}

}  // namespace ds4q

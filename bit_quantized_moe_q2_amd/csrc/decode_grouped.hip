// Decode of 2..64 tokens on Q2_K or Q4_1 weights: expert-grouped, streaming.
//
// At decode sizes an expert holds a few of the call's token-expert pairs,
// so the work is the weight stream of the routed experts ("【#2】ds4.c
// 해독하기": only the routed experts' bytes move per token).  A work item is an
// m-tile of at most DECODE_TILE_M (4) sorted pairs of one expert and an
// n-tile of weight rows; each of the eight waves owns 16 weight rows over a
// quarter or half of K (four 256-value blocks).  The workgroups are
// persistent and stream the next item's weights while computing the current
// one (see decode_grouped_kernel).
//
// Arithmetic.  For one block of a weight row ("【#2】ds4.c 해독하기", Q2_K
// block-layout table) and an activation row a,
//   sum_v w_v a_v = d * sum_v (sc*q)_v a_v  -  dmin * sum_s mn_s A_s,
// A_s the sums of a over the 16 sub-blocks.  Each activation row is prepared
// once per call (prep_d3_kernel): sigma = max|a| / 127 over the row and
// N = round(a / sigma * 65536) as three balanced base-256 digits a0 (high),
// a1, a2, all int8, so a = sigma * (a0 + a1/256 + a2/65536) up to
// sigma/131072 (2^-24 of the row maximum).  On v_mfma_i32_16x16x64_i8 the 16
// A rows are the 4 pairs x 4 (three digits and an unused row: row
// 4*pair + digit), so each lane's four accumulator rows are one pair's
// digits.  Two B operands per block: the integer weights sc*q in 0..45
// (v_perm of the byte table [0, sc, 2sc, 3sc] with the 2-bit codes), and the
// min nibble of each value's sub-block (min_bfrag), whose MFMAs sum to
// sum_s mn_s A_s; both sums are exact in int32 and meet d and dmin in fp32.
// A Q4_1 block (ThakiCloud "...GGUF Q4_1 재부호화", Q4_1 block section: 32
// values, y = d*q + m) gives d * sum q a + m * sum a: the integer sums on
// the same MFMA (see the kernel), the sums of a prepared with the digits.
//
// LDS: the digit rows (GLayout), then the K parts, then (Q4_1) the m-tile's
// sums of 32 values.
#include <type_traits>

#include "common.h"
#include "i8_ops.h"
#include "launch.h"

namespace ds4q {
namespace {

constexpr int GT = DECODE_TILE_M;
static_assert(GT == 4, "the A operand holds 4 pairs x 4 rows");
constexpr int QROW3 = 768;  // digit bytes of one row's 256-column block (3 digits)

// One workgroup per activation row, one thread per 16-value sub-block: the
// row (times inv_rms[row] when given) as three digit rows per 256-value block
// in the B order of the weights, and sigma.  Q2_K order: byte i of dword k of
// chunk 4j+g is value 128(g>>1) + 32k + 16(g&1) + 4j + i.  Q4_1 order (K tile
// j holds the 32-value blocks 2j and 2j+1, lane group g half g&1 of block
// 2j + (g>>1): the low nibbles of its 8 code bytes, then the high ones):
// value 64j + 32(g>>1) + 16(k>>1) + 8(g&1) + 4(k&1) + i; with it, the sum of
// each 32 values over sigma.
template <bool Q41>
__global__ __launch_bounds__(256) void prep_d3_kernel(const float *__restrict__ src,
                                                      const float *__restrict__ inv_rms, int K,
                                                      uint8_t *__restrict__ aq, float *__restrict__ asig,
                                                      float *__restrict__ axs) {
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nsub = K >> 4, nb = K >> 8;
  __shared__ float red[4];
  float v[16];
  float m = 0.f;
  const bool act = t < nsub;
  if (act) {
    const float sc = inv_rms ? inv_rms[row] : 1.0f;
    const float4 *x = reinterpret_cast<const float4 *>(src + row * K + 16 * t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = x[i];
      v[4 * i] = f.x * sc;
      v[4 * i + 1] = f.y * sc;
      v[4 * i + 2] = f.z * sc;
      v[4 * i + 3] = f.w * sc;
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
  if constexpr (Q41) {
    // threads t and t ^ 1 hold the two halves of 32-value block t / 2
    float sm = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sm += v[i];
    sm += __shfl_xor(sm, 1, 64);
    if ((t & 1) == 0) axs[row * (K >> 5) + (t >> 1)] = sm * inv;
  }
  uint32_t *qb = reinterpret_cast<uint32_t *>(aq + (row * nb + b) * QROW3);
  const float scale = inv * 65536.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // N + 0x808080 = 65536 (a0 + 128) + 256 (a1 + 128) + (a2 + 128), in
    // [0, 2^24) for |N| <= 127 * 65536 (an integer-valued float there)
    uint32_t n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) n[i] = (uint32_t)__builtin_rintf(fmaf(v[4 * j + i], scale, 8421504.0f));
    const uint32_t p01 = __builtin_amdgcn_perm(n[1], n[0], 0x05010400u);  // bytes 0, 1
    const uint32_t p23 = __builtin_amdgcn_perm(n[3], n[2], 0x05010400u);
    const uint32_t q01 = __builtin_amdgcn_perm(n[1], n[0], 0x0C0C0602u);  // byte 2
    const uint32_t q23 = __builtin_amdgcn_perm(n[3], n[2], 0x0C0C0602u);
    // values 16s + 4j .. +3 of the block
    int off;
    if constexpr (Q41) off = (4 * (s >> 2) + 2 * ((s >> 1) & 1) + (j >> 1)) * 4 + 2 * (s & 1) + (j & 1);
    else off = (4 * j + 2 * (s >> 3) + (s & 1)) * 4 + ((s >> 1) & 3);
    qb[off] = __builtin_amdgcn_perm(q23, q01, 0x05040100u) ^ 0x80808080u;        // a0
    qb[64 + off] = __builtin_amdgcn_perm(p23, p01, 0x07060302u) ^ 0x80808080u;   // a1
    qb[128 + off] = __builtin_amdgcn_perm(p23, p01, 0x05040100u) ^ 0x80808080u;  // a2
  }
}

// Eight waves of at most four blocks each, two workgroups per CU.  (Four
// waves of up to eight blocks, three workgroups per CU, hold half as many
// weight bytes in flight again and measured the same for the down rows and
// slower for gate/up: the weight stream of this access pattern runs at the
// same rate either way.)
constexpr int NWV = 8;   // waves per workgroup
constexpr int BPWM = 4;  // blocks of K per wave at most
constexpr int WG_PER_CU = 2;

// LDS digit rows: 12 rows (4 * digit + pair) of NB * 256 bytes.  With four
// or more blocks a row is followed by 16 bytes of padding (row stride
// NB*256 + 16), so the lanes reading one 16-byte chunk column of the 12 rows
// hit 12 different bank groups and a lane's reads are one base address plus
// immediate offsets; with fewer blocks the rows are packed and the chunks of
// row r are XOR-swizzled by r instead.
template <int NB, bool Q41>
struct GLayout {
  static constexpr int BPW = NB < BPWM ? NB : BPWM;  // blocks per wave
  static constexpr int KS = NB / BPW;           // K parts
  static constexpr bool PAD = NB >= 4;
  static constexpr int RSTRIDE = NB * 256 + (PAD ? 16 : 0);
  static constexpr int DIG = 12 * RSTRIDE;      // digit rows
  static constexpr int NDMA = 12 * NB / 4;      // 1-KiB direct loads of the digit rows
  static constexpr int PART = NWV * 64 * 4;     // K parts of the waves (a float per lane)
  // Q4_1: the 4 pairs' sums of 32 values (NB * 8 floats each), brought in by
  // NXD direct loads of 1 KiB
  static constexpr int NXD = Q41 ? (NB * 128 + 1023) / 1024 : 0;
  static constexpr int XB = 1024 * NXD;
  static constexpr int BYTES = DIG + PART + XB;
  static constexpr int CHUNK = Q41 ? 8 * BB_Q41 : BB_Q2K;  // weight bytes per 256 values of a row
};

// Weight rows of one work item: 16 per wave over the waves that share a K part.
constexpr int rows_per_item(bool swiglu, int nb) {
  return 16 * NWV / ((swiglu ? 2 : 1) * (nb < BPWM ? 1 : nb / BPWM));
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) i32x2 *const_i32x2_ptr;

// Barrier for LDS only: the workgroup's LDS accesses so far are complete;
// global loads in flight stay in flight (a full __syncthreads would wait for
// them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Barrier after every load of the wave has landed (direct loads to LDS
// included).
__device__ __forceinline__ void full_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x3g __attribute__((ext_vector_type(3), aligned(4)));

// Raw bytes of one Q4_1 chunk (256 values = 8 blocks of one row) for lane
// group g: per K tile j, 12 bytes of block 2j + (g>>1) at offset 8(g&1) (the
// even group: d|m and code bytes 0..7; the odd one: code bytes 4..15, of
// which 8..15 are its own).
struct RawQ41 {
  u32x3 v[4];
  __device__ __forceinline__ void load(const uint8_t *__restrict__ chunk, int g) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = *reinterpret_cast<const u32x3g *>(chunk + (2 * j + (g >> 1)) * BB_Q41 + 8 * (g & 1));
  }
};

// Integer B fragment of the min term: dword k is the min nibble of the
// lane's sub-block for bit pair k (the sub-block of that dword in every
// K-tile's code fragment) in all four bytes, so the K-tiles' MFMAs against
// the digit rows sum to sum_s mn_s A_s exactly.  sel_lo / sel_hi replicate
// byte p / 2 + p (p = g & 1) of a dword.
__device__ __forceinline__ i32x4 min_bfrag(const Q2KPart &r, uint32_t sel_lo, uint32_t sel_hi) {
  const uint32_t m0 = (r.s0 >> 4) & 0x0F0F0F0Fu, m1 = (r.s1 >> 4) & 0x0F0F0F0Fu;
  i32x4 b;
  b.x = (int)__builtin_amdgcn_perm(0u, m0, sel_lo);
  b.y = (int)__builtin_amdgcn_perm(0u, m0, sel_hi);
  b.z = (int)__builtin_amdgcn_perm(0u, m1, sel_lo);
  b.w = (int)__builtin_amdgcn_perm(0u, m1, sel_hi);
  return b;
}

// The three digit sums of a pair as one value in units of the high digit:
// C0 + C1/256 + C2/65536 (C0*256 + C1 is exact in int32).
__device__ __forceinline__ float digits3(i32x4 c) {
  return fmaf((float)c.z, 1.0f / 65536.0f, (float)((c.x << 8) + c.y) * (1.0f / 256.0f));
}

// Q4_1 (Q41): per K tile the lane's 8 code bytes give the B operand (low
// nibbles, then high nibbles, in the prepared activation order), once masked
// to lane groups 0-1 (block 2j) and once to groups 2-3 (block 2j+1), so the
// two MFMAs sum each 32-value block on its own; lane (g, n) then holds both
// blocks' sums for pair g and weight row n and takes both blocks' (d, m) by
// two lane exchanges: sum w a = d * sum q a + m * sum a, the last from the
// prepared sums of 32 values.
//
// SWIGLU: W0 = gate, W1 = up, rows = n_ff, the A rows are the pairs' token
// rows (gathered through the sorted pair list); out = SwiGLU rows [pos][n_ff].
// Otherwise W0 = down, rows = n_embd, the A rows are the sorted positions;
// out = down rows [pos][n_embd].  Waves: w = (mat * RG + rg) * KS + kq; a
// wave owns 16 weight rows over BPW blocks of K.
//
// Persistent, WG_PER_CU workgroups per CU: workgroup i takes the contiguous run of
// work items [i n / G, (i + 1) n / G) (item = m-tile * n_ntiles + n-tile, n
// counted on the device), so consecutive items mostly share their m-tile and
// its digit rows stay in LDS.  The next item's weights stream in while the
// current one is computed: once a block's MFMAs are issued, the registers
// that held its raw bytes receive the same block of the next item.
// Barriers wait for LDS only, so those loads stay in flight across them.
// When the m-tile changes, the new digit rows are requested once the old
// ones are no longer read, and waited for then.  An item's outputs are
// stored once the next item has started, so no wait covers their completion.
template <bool SWIGLU, int NB, bool Q41>
__global__ __launch_bounds__(64 * NWV, WG_PER_CU) void decode_grouped_kernel(
    const uint8_t *__restrict__ W0, const uint8_t *__restrict__ W1, int rows_per_expert,
    const uint8_t *__restrict__ aq, const float *__restrict__ asig, const float *__restrict__ axs, int kslots,
    int n_pairs, RouteBufs rb, int n_ntiles, float *__restrict__ out) {
  using L = GLayout<NB, Q41>;
  constexpr int BPW = L::BPW, KS = L::KS, NMAT = SWIGLU ? 2 : 1, RG = NWV / (NMAT * KS);
  constexpr int ROWS = RG * 16;  // weight rows per work item
  static_assert(NMAT * KS * RG == NWV && ROWS == rows_per_item(SWIGLU, NB), "waves");
  static_assert(GT * ROWS <= 64 * NWV, "one output per thread and item");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::BYTES];
  __shared__ float sig_s[GT];

  const int n_items = *rb.n_tiles * n_ntiles;
  const int G = gridDim.x;
  int item = (int)((int64_t)blockIdx.x * n_items / G);
  const int item_end = (int)((int64_t)(blockIdx.x + 1) * n_items / G);
  if (item >= item_end) return;  // uniform
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int kq = w % KS, rg = (w / KS) % RG, mat = w / (KS * RG);
  const int64_t rbytes = (int64_t)NB * L::CHUNK;
  const uint8_t *wm = mat ? W1 : W0;
  const uint32_t sel_lo = (g & 1) ? 0x01010101u : 0x00000000u;
  const uint32_t sel_hi = (g & 1) ? 0x03030303u : 0x02020202u;
  const uint32_t mask_e = g < 2 ? 0x0F0F0F0Fu : 0u, mask_o = mask_e ^ 0x0F0F0F0Fu;  // Q4_1 code masks

  // m-tile context: expert, first sorted position, pairs present (>= 1), the
  // lane's pair-list entry (SWIGLU; entries past the tile's end are never
  // used) and the row scale of pair tid (tid < GT).  The tile entry is read
  // through the scalar cache (uniform); the pair count and list entry are
  // requested early and taken (tile_take) when they are needed.
  struct MTile {
    int e, start, valid, pr;
    float sig;
  };
  auto tile_head = [&](int mt, MTile &c) {
    const i32x2 v = *((const_i32x2_ptr)(const void *)rb.tiles + mt);
    c.e = v.x;
    c.start = v.y;
  };
  auto tile_rest = [&](MTile &c) {
    c.valid = *((const __attribute__((address_space(4))) int *)(const void *)rb.offsets + c.e + 1);
    c.pr = 0;
    if constexpr (SWIGLU) c.pr = rb.pairs[min(c.start + (lane & (GT - 1)), n_pairs - 1)];
  };
  auto tile_take = [&](MTile &c) { c.valid = min(c.valid - c.start, GT); };
  // source row of pair m (m < GT; pairs past the end repeat the last one)
  auto arow = [&](const MTile &c, int m) {
    const int mm = min(m, c.valid - 1);
    if constexpr (SWIGLU) return __shfl(c.pr, mm, 64) / kslots;
    else return c.start + mm;
  };
  // raw bytes of block b of the wave's K part: row nt*ROWS + rg*16 + n
  using Raw = typename std::conditional<Q41, RawQ41, RawBlk>::type;
  auto load_block = [&](int e, int nt, int b, Raw &r) {
    const int row = nt * ROWS + rg * 16 + n;
    r.load(wm + ((int64_t)e * rows_per_expert + row) * rbytes + (int64_t)(kq * BPW + b) * L::CHUNK, g);
  };
  // Digit rows of an m-tile to LDS as NDMA direct loads of 1 KiB (64 lanes
  // x 16 bytes), load u by wave u % NWV.  With four or more blocks a load
  // holds four blocks of one (digit, pair) row, and loads of absent pairs
  // are skipped.  The row scales go to registers until the K parts meet.
  const DmaSrc qsrc(aq), xssrc(axs);
  auto issue_act = [&](MTile &c) {
    const int src_row = arow(c, lane & 3);  // source row of pair lane & 3
#pragma unroll
    for (int u0 = 0; u0 < L::NDMA; u0 += NWV) {
      int u = u0 + w;
      asm volatile("" : "+s"(u));  // the slot arithmetic below stays here (not hoisted out of the loop)
      if (u < L::NDMA) {
        if constexpr (L::PAD) {
          const int rix = u / (NB / 4), pair = rix & 3, d = rix >> 2;  // uniform
          const int blk = 4 * (u % (NB / 4)) + (lane >> 4);
          if (pair < c.valid)
            qsrc.copy16(blk * QROW3 + d * 256 + (lane & 15) * 16,
                        (uint32_t)__builtin_amdgcn_readlane(src_row, pair) * (NB * QROW3),
                        lds + rix * L::RSTRIDE + (u % (NB / 4)) * 1024);
        } else {
          const int sl = 64 * u + lane;    // 16-byte slot
          const int rix = sl / (NB * 16);  // 4 * digit + pair
          const int pair = rix & 3, d = rix >> 2;
          const int blk = (sl >> 4) & (NB - 1), pos = sl & 15;
          qsrc.copy16((uint32_t)__shfl(src_row, pair, 64) * (NB * QROW3) +
                          (blk * QROW3 + d * 256 + ((pos ^ (4 * pair + d)) << 4)),
                      0, lds + 1024 * u);
        }
      }
    }
    if constexpr (Q41) {
      // the sums of 32 values: byte o of the area is pair o / (NB*32)'s
      // byte o % (NB*32); lanes past the area re-read pair 0 (never used)
      for (int u = w; u < L::NXD; u += NWV) {
        const int o = 1024 * u + 16 * lane;
        const bool in = o < NB * 128;
        const int pair = in ? o / (NB * 32) : 0, off = in ? o % (NB * 32) : 0;
        xssrc.copy16((uint32_t)arow(c, pair) * (NB * 32) + off, 0, lds + L::DIG + L::PART + 1024 * u);
      }
    }
    c.sig = tid < GT ? asig[arow(c, tid)] : 0.f;
  };

  int mt = item / n_ntiles, nt = item % n_ntiles;
  MTile cur;
  tile_head(mt, cur);
  tile_rest(cur);
  Raw raw[BPW];
#pragma unroll
  for (int b = 0; b < BPW; ++b) load_block(cur.e, nt, b, raw[b]);
  tile_take(cur);
  issue_act(cur);
  full_barrier();

  // the previous item's output: value and index, or index < 0
  float pv = 0.f;
  int pi = -1;

  // A row of this lane: pair n >> 2, digit n & 3 (row 3 of a pair repeats
  // digit 2; its results are not used)
  const int arw = 4 * (n >> 2) + min(n & 3, 2);
  const int rixa = 4 * (arw & 3) + (n >> 2);  // LDS row: 4 * digit + pair
  const int aoff = L::PAD ? rixa * L::RSTRIDE + 16 * g : rixa * L::RSTRIDE;
  float *part = reinterpret_cast<float *>(lds + L::DIG);
  const float *xsl = reinterpret_cast<const float *>(lds + L::DIG + L::PART) + g * (NB * 8);  // pair g's sums
  for (;;) {
    const bool more = item + 1 < item_end;  // uniform
    const int mt2 = (item + 1) / n_ntiles, nt2 = (item + 1) % n_ntiles;
    const bool newm = more && mt2 != mt;
    MTile nx = cur;
    if (newm) {
      tile_head(mt2, nx);
      tile_rest(nx);
    }
    if (pi >= 0) out[pi] = pv;
    // the next item's weights (on the last item: this item's again, so every
    // path issues the same requests)
    const int e_next = more ? nx.e : cur.e, nt_next = more ? nt2 : nt;

    float acc = 0.f;  // pair g, weight row n
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      const int kb = kq * BPW + b;
      // A fragment of K tile j (the digit rows), read one K tile ahead
      auto afrag = [&](int j) {
        if constexpr (L::PAD) return *reinterpret_cast<const i32x4 *>(lds + aoff + kb * 256 + 64 * j);
        else return *reinterpret_cast<const i32x4 *>(lds + aoff + kb * 256 + (((4 * j + g) ^ arw) << 4));
      };
      i32x4 aj = afrag(0);
      if constexpr (!Q41) {
        // this block's operands from its raw bytes (the B fragments one K tile
        // at a time); once its MFMAs are issued, the raw registers take the
        // same block of the next item in place
        const Q2KPart rc = take_block(raw[b]);
        WTab tb;
        tb.build(rc, g);
        const i32x4 bmn = min_bfrag(rc, sel_lo, sel_hi);
        float dsc = f16lo(rc.dd), ndm = -f16hi(rc.dd);
        asm volatile("" : "+v"(dsc), "+v"(ndm));  // computed here, so d|dmin is free before the reload
        // per K tile the code and min MFMAs as one fenced group
        i32x4 c, cm;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const i32x4 an = afrag(j < 3 ? j + 1 : 3);
          const i32x4 bj = tb.bfrag(rc, j);
          mfma_group_begin();
          c = __builtin_amdgcn_mfma_i32_16x16x64_i8(aj, bj, j ? c : (i32x4){0, 0, 0, 0}, 0, 0, 0);
          cm = __builtin_amdgcn_mfma_i32_16x16x64_i8(aj, bmn, j ? cm : (i32x4){0, 0, 0, 0}, 0, 0, 0);
          mfma_fence();
          aj = an;
        }
        load_block(e_next, nt_next, b, raw[b]);
        acc = fmaf(dsc, digits3(c), acc);
        acc = fmaf(ndm, digits3(cm), acc);
      } else {
        // per K tile: the two blocks' MFMAs as one fenced group; the sums of
        // K tile j are scaled while the MFMAs of tile j + 1 run
        i32x4 ce[2], co[2];
        uint32_t dme[2], dmo[2];
        float2 xv[2];
        auto scale = [&](int q) {
          acc = fmaf(f16lo(dme[q]), digits3(ce[q]), acc);
          acc = fmaf(f16lo(dmo[q]), digits3(co[q]), acc);
          acc = fmaf(f16hi(dme[q]), xv[q].x, acc);
          acc = fmaf(f16hi(dmo[q]), xv[q].y, acc);
          asm volatile("" : "+v"(acc));  // here, not sunk below later MFMAs (their results would pile up)
        };
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = j & 1;
          const i32x4 an = afrag(j < 3 ? j + 1 : 3);
          const u32x3 rv = raw[b].v[j];
          const uint32_t h1 = rv.y >> 4, h2 = rv.z >> 4;
          const i32x4 be = {(int)(rv.y & mask_e), (int)(rv.z & mask_e), (int)(h1 & mask_e), (int)(h2 & mask_e)};
          const i32x4 bo = {(int)(rv.y & mask_o), (int)(rv.z & mask_o), (int)(h1 & mask_o), (int)(h2 & mask_o)};
          mfma_group_begin();
          ce[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aj, be, (i32x4){0, 0, 0, 0}, 0, 0, 0);
          co[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aj, bo, (i32x4){0, 0, 0, 0}, 0, 0, 0);
          mfma_fence();
          // d|m of block 2j + (g>>1) from the even lane group, then of blocks
          // 2j (lower half of the wave) and 2j + 1 (upper half) to every lane
          const uint32_t own = __builtin_amdgcn_permlane16_swap(rv.x, rv.x, false, false)[0];
          const auto pr = __builtin_amdgcn_permlane32_swap(own, own, false, false);
          dme[q] = pr[0];
          dmo[q] = pr[1];
          xv[q] = *reinterpret_cast<const float2 *>(xsl + kb * 8 + 2 * j);
          if (j) scale(q ^ 1);
          aj = an;
        }
        load_block(e_next, nt_next, b, raw[b]);
        scale(1);
      }
    }

    // every wave is done with the digit rows; the K parts meet
    lds_barrier();
    if (tid < GT) sig_s[tid] = cur.sig;
    part[(w * GT + g) * 16 + n] = acc;
    lds_barrier();
    pi = -1;
    if (tid < GT * ROWS) {
      const int m = tid / ROWS, r = tid % ROWS;
      if (m < cur.valid) {
        const int rgi = r / 16, rr = r % 16;
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int q = 0; q < KS; ++q) {
          v0 += part[(((0 * RG + rgi) * KS + q) * GT + m) * 16 + rr];
          if constexpr (SWIGLU) v1 += part[(((1 * RG + rgi) * KS + q) * GT + m) * 16 + rr];
        }
        const float sg = sig_s[m];
        if constexpr (SWIGLU) pv = silu(v0 * sg) * (v1 * sg);
        else pv = v0 * sg;
        pi = (cur.start + m) * rows_per_expert + nt * ROWS + r;
      }
    }
    if (!more) break;
    if (newm) {
      // the digit rows are no longer read: the new m-tile's land, and are
      // waited for here (with the weights in flight)
      tile_take(nx);
      issue_act(nx);
      full_barrier();
    }
    cur = nx;
    mt = mt2;
    nt = nt2;
    ++item;
  }
  if (pi >= 0) out[pi] = pv;
}

template <bool SWIGLU, bool Q41>
hipError_t launch_nb(int nb, const uint8_t *W0, const uint8_t *W1, int rows, const PrepD3 &a, int k,
                     int P, const RouteBufs &rb, int max_tiles, int n_cu, float *out, hipStream_t s) {
  const int nn = rows / rows_per_item(SWIGLU, nb);
  // persistent workgroups, WG_PER_CU per CU (at most one per item)
  const int64_t items = (int64_t)max_tiles * nn;
  const dim3 grid((unsigned)(items < WG_PER_CU * n_cu ? items : WG_PER_CU * n_cu));
#define DS4Q_DG(NBV)                                                                                      \
  hipLaunchKernelGGL((decode_grouped_kernel<SWIGLU, NBV, Q41>), grid, dim3(64 * NWV), 0, s, W0, W1, rows, a.q, \
                     a.sig, a.xs, k, P, rb, nn, out)
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

size_t prep_d3_bytes(int64_t rows, int K) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return up((size_t)rows * (K / 256) * QROW3) + up((size_t)rows * 4) + up((size_t)rows * (K / 32) * 4);
}

PrepD3 prep_d3_view(void *base, int64_t rows, int K) {
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  PrepD3 p;
  p.q = static_cast<uint8_t *>(base);
  p.sig = reinterpret_cast<float *>(p.q + up((size_t)rows * (K / 256) * QROW3));
  p.xs = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(p.sig) + up((size_t)rows * 4));
  return p;
}

hipError_t launch_prep_d3(const float *src, const float *inv_rms, int64_t rows, int K, int type,
                          const PrepD3 &p, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (type == TYPE_Q4_1)
    hipLaunchKernelGGL(prep_d3_kernel<true>, dim3((unsigned)rows), dim3(256), 0, s, src, inv_rms, K, p.q, p.sig,
                       p.xs);
  else
    hipLaunchKernelGGL(prep_d3_kernel<false>, dim3((unsigned)rows), dim3(256), 0, s, src, inv_rms, K, p.q, p.sig,
                       p.xs);
  return hipGetLastError();
}

hipError_t launch_decode_grouped(const MoeDims &m, const PrepD3 &a, int T, const RouteBufs &rb,
                                 int max_tiles, float *out, int phase, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T > 64) return hipErrorInvalidValue;
  const int P = T * m.k;
  int n_cu = 256;
  const hipError_t err = cu_count(&n_cu);
  if (err != hipSuccess) return err;
  if (phase == 1)
    return m.tg == TYPE_Q4_1
               ? launch_nb<true, true>(m.D / 256, m.gate, m.up, m.F, a, m.k, P, rb, max_tiles, n_cu, out, s)
               : launch_nb<true, false>(m.D / 256, m.gate, m.up, m.F, a, m.k, P, rb, max_tiles, n_cu, out, s);
  if (phase == 2)
    return m.td == TYPE_Q4_1
               ? launch_nb<false, true>(m.F / 256, m.down, nullptr, m.D, a, m.k, P, rb, max_tiles, n_cu, out, s)
               : launch_nb<false, false>(m.F / 256, m.down, nullptr, m.D, a, m.k, P, rb, max_tiles, n_cu, out, s);
  return hipErrorInvalidValue;
}

}  // namespace ds4q

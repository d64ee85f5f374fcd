// Host-side launchers of the gfx950 kernels (one translation unit per kernel
// family).  Called only from abi.cpp after argument validation.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ds4q {

hipError_t launch_dequant(int src_type, const void *src, int64_t rows, int64_t cols, bool bf16,
                          void *dst, hipStream_t s);

hipError_t launch_matvec(int w_type, const void *w, int64_t rows, int64_t cols, const float *x,
                         int n_tok, float *y, hipStream_t s);

// Routing workspace views (all device pointers).
struct RouteBufs {
  int32_t *ids;        // [T][k]
  float *w;            // [T][k]
  float *inv_rms;      // [T]  (written when x != NULL)
  int32_t *counts;     // [E]
  int32_t *offsets;    // [E+1]
  int32_t *pairs;      // [T*k] sorted by (expert, token, slot)
  int32_t *pair_pos;   // [T*k] inverse of pairs
  int32_t *act_expert; // [E]   active experts (count > 0), in expert order
  int32_t *act_begin;  // [E+1] start of each active expert's run in pairs
  int32_t *n_active;   // [1]
  int32_t *tiles;      // [max_tiles][2] (expert, first sorted position) m-tiles
  int32_t *n_tiles;    // [1]
  int32_t *tiles_sz;   // [max_tiles][2] prefill: the same m-tiles, full ones first, then by
                       // falling count of 16-pair groups (each class in expert order)
};

// Top-k + softmax per token; with x != NULL also the per-token inverse RMS.
hipError_t launch_topk(const float *logits, int T, int E, int k, const float *x, int D, float eps,
                       const RouteBufs &rb, hipStream_t s);
// Counting-sort grouping of the T*k pairs; tile_m > 0 also builds m-tiles,
// by_size also their size-ordered copy (rb.tiles_sz).
hipError_t launch_group(int T, int E, int k, int tile_m, bool by_size, const RouteBufs &rb, hipStream_t s);

// Directional steering of a layer's MoE output (dir == nullptr: none).
// stage ([D] f32) is one-token decode workspace: the down kernel writes the
// unsteered row there and launch_steer writes y from it.
struct SteerArgs {
  const float *dir = nullptr;
  float scale = 0.f;
  float *stage = nullptr;
};

struct MoeDims {
  int D, F, E, k;
  int tg, tu, td;  // block types of gate, up, down
  const uint8_t *gate, *up, *down;
};

// Single-token Q2_K decode on int8 matrix cores, in two phases: 1 = routing
// (into rb.ids / rb.w) + gate/up + SwiGLU into h, 2 = down + weighted combine
// into y.
hipError_t launch_decode_q2k_t1(const MoeDims &m, const float *x, const float *logits,
                                bool rmsnorm, float eps, const RouteBufs &rb, float *h, float *y,
                                bool accumulate, int phase, const SteerArgs &st, hipStream_t s);
// The same two phases on Q4_1 tensors (decode_q41.hip).  The gate/up and down
// kernels of the two formats share the workspace contract, so a layer may mix
// them (phase 1 by the gate/up type, phase 2 by the down type).
hipError_t launch_decode_q41_t1(const MoeDims &m, const float *x, const float *logits,
                                bool rmsnorm, float eps, const RouteBufs &rb, float *h, float *y,
                                bool accumulate, int phase, const SteerArgs &st, hipStream_t s);
// y[t] (+)= sum_j w[t][j] * o[row(t, j)]; row = pair index, or sorted
// position (via pair_pos) when by_pos.
// With st.dir set, each token row is steered before it is written (one
// workgroup per row).
hipError_t launch_combine(const float *o, const RouteBufs &rb, int T, int k, int D, bool by_pos,
                          float *y, bool accumulate, const SteerArgs &st, hipStream_t s);
// The same with o in bf16 (the prefill's down rows).
hipError_t launch_combine(const uint16_t *o, const RouteBufs &rb, int T, int k, int D, bool by_pos,
                          float *y, bool accumulate, const SteerArgs &st, hipStream_t s);

// Prefill on fp16 matrix cores, Q2_K or Q4_1 weights per tensor
// (prefill_f16.hip): activation rows scaled per row by a power of two and
// stored as fp16 in the MFMA fragment order of the weights they meet, with
// the factor that undoes the scaling.
struct PrepF16 {
  uint16_t *q;  // [rows][K/256][32][8] fp16
  float *sig;   // [rows]
};
size_t prep_f16_bytes(int64_t rows, int K);
PrepF16 prep_f16_view(void *base, int64_t rows, int K);
// src: f32 (f32in; times inv_rms[row] when given, then rounded to bf16 when
// round_bf16) or bf16 rows [rows][K]; wtype: the weight format (Q2_K or
// Q4_1) whose K order the rows are written in.
hipError_t launch_prep_f16(const void *src, bool f32in, bool round_bf16, const float *inv_rms,
                           int64_t rows, int K, int wtype, const PrepF16 &p, hipStream_t s);
hipError_t launch_prefill_f16_gateup(const MoeDims &m, const PrepF16 &a, int T, const RouteBufs &rb,
                                     int max_tiles, uint16_t *hb, hipStream_t s);
hipError_t launch_prefill_f16_down(const MoeDims &m, const PrepF16 &a, int T, const RouteBufs &rb,
                                   int max_tiles, uint16_t *ob, hipStream_t s);
// Decode of 2..64 tokens (decode_grouped.hip): activation rows prepared as
// three int8 digits per value, in the MFMA fragment order of the weight
// format they meet, and a per-row scale (plus, for Q4_1, the sums of every
// 32 values); m-tiles of at most DECODE_TILE_M sorted pairs; phase 1 writes
// the fp32 SwiGLU rows [T*k][F] from the prepared token rows, phase 2 the
// down rows [T*k][D] from the prepared SwiGLU rows, both in sorted-pair order.
struct PrepD3 {
  uint8_t *q;  // [rows][K/256][3][256]
  float *sig;  // [rows]
  float *xs;   // [rows][K/32]: sums of 32 values over sig (Q4_1 order only)
};
size_t prep_d3_bytes(int64_t rows, int K);
PrepD3 prep_d3_view(void *base, int64_t rows, int K);
// src: f32 rows [rows][K], times inv_rms[row] when given; type: the weight
// format (DS4Q_TYPE_Q2_K or DS4Q_TYPE_Q4_1) whose fragment order to write.
hipError_t launch_prep_d3(const float *src, const float *inv_rms, int64_t rows, int K, int type,
                          const PrepD3 &p, hipStream_t s);
hipError_t launch_decode_grouped(const MoeDims &m, const PrepD3 &a, int T, const RouteBufs &rb,
                                 int max_tiles, float *out, int phase, hipStream_t s);

// Directional steering: out_r (+)= y_r - scale * dir * (dir . y_r), rows of n
// floats (n % 4 == 0, 16-byte aligned); out may be y.
hipError_t launch_steer(const float *dir, float scale, const float *y, int64_t n_rows, int n,
                        float *out, bool accumulate, hipStream_t s);
// Activation wire formats: bits 32 (copy), 16 (f16) or 8 (E4M3).
hipError_t launch_act_encode(const float *src, int64_t n, int bits, void *dst, hipStream_t s);
hipError_t launch_act_decode(const void *src, int64_t n, int bits, float *dst, hipStream_t s);

// Device address of the current device's static scratch (scratch.hip),
// DS4Q_SCRATCH_BYTES long; looked up once per device.
hipError_t scratch_address(void **out);

constexpr int PREFILL_TILE_M = 128;
// Compute units of the current device, looked up once per device.
inline hipError_t cu_count(int *out) {
  static int cache[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!cache[dev]) {
    int v = 0;
    err = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    cache[dev] = v > 0 ? v : 256;
  }
  *out = cache[dev];
  return hipSuccess;
}
constexpr int DECODE_TILE_M = 4;

// imatrix statistics of one layer call (imatrix.hip).  Segments of an
// expert's pairs: the k slots of one token, the active experts (pairs grouped
// without m-tiles), or the m-tiles.
enum { IMAT_SEG_SLOTS = 0, IMAT_SEG_ACTIVE = 1, IMAT_SEG_TILES = 2 };
// Where a statistic reads its rows.  Input statistic: rows of x by token
// (f32 or bf16), times inv_rms[token] when given (or the row's own inverse
// RMS computed in place when norm_self: one token), rounded to bf16 when
// round_bf16.  Down statistic: SwiGLU rows (f32 or bf16) at the sorted
// position (by_sorted) or the pair index, times the pair's routing weight.
struct ImatRows {
  const void *rows = nullptr;
  bool bf16 = false;
  const float *inv_rms = nullptr;
  bool norm_self = false;
  float eps = 0.f;
  bool round_bf16 = false;
  bool by_sorted = false;
};
// stat_in [E][D] and stat_down [E][F] (either may be null) += the statistics;
// partial: [max_seg][max(D, F)] f32 workspace for IMAT_SEG_TILES.
hipError_t launch_imatrix(const MoeDims &m, const RouteBufs &rb, int seg_mode, int max_seg,
                          const ImatRows &in, float *stat_in, const ImatRows &h, float *stat_down,
                          float *partial, hipStream_t s);

}  // namespace ds4q

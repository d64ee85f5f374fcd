// Host side of libds4q.so: argument validation, workspace layout and kernel
// launches behind the extern "C" entry points declared in include/ds4q.h.
// Every check runs before anything is enqueued; no device memory is
// allocated here (the one library-owned device buffer is the static scratch
// of scratch.hip).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <utility>

#include "../../include/ds4q.h"
#include "launch.h"

#define DS4Q_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace ds4q;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

bool quant_type(int t) { return t == DS4Q_TYPE_Q2_K || t == DS4Q_TYPE_Q4_1; }

int qk_of(int t) { return t == DS4Q_TYPE_Q2_K ? 256 : 32; }

int64_t row_bytes(int t, int64_t cols) { return t == DS4Q_TYPE_Q2_K ? cols / 256 * 84 : cols / 32 * 20; }

bool path_dim(int32_t d) { return d == 256 || d == 512 || d == 1024 || d == 2048 || d == 4096; }

constexpr size_t ALIGN = 256;
size_t up(size_t v) { return (v + ALIGN - 1) & ~(ALIGN - 1); }

// Upper bound of the m-tiles of tile_m pairs: every active expert's last
// tile may be partial.
int max_tiles(int T, int E, int k, int tile_m) {
  const int P = T * k;
  return (P < E ? P : E) + P / tile_m + 1;
}

// Workspace carving; with base == nullptr only the size is computed.
struct Workspace {
  RouteBufs rb{};
  float *h = nullptr;      // decode: [T*k][F] f32
  uint16_t *hb = nullptr;  // prefill: [T*k][F] bf16 (sorted order)
  float *o = nullptr;      // decode: [T*k][D] f32
  uint16_t *ob = nullptr;  // prefill: [T*k][D] bf16 (sorted order)
  float *stage = nullptr;  // decode of one token: [D] f32, the unsteered output before steering
  float *imat_part = nullptr;  // imatrix on m-tiles: [max_tiles][max(D, F)] f32 partial rows
  PrepF16 xq{}, hq{};      // prefill: fp16 rows of x and of hb
  PrepD3 xd{}, hd{};       // decode of 2..64 tokens: int8 digit rows of x and of h
  size_t bytes = 0;

  // mode 0 = decode, 1 = prefill, 2 = routing only; stats: the imatrix
  // partial rows of the prefill
  Workspace(uint8_t *base, int D, int F, int E, int k, int T, int mode, bool stats = false) {
    size_t off = 0;
    auto take = [&](size_t n) -> void * {
      void *p = base ? base + off : nullptr;
      off += up(n);
      return p;
    };
    const size_t P = (size_t)T * k;
    rb.ids = (int32_t *)take(P * 4);
    rb.w = (float *)take(P * 4);
    rb.inv_rms = (float *)take((size_t)T * 4);
    rb.counts = (int32_t *)take((size_t)E * 4);
    rb.offsets = (int32_t *)take((size_t)(E + 1) * 4);
    rb.pairs = (int32_t *)take(P * 4);
    rb.pair_pos = (int32_t *)take(P * 4);
    rb.act_expert = (int32_t *)take((size_t)E * 4);
    rb.act_begin = (int32_t *)take((size_t)(E + 1) * 4);
    rb.n_active = (int32_t *)take(4);
    rb.n_tiles = (int32_t *)take(4);
    if (mode == 2) {
      // routing only
    } else if (mode == 0) {
      h = (float *)take(P * F * 4);
      if (T == 1) {
        stage = (float *)take((size_t)D * 4);
      } else {  // decode of 2..64 tokens: the grouped int8 kernels
        o = (float *)take(P * D * 4);
        rb.tiles = (int32_t *)take((size_t)max_tiles(T, E, k, DECODE_TILE_M) * 8);
        void *p = take(prep_d3_bytes(T, D));
        if (base) xd = prep_d3_view(p, T, D);
        p = take(prep_d3_bytes(P, F));
        if (base) hd = prep_d3_view(p, P, F);
      }
    } else {
      rb.tiles = (int32_t *)take((size_t)max_tiles(T, E, k, PREFILL_TILE_M) * 8);
      rb.tiles_sz = (int32_t *)take((size_t)max_tiles(T, E, k, PREFILL_TILE_M) * 8);
      hb = (uint16_t *)take(P * F * 2);
      ob = (uint16_t *)take(P * D * 2);
      {
        void *p = take(prep_f16_bytes(T, D));
        if (base) xq = prep_f16_view(p, T, D);
        p = take(prep_f16_bytes(P, F));
        if (base) hq = prep_f16_view(p, P, F);
      }
      if (stats) imat_part = (float *)take((size_t)max_tiles(T, E, k, PREFILL_TILE_M) * (D > F ? D : F) * 4);
    }
    bytes = off;
  }
};

int check_layer(const ds4q_moe_layer *L) {
  if (!L) return DS4Q_E_INVAL;
  for (int t : {L->type_gate, L->type_up, L->type_down})
    if (!quant_type(t)) return DS4Q_E_UNSUPPORTED;
  if (L->type_gate != L->type_up) return DS4Q_E_UNSUPPORTED;
  if (L->n_expert < 1 || L->n_expert > 1024 || L->n_expert_used < 1 || L->n_expert_used > 8 ||
      L->n_expert_used > L->n_expert)
    return DS4Q_E_INVAL;
  if (!path_dim(L->n_embd) || !path_dim(L->n_ff)) return DS4Q_E_SHAPE;
  if (!L->gate || !L->up || !L->down) return DS4Q_E_INVAL;
  if (!aligned(L->gate, 16) || !aligned(L->up, 16) || !aligned(L->down, 16)) return DS4Q_E_ALIGN;
  if (L->flags & ~(DS4Q_F_ACCUMULATE | DS4Q_F_RMSNORM_INPUT)) return DS4Q_E_INVAL;
  if (!(L->norm_eps >= 0.0f) || !isfinite(L->norm_eps)) return DS4Q_E_INVAL;
  if (L->steer_dir) {
    if (!aligned(L->steer_dir, 16)) return DS4Q_E_ALIGN;
    if (!isfinite(L->steer_scale)) return DS4Q_E_INVAL;
  }
  if (!aligned(L->imatrix_in, 16) || !aligned(L->imatrix_down, 16)) return DS4Q_E_ALIGN;
  if (L->imatrix_in && L->imatrix_down &&
      overlap(L->imatrix_in, (size_t)L->n_expert * L->n_embd * 4, L->imatrix_down,
              (size_t)L->n_expert * L->n_ff * 4))
    return DS4Q_E_ALIAS;
  return DS4Q_OK;
}

SteerArgs steer_of(const ds4q_moe_layer *L, float *stage) {
  SteerArgs st;
  if (L->steer_dir) {
    st.dir = L->steer_dir;
    st.scale = L->steer_scale;
    st.stage = stage;
  }
  return st;
}


bool wants_stats(const ds4q_moe_layer *L) { return L->imatrix_in || L->imatrix_down; }

MoeDims dims_of(const ds4q_moe_layer *L) {
  MoeDims m;
  m.D = L->n_embd; m.F = L->n_ff; m.E = L->n_expert; m.k = L->n_expert_used;
  m.tg = L->type_gate; m.tu = L->type_up; m.td = L->type_down;
  m.gate = static_cast<const uint8_t *>(L->gate);
  m.up = static_cast<const uint8_t *>(L->up);
  m.down = static_cast<const uint8_t *>(L->down);
  return m;
}

// ---------------------------------------------------------------- timing
// While enabled, each launcher call is bracketed by two HIP events recorded on
// the caller's stream; ds4q_timing_read() resolves them per launcher name.
struct TimingRec {
  const char *name;
  hipEvent_t start, stop;
};
constexpr int MAX_TIMING = 1 << 16;
constexpr int MAX_NAMES = 32;
bool g_timing = false;
int g_n_rec = 0;
TimingRec g_rec[MAX_TIMING];

struct Timed {
  TimingRec *rec = nullptr;
  hipStream_t s;
  Timed(const char *name, hipStream_t st) : s(st) {
    if (!g_timing || g_n_rec >= MAX_TIMING) return;
    TimingRec &r = g_rec[g_n_rec];
    if (hipEventCreate(&r.start) != hipSuccess) return;
    if (hipEventCreate(&r.stop) != hipSuccess) {
      (void)hipEventDestroy(r.start);
      return;
    }
    r.name = name;
    if (hipEventRecord(r.start, s) != hipSuccess) {
      (void)hipEventDestroy(r.start);
      (void)hipEventDestroy(r.stop);
      return;
    }
    rec = &r;
    ++g_n_rec;
  }
  ~Timed() {
    if (rec) (void)hipEventRecord(rec->stop, s);
  }
};

#define HIP_TRY(expr)                                \
  do {                                               \
    if ((expr) != hipSuccess) return DS4Q_E_HIP;     \
  } while (0)

#define TIMED_TRY(name, expr)                        \
  do {                                               \
    Timed timed_(name, s);                           \
    if ((expr) != hipSuccess) return DS4Q_E_HIP;     \
  } while (0)

// Copy the requested routing outputs out of the workspace.
int copy_route(const ds4q_route_out *route, const RouteBufs &rb, int T, int E, int k,
               hipStream_t s) {
  if (!route) return DS4Q_OK;
  const size_t P = (size_t)T * k;
  auto cp = [&](void *dst, const void *src, size_t n) -> bool {
    return !dst || n == 0 || hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, s) == hipSuccess;
  };
  if (!cp(route->topk_ids, rb.ids, P * 4) || !cp(route->topk_w, rb.w, P * 4) ||
      !cp(route->expert_counts, rb.counts, (size_t)E * 4) ||
      !cp(route->expert_offsets, rb.offsets, (size_t)(E + 1) * 4) ||
      !cp(route->sorted_pairs, rb.pairs, P * 4))
    return DS4Q_E_HIP;
  return DS4Q_OK;
}

bool route_overlaps(const ds4q_route_out *r, int T, int E, int k, const void *p, size_t n) {
  if (!r) return false;
  const size_t P = (size_t)T * k;
  return overlap(r->topk_ids, P * 4, p, n) || overlap(r->topk_w, P * 4, p, n) ||
         overlap(r->expert_counts, (size_t)E * 4, p, n) ||
         overlap(r->expert_offsets, (size_t)(E + 1) * 4, p, n) ||
         overlap(r->sorted_pairs, P * 4, p, n);
}

bool route_misaligned(const ds4q_route_out *r) {
  if (!r) return false;
  return !aligned(r->topk_ids, 4) || !aligned(r->topk_w, 4) || !aligned(r->expert_counts, 4) ||
         !aligned(r->expert_offsets, 4) || !aligned(r->sorted_pairs, 4);
}

bool wants_grouping(const ds4q_route_out *r) {
  return r && (r->expert_counts || r->expert_offsets || r->sorted_pairs);
}

// Shared argument checks of the decode / prefill layer calls.  With
// STATIC_WS the workspace is the library's static scratch (its size is
// checked by the caller; no caller buffer can overlap it): ws is ignored.
constexpr void *STATIC_WS = nullptr;
int check_call(const ds4q_moe_layer *L, const void *x, size_t x_elem, const float *logits, int32_t T,
               int32_t max_T, const float *y, const ds4q_route_out *route, void *ws, size_t ws_bytes,
               int mode, bool static_ws = false) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0 || T > max_T) return DS4Q_E_SHAPE;
  if (T == 0) return DS4Q_OK;
  if (!x || !logits || !y) return DS4Q_E_INVAL;
  if (!ws && !static_ws) return DS4Q_E_WORKSPACE;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(logits, 4) || !aligned(ws, ALIGN) ||
      route_misaligned(route))
    return DS4Q_E_ALIGN;
  const Workspace need(nullptr, L->n_embd, L->n_ff, L->n_expert, L->n_expert_used, T, mode, wants_stats(L));
  if (static_ws) {
    if (need.bytes > DS4Q_SCRATCH_BYTES) return DS4Q_E_SCRATCH;
  } else if (ws_bytes < need.bytes) {
    return DS4Q_E_WORKSPACE;
  }
  const size_t xb = (size_t)T * L->n_embd * x_elem, yb = (size_t)T * L->n_embd * 4;
  const size_t lb = (size_t)T * L->n_expert * 4;
  if (overlap(ws, need.bytes, x, xb) || overlap(ws, need.bytes, y, yb) ||
      overlap(ws, need.bytes, logits, lb))
    return DS4Q_E_ALIAS;
  if ((const void *)y != x && overlap(y, yb, x, xb)) return DS4Q_E_ALIAS;
  if (L->steer_dir) {
    const size_t db = (size_t)L->n_embd * 4;
    if (overlap(L->steer_dir, db, y, yb) || overlap(L->steer_dir, db, ws, need.bytes))
      return DS4Q_E_ALIAS;
  }
  // the statistics are written: they overlap no input, output or workspace
  const std::pair<const void *, size_t> stats[2] = {
      {L->imatrix_in, (size_t)L->n_expert * L->n_embd * 4},
      {L->imatrix_down, (size_t)L->n_expert * L->n_ff * 4}};
  for (const auto &st : stats) {
    if (!st.first) continue;
    if (overlap(st.first, st.second, x, xb) || overlap(st.first, st.second, y, yb) ||
        overlap(st.first, st.second, logits, lb) || overlap(st.first, st.second, ws, need.bytes) ||
        (L->steer_dir && overlap(st.first, st.second, L->steer_dir, (size_t)L->n_embd * 4)) ||
        overlap(st.first, st.second, L->gate, (size_t)L->n_expert * L->n_ff * row_bytes(L->type_gate, L->n_embd)) ||
        overlap(st.first, st.second, L->up, (size_t)L->n_expert * L->n_ff * row_bytes(L->type_up, L->n_embd)) ||
        overlap(st.first, st.second, L->down, (size_t)L->n_expert * L->n_embd * row_bytes(L->type_down, L->n_ff)) ||
        route_overlaps(route, T, L->n_expert, L->n_expert_used, st.first, st.second))
      return DS4Q_E_ALIAS;
  }
  if (overlap(y, yb, logits, lb)) return DS4Q_E_ALIAS;
  if (route_overlaps(route, T, L->n_expert, L->n_expert_used, ws, need.bytes) ||
      route_overlaps(route, T, L->n_expert, L->n_expert_used, y, yb) ||
      route_overlaps(route, T, L->n_expert, L->n_expert_used, x, xb) ||
      route_overlaps(route, T, L->n_expert, L->n_expert_used, logits, lb))
    return DS4Q_E_ALIAS;
  return DS4Q_OK;
}

// imatrix statistics of a call, launched once the routing and the SwiGLU
// rows exist and before anything writes y (which may be x).
hipError_t launch_stats(const ds4q_moe_layer *L, const MoeDims &m, const Workspace &w, int seg_mode,
                        int max_seg, const ImatRows &in, const ImatRows &h, hipStream_t s) {
  if (!wants_stats(L)) return hipSuccess;
  return launch_imatrix(m, w.rb, seg_mode, max_seg, in, L->imatrix_in, h, L->imatrix_down,
                        w.imat_part, s);
}

ImatRows rows_of(const void *p, bool bf16, const float *inv_rms, bool by_sorted) {
  ImatRows r;
  r.rows = p;
  r.bf16 = bf16;
  r.inv_rms = inv_rms;
  r.by_sorted = by_sorted;
  return r;
}

// The decode launches in three phases (DS4Q_PHASE_*): routing and input
// preparation, gate/up + SwiGLU, down + combine.  Each phase reads only what
// the earlier ones left in the workspace.
int run_decode(const ds4q_moe_layer *L, const float *x, const float *logits, int32_t T, float *y,
               const ds4q_route_out *route, void *ws, hipStream_t s, uint32_t flags,
               uint32_t phases = DS4Q_PHASE_ALL) {
  const MoeDims m = dims_of(L);
  Workspace w(static_cast<uint8_t *>(ws), m.D, m.F, m.E, m.k, T, 0, wants_stats(L));
  const bool norm = flags & DS4Q_F_RMSNORM_INPUT, acc = flags & DS4Q_F_ACCUMULATE;
  const SteerArgs st = steer_of(L, w.stage);
  const bool p_route = phases & DS4Q_PHASE_ROUTE, p_gu = phases & DS4Q_PHASE_GATEUP,
             p_down = phases & DS4Q_PHASE_DOWN;
  if (T == 1) {
    // One token on int8 matrix cores (either block format, chosen per
    // tensor): the gate/up launch routes the token itself, so the routing
    // phase has nothing of its own to launch and the routing outputs follow
    // the gate/up launch.
    auto t1 = [&](int phase) {
      const int type = phase == 1 ? m.tg : m.td;
      return type == DS4Q_TYPE_Q2_K
                 ? launch_decode_q2k_t1(m, x, logits, norm, L->norm_eps, w.rb, w.h, y, acc, phase, st, s)
                 : launch_decode_q41_t1(m, x, logits, norm, L->norm_eps, w.rb, w.h, y, acc, phase, st, s);
    };
    if (p_gu) {
      TIMED_TRY("decode_gateup", t1(1));
      // the grouping pass (expert order) runs only when asked for
      if (wants_grouping(route)) TIMED_TRY("group", launch_group(T, m.E, m.k, 0, false, w.rb, s));
      ImatRows in = rows_of(x, false, nullptr, false);
      in.norm_self = norm;  // the gate/up launch keeps the inverse RMS to itself
      in.eps = L->norm_eps;
      if (wants_stats(L)) TIMED_TRY("imatrix", launch_stats(L, m, w, IMAT_SEG_SLOTS, m.k, in, rows_of(w.h, false, nullptr, false), s));
    }
    if (p_down) TIMED_TRY("decode_down", t1(2));
    return p_gu ? copy_route(route, w.rb, T, m.E, m.k, s) : DS4Q_OK;
  }
  // 2..64 tokens: expert-grouped m-tiles of at most DECODE_TILE_M pairs on
  // int8 matrix cores, either format per tensor; h and o in sorted-pair order
  const int mt = max_tiles(T, m.E, m.k, DECODE_TILE_M);
  if (p_route) {
    TIMED_TRY("topk", launch_topk(logits, T, m.E, m.k, norm ? x : nullptr, m.D, L->norm_eps, w.rb, s));
    TIMED_TRY("group", launch_group(T, m.E, m.k, DECODE_TILE_M, false, w.rb, s));
  }
  if (p_gu) {
    TIMED_TRY("prep_d3", launch_prep_d3(x, norm ? w.rb.inv_rms : nullptr, T, m.D, m.tg, w.xd, s));
    TIMED_TRY("decode_gateup", launch_decode_grouped(m, w.xd, T, w.rb, mt, w.h, 1, s));
    const int na = T * m.k < m.E ? T * m.k : m.E;
    if (wants_stats(L)) TIMED_TRY("imatrix", launch_stats(L, m, w, IMAT_SEG_ACTIVE, na, rows_of(x, false, norm ? w.rb.inv_rms : nullptr, false),
                                      rows_of(w.h, false, nullptr, true), s));
  }
  if (p_down) {
    TIMED_TRY("prep_d3", launch_prep_d3(w.h, nullptr, (int64_t)T * m.k, m.F, m.td, w.hd, s));
    TIMED_TRY("decode_down", launch_decode_grouped(m, w.hd, T, w.rb, mt, w.o, 2, s));
    TIMED_TRY("combine", launch_combine(w.o, w.rb, T, m.k, m.D, true, y, acc, st, s));
  }
  return p_route ? copy_route(route, w.rb, T, m.E, m.k, s) : DS4Q_OK;
}

int run_prefill(const ds4q_moe_layer *L, const void *x, int32_t x_type, const float *logits,
                int32_t T, float *y, const ds4q_route_out *route, void *ws, hipStream_t s,
                uint32_t flags) {
  const MoeDims m = dims_of(L);
  Workspace w(static_cast<uint8_t *>(ws), m.D, m.F, m.E, m.k, T, 1, wants_stats(L));
  const bool norm = flags & DS4Q_F_RMSNORM_INPUT, acc = flags & DS4Q_F_ACCUMULATE;
  const float *xf = x_type == DS4Q_TYPE_F32 ? static_cast<const float *>(x) : nullptr;
  TIMED_TRY("topk", launch_topk(logits, T, m.E, m.k, norm ? xf : nullptr, m.D, L->norm_eps, w.rb, s));
  TIMED_TRY("group", launch_group(T, m.E, m.k, PREFILL_TILE_M, true, w.rb, s));
  const int mt = max_tiles(T, m.E, m.k, PREFILL_TILE_M);
  TIMED_TRY("prep_f16", launch_prep_f16(x, xf != nullptr, true, norm && xf ? w.rb.inv_rms : nullptr, T, m.D,
                                        m.tg, w.xq, s));
  TIMED_TRY("prefill_gateup", launch_prefill_f16_gateup(m, w.xq, T, w.rb, mt, w.hb, s));
  {
    ImatRows in = rows_of(x, xf == nullptr, norm && xf ? w.rb.inv_rms : nullptr, false);
    in.round_bf16 = xf != nullptr;  // the expert GEMMs read the bf16 rounding of the f32 input
    if (wants_stats(L)) TIMED_TRY("imatrix", launch_stats(L, m, w, IMAT_SEG_TILES, mt, in, rows_of(w.hb, true, nullptr, true), s));
  }
  const int64_t P = (int64_t)T * m.k;
  TIMED_TRY("prep_f16", launch_prep_f16(w.hb, false, false, nullptr, P, m.F, m.td, w.hq, s));
  TIMED_TRY("prefill_down", launch_prefill_f16_down(m, w.hq, T, w.rb, mt, w.ob, s));
  TIMED_TRY("combine", launch_combine(w.ob, w.rb, T, m.k, m.D, true, y, acc, steer_of(L, nullptr), s));
  return copy_route(route, w.rb, T, m.E, m.k, s);
}

}  // namespace

DS4Q_API int ds4q_abi_version(void) { return DS4Q_ABI_VERSION; }

DS4Q_API const char *ds4q_strerror(int status) {
  switch (status) {
    case DS4Q_OK: return "ok";
    case DS4Q_E_INVAL: return "invalid argument";
    case DS4Q_E_UNSUPPORTED: return "unsupported tensor type";
    case DS4Q_E_SHAPE: return "unsupported or inconsistent shape";
    case DS4Q_E_ALIGN: return "misaligned pointer";
    case DS4Q_E_WORKSPACE: return "workspace missing or too small";
    case DS4Q_E_ALIAS: return "output overlaps an input or the workspace";
    case DS4Q_E_HIP: return "HIP runtime error";
    case DS4Q_E_SCRATCH: return "call needs more than the static scratch (DS4Q_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

DS4Q_API int ds4q_dequant(int32_t src_type, const void *src, int64_t rows, int64_t cols,
                          int32_t dst_type, void *dst, void *stream) {
  if (!quant_type(src_type)) return DS4Q_E_UNSUPPORTED;
  if (dst_type != DS4Q_TYPE_F32 && dst_type != DS4Q_TYPE_BF16) return DS4Q_E_UNSUPPORTED;
  if (rows < 0 || cols <= 0) return DS4Q_E_SHAPE;
  if (cols % qk_of(src_type)) return DS4Q_E_SHAPE;
  if (rows == 0) return DS4Q_OK;
  if (!src || !dst) return DS4Q_E_INVAL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return DS4Q_E_ALIGN;
  const size_t sb = (size_t)rows * row_bytes(src_type, cols);
  const size_t db = (size_t)rows * cols * (dst_type == DS4Q_TYPE_F32 ? 4 : 2);
  if (overlap(src, sb, dst, db)) return DS4Q_E_ALIAS;
  HIP_TRY(launch_dequant(src_type, src, rows, cols, dst_type == DS4Q_TYPE_BF16, dst,
                         static_cast<hipStream_t>(stream)));
  return DS4Q_OK;
}

DS4Q_API int ds4q_matvec(int32_t w_type, const void *w, int64_t rows, int64_t cols, const float *x,
                         int32_t n_tok, float *y, void *stream) {
  if (!quant_type(w_type)) return DS4Q_E_UNSUPPORTED;
  if (rows < 0 || n_tok < 0 || n_tok > 64) return DS4Q_E_SHAPE;
  if (!path_dim((int32_t)cols) || cols != (int32_t)cols) return DS4Q_E_SHAPE;
  if (rows == 0 || n_tok == 0) return DS4Q_OK;
  if (!w || !x || !y) return DS4Q_E_INVAL;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return DS4Q_E_ALIGN;
  const size_t wb = (size_t)rows * row_bytes(w_type, cols);
  if (overlap(y, (size_t)rows * n_tok * 4, x, (size_t)cols * n_tok * 4) ||
      overlap(y, (size_t)rows * n_tok * 4, w, wb))
    return DS4Q_E_ALIAS;
  HIP_TRY(launch_matvec(w_type, w, rows, cols, x, n_tok, y, static_cast<hipStream_t>(stream)));
  return DS4Q_OK;
}

DS4Q_API size_t ds4q_route_workspace_size(int32_t n_tok, int32_t n_expert, int32_t k) {
  if (n_expert < 1 || n_expert > 1024 || k < 1 || k > 8 || k > n_expert || n_tok < 0 ||
      n_tok > 65536)
    return 0;
  return Workspace(nullptr, 0, 0, n_expert, k, n_tok > 0 ? n_tok : 1, 2).bytes;
}

DS4Q_API int ds4q_route(const float *logits, int32_t n_tok, int32_t n_expert, int32_t k,
                        const ds4q_route_out *out, void *workspace, size_t workspace_bytes,
                        void *stream) {
  if (n_expert < 1 || n_expert > 1024 || k < 1 || k > 8 || k > n_expert) return DS4Q_E_INVAL;
  if (n_tok < 0 || n_tok > 65536) return DS4Q_E_SHAPE;
  if (n_tok == 0) return DS4Q_OK;
  if (!logits || !out) return DS4Q_E_INVAL;
  if (!workspace) return DS4Q_E_WORKSPACE;
  if (!aligned(logits, 4) || route_misaligned(out) || !aligned(workspace, ALIGN))
    return DS4Q_E_ALIGN;
  const Workspace need(nullptr, 0, 0, n_expert, k, n_tok, 2);
  if (workspace_bytes < need.bytes) return DS4Q_E_WORKSPACE;
  const size_t lb = (size_t)n_tok * n_expert * 4;
  if (route_overlaps(out, n_tok, n_expert, k, logits, lb) ||
      route_overlaps(out, n_tok, n_expert, k, workspace, need.bytes) ||
      overlap(workspace, need.bytes, logits, lb))
    return DS4Q_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace w(static_cast<uint8_t *>(workspace), 0, 0, n_expert, k, n_tok, 2);
  HIP_TRY(launch_topk(logits, n_tok, n_expert, k, nullptr, 0, 0.f, w.rb, s));
  if (wants_grouping(out)) HIP_TRY(launch_group(n_tok, n_expert, k, 0, false, w.rb, s));
  return copy_route(out, w.rb, n_tok, n_expert, k, s);
}

DS4Q_API size_t ds4q_moe_workspace_size(const ds4q_moe_layer *L, int32_t max_tok, int32_t mode) {
  if (check_layer(L) || max_tok < 0 || (mode != 0 && mode != 1)) return 0;
  const int T = max_tok > 0 ? max_tok : 1;
  return Workspace(nullptr, L->n_embd, L->n_ff, L->n_expert, L->n_expert_used, T, mode, wants_stats(L)).bytes;
}

DS4Q_API int ds4q_moe_decode(const ds4q_moe_layer *L, const float *x, const float *logits,
                             int32_t n_tok, float *y, const ds4q_route_out *route, void *workspace,
                             size_t workspace_bytes, void *stream) {
  int rc = check_call(L, x, 4, logits, n_tok, 64, y, route, workspace, workspace_bytes, 0);
  if (rc || n_tok == 0) return rc;
  return run_decode(L, x, logits, n_tok, y, route, workspace, static_cast<hipStream_t>(stream),
                    L->flags);
}

DS4Q_API int ds4q_moe_decode_static(const ds4q_moe_layer *L, const float *x, const float *logits,
                                    int32_t n_tok, float *y, const ds4q_route_out *route,
                                    void *stream) {
  // every argument check first (the same as ds4q_moe_decode's), then the
  // scratch's device address
  const int rc = check_call(L, x, 4, logits, n_tok, 64, y, route, STATIC_WS, 0, 0, true);
  if (rc || n_tok == 0) return rc;
  void *ws = nullptr;
  HIP_TRY(scratch_address(&ws));
  return run_decode(L, x, logits, n_tok, y, route, ws, static_cast<hipStream_t>(stream), L->flags);
}

DS4Q_API int ds4q_moe_decode_phases(const ds4q_moe_layer *L, const float *x, const float *logits,
                                    int32_t n_tok, float *y, const ds4q_route_out *route,
                                    void *workspace, size_t workspace_bytes, uint32_t phases,
                                    void *stream) {
  if (phases == 0 || (phases & ~(uint32_t)DS4Q_PHASE_ALL)) return DS4Q_E_INVAL;
  int rc = check_call(L, x, 4, logits, n_tok, 64, y, route, workspace, workspace_bytes, 0);
  if (rc || n_tok == 0) return rc;
  return run_decode(L, x, logits, n_tok, y, route, workspace, static_cast<hipStream_t>(stream),
                    L->flags, phases);
}

DS4Q_API int ds4q_moe_prefill(const ds4q_moe_layer *L, const void *x, int32_t x_type,
                              const float *logits, int32_t n_tok, float *y,
                              const ds4q_route_out *route, void *workspace, size_t workspace_bytes,
                              void *stream) {
  if (x_type != DS4Q_TYPE_BF16 && x_type != DS4Q_TYPE_F32) return DS4Q_E_UNSUPPORTED;
  if (x_type == DS4Q_TYPE_BF16 && L && (L->flags & DS4Q_F_RMSNORM_INPUT)) return DS4Q_E_INVAL;
  int rc = check_call(L, x, x_type == DS4Q_TYPE_F32 ? 4 : 2, logits, n_tok, 65536, y, route,
                      workspace, workspace_bytes, 1);
  if (rc || n_tok == 0) return rc;
  if (x_type == DS4Q_TYPE_BF16 && overlap(y, (size_t)n_tok * L->n_embd * 4, x,
                                          (size_t)n_tok * L->n_embd * 2))
    return DS4Q_E_ALIAS;
  return run_prefill(L, x, x_type, logits, n_tok, y, route, workspace,
                     static_cast<hipStream_t>(stream), L->flags);
}

DS4Q_API int ds4q_steer(const float *dir, float scale, const float *y, int32_t n_rows, int32_t n_embd,
                        float *out, uint32_t flags, void *stream) {
  if (flags & ~DS4Q_F_ACCUMULATE) return DS4Q_E_INVAL;
  if (n_rows < 0 || n_embd < 4 || n_embd > 65536 || n_embd % 4) return DS4Q_E_SHAPE;
  if (n_rows == 0) return DS4Q_OK;
  if (!dir || !y || !out || !isfinite(scale)) return DS4Q_E_INVAL;
  if (!aligned(dir, 16) || !aligned(y, 16) || !aligned(out, 16)) return DS4Q_E_ALIGN;
  const size_t rb = (size_t)n_rows * n_embd * 4;
  if (overlap(dir, (size_t)n_embd * 4, out, rb)) return DS4Q_E_ALIAS;
  if ((const void *)y != out && overlap(y, rb, out, rb)) return DS4Q_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TIMED_TRY("steer", launch_steer(dir, scale, y, n_rows, n_embd, out, flags & DS4Q_F_ACCUMULATE, s));
  return DS4Q_OK;
}

DS4Q_API int ds4q_act_encode(const float *src, int64_t n, int32_t bits, void *dst, void *stream) {
  if (bits != 32 && bits != 16 && bits != 8) return DS4Q_E_INVAL;
  if (n < 0) return DS4Q_E_SHAPE;
  if (n == 0) return DS4Q_OK;
  if (!src || !dst) return DS4Q_E_INVAL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return DS4Q_E_ALIGN;
  if (overlap(src, (size_t)n * 4, dst, (size_t)n * bits / 8)) return DS4Q_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TIMED_TRY("act_encode", launch_act_encode(src, n, bits, dst, s));
  return DS4Q_OK;
}

DS4Q_API int ds4q_act_decode(const void *src, int64_t n, int32_t bits, float *dst, void *stream) {
  if (bits != 32 && bits != 16 && bits != 8) return DS4Q_E_INVAL;
  if (n < 0) return DS4Q_E_SHAPE;
  if (n == 0) return DS4Q_OK;
  if (!src || !dst) return DS4Q_E_INVAL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return DS4Q_E_ALIGN;
  if (overlap(src, (size_t)n * bits / 8, dst, (size_t)n * 4)) return DS4Q_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TIMED_TRY("act_decode", launch_act_decode(src, n, bits, dst, s));
  return DS4Q_OK;
}

DS4Q_API int ds4q_moe_stack(const ds4q_moe_layer *layers, int32_t n_layers, int32_t mode, float *x,
                            const float *logits, int32_t n_tok, void *workspace,
                            size_t workspace_bytes, void *stream) {
  if (!layers || n_layers < 0 || (mode != 0 && mode != 1)) return DS4Q_E_INVAL;
  if (n_layers == 0 || n_tok == 0) return n_tok < 0 ? DS4Q_E_SHAPE : DS4Q_OK;
  const ds4q_moe_layer &l0 = layers[0];
  for (int32_t l = 0; l < n_layers; ++l) {
    const ds4q_moe_layer &L = layers[l];
    int rc = check_layer(&L);
    if (rc) return rc;
    if (L.n_embd != l0.n_embd || L.n_ff != l0.n_ff || L.n_expert != l0.n_expert ||
        L.n_expert_used != l0.n_expert_used)
      return DS4Q_E_SHAPE;
    rc = check_call(&L, x, 4, logits + (size_t)l * n_tok * L.n_expert, n_tok, mode ? 65536 : 64, x,
                    nullptr, workspace, workspace_bytes, mode);
    if (rc) return rc;
  }
  const size_t lb = (size_t)n_layers * n_tok * l0.n_expert * 4;
  if (overlap(x, (size_t)n_tok * l0.n_embd * 4, logits, lb) ||
      overlap(workspace, workspace_bytes, logits, lb))
    return DS4Q_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t flags = DS4Q_F_RMSNORM_INPUT | DS4Q_F_ACCUMULATE;
  for (int32_t l = 0; l < n_layers; ++l) {
    const float *lg = logits + (size_t)l * n_tok * l0.n_expert;
    const int rc = mode == 0 ? run_decode(&layers[l], x, lg, n_tok, x, nullptr, workspace, s, flags)
                             : run_prefill(&layers[l], x, DS4Q_TYPE_F32, lg, n_tok, x, nullptr,
                                           workspace, s, flags);
    if (rc) return rc;
  }
  return DS4Q_OK;
}

DS4Q_API int ds4q_timing_enable(int on) {
  g_timing = on != 0;
  return DS4Q_OK;
}

DS4Q_API int ds4q_timing_read(char *names, int name_len, double *total_ms, int64_t *count,
                              int max_names, int *n_names) {
  if (!names || !total_ms || !count || !n_names || name_len < 2 || max_names < 1)
    return DS4Q_E_INVAL;
  const char *seen[MAX_NAMES];
  int n = 0, rc = DS4Q_OK;
  for (int i = 0; i < g_n_rec; ++i) {
    TimingRec &r = g_rec[i];
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      rc = DS4Q_E_HIP;
    int j = 0;
    while (j < n && strcmp(seen[j], r.name) != 0) ++j;
    if (j == n && n < max_names && n < MAX_NAMES) {
      seen[n] = r.name;
      strncpy(names + (size_t)n * name_len, r.name, (size_t)name_len - 1);
      names[(size_t)n * name_len + name_len - 1] = 0;
      total_ms[n] = 0.0;
      count[n] = 0;
      ++n;
    }
    if (j < n) {
      total_ms[j] += ms;
      count[j] += 1;
    }
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_n_rec = 0;
  *n_names = n;
  return rc;
}

// Drives every entry point of the ABI's host code (abi.cpp, linked with the
// host-only stand-ins of stub_device.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer: valid calls on every path (decode of 1, 5 and
// 64 tokens on Q2_K, Q4_1 and mixed layers; prefill; the 43-layer stack with
// every layer steered, in both modes; routing outputs, imatrix, the static
// scratch, timing records past their capacity) and invalid ones.  Buffers the
// host code may touch (workspaces, routing outputs) are real host
// allocations of the documented sizes; weight tensors, which the host code
// only does address arithmetic on, are fake aligned addresses.  Exits 0 when
// every status is the expected one.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/ds4q.h"

extern long g_launches;
static int g_fail = 0;
#define EXPECT(call, want)                                                          \
  do {                                                                              \
    const int rc_ = (call);                                                         \
    if (rc_ != (want)) {                                                            \
      fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, rc_, (want)); \
      g_fail = 1;                                                                   \
    }                                                                               \
  } while (0)

static void *fake(int i) { return (void *)(uintptr_t)((uint64_t)(i + 1) << 40); }

struct Buf {
  void *p = nullptr;
  // exactly n bytes (the sanitizer's redzone starts right after them), 256-byte aligned
  explicit Buf(size_t n) {
    if (posix_memalign(&p, 256, n ? n : 1)) abort();
    memset(p, 0, n);
  }
  ~Buf() { free(p); }
  template <class T> T *as() const { return static_cast<T *>(p); }
};

static ds4q_moe_layer layer(int tg, int td, int D = 4096, int F = 2048, int E = 256, int k = 6) {
  ds4q_moe_layer L;
  memset(&L, 0, sizeof L);
  L.n_embd = D; L.n_ff = F; L.n_expert = E; L.n_expert_used = k;
  L.type_gate = L.type_up = tg; L.type_down = td;
  L.gate = fake(1); L.up = fake(2); L.down = fake(3);
  L.norm_eps = 1e-6f;
  return L;
}

static void decode_case(int tg, int td, int T, bool steer, bool stats) {
  ds4q_moe_layer L = layer(tg, td);
  Buf x((size_t)T * 4096 * 4), y((size_t)T * 4096 * 4), lg((size_t)T * 256 * 4), dir(4096 * 4);
  Buf si(256 * 4096 * 4), sd(256 * 2048 * 4);
  if (steer) { L.steer_dir = dir.as<float>(); L.steer_scale = 0.5f; }
  if (stats) { L.imatrix_in = si.as<float>(); L.imatrix_down = sd.as<float>(); }
  const size_t wb = ds4q_moe_workspace_size(&L, T, 0);
  Buf ws(wb);
  Buf ids((size_t)T * 6 * 4), w((size_t)T * 6 * 4), cnt(256 * 4), off(257 * 4), pairs((size_t)T * 6 * 4);
  ds4q_route_out r = {ids.as<int32_t>(), w.as<float>(), cnt.as<int32_t>(), off.as<int32_t>(), pairs.as<int32_t>()};
  L.flags = DS4Q_F_RMSNORM_INPUT;
  EXPECT(ds4q_moe_decode(&L, x.as<float>(), lg.as<float>(), T, y.as<float>(), &r, ws.p, wb, nullptr), DS4Q_OK);
  L.flags = DS4Q_F_ACCUMULATE;
  EXPECT(ds4q_moe_decode(&L, x.as<float>(), lg.as<float>(), T, x.as<float>(), &r, ws.p, wb, nullptr), DS4Q_OK);
  for (uint32_t ph : {DS4Q_PHASE_ROUTE, DS4Q_PHASE_GATEUP, DS4Q_PHASE_DOWN})
    EXPECT(ds4q_moe_decode_phases(&L, x.as<float>(), lg.as<float>(), T, y.as<float>(), &r, ws.p, wb, ph, nullptr),
           DS4Q_OK);
  EXPECT(ds4q_moe_decode(&L, x.as<float>(), lg.as<float>(), T, y.as<float>(), &r, ws.p, wb - 1, nullptr),
         DS4Q_E_WORKSPACE);
  EXPECT(ds4q_moe_decode_static(&L, x.as<float>(), lg.as<float>(), T, y.as<float>(), &r, nullptr), DS4Q_OK);
}

static void prefill_case(int tg, int td, int T, bool steer, bool stats) {
  ds4q_moe_layer L = layer(tg, td);
  Buf x((size_t)T * 4096 * 4), y((size_t)T * 4096 * 4), lg((size_t)T * 256 * 4), dir(4096 * 4);
  Buf si(256 * 4096 * 4), sd(256 * 2048 * 4);
  if (steer) { L.steer_dir = dir.as<float>(); L.steer_scale = -0.5f; }
  if (stats) { L.imatrix_in = si.as<float>(); L.imatrix_down = sd.as<float>(); }
  const size_t wb = ds4q_moe_workspace_size(&L, T, 1);
  Buf ws(wb);
  Buf ids((size_t)T * 6 * 4), cnt(256 * 4), off(257 * 4), pairs((size_t)T * 6 * 4);
  ds4q_route_out r = {ids.as<int32_t>(), nullptr, cnt.as<int32_t>(), off.as<int32_t>(), pairs.as<int32_t>()};
  EXPECT(ds4q_moe_prefill(&L, x.p, DS4Q_TYPE_BF16, lg.as<float>(), T, y.as<float>(), &r, ws.p, wb, nullptr), DS4Q_OK);
  L.flags = DS4Q_F_RMSNORM_INPUT | DS4Q_F_ACCUMULATE;
  EXPECT(ds4q_moe_prefill(&L, x.p, DS4Q_TYPE_F32, lg.as<float>(), T, x.as<float>(), nullptr, ws.p, wb, nullptr), DS4Q_OK);
  EXPECT(ds4q_moe_prefill(&L, x.p, DS4Q_TYPE_BF16, lg.as<float>(), T, y.as<float>(), &r, ws.p, wb, nullptr),
         DS4Q_E_INVAL);  // bf16 input with RMSNORM_INPUT
}

static void stack_case(int mode, int T) {
  const int NL = 43;
  std::vector<ds4q_moe_layer> lays;
  Buf dirs((size_t)NL * 4096 * 4), x((size_t)T * 4096 * 4), lg((size_t)NL * T * 256 * 4);
  for (int l = 0; l < NL; ++l) {
    ds4q_moe_layer L = layer(l < 37 ? DS4Q_TYPE_Q2_K : DS4Q_TYPE_Q4_1, l < 37 ? DS4Q_TYPE_Q2_K : DS4Q_TYPE_Q4_1);
    L.gate = fake(10 + 3 * l); L.up = fake(11 + 3 * l); L.down = fake(12 + 3 * l);
    L.steer_dir = dirs.as<float>() + (size_t)l * 4096;
    L.steer_scale = 1.0f;
    lays.push_back(L);
  }
  size_t wb = 0;
  for (const auto &L : lays) {
    const size_t b = ds4q_moe_workspace_size(&L, T, mode);
    wb = b > wb ? b : wb;
  }
  Buf ws(wb);
  EXPECT(ds4q_moe_stack(lays.data(), NL, mode, x.as<float>(), lg.as<float>(), T, ws.p, wb, nullptr), DS4Q_OK);
  EXPECT(ds4q_moe_stack(lays.data(), NL, mode, x.as<float>(), lg.as<float>(), T, ws.p, wb - 256, nullptr),
         DS4Q_E_WORKSPACE);
  lays[7].n_ff = 1024;
  EXPECT(ds4q_moe_stack(lays.data(), NL, mode, x.as<float>(), lg.as<float>(), T, ws.p, wb, nullptr), DS4Q_E_SHAPE);
}

int main() {
  // timing records on while everything runs, read at the end
  EXPECT(ds4q_timing_enable(1), DS4Q_OK);
  for (int tg : {DS4Q_TYPE_Q2_K, DS4Q_TYPE_Q4_1})
    for (int td : {DS4Q_TYPE_Q2_K, DS4Q_TYPE_Q4_1})
      for (int T : {1, 5, 64}) decode_case(tg, td, T, T != 5, T != 1);
  for (int tg : {DS4Q_TYPE_Q2_K, DS4Q_TYPE_Q4_1})
    for (int T : {1, 300, 4096}) prefill_case(tg, tg, T, T == 300, T != 1);
  stack_case(0, 1);
  stack_case(1, 64);
  {
    // routing alone, dequant, matvec, steering, codec
    Buf lg(4096 * 256 * 4), ws(ds4q_route_workspace_size(4096, 256, 6));
    Buf ids(4096 * 6 * 4), w(4096 * 6 * 4), cnt(256 * 4), off(257 * 4), pairs(4096 * 6 * 4);
    ds4q_route_out r = {ids.as<int32_t>(), w.as<float>(), cnt.as<int32_t>(), off.as<int32_t>(), pairs.as<int32_t>()};
    EXPECT(ds4q_route(lg.as<float>(), 4096, 256, 6, &r, ws.p, ds4q_route_workspace_size(4096, 256, 6), nullptr), DS4Q_OK);
    EXPECT(ds4q_dequant(DS4Q_TYPE_Q2_K, fake(1), 2048, 4096, DS4Q_TYPE_F32, fake(2), nullptr), DS4Q_OK);
    EXPECT(ds4q_matvec(DS4Q_TYPE_Q4_1, fake(1), 2048, 4096, (const float *)fake(2), 3, (float *)fake(3), nullptr), DS4Q_OK);
    EXPECT(ds4q_steer((const float *)fake(1), 0.5f, (const float *)fake(2), 7, 4096, (float *)fake(3), DS4Q_F_ACCUMULATE, nullptr), DS4Q_OK);
    EXPECT(ds4q_act_encode((const float *)fake(1), 1000, 8, fake(2), nullptr), DS4Q_OK);
    EXPECT(ds4q_act_decode(fake(2), 1000, 16, (float *)fake(1), nullptr), DS4Q_OK);
    EXPECT(ds4q_act_encode((const float *)fake(1), 1000, 12, fake(2), nullptr), DS4Q_E_INVAL);
  }
  // more launches than the timing record holds (65536): the rest are not recorded
  for (int i = 0; i < 70000; ++i)
    EXPECT(ds4q_act_encode((const float *)fake(1), 16, 32, fake(2), nullptr), DS4Q_OK);
  char names[32 * 32];
  double ms[32];
  int64_t count[32];
  int n = 0;
  EXPECT(ds4q_timing_read(names, 32, ms, count, 32, &n), DS4Q_OK);
  int64_t total = 0;
  for (int i = 0; i < n; ++i) total += count[i];
  if (n <= 0 || total != 65536) { fprintf(stderr, "timing records: %d names, %lld launches\n", n, (long long)total); g_fail = 1; }
  EXPECT(ds4q_timing_read(names, 32, ms, count, 32, &n), DS4Q_OK);
  if (n != 0) { fprintf(stderr, "timing record not cleared\n"); g_fail = 1; }
  EXPECT(ds4q_timing_enable(0), DS4Q_OK);
  printf("%s: %ld launches\n", g_fail ? "FAIL" : "ok", g_launches);
  return g_fail;
}

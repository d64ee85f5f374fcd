/* Drives the oracle's functions on small inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure only).  Exits 0 when every
 * call returns its success status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/ds4q_oracle.h"

static uint64_t s = 88172645463325252ull;
static uint32_t rnd(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return (uint32_t)s; }
static void fill(uint8_t *p, size_t n) { for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)rnd(); }
static void fillf(float *p, size_t n) { for (size_t i = 0; i < n; ++i) p[i] = ((int)(rnd() % 2001) - 1000) / 500.0f; }

int main(void) {
  int fail = 0;
  const int D = 512, F = 256, E = 8, k = 3, T = 5, L = 2;
  for (int type = 0; type < 2; ++type) {
    const int qt = type ? ORC_Q4_1 : ORC_Q2_K, qk = type ? 32 : 256, bb = type ? 20 : 84;
    /* d and dmin fields stay finite: random bits may be NaN, which is fine
       for the oracle but keep the run free of float-cast-overflow reports */
    const size_t gb = (size_t)E * F * (D / qk) * bb, db = (size_t)E * D * (F / qk) * bb;
    uint8_t *g = malloc(gb * L), *u = malloc(gb * L), *d = malloc(db * L);
    fill(g, gb * L); fill(u, gb * L); fill(d, db * L);
    for (size_t b = 0; b < gb * L / bb; ++b) {
      uint8_t *pg = g + b * bb + (type ? 0 : 80), *pu = u + b * bb + (type ? 0 : 80);
      pg[1] &= 0x3B; pg[3] &= 0x3B; pu[1] &= 0x3B; pu[3] &= 0x3B;  /* small exponents */
    }
    for (size_t b = 0; b < db * L / bb; ++b) {
      uint8_t *pd = d + b * bb + (type ? 0 : 80);
      pd[1] &= 0x3B; pd[3] &= 0x3B;
    }
    float *x = malloc(sizeof(float) * T * D), *lg = malloc(sizeof(float) * L * T * E);
    fillf(x, (size_t)T * D); fillf(lg, (size_t)L * T * E);
    float *deq = malloc(sizeof(float) * F * D);
    uint16_t *deqb = malloc(2 * (size_t)F * D);
    double *y = malloc(sizeof(double) * T * D), *ia = calloc((size_t)E * D, 8), *id = calloc((size_t)E * F, 8);
    if (orc_dequant_f32(qt, g, F, D, deq) || orc_dequant_bf16(qt, g, F, D, deqb)) fail = 1;
    if (orc_matvec(qt, g, F, D, x, y)) fail = 1;
    orc_layer lay[2];
    for (int l = 0; l < L; ++l) {
      lay[l].n_embd = D; lay[l].n_ff = F; lay[l].n_expert = E; lay[l].n_expert_used = k;
      lay[l].type_gate = lay[l].type_up = lay[l].type_down = qt;
      lay[l].gate = g + l * gb; lay[l].up = u + l * gb; lay[l].down = d + l * db;
    }
    if (orc_moe(&lay[0], x, lg, T, y, 2)) fail = 1;
    if (orc_moe_imatrix(&lay[0], x, lg, T, ia, id, 2)) fail = 1;
    float *dirs = malloc(sizeof(float) * L * D);
    fillf(dirs, (size_t)L * D);
    if (orc_stack(lay, L, type, x, lg, T, 1e-6, 2, dirs, 0.5)) fail = 1;
    if (orc_stack(lay, L, 0, x, lg, T, 1e-6, 2, NULL, 0.0)) fail = 1;
    int32_t ids[T * 3], cnt[E], off[E + 1], pairs[T * 3];
    double w[T * 3];
    orc_route(lg, T, E, k, ids, w);
    orc_group(ids, T, k, E, cnt, off, pairs);
    float *yo = malloc(sizeof(float) * T * D);
    orc_steer(dirs, 0.25, x, T, D, x, yo);
    orc_steer_f64(dirs, 0.25, y, T, D);
    free(g); free(u); free(d); free(x); free(lg); free(deq); free(deqb); free(y); free(ia); free(id);
    free(dirs); free(yo);
  }
  /* block codecs, the re-encode and the wire formats */
  uint8_t sc[16], mn[16], q[256], blk[84], q4[32], b41[20];
  for (int i = 0; i < 16; ++i) { sc[i] = rnd() & 15; mn[i] = rnd() & 15; }
  for (int i = 0; i < 256; ++i) q[i] = rnd() & 3;
  for (int i = 0; i < 32; ++i) q4[i] = rnd() & 15;
  orc_q2k_encode_block(sc, mn, q, 0x3c00, 0x3800, blk);
  orc_q41_encode_block(q4, 0x3c00, 0xb800, b41);
  float out[256];
  orc_q2k_decode_block(blk, out);
  orc_q41_decode_block(b41, out);
  uint8_t codes[128];
  uint16_t scl[4], mns[4];
  for (int i = 0; i < 128; ++i) codes[i] = rnd() & 7;
  for (int i = 0; i < 4; ++i) { scl[i] = 0x3400; mns[i] = 0xb400; }
  uint8_t re[4 * 20];
  if (orc_q41_reencode(codes, scl, mns, 128, 32, 3, re)) fail = 1;
  for (int i = 0; i < 100000; ++i) {
    uint32_t bits = rnd();
    float f;
    memcpy(&f, &bits, 4);
    (void)orc_f16_rne(f);
    (void)orc_e4m3_rne(f);
    (void)orc_e4m3_value((uint8_t)bits);
    (void)orc_f16_value((uint16_t)bits);
    (void)orc_bf16_rne(f);
  }
  printf("%s\n", fail ? "FAIL" : "ok");
  return fail;
}

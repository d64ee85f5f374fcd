/* ds4q oracle — TEST INFRASTRUCTURE ONLY (see ds4q_oracle.h for sources and
 * the readings taken).  Plain, slow, fp64, no blocking or fusion beyond what
 * each definition states.  Threads (OpenMP) only split independent rows or
 * tokens; every output element is summed sequentially by one thread. */
#include "ds4q_oracle.h"
#include <math.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE binary16 by definition: sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 = subnormal, 31 = Inf/NaN. */
double orc_f16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* float32 -> bfloat16, round to nearest even; NaN stays a (quiet) NaN. */
uint16_t orc_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void orc_f32_to_bf16(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(in[i]);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* [P1] Q2_K layout table: scales @0 (16 B, one scale/min nibble byte per
 * 16-value sub-block), qs @16 (64 B of 2-bit codes), d @80, dmin @82 (fp16).
 * [P1] packing expression: byte qs[j/4 + l] (j = 0 or 128, l = 0..31) holds
 * codes L[j+l], L[j+l+32], L[j+l+64], L[j+l+96] at bit offsets 0, 2, 4, 6.
 * Value = fl32(d*sc*q - dmin*mn): the products are exact in double, so the
 * only rounding is the final cast. */
void orc_q2k_decode_block(const uint8_t *blk, float out[256]) {
  const uint8_t *scales = blk, *qs = blk + 16;
  double d = orc_f16_value(rd16(blk + 80));
  double dmin = orc_f16_value(rd16(blk + 82));
  for (int j = 0; j < 256; j += 128) {
    for (int l = 0; l < 32; ++l) {
      uint8_t byte = qs[j / 4 + l];
      for (int pair = 0; pair < 4; ++pair) {
        int e = j + l + 32 * pair;
        int q = (byte >> (2 * pair)) & 3;
        int s = e / 16;
        int sc = scales[s] & 15, mn = scales[s] >> 4;
        out[e] = (float)(d * sc * q - dmin * mn);
      }
    }
  }
}

/* [P5] Q4_1 block section: fp16 d, fp16 m, uint8 qs[16] (20 B, 32 values);
 * low nibble of qs[j] is value j, high nibble is value j+16; y = d*q + m. */
void orc_q41_decode_block(const uint8_t *blk, float out[32]) {
  double d = orc_f16_value(rd16(blk));
  double m = orc_f16_value(rd16(blk + 2));
  for (int j = 0; j < 16; ++j) {
    out[j] = (float)(d * (blk[4 + j] & 15) + m);
    out[j + 16] = (float)(d * (blk[4 + j] >> 4) + m);
  }
}

static int type_geom(int type, int64_t *qk, int64_t *bytes) {
  if (type == ORC_Q2_K) { *qk = 256; *bytes = 84; return 0; }
  if (type == ORC_Q4_1) { *qk = 32; *bytes = 20; return 0; }
  return -1;
}

/* Element (r, c) of a [rows][cols] tensor is value c % QK of block c / QK of
 * row r; rows are stored one after another (GGUF: ne[0] is the input dim). */
int orc_dequant_f32(int type, const uint8_t *src, int64_t rows, int64_t cols, float *dst) {
  int64_t qk, bb;
  if (type_geom(type, &qk, &bb) || cols % qk) return -1;
  int64_t nb = cols / qk;
  float tmp[256];
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t *blk = src + (r * nb + b) * bb;
      if (type == ORC_Q2_K) orc_q2k_decode_block(blk, tmp);
      else orc_q41_decode_block(blk, tmp);
      memcpy(dst + r * cols + b * qk, tmp, (size_t)qk * sizeof(float));
    }
  return 0;
}

int orc_dequant_bf16(int type, const uint8_t *src, int64_t rows, int64_t cols, uint16_t *dst) {
  int64_t qk, bb;
  if (type_geom(type, &qk, &bb) || cols % qk) return -1;
  float *tmp = (float *)malloc((size_t)(rows * cols) * sizeof(float));
  if (!tmp) return -2;
  orc_dequant_f32(type, src, rows, cols, tmp);
  orc_f32_to_bf16(tmp, dst, rows * cols);
  free(tmp);
  return 0;
}

/* Inverse of orc_q2k_decode_block's byte reading: the [P1] packing with the
 * fourth bit pair at << 6. */
void orc_q2k_encode_block(const uint8_t sc[16], const uint8_t mn[16], const uint8_t q[256],
                          uint16_t d_bits, uint16_t dmin_bits, uint8_t out[84]) {
  for (int s = 0; s < 16; ++s) out[s] = (uint8_t)((sc[s] & 15) | ((mn[s] & 15) << 4));
  for (int j = 0; j < 256; j += 128)
    for (int l = 0; l < 32; ++l)
      out[16 + j / 4 + l] = (uint8_t)((q[j + l] & 3) | ((q[j + l + 32] & 3) << 2) |
                                      ((q[j + l + 64] & 3) << 4) | ((q[j + l + 96] & 3) << 6));
  out[80] = (uint8_t)(d_bits & 0xFF); out[81] = (uint8_t)(d_bits >> 8);
  out[82] = (uint8_t)(dmin_bits & 0xFF); out[83] = (uint8_t)(dmin_bits >> 8);
}

void orc_q41_encode_block(const uint8_t q[32], uint16_t d_bits, uint16_t m_bits, uint8_t out[20]) {
  out[0] = (uint8_t)(d_bits & 0xFF); out[1] = (uint8_t)(d_bits >> 8);
  out[2] = (uint8_t)(m_bits & 0xFF); out[3] = (uint8_t)(m_bits >> 8);
  for (int j = 0; j < 16; ++j) out[4 + j] = (uint8_t)((q[j] & 15) | ((q[j + 16] & 15) << 4));
}

/* [P5] lossless re-encode: valid only when the group size is a multiple of 32
 * and codes have at most 4 bits (section on the two lossless conditions).  Each
 * group's fp16 (scale, min) is copied into every 32-value block the group
 * spans; codes fold into nibbles (low = j, high = j+16).  Returns -1 (no
 * fallback) when a condition fails or a code exceeds the nibble. */
int orc_q41_reencode(const uint8_t *codes, const uint16_t *scale, const uint16_t *mins,
                     int64_t n_values, int group, int bits, uint8_t *out) {
  if (group <= 0 || group % 32 || bits < 1 || bits > 4 || n_values % group) return -1;
  int64_t nb = n_values / 32;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t g = (b * 32) / group;
    for (int j = 0; j < 32; ++j)
      if (codes[b * 32 + j] >= (1u << bits)) return -1;
    orc_q41_encode_block(codes + b * 32, scale[g], mins[g], out + b * 20);
  }
  return 0;
}

/* y_r = sum_c w_rc * x_c, summed in fp64 in column order. */
int orc_matvec(int type, const uint8_t *w, int64_t rows, int64_t cols, const float *x, double *y) {
  int64_t qk, bb;
  if (type_geom(type, &qk, &bb) || cols % qk) return -1;
  int64_t nb = cols / qk;
  float tmp[256];
  for (int64_t r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t *blk = w + (r * nb + b) * bb;
      if (type == ORC_Q2_K) orc_q2k_decode_block(blk, tmp);
      else orc_q41_decode_block(blk, tmp);
      for (int64_t i = 0; i < qk; ++i) acc += (double)tmp[i] * (double)x[b * qk + i];
    }
    y[r] = acc;
  }
  return 0;
}

/* [P2] 6 of 256 routed experts per token.  Selection order (logit desc,
 * index asc); weights = softmax over the selected logits (max-subtracted). */
void orc_route(const float *logits, int32_t n_tok, int32_t n_expert, int32_t k,
               int32_t *ids, double *w) {
  char *taken = (char *)malloc((size_t)n_expert);
  for (int32_t t = 0; t < n_tok; ++t) {
    const float *l = logits + (int64_t)t * n_expert;
    memset(taken, 0, (size_t)n_expert);
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < n_expert; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      ids[t * k + j] = best;
    }
    double mx = l[ids[t * k]];
    double den = 0.0;
    for (int32_t j = 0; j < k; ++j) den += exp((double)l[ids[t * k + j]] - mx);
    for (int32_t j = 0; j < k; ++j) w[t * k + j] = exp((double)l[ids[t * k + j]] - mx) / den;
  }
  free(taken);
}

/* Token->expert grouping: counts per expert, exclusive offsets, and pair
 * indices p = token*k + slot ordered by (expert, token, slot). */
void orc_group(const int32_t *ids, int32_t n_tok, int32_t k, int32_t n_expert,
               int32_t *counts, int32_t *offsets, int32_t *pairs) {
  for (int32_t e = 0; e < n_expert; ++e) counts[e] = 0;
  for (int64_t p = 0; p < (int64_t)n_tok * k; ++p) counts[ids[p]]++;
  offsets[0] = 0;
  for (int32_t e = 0; e < n_expert; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t pos = 0;
  for (int32_t e = 0; e < n_expert; ++e)
    for (int64_t p = 0; p < (int64_t)n_tok * k; ++p)
      if (ids[p] == e) pairs[pos++] = (int32_t)p;
}

static int64_t tensor_bytes(int type, int64_t rows, int64_t cols) {
  int64_t qk, bb;
  if (type_geom(type, &qk, &bb) || cols % qk) return -1;
  return rows * (cols / qk) * bb;
}

static double dot_row(int type, const uint8_t *row, int64_t cols, const double *x) {
  int64_t qk = 1, bb = 0;
  if (type_geom(type, &qk, &bb)) return NAN;
  float tmp[256];
  double acc = 0.0;
  for (int64_t b = 0; b < cols / qk; ++b) {
    if (type == ORC_Q2_K) orc_q2k_decode_block(row + b * bb, tmp);
    else orc_q41_decode_block(row + b * bb, tmp);
    for (int64_t i = 0; i < qk; ++i) acc += (double)tmp[i] * x[b * qk + i];
  }
  return acc;
}

/* One routed expert on one token, all fp64: g = W1 x, u = W3 x,
 * h = silu(g) * u, o = W2 h  ([P1]: w1 = gate, w3 = up, w2 = down). */
/* The expert's SwiGLU row h = silu(W1 x) * (W3 x), [n_ff]. */
int orc_expert_swiglu(const orc_layer *L, int32_t e, const double *x, double *h) {
  int64_t D = L->n_embd, F = L->n_ff;
  int64_t gb = tensor_bytes(L->type_gate, F, D), ub = tensor_bytes(L->type_up, F, D);
  if (gb < 0 || ub < 0) return -1;
  const uint8_t *G = L->gate + e * gb, *U = L->up + e * ub;
  for (int64_t r = 0; r < F; ++r) {
    double g = dot_row(L->type_gate, G + r * (gb / F), D, x);
    double u = dot_row(L->type_up, U + r * (ub / F), D, x);
    h[r] = g / (1.0 + exp(-g)) * u;
  }
  return 0;
}

int orc_expert_ffn(const orc_layer *L, int32_t e, const double *x, double *o) {
  int64_t D = L->n_embd, F = L->n_ff;
  int64_t db = tensor_bytes(L->type_down, D, F);
  if (db < 0) return -1;
  const uint8_t *W2 = L->down + e * db;
  double *h = (double *)malloc((size_t)F * sizeof(double));
  int rc = orc_expert_swiglu(L, e, x, h);
  if (!rc)
    for (int64_t i = 0; i < D; ++i) o[i] = dot_row(L->type_down, W2 + i * (db / D), F, h);
  free(h);
  return rc;
}

/* y_t = sum over slots j (in slot order) of p_j * expert_{id_j}(x_t). */
int orc_moe(const orc_layer *L, const float *x, const float *logits, int32_t n_tok,
            double *y, int n_threads) {
  int32_t k = L->n_expert_used, E = L->n_expert, D = L->n_embd;
  if (tensor_bytes(L->type_gate, L->n_ff, D) < 0 || tensor_bytes(L->type_up, L->n_ff, D) < 0 ||
      tensor_bytes(L->type_down, D, L->n_ff) < 0)
    return -1;
  int32_t *ids = (int32_t *)malloc((size_t)n_tok * k * sizeof(int32_t));
  double *w = (double *)malloc((size_t)n_tok * k * sizeof(double));
  orc_route(logits, n_tok, E, k, ids, w);
  int rc = 0;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int32_t t = 0; t < n_tok; ++t) {
    double *xt = (double *)malloc((size_t)D * sizeof(double));
    double *o = (double *)malloc((size_t)D * sizeof(double));
    for (int32_t i = 0; i < D; ++i) xt[i] = x[(int64_t)t * D + i];
    for (int32_t i = 0; i < D; ++i) y[(int64_t)t * D + i] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      orc_expert_ffn(L, ids[t * k + j], xt, o);
      for (int32_t i = 0; i < D; ++i) y[(int64_t)t * D + i] += w[t * k + j] * o[i];
    }
    free(xt);
    free(o);
  }
  free(ids);
  free(w);
  return rc;
}

/* [P1] imatrix passage: the activation statistics collected on the routed
 * experts, per expert and input column, expert-major:
 *   imat_in   [n_expert][n_embd] += sum over the tokens routed to the expert
 *             of x[col]^2, x the MoE input row (one vector serves the gate and
 *             the up tensor, which read the same input);
 *   imat_down [n_expert][n_ff]   += sum over the same (token, slot) pairs of
 *             (p * h[col])^2, h the expert's SwiGLU row and p the pair's
 *             routing weight (the down projection's input).
 * fp64, tokens then slots in order; experts are independent (one thread
 * each). */
int orc_moe_imatrix(const orc_layer *L, const float *x, const float *logits, int32_t n_tok,
                    double *imat_in, double *imat_down, int n_threads) {
  int32_t k = L->n_expert_used, E = L->n_expert, D = L->n_embd, F = L->n_ff;
  if (tensor_bytes(L->type_gate, F, D) < 0 || tensor_bytes(L->type_up, F, D) < 0) return -1;
  int32_t *ids = (int32_t *)malloc((size_t)n_tok * k * sizeof(int32_t));
  double *w = (double *)malloc((size_t)n_tok * k * sizeof(double));
  orc_route(logits, n_tok, E, k, ids, w);
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int32_t e = 0; e < E; ++e) {
    double *xt = (double *)malloc((size_t)D * sizeof(double));
    double *h = (double *)malloc((size_t)F * sizeof(double));
    for (int32_t t = 0; t < n_tok; ++t)
      for (int32_t j = 0; j < k; ++j) {
        if (ids[t * k + j] != e) continue;
        for (int32_t i = 0; i < D; ++i) {
          xt[i] = x[(int64_t)t * D + i];
          imat_in[(int64_t)e * D + i] += xt[i] * xt[i];
        }
        orc_expert_swiglu(L, e, xt, h);
        for (int32_t i = 0; i < F; ++i) {
          const double v = w[t * k + j] * h[i];
          imat_down[(int64_t)e * F + i] += v * v;
        }
      }
    free(xt);
    free(h);
  }
  free(ids);
  free(w);
  return 0;
}

/* Parameter-free RMS norm: n = x / sqrt(mean(x^2) + eps). */
void orc_rmsnorm(const float *x, int32_t n, double eps, double *out) {
  double ss = 0.0;
  for (int32_t i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
  double r = 1.0 / sqrt(ss / n + eps);
  for (int32_t i = 0; i < n; ++i) out[i] = (double)x[i] * r;
}

/* Layer stack: x <- x + MoE_l(rmsnorm(x)) for l = 0..n_layers-1, with the
 * layer's own router logits ([n_layers][n_tok][n_expert]).  When
 * prefill_bf16 is set, the normalised input is rounded to fp32 then bf16
 * before the experts see it.  x is the fp32 residual stream, updated in place
 * (the sum x + y is rounded to fp32 after each layer). */
int orc_stack(const orc_layer *layers, int32_t n_layers, int prefill_bf16, float *x,
              const float *logits, int32_t n_tok, double eps, int n_threads,
              const float *dirs, double steer_scale) {
  int32_t D = layers[0].n_embd, E = layers[0].n_expert;
  float *n32 = (float *)malloc((size_t)n_tok * D * sizeof(float));
  double *nd = (double *)malloc((size_t)D * sizeof(double));
  double *y = (double *)malloc((size_t)n_tok * D * sizeof(double));
  int rc = 0;
  for (int32_t l = 0; l < n_layers && !rc; ++l) {
    for (int32_t t = 0; t < n_tok; ++t) {
      orc_rmsnorm(x + (int64_t)t * D, D, eps, nd);
      for (int32_t i = 0; i < D; ++i) {
        float v = (float)nd[i];
        if (prefill_bf16) {
          uint32_t u = (uint32_t)orc_bf16_rne(v) << 16;
          memcpy(&v, &u, 4);
        }
        n32[(int64_t)t * D + i] = v;
      }
    }
    rc = orc_moe(&layers[l], n32, logits + (int64_t)l * n_tok * E, n_tok, y, n_threads);
    /* [P3]: the layer's own direction (row l of the layer-major table) is
     * projected out of its FFN output before the residual add */
    if (dirs) orc_steer_f64(dirs + (int64_t)l * D, steer_scale, y, n_tok, D);
    for (int64_t i = 0; i < (int64_t)n_tok * D; ++i) x[i] = (float)((double)x[i] + y[i]);
  }
  free(n32);
  free(nd);
  free(y);
  return rc;
}

/* ---------------------------------------------------------------- steering
 * [P3] directional-steering section: the projection of the layer's direction
 * is subtracted from the FFN output, y - scale * dir * (dir . y). */
void orc_steer(const float *dir, double scale, const float *y, int32_t n_rows, int32_t n,
               const float *residual, float *out) {
  for (int32_t r = 0; r < n_rows; ++r) {
    const float *yr = y + (int64_t)r * n;
    double d = 0.0;
    for (int32_t i = 0; i < n; ++i) d += (double)dir[i] * (double)yr[i];
    for (int32_t i = 0; i < n; ++i) {
      double v = (double)yr[i] - scale * (double)dir[i] * d;
      if (residual) v += (double)residual[(int64_t)r * n + i];
      out[(int64_t)r * n + i] = (float)v;
    }
  }
}

void orc_steer_f64(const float *dir, double scale, double *y, int32_t n_rows, int32_t n) {
  for (int32_t r = 0; r < n_rows; ++r) {
    double *yr = y + (int64_t)r * n;
    double d = 0.0;
    for (int32_t i = 0; i < n; ++i) d += (double)dir[i] * yr[i];
    for (int32_t i = 0; i < n; ++i) yr[i] -= scale * (double)dir[i] * d;
  }
}

/* ---------------------------------------------------------------- codec
 * [P4] distributed-transport passage: 32-bit floats, or 16 bits (f16) or
 * 8 bits (E4M3) on the wire, decoded back to float by the receiver.
 *
 * Both encoders take the value of the fp32 input exactly (as a double) and
 * pick the representable neighbour by comparing distances: a plain
 * statement of round-to-nearest-even over the target grid. */

/* Round |v| (finite, >= 0) to the grid m * 2^e, m integer, ties to even m. */
static double round_grid(double v, int e) {
  const double m = ldexp(v, -e);
  double f = floor(m);
  const double r = m - f;
  if (r > 0.5 || (r == 0.5 && fmod(f, 2.0) != 0.0)) f += 1.0;
  return ldexp(f, e);
}

uint16_t orc_f16_rne(float f) {
  const double v = (double)f;
  const uint16_t sign = signbit(f) ? 0x8000u : 0u;
  if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
  const double a = fabs(v);
  if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
  /* binary16: normals (1 + m/1024) 2^(e-15), e = 1..30; subnormals m 2^-24 */
  int e2 = a > 0.0 ? ilogb(a) : -25;
  if (e2 < -14) e2 = -14;                 /* subnormal spacing 2^-24 */
  double q = round_grid(a, e2 - 10);      /* 10 fraction bits */
  if (q >= 65520.0 || q > 65504.0) return (uint16_t)(sign | 0x7C00u);
  if (q == 0.0) return sign;
  int eq = ilogb(q);
  if (eq < -14) return (uint16_t)(sign | (uint16_t)ldexp(q, 24));  /* subnormal */
  const uint16_t mant = (uint16_t)(ldexp(q, 10 - eq) - 1024.0);
  return (uint16_t)(sign | (uint16_t)((eq + 15) << 10) | mant);
}

double orc_e4m3_value(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexp((double)m, -9);         /* subnormal: m/8 * 2^-6 */
  else v = ldexp((double)(8 + m), e - 10);           /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

uint8_t orc_e4m3_rne(float f) {
  const uint8_t sign = signbit(f) ? 0x80u : 0u;
  if (isnan(f)) return (uint8_t)(sign | 0x7Fu);
  const double a = fabs((double)f);
  if (isinf(f) || a >= 464.0) return (uint8_t)(sign | 0x7Eu); /* 464 = midpoint 448|480: even -> 480 out of range */
  int e2 = a > 0.0 ? ilogb(a) : -10;
  if (e2 < -6) e2 = -6;                   /* subnormal spacing 2^-9 */
  double q = round_grid(a, e2 - 3);       /* 3 fraction bits */
  if (q > 448.0) return (uint8_t)(sign | 0x7Eu);
  if (q == 0.0) return sign;
  int eq = ilogb(q);
  if (eq < -6) return (uint8_t)(sign | (uint8_t)ldexp(q, 9));    /* subnormal */
  const uint8_t mant = (uint8_t)(ldexp(q, 3 - eq) - 8.0);
  return (uint8_t)(sign | (uint8_t)((eq + 7) << 3) | mant);
}

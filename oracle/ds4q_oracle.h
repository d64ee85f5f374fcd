/* ds4q oracle — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, CPU-only fp64 statement of what the routed-MoE expert path on
 * Q2_K / Q4_1 weights computes.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code with the GPU
 * library and includes none of its headers.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "【#2】ds4.c 해독하기" (molayo1419.me) — Q2_K layout table and
 *       the code-packing expression; routed-expert tensors w1=gate, w2=down,
 *       w3=up; imatrix passage saying the down input is the routed SwiGLU row
 *       after the routing weight.
 *  [P2] "ds4.c 해독하기 1/8" (molayo1419.me) — DS4_SHAPE_FLASH passage:
 *       256 routed experts, 6 used per token.
 *  [P3] "【#8】ds4.c 해독하기" (molayo1419.me) — directional steering: per
 *       layer a direction dir, applied to the FFN output as
 *       y - scale * dir * (dir . y).
 *  [P4] "【#6】ds4.c 분석하기" (molayo1419.me) — distributed transport: the
 *       activations between graph slices travel as 32-bit floats or are
 *       packed to 16 bits (f16) or 8 bits (E4M3) and decoded back to float.
 *  [P5] "자체 저비트 포맷을 llama.cpp로 옮기기: 복원값이 비트까지 같은 GGUF Q4_1
 *       재부호화" (ThakiCloud) — section on the Q4_1 block (struct, nibble
 *       order, y = d*q + m), section on the two lossless conditions, the
 *       q41_blocks code section, the read-back section.
 *
 * Readings taken where the pages are silent:
 *  - Q2_K value = d*sc*q - dmin*mn, sc = low nibble, mn = high nibble of the
 *    sub-block byte (the pages give only "scale/min nibble per 16 values").
 *  - 4th bit pair of the Q2_K pack = L[j+l+96] << 6 (elided on the page).
 *  - fp16 fields little-endian; fp32 value rounded once (RNE).
 *  - routing: top-k by (logit desc, index asc); weights = softmax over the k
 *    selected logits.
 *  - SwiGLU h = silu(gate) * up; expert output down*h; token output is the
 *    routing-weighted sum over slots in slot order.
 *  - stack: x_{l+1} = x_l + MoE_l(rmsnorm(x_l)), parameter-free RMS norm.
 *  - steering: the dot product and the update in fp64, one rounding to f32
 *    (optionally after adding to a residual row); dir used as given.
 *  - activation codec: f16 = IEEE binary16 with round-to-nearest-even,
 *    overflow to +-inf, NaN to the quiet NaN sign|0x7E00; E4M3 = the OCP
 *    8-bit E4M3 ("FN") encoding: bias 7, subnormals, no infinities, NaN =
 *    sign|0x7F, largest finite 448; round to nearest even, magnitudes that
 *    round beyond 448 (and +-inf) saturate to +-448, NaN to sign|0x7F.
 */
#ifndef DS4Q_ORACLE_H
#define DS4Q_ORACLE_H
#include <stdint.h>
#include <stddef.h>
#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_Q4_1 = 3, ORC_Q2_K = 10 };

double orc_f16_value(uint16_t h);
uint16_t orc_bf16_rne(float f);
void orc_f32_to_bf16(const float *in, uint16_t *out, int64_t n);

void orc_q2k_decode_block(const uint8_t *blk, float out[256]);
void orc_q41_decode_block(const uint8_t *blk, float out[32]);
int orc_dequant_f32(int type, const uint8_t *src, int64_t rows, int64_t cols, float *dst);
int orc_dequant_bf16(int type, const uint8_t *src, int64_t rows, int64_t cols, uint16_t *dst);

void orc_q2k_encode_block(const uint8_t sc[16], const uint8_t mn[16], const uint8_t q[256],
                          uint16_t d_bits, uint16_t dmin_bits, uint8_t out[84]);
void orc_q41_encode_block(const uint8_t q[32], uint16_t d_bits, uint16_t m_bits, uint8_t out[20]);
int orc_q41_reencode(const uint8_t *codes, const uint16_t *scale, const uint16_t *mins,
                     int64_t n_values, int group, int bits, uint8_t *out);

int orc_matvec(int type, const uint8_t *w, int64_t rows, int64_t cols,
               const float *x, double *y);

void orc_route(const float *logits, int32_t n_tok, int32_t n_expert, int32_t k,
               int32_t *ids, double *w);
void orc_group(const int32_t *ids, int32_t n_tok, int32_t k, int32_t n_expert,
               int32_t *counts, int32_t *offsets, int32_t *pairs);

typedef struct {
  int32_t n_embd, n_ff, n_expert, n_expert_used;
  int32_t type_gate, type_up, type_down;
  const uint8_t *gate, *up, *down;   /* [n_expert][rows][blocks] */
} orc_layer;

int orc_expert_swiglu(const orc_layer *L, int32_t e, const double *x, double *h);
int orc_expert_ffn(const orc_layer *L, int32_t e, const double *x, double *o);
/* [P1] imatrix statistics of one layer call on MoE input rows x (see the .c). */
int orc_moe_imatrix(const orc_layer *L, const float *x, const float *logits, int32_t n_tok,
                    double *imat_in, double *imat_down, int n_threads);
int orc_moe(const orc_layer *L, const float *x, const float *logits, int32_t n_tok,
            double *y, int n_threads);
void orc_rmsnorm(const float *x, int32_t n, double eps, double *out);
/* dirs (nullable): layer-major steering directions [n_layers][n_embd]; when
 * given, layer l's MoE output is steered with dirs + l*n_embd and
 * steer_scale (fp64, before the residual add). */
int orc_stack(const orc_layer *layers, int32_t n_layers, int prefill_bf16, float *x,
              const float *logits, int32_t n_tok, double eps, int n_threads,
              const float *dirs, double steer_scale);

/* [P3] directional steering: out_r (+)= y_r - scale * dir * (dir . y_r)
 * for each row r of y [n_rows][n]; residual (nullable) is added first. */
void orc_steer(const float *dir, double scale, const float *y, int32_t n_rows, int32_t n,
               const float *residual, float *out);
/* The same on fp64 rows, in place, without rounding. */
void orc_steer_f64(const float *dir, double scale, double *y, int32_t n_rows, int32_t n);

/* [P4] activation wire formats. */
uint16_t orc_f16_rne(float f);
uint8_t orc_e4m3_rne(float f);
double orc_e4m3_value(uint8_t b);

#ifdef __cplusplus
}
#endif
#endif

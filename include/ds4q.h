/* ds4q — routed-MoE expert FFN on Q2_K / Q4_1 block-quantised weights for
 * AMD Instinct MI355X (gfx950).  C ABI of libds4q.so.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "【#2】ds4.c 해독하기" (molayo1419.me): the Q2_K block-layout table
 *       (scales @0, qs @16, d @80, dmin @82; 256 values in 84 B) and the
 *       printed code-packing expression; routed-expert tensors
 *       blk.N.ffn_{gate,up,down}_exps with w1 = gate, w2 = down, w3 = up;
 *       the imatrix passage stating that the down projection's input is the
 *       routed SwiGLU row after the routing weight.
 *  [P2] "ds4.c 해독하기 1/8" (molayo1419.me): the DS4_SHAPE_FLASH passage —
 *       256 routed experts per layer, 6 used per token, 43 layers.
 *  [P5] ThakiCloud, "자체 저비트 포맷을 llama.cpp로 옮기기: 복원값이 비트까지
 *       같은 GGUF Q4_1 재부호화": the Q4_1 block section (fp16 d, fp16 m,
 *       qs[16]; low nibble = value j, high nibble = value j+16;
 *       y = d*q + m); the section on reading bits/group from metadata, never
 *       from byte counts; the raw_shape section (byte shape vs element shape);
 *       the tensor-name section (GGUF ne[0] is the input dimension).
 *
 * Conventions for every entry point:
 *  - Types are always explicit (never inferred from a byte count, [P5]).
 *  - Shapes are ELEMENT shapes; the library derives byte strides
 *    (row bytes = cols / QK * block_bytes).  A matrix [rows][cols] stores its
 *    rows one after another, each row a run of blocks along cols (the input
 *    dimension, [P5]).  An expert tensor is [n_expert][rows][cols], expert
 *    major ([P1] ffn_*_exps).
 *  - Every pointer argument named *_dev or documented "device" is device memory
 *    the caller owns; the library allocates no device memory and keeps no
 *    device state, except one static scratch array per device that only
 *    ds4q_moe_decode_static uses.  Structs are read on the host during the
 *    call only.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; the call returns once it is enqueued.
 *  - All validation happens on the host before anything is enqueued; on an
 *    error nothing is launched.  Block contents are never validated: every bit
 *    pattern is a valid block, and NaN/Inf in fp16 fields propagate.
 *  - Calls on distinct streams with disjoint outputs and workspaces may run
 *    concurrently.
 */
#ifndef DS4Q_H
#define DS4Q_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

#define DS4Q_ABI_VERSION 6

/* Tensor types.  Numeric values follow the public GGML/GGUF type ids. */
typedef enum {
  DS4Q_TYPE_F32 = 0,
  DS4Q_TYPE_F16 = 1,      /* not accepted by any entry point */
  DS4Q_TYPE_Q4_1 = 3,     /* 32 values in 20 B, [P5] */
  DS4Q_TYPE_Q2_K = 10,    /* 256 values in 84 B, [P1] */
  DS4Q_TYPE_IQ2_XXS = 16, /* known but unsupported: its grid codebook is not on the pages */
  DS4Q_TYPE_BF16 = 30
} ds4q_type;

/* Status codes (0 = success, negative = error). */
enum {
  DS4Q_OK = 0,
  DS4Q_E_INVAL = -1,        /* NULL pointer, negative size, bad k / n_expert, unknown flag */
  DS4Q_E_UNSUPPORTED = -2,  /* type not handled (IQ2_XXS, F16, unknown); no fallback path */
  DS4Q_E_SHAPE = -3,        /* cols not a multiple of the block size, or a shape the path does not take */
  DS4Q_E_ALIGN = -4,        /* a pointer misses its required alignment */
  DS4Q_E_WORKSPACE = -5,    /* workspace NULL or smaller than ds4q_moe_workspace_size() */
  DS4Q_E_ALIAS = -6,        /* an output overlaps an input or the workspace */
  DS4Q_E_HIP = -7,          /* a HIP runtime call or launch failed */
  DS4Q_E_SCRATCH = -8       /* the call needs more than DS4Q_SCRATCH_BYTES of static scratch */
};

/* Flags of ds4q_moe_layer.flags. */
#define DS4Q_F_ACCUMULATE 0x1u    /* y += MoE(x) instead of y = MoE(x) */
#define DS4Q_F_RMSNORM_INPUT 0x2u /* experts see x / sqrt(mean(x^2) + norm_eps) (per token) */

/* One routed-MoE layer.  gate/up: [n_expert][n_ff][n_embd]; down:
 * [n_expert][n_embd][n_ff] (element shapes; rows run along the last index).
 * w1 = gate, w3 = up, w2 = down ([P1]).  Each tensor is Q2_K or Q4_1; gate
 * and up must share a type, down may differ.  Device pointers, 16-byte
 * aligned.  n_embd and n_ff each one of 256, 512, 1024, 2048, 4096
 * (DS4_SHAPE_FLASH: 4096 and 2048); n_expert 1..1024; n_expert_used 1..8 and
 * <= n_expert; norm_eps finite and >= 0.
 *
 * Directional steering of the layer's FFN output ("【#8】ds4.c 해독하기",
 * directional-steering section: each layer projects its own direction out of
 * its FFN output): with steer_dir non-NULL, every token's MoE output v is
 * replaced by v - steer_scale * dir * (dir . v) before it is written or
 * accumulated (fp32; the dot product reduced in fp32 in a fixed order).
 * steer_dir: device f32 [n_embd], 16-byte aligned, used as given (a unit
 * vector makes this a projection), must not overlap y or the workspace;
 * steer_scale finite (> 0 suppresses the direction, < 0 amplifies it).  For a
 * layer-major table dirs [n_layers][n_embd], layer l takes dirs + l*n_embd.
 * NULL = no steering (steer_scale ignored).
 *
 * imatrix statistics ([P1] imatrix passage: per routed expert and input
 * column, the sum of squares of the activations the expert's projections
 * read; one entry per tensor of n_expert * n_columns values, expert-major):
 * with imatrix_in non-NULL, every call adds, for each (token, slot) pair
 * routed to expert e, n[c]^2 to imatrix_in[e][c] (device f32
 * [n_expert][n_embd]), n the MoE input row as the path feeds it to the
 * gate/up projections (decode: fp32, RMS-normalised with
 * DS4Q_F_RMSNORM_INPUT; prefill: the bf16 row).  The one vector serves both
 * the gate and the up tensor.  With imatrix_down non-NULL it adds
 * (p * h[c])^2 to imatrix_down[e][c] (device f32 [n_expert][n_ff]), h the
 * SwiGLU row as the path feeds it to the down projection (decode fp32,
 * prefill bf16) and p the pair's routing weight.  Sums are fp32, over an
 * expert's pairs in sorted order, then added to the arrays (deterministic, no
 * atomics; accumulate over calls, the caller zeroes them).  16-byte aligned,
 * overlapping nothing else.  When either is set the workspace of the prefill
 * grows by (min(P, n_expert) + P/128 + 1) * max(n_embd, n_ff) * 4 bytes,
 * P = n_tok * n_expert_used (ds4q_moe_workspace_size reads the descriptor). */
typedef struct {
  int32_t n_embd, n_ff, n_expert, n_expert_used;
  int32_t type_gate, type_up, type_down; /* ds4q_type */
  const void *gate, *up, *down;
  uint32_t flags;
  float norm_eps;
  const float *steer_dir;
  float steer_scale;
  float *imatrix_in;
  float *imatrix_down;
} ds4q_moe_layer;

/* Optional routing outputs (device pointers; any may be NULL). */
typedef struct {
  int32_t *topk_ids;       /* [T][k]  experts by (logit desc, index asc) */
  float *topk_w;           /* [T][k]  softmax over the k selected logits */
  int32_t *expert_counts;  /* [n_expert]   pairs per expert */
  int32_t *expert_offsets; /* [n_expert+1] exclusive prefix of counts */
  int32_t *sorted_pairs;   /* [T*k]  p = token*k + slot, ordered by (expert, token, slot) */
} ds4q_route_out;

/* Dequantise a [rows][cols] tensor ([P1] Q2_K table, [P5] Q4_1 section).
 * src_type: Q2_K (cols % 256 == 0) or Q4_1 (cols % 32 == 0); src 16-byte
 * aligned device pointer to rows*cols/QK blocks (read in 16-byte chunks;
 * never past the last block).  dst_type: F32 (value =
 * fp32 of d*sc*q - dmin*mn, resp. d*q + m, rounded once) or BF16 (that fp32
 * value rounded to nearest even); dst device [rows][cols], 16-byte aligned,
 * not overlapping src.  rows == 0 is a no-op. */
int ds4q_dequant(int32_t src_type, const void *src, int64_t rows, int64_t cols,
                 int32_t dst_type, void *dst, void *stream);

/* y[t][r] = sum_c W[r][c] * x[t][c] for t < n_tok, fp32 accumulation
 * (one token per call in the decode use; [P1] layouts).  w: device blocks of
 * a [rows][cols] Q2_K or Q4_1 tensor, 16-byte aligned, cols one of 256, 512,
 * 1024, 2048, 4096; x: device f32 [n_tok][cols], 16-byte aligned; y: device
 * f32 [n_tok][rows], must not overlap x or w.  n_tok in 0..64. */
int ds4q_matvec(int32_t w_type, const void *w, int64_t rows, int64_t cols,
                const float *x, int32_t n_tok, float *y, void *stream);

/* Bytes of device workspace ds4q_route needs for n_tok tokens; 0 for invalid
 * arguments. */
size_t ds4q_route_workspace_size(int32_t n_tok, int32_t n_expert, int32_t k);

/* Routing alone ([P2]: k of n_expert experts per token; n_expert 1..1024,
 * k 1..8, n_tok 0..65536).  logits: device f32 [n_tok][n_expert], finite
 * values expected.  Writes the non-NULL members of *out (device arrays; see
 * ds4q_route_out).  workspace: device, 256-byte aligned, at least
 * ds4q_route_workspace_size() bytes, overlapping nothing else. */
int ds4q_route(const float *logits, int32_t n_tok, int32_t n_expert, int32_t k,
               const ds4q_route_out *out, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace a decode (mode 0) or prefill (mode 1) call with
 * up to max_tok tokens needs; 0 for an invalid layer. */
size_t ds4q_moe_workspace_size(const ds4q_moe_layer *L, int32_t max_tok, int32_t mode);

/* Decode-path MoE layer ([P1] SwiGLU expert FFN with the routing weight on the
 * down input; [P2] top-k routing): for each token t,
 *   y_t (+)= sum_j p_tj * W2[e_tj] (silu(W1[e_tj] n_t) * (W3[e_tj] n_t)),
 * n_t = x_t (or its RMS norm with DS4Q_F_RMSNORM_INPUT), fp32 in and out.
 * One token runs on int8 matrix cores for either format (chosen per tensor):
 * the input and SwiGLU vectors enter as three int8 digits per value times a
 * scale per 256 values (residual below 2^-23 of the chunk maximum) against
 * the exact integers sc*q (Q2_K) or q (Q4_1), with the min / offset term in
 * fp32.  2..64 tokens run on int8 matrix cores grouped by expert in tiles of
 * at most 4 token-expert pairs (either format per tensor), with three int8
 * digits per value and a scale per row (residual below 2^-24 of the row
 * maximum); the Q2_K min term is exact in int32, the Q4_1 offset term takes
 * fp32 sums of 32 input values.  The SwiGLU rows stay fp32.
 * x: device f32 [n_tok][n_embd]; logits: device f32 [n_tok][n_expert];
 * y: device f32 [n_tok][n_embd] — may be the same pointer as x (in-place
 * residual with DS4Q_F_ACCUMULATE), must not partially overlap it.
 * n_tok in 0..64.  route may be NULL.  workspace: device, 256-byte aligned,
 * >= ds4q_moe_workspace_size(L, n_tok, 0) bytes, not overlapping any other
 * argument. */
int ds4q_moe_decode(const ds4q_moe_layer *L, const float *x, const float *logits, int32_t n_tok,
                    float *y, const ds4q_route_out *route, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Size of the library's static device scratch: one array of this many bytes
 * per device, reserved when the library's code is loaded on that device and
 * kept until the process ends.  It holds the workspace of every decode call
 * the ABI accepts (the largest, n_tok 64 with n_embd = n_ff = 4096, 1024
 * experts and 8 slots, needs 21.1 MiB). */
#define DS4Q_SCRATCH_BYTES (24u << 20)

/* ds4q_moe_decode without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid the allocator.  Same mathematics, kernels, argument
 * rules and errors as ds4q_moe_decode, with the workspace taken from the
 * static scratch of the calling thread's current device (the stream must
 * belong to that device).  The call itself allocates nothing: the scratch's
 * device address is looked up once per device (first call on it) and kept.
 * DS4Q_E_SCRATCH if the call would need more than DS4Q_SCRATCH_BYTES (no
 * shape the ABI accepts does).  All calls on one device share its scratch:
 * calls that overlap in time on one device (concurrent streams, threads)
 * race and must be serialised by the caller; a call leaves its workspace
 * contents in the scratch, and no call reads scratch bytes it did not write
 * itself. */
int ds4q_moe_decode_static(const ds4q_moe_layer *L, const float *x, const float *logits,
                           int32_t n_tok, float *y, const ds4q_route_out *route, void *stream);

/* Phases of the decode launches, for ds4q_moe_decode_phases. */
#define DS4Q_PHASE_ROUTE 0x1u  /* routing (nothing of its own for one Q2_K token, see below) */
#define DS4Q_PHASE_GATEUP 0x2u /* gate/up projections + SwiGLU into the workspace */
#define DS4Q_PHASE_DOWN 0x4u   /* down projection + weighted combine into y */
#define DS4Q_PHASE_ALL 0x7u

/* ds4q_moe_decode restricted to the launches of the phases set in `phases`
 * (a non-empty subset of DS4Q_PHASE_ALL, else DS4Q_E_INVAL), for timing one
 * kernel family at a time.  A phase reads only what the earlier phases left
 * in the workspace, so a sequence of calls with the same arguments and
 * workspace that covers ROUTE, GATEUP and DOWN in that order computes
 * exactly what one ds4q_moe_decode call computes.  Repeating GATEUP or DOWN
 * alone is idempotent without DS4Q_F_ACCUMULATE; with it each DOWN adds
 * again (and each GATEUP adds the imatrix statistics again).  Same argument rules and errors as ds4q_moe_decode.  route is
 * written by the phase that routes: ROUTE, except for a single token with
 * Q2_K gate/up and down, whose GATEUP launch routes the token itself. */
int ds4q_moe_decode_phases(const ds4q_moe_layer *L, const float *x, const float *logits,
                           int32_t n_tok, float *y, const ds4q_route_out *route, void *workspace,
                           size_t workspace_bytes, uint32_t phases, void *stream);

/* Prefill-path MoE layer ("【#6】ds4.c 분석하기", chunked-prefill passage: the
 * prompt is processed in chunks of 4096 tokens; "【#2】ds4.c 해독하기": the
 * routed expert is a SwiGLU FFN, w1 = gate, w3 = up, w2 = down, and the
 * routing weight scales the SwiGLU row that the down projection reads): the
 * same mathematics as ds4q_moe_decode for a chunk of n_tok tokens
 * (0..65536), computed as grouped GEMMs on matrix cores with fp32
 * accumulation.  The expert input rows are bf16 (x_type BF16, or
 * x_type F32 which is normalised per DS4Q_F_RMSNORM_INPUT if set and rounded
 * to bf16); the SwiGLU row is rounded to bf16 before the down projection.
 * The weights are dequantised to fp16 for fp16 MFMA: Q2_K weights as the
 * fp32 value d*sc*q - dmin*mn (exact up to its one fp32 rounding) rounded
 * once to fp16, Q4_1 weights as d*q + m by one fp16 fma (one rounding); each
 * bf16 input or SwiGLU row is scaled by the power of two that puts its
 * largest magnitude in [2^14, 2^15) and stored as fp16 (exact down to 2^-17
 * of the scaled maximum; the scale is undone in fp32).
 * Each pair's down row is rounded to bf16 once; routing and the final
 * weighted combine are fp32.  x: device [n_tok][n_embd] of x_type; y: device f32 [n_tok][n_embd]
 * (may equal x only when x_type is F32).  workspace
 * >= ds4q_moe_workspace_size(L, n_tok, 1). */
int ds4q_moe_prefill(const ds4q_moe_layer *L, const void *x, int32_t x_type, const float *logits,
                     int32_t n_tok, float *y, const ds4q_route_out *route, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Layer stack ([P2]: 43 layers in the Flash shape): for l in 0..n_layers-1,
 *   x <- x + MoE_l(rmsnorm(x))   (MoE_l steered when layers[l].steer_dir is set)
 * with layer l's descriptor layers[l] (its flags are ignored: RMSNORM_INPUT
 * and ACCUMULATE are implied) and router logits logits + l*n_tok*n_expert.
 * mode 0 = decode path (n_tok <= 64), 1 = prefill path.  x: device f32
 * [n_tok][n_embd], updated in place.  All layers must share n_embd, n_ff,
 * n_expert, n_expert_used.  workspace >= max over layers of
 * ds4q_moe_workspace_size(layers[l], n_tok, mode). */
int ds4q_moe_stack(const ds4q_moe_layer *layers, int32_t n_layers, int32_t mode, float *x,
                   const float *logits, int32_t n_tok, void *workspace, size_t workspace_bytes,
                   void *stream);

/* Directional steering ("【#8】ds4.c 해독하기", directional-steering section:
 * the layer's direction is projected out of its FFN output): for each row r
 * of y [n_rows][n_embd] f32,
 *   out_r (+)= y_r - scale * dir * (dir . y_r)
 * (+= with DS4Q_F_ACCUMULATE, e.g. onto the residual stream; the only flag).
 * dir: device f32 [n_embd], used as given (a unit vector makes this a
 * projection).  fp32 arithmetic: the dot product reduced in fp32, one fma per
 * value.  n_embd: multiple of 4, 4..65536; n_rows >= 0.  dir, y, out: device,
 * 16-byte aligned; out may be y (in place), dir may not overlap out. */
int ds4q_steer(const float *dir, float scale, const float *y, int32_t n_rows, int32_t n_embd,
               float *out, uint32_t flags, void *stream);

/* Activation wire formats ("【#6】ds4.c 분석하기", distributed-transport
 * passage: activations between pipeline stages travel as 32-bit floats or
 * packed to 16 or 8 bits and are decoded back to float).  bits = 32: plain
 * copy; 16: IEEE binary16, round to nearest even, overflow to +-inf, NaN to
 * sign|0x7E00; 8: OCP E4M3 (bias 7, subnormals, largest finite 448, NaN
 * sign|0x7F, no infinities), round to nearest even, magnitudes beyond 448
 * and +-inf saturate to +-448.  Decoding is exact.  n >= 0 values; src and dst
 * device, 16-byte aligned, not overlapping; dst holds n * bits / 8 bytes
 * (encode) or n floats (decode).  Other bit widths: DS4Q_E_INVAL. */
int ds4q_act_encode(const float *src, int64_t n, int32_t bits, void *dst, void *stream);
int ds4q_act_decode(const void *src, int64_t n, int32_t bits, float *dst, void *stream);

/* Per-kernel timing for profiling harnesses (not thread-safe; intended for a
 * single benchmarking thread).  While enabled, every kernel launch made by
 * the calls above is bracketed by two HIP events recorded on the call's
 * stream (the kernels themselves are unchanged; the gaps between launches
 * grow by the event records).  At most 65536 launches are recorded. */
int ds4q_timing_enable(int on);
/* Waits for the recorded events, then returns one entry per launch site:
 * names (max_names x name_len chars, NUL-terminated: "topk", "group",
 * "decode_gateup", "decode_down",
 * "prep_f16", "prefill_gateup", "prefill_down", "combine", "steer", "act_encode",
 * "act_decode"), summed milliseconds and
 * launch counts (host arrays).  Clears the record. */
int ds4q_timing_read(char *names, int name_len, double *total_ms, int64_t *count, int max_names,
                     int *n_names);

/* Static description of a status code. */
const char *ds4q_strerror(int status);
/* DS4Q_ABI_VERSION of the loaded library. */
int ds4q_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DS4Q_H */

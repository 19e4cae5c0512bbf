/*
 * CPU oracle for the decode step of a DeepSeek-V4.1-style MoE layer half.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU baseline may call it; the GPU library never links or calls
 * it, and it shares no code with the GPU library.
 *
 * Plain, slow and unfused: every sum or dot product accumulates in f64 and is
 * rounded to f32 once per defined f32 tensor, then to bf16 where the step
 * stores bf16 (rounding points as listed by the ds4 page, "v41: fuse the
 * single-box decode glue (HC, MoE, attention)", in its "What" section and its
 * router/shared-expert commit). Threads only split independent output
 * elements; they never change an element's arithmetic.
 *
 * Storage: f32 tensors are float; "act" tensors (state, x, norm, h, shared,
 * block, new state) are float when act == OR_F32 and bf16 bit patterns
 * (uint16) when act == OR_BF16. All arrays are host memory, row-major.
 *
 * Every function returns 0 on success and a negative value on bad arguments
 * or a missing expert matrix.
 */
#ifndef MONO_ORACLE_H
#define MONO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_Q8_0 = 2, OR_MXFP4 = 3 };
/* Activation quantisation for the expert matvecs: none, or MXFP8 (E4M3 values, e8m0 scale per
 * 32) for every matrix stored in MXFP4. */
enum { OR_AQ_NONE = 0, OR_AQ_MXFP8 = 1 };

typedef struct {
  int rows;         /* R */
  int hidden;       /* H; the HC row has 4 * H values */
  int n_experts;    /* E */
  int top_k;        /* k */
  int inter;        /* routed expert intermediate width I */
  int shared_inter; /* shared expert intermediate width Is */
  int act;          /* OR_F32 or OR_BF16 */
  int sinkhorn_iters;
  double routed_scale; /* rho */
  double eps_hc, eps_norm;
  int act_quant;       /* OR_AQ_NONE or OR_AQ_MXFP8 */
} or_shape;

/* One [rows][k] weight matrix. values: f32 | bf16 bits | int8 | packed e2m1 pairs (low nibble =
 * even element); scales (blocks of 32 along k, [rows][k/32]): NULL | fp16 bits | e8m0 bytes. */
typedef struct {
  int fmt;
  const void* values;
  const void* scales;
} or_mat;

/* gate [inter][H], up [inter][H], down [H][inter]; values == NULL marks an absent expert. */
typedef struct {
  or_mat gate, up, down;
} or_expert;

/* mixes[r][j] (j < 24) from the state row, or from a carry [R][25] when carry != NULL. */
int or_mix(const or_shape* s, const void* state, const float* w_mix, const float* carry,
           float* mixes);
/* pre [R][4], post [R][4], comb [R][4][4] from mixes, hc_scale [3], hc_base [24]. */
int or_split(const or_shape* s, const float* mixes, const float* hc_scale, const float* hc_base,
             float* pre, float* post, float* comb);
/* x, norm [R][H] (act) from the state, pre and w_norm [H] (act). */
int or_collapse_norm(const or_shape* s, const void* state, const float* pre, const void* w_norm,
                     void* x, void* norm);
/* Model tail: pre [R][4] (optional), x, norm [R][H] (act) from the state, the head's mix
 * w_head [4][4H], head_scale [1], head_base [4] and the output norm weight [H] (act); no split. */
int or_head(const or_shape* s, const void* state, const float* w_head, const float* head_scale,
            const float* head_base, const void* w_norm, float* pre, void* x, void* norm);
/* logits [R][E] from norm and w_router [E][H]. */
int or_router_logits(const or_shape* s, const void* norm, const float* w_router, float* logits);
/* idx [R][k], weights [R][k] from logits and bias [E]; beta_sorted [R][E] (optional) receives the
 * biased scores in selection order (for gap checks). */
int or_select(const or_shape* s, const float* logits, const float* bias, int32_t* idx,
              float* weights, float* beta_sorted);
/* One expert's SwiGLU hidden for one activation row: h [inter] (act). */
int or_expert_hidden(const or_shape* s, int inter, const or_expert* ex, const void* norm_row,
                     void* h);
/* Routed + shared experts. routed[E], shared[1]. h_routed [R][k][I] and h_shared [R][Is] are
 * outputs, or inputs when force_h != 0 (the down projections then use the given hidden rows).
 * Outputs: shared_out [R][H] (act), routed_out [R][H] (f32), block [R][H] (act). */
int or_moe(const or_shape* s, const void* norm, const int32_t* idx, const float* weights,
           const or_expert* routed, const or_expert* shared, int force_h, void* h_routed,
           void* h_shared, void* shared_out, float* routed_out, void* block);
/* new_state [R][4][H] (act) and, when w_mix_next != NULL, carry [R][25] (raw mix sums, sumsq). */
int or_expand(const or_shape* s, const void* state, const void* block, const float* post,
              const float* comb, const float* w_mix_next, void* new_state, float* carry);

/* Format helpers (exact decodes), exposed for the tests' decode tables. */
double or_bf16_to_f64(uint16_t b);
uint16_t or_f32_to_bf16(float f);
double or_f16_to_f64(uint16_t h);
double or_e2m1_to_f64(unsigned code);
double or_e8m0_to_f64(uint8_t e);
double or_e4m3_to_f64(uint8_t c);
/* MXFP8 quantisation of v[0 .. n) (n a multiple of 32): E4M3 codes [n] and e8m0 scales [n/32]. */
int or_mxfp8_quant(const double* v, int n, uint8_t* codes, uint8_t* scales);
/* Element (row, col) of a matrix with k columns, exactly, in f64. */
double or_mat_elem(const or_mat* m, int64_t k, int64_t row, int64_t col);

/* Number of threads the oracle's parallel loops use, and a way to set it (n >= 1). */
int or_threads(void);
void or_set_threads(int n);

#ifdef __cplusplus
}
#endif

#endif /* MONO_ORACLE_H */

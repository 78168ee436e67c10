/*
 * vlb_oracle.h -- plain fp64 CPU oracle of the vision-to-language bridge.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  It shares
 * no code, header, table or helper with the HIP path in patch_merge_mlp_amd/.
 *
 * Every value is a double.  Inputs that were stored in bf16 or fp32 are widened
 * to double exactly by the caller; the oracle itself never rounds to a narrower
 * type.
 *
 * Sources (web pages; cited by title and section):
 *   [VL2]  "feat(models): port DeepSeek-VL2 (MoE text + SigLIP/SAM vision)",
 *          mlxcel issue #533 -- sections "Projector (downsample_mlp_gelu)",
 *          "Tile-sequence assembly (tile_tag 2D)", "Processor" step 7,
 *          "Validation and acceptance criteria".
 *   [V4V]  "DeepSeek-V4-Flash-Vision-BF16" model card -- header paragraph
 *          (2x2 PatchMerger, 4608 -> 4096, 40,119,040 projector parameters).
 *   [VOIE] "La voie visuelle" (DeepSeek-V4.1-Flash architecture notes) --
 *          sections "Le pixel-unshuffle 3x3" and "Le calcul".
 *   [HYB]  "DeepSeek-VL Hybrid" (KerasFormers docs) -- processor argument
 *          num_image_tokens = 576.
 */
#ifndef VLB_ORACLE_H
#define VLB_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Activation between the two projector Linears. */
enum { ORC_GELU_ERF = 0, ORC_GELU_TANH = 1, ORC_ACT_NONE = 2 };

/* Source codes of an assembled slot that is not a projected token row. */
enum { ORC_SRC_NEWLINE = -1, ORC_SRC_SEPARATOR = -2 };

/* One bridge problem.  Views are stored back to back, each (gh, gw, C)
 * channels-last; images own consecutive views.  For the tiled layout an image
 * has 1 + tile_w*tile_h views, the global view first. */
typedef struct {
  int32_t n_views;
  const int32_t *grid_h, *grid_w;   /* [n_views] */
  int32_t C, k, hidden, out_dim;
  int32_t has_ln;
  double ln_eps;
  int32_t act;                      /* ORC_GELU_ERF / ORC_GELU_TANH / ORC_ACT_NONE */
  int32_t n_images;
  const int32_t *views_per_image;   /* [n_images] */
  int32_t tiled;                    /* 0: tokens in order; 1: 2D tile assembly */
  const int32_t *tile_w, *tile_h;   /* [n_images], tiled only */
  int32_t global_tail;              /* tiled only: 1 = [local, sep, global] */
  int32_t n_mid;                    /* hidden -> hidden Linears between the two (depth - 2);
                                       their weights go to orc_project_rows_deep */
} orc_spec;

/* ceil(g / k): side of the merged grid after high-end zero padding [VL2 Projector 1-2]. */
int64_t orc_merged_side(int64_t g, int64_t k);
/* Projected token rows of one view. */
int64_t orc_view_tokens(int64_t gh, int64_t gw, int64_t k);
/* Total projected token rows of the problem (views concatenated in order). */
int64_t orc_total_tokens(const orc_spec *s);
/* Placeholder count of one tiled image by the closed formula of [VL2 Processor step 7]. */
int64_t orc_tiled_placeholders(int64_t hp, int64_t wp, int64_t tw, int64_t th);
/* Parameter count of LN(C, affine, optional) + Linear(C k^2 -> hidden) + Linear(hidden -> out). */
int64_t orc_param_count(int64_t C, int64_t k, int64_t hidden, int64_t out_dim, int32_t has_ln);

/* Per-pixel LayerNorm over the C channels of npix pixels (biased variance,
 * eps inside the square root, affine gamma/beta). */
void orc_layer_norm(const double *x, int64_t npix, int32_t C, const double *gamma,
                    const double *beta, double eps, double *out);

/* Pad one (gh, gw, C) view with zeros at the high end to a multiple of k and
 * apply the k x k space-to-depth: out[t][c*k*k + dy*k + dx], t row-major over
 * the merged grid [VL2 Projector 1-2].  out has orc_view_tokens() rows of C*k*k. */
void orc_merge_view(const double *x, int32_t gh, int32_t gw, int32_t C, int32_t k, double *out);
/* Inverse of orc_merge_view on the unpadded cells (the merge is lossless [VOIE]). */
void orc_unmerge_view(const double *merged, int32_t gh, int32_t gw, int32_t C, int32_t k,
                      double *x);

/* out[r][j] = b[j] + sum_i in[r][i] * W[j][i]; W stored (out_dim, in_dim). */
void orc_linear(const double *in, int64_t rows, int32_t in_dim, const double *W,
                const double *b, int32_t out_dim, double *out, int32_t nthreads);
/* In-place activations. */
void orc_gelu_erf(double *x, int64_t n);
void orc_gelu_tanh(double *x, int64_t n);

/* Merged (LN -> pad -> space-to-depth) feature row of projected token row r of
 * the whole problem.  x holds all views; gamma/beta may be NULL when has_ln=0. */
void orc_merged_row(const orc_spec *s, const double *x, const double *gamma,
                    const double *beta, int64_t r, double *out);

/* Projected rows (merge -> Linear -> act -> Linear) for the listed token rows.
 * out is [n_rows][out_dim]. */
void orc_project_rows(const orc_spec *s, const double *x, const double *gamma,
                      const double *beta, const double *W1, const double *b1,
                      const double *W2, const double *b2, const int64_t *row_ids,
                      int64_t n_rows, double *out, int32_t nthreads);

/* The same for a projector of depth 2 + n_mid [VL2 Projector 3: with depth > 2
 * further act + Linear(hidden -> hidden) pairs sit between the two]: merge ->
 * Linear1 -> (act -> Linear_mid[i]) for each i -> act -> Linear2.  W_mid is
 * [n_mid][hidden][hidden] (each stored (out, in)), b_mid [n_mid][hidden]. */
void orc_project_rows_deep(const orc_spec *s, const double *x, const double *gamma,
                           const double *beta, const double *W1, const double *b1,
                           const double *W_mid, const double *b_mid, const double *W2,
                           const double *b2, const int64_t *row_ids, int64_t n_rows, double *out,
                           int32_t nthreads);

/* Assembly order of all images [VL2 Tile-sequence assembly].  Writes the
 * source of every placeholder slot into src (token row >= 0, or
 * ORC_SRC_NEWLINE / ORC_SRC_SEPARATOR) and returns the slot count P.  src may
 * be NULL to count only; otherwise it must hold cap entries (returns -1 if
 * P > cap). */
int64_t orc_assemble(const orc_spec *s, int64_t *src, int64_t cap);

/* Overwrite seq (S x D) at the mask==1 positions, in order, with the assembled
 * rows [VL2 Tile-sequence assembly, last paragraph].  rows is [T][D] indexed by
 * token row.  Returns 0, or -1 without writing anything if the number of
 * placeholder positions differs from P [VL2 Validation]. */
int32_t orc_scatter(const int64_t *src, int64_t P, const double *rows, const double *newline,
                    const double *separator, const uint8_t *mask, int64_t S, int32_t D,
                    double *seq);

/* The whole embedded sequence [VL2 Tile-sequence assembly, last paragraph;
 * language config vocab_size, image_token_index]: position s holds row ids[s]
 * of the token-embedding table E [vocab][D] unless ids[s] == image_id; the
 * positions holding image_id take the assembled rows in order (as
 * orc_scatter).  E is given in its stored form, as bf16 bit patterns (e_bf16)
 * when that is non-NULL, else as doubles (e_f64); it is widened exactly.
 * Returns 0; -1 if the number of image_id positions differs from P; else -2
 * if a text id lies outside [0, vocab).  On error seq is left untouched. */
int32_t orc_embed_scatter(const int64_t *src, int64_t P, const double *rows,
                          const double *newline, const double *separator, const int32_t *ids,
                          int64_t S, int32_t image_id, const uint16_t *e_bf16,
                          const double *e_f64, int64_t vocab, int32_t D, double *seq);

/* ---- backward (training the projector [V4V header]; [VOIE] "Pendant le
 * pré-entraînement du squelette") ------------------------------------------- */

/* Gradient of orc_scatter: given dseq (S x D), the gradient of each scattered
 * token row (drows [T][D]; each row sits in exactly one slot) and of the
 * newline and separator vectors (summed over every slot that holds them).
 * Returns 0, or -1 (nothing written) on a placeholder-count mismatch. */
int32_t orc_scatter_backward(const int64_t *src, int64_t P, const uint8_t *mask, int64_t S,
                             int32_t D, const double *dseq, int64_t T, double *drows,
                             double *dnewline, double *dseparator);

/* orc_project_backward, orc_hidden_unit_grads and orc_pixel_grad take a
 * projector of depth 2 (s->n_mid is not read); orc_project_backward_deep any. */

/* Gradients of the projector for the gradient dY [T][out_dim] of its output
 * rows: dx [n_pixels][C] (of the features), dW1 [hidden][C*k*k] (pages' feature
 * order), db1 [hidden], dW2 [out_dim][hidden], db2 [out_dim], and with the
 * LayerNorm dgamma, dbeta [C] (untouched, may be NULL, without it).  Padded
 * cells take no gradient. */
void orc_project_backward(const orc_spec *s, const double *x, const double *gamma,
                          const double *beta, const double *W1, const double *b1,
                          const double *W2, const double *dY, double *dx, double *dW1,
                          double *db1, double *dW2, double *db2, double *dgamma,
                          double *dbeta);

/* orc_project_backward for a projector of depth 2 + s->n_mid: also the
 * gradients of the middle Linears, dW_mid [n_mid][hidden][hidden] and db_mid
 * [n_mid][hidden] (W_mid, b_mid as for orc_project_rows_deep). */
void orc_project_backward_deep(const orc_spec *s, const double *x, const double *gamma,
                               const double *beta, const double *W1, const double *b1,
                               const double *W_mid, const double *b_mid, const double *W2,
                               const double *dY, double *dx, double *dW1, double *db1,
                               double *dW_mid, double *db_mid, double *dW2, double *db2,
                               double *dgamma, double *dbeta);

/* The same gradients restricted to hidden unit h: row h of dW1, db1[h] and
 * column h of dW2 (dW2_col [out_dim]). */
void orc_hidden_unit_grads(const orc_spec *s, const double *x, const double *gamma,
                           const double *beta, const double *W1, const double *b1,
                           const double *W2, const double *dY, int32_t h, double *dW1_row,
                           double *db1_h, double *dW2_col);

/* The feature gradient of one pixel (view v, row y, column xx): dx_out [C]. */
void orc_pixel_grad(const orc_spec *s, const double *x, const double *gamma, const double *beta,
                    const double *W1, const double *b1, const double *W2, const double *dY,
                    int32_t v, int32_t y, int32_t xx, double *dx_out);

#ifdef __cplusplus
}
#endif
#endif

/*
 * vlb_oracle.c -- plain fp64 CPU oracle of the vision-to-language bridge.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: only tests/, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It is written from the pages' text,
 * step by step, with no blocking, fusion or reordering; the one liberty is
 * that independent output rows of a Linear may be computed on several threads,
 * which does not change any summation order.
 *
 * Pages (cited by title and section; see vlb_oracle.h for the short tags):
 *   [VL2]  mlxcel issue #533 "port DeepSeek-VL2"
 *   [V4V]  "DeepSeek-V4-Flash-Vision-BF16" model card
 *   [VOIE] "La voie visuelle" (DeepSeek-V4.1-Flash)
 *
 * Readings taken where the pages leave a step open (each is listed in the
 * design notes of the repository):
 *   - the projector's GELU is the exact erf form; the tanh form is a flag;
 *   - the pre-merge LayerNorm is per patch over C, biased variance, eps inside
 *     the square root, affine (the only form matching the 40,119,040 count);
 *   - padding is applied after the LayerNorm (padded cells are exactly zero);
 *   - rectangular grids pad and merge each axis independently.
 */
#include "vlb_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- sizes ------------------------------------------------------------- */

/* [VL2 Projector 1]: pad "at the high end up to g_pad, the next multiple of
 * ds"; the merged side is g_pad / ds. */
int64_t orc_merged_side(int64_t g, int64_t k) {
  int64_t g_pad = g;
  while (g_pad % k != 0) g_pad++;
  return g_pad / k;
}

/* [VL2 Projector 2]: N' = (g_pad / ds)^2 for a square grid. */
int64_t orc_view_tokens(int64_t gh, int64_t gw, int64_t k) {
  return orc_merged_side(gh, k) * orc_merged_side(gw, k);
}

int64_t orc_total_tokens(const orc_spec *s) {
  int64_t t = 0;
  for (int32_t v = 0; v < s->n_views; v++) t += orc_view_tokens(s->grid_h[v], s->grid_w[v], s->k);
  return t;
}

/* [VL2 Processor step 7]: h'*(w'+1) + 1 + (th*h')*(tw*w'+1). */
int64_t orc_tiled_placeholders(int64_t hp, int64_t wp, int64_t tw, int64_t th) {
  return hp * (wp + 1) + 1 + (th * hp) * (tw * wp + 1);
}

/* LN(C): gamma and beta (2C); Linear(C k^2 -> hidden): weight + bias;
 * Linear(hidden -> out): weight + bias.  [V4V header] quotes the total. */
int64_t orc_param_count(int64_t C, int64_t k, int64_t hidden, int64_t out_dim, int32_t has_ln) {
  int64_t K1 = C * k * k;
  int64_t n = K1 * hidden + hidden + hidden * out_dim + out_dim;
  if (has_ln) n += 2 * C;
  return n;
}

/* ---- LayerNorm --------------------------------------------------------- */

void orc_layer_norm(const double *x, int64_t npix, int32_t C, const double *gamma,
                    const double *beta, double eps, double *out) {
  for (int64_t p = 0; p < npix; p++) {
    const double *xp = x + p * C;
    double mean = 0.0;
    for (int32_t c = 0; c < C; c++) mean += xp[c];
    mean /= C;
    double var = 0.0;
    for (int32_t c = 0; c < C; c++) var += (xp[c] - mean) * (xp[c] - mean);
    var /= C;
    double inv = 1.0 / sqrt(var + eps);
    for (int32_t c = 0; c < C; c++) out[p * C + c] = (xp[c] - mean) * inv * gamma[c] + beta[c];
  }
}

/* ---- space-to-depth ---------------------------------------------------- */

/* Value of padded cell (y, x) of a view: the stored value inside the grid,
 * zero in the padding [VL2 Projector 1]. */
static double padded_cell(const double *x, int32_t gh, int32_t gw, int32_t C, int64_t y,
                          int64_t xx, int32_t c) {
  if (y >= gh || xx >= gw) return 0.0;
  return x[(y * gw + xx) * C + c];
}

/* [VL2 Projector 2]: blocks scanned row-major; inside a block the feature
 * index is c*ds*ds + dy*ds + dx.  [VOIE] calls the same rearrangement a
 * pixel-unshuffle. */
void orc_merge_view(const double *x, int32_t gh, int32_t gw, int32_t C, int32_t k, double *out) {
  int64_t hp = orc_merged_side(gh, k), wp = orc_merged_side(gw, k);
  int64_t K1 = (int64_t)C * k * k;
  for (int64_t ty = 0; ty < hp; ty++)
    for (int64_t tx = 0; tx < wp; tx++) {
      int64_t t = ty * wp + tx;
      for (int32_t c = 0; c < C; c++)
        for (int32_t dy = 0; dy < k; dy++)
          for (int32_t dx = 0; dx < k; dx++)
            out[t * K1 + (int64_t)c * k * k + dy * k + dx] =
                padded_cell(x, gh, gw, C, ty * k + dy, tx * k + dx, c);
    }
}

void orc_unmerge_view(const double *merged, int32_t gh, int32_t gw, int32_t C, int32_t k,
                      double *x) {
  int64_t wp = orc_merged_side(gw, k);
  int64_t K1 = (int64_t)C * k * k;
  for (int64_t y = 0; y < gh; y++)
    for (int64_t xx = 0; xx < gw; xx++) {
      int64_t t = (y / k) * wp + (xx / k);
      int64_t dy = y % k, dx = xx % k;
      for (int32_t c = 0; c < C; c++)
        x[(y * gw + xx) * C + c] = merged[t * K1 + (int64_t)c * k * k + dy * k + dx];
    }
}

/* ---- Linear and activations ------------------------------------------- */

typedef struct {
  const double *in, *W, *b;
  double *out;
  int64_t r0, r1;
  int32_t in_dim, out_dim;
} linear_job;

static void linear_rows(const linear_job *j) {
  for (int64_t r = j->r0; r < j->r1; r++)
    for (int32_t o = 0; o < j->out_dim; o++) {
      double acc = 0.0;
      const double *w = j->W + (int64_t)o * j->in_dim;
      const double *a = j->in + r * j->in_dim;
      for (int32_t i = 0; i < j->in_dim; i++) acc += a[i] * w[i];
      j->out[r * j->out_dim + o] = acc + (j->b ? j->b[o] : 0.0);
    }
}

static void *linear_thread(void *arg) {
  linear_rows((const linear_job *)arg);
  return NULL;
}

/* [VL2 Weight loading]: Linear weights are stored (out_features, in_features)
 * and used as-is. */
void orc_linear(const double *in, int64_t rows, int32_t in_dim, const double *W,
                const double *b, int32_t out_dim, double *out, int32_t nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = rows > 0 ? (int32_t)rows : 1;
  linear_job jobs[256];
  pthread_t th[256];
  if (nthreads > 256) nthreads = 256;
  for (int32_t t = 0; t < nthreads; t++) {
    jobs[t].in = in; jobs[t].W = W; jobs[t].b = b; jobs[t].out = out;
    jobs[t].in_dim = in_dim; jobs[t].out_dim = out_dim;
    jobs[t].r0 = rows * t / nthreads;
    jobs[t].r1 = rows * (t + 1) / nthreads;
  }
  if (nthreads == 1) {
    linear_rows(&jobs[0]);
    return;
  }
  for (int32_t t = 0; t < nthreads; t++) pthread_create(&th[t], NULL, linear_thread, &jobs[t]);
  for (int32_t t = 0; t < nthreads; t++) pthread_join(th[t], NULL);
}

/* GELU(x) = x * Phi(x) with Phi the standard normal CDF (Hendrycks & Gimpel). */
void orc_gelu_erf(double *x, int64_t n) {
  for (int64_t i = 0; i < n; i++) x[i] = 0.5 * x[i] * (1.0 + erf(x[i] / sqrt(2.0)));
}

/* The tanh approximation of GELU (Hendrycks & Gimpel, sec. 2). */
void orc_gelu_tanh(double *x, int64_t n) {
  const double a = sqrt(2.0 / M_PI);
  for (int64_t i = 0; i < n; i++)
    x[i] = 0.5 * x[i] * (1.0 + tanh(a * (x[i] + 0.044715 * x[i] * x[i] * x[i])));
}

/* ---- one token row through the whole projector ------------------------- */

/* Locate token row r: its view, and its token index inside that view. */
static void locate_row(const orc_spec *s, int64_t r, int32_t *view, int64_t *pixel_base,
                       int64_t *tok) {
  int64_t pix = 0;
  for (int32_t v = 0; v < s->n_views; v++) {
    int64_t n = orc_view_tokens(s->grid_h[v], s->grid_w[v], s->k);
    if (r < n) {
      *view = v;
      *pixel_base = pix;
      *tok = r;
      return;
    }
    r -= n;
    pix += (int64_t)s->grid_h[v] * s->grid_w[v];
  }
  *view = -1;
  *pixel_base = 0;
  *tok = 0;
}

void orc_merged_row(const orc_spec *s, const double *x, const double *gamma,
                    const double *beta, int64_t r, double *out) {
  int32_t v;
  int64_t pix, tok;
  locate_row(s, r, &v, &pix, &tok);
  int32_t gh = s->grid_h[v], gw = s->grid_w[v], C = s->C, k = s->k;
  int64_t wp = orc_merged_side(gw, k);
  int64_t ty = tok / wp, tx = tok % wp;
  double *normed = (double *)malloc(sizeof(double) * C);
  for (int32_t dy = 0; dy < k; dy++)
    for (int32_t dx = 0; dx < k; dx++) {
      int64_t y = ty * k + dy, xx = tx * k + dx;
      int inside = (y < gh && xx < gw);
      if (inside) {
        const double *px = x + (pix + y * gw + xx) * C;
        if (s->has_ln)
          orc_layer_norm(px, 1, C, gamma, beta, s->ln_eps, normed);
        else
          memcpy(normed, px, sizeof(double) * C);
      }
      for (int32_t c = 0; c < C; c++)
        out[(int64_t)c * k * k + dy * k + dx] = inside ? normed[c] : 0.0;
    }
  free(normed);
}

typedef struct {
  const orc_spec *s;
  const double *x, *gamma, *beta, *W1, *b1, *W_mid, *b_mid, *W2, *b2;
  const int64_t *row_ids;
  double *out;
  int64_t i0, i1;
} project_job;

static void apply_act(int32_t act, double *h, int64_t n) {
  if (act == ORC_GELU_ERF) orc_gelu_erf(h, n);
  else if (act == ORC_GELU_TANH) orc_gelu_tanh(h, n);
}

static void project_range(const project_job *j) {
  const orc_spec *s = j->s;
  int32_t K1 = s->C * s->k * s->k;
  const int32_t H = s->hidden;
  double *m = (double *)malloc(sizeof(double) * K1);
  double *h = (double *)malloc(sizeof(double) * H);
  double *h2 = (double *)malloc(sizeof(double) * H);
  for (int64_t i = j->i0; i < j->i1; i++) {
    orc_merged_row(s, j->x, j->gamma, j->beta, j->row_ids[i], m);
    /* [VL2 Projector 3]: Linear -> GELU -> Linear, with (GELU -> Linear(hidden ->
     * hidden)) pairs in the middle when the depth is above 2. */
    orc_linear(m, 1, K1, j->W1, j->b1, H, h, 1);
    for (int32_t q = 0; q < s->n_mid; q++) {
      apply_act(s->act, h, H);
      orc_linear(h, 1, H, j->W_mid + (int64_t)q * H * H, j->b_mid + (int64_t)q * H, H, h2, 1);
      memcpy(h, h2, sizeof(double) * H);
    }
    apply_act(s->act, h, H);
    orc_linear(h, 1, H, j->W2, j->b2, s->out_dim, j->out + i * s->out_dim, 1);
  }
  free(m);
  free(h);
  free(h2);
}

static void *project_thread(void *arg) {
  project_range((const project_job *)arg);
  return NULL;
}

void orc_project_rows(const orc_spec *s, const double *x, const double *gamma,
                      const double *beta, const double *W1, const double *b1,
                      const double *W2, const double *b2, const int64_t *row_ids,
                      int64_t n_rows, double *out, int32_t nthreads) {
  orc_spec s2 = *s;
  s2.n_mid = 0;
  orc_project_rows_deep(&s2, x, gamma, beta, W1, b1, NULL, NULL, W2, b2, row_ids, n_rows, out,
                        nthreads);
}

void orc_project_rows_deep(const orc_spec *s, const double *x, const double *gamma,
                           const double *beta, const double *W1, const double *b1,
                           const double *W_mid, const double *b_mid, const double *W2,
                           const double *b2, const int64_t *row_ids, int64_t n_rows, double *out,
                           int32_t nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > n_rows) nthreads = n_rows > 0 ? (int32_t)n_rows : 1;
  project_job jobs[256];
  pthread_t th[256];
  for (int32_t t = 0; t < nthreads; t++) {
    project_job j = {s, x, gamma, beta, W1, b1, W_mid, b_mid, W2, b2, row_ids, out,
                     n_rows * t / nthreads, n_rows * (t + 1) / nthreads};
    jobs[t] = j;
  }
  if (nthreads == 1) {
    project_range(&jobs[0]);
    return;
  }
  for (int32_t t = 0; t < nthreads; t++) pthread_create(&th[t], NULL, project_thread, &jobs[t]);
  for (int32_t t = 0; t < nthreads; t++) pthread_join(th[t], NULL);
}

/* ---- assembly and scatter --------------------------------------------- */

static int64_t emit(int64_t *src, int64_t cap, int64_t n, int64_t value) {
  if (src && n < cap) src[n] = value;
  return n + 1;
}

/* [VL2 Tile-sequence assembly], one tiled image whose views start at token row
 * base.  The global view gets a newline column; the local views are laid out
 * as the (th, tw, h', w') -> (th, h', tw, w') transposed mosaic with one
 * newline per mosaic row; the separator sits between them. */
static int64_t emit_global(int64_t *src, int64_t cap, int64_t n, int64_t base, int64_t hp,
                           int64_t wp) {
  for (int64_t y = 0; y < hp; y++) {
    for (int64_t x = 0; x < wp; x++) n = emit(src, cap, n, base + y * wp + x);
    n = emit(src, cap, n, ORC_SRC_NEWLINE);
  }
  return n;
}

static int64_t emit_local(int64_t *src, int64_t cap, int64_t n, int64_t base, int64_t hp,
                          int64_t wp, int64_t tw, int64_t th) {
  int64_t per_view = hp * wp;
  for (int64_t i = 0; i < th; i++)
    for (int64_t y = 0; y < hp; y++) {
      for (int64_t j = 0; j < tw; j++)
        for (int64_t x = 0; x < wp; x++)
          n = emit(src, cap, n, base + (1 + i * tw + j) * per_view + y * wp + x);
      n = emit(src, cap, n, ORC_SRC_NEWLINE);
    }
  return n;
}

int64_t orc_assemble(const orc_spec *s, int64_t *src, int64_t cap) {
  int64_t n = 0, row = 0;
  int32_t v = 0;
  for (int32_t im = 0; im < s->n_images; im++) {
    int32_t nv = s->views_per_image[im];
    if (!s->tiled) {
      for (int32_t q = 0; q < nv; q++, v++) {
        int64_t t = orc_view_tokens(s->grid_h[v], s->grid_w[v], s->k);
        for (int64_t i = 0; i < t; i++) n = emit(src, cap, n, row + i);
        row += t;
      }
      continue;
    }
    int64_t hp = orc_merged_side(s->grid_h[v], s->k), wp = orc_merged_side(s->grid_w[v], s->k);
    int64_t tw = s->tile_w[im], th = s->tile_h[im];
    if (!s->global_tail) {
      n = emit_global(src, cap, n, row, hp, wp);
      n = emit(src, cap, n, ORC_SRC_SEPARATOR);
      n = emit_local(src, cap, n, row, hp, wp, tw, th);
    } else {
      n = emit_local(src, cap, n, row, hp, wp, tw, th);
      n = emit(src, cap, n, ORC_SRC_SEPARATOR);
      n = emit_global(src, cap, n, row, hp, wp);
    }
    row += (int64_t)nv * hp * wp;
    v += nv;
  }
  if (src && n > cap) return -1;
  return n;
}

/* [VL2 Tile-sequence assembly]: the assembled rows overwrite the embeddings at
 * the placeholder positions, in order.  [VL2 Validation]: the placeholder
 * count must equal the number of scattered rows; on a mismatch nothing is
 * written. */
int32_t orc_scatter(const int64_t *src, int64_t P, const double *rows, const double *newline,
                    const double *separator, const uint8_t *mask, int64_t S, int32_t D,
                    double *seq) {
  int64_t count = 0;
  for (int64_t i = 0; i < S; i++) count += mask[i] != 0;
  if (count != P) return -1;
  int64_t j = 0;
  for (int64_t i = 0; i < S; i++) {
    if (!mask[i]) continue;
    const double *from = src[j] >= 0                  ? rows + src[j] * D
                         : src[j] == ORC_SRC_NEWLINE ? newline
                                                      : separator;
    memcpy(seq + i * D, from, sizeof(double) * D);
    j++;
  }
  return 0;
}

/* bf16 bit pattern -> double (exact: bf16 is the upper half of an fp32). */
static double bf16_bits(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int32_t orc_embed_scatter(const int64_t *src, int64_t P, const double *rows,
                          const double *newline, const double *separator, const int32_t *ids,
                          int64_t S, int32_t image_id, const uint16_t *e_bf16,
                          const double *e_f64, int64_t vocab, int32_t D, double *seq) {
  int64_t n_img = 0;
  int bad_id = 0;
  for (int64_t i = 0; i < S; i++) {
    if (ids[i] == image_id) n_img++;
    else if (ids[i] < 0 || ids[i] >= vocab) bad_id = 1;
  }
  if (n_img != P) return -1;
  if (bad_id) return -2;
  int64_t j = 0;
  for (int64_t i = 0; i < S; i++) {
    double *to = seq + i * D;
    if (ids[i] == image_id) {
      const double *from = src[j] >= 0                  ? rows + src[j] * D
                           : src[j] == ORC_SRC_NEWLINE ? newline
                                                        : separator;
      memcpy(to, from, sizeof(double) * D);
      j++;
    } else {
      const int64_t e = (int64_t)ids[i] * D;
      for (int32_t d = 0; d < D; d++) to[d] = e_bf16 ? bf16_bits(e_bf16[e + d]) : e_f64[e + d];
    }
  }
  return 0;
}

/* ---- backward --------------------------------------------------------- */
/*
 * The projector is the trained part of the bridge: [V4V header] trains only its
 * parameters (the LayerNorm, both Linears) with tower and text model frozen,
 * and [VOIE "Pendant le pré-entraînement du squelette"] keeps the projector
 * (and the tower's final norm, whose gradient is the one reaching the features)
 * trainable.  The gradients below are the chain rule taken through the forward
 * steps in reverse: scatter, Linear2, activation, Linear1, space-to-depth,
 * LayerNorm.
 */

/* d/dz of the activation. erf form: Phi(z) + z phi(z). tanh form: the
 * derivative of 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3). */
static double act_slope(int32_t act, double z) {
  if (act == ORC_GELU_ERF)
    return 0.5 * (1.0 + erf(z / sqrt(2.0))) + z * exp(-0.5 * z * z) / sqrt(2.0 * M_PI);
  if (act == ORC_GELU_TANH) {
    const double a = sqrt(2.0 / M_PI);
    const double t = tanh(a * (z + 0.044715 * z * z * z));
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * a * (1.0 + 3.0 * 0.044715 * z * z);
  }
  return 1.0;
}

static double act_value(int32_t act, double z) {
  if (act == ORC_GELU_ERF) orc_gelu_erf(&z, 1);
  else if (act == ORC_GELU_TANH) orc_gelu_tanh(&z, 1);
  return z;
}

int32_t orc_scatter_backward(const int64_t *src, int64_t P, const uint8_t *mask, int64_t S,
                             int32_t D, const double *dseq, int64_t T, double *drows,
                             double *dnewline, double *dseparator) {
  int64_t count = 0;
  for (int64_t i = 0; i < S; i++) count += mask[i] != 0;
  if (count != P) return -1;
  memset(drows, 0, sizeof(double) * T * D);
  memset(dnewline, 0, sizeof(double) * D);
  memset(dseparator, 0, sizeof(double) * D);
  int64_t j = 0;
  for (int64_t i = 0; i < S; i++) {
    if (!mask[i]) continue;
    const double *g = dseq + i * D;
    if (src[j] >= 0) {
      memcpy(drows + src[j] * D, g, sizeof(double) * D);
    } else {
      double *to = src[j] == ORC_SRC_NEWLINE ? dnewline : dseparator;
      for (int32_t d = 0; d < D; d++) to[d] += g[d];
    }
    j++;
  }
  return 0;
}

/* Backward of the LayerNorm of one pixel: x its C inputs, dn the gradient of
 * its normalised output.  With xh = (x - mean) * r, r = 1 / sqrt(var + eps)
 * and n = gamma * xh + beta:
 *   dgamma += dn * xh,  dbeta += dn,
 *   dx = r * (g - mean(g) - xh * mean(g * xh)),  g = gamma * dn. */
static void ln_backward_pixel(const double *x, const double *dn, int32_t C, const double *gamma,
                              double eps, double *dx, double *dgamma, double *dbeta) {
  double mean = 0.0;
  for (int32_t c = 0; c < C; c++) mean += x[c];
  mean /= C;
  double var = 0.0;
  for (int32_t c = 0; c < C; c++) var += (x[c] - mean) * (x[c] - mean);
  var /= C;
  const double r = 1.0 / sqrt(var + eps);
  double mg = 0.0, mgx = 0.0;
  for (int32_t c = 0; c < C; c++) {
    const double xh = (x[c] - mean) * r, g = gamma[c] * dn[c];
    if (dgamma) dgamma[c] += dn[c] * xh;
    if (dbeta) dbeta[c] += dn[c];
    mg += g;
    mgx += g * xh;
  }
  mg /= C;
  mgx /= C;
  for (int32_t c = 0; c < C; c++) {
    const double xh = (x[c] - mean) * r;
    dx[c] = r * (gamma[c] * dn[c] - mg - xh * mgx);
  }
}

/* First pixel of view v and the first token row of view v. */
static void view_bases(const orc_spec *s, int32_t v, int64_t *pix, int64_t *row) {
  *pix = 0;
  *row = 0;
  for (int32_t q = 0; q < v; q++) {
    *pix += (int64_t)s->grid_h[q] * s->grid_w[q];
    *row += orc_view_tokens(s->grid_h[q], s->grid_w[q], s->k);
  }
}

void orc_project_backward(const orc_spec *s, const double *x, const double *gamma,
                          const double *beta, const double *W1, const double *b1,
                          const double *W2, const double *dY, double *dx, double *dW1,
                          double *db1, double *dW2, double *db2, double *dgamma,
                          double *dbeta) {
  orc_spec s2 = *s;
  s2.n_mid = 0;
  orc_project_backward_deep(&s2, x, gamma, beta, W1, b1, NULL, NULL, W2, dY, dx, dW1, db1, NULL,
                            NULL, dW2, db2, dgamma, dbeta);
}

void orc_project_backward_deep(const orc_spec *s, const double *x, const double *gamma,
                               const double *beta, const double *W1, const double *b1,
                               const double *W_mid, const double *b_mid, const double *W2,
                               const double *dY, double *dx, double *dW1, double *db1,
                               double *dW_mid, double *db_mid, double *dW2, double *db2,
                               double *dgamma, double *dbeta) {
  const int32_t C = s->C, k = s->k, H = s->hidden, O = s->out_dim, n_mid = s->n_mid;
  const int64_t K1 = (int64_t)C * k * k;
  int64_t npix = 0;
  for (int32_t v = 0; v < s->n_views; v++) npix += (int64_t)s->grid_h[v] * s->grid_w[v];
  memset(dW1, 0, sizeof(double) * H * K1);
  memset(db1, 0, sizeof(double) * H);
  memset(dW2, 0, sizeof(double) * O * H);
  memset(db2, 0, sizeof(double) * O);
  if (n_mid > 0) {
    memset(dW_mid, 0, sizeof(double) * n_mid * H * H);
    memset(db_mid, 0, sizeof(double) * n_mid * H);
  }
  if (s->has_ln) {
    memset(dgamma, 0, sizeof(double) * C);
    memset(dbeta, 0, sizeof(double) * C);
  }
  double *m = (double *)malloc(sizeof(double) * K1);
  double *zs = (double *)malloc(sizeof(double) * (n_mid + 1) * H); /* pre-activations per Linear */
  double *a = (double *)malloc(sizeof(double) * H);
  double *dz = (double *)malloc(sizeof(double) * H);
  double *dzp = (double *)malloc(sizeof(double) * H);
  double *dm = (double *)malloc(sizeof(double) * K1);
  double *dn = (double *)calloc((size_t)npix * C, sizeof(double)); /* d(LN output) per pixel */
  int64_t r = 0, pix = 0;
  for (int32_t v = 0; v < s->n_views; v++) {
    const int32_t gh = s->grid_h[v], gw = s->grid_w[v];
    const int64_t wp = orc_merged_side(gw, k), nt = orc_view_tokens(gh, gw, k);
    for (int64_t t = 0; t < nt; t++, r++) {
      const double *dy = dY + r * O;
      /* forward of the row: merged features, Linear1 pre-activation, then the
       * middle Linears' pre-activations z_{q+1} = W_mid[q] act(z_q) + b_mid[q] */
      orc_merged_row(s, x, gamma, beta, r, m);
      orc_linear(m, 1, (int32_t)K1, W1, b1, H, zs, 1);
      for (int32_t q = 0; q < n_mid; q++) {
        for (int32_t h = 0; h < H; h++) a[h] = act_value(s->act, zs[(int64_t)q * H + h]);
        orc_linear(a, 1, H, W_mid + (int64_t)q * H * H, b_mid + (int64_t)q * H, H,
                   zs + (int64_t)(q + 1) * H, 1);
      }
      const double *z = zs + (int64_t)n_mid * H; /* the last pre-activation */
      /* Linear2: y = W2 a + b2 */
      for (int32_t o = 0; o < O; o++) db2[o] += dy[o];
      for (int32_t o = 0; o < O; o++)
        for (int32_t h = 0; h < H; h++) dW2[(int64_t)o * H + h] += dy[o] * act_value(s->act, z[h]);
      /* the last activation */
      for (int32_t h = 0; h < H; h++) {
        double da = 0.0;
        for (int32_t o = 0; o < O; o++) da += dy[o] * W2[(int64_t)o * H + h];
        dz[h] = da * act_slope(s->act, z[h]);
      }
      /* middle Linears, last to first: layer q maps act(z_q) to z_{q+1} */
      for (int32_t q = n_mid - 1; q >= 0; q--) {
        const double *zq = zs + (int64_t)q * H;
        const double *Wq = W_mid + (int64_t)q * H * H;
        for (int32_t j = 0; j < H; j++) {
          db_mid[(int64_t)q * H + j] += dz[j];
          for (int32_t h = 0; h < H; h++)
            dW_mid[((int64_t)q * H + j) * H + h] += dz[j] * act_value(s->act, zq[h]);
        }
        for (int32_t h = 0; h < H; h++) {
          double da = 0.0;
          for (int32_t j = 0; j < H; j++) da += dz[j] * Wq[(int64_t)j * H + h];
          dzp[h] = da * act_slope(s->act, zq[h]);
        }
        memcpy(dz, dzp, sizeof(double) * H);
      }
      /* Linear1: z_0 = W1 m + b1 */
      for (int32_t h = 0; h < H; h++) {
        db1[h] += dz[h];
        for (int64_t i = 0; i < K1; i++) dW1[h * K1 + i] += dz[h] * m[i];
      }
      for (int64_t i = 0; i < K1; i++) {
        double acc = 0.0;
        for (int32_t h = 0; h < H; h++) acc += dz[h] * W1[h * K1 + i];
        dm[i] = acc;
      }
      /* space-to-depth, reversed: feature c*k*k + dy*k + dx of token (ty, tx)
       * came from cell (ty*k + dy, tx*k + dx); padded cells take no gradient */
      const int64_t ty = t / wp, tx = t % wp;
      for (int32_t ddy = 0; ddy < k; ddy++)
        for (int32_t ddx = 0; ddx < k; ddx++) {
          const int64_t y = ty * k + ddy, xx = tx * k + ddx;
          if (y >= gh || xx >= gw) continue;
          for (int32_t c = 0; c < C; c++)
            dn[(pix + y * gw + xx) * C + c] = dm[(int64_t)c * k * k + ddy * k + ddx];
        }
    }
    pix += (int64_t)gh * gw;
  }
  /* LayerNorm, reversed (or the identity without it) */
  for (int64_t p = 0; p < npix; p++) {
    if (s->has_ln)
      ln_backward_pixel(x + p * C, dn + p * C, C, gamma, s->ln_eps, dx + p * C, dgamma, dbeta);
    else
      memcpy(dx + p * C, dn + p * C, sizeof(double) * C);
  }
  free(m);
  free(zs);
  free(a);
  free(dz);
  free(dzp);
  free(dm);
  free(dn);
}

void orc_hidden_unit_grads(const orc_spec *s, const double *x, const double *gamma,
                           const double *beta, const double *W1, const double *b1,
                           const double *W2, const double *dY, int32_t h, double *dW1_row,
                           double *db1_h, double *dW2_col) {
  const int32_t C = s->C, k = s->k, H = s->hidden, O = s->out_dim;
  const int64_t K1 = (int64_t)C * k * k, T = orc_total_tokens(s);
  double *m = (double *)malloc(sizeof(double) * K1);
  memset(dW1_row, 0, sizeof(double) * K1);
  memset(dW2_col, 0, sizeof(double) * O);
  *db1_h = 0.0;
  for (int64_t r = 0; r < T; r++) {
    const double *dy = dY + r * O;
    orc_merged_row(s, x, gamma, beta, r, m);
    double z = 0.0;
    for (int64_t i = 0; i < K1; i++) z += m[i] * W1[(int64_t)h * K1 + i];
    z += b1[h];
    const double a = act_value(s->act, z);
    double da = 0.0;
    for (int32_t o = 0; o < O; o++) {
      dW2_col[o] += dy[o] * a;
      da += dy[o] * W2[(int64_t)o * H + h];
    }
    const double dz = da * act_slope(s->act, z);
    *db1_h += dz;
    for (int64_t i = 0; i < K1; i++) dW1_row[i] += dz * m[i];
  }
  free(m);
}

void orc_pixel_grad(const orc_spec *s, const double *x, const double *gamma, const double *beta,
                    const double *W1, const double *b1, const double *W2, const double *dY,
                    int32_t v, int32_t y, int32_t xx, double *dx_out) {
  const int32_t C = s->C, k = s->k, H = s->hidden, O = s->out_dim;
  const int64_t K1 = (int64_t)C * k * k;
  int64_t pix0, row0;
  view_bases(s, v, &pix0, &row0);
  const int32_t gw = s->grid_w[v];
  const int64_t r = row0 + (y / k) * orc_merged_side(gw, k) + xx / k;
  const int32_t p = (y % k) * k + xx % k;
  double *m = (double *)malloc(sizeof(double) * K1);
  double *z = (double *)malloc(sizeof(double) * H);
  double *dn = (double *)malloc(sizeof(double) * C);
  orc_merged_row(s, x, gamma, beta, r, m);
  orc_linear(m, 1, (int32_t)K1, W1, b1, H, z, 1);
  const double *dy = dY + r * O;
  for (int32_t c = 0; c < C; c++) dn[c] = 0.0;
  for (int32_t h = 0; h < H; h++) {
    double da = 0.0;
    for (int32_t o = 0; o < O; o++) da += dy[o] * W2[(int64_t)o * H + h];
    const double dz = da * act_slope(s->act, z[h]);
    for (int32_t c = 0; c < C; c++) dn[c] += dz * W1[(int64_t)h * K1 + (int64_t)c * k * k + p];
  }
  const double *px = x + (pix0 + (int64_t)y * gw + xx) * C;
  if (s->has_ln)
    ln_backward_pixel(px, dn, C, gamma, s->ln_eps, dx_out, NULL, NULL);
  else
    memcpy(dx_out, dn, sizeof(double) * C);
  free(m);
  free(z);
  free(dn);
}

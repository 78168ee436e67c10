/*
 * vlbridge.h -- C ABI of the vision-to-language bridge for AMD Instinct MI355X
 * (gfx950): k x k space-to-depth merge of a ViT patch grid, two-Linear GELU
 * projector, and scatter of the projected tokens into a text-embedding
 * sequence at the image-placeholder positions.
 *
 * Pages that define the operations (cited by title and section):
 *   [VL2]  mlxcel issue #533, "feat(models): port DeepSeek-VL2" -- sections
 *          "Projector (downsample_mlp_gelu)", "Tile-sequence assembly
 *          (tile_tag 2D)", "Processor" step 7, "Weight loading and sanitize",
 *          "Validation and acceptance criteria".
 *   [V4V]  "DeepSeek-V4-Flash-Vision-BF16" model card, header paragraph
 *          (2x2 PatchMerger, 4608 -> 4096).
 *   [VOIE] "La voie visuelle" (DeepSeek-V4.1-Flash), sections "Le chemin d'une
 *          image" and "Le pixel-unshuffle 3x3".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE memory owned by the caller unless marked (host).  The
 *    library allocates nothing on the device and keeps no state between calls
 *    (apart from the optional profiling records below); calls with distinct
 *    workspaces may run concurrently on different streams.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    Work is enqueued asynchronously on it.
 *  - Every argument and shape is validated on the host before anything is
 *    enqueued; on error nothing is launched and the status is returned.  No
 *    HIP call is made before validation has passed.
 *  - dtype: one type for features, LayerNorm parameters, weights, biases,
 *    newline/separator vectors, projected rows and the sequence.  VLB_BF16
 *    computes with fp32 accumulation and keeps the hidden activation in bf16;
 *    VLB_F32 computes in fp32 throughout.
 *  - Features: views stored back to back, each (grid_h, grid_w, C) row-major
 *    channels-last: the tower's per-view token sequence with its token index
 *    read as grid row, then column [VL2 Projector 1].  Images own consecutive
 *    views; for the 2D tile layout an image's views are [global, local tiles
 *    row-major].
 *  - Token rows: the projected tokens of all views, concatenated in view order,
 *    each view's tokens row-major over its merged grid [VL2 Projector, Output].
 *  - Alignment: every device pointer must be 16-byte aligned.
 *  - Supported shapes: k in {1, 2, 3}; C, hidden and out_dim multiples of 8
 *    (VLB_BF16 additionally: C and hidden multiples of 64, C <= 4096); with
 *    LayerNorm, C <= 2048 for VLB_F32.
 */
#ifndef VLBRIDGE_H
#define VLBRIDGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VLB_OK = 0,
  VLB_ERR_NULL = 1,        /* a required pointer is NULL */
  VLB_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  VLB_ERR_DTYPE = 3,       /* unknown dtype */
  VLB_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  VLB_ERR_WORKSPACE = 5,   /* workspace smaller than vlb_workspace_bytes() */
  VLB_ERR_MASK_COUNT = 6,  /* placeholder count != assembled slots (device-detected) */
  VLB_ERR_UNSUPPORTED = 7, /* a valid but unsupported setting */
  VLB_ERR_HIP = 8,         /* a HIP runtime call failed */
  VLB_ERR_TOKEN_ID = 9,    /* a text token id outside [0, vocab) (device-detected) */
  VLB_ERR_SCRATCH = 10     /* the problem's workspace exceeds VLB_NOALLOC_SCRATCH_BYTES */
} vlb_status;

typedef enum { VLB_F32 = 0, VLB_BF16 = 1 } vlb_dtype;

/* Activation between the two Linears.  The projector of [VL2 Projector 3] is
 * Linear -> GELU -> Linear; the exact (erf) GELU is the default, the tanh
 * approximation and no activation are available as flags. */
typedef enum { VLB_GELU_ERF = 0, VLB_GELU_TANH = 1, VLB_ACT_NONE = 2 } vlb_act;

/* PLAIN: every image's token rows go to its placeholders in token order
 * (MoonViT / DeepSeek-ViT style, [V4V], [VOIE]).  TILED_2D: the global view
 * with one newline per token row, the separator, then the local views as one
 * mosaic with one newline per mosaic row [VL2 Tile-sequence assembly]. */
typedef enum { VLB_LAYOUT_PLAIN = 0, VLB_LAYOUT_TILED_2D = 1 } vlb_layout;

/* VLB_GATHER_ON: the first Linear reads each merged token straight from the
 * patch grid -- the space-to-depth [VL2 Projector 2] happens inside its operand
 * loads -- so the merged tokens never exist in memory and the workspace is
 * T * C * k * k * 2 bytes smaller (T rounded up to 256).  VLB_BF16 without
 * LayerNorm only (else VLB_ERR_UNSUPPORTED).  VLB_GATHER_OFF: the grid is first
 * merged (with the LayerNorm, when on) into the GEMM's blocked operand.
 * VLB_GATHER_AUTO: the library chooses -- the gather for VLB_BF16 without
 * LayerNorm and hidden <= 4096, where the merge pass costs more than the
 * slower gathered loads.  Both forms give the same bits.  The training forward
 * keeps the merged tokens, so it always merges. */
typedef enum { VLB_GATHER_AUTO = 0, VLB_GATHER_ON = 1, VLB_GATHER_OFF = 2 } vlb_gather;

/* The projector: LN(C) (optional, per patch, biased variance, eps inside the
 * square root, affine) -> pad to a multiple of k -> k x k space-to-depth with
 * feature index c*k*k + dy*k + dx [VL2 Projector 1-2] -> Linear(C*k*k ->
 * hidden) -> act -> Linear(hidden -> out_dim) [VL2 Projector 3].  With depth
 * d > 2 (the projector config's "depth", d Linears in all), d - 2 further
 * (act -> Linear(hidden -> hidden)) pairs sit between the two [VL2 Projector
 * 3]. */
typedef struct {
  int32_t dtype;     /* vlb_dtype */
  int32_t C;         /* channels of the patch grid */
  int32_t k;         /* merge factor: 1, 2 or 3 */
  int32_t hidden;    /* width of the first Linear's output */
  int32_t out_dim;   /* width of the projected tokens (the text model's width) */
  int32_t has_ln;    /* 1: LayerNorm over C before the merge */
  float ln_eps;      /* LayerNorm epsilon */
  int32_t act;       /* vlb_act */
  int32_t packed;    /* 1: weights.w1 / weights.w2 are the packed forms made by
                        vlb_pack_weights, and weights.w_mid[i] those made by
                        vlb_pack_mid (VLB_BF16 only) */
  int32_t depth;     /* Linears in the projector: 2..16; 0 is read as 2 */
  int32_t gather;    /* vlb_gather: where the first Linear's operand comes from */
} vlb_projector;

/* Weights in PyTorch Linear layout (out_features, in_features), as stored and
 * used as-is [VL2 Weight loading]. */
typedef struct {
  const void *ln_gamma, *ln_beta; /* [C] each, or NULL when has_ln == 0 */
  const void *w1;                 /* [hidden][C*k*k]; or its packed form */
  const void *b1;                 /* [hidden] */
  const void *w2;                 /* [out_dim][hidden]; or its packed form */
  const void *b2;                 /* [out_dim] */
  const void *const *w_mid;       /* (host) [depth - 2] device pointers, each [hidden][hidden]
                                     (or its packed form), in order; NULL when depth <= 2 */
  const void *const *b_mid;       /* (host) [depth - 2] device pointers, each [hidden] */
} vlb_weights;

/* Batch description; all arrays are (host) memory read during the call only. */
typedef struct {
  int32_t n_views;                 /* >= 0; 0 = text only (the bridge is a no-op) */
  const int32_t *grid_h, *grid_w;  /* (host) [n_views], each in [1, 32767] */
  int32_t n_images;                /* images; their views sum to n_views */
  const int32_t *views_per_image;  /* (host) [n_images] */
  int32_t layout;                  /* vlb_layout */
  const int32_t *tile_w, *tile_h;  /* (host) [n_images], TILED_2D only: the [tw, th]
                                      tile grid, width count first [VL2 Processor 6];
                                      each image then has 1 + tw*th views of one
                                      common grid */
  int32_t global_view_tail;        /* TILED_2D: 0 = [global, sep, local] ("head"),
                                      1 = [local, sep, global] ("tail") */
} vlb_batch;

/* ---- sizing (host only, no HIP call) ---------------------------------- */

/* Projected token rows T of the batch, or -(vlb_status) on invalid input. */
int64_t vlb_num_tokens(const vlb_projector *p, const vlb_batch *b);
/* Assembled placeholder slots P = T + newlines + separators [VL2 Processor 7],
 * or -(vlb_status). */
int64_t vlb_num_slots(const vlb_projector *p, const vlb_batch *b);
/* Slots of each image, written to (host) out[n_images]; returns the total P or
 * -(vlb_status). */
int64_t vlb_image_slots(const vlb_projector *p, const vlb_batch *b, int64_t *out);
/* Device workspace bytes needed by any entry point below for this batch and a
 * sequence of seq_len rows (0 when only vlb_merge_project is used); 0 on
 * invalid input. */
size_t vlb_workspace_bytes(const vlb_projector *p, const vlb_batch *b, int64_t seq_len);

/* ---- entry points (asynchronous on stream) ---------------------------- */

/* Bytes of the packed form of W1 (which = 1), W2 (which = 2) or one middle
 * weight (which = 3); 0 on invalid input or for VLB_F32 (which has no packed
 * form). */
size_t vlb_packed_bytes(const vlb_projector *p, int32_t which);

/* One-time re-layout of the weights into the GEMMs' tile-blocked forms
 * (VLB_BF16 only).  Packed W is [ceil(N/256)][K/32][256][32]: for every
 * 256-row block of outputs and every 32-wide K slice, the block's 256 rows of
 * that slice are one contiguous 16 KiB run (rows past N are zero).  For W1 the
 * K axis is also reordered position-major (index p*C + c instead of the
 * pages' c*k*k + p) so a K slice is contiguous channels of one pixel; only the
 * summation order of the first Linear changes.  w1 [hidden][C*k*k] and w2
 * [out_dim][hidden] are read; w1_packed / w2_packed (vlb_packed_bytes each)
 * are written and must not overlap the inputs. */
vlb_status vlb_pack_weights(const vlb_projector *p, const void *w1, const void *w2,
                            void *w1_packed, void *w2_packed, void *stream);

/* The same re-layout for one middle weight [hidden][hidden] of a projector of
 * depth > 2 (no reordering, like W2); w_packed holds vlb_packed_bytes(p, 3)
 * bytes and must not overlap w. */
vlb_status vlb_pack_mid(const vlb_projector *p, const void *w, void *w_packed, void *stream);

/* LN (if enabled) -> pad -> space-to-depth, materialised: merged[T][C*k*k] in
 * the pages' feature order c*k*k + dy*k + dx [VL2 Projector 1-2], [VOIE
 * pixel-unshuffle].  ws: workspace of vlb_workspace_bytes(p, b, 0) bytes (used
 * only when has_ln). */
vlb_status vlb_merge_tokens(const vlb_projector *p, const vlb_batch *b, const void *features,
                            const void *ln_gamma, const void *ln_beta, void *merged, void *ws,
                            size_t ws_bytes, void *stream);

/* The projector: rows[T][out_dim] = Linear2(act(Linear1(merge(LN(features)))))
 * [VL2 Projector 1-3]. */
vlb_status vlb_merge_project(const vlb_projector *p, const vlb_batch *b, const void *features,
                             const vlb_weights *w, void *rows, void *ws, size_t ws_bytes,
                             void *stream);

/* Assembly and scatter [VL2 Tile-sequence assembly]: the assembled rows (token
 * rows, plus newline/separator for TILED_2D) overwrite seq[seq_len][out_dim]
 * in place at the positions where mask[seq_len] (uint8) is nonzero, in order;
 * all other rows of seq are untouched.  newline/separator: [out_dim] each
 * (TILED_2D; may be NULL for PLAIN).  If the number of nonzero mask entries
 * differs from P [VL2 Validation], the device writes nothing to seq and
 * records VLB_ERR_MASK_COUNT, which vlb_check returns.  T == 0 is a no-op. */
vlb_status vlb_scatter_tokens(const vlb_projector *p, const vlb_batch *b, const void *rows,
                              const void *newline, const void *separator, const uint8_t *mask,
                              int64_t seq_len, void *seq, void *ws, size_t ws_bytes,
                              void *stream);

/* vlb_merge_project followed by vlb_scatter_tokens without materialising the
 * projected rows: the second GEMM writes each row straight to its placeholder
 * slot.  Same arguments and error behaviour as the two calls. */
vlb_status vlb_bridge_fused(const vlb_projector *p, const vlb_batch *b, const void *features,
                            const vlb_weights *w, const void *newline, const void *separator,
                            const uint8_t *mask, int64_t seq_len, void *seq, void *ws,
                            size_t ws_bytes, void *stream);

/* vlb_bridge_fused for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The workspace is a library-owned device array of
 * VLB_NOALLOC_SCRATCH_BYTES (256 MiB) that every GPU running the library
 * holds until the process ends; the call makes no allocation of any kind on
 * the device.  Inputs, outputs and errors as vlb_bridge_fused, plus:
 *   status: (device) int32[4], 16-byte aligned, written with the call's
 *     status words (all zero when there are no token rows); vlb_check(status,
 *     stream) returns VLB_ERR_MASK_COUNT for a placeholder-count mismatch.
 *   VLB_GATHER_AUTO is taken as VLB_GATHER_ON where that is allowed, so the
 *     merged tokens take no scratch; the bits are the same.
 *   VLB_ERR_SCRATCH (nothing launched): vlb_workspace_bytes of the problem
 *     (with that gather choice) exceeds VLB_NOALLOC_SCRATCH_BYTES.
 * Every call on a GPU uses that GPU's one array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller. */
#define VLB_NOALLOC_SCRATCH_BYTES (256u << 20)
vlb_status vlb_bridge_fused_noalloc(const vlb_projector *p, const vlb_batch *b,
                                    const void *features, const vlb_weights *w,
                                    const void *newline, const void *separator,
                                    const uint8_t *mask, int64_t seq_len, void *seq,
                                    int32_t *status, void *stream);

/* The whole embedded sequence in one call [VL2 Tile-sequence assembly, last
 * paragraph; VL2 language config: vocab_size 102400, image_token_index
 * 100015]: every position s of seq [seq_len][out_dim] whose id is not
 * image_token_id receives row ids[s] of the token-embedding table embed
 * [vocab][out_dim]; the positions holding image_token_id receive the
 * projected visual rows (and newline / separator rows), in order, exactly as
 * vlb_bridge_fused places them.  Every row of seq is written.
 *   ids: int32 [seq_len] (device).  embed: dtype, row-major.
 *   Device-detected errors (reported by vlb_check; nothing is written): the
 *   number of image_token_id positions differs from vlb_num_slots
 *   (VLB_ERR_MASK_COUNT), else a text id lies outside [0, vocab)
 *   (VLB_ERR_TOKEN_ID).  A batch without images (n_views = 0) writes the
 *   text embeddings only.  Workspace: vlb_workspace_bytes(p, b, seq_len). */
vlb_status vlb_bridge_embed(const vlb_projector *p, const vlb_batch *b, const void *features,
                            const vlb_weights *w, const void *newline, const void *separator,
                            const int32_t *ids, int32_t image_token_id, const void *embed,
                            int64_t vocab, int64_t seq_len, void *seq, void *ws, size_t ws_bytes,
                            void *stream);

/* ---- training the projector ------------------------------------------- */
/*
 * The projector is the trained part of the bridge: [V4V header] trains only
 * its parameters (tower and text model frozen), and [VOIE "Pendant le
 * pré-entraînement du squelette"] keeps it trainable while the tower is
 * frozen.  A training step calls vlb_bridge_fused_train (the forward, keeping
 * what the backward needs in `saved`) and then vlb_bridge_backward with the
 * gradient of the loss with respect to the sequence.  The gradients are the
 * chain rule through [VL2 Projector 1-3] and [VL2 Tile-sequence assembly].
 */

/* Bytes of the saved-activation buffer of a batch (the merged tokens and the
 * pre-activation of the first and every middle Linear, and for VLB_BF16 their
 * activations too: tile-blocked for VLB_BF16, row-major for VLB_F32; the
 * contents are opaque); 0 on invalid input. */
size_t vlb_saved_bytes(const vlb_projector *p, const vlb_batch *b);

/* Device workspace bytes of vlb_bridge_backward for this batch and sequence
 * length; 0 on invalid input or an unsupported setting (see below). */
size_t vlb_backward_workspace_bytes(const vlb_projector *p, const vlb_batch *b, int64_t seq_len);

/* vlb_bridge_fused (same arguments, errors and sequence values), and the
 * activations the backward needs written to saved (vlb_saved_bytes bytes,
 * which must not overlap any other argument). */
vlb_status vlb_bridge_fused_train(const vlb_projector *p, const vlb_batch *b,
                                  const void *features, const vlb_weights *w,
                                  const void *newline, const void *separator,
                                  const uint8_t *mask, int64_t seq_len, void *seq, void *saved,
                                  size_t saved_bytes, void *ws, size_t ws_bytes, void *stream);

/* Gradient outputs of vlb_bridge_backward: fp32 unless marked, each written
 * whole (not accumulated into). */
typedef struct {
  void *d_features;               /* [n_pixels][C] in the projector dtype; NULL: skipped */
  float *d_w1;                    /* [hidden][C*k*k], the pages' feature order */
  float *d_b1;                    /* [hidden] */
  float *d_w2;                    /* [out_dim][hidden] */
  float *d_b2;                    /* [out_dim] */
  float *d_ln_gamma, *d_ln_beta;  /* [C]; has_ln only (ignored otherwise) */
  float *d_newline, *d_separator; /* [out_dim]; TILED_2D only (ignored otherwise) */
  float *const *d_w_mid;          /* (host) [depth - 2] device pointers, each [hidden][hidden];
                                     depth > 2 only */
  float *const *d_b_mid;          /* (host) [depth - 2] device pointers, each [hidden] */
} vlb_grads;

/* Backward of the bridge.  dseq [seq_len][out_dim] (dtype) is the gradient of
 * the loss with respect to the sequence vlb_bridge_fused_train wrote; its rows
 * at text positions (mask == 0) are not read.  features, w, mask and saved
 * must be those of that forward call (features and w->ln_gamma are read only
 * with the LayerNorm; w->w1, w->w2 and w->w_mid as the projector says,
 * unpacked or packed -- unpacked ones are packed into the workspace first;
 * biases and ln_beta are not read).  Every token row's gradient is the dseq row of its
 * slot; the newline and separator gradients sum the rows of all their slots;
 * padded merge cells take no gradient.
 * Unsupported (VLB_ERR_UNSUPPORTED): has_ln with C > 2048.  Device-detected placeholder-count mismatch: nothing is written
 * and vlb_check(ws) returns VLB_ERR_MASK_COUNT.  With no token rows
 * (n_views = 0) every gradient is set to zero and the mask is not read.
 * Workspace: vlb_backward_workspace_bytes(p, b, seq_len). */
vlb_status vlb_bridge_backward(const vlb_projector *p, const vlb_batch *b, const void *features,
                               const vlb_weights *w, const uint8_t *mask, int64_t seq_len,
                               const void *dseq, const void *saved, size_t saved_bytes,
                               const vlb_grads *g, void *ws, size_t ws_bytes, void *stream);

/* Waits for stream and returns the status recorded on the device by the last
 * vlb_scatter_tokens / vlb_bridge_fused / vlb_bridge_fused_train /
 * vlb_bridge_embed / vlb_bridge_backward that used this workspace (VLB_OK,
 * VLB_ERR_MASK_COUNT or VLB_ERR_TOKEN_ID), or VLB_ERR_HIP. */
vlb_status vlb_check(void *ws, void *stream);

const char *vlb_status_str(vlb_status s);

/* ---- request planning (host only, no HIP call) -------------------------- */
/*
 * The processor steps that decide the batch [VL2 Processor]: step 1 (crop
 * only when a request has at most 2 images), step 2 (best-fit candidate
 * resolution), step 6 (the [tw, th] tile grid, width count first) and step 7
 * (placeholder count and expansion of the prompt).  A planned image has
 * 1 + tw*th views of floor(image_size / patch_size)^2 patches each.
 */
typedef struct {
  const int32_t *candidates; /* (host) [n_candidates][2] (W, H) in pixels, whole multiples of
                                image_size = candidates[0][0] */
  int32_t n_candidates;
  int32_t patch_size;        /* the tower's patch size */
  int32_t downsample;        /* the projector's merge factor k */
} vlb_processor;

/* [VL2 Processor step 2] for an image of w0 x h0 pixels: per candidate,
 * scale = min(W / w0, H / h0) and effective = min(floor(w0 * scale) *
 * floor(h0 * scale), w0 * h0) in IEEE double; the largest effective area
 * wins, then the smallest W * H - effective, then the first listed.  best:
 * (host) int32[2] = (W, H).  Errors: VLB_ERR_NULL, VLB_ERR_SHAPE (sizes < 1,
 * candidates not whole tiles, image_size < patch_size). */
vlb_status vlb_select_resolution(const vlb_processor *pc, int32_t w0, int32_t h0, int32_t *best);

/* [VL2 Processor steps 1, 2, 6, 7] for the n_images images of one request,
 * sizes (host) [n_images][2] = (w0, h0): cropping only when n_images <= 2
 * (otherwise every image is 1 x 1); tiles (host, out) [n_images][2] =
 * [tw, th]; slots (host, out) [n_images] = h'(w'+1) + 1 + (th h')(tw w' + 1)
 * with h' = w' = ceil(floor(image_size / patch_size) / downsample), the
 * image's placeholder count (vlb_image_slots of the planned batch). */
vlb_status vlb_plan_request(const vlb_processor *pc, int32_t n_images, const int32_t *sizes,
                            int32_t *tiles, int64_t *slots);

/* [VL2 Processor step 7] placeholder expansion of a prompt holding one
 * image_token_id per image: out (host) = bos_id, then ids with its i-th
 * image_token_id replaced by slots[i] copies of it.  Returns the length
 * (with out == NULL: the length only), or -VLB_ERR_SHAPE when the prompt's
 * image tokens differ from n_images or the length exceeds cap, -VLB_ERR_NULL. */
int64_t vlb_expand_prompt(const int32_t *ids, int64_t n_ids, int32_t image_token_id,
                          int32_t bos_id, const int64_t *slots, int32_t n_images, int32_t *out,
                          int64_t cap);

/* ---- optional per-kernel timing ---------------------------------------- */

/* Kernel ids for the timing records. */
enum {
  VLB_K_PLAN = 0,    /* per-token gather descriptors */
  VLB_K_SCAN = 1,    /* mask / token-id prefix sum -> slot positions (on the plain bf16
                        path of the fused calls it runs inside the merge launch, timed
                        as VLB_K_LN or VLB_K_MERGE) */
  VLB_K_PLACE = 2,   /* assembly map, newline/separator rows */
  VLB_K_LN = 3,      /* LayerNorm (bf16: fused with the merge into Linear1's operand) */
  VLB_K_GEMM1 = 4,   /* Linear1 + bias + activation (fp32: gathering the merge itself) */
  VLB_K_GEMM2 = 5,   /* Linear2 + bias + row/slot store */
  VLB_K_SCATTER = 6, /* standalone row scatter */
  VLB_K_MERGE = 7,   /* space-to-depth (bf16 without LayerNorm: into Linear1's operand) */
  VLB_K_PACK = 8,    /* weight re-layout */
  VLB_K_EMBED = 9,   /* token-embedding rows */
  VLB_K_BWD_PACK = 10,    /* backward: gradient gather and operand transposes */
  VLB_K_BWD_DW2 = 11,     /* backward: dW2 = dY^T act(Z1) (and the sum of its K-split tail tiles) */
  VLB_K_BWD_DA1 = 12,     /* backward: dA1 = dY W2 */
  VLB_K_BWD_DW1 = 13,     /* backward: dW1 = dZ1^T Xm (and the sum of its K-split tail tiles) */
  VLB_K_BWD_DX = 14,      /* backward: dXm = dZ1 W1 */
  VLB_K_BWD_UNMERGE = 15, /* backward: unmerge + LayerNorm backward */
  VLB_K_BWD_SUM = 16,     /* backward: bias / LayerNorm / newline sums */
  VLB_K_GEMM_MID = 17,    /* middle Linears (depth > 2) */
  VLB_K_COUNT = 18
};

/* Launch timing.  mask bit kid (1 << VLB_K_*) enables timing of that kernel
 * id: each such launch is bracketed by HIP events recorded on the stream it
 * runs on.  A nonzero mask clears earlier records; 0 stops recording; -1
 * times every kernel. */
vlb_status vlb_prof_enable(int32_t mask);
/* Sets the mask like vlb_prof_enable but keeps the records taken so far, so
 * that only some launches of a run are bracketed (0 pauses recording). */
vlb_status vlb_prof_resume(int32_t mask);
/* Waits for the recorded events and returns, for kernel id kid, the number of
 * launches and their summed duration in milliseconds. */
vlb_status vlb_prof_read(int32_t kid, int64_t *launches, double *total_ms);

#ifdef __cplusplus
}
#endif
#endif /* VLBRIDGE_H */

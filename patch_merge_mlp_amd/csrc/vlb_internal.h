// Internal declarations shared by the host planner (vlb_api.hip) and the HIP
// kernels (vlb_data.hip, vlb_gemm.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace vlb {

// ---- per-token gather descriptor ------------------------------------------
// pix: index (in pixels, over all views) of the top-left pixel of the token's
//      k x k block.
// geo: bits 0..15  the view's grid width (pixel stride of one grid row);
//      bits 16..24 bit (dy*k + dx) set when that block position lies inside the
//                  grid (clear = high-end zero padding).
// A token row past the end of the batch is never read.
struct RowDesc {
  int32_t pix;
  int32_t geo;
};

// Views handled by one launch of the descriptor or blocked-merge kernel
// (kernel-argument table; one view per lane of a wave in the latter).
constexpr int kPlanViews = 64;
struct PlanChunk {
  int32_t n;                     // views in this chunk
  int32_t k;                     // merge factor
  int32_t tok0[kPlanViews + 1];  // first token row of each view; tok0[n] = end
  int32_t pix0[kPlanViews];      // first pixel of each view
  int16_t gh[kPlanViews], gw[kPlanViews];
};

// Tiled images handled by one launch of the placement kernel.
constexpr int kPlaceImages = 64;
struct PlaceChunk {
  int32_t n;                        // images in this chunk
  int32_t tail;                     // 1: [local, separator, global]
  int32_t slot0[kPlaceImages + 1];  // first assembled slot of each image; slot0[n] = end
  int32_t row0[kPlaceImages];       // first token row of each image (its global view)
  int16_t hp[kPlaceImages], wp[kPlaceImages];  // merged grid of every view of the image
  int16_t tw[kPlaceImages], th[kPlaceImages];  // local tile grid, width count first
  // Recording mode (gradients): newline slots of image i go to list entries
  // nl0[i] + ordinal (ordinal in assembly order), its separator to entry img0 + i.
  int32_t nl0[kPlaceImages];
  int32_t img0;
};

// Status words at the start of the workspace.
enum { kStatusWord = 0, kCountWord = 1 };

// ---- GEMM arguments -------------------------------------------------------
// out[dst(m)][n] = act(sum_k A[m][k] * B[n][k] + bias[n]) for m < M, n < N.
// bf16 path: A and B are tile-blocked (see blocked_elems).  Linear1 takes the
// merged tokens with K ordered position-major (k' = p*C + c) and the packed
// W1, and writes its output tile-blocked; Linear2 takes that blocked A and
// writes plain rows to dst(m).  fp32 path: plain row-major B; Linear1 gathers
// A through RowDesc from the patch grid with K of W1 in the pages' order.
struct GemmArgs {
  const void *A;          // activations, or the (normalised) patch grid (fp32 gather)
  const RowDesc *desc;    // gather descriptors (fp32 gather mode only)
  const void *B;          // weights
  const void *bias;       // [N]
  void *out;              // output rows
  const int32_t *dst_row; // nullptr: row m -> out + m*ldo; else dst_row[m] (< 0: skipped)
  int32_t M, N, K, ldo;
  int32_t C, k;           // fp32 gather mode: channels and merge factor
  int32_t act;            // vlb_act
  int32_t tiles_m, tiles_n;
  uint32_t a_bytes, b_bytes;  // extent of A and B in bytes (< 2^31): loads past it read 0
  // bf16 path: tiles [0, n_full) of the 256-grid are computed as 256x256
  // tiles, the rest as 128x128 tiles (see tile_plan).
  int32_t n_full;
  void *out2;              // kGemmBlockedSave: the pre-activation, tile-blocked like out
  const int32_t *status;   // kGemmF32 / fp32: nothing is written when status[0] != 0 (may be null)
  // fp32 path, not gather mode: element (m, k) of A at A[m * sa_m + k * sa_k] and
  // (n, k) of B at B[n * sb_n + k * sb_k]; sa_k == 0 (sb_k == 0) means row-major.
  int64_t sa_m, sa_k, sb_n, sb_k;
  // kGemmRows: 1 = rows written with non-temporal stores (rows nobody reads
  // back soon: Linear2's rows into the sequence), 0 = ordinary stores.
  int32_t stream_out;
  // kGemmF32 only: with split_part set (gemm_split_bytes of room), tiles past
  // n_full that gemm_k_splits splits are computed as k_splits K ranges each,
  // every range a whole 256x256 fp32 tile in split_part, and the ranges of a
  // tile are added in order into out by a second kernel.  Set by the launcher.
  float *split_part;
  int32_t k_splits;
  // bf16 path, b_tmaj: B is token-major, stored tile-blocked with the
  // contraction index as its row -- [K][W] with element (k, n) at
  // ((k/256 * W/32 + n/32) * 256 + k%256) * 32 + n%32 -- so a product that
  // contracts over tokens reads it as the producing kernel wrote it, and a
  // packed weight [N][K] serves as the B of the product with its transpose.
  // tb_w: the stored width W (a multiple of 32); contraction indices at or
  // past k_valid read zero.
  int32_t b_tmaj;
  int32_t tb_w, k_valid;
};

// Epilogues of the bf16 GEMM.
enum GemmMode {
  kGemmBlocked = 0,      // bias + activation, bf16 tile-blocked output (Linear1)
  kGemmRows = 1,         // bias, bf16 rows to dst(m) (Linear2)
  kGemmF32 = 2,          // fp32 rows out + m*ldo, no bias (weight gradients)
  kGemmBlockedSave = 3,  // kGemmBlocked, and bias without activation to out2 as well
  // kGemmBlocked with A gathered from the bf16 patch grid (NHWC, g.A) through
  // the per-token descriptors g.desc: the merge is never materialised.  K runs
  // position-major (the packed W1's order); g.C (a multiple of 32) and g.k
  // give the block geometry, g.a_bytes the grid's extent.
  kGemmGatherBlocked = 4,
};

// Tile plan of the bf16 GEMM.  256x256 tiles keep the MFMAs busiest, but on
// 256 compute units a last round that is at most half full wastes most of a
// round; those tiles are computed as four 128x128 tiles each instead, so the
// last round fills the chip.  Problems with fewer than 128 big tiles use
// 128x128 tiles throughout.
constexpr int kGemmBK = 32;         // K per pipeline step
constexpr int kGemmStages = 4;      // pipeline stages
constexpr int kPlanCUs = 256;       // compute units of MI355X
struct TilePlan {
  int32_t tiles_m, tiles_n;  // 256-grid
  int32_t n_full;            // 256x256 tiles (one workgroup each)
  int32_t blocks128;         // 128x128 tiles (one workgroup each)
};
inline TilePlan tile_plan(int64_t M, int64_t N) {
  TilePlan tp{};
  tp.tiles_m = static_cast<int32_t>((M + 255) / 256);
  tp.tiles_n = static_cast<int32_t>((N + 255) / 256);
  const int32_t tiles = tp.tiles_m * tp.tiles_n;
  const int32_t rem = tiles % kPlanCUs;
  if (tiles < kPlanCUs / 2) {
    tp.n_full = 0;
    tp.blocks128 = static_cast<int32_t>(((M + 127) / 128) * ((N + 127) / 128));
  } else if (rem > 0 && rem <= kPlanCUs / 2) {
    tp.n_full = tiles - rem;
    tp.blocks128 = 4 * rem;
  } else {
    tp.n_full = tiles;
    tp.blocks128 = 0;
  }
  return tp;
}

// K splits of the tiles past n_full of an fp32-output product (weight
// gradients: K = tokens, long).  Their quarter tiles would need two rounds
// (more than 256 of them), or each would run the whole K through a 128x128
// tile at about two thirds of a whole tile's rate; as S whole 256x256 tiles
// over a K range each (S * rem <= 256 CUs, one round) they finish in about
// 1/S of a whole tile's time, plus a pass adding the S partial tiles.
// 1: no split.
inline int gemm_k_splits(const TilePlan &tp, int64_t K) {
  const int rem = tp.tiles_m * tp.tiles_n - tp.n_full;
  if (tp.n_full == 0 || tp.blocks128 == 0 || rem <= 0) return 1;
  const int S = std::min(8, kPlanCUs / rem);
  if (S < 2 || K / kGemmBK < 16 * S) return 1;  // at least 16 K steps per range
  return (4 * rem > kPlanCUs || S >= 6) ? S : 1;
}
// Bytes of GemmArgs::split_part that an M x N x K kGemmF32 product needs (0: none).
inline size_t gemm_split_bytes(int64_t M, int64_t N, int64_t K) {
  const TilePlan tp = tile_plan(M, N);
  const int S = gemm_k_splits(tp, K);
  if (S < 2) return 0;
  return static_cast<size_t>(tp.tiles_m * tp.tiles_n - tp.n_full) * S * 256 * 256 * sizeof(float);
}

// ---- launchers (return the launch error, hipSuccess otherwise) ------------
// Placeholder scan over a uint8 mask (ids == nullptr) or over token ids
// (placeholder = image_id; other ids must lie in [0, vocab)).
// direct (plain layout): slot_pos is dst_row [P] and receives the positions
// themselves, or -1 everywhere when the input is invalid.
hipError_t launch_scan(const uint8_t *mask, const int32_t *ids, int32_t image_id, int64_t vocab,
                       int64_t S, int64_t P, int32_t *slot_pos, int32_t *status, bool direct,
                       hipStream_t s, int32_t *text = nullptr);
// The same scan, carried by a merge launch (launch_merge_blocked) as one extra
// workgroup that runs beside the merge: it reads neither the features nor
// the merged rows, so the two need no ordering.
struct ScanJob {
  const uint8_t *mask;
  const int32_t *ids;
  int32_t image_id;
  int64_t vocab;
  int64_t S, P;
  int32_t *slot_pos;
  int32_t *status;
  bool direct;
  // token-id form, optional: the (position, id) pairs of the text positions,
  // in order ([S][2] int32 of room: a count mismatch may leave more than S - P)
  int32_t *text = nullptr;
};
// dst[0..3] = src[0..3] (the status words), or zeros when src is null.
hipError_t launch_copy_status(const int32_t *src, int32_t *dst, hipStream_t s);
// Gather descriptors of the token rows of one chunk of views; with scan
// non-null, the launch also runs that placeholder scan (one extra workgroup).
hipError_t launch_plan(const PlanChunk &c, RowDesc *desc, hipStream_t s,
                       const ScanJob *scan = nullptr);
// seq[q] = embed[id] for the first n (q, id) pairs of text, the list the
// token-id scan writes (nothing if the scan failed).
hipError_t launch_embed_rows(int dtype, const int32_t *text, int64_t n, const void *embed, int D,
                             const int32_t *status, void *seq, hipStream_t s);
hipError_t launch_place_tiled(int dtype, const PlaceChunk &c, const int32_t *slot_pos,
                              const int32_t *status, int32_t *dst_row, const void *newline,
                              const void *separator, void *seq, int D, hipStream_t s);
// The same decode without writing the sequence: dst_row as above, and the
// sequence positions of the newline and separator slots into nl_pos / sep_pos
// (see PlaceChunk::nl0, img0).
hipError_t launch_place_tiled_record(const PlaceChunk &c, const int32_t *slot_pos,
                                     const int32_t *status, int32_t *dst_row, int32_t *nl_pos,
                                     int32_t *sep_pos, hipStream_t s);
// Largest C the LayerNorm kernel keeps in registers.
int layernorm_max_channels(int dtype);
hipError_t launch_layernorm(int dtype, const void *x, int64_t npix, int C, const void *gamma,
                            const void *beta, float eps, void *out, hipStream_t s);
hipError_t launch_scatter(int dtype, const void *rows, int64_t T, int D, const int32_t *dst_row,
                          void *seq, hipStream_t s);
hipError_t launch_merge(int dtype, const void *x, const RowDesc *desc, int64_t T, int C, int k,
                        void *merged, hipStream_t s);
// Tile-blocked operand layout of the bf16 GEMMs: a [R][K] bf16 matrix is kept
// as [ceil(R/256)][K/32][256][32], i.e. element (r, c) at
// ((r/256 * K/32 + c/32) * 256 + r%256) * 32 + c%32, so the 256 rows of one
// 32-wide K slice of a row block are one contiguous 16 KiB run.  Rows past R
// are zero (weights) or unused (the hidden activation).
inline int64_t blocked_elems(int64_t R, int64_t K) { return (R + 255) / 256 * 256 * K; }
// Packs w [R][K] into the blocked layout.  With k > 1 (W1) the K axis is also
// reordered position-major: packed column j = p*C + c takes w[r][c*k*k + p].
hipError_t launch_pack(const void *w, int64_t R, int64_t K, int C, int k, void *packed,
                       hipStream_t s);
// Space-to-depth of the (bf16) patch grid into the blocked [T][C*k*k] operand
// of Linear1 for the token rows of one chunk of views, K position-major, zeros
// for cells past the grid; LayerNorm over C applied on the way when gamma is
// non-null (C <= layernorm_max_channels).
// With scan non-null, the launch also runs that placeholder scan (workgroup 0).
hipError_t launch_merge_blocked(const void *x, const PlanChunk &c, int C, const void *gamma,
                                const void *beta, float eps, void *out, hipStream_t s,
                                const ScanJob *scan = nullptr);

// bf16 MFMA GEMMs on blocked operands (K a multiple of 32), epilogue by mode
// (GemmMode).  A null bias counts as zero.
hipError_t launch_gemm_bf16(int mode, GemmArgs g, hipStream_t s);
// fp32 GEMMs (FMA).  In gather mode K follows the pages' order c*k*k + p and B
// is the unpacked W1.
hipError_t launch_gemm_f32(bool gather, GemmArgs g, hipStream_t s);

// ---- projector backward (bf16; see vlb_backward.hip) ------------------------
// T: token rows; Tk = T rounded up to 32 (the K extent of every contraction
// over tokens); Op = out_dim rounded up to 32.  Tile-blocked operands as above.
constexpr int kBwdMaxChannels = 2048;  // the LayerNorm backward keeps a pixel in registers
constexpr int kBwdUnmergeGrid = 768;   // most workgroups of one unmerge launch (3 per CU)
int bwd_unmerge_grid(int64_t items);   // workgroups for items (token row, position) pairs
// dY rows gathered from G [S][O] at dst_row (zero where negative) -> dY [T][Op],
// dY^T [O][Tk], part [Tk/32][O] (column sums per 32-row slice).
hipError_t launch_bwd_gather_dy(const void *G, const int32_t *dst_row, int32_t T, int32_t O,
                                int32_t Op, int32_t Tk, void *dy, void *dyt, float *part,
                                hipStream_t s);
// Merged tokens Xm [T][C*k*k] (K position-major) -> Xm^T [C*k*k][Tk], rows in
// the pages' feature order.
hipError_t launch_bwd_xm_t(const void *xm, int32_t T, int32_t C, int32_t k, int32_t Tk, void *xmt,
                           hipStream_t s);
// dZ1 = dA1 * act'(Z1) -> dZ1 [T][H], dZ1^T [H][Tk], part [Tk/32][H].
hipError_t launch_bwd_dact(int act, const void *da1, const void *z1, int32_t T, int32_t H,
                           int32_t Tk, void *dz1, void *dz1t, float *part, hipStream_t s);
// Feature gradient of one chunk of views from dXm (row-major [T][C*k*k], K
// position-major) through the LayerNorm (gamma non-null) or not; grid rows of
// part_g / part_b ([grid][C]) take the per-workgroup dgamma / dbeta sums.
hipError_t launch_bwd_unmerge(const void *dxm, const void *x, const PlanChunk &c, int C,
                              const void *gamma, float eps, void *dx, float *part_g,
                              float *part_b, const int32_t *status, int grid, hipStream_t s);
// out[n] = sum_r part[r][n], rows in order; nothing when status[0] != 0.
hipError_t launch_colsum(const float *part, int32_t R, int32_t N, float *out,
                         const int32_t *status, hipStream_t s);
// part[ceil(n/64)][O]: sums of G rows pos[i] (negative: none), 64 entries per row.
hipError_t launch_rows_sum(int dtype, const void *G, const int32_t *pos, int32_t n, int32_t O,
                           float *part, hipStream_t s);
// fp32: dY[t] = G[dst_row[t]] (zero where negative), row-major [T][O].
hipError_t launch_gather_rows_f32(const void *G, const int32_t *dst_row, int32_t T, int32_t O,
                                  void *dy, hipStream_t s);
// fp32: a = act(z) when da is null, else da *= act'(z) in place (n elements).
hipError_t launch_act_f32(int act, const void *z, int64_t n, void *a, void *da, hipStream_t s);
// fp32 feature gradient of one chunk of views from dXm (row-major [T][C*k*k],
// the pages' feature order), as launch_bwd_unmerge (C <= 2048).
hipError_t launch_bwd_unmerge_f32(const void *dxm, const void *x, const PlanChunk &c, int C,
                                  const void *gamma, float eps, void *dx, float *part_g,
                                  float *part_b, const int32_t *status, int grid, hipStream_t s);

}  // namespace vlb

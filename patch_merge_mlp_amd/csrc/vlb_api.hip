// Host side of the vlbridge C ABI: argument validation, the batch planner
// (token rows, assembled slots, workspace carving) and kernel launches.
//
// Sizes follow mlxcel issue #533 "port DeepSeek-VL2": section "Projector
// (downsample_mlp_gelu)" (N' = (g_pad/k)^2 tokens per view, g_pad the next
// multiple of k) and section "Processor" step 7 (h'(w'+1) + 1 + (th h')(tw w'+1)
// placeholder slots per tiled image).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "vlbridge.h"
#include "vlb_internal.h"

namespace {

using vlb::PlaceChunk;
using vlb::PlanChunk;
using vlb::RowDesc;

constexpr int64_t kI32Max = 2147483647;

struct Plan {
  int64_t T = 0, P = 0, npix = 0, K1 = 0;
  int es = 2;                          // element size in bytes
  std::vector<int32_t> view_tok0;      // [n_views + 1]
  std::vector<int32_t> view_pix0;      // [n_views]
  std::vector<int32_t> img_slot0;      // [n_images + 1]
  std::vector<int32_t> img_row0;       // [n_images]
  std::vector<int32_t> img_view0;      // [n_images]
  // workspace carving (bytes)
  size_t off_status = 0, off_dst = 0, off_desc = 0, off_xn = 0, off_h = 0, off_w1p = 0,
         off_w2p = 0, off_slot = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

vlb_status check_projector(const vlb_projector *p) {
  if (!p) return VLB_ERR_NULL;
  if (p->dtype != VLB_F32 && p->dtype != VLB_BF16) return VLB_ERR_DTYPE;
  if (p->k < 1 || p->k > 3) return VLB_ERR_UNSUPPORTED;
  if (p->C <= 0 || p->hidden <= 0 || p->out_dim <= 0) return VLB_ERR_SHAPE;
  if (p->C % 8 || p->hidden % 8 || p->out_dim % 8) return VLB_ERR_UNSUPPORTED;
  if (p->dtype == VLB_BF16 && (p->C % 64 || p->hidden % 64)) return VLB_ERR_UNSUPPORTED;
  if (p->act < VLB_GELU_ERF || p->act > VLB_ACT_NONE) return VLB_ERR_UNSUPPORTED;
  if (p->has_ln != 0 && p->has_ln != 1) return VLB_ERR_UNSUPPORTED;
  if (p->has_ln && !(p->ln_eps > 0.f)) return VLB_ERR_SHAPE;
  // LayerNorm holds a pixel in registers; the bf16 merge stages 16 of them in LDS
  if ((p->has_ln || p->dtype == VLB_BF16) && p->C > vlb::layernorm_max_channels(p->dtype))
    return VLB_ERR_UNSUPPORTED;
  if (p->packed && p->dtype != VLB_BF16) return VLB_ERR_UNSUPPORTED;
  const int64_t K1 = static_cast<int64_t>(p->C) * p->k * p->k;
  // 32-bit byte offsets address the weights (bf16: padded and tile-blocked)
  const int64_t es = p->dtype == VLB_BF16 ? 2 : 4;
  if (vlb::blocked_elems(p->hidden, K1) * es > kI32Max ||
      vlb::blocked_elems(p->out_dim, p->hidden) * es > kI32Max)
    return VLB_ERR_SHAPE;
  return VLB_OK;
}

// Validates the batch and fills the planner tables and workspace offsets.
vlb_status make_plan(const vlb_projector *p, const vlb_batch *b, int64_t seq_len, Plan *pl) {
  vlb_status st = check_projector(p);
  if (st != VLB_OK) return st;
  if (!b) return VLB_ERR_NULL;
  if (b->n_views < 0 || b->n_images < 0 || seq_len < 0) return VLB_ERR_SHAPE;
  if (b->layout != VLB_LAYOUT_PLAIN && b->layout != VLB_LAYOUT_TILED_2D)
    return VLB_ERR_UNSUPPORTED;
  if (b->n_views > 0 && (!b->grid_h || !b->grid_w)) return VLB_ERR_NULL;
  if (b->n_images > 0 && !b->views_per_image) return VLB_ERR_NULL;
  const bool tiled = b->layout == VLB_LAYOUT_TILED_2D;
  if (tiled && b->n_images > 0 && (!b->tile_w || !b->tile_h)) return VLB_ERR_NULL;
  if (tiled && b->global_view_tail != 0 && b->global_view_tail != 1) return VLB_ERR_UNSUPPORTED;
  const int k = p->k;
  pl->es = p->dtype == VLB_BF16 ? 2 : 4;
  pl->K1 = static_cast<int64_t>(p->C) * k * k;
  pl->view_tok0.assign(b->n_views + 1, 0);
  pl->view_pix0.assign(b->n_views, 0);
  int64_t tok = 0, pix = 0;
  for (int v = 0; v < b->n_views; ++v) {
    const int gh = b->grid_h[v], gw = b->grid_w[v];
    if (gh < 1 || gw < 1 || gh > 32767 || gw > 32767) return VLB_ERR_SHAPE;
    pl->view_tok0[v] = static_cast<int32_t>(tok);
    pl->view_pix0[v] = static_cast<int32_t>(pix);
    tok += ceil_div(gh, k) * ceil_div(gw, k);
    pix += static_cast<int64_t>(gh) * gw;
    if (tok > kI32Max || pix * p->C > kI32Max) return VLB_ERR_SHAPE;
  }
  pl->view_tok0[b->n_views] = static_cast<int32_t>(tok);
  pl->T = tok;
  pl->npix = pix;
  pl->img_slot0.assign(b->n_images + 1, 0);
  pl->img_row0.assign(b->n_images, 0);
  pl->img_view0.assign(b->n_images, 0);
  int64_t slot = 0;
  int v = 0;
  for (int im = 0; im < b->n_images; ++im) {
    const int nv = b->views_per_image[im];
    if (nv < 1 || v + nv > b->n_views) return VLB_ERR_SHAPE;
    pl->img_slot0[im] = static_cast<int32_t>(slot);
    pl->img_row0[im] = pl->view_tok0[v];
    pl->img_view0[im] = v;
    if (tiled) {
      const int tw = b->tile_w[im], th = b->tile_h[im];
      if (tw < 1 || th < 1 || static_cast<int64_t>(tw) * th + 1 != nv) return VLB_ERR_SHAPE;
      for (int q = 1; q < nv; ++q)
        if (b->grid_h[v + q] != b->grid_h[v] || b->grid_w[v + q] != b->grid_w[v])
          return VLB_ERR_SHAPE;
      const int64_t hp = ceil_div(b->grid_h[v], k), wp = ceil_div(b->grid_w[v], k);
      if (hp * th > 32767 || wp * tw > 32767) return VLB_ERR_SHAPE;
      slot += hp * (wp + 1) + 1 + (th * hp) * (tw * wp + 1);
    } else {
      slot += pl->view_tok0[v + nv] - pl->view_tok0[v];
    }
    if (slot > kI32Max) return VLB_ERR_SHAPE;
    v += nv;
  }
  if (v != b->n_views) return VLB_ERR_SHAPE;
  pl->img_slot0[b->n_images] = static_cast<int32_t>(slot);
  pl->P = slot;
  if (pl->T * std::max<int64_t>(p->hidden, p->out_dim) > kI32Max) return VLB_ERR_SHAPE;
  if (seq_len * p->out_dim > kI32Max) return VLB_ERR_SHAPE;
  // The GEMMs address their operands with 32-bit byte offsets (buffer loads).
  if (pl->npix * p->C * pl->es > kI32Max || vlb::blocked_elems(pl->T, p->hidden) * pl->es > kI32Max ||
      vlb::blocked_elems(pl->T, pl->K1) * pl->es > kI32Max)
    return VLB_ERR_SHAPE;

  size_t off = 0;
  pl->off_status = off;
  off = align256(off + 16);
  pl->off_dst = off;
  off = align256(off + static_cast<size_t>(pl->T) * 4);
  pl->off_desc = off;
  off = align256(off + static_cast<size_t>(pl->T) * sizeof(RowDesc));
  pl->off_xn = off;  // bf16: merged tokens, tile-blocked; fp32: the normalised grid
  if (p->dtype == VLB_BF16)
    off = align256(off + static_cast<size_t>(vlb::blocked_elems(pl->T, pl->K1)) * 2);
  else if (p->has_ln)
    off = align256(off + static_cast<size_t>(pl->npix) * p->C * pl->es);
  pl->off_h = off;  // hidden activation: tile-blocked (bf16) or row-major (fp32)
  if (p->dtype == VLB_BF16)
    off = align256(off + static_cast<size_t>(vlb::blocked_elems(pl->T, p->hidden)) * pl->es);
  else
    off = align256(off + static_cast<size_t>(pl->T) * p->hidden * pl->es);
  pl->off_w1p = off;  // weights packed per call when they are not pre-packed
  if (p->dtype == VLB_BF16 && !p->packed) {
    off = align256(off + static_cast<size_t>(vlb::blocked_elems(p->hidden, pl->K1)) * 2);
    pl->off_w2p = off;
    off = align256(off + static_cast<size_t>(vlb::blocked_elems(p->out_dim, p->hidden)) * 2);
  }
  pl->off_slot = off;
  off = align256(off + static_cast<size_t>(seq_len) * 4);
  pl->total = off;
  return VLB_OK;
}

// ---- optional per-kernel timing ---------------------------------------------
struct ProfRec {
  int kid;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
uint32_t g_prof_mask = 0;  // bit kid: time kernel id kid
std::vector<ProfRec> g_prof;
size_t g_prof_used = 0;

int prof_begin(int kid, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!((g_prof_mask >> kid) & 1u)) return -1;
  if (g_prof_used == g_prof.size()) {
    ProfRec r{kid, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return -1;
    g_prof.push_back(r);
  }
  ProfRec &r = g_prof[g_prof_used];
  r.kid = kid;
  if (hipEventRecord(r.a, s) != hipSuccess) return -1;
  return static_cast<int>(g_prof_used++);
}

void prof_end(int idx, hipStream_t s) {
  if (idx < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  (void)hipEventRecord(g_prof[idx].b, s);
}

#define VLB_LAUNCH(kid, stream, expr)                 \
  do {                                                \
    const int _pi = prof_begin((kid), (stream));      \
    const hipError_t _e = (expr);                     \
    prof_end(_pi, (stream));                          \
    if (_e != hipSuccess) return VLB_ERR_HIP;         \
  } while (0)

// The planner table of views [v0, v0 + kPlanViews) (clipped to the batch).
PlanChunk view_chunk(const vlb_projector *p, const vlb_batch *b, const Plan &pl, int v0) {
  PlanChunk c{};
  c.n = std::min(vlb::kPlanViews, b->n_views - v0);
  c.k = p->k;
  for (int i = 0; i < c.n; ++i) {
    c.tok0[i] = pl.view_tok0[v0 + i];
    c.pix0[i] = pl.view_pix0[v0 + i];
    c.gh[i] = static_cast<int16_t>(b->grid_h[v0 + i]);
    c.gw[i] = static_cast<int16_t>(b->grid_w[v0 + i]);
  }
  c.tok0[c.n] = pl.view_tok0[v0 + c.n];
  return c;
}

// Per-token gather descriptors, one launch per kPlanViews views.
vlb_status run_plan(const vlb_projector *p, const vlb_batch *b, const Plan &pl, RowDesc *desc,
                    hipStream_t s) {
  for (int v0 = 0; v0 < b->n_views; v0 += vlb::kPlanViews)
    VLB_LAUNCH(VLB_K_PLAN, s, vlb::launch_plan(view_chunk(p, b, pl, v0), desc, s));
  return VLB_OK;
}

// LN (optional) + both GEMMs.  dst_row == nullptr: rows[m] = projected row m;
// otherwise row m goes to out + dst_row[m] * out_dim.
vlb_status run_project(const vlb_projector *p, const vlb_batch *b, const Plan &pl,
                       const void *features, const vlb_weights *w, void *out,
                       const int32_t *dst_row, uint8_t *ws, hipStream_t s) {
  RowDesc *desc = reinterpret_cast<RowDesc *>(ws + pl.off_desc);
  const void *x = features;
  if (p->dtype == VLB_BF16) {  // LN (optional) + merge into Linear1's blocked operand
    void *xm = ws + pl.off_xn;
    for (int v0 = 0; v0 < b->n_views; v0 += vlb::kPlanViews)
      VLB_LAUNCH(p->has_ln ? VLB_K_LN : VLB_K_MERGE, s,
                 vlb::launch_merge_blocked(features, view_chunk(p, b, pl, v0), p->C,
                                           p->has_ln ? w->ln_gamma : nullptr,
                                           p->has_ln ? w->ln_beta : nullptr, p->ln_eps, xm, s));
    x = xm;
  } else {
    vlb_status st = run_plan(p, b, pl, desc, s);
    if (st != VLB_OK) return st;
    if (p->has_ln) {
      void *xn = ws + pl.off_xn;
      VLB_LAUNCH(VLB_K_LN, s,
                 vlb::launch_layernorm(p->dtype, features, pl.npix, p->C, w->ln_gamma,
                                       w->ln_beta, p->ln_eps, xn, s));
      x = xn;
    }
  }
  void *hbuf = ws + pl.off_h;
  vlb::GemmArgs g1{};
  g1.A = x;
  g1.desc = desc;
  g1.bias = w->b1;
  g1.out = hbuf;
  g1.dst_row = nullptr;
  g1.M = static_cast<int32_t>(pl.T);
  g1.N = p->hidden;
  g1.K = static_cast<int32_t>(pl.K1);
  g1.ldo = p->hidden;
  g1.C = p->C;
  g1.k = p->k;
  g1.act = p->act;
  g1.a_bytes = static_cast<uint32_t>(pl.npix * p->C * pl.es);
  g1.b_bytes = static_cast<uint32_t>(pl.K1 * p->hidden * pl.es);
  vlb::GemmArgs g2{};
  g2.A = hbuf;
  g2.B = w->w2;
  g2.bias = w->b2;
  g2.out = out;
  g2.dst_row = dst_row;
  g2.M = static_cast<int32_t>(pl.T);
  g2.N = p->out_dim;
  g2.K = p->hidden;
  g2.ldo = p->out_dim;
  g2.act = VLB_ACT_NONE;
  g2.a_bytes = static_cast<uint32_t>(pl.T * p->hidden * pl.es);
  g2.b_bytes = static_cast<uint32_t>(static_cast<int64_t>(p->out_dim) * p->hidden * pl.es);
  if (p->dtype == VLB_BF16) {
    const void *w1p = w->w1, *w2p = w->w2;
    if (!p->packed) {
      VLB_LAUNCH(VLB_K_PACK, s,
                 vlb::launch_pack(w->w1, p->hidden, pl.K1, p->C, p->k, ws + pl.off_w1p, s));
      VLB_LAUNCH(VLB_K_PACK, s,
                 vlb::launch_pack(w->w2, p->out_dim, p->hidden, p->C, 1, ws + pl.off_w2p, s));
      w1p = ws + pl.off_w1p;
      w2p = ws + pl.off_w2p;
    }
    g1.B = w1p;
    g1.b_bytes = static_cast<uint32_t>(vlb::blocked_elems(p->hidden, pl.K1) * 2);
    g2.B = w2p;
    g2.b_bytes = static_cast<uint32_t>(vlb::blocked_elems(p->out_dim, p->hidden) * 2);
    g1.a_bytes = static_cast<uint32_t>(vlb::blocked_elems(pl.T, pl.K1) * 2);
    g2.a_bytes = static_cast<uint32_t>(vlb::blocked_elems(pl.T, p->hidden) * 2);
    VLB_LAUNCH(VLB_K_GEMM1, s, vlb::launch_gemm_bf16(true, g1, s));
    VLB_LAUNCH(VLB_K_GEMM2, s, vlb::launch_gemm_bf16(false, g2, s));
  } else {
    g1.B = w->w1;
    VLB_LAUNCH(VLB_K_GEMM1, s, vlb::launch_gemm_f32(true, g1, s));
    VLB_LAUNCH(VLB_K_GEMM2, s, vlb::launch_gemm_f32(false, g2, s));
  }
  return VLB_OK;
}

// Prefix sum of the mask and the assembly map -> dst_row; newline / separator
// rows are written to their slots here.
// Where the placeholders are: a uint8 mask, or token ids equal to image_id
// (the other ids must lie in [0, vocab)).
struct PlaceSrc {
  const uint8_t *mask;
  const int32_t *ids;
  int32_t image_id;
  int64_t vocab;
};

vlb_status run_place(const vlb_projector *p, const vlb_batch *b, const Plan &pl,
                     const void *newline, const void *separator, const PlaceSrc &src,
                     int64_t seq_len, void *seq, uint8_t *ws, hipStream_t s) {
  int32_t *status = reinterpret_cast<int32_t *>(ws + pl.off_status);
  int32_t *slot_pos = reinterpret_cast<int32_t *>(ws + pl.off_slot);
  int32_t *dst_row = reinterpret_cast<int32_t *>(ws + pl.off_dst);
  if (b->layout == VLB_LAYOUT_PLAIN) {  // token row r -> the r-th placeholder: the scan writes dst_row
    VLB_LAUNCH(VLB_K_SCAN, s,
               vlb::launch_scan(src.mask, src.ids, src.image_id, src.vocab, seq_len, pl.P, dst_row,
                                status, true, s));
    return VLB_OK;
  }
  VLB_LAUNCH(VLB_K_SCAN, s,
             vlb::launch_scan(src.mask, src.ids, src.image_id, src.vocab, seq_len, pl.P, slot_pos,
                              status, false, s));
  for (int i0 = 0; i0 < b->n_images; i0 += vlb::kPlaceImages) {
    PlaceChunk c{};
    c.n = std::min(vlb::kPlaceImages, b->n_images - i0);
    c.tail = b->global_view_tail;
    for (int i = 0; i < c.n; ++i) {
      const int im = i0 + i, v = pl.img_view0[im];
      c.slot0[i] = pl.img_slot0[im];
      c.row0[i] = pl.img_row0[im];
      c.hp[i] = static_cast<int16_t>(ceil_div(b->grid_h[v], p->k));
      c.wp[i] = static_cast<int16_t>(ceil_div(b->grid_w[v], p->k));
      c.tw[i] = static_cast<int16_t>(b->tile_w[im]);
      c.th[i] = static_cast<int16_t>(b->tile_h[im]);
    }
    c.slot0[c.n] = pl.img_slot0[i0 + c.n];
    VLB_LAUNCH(VLB_K_PLACE, s,
               vlb::launch_place_tiled(p->dtype, c, slot_pos, status, dst_row, newline, separator,
                                       seq, p->out_dim, s));
  }
  return VLB_OK;
}

vlb_status check_weights(const vlb_projector *p, const vlb_weights *w) {
  if (!w) return VLB_ERR_NULL;
  if (!w->w1 || !w->b1 || !w->w2 || !w->b2) return VLB_ERR_NULL;
  if (p->has_ln && (!w->ln_gamma || !w->ln_beta)) return VLB_ERR_NULL;
  if (!aligned16(w->w1) || !aligned16(w->b1) || !aligned16(w->w2) || !aligned16(w->b2))
    return VLB_ERR_ALIGN;
  if (p->has_ln && (!aligned16(w->ln_gamma) || !aligned16(w->ln_beta))) return VLB_ERR_ALIGN;
  return VLB_OK;
}

vlb_status check_scatter_args(const vlb_projector *p, const vlb_batch *b, const void *newline,
                              const void *separator, const uint8_t *mask, int64_t seq_len,
                              const void *seq) {
  if (!mask || !seq) return VLB_ERR_NULL;
  if (!aligned16(mask) || !aligned16(seq)) return VLB_ERR_ALIGN;
  if (seq_len < 1) return VLB_ERR_SHAPE;
  if (b->layout == VLB_LAYOUT_TILED_2D) {
    if (!newline || !separator) return VLB_ERR_NULL;
    if (!aligned16(newline) || !aligned16(separator)) return VLB_ERR_ALIGN;
  }
  (void)p;
  return VLB_OK;
}

}  // namespace

extern "C" {

int64_t vlb_num_tokens(const vlb_projector *p, const vlb_batch *b) {
  Plan pl;
  const vlb_status st = make_plan(p, b, 0, &pl);
  return st == VLB_OK ? pl.T : -static_cast<int64_t>(st);
}

int64_t vlb_num_slots(const vlb_projector *p, const vlb_batch *b) {
  Plan pl;
  const vlb_status st = make_plan(p, b, 0, &pl);
  return st == VLB_OK ? pl.P : -static_cast<int64_t>(st);
}

int64_t vlb_image_slots(const vlb_projector *p, const vlb_batch *b, int64_t *out) {
  Plan pl;
  const vlb_status st = make_plan(p, b, 0, &pl);
  if (st != VLB_OK) return -static_cast<int64_t>(st);
  if (!out && b->n_images > 0) return -static_cast<int64_t>(VLB_ERR_NULL);
  for (int i = 0; i < b->n_images; ++i) out[i] = pl.img_slot0[i + 1] - pl.img_slot0[i];
  return pl.P;
}

size_t vlb_workspace_bytes(const vlb_projector *p, const vlb_batch *b, int64_t seq_len) {
  Plan pl;
  return make_plan(p, b, seq_len, &pl) == VLB_OK ? pl.total : 0;
}

size_t vlb_packed_bytes(const vlb_projector *p, int32_t which) {
  if (check_projector(p) != VLB_OK || p->dtype != VLB_BF16) return 0;
  const int64_t K1 = static_cast<int64_t>(p->C) * p->k * p->k;
  if (which == 1) return static_cast<size_t>(vlb::blocked_elems(p->hidden, K1)) * 2;
  if (which == 2) return static_cast<size_t>(vlb::blocked_elems(p->out_dim, p->hidden)) * 2;
  return 0;
}

vlb_status vlb_pack_weights(const vlb_projector *p, const void *w1, const void *w2,
                            void *w1_packed, void *w2_packed, void *stream) {
  vlb_status st = check_projector(p);
  if (st != VLB_OK) return st;
  if (p->dtype != VLB_BF16) return VLB_ERR_UNSUPPORTED;
  if (!w1 || !w2 || !w1_packed || !w2_packed) return VLB_ERR_NULL;
  if (!aligned16(w1) || !aligned16(w2) || !aligned16(w1_packed) || !aligned16(w2_packed))
    return VLB_ERR_ALIGN;
  const int64_t K1 = static_cast<int64_t>(p->C) * p->k * p->k;
  auto overlap = [](const void *a, size_t na, const void *b, size_t nb) {
    const uint8_t *x = static_cast<const uint8_t *>(a), *y = static_cast<const uint8_t *>(b);
    return x < y + nb && y < x + na;
  };
  const size_t n1 = static_cast<size_t>(p->hidden) * K1 * 2, n2 = static_cast<size_t>(p->out_dim) * p->hidden * 2;
  const size_t m1 = vlb_packed_bytes(p, 1), m2 = vlb_packed_bytes(p, 2);
  if (overlap(w1_packed, m1, w1, n1) || overlap(w1_packed, m1, w2, n2) ||
      overlap(w2_packed, m2, w1, n1) || overlap(w2_packed, m2, w2, n2) ||
      overlap(w1_packed, m1, w2_packed, m2))
    return VLB_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  VLB_LAUNCH(VLB_K_PACK, s, vlb::launch_pack(w1, p->hidden, K1, p->C, p->k, w1_packed, s));
  VLB_LAUNCH(VLB_K_PACK, s, vlb::launch_pack(w2, p->out_dim, p->hidden, p->C, 1, w2_packed, s));
  return VLB_OK;
}

vlb_status vlb_merge_tokens(const vlb_projector *p, const vlb_batch *b, const void *features,
                            const void *ln_gamma, const void *ln_beta, void *merged, void *ws,
                            size_t ws_bytes, void *stream) {
  Plan pl;
  vlb_status st = make_plan(p, b, 0, &pl);
  if (st != VLB_OK) return st;
  if (pl.T == 0) return VLB_OK;
  if (!features || !merged || !ws) return VLB_ERR_NULL;
  if (p->has_ln && (!ln_gamma || !ln_beta)) return VLB_ERR_NULL;
  if (!aligned16(features) || !aligned16(merged) || !aligned16(ws)) return VLB_ERR_ALIGN;
  if (p->has_ln && (!aligned16(ln_gamma) || !aligned16(ln_beta))) return VLB_ERR_ALIGN;
  if (ws_bytes < pl.total) return VLB_ERR_WORKSPACE;
  if (pl.K1 * pl.es > 65536) return VLB_ERR_UNSUPPORTED;  // one token's pixels staged in LDS
  if (pl.T * pl.K1 > kI32Max) return VLB_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  RowDesc *desc = reinterpret_cast<RowDesc *>(w8 + pl.off_desc);
  st = run_plan(p, b, pl, desc, s);
  if (st != VLB_OK) return st;
  const void *x = features;
  if (p->has_ln) {
    VLB_LAUNCH(VLB_K_LN, s,
               vlb::launch_layernorm(p->dtype, features, pl.npix, p->C, ln_gamma, ln_beta,
                                     p->ln_eps, w8 + pl.off_xn, s));
    x = w8 + pl.off_xn;
  }
  VLB_LAUNCH(VLB_K_MERGE, s, vlb::launch_merge(p->dtype, x, desc, pl.T, p->C, p->k, merged, s));
  return VLB_OK;
}

vlb_status vlb_merge_project(const vlb_projector *p, const vlb_batch *b, const void *features,
                             const vlb_weights *w, void *rows, void *ws, size_t ws_bytes,
                             void *stream) {
  Plan pl;
  vlb_status st = make_plan(p, b, 0, &pl);
  if (st != VLB_OK) return st;
  if (pl.T == 0) return VLB_OK;
  if ((st = check_weights(p, w)) != VLB_OK) return st;
  if (!features || !rows || !ws) return VLB_ERR_NULL;
  if (!aligned16(features) || !aligned16(rows) || !aligned16(ws)) return VLB_ERR_ALIGN;
  if (ws_bytes < pl.total) return VLB_ERR_WORKSPACE;
  return run_project(p, b, pl, features, w, rows, nullptr, static_cast<uint8_t *>(ws),
                     static_cast<hipStream_t>(stream));
}

vlb_status vlb_scatter_tokens(const vlb_projector *p, const vlb_batch *b, const void *rows,
                              const void *newline, const void *separator, const uint8_t *mask,
                              int64_t seq_len, void *seq, void *ws, size_t ws_bytes,
                              void *stream) {
  Plan pl;
  vlb_status st = make_plan(p, b, seq_len, &pl);
  if (st != VLB_OK) return st;
  if (pl.T == 0) return VLB_OK;
  if ((st = check_scatter_args(p, b, newline, separator, mask, seq_len, seq)) != VLB_OK) return st;
  if (!rows || !ws) return VLB_ERR_NULL;
  if (!aligned16(rows) || !aligned16(ws)) return VLB_ERR_ALIGN;
  if (ws_bytes < pl.total) return VLB_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  st = run_place(p, b, pl, newline, separator, PlaceSrc{mask, nullptr, 0, 0}, seq_len, seq, w8, s);
  if (st != VLB_OK) return st;
  VLB_LAUNCH(VLB_K_SCATTER, s,
             vlb::launch_scatter(p->dtype, rows, pl.T, p->out_dim,
                                 reinterpret_cast<const int32_t *>(w8 + pl.off_dst), seq, s));
  return VLB_OK;
}

vlb_status vlb_bridge_fused(const vlb_projector *p, const vlb_batch *b, const void *features,
                            const vlb_weights *w, const void *newline, const void *separator,
                            const uint8_t *mask, int64_t seq_len, void *seq, void *ws,
                            size_t ws_bytes, void *stream) {
  Plan pl;
  vlb_status st = make_plan(p, b, seq_len, &pl);
  if (st != VLB_OK) return st;
  if (pl.T == 0) return VLB_OK;
  if ((st = check_weights(p, w)) != VLB_OK) return st;
  if ((st = check_scatter_args(p, b, newline, separator, mask, seq_len, seq)) != VLB_OK) return st;
  if (!features || !ws) return VLB_ERR_NULL;
  if (!aligned16(features) || !aligned16(ws)) return VLB_ERR_ALIGN;
  if (ws_bytes < pl.total) return VLB_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  st = run_place(p, b, pl, newline, separator, PlaceSrc{mask, nullptr, 0, 0}, seq_len, seq, w8, s);
  if (st != VLB_OK) return st;
  return run_project(p, b, pl, features, w, seq,
                     reinterpret_cast<const int32_t *>(w8 + pl.off_dst), w8, s);
}

vlb_status vlb_bridge_embed(const vlb_projector *p, const vlb_batch *b, const void *features,
                            const vlb_weights *w, const void *newline, const void *separator,
                            const int32_t *ids, int32_t image_token_id, const void *embed,
                            int64_t vocab, int64_t seq_len, void *seq, void *ws, size_t ws_bytes,
                            void *stream) {
  Plan pl;
  vlb_status st = make_plan(p, b, seq_len, &pl);
  if (st != VLB_OK) return st;
  if (!ids || !embed || !seq || !ws) return VLB_ERR_NULL;
  if (!aligned16(ids) || !aligned16(embed) || !aligned16(seq) || !aligned16(ws))
    return VLB_ERR_ALIGN;
  if (seq_len < 1 || vocab < 1 || vocab > kI32Max) return VLB_ERR_SHAPE;
  if (pl.T > 0) {
    if ((st = check_weights(p, w)) != VLB_OK) return st;
    if (!features) return VLB_ERR_NULL;
    if (!aligned16(features)) return VLB_ERR_ALIGN;
    if (b->layout == VLB_LAYOUT_TILED_2D) {
      if (!newline || !separator) return VLB_ERR_NULL;
      if (!aligned16(newline) || !aligned16(separator)) return VLB_ERR_ALIGN;
    }
  }
  if (ws_bytes < pl.total) return VLB_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  st = run_place(p, b, pl, newline, separator, PlaceSrc{nullptr, ids, image_token_id, vocab},
                 seq_len, seq, w8, s);
  if (st != VLB_OK) return st;
  VLB_LAUNCH(VLB_K_EMBED, s,
             vlb::launch_embed_rows(p->dtype, ids, seq_len, image_token_id, embed, p->out_dim,
                                    reinterpret_cast<const int32_t *>(w8 + pl.off_status), seq, s));
  if (pl.T == 0) return VLB_OK;
  return run_project(p, b, pl, features, w, seq,
                     reinterpret_cast<const int32_t *>(w8 + pl.off_dst), w8, s);
}

vlb_status vlb_check(void *ws, void *stream) {
  if (!ws) return VLB_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return VLB_ERR_HIP;
  int32_t word[2] = {0, 0};
  if (hipMemcpy(word, ws, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return VLB_ERR_HIP;
  return word[0] == 0 ? VLB_OK : static_cast<vlb_status>(word[0]);
}

const char *vlb_status_str(vlb_status s) {
  switch (s) {
    case VLB_OK: return "ok";
    case VLB_ERR_NULL: return "null pointer";
    case VLB_ERR_SHAPE: return "invalid shape";
    case VLB_ERR_DTYPE: return "invalid dtype";
    case VLB_ERR_ALIGN: return "pointer not 16-byte aligned";
    case VLB_ERR_WORKSPACE: return "workspace too small";
    case VLB_ERR_MASK_COUNT: return "placeholder count differs from assembled slots";
    case VLB_ERR_UNSUPPORTED: return "unsupported setting";
    case VLB_ERR_HIP: return "HIP runtime error";
    case VLB_ERR_TOKEN_ID: return "text token id outside the vocabulary";
  }
  return "unknown status";
}

vlb_status vlb_prof_enable(int32_t mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = static_cast<uint32_t>(mask);
  if (g_prof_mask) g_prof_used = 0;
  return VLB_OK;
}

vlb_status vlb_prof_read(int32_t kid, int64_t *launches, double *total_ms) {
  if (!launches || !total_ms) return VLB_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int64_t n = 0;
  double ms = 0.0;
  for (size_t i = 0; i < g_prof_used; ++i) {
    if (g_prof[i].kid != kid) continue;
    if (hipEventSynchronize(g_prof[i].b) != hipSuccess) return VLB_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_prof[i].a, g_prof[i].b) != hipSuccess) return VLB_ERR_HIP;
    ++n;
    ms += t;
  }
  *launches = n;
  *total_ms = ms;
  return VLB_OK;
}

}  // extern "C"

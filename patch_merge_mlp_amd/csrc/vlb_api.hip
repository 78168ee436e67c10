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
  size_t off_status = 0, off_dst = 0, off_desc = 0, off_xn = 0, off_h = 0, off_h2 = 0,
         off_w1p = 0, off_w2p = 0, off_wmp = 0, off_slot = 0, off_text = 0, total = 0;
};

constexpr int kMaxDepth = 16;

// Linears in the projector (the depth field; 0 means the pages' default 2).
int proj_depth(const vlb_projector *p) { return p->depth == 0 ? 2 : p->depth; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Linear1 reads the merged tokens straight from the grid (vlb_projector.gather).
// Gathered operand loads slow Linear1 by 8-11% (16 separate 64-byte pieces per
// load instruction instead of one contiguous KiB), which grows with its
// hidden width, while the merge pass it saves moves a fixed T * C * k * k * 4
// bytes.  Measured: hidden 2560 (the tiled 2x2 workload) runs 3% faster per
// call with the gather, hidden 5120 (both 3x3 workloads) from 1% faster to
// 1.7% slower, depending on the run; the automatic choice takes the gather up
// to hidden 4096.
constexpr int kGatherMaxHidden = 4096;
bool gathers(const vlb_projector *p) {
  if (p->dtype != VLB_BF16 || p->has_ln || p->gather == VLB_GATHER_OFF) return false;
  return p->gather == VLB_GATHER_ON || p->hidden <= kGatherMaxHidden;
}

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
  if (p->gather < VLB_GATHER_AUTO || p->gather > VLB_GATHER_OFF) return VLB_ERR_UNSUPPORTED;
  if (p->gather == VLB_GATHER_ON && (p->dtype != VLB_BF16 || p->has_ln))
    return VLB_ERR_UNSUPPORTED;
  if (p->depth < 0 || p->depth == 1) return VLB_ERR_SHAPE;
  if (p->depth > kMaxDepth) return VLB_ERR_UNSUPPORTED;
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
  // bf16: the (normalised) merged tokens, tile-blocked -- not kept when
  // Linear1 gathers its operand from the grid; fp32: the normalised grid
  pl->off_xn = off;
  if (p->dtype == VLB_BF16 && !gathers(p))
    off = align256(off + static_cast<size_t>(vlb::blocked_elems(pl->T, pl->K1)) * 2);
  else if (p->has_ln)
    off = align256(off + static_cast<size_t>(pl->npix) * p->C * pl->es);
  // hidden activation: tile-blocked (bf16) or row-major (fp32); a second
  // buffer for the middle Linears (depth > 2) to alternate with
  const size_t hbytes = p->dtype == VLB_BF16
                            ? static_cast<size_t>(vlb::blocked_elems(pl->T, p->hidden)) * 2
                            : static_cast<size_t>(pl->T) * p->hidden * pl->es;
  pl->off_h = off;
  off = align256(off + hbytes);
  pl->off_h2 = off;
  if (proj_depth(p) > 2) off = align256(off + hbytes);
  pl->off_w1p = off;  // weights packed per call when they are not pre-packed
  if (p->dtype == VLB_BF16 && !p->packed) {
    off = align256(off + static_cast<size_t>(vlb::blocked_elems(p->hidden, pl->K1)) * 2);
    pl->off_w2p = off;
    off = align256(off + static_cast<size_t>(vlb::blocked_elems(p->out_dim, p->hidden)) * 2);
    pl->off_wmp = off;  // one middle weight at a time
    if (proj_depth(p) > 2)
      off = align256(off + static_cast<size_t>(vlb::blocked_elems(p->hidden, p->hidden)) * 2);
  }
  pl->off_slot = off;
  off = align256(off + static_cast<size_t>(seq_len) * 4);
  // the token-id form's text positions and ids (vlb_bridge_embed)
  pl->off_text = off;
  off = align256(off + static_cast<size_t>(seq_len) * 8);
  pl->total = off;
  return VLB_OK;
}

// Saved activations of a training forward: the merged tokens (Linear1's
// operand) and the pre-activation of Linear1 and of every middle Linear,
// tile-blocked (bf16) or row-major (fp32); bf16 keeps their activations as
// well (the next Linear's operand, written there instead of the workspace),
// which the weight gradients read token-major.
struct SavedLayout {
  size_t off_xm = 0, off_z1 = 0, off_a1 = 0, z_stride = 0, total = 0;
  // pre-activation of Linear1 (q = 0) or of middle Linear q (1 <= q <= depth - 2)
  size_t off_z(int q) const { return off_z1 + static_cast<size_t>(q) * z_stride; }
  // its activation (bf16)
  size_t off_a(int q) const { return off_a1 + static_cast<size_t>(q) * z_stride; }
};

SavedLayout saved_layout(const vlb_projector *p, const Plan &pl) {
  SavedLayout L;
  size_t off = 0;
  const int nz = proj_depth(p) - 1;  // pre-activations kept: Linear1 and the middle ones
  if (p->dtype == VLB_F32) {  // row-major merged rows (the pages' order) and Z per Linear
    L.off_xm = off;
    off = align256(off + static_cast<size_t>(pl.T) * pl.K1 * 4);
    L.off_z1 = off;
    L.z_stride = align256(static_cast<size_t>(pl.T) * p->hidden * 4);
    L.total = off + nz * L.z_stride;
    return L;
  }
  L.off_xm = off;
  off = align256(off + static_cast<size_t>(vlb::blocked_elems(pl.T, pl.K1)) * 2);
  L.off_z1 = off;
  L.z_stride = align256(static_cast<size_t>(vlb::blocked_elems(pl.T, p->hidden)) * 2);
  L.off_a1 = off + nz * L.z_stride;
  L.total = L.off_a1 + nz * L.z_stride;
  return L;
}

// Workspace of the backward (bf16).  Tk = T and Op = out_dim rounded up to 32.
struct BwdLayout {
  int64_t Tk = 0, Op = 0, NL = 0;  // NL: newline slots of the batch
  size_t off_status = 0, off_dst = 0, off_slot = 0, off_nl = 0, off_sep = 0, off_dy = 0,
         off_dyt = 0, off_a1t = 0, off_w1p = 0, off_w2p = 0, off_wmp = 0, off_da1 = 0,
         off_dz1 = 0, off_dz1t = 0, off_xmt = 0, off_dxm = 0, off_pb2 = 0, off_pb1 = 0, off_pln = 0,
         off_pnl = 0, off_psep = 0, off_split = 0, total = 0;
  size_t split_bytes = 0;    // K-split partial tiles of the weight gradients (0: none)
  std::vector<int> ln_grid;  // unmerge workgroups per chunk of views
  int64_t ln_rows = 0;       // their sum: rows of each LayerNorm partial
};

vlb_status bwd_layout(const vlb_projector *p, const vlb_batch *b, const Plan &pl,
                      int64_t seq_len, BwdLayout *L) {
  if (p->has_ln && p->C > vlb::kBwdMaxChannels) return VLB_ERR_UNSUPPORTED;
  const int64_t T = pl.T, H = p->hidden, O = p->out_dim, K1 = pl.K1;
  L->Tk = (T + 31) / 32 * 32;
  L->Op = (O + 31) / 32 * 32;
  L->NL = 0;
  if (b->layout == VLB_LAYOUT_TILED_2D)
    for (int im = 0; im < b->n_images; ++im) {
      const int v = pl.img_view0[im];
      L->NL += ceil_div(b->grid_h[v], p->k) * (1 + b->tile_h[im]);
    }
  // 32-bit byte extents of the bf16 GEMM operands
  const int64_t Tk = L->Tk, Op = L->Op;
  if (p->dtype == VLB_BF16)
    for (const int64_t e : {vlb::blocked_elems(T, Op), vlb::blocked_elems(O, Tk),
                            vlb::blocked_elems(H, Tk), vlb::blocked_elems(O, H),
                            vlb::blocked_elems(K1, Tk), vlb::blocked_elems(H, K1),
                            vlb::blocked_elems(T, H)})
      if (e * 2 > kI32Max) return VLB_ERR_SHAPE;
  L->ln_grid.clear();
  L->ln_rows = 0;
  for (int v0 = 0; v0 < b->n_views; v0 += vlb::kPlanViews) {
    const int v1 = std::min(b->n_views, v0 + vlb::kPlanViews);
    const int g = vlb::bwd_unmerge_grid(
        static_cast<int64_t>(pl.view_tok0[v1] - pl.view_tok0[v0]) * p->k * p->k);
    L->ln_grid.push_back(g);
    L->ln_rows += g;
  }
  auto take = [](size_t &off, size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  size_t off = 0;
  L->off_status = take(off, 16);
  L->off_dst = take(off, static_cast<size_t>(T) * 4);
  L->off_slot = take(off, static_cast<size_t>(seq_len) * 4);
  L->off_nl = take(off, static_cast<size_t>(L->NL) * 4);
  L->off_sep = take(off, static_cast<size_t>(b->n_images) * 4);
  if (p->dtype == VLB_F32) {  // row-major: dY [T][O], act(Z1) [T][H], dA1 / dZ1 [T][H], dXm [T][K1]
    L->off_dy = take(off, static_cast<size_t>(T) * O * 4);
    L->off_a1t = take(off, static_cast<size_t>(T) * H * 4);
    L->off_da1 = take(off, static_cast<size_t>(T) * H * 4);
    L->off_dxm = take(off, static_cast<size_t>(T) * K1 * 4);
    L->off_pln = take(off, static_cast<size_t>(2 * L->ln_rows) * p->C * 4);
    L->off_pnl = take(off, static_cast<size_t>(ceil_div(L->NL, 64)) * O * 4);
    L->off_psep = take(off, static_cast<size_t>(ceil_div(b->n_images, 64)) * O * 4);
    L->total = off;
    return VLB_OK;
  }
  L->off_dy = take(off, static_cast<size_t>(vlb::blocked_elems(T, Op)) * 2);
  L->off_dyt = take(off, static_cast<size_t>(vlb::blocked_elems(O, Tk)) * 2);
  L->off_da1 = take(off, static_cast<size_t>(vlb::blocked_elems(T, H)) * 2);
  L->off_dz1 = take(off, static_cast<size_t>(vlb::blocked_elems(T, H)) * 2);
  L->off_dz1t = take(off, static_cast<size_t>(vlb::blocked_elems(H, Tk)) * 2);
  L->off_xmt = take(off, static_cast<size_t>(vlb::blocked_elems(K1, Tk)) * 2);
  if (!p->packed) {  // weights passed unpacked: packed here (the products read them token-major)
    L->off_w1p = take(off, static_cast<size_t>(vlb::blocked_elems(H, K1)) * 2);
    L->off_w2p = take(off, static_cast<size_t>(vlb::blocked_elems(O, H)) * 2);
    if (proj_depth(p) > 2)  // one middle weight at a time
      L->off_wmp = take(off, static_cast<size_t>(vlb::blocked_elems(H, H)) * 2);
  }
  L->off_dxm = take(off, static_cast<size_t>(T) * K1 * 2);
  L->off_pb2 = take(off, static_cast<size_t>(Tk / 32) * O * 4);
  L->off_pb1 = take(off, static_cast<size_t>(Tk / 32) * H * 4);
  L->off_pln = take(off, static_cast<size_t>(2 * L->ln_rows) * p->C * 4);
  L->off_pnl = take(off, static_cast<size_t>(ceil_div(L->NL, 64)) * O * 4);
  L->off_psep = take(off, static_cast<size_t>(ceil_div(b->n_images, 64)) * O * 4);
  // partial tiles of the weight-gradient products' split K ranges
  L->split_bytes = std::max(vlb::gemm_split_bytes(O, H, Tk), vlb::gemm_split_bytes(H, K1, Tk));
  if (proj_depth(p) > 2) L->split_bytes = std::max(L->split_bytes, vlb::gemm_split_bytes(H, H, Tk));
  L->off_split = take(off, L->split_bytes);
  L->total = off;
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

// The tiled slot map (defined below), and what it needs when run_project
// launches it after the merge.
vlb_status run_place_tiled(const vlb_projector *p, const vlb_batch *b, const Plan &pl,
                           const void *newline, const void *separator, void *seq, uint8_t *ws,
                           hipStream_t s);
struct TiledPlace {
  const void *newline, *separator;
  void *seq;
};

// LN (optional) + merge + the Linears.  dst_row == nullptr: rows[m] =
// projected row m; otherwise row m goes to out + dst_row[m] * out_dim.
// saved (training forward, else null): the merged tokens and the
// pre-activation of every Linear but the last are kept there (saved_layout).
// scan (bf16 fused calls, else null): the placeholder scan, carried by the
// first merge launch.  place (tiled layout with scan, else null): the slot
// map, launched after the merge and before the Linears.
vlb_status run_project(const vlb_projector *p, const vlb_batch *b, const Plan &pl,
                       const void *features, const vlb_weights *w, void *out,
                       const int32_t *dst_row, uint8_t *ws, hipStream_t s,
                       uint8_t *saved = nullptr, const vlb::ScanJob *scan = nullptr,
                       const TiledPlace *place = nullptr) {
  RowDesc *desc = reinterpret_cast<RowDesc *>(ws + pl.off_desc);
  const void *x = features;
  const SavedLayout sl = saved ? saved_layout(p, pl) : SavedLayout{};
  vlb_status st;
  if (scan && (p->dtype != VLB_BF16 || b->n_views < 1)) {  // no merge launch to carry it
    VLB_LAUNCH(VLB_K_SCAN, s,
               vlb::launch_scan(scan->mask, scan->ids, scan->image_id, scan->vocab, scan->S,
                                scan->P, scan->slot_pos, scan->status, scan->direct, s, scan->text));
    scan = nullptr;
  }
  // Gather mode (the projector's gather flag; bf16 without LayerNorm, and no
  // merged tokens to keep): Linear1 reads its operand straight from the grid
  // through per-token descriptors, and the scan rides in the descriptor launch.
  const bool gather = gathers(p) && !saved;
  if (gather) {
    for (int v0 = 0; v0 < b->n_views; v0 += vlb::kPlanViews)
      VLB_LAUNCH(VLB_K_PLAN, s,
                 vlb::launch_plan(view_chunk(p, b, pl, v0), desc, s, v0 == 0 ? scan : nullptr));
  } else if (p->dtype == VLB_BF16) {  // LN (optional) + merge into Linear1's blocked operand
    void *xm = saved ? saved + sl.off_xm : ws + pl.off_xn;
    for (int v0 = 0; v0 < b->n_views; v0 += vlb::kPlanViews)
      VLB_LAUNCH(p->has_ln ? VLB_K_LN : VLB_K_MERGE, s,
                 vlb::launch_merge_blocked(features, view_chunk(p, b, pl, v0), p->C,
                                           p->has_ln ? w->ln_gamma : nullptr,
                                           p->has_ln ? w->ln_beta : nullptr, p->ln_eps, xm, s,
                                           v0 == 0 ? scan : nullptr));
    x = xm;
  } else {
    if ((st = run_plan(p, b, pl, desc, s)) != VLB_OK) return st;
    if (p->has_ln) {
      void *xn = ws + pl.off_xn;
      VLB_LAUNCH(VLB_K_LN, s,
                 vlb::launch_layernorm(p->dtype, features, pl.npix, p->C, w->ln_gamma,
                                       w->ln_beta, p->ln_eps, xn, s));
      x = xn;
    }
    if (saved)  // the training forward keeps the merged rows (Linear1 then reads them)
      VLB_LAUNCH(VLB_K_MERGE, s,
                 vlb::launch_merge(p->dtype, x, desc, pl.T, p->C, p->k, saved + sl.off_xm, s));
  }
  // Tiled: the slot map follows the merge that carried the scan (Linear2 is
  // the first reader of dst_row).
  if (place && (st = run_place_tiled(p, b, pl, place->newline, place->separator, place->seq, ws,
                                     s)) != VLB_OK)
    return st;
  // the hidden activation: the workspace, or the saved activation of Linear1
  // in a bf16 training forward
  void *hbuf = saved && p->dtype == VLB_BF16 ? saved + sl.off_a(0) : ws + pl.off_h;
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
    g1.a_bytes = gather ? static_cast<uint32_t>(pl.npix * p->C * 2)
                        : static_cast<uint32_t>(vlb::blocked_elems(pl.T, pl.K1) * 2);
    g2.a_bytes = static_cast<uint32_t>(vlb::blocked_elems(pl.T, p->hidden) * 2);
    g1.out2 = saved ? saved + sl.off_z1 : nullptr;
    VLB_LAUNCH(VLB_K_GEMM1, s,
               vlb::launch_gemm_bf16(saved    ? vlb::kGemmBlockedSave
                                     : gather ? vlb::kGemmGatherBlocked
                                              : vlb::kGemmBlocked,
                                     g1, s));
    // middle Linears: act(H W^T + b), blocked in and out, alternating buffers
    for (int q = 0; q + 2 < proj_depth(p); ++q) {
      const void *wm = w->w_mid[q];
      if (!p->packed) {
        VLB_LAUNCH(VLB_K_PACK, s,
                   vlb::launch_pack(wm, p->hidden, p->hidden, p->C, 1, ws + pl.off_wmp, s));
        wm = ws + pl.off_wmp;
      }
      vlb::GemmArgs gm{};
      gm.A = g2.A;
      gm.B = wm;
      gm.bias = w->b_mid[q];
      gm.out = saved ? saved + sl.off_a(q + 1)
               : g2.A == ws + pl.off_h ? ws + pl.off_h2 : ws + pl.off_h;
      gm.M = static_cast<int32_t>(pl.T);
      gm.N = p->hidden;
      gm.K = p->hidden;
      gm.ldo = p->hidden;
      gm.act = p->act;
      gm.a_bytes = g2.a_bytes;
      gm.b_bytes = static_cast<uint32_t>(vlb::blocked_elems(p->hidden, p->hidden) * 2);
      gm.out2 = saved ? saved + sl.off_z(q + 1) : nullptr;
      VLB_LAUNCH(VLB_K_GEMM_MID, s,
                 vlb::launch_gemm_bf16(saved ? vlb::kGemmBlockedSave : vlb::kGemmBlocked, gm, s));
      g2.A = gm.out;
    }
    g2.stream_out = 1;  // the sequence rows are not read back here
    VLB_LAUNCH(VLB_K_GEMM2, s, vlb::launch_gemm_bf16(vlb::kGemmRows, g2, s));
  } else {
    g1.B = w->w1;
    if (saved) {  // from the kept merged rows, keeping Z1 as well
      g1.A = saved + sl.off_xm;
      g1.out2 = saved + sl.off_z1;
    }
    VLB_LAUNCH(VLB_K_GEMM1, s, vlb::launch_gemm_f32(!saved, g1, s));
    for (int q = 0; q + 2 < proj_depth(p); ++q) {
      vlb::GemmArgs gm{};
      gm.A = g2.A;
      gm.B = w->w_mid[q];
      gm.bias = w->b_mid[q];
      gm.out = g2.A == ws + pl.off_h ? ws + pl.off_h2 : ws + pl.off_h;
      gm.M = static_cast<int32_t>(pl.T);
      gm.N = p->hidden;
      gm.K = p->hidden;
      gm.ldo = p->hidden;
      gm.act = p->act;
      gm.out2 = saved ? saved + sl.off_z(q + 1) : nullptr;
      VLB_LAUNCH(VLB_K_GEMM_MID, s, vlb::launch_gemm_f32(false, gm, s));
      g2.A = gm.out;
    }
    VLB_LAUNCH(VLB_K_GEMM2, s, vlb::launch_gemm_f32(false, g2, s));
  }
  return VLB_OK;
}

// Where the placeholders are: a uint8 mask, or token ids equal to image_id
// (the other ids must lie in [0, vocab)).
struct PlaceSrc {
  const uint8_t *mask;
  const int32_t *ids;
  int32_t image_id;
  int64_t vocab;
};

// Slot map of a tiled batch from the scan's slot positions: dst_row of every
// token row; newline and separator rows written to their slots.
vlb_status run_place_tiled(const vlb_projector *p, const vlb_batch *b, const Plan &pl,
                           const void *newline, const void *separator, void *seq, uint8_t *ws,
                           hipStream_t s) {
  int32_t *status = reinterpret_cast<int32_t *>(ws + pl.off_status);
  int32_t *slot_pos = reinterpret_cast<int32_t *>(ws + pl.off_slot);
  int32_t *dst_row = reinterpret_cast<int32_t *>(ws + pl.off_dst);
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

// Prefix sum of the placeholders and (tiled) the assembly map -> dst_row, as
// launches of their own; newline / separator rows are written to their slots.
vlb_status run_place(const vlb_projector *p, const vlb_batch *b, const Plan &pl,
                     const void *newline, const void *separator, const PlaceSrc &src,
                     int64_t seq_len, void *seq, uint8_t *ws, hipStream_t s) {
  int32_t *status = reinterpret_cast<int32_t *>(ws + pl.off_status);
  int32_t *slot_pos = reinterpret_cast<int32_t *>(ws + pl.off_slot);
  int32_t *dst_row = reinterpret_cast<int32_t *>(ws + pl.off_dst);
  // the token-id form also lists the text positions and their ids
  int32_t *text = src.ids ? reinterpret_cast<int32_t *>(ws + pl.off_text) : nullptr;
  if (b->layout == VLB_LAYOUT_PLAIN) {  // token row r -> the r-th placeholder: the scan writes dst_row
    VLB_LAUNCH(VLB_K_SCAN, s,
               vlb::launch_scan(src.mask, src.ids, src.image_id, src.vocab, seq_len, pl.P, dst_row,
                                status, true, s, text));
    return VLB_OK;
  }
  VLB_LAUNCH(VLB_K_SCAN, s,
             vlb::launch_scan(src.mask, src.ids, src.image_id, src.vocab, seq_len, pl.P, slot_pos,
                              status, false, s, text));
  return run_place_tiled(p, b, pl, newline, separator, seq, ws, s);
}

// bf16: the placeholder scan runs as one extra workgroup of the first merge
// launch instead of a launch of its own.  In the plain layout it writes
// dst_row itself; in the tiled layout it writes the slot positions, and the
// slot map runs after the merge (TiledPlace).  Linear2, the first reader of
// dst_row, comes after both either way.
bool scan_in_merge(const vlb_projector *p) { return p->dtype == VLB_BF16; }

// The scan of the mask (ids == nullptr) or of the token ids.
vlb::ScanJob merge_scan(const vlb_batch *b, const Plan &pl, const uint8_t *mask,
                        const int32_t *ids, int32_t image_id, int64_t vocab, int64_t seq_len,
                        uint8_t *ws) {
  const bool plain = b->layout == VLB_LAYOUT_PLAIN;
  return vlb::ScanJob{mask, ids, image_id, vocab, seq_len, pl.P,
                      reinterpret_cast<int32_t *>(ws + (plain ? pl.off_dst : pl.off_slot)),
                      reinterpret_cast<int32_t *>(ws + pl.off_status), plain,
                      ids ? reinterpret_cast<int32_t *>(ws + pl.off_text) : nullptr};
}

vlb_status check_weights(const vlb_projector *p, const vlb_weights *w) {
  if (!w) return VLB_ERR_NULL;
  if (!w->w1 || !w->b1 || !w->w2 || !w->b2) return VLB_ERR_NULL;
  if (p->has_ln && (!w->ln_gamma || !w->ln_beta)) return VLB_ERR_NULL;
  if (!aligned16(w->w1) || !aligned16(w->b1) || !aligned16(w->w2) || !aligned16(w->b2))
    return VLB_ERR_ALIGN;
  if (p->has_ln && (!aligned16(w->ln_gamma) || !aligned16(w->ln_beta))) return VLB_ERR_ALIGN;
  if (proj_depth(p) > 2) {
    if (!w->w_mid || !w->b_mid) return VLB_ERR_NULL;
    for (int q = 0; q + 2 < proj_depth(p); ++q) {
      if (!w->w_mid[q] || !w->b_mid[q]) return VLB_ERR_NULL;
      if (!aligned16(w->w_mid[q]) || !aligned16(w->b_mid[q])) return VLB_ERR_ALIGN;
    }
  }
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
  if (which == 3) return static_cast<size_t>(vlb::blocked_elems(p->hidden, p->hidden)) * 2;
  return 0;
}

vlb_status vlb_pack_mid(const vlb_projector *p, const void *w, void *w_packed, void *stream) {
  vlb_status st = check_projector(p);
  if (st != VLB_OK) return st;
  if (p->dtype != VLB_BF16) return VLB_ERR_UNSUPPORTED;
  if (!w || !w_packed) return VLB_ERR_NULL;
  if (!aligned16(w) || !aligned16(w_packed)) return VLB_ERR_ALIGN;
  const size_t n = static_cast<size_t>(p->hidden) * p->hidden * 2;
  if (overlaps(w_packed, vlb_packed_bytes(p, 3), w, n)) return VLB_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  VLB_LAUNCH(VLB_K_PACK, s, vlb::launch_pack(w, p->hidden, p->hidden, p->C, 1, w_packed, s));
  return VLB_OK;
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

}  // extern "C"

namespace {

// The fused call's launches on a validated plan, with workspace w8.
vlb_status run_fused(const vlb_projector *p, const vlb_batch *b, const Plan &pl,
                     const void *features, const vlb_weights *w, const void *newline,
                     const void *separator, const uint8_t *mask, int64_t seq_len, void *seq,
                     uint8_t *w8, hipStream_t s) {
  vlb_status st;
  const vlb::ScanJob sj = merge_scan(b, pl, mask, nullptr, 0, 0, seq_len, w8);
  const TiledPlace tp{newline, separator, seq};
  const bool fused_scan = scan_in_merge(p), tiled = b->layout == VLB_LAYOUT_TILED_2D;
  if (!fused_scan) {
    st = run_place(p, b, pl, newline, separator, PlaceSrc{mask, nullptr, 0, 0}, seq_len, seq, w8,
                   s);
    if (st != VLB_OK) return st;
  }
  return run_project(p, b, pl, features, w, seq,
                     reinterpret_cast<const int32_t *>(w8 + pl.off_dst), w8, s, nullptr,
                     fused_scan ? &sj : nullptr, fused_scan && tiled ? &tp : nullptr);
}

// Argument checks of the fused call (after make_plan), workspace aside.
vlb_status check_fused_args(const vlb_projector *p, const vlb_batch *b, const void *features,
                            const vlb_weights *w, const void *newline, const void *separator,
                            const uint8_t *mask, int64_t seq_len, const void *seq) {
  vlb_status st;
  if ((st = check_weights(p, w)) != VLB_OK) return st;
  if ((st = check_scatter_args(p, b, newline, separator, mask, seq_len, seq)) != VLB_OK) return st;
  if (!features) return VLB_ERR_NULL;
  if (!aligned16(features)) return VLB_ERR_ALIGN;
  return VLB_OK;
}

}  // namespace

extern "C" {

vlb_status vlb_bridge_fused(const vlb_projector *p, const vlb_batch *b, const void *features,
                            const vlb_weights *w, const void *newline, const void *separator,
                            const uint8_t *mask, int64_t seq_len, void *seq, void *ws,
                            size_t ws_bytes, void *stream) {
  Plan pl;
  vlb_status st = make_plan(p, b, seq_len, &pl);
  if (st != VLB_OK) return st;
  if (pl.T == 0) return VLB_OK;
  if ((st = check_fused_args(p, b, features, w, newline, separator, mask, seq_len, seq)) != VLB_OK)
    return st;
  if (!ws) return VLB_ERR_NULL;
  if (!aligned16(ws)) return VLB_ERR_ALIGN;
  if (ws_bytes < pl.total) return VLB_ERR_WORKSPACE;
  return run_fused(p, b, pl, features, w, newline, separator, mask, seq_len, seq,
                   static_cast<uint8_t *>(ws), static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- the allocation-free fused call -----------------------------------------
// The workspace of vlb_bridge_fused_noalloc: one array per GPU (every device
// that runs the library holds its own copy until the process ends).  Host code
// never uses the array's name as an address -- on the host it is a stand-in --
// but the device address that hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) uint8_t scratch[VLB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];  // scratch's device address on each device, once taken

// scratch's address on the current device, taken on the first call there.
vlb_status scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VLB_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return VLB_ERR_HIP;
    g_scratch[dev] = a;
  }
  *out = g_scratch[dev];
  return VLB_OK;
}

}  // namespace

extern "C" {

vlb_status vlb_bridge_fused_noalloc(const vlb_projector *p, const vlb_batch *b,
                                    const void *features, const vlb_weights *w,
                                    const void *newline, const void *separator,
                                    const uint8_t *mask, int64_t seq_len, void *seq,
                                    int32_t *status, void *stream) {
  if (!p) return VLB_ERR_NULL;
  vlb_projector q = *p;  // the gather keeps the merged tokens out of the scratch
  if (q.gather == VLB_GATHER_AUTO && q.dtype == VLB_BF16 && !q.has_ln) q.gather = VLB_GATHER_ON;
  Plan pl;
  vlb_status st = make_plan(&q, b, seq_len, &pl);
  if (st != VLB_OK) return st;
  if (!status) return VLB_ERR_NULL;
  if (!aligned16(status)) return VLB_ERR_ALIGN;
  if (pl.T > 0 &&
      (st = check_fused_args(&q, b, features, w, newline, separator, mask, seq_len, seq)) != VLB_OK)
    return st;
  if (pl.total > VLB_NOALLOC_SCRATCH_BYTES) return VLB_ERR_SCRATCH;
  void *scr = nullptr;
  if ((st = scratch_address(&scr)) != VLB_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *w8 = static_cast<uint8_t *>(scr);
  if (pl.T > 0 &&
      (st = run_fused(&q, b, pl, features, w, newline, separator, mask, seq_len, seq, w8, s)) !=
          VLB_OK)
    return st;
  // The call's status words, into the caller's buffer (zeros when nothing ran).
  VLB_LAUNCH(VLB_K_SCAN, s,
             vlb::launch_copy_status(
                 pl.T > 0 ? reinterpret_cast<const int32_t *>(w8 + pl.off_status) : nullptr,
                 status, s));
  return VLB_OK;
}

size_t vlb_saved_bytes(const vlb_projector *p, const vlb_batch *b) {
  Plan pl;
  if (make_plan(p, b, 0, &pl) != VLB_OK) return 0;
  return saved_layout(p, pl).total;
}

size_t vlb_backward_workspace_bytes(const vlb_projector *p, const vlb_batch *b, int64_t seq_len) {
  Plan pl;
  BwdLayout L;
  if (make_plan(p, b, seq_len, &pl) != VLB_OK || bwd_layout(p, b, pl, seq_len, &L) != VLB_OK)
    return 0;
  return L.total;
}

vlb_status vlb_bridge_fused_train(const vlb_projector *p, const vlb_batch *b,
                                  const void *features, const vlb_weights *w,
                                  const void *newline, const void *separator,
                                  const uint8_t *mask, int64_t seq_len, void *seq, void *saved,
                                  size_t saved_bytes, void *ws, size_t ws_bytes, void *stream) {
  Plan pl;
  vlb_status st = make_plan(p, b, seq_len, &pl);
  if (st != VLB_OK) return st;
  if (pl.T == 0) return VLB_OK;
  if ((st = check_weights(p, w)) != VLB_OK) return st;
  if ((st = check_scatter_args(p, b, newline, separator, mask, seq_len, seq)) != VLB_OK) return st;
  if (!features || !ws || !saved) return VLB_ERR_NULL;
  if (!aligned16(features) || !aligned16(ws) || !aligned16(saved)) return VLB_ERR_ALIGN;
  if (ws_bytes < pl.total) return VLB_ERR_WORKSPACE;
  const size_t need = saved_layout(p, pl).total;
  if (saved_bytes < need) return VLB_ERR_WORKSPACE;
  const size_t seq_bytes = static_cast<size_t>(seq_len) * p->out_dim * pl.es;
  if (overlaps(saved, need, ws, pl.total) || overlaps(saved, need, seq, seq_bytes))
    return VLB_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  const vlb::ScanJob sj = merge_scan(b, pl, mask, nullptr, 0, 0, seq_len, w8);
  const TiledPlace tp{newline, separator, seq};
  const bool fused_scan = scan_in_merge(p), tiled = b->layout == VLB_LAYOUT_TILED_2D;
  if (!fused_scan) {
    st = run_place(p, b, pl, newline, separator, PlaceSrc{mask, nullptr, 0, 0}, seq_len, seq, w8,
                   s);
    if (st != VLB_OK) return st;
  }
  return run_project(p, b, pl, features, w, seq,
                     reinterpret_cast<const int32_t *>(w8 + pl.off_dst), w8, s,
                     static_cast<uint8_t *>(saved), fused_scan ? &sj : nullptr,
                     fused_scan && tiled ? &tp : nullptr);
}

vlb_status vlb_bridge_backward(const vlb_projector *p, const vlb_batch *b, const void *features,
                               const vlb_weights *w, const uint8_t *mask, int64_t seq_len,
                               const void *dseq, const void *saved, size_t saved_bytes,
                               const vlb_grads *g, void *ws, size_t ws_bytes, void *stream) {
  Plan pl;
  vlb_status st = make_plan(p, b, seq_len, &pl);
  if (st != VLB_OK) return st;
  BwdLayout L;
  if ((st = bwd_layout(p, b, pl, seq_len, &L)) != VLB_OK) return st;
  const bool ln = p->has_ln != 0, tiled = b->layout == VLB_LAYOUT_TILED_2D;
  if (!g || !w || !mask || !dseq || !saved || !ws) return VLB_ERR_NULL;
  if (!g->d_w1 || !g->d_b1 || !g->d_w2 || !g->d_b2 || !w->w1 || !w->w2) return VLB_ERR_NULL;
  const int n_mid = proj_depth(p) - 2;
  if (n_mid > 0) {
    if (!w->w_mid || !g->d_w_mid || !g->d_b_mid) return VLB_ERR_NULL;
    for (int q = 0; q < n_mid; ++q) {
      if (!w->w_mid[q] || !g->d_w_mid[q] || !g->d_b_mid[q]) return VLB_ERR_NULL;
      if (!aligned16(w->w_mid[q]) || !aligned16(g->d_w_mid[q]) || !aligned16(g->d_b_mid[q]))
        return VLB_ERR_ALIGN;
    }
  }
  if (ln && (!g->d_ln_gamma || !g->d_ln_beta || !w->ln_gamma)) return VLB_ERR_NULL;
  if (ln && pl.T > 0 && !features) return VLB_ERR_NULL;
  if (tiled && (!g->d_newline || !g->d_separator)) return VLB_ERR_NULL;
  const void *ptrs[] = {mask, dseq, saved, ws, g->d_w1, g->d_b1, g->d_w2, g->d_b2, w->w1, w->w2,
                        g->d_features, features, w->ln_gamma, g->d_ln_gamma, g->d_ln_beta,
                        g->d_newline, g->d_separator};
  for (const void *q : ptrs)
    if (!aligned16(q)) return VLB_ERR_ALIGN;
  if (seq_len < 1) return VLB_ERR_SHAPE;
  if (ws_bytes < L.total) return VLB_ERR_WORKSPACE;
  if (saved_bytes < saved_layout(p, pl).total) return VLB_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = pl.T, H = p->hidden, O = p->out_dim, K1 = pl.K1, C = p->C;
  if (T == 0) {  // no token rows: every gradient is zero
    auto zero = [&](void *q, size_t bytes) {
      return q == nullptr || hipMemsetAsync(q, 0, bytes, s) == hipSuccess;
    };
    bool ok = true;
    for (int q = 0; q < n_mid; ++q)
      ok = ok && zero(g->d_w_mid[q], H * H * 4) && zero(g->d_b_mid[q], H * 4);
    ok = ok && zero(g->d_w1, H * K1 * 4) && zero(g->d_b1, H * 4) &&
                    zero(g->d_w2, O * H * 4) && zero(g->d_b2, O * 4) &&
                    (!ln || (zero(g->d_ln_gamma, C * 4) && zero(g->d_ln_beta, C * 4))) &&
                    (!tiled || (zero(g->d_newline, O * 4) && zero(g->d_separator, O * 4))) &&
                    zero(g->d_features, static_cast<size_t>(pl.npix) * C * pl.es);
    return ok ? VLB_OK : VLB_ERR_HIP;
  }
  uint8_t *w8 = static_cast<uint8_t *>(ws);
  const uint8_t *sv = static_cast<const uint8_t *>(saved);
  const SavedLayout sl = saved_layout(p, pl);
  int32_t *status = reinterpret_cast<int32_t *>(w8 + L.off_status);
  int32_t *dst_row = reinterpret_cast<int32_t *>(w8 + L.off_dst);
  int32_t *slot_pos = reinterpret_cast<int32_t *>(w8 + L.off_slot);
  int32_t *nl_pos = reinterpret_cast<int32_t *>(w8 + L.off_nl);
  int32_t *sep_pos = reinterpret_cast<int32_t *>(w8 + L.off_sep);
  const int32_t Tk = static_cast<int32_t>(L.Tk), Op = static_cast<int32_t>(L.Op);
  const int32_t Ti = static_cast<int32_t>(T), Hi = static_cast<int32_t>(H),
                Oi = static_cast<int32_t>(O), K1i = static_cast<int32_t>(K1);

  // 1. slot of every token row (and of every newline / separator)
  if (!tiled) {
    VLB_LAUNCH(VLB_K_SCAN, s,
               vlb::launch_scan(mask, nullptr, 0, 0, seq_len, pl.P, dst_row, status, true, s));
  } else {
    VLB_LAUNCH(VLB_K_SCAN, s,
               vlb::launch_scan(mask, nullptr, 0, 0, seq_len, pl.P, slot_pos, status, false, s));
    int32_t nl0 = 0;
    for (int i0 = 0; i0 < b->n_images; i0 += vlb::kPlaceImages) {
      PlaceChunk c{};
      c.n = std::min(vlb::kPlaceImages, b->n_images - i0);
      c.tail = b->global_view_tail;
      c.img0 = i0;
      for (int i = 0; i < c.n; ++i) {
        const int im = i0 + i, v = pl.img_view0[im];
        c.slot0[i] = pl.img_slot0[im];
        c.row0[i] = pl.img_row0[im];
        c.hp[i] = static_cast<int16_t>(ceil_div(b->grid_h[v], p->k));
        c.wp[i] = static_cast<int16_t>(ceil_div(b->grid_w[v], p->k));
        c.tw[i] = static_cast<int16_t>(b->tile_w[im]);
        c.th[i] = static_cast<int16_t>(b->tile_h[im]);
        c.nl0[i] = nl0;
        nl0 += c.hp[i] * (1 + c.th[i]);
      }
      c.slot0[c.n] = pl.img_slot0[i0 + c.n];
      VLB_LAUNCH(VLB_K_PLACE, s,
                 vlb::launch_place_tiled_record(c, slot_pos, status, dst_row, nl_pos, sep_pos, s));
    }
  }
  if (p->dtype == VLB_F32) {  // row-major operands, strided fp32 GEMMs
    float *dy = reinterpret_cast<float *>(w8 + L.off_dy);
    float *a1 = reinterpret_cast<float *>(w8 + L.off_a1t);
    float *dz = reinterpret_cast<float *>(w8 + L.off_da1);
    float *dxm = reinterpret_cast<float *>(w8 + L.off_dxm);
    const void *xm = sv + sl.off_xm;
    VLB_LAUNCH(VLB_K_BWD_PACK, s, vlb::launch_gather_rows_f32(dseq, dst_row, Ti, Oi, dy, s));
    VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_colsum(dy, Ti, Oi, g->d_b2, status, s));
    const void *zl = sv + sl.off_z(n_mid);  // the last Linear's input is act(Z_last)
    VLB_LAUNCH(VLB_K_BWD_PACK, s, vlb::launch_act_f32(p->act, zl, T * H, a1, nullptr, s));
    auto gemm = [&](const void *A, int64_t sam, int64_t sak, const void *B, int64_t sbn,
                    int64_t sbk, void *out, int64_t M, int64_t N, int64_t K,
                    const int32_t *st_word) {
      vlb::GemmArgs ga{};
      ga.A = A;
      ga.B = B;
      ga.out = out;
      ga.M = static_cast<int32_t>(M);
      ga.N = static_cast<int32_t>(N);
      ga.K = static_cast<int32_t>(K);
      ga.ldo = static_cast<int32_t>(N);
      ga.act = VLB_ACT_NONE;
      ga.sa_m = sam;
      ga.sa_k = sak;
      ga.sb_n = sbn;
      ga.sb_k = sbk;
      ga.status = st_word;
      return ga;
    };
    // dW2[o][h] = sum_t dY[t][o] act(Z1)[t][h]; dA1[t][h] = sum_o dY[t][o] W2[o][h]
    VLB_LAUNCH(VLB_K_BWD_DW2, s,
               vlb::launch_gemm_f32(false, gemm(dy, 1, O, a1, 1, H, g->d_w2, O, H, T, status), s));
    VLB_LAUNCH(VLB_K_BWD_DA1, s,
               vlb::launch_gemm_f32(false, gemm(dy, O, 1, w->w2, 1, H, dz, T, H, O, nullptr), s));
    VLB_LAUNCH(VLB_K_BWD_PACK, s, vlb::launch_act_f32(p->act, zl, T * H, nullptr, dz, s));
    // middle Linears, last to first: layer q maps act(Z_{q-1}) to Z_q
    for (int q = n_mid; q >= 1; --q) {
      const void *zp = sv + sl.off_z(q - 1);
      VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_colsum(dz, Ti, Hi, g->d_b_mid[q - 1], status, s));
      VLB_LAUNCH(VLB_K_BWD_PACK, s, vlb::launch_act_f32(p->act, zp, T * H, a1, nullptr, s));
      VLB_LAUNCH(VLB_K_BWD_DW2, s,
                 vlb::launch_gemm_f32(
                     false, gemm(dz, 1, H, a1, 1, H, g->d_w_mid[q - 1], H, H, T, status), s));
      VLB_LAUNCH(VLB_K_BWD_DA1, s,
                 vlb::launch_gemm_f32(false, gemm(dz, H, 1, w->w_mid[q - 1], 1, H, a1, T, H, H,
                                                  nullptr), s));
      VLB_LAUNCH(VLB_K_BWD_PACK, s, vlb::launch_act_f32(p->act, zp, T * H, nullptr, a1, s));
      std::swap(dz, a1);  // dZ_{q-1}
    }
    VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_colsum(dz, Ti, Hi, g->d_b1, status, s));
    // dW1[h][i] = sum_t dZ1[t][h] Xm[t][i]; dXm[t][i] = sum_h dZ1[t][h] W1[h][i]
    VLB_LAUNCH(VLB_K_BWD_DW1, s,
               vlb::launch_gemm_f32(false, gemm(dz, 1, H, xm, 1, K1, g->d_w1, H, K1, T, status),
                                    s));
    if (ln || g->d_features) {
      VLB_LAUNCH(VLB_K_BWD_DX, s,
                 vlb::launch_gemm_f32(false, gemm(dz, H, 1, w->w1, 1, K1, dxm, T, K1, H, nullptr),
                                      s));
      float *pg = reinterpret_cast<float *>(w8 + L.off_pln);
      float *pbeta = pg + L.ln_rows * C;
      int64_t row = 0;
      for (int v0 = 0, ci = 0; v0 < b->n_views; v0 += vlb::kPlanViews, ++ci) {
        const int grid = L.ln_grid[ci];
        VLB_LAUNCH(VLB_K_BWD_UNMERGE, s,
                   vlb::launch_bwd_unmerge_f32(dxm, features, view_chunk(p, b, pl, v0), p->C,
                                               ln ? w->ln_gamma : nullptr, p->ln_eps,
                                               g->d_features, pg + row * C, pbeta + row * C,
                                               status, grid, s));
        row += grid;
      }
      if (ln) {
        const int32_t R = static_cast<int32_t>(L.ln_rows);
        VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_colsum(pg, R, p->C, g->d_ln_gamma, status, s));
        VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_colsum(pbeta, R, p->C, g->d_ln_beta, status, s));
      }
    }
    if (tiled) {
      float *pnl = reinterpret_cast<float *>(w8 + L.off_pnl);
      float *psep = reinterpret_cast<float *>(w8 + L.off_psep);
      const int32_t NL = static_cast<int32_t>(L.NL);
      VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_rows_sum(p->dtype, dseq, nl_pos, NL, Oi, pnl, s));
      VLB_LAUNCH(VLB_K_BWD_SUM, s,
                 vlb::launch_colsum(pnl, (NL + 63) / 64, Oi, g->d_newline, status, s));
      VLB_LAUNCH(VLB_K_BWD_SUM, s,
                 vlb::launch_rows_sum(p->dtype, dseq, sep_pos, b->n_images, Oi, psep, s));
      VLB_LAUNCH(VLB_K_BWD_SUM, s,
                 vlb::launch_colsum(psep, (b->n_images + 63) / 64, Oi, g->d_separator, status,
                                    s));
    }
    return VLB_OK;
  }
  // 2. dY, its transpose, db2
  float *pb2 = reinterpret_cast<float *>(w8 + L.off_pb2);
  VLB_LAUNCH(VLB_K_BWD_PACK, s,
             vlb::launch_bwd_gather_dy(dseq, dst_row, Ti, Oi, Op, Tk, w8 + L.off_dy,
                                       w8 + L.off_dyt, pb2, s));
  VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_colsum(pb2, Tk / 32, Oi, g->d_b2, status, s));
  // dW2 and the middle weight gradients read the saved activations
  // token-major (GemmArgs::b_tmaj, rows past T read zero), and the products
  // with a weight read the packed weight token-major, so neither needs a
  // transposing pass; weights passed unpacked are packed here first.  dW1
  // takes Xm^T, whose rows are in the pages' feature order (Xm's columns are
  // position-major), so the gradient comes out in the pages' order.
  float *split_part = L.split_bytes ? reinterpret_cast<float *>(w8 + L.off_split) : nullptr;
  auto tmaj_b = [&](vlb::GemmArgs &g, const void *B, int32_t width, int32_t k_valid,
                    int64_t stored_rows) {
    g.B = B;
    g.b_tmaj = 1;
    g.tb_w = width;
    g.k_valid = k_valid;
    g.b_bytes = static_cast<uint32_t>(vlb::blocked_elems(stored_rows, width) * 2);
  };
  auto packed_weight = [&](const void *w_in, int64_t R, int64_t Kw, int kmerge, size_t off,
                           const void **out) -> vlb_status {
    if (p->packed) {
      *out = w_in;
      return VLB_OK;
    }
    VLB_LAUNCH(VLB_K_PACK, s, vlb::launch_pack(w_in, R, Kw, p->C, kmerge, w8 + off, s));
    *out = w8 + off;
    return VLB_OK;
  };
  vlb_status pst;
  // 3. dW2 = dY^T act(Z1)
  vlb::GemmArgs gw2{};
  gw2.A = w8 + L.off_dyt;
  gw2.out = g->d_w2;
  gw2.status = status;
  gw2.M = Oi;
  gw2.N = Hi;
  gw2.K = Tk;
  gw2.ldo = Hi;
  gw2.act = VLB_ACT_NONE;
  gw2.a_bytes = static_cast<uint32_t>(vlb::blocked_elems(O, Tk) * 2);
  tmaj_b(gw2, sv + sl.off_a(n_mid), Hi, Ti, T);
  gw2.split_part = split_part;
  VLB_LAUNCH(VLB_K_BWD_DW2, s, vlb::launch_gemm_bf16(vlb::kGemmF32, gw2, s));
  // 4. dA1 = dY W2, then dZ1 = dA1 * act'(Z1) and db1
  const void *w2p = nullptr;
  if ((pst = packed_weight(w->w2, O, H, 1, L.off_w2p, &w2p)) != VLB_OK) return pst;
  vlb::GemmArgs ga{};
  ga.A = w8 + L.off_dy;
  ga.out = w8 + L.off_da1;
  ga.M = Ti;
  ga.N = Hi;
  ga.K = Op;
  ga.ldo = Hi;
  ga.act = VLB_ACT_NONE;
  ga.a_bytes = static_cast<uint32_t>(vlb::blocked_elems(T, Op) * 2);
  tmaj_b(ga, w2p, Hi, Op, O);  // packed W2 [O][H]: rows past O are zero
  VLB_LAUNCH(VLB_K_BWD_DA1, s, vlb::launch_gemm_bf16(vlb::kGemmBlocked, ga, s));
  float *pb1 = reinterpret_cast<float *>(w8 + L.off_pb1);
  VLB_LAUNCH(VLB_K_BWD_PACK, s,
             vlb::launch_bwd_dact(p->act, w8 + L.off_da1, sv + sl.off_z(n_mid), Ti, Hi, Tk,
                                  w8 + L.off_dz1, w8 + L.off_dz1t, pb1, s));
  // middle Linears, last to first: layer q maps act(Z_{q-1}) to Z_q
  for (int q = n_mid; q >= 1; --q) {
    VLB_LAUNCH(VLB_K_BWD_SUM, s,
               vlb::launch_colsum(pb1, Tk / 32, Hi, g->d_b_mid[q - 1], status, s));
    // dW_q = dZ_q^T act(Z_{q-1})
    vlb::GemmArgs gwm{};
    gwm.A = w8 + L.off_dz1t;
    gwm.out = g->d_w_mid[q - 1];
    gwm.status = status;
    gwm.M = Hi;
    gwm.N = Hi;
    gwm.K = Tk;
    gwm.ldo = Hi;
    gwm.act = VLB_ACT_NONE;
    gwm.a_bytes = static_cast<uint32_t>(vlb::blocked_elems(H, Tk) * 2);
    tmaj_b(gwm, sv + sl.off_a(q - 1), Hi, Ti, T);
    gwm.split_part = split_part;
    VLB_LAUNCH(VLB_K_BWD_DW2, s, vlb::launch_gemm_bf16(vlb::kGemmF32, gwm, s));
    // dA_{q-1} = dZ_q W_q, then dZ_{q-1} = dA_{q-1} * act'(Z_{q-1})
    const void *wqp = nullptr;
    if ((pst = packed_weight(w->w_mid[q - 1], H, H, 1, L.off_wmp, &wqp)) != VLB_OK) return pst;
    vlb::GemmArgs gam{};
    gam.A = w8 + L.off_dz1;
    gam.out = w8 + L.off_da1;
    gam.M = Ti;
    gam.N = Hi;
    gam.K = Hi;
    gam.ldo = Hi;
    gam.act = VLB_ACT_NONE;
    gam.a_bytes = static_cast<uint32_t>(vlb::blocked_elems(T, H) * 2);
    tmaj_b(gam, wqp, Hi, Hi, H);
    VLB_LAUNCH(VLB_K_BWD_DA1, s, vlb::launch_gemm_bf16(vlb::kGemmBlocked, gam, s));
    VLB_LAUNCH(VLB_K_BWD_PACK, s,
               vlb::launch_bwd_dact(p->act, w8 + L.off_da1, sv + sl.off_z(q - 1), Ti, Hi, Tk,
                                    w8 + L.off_dz1, w8 + L.off_dz1t, pb1, s));
  }
  VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_colsum(pb1, Tk / 32, Hi, g->d_b1, status, s));
  // 5. dW1 = dZ1^T Xm (columns in the pages' order)
  VLB_LAUNCH(VLB_K_BWD_PACK, s,
             vlb::launch_bwd_xm_t(sv + sl.off_xm, Ti, p->C, p->k, Tk, w8 + L.off_xmt, s));
  vlb::GemmArgs gw1{};
  gw1.A = w8 + L.off_dz1t;
  gw1.out = g->d_w1;
  gw1.status = status;
  gw1.M = Hi;
  gw1.N = K1i;
  gw1.K = Tk;
  gw1.ldo = K1i;
  gw1.act = VLB_ACT_NONE;
  gw1.a_bytes = static_cast<uint32_t>(vlb::blocked_elems(H, Tk) * 2);
  gw1.B = w8 + L.off_xmt;
  gw1.b_bytes = static_cast<uint32_t>(vlb::blocked_elems(K1, Tk) * 2);
  gw1.split_part = split_part;
  VLB_LAUNCH(VLB_K_BWD_DW1, s, vlb::launch_gemm_bf16(vlb::kGemmF32, gw1, s));
  // 6. dXm = dZ1 W1 (K position-major, the packed W1's order), unmerge,
  // LayerNorm backward
  if (ln || g->d_features) {
    const void *w1p = nullptr;
    if ((pst = packed_weight(w->w1, H, K1, p->k, L.off_w1p, &w1p)) != VLB_OK) return pst;
    vlb::GemmArgs gx{};
    gx.A = w8 + L.off_dz1;
    gx.out = w8 + L.off_dxm;
    gx.M = Ti;
    gx.N = K1i;
    gx.K = Hi;
    gx.ldo = K1i;
    gx.act = VLB_ACT_NONE;
    gx.a_bytes = static_cast<uint32_t>(vlb::blocked_elems(T, H) * 2);
    tmaj_b(gx, w1p, K1i, Hi, H);
    VLB_LAUNCH(VLB_K_BWD_DX, s, vlb::launch_gemm_bf16(vlb::kGemmRows, gx, s));
    float *pg = reinterpret_cast<float *>(w8 + L.off_pln);
    float *pbeta = pg + L.ln_rows * C;
    int64_t row = 0;
    for (int v0 = 0, ci = 0; v0 < b->n_views; v0 += vlb::kPlanViews, ++ci) {
      const int grid = L.ln_grid[ci];
      VLB_LAUNCH(VLB_K_BWD_UNMERGE, s,
                 vlb::launch_bwd_unmerge(w8 + L.off_dxm, features, view_chunk(p, b, pl, v0),
                                         p->C, ln ? w->ln_gamma : nullptr, p->ln_eps,
                                         g->d_features, pg + row * C, pbeta + row * C, status,
                                         grid, s));
      row += grid;
    }
    if (ln) {
      const int32_t R = static_cast<int32_t>(L.ln_rows);
      VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_colsum(pg, R, p->C, g->d_ln_gamma, status, s));
      VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_colsum(pbeta, R, p->C, g->d_ln_beta, status, s));
    }
  }
  // 7. newline and separator: sums over their slots
  if (tiled) {
    float *pnl = reinterpret_cast<float *>(w8 + L.off_pnl);
    float *psep = reinterpret_cast<float *>(w8 + L.off_psep);
    const int32_t NL = static_cast<int32_t>(L.NL);
    VLB_LAUNCH(VLB_K_BWD_SUM, s, vlb::launch_rows_sum(p->dtype, dseq, nl_pos, NL, Oi, pnl, s));
    VLB_LAUNCH(VLB_K_BWD_SUM, s,
               vlb::launch_colsum(pnl, (NL + 63) / 64, Oi, g->d_newline, status, s));
    VLB_LAUNCH(VLB_K_BWD_SUM, s,
               vlb::launch_rows_sum(p->dtype, dseq, sep_pos, b->n_images, Oi, psep, s));
    VLB_LAUNCH(VLB_K_BWD_SUM, s,
               vlb::launch_colsum(psep, (b->n_images + 63) / 64, Oi, g->d_separator, status, s));
  }
  return VLB_OK;
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
  const int32_t *status = reinterpret_cast<const int32_t *>(w8 + pl.off_status);
  const int32_t *dst_row = reinterpret_cast<const int32_t *>(w8 + pl.off_dst);
  // (position, id) of every text position, written by the token-id scan
  const int32_t *text = reinterpret_cast<const int32_t *>(w8 + pl.off_text);
  if (pl.T > 0 && scan_in_merge(p)) {
    // The token-id scan rides in the first merge launch (the tiled slot map
    // follows the merge); the text rows, which wait for its verdict, follow
    // the projector (they touch other rows).
    const vlb::ScanJob sj = merge_scan(b, pl, nullptr, ids, image_token_id, vocab, seq_len, w8);
    const TiledPlace tp{newline, separator, seq};
    st = run_project(p, b, pl, features, w, seq, dst_row, w8, s, nullptr, &sj,
                     b->layout == VLB_LAYOUT_TILED_2D ? &tp : nullptr);
    if (st != VLB_OK) return st;
    VLB_LAUNCH(VLB_K_EMBED, s,
               vlb::launch_embed_rows(p->dtype, text, seq_len - pl.P, embed, p->out_dim, status,
                                      seq, s));
    return VLB_OK;
  }
  st = run_place(p, b, pl, newline, separator, PlaceSrc{nullptr, ids, image_token_id, vocab},
                 seq_len, seq, w8, s);
  if (st != VLB_OK) return st;
  VLB_LAUNCH(VLB_K_EMBED, s,
             vlb::launch_embed_rows(p->dtype, text, seq_len - pl.P, embed, p->out_dim, status, seq,
                                    s));
  if (pl.T == 0) return VLB_OK;
  return run_project(p, b, pl, features, w, seq, dst_row, w8, s);
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
    case VLB_ERR_SCRATCH: return "problem too large for the no-allocation scratch";
  }
  return "unknown status";
}

vlb_status vlb_prof_enable(int32_t mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = static_cast<uint32_t>(mask);
  if (g_prof_mask) g_prof_used = 0;
  return VLB_OK;
}

vlb_status vlb_prof_resume(int32_t mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = static_cast<uint32_t>(mask);
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

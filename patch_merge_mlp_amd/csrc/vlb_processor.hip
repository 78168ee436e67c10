// Request planning of the DeepSeek-VL2 processor (host only, no HIP call):
// which candidate resolution an image is tiled at, its [tw, th] tile grid,
// its placeholder count, and the expansion of the prompt's image tokens.
// mlxcel issue #533 "port DeepSeek-VL2", section "Processor", steps 1, 2, 6, 7.
#include <cmath>
#include <cstdint>

#include "vlbridge.h"

// The best fit compares floors of double products; keep every product a
// plain IEEE double multiply (no fused multiply-add), as the page evaluates it.
#pragma clang fp contract(off)

namespace {

vlb_status check_processor(const vlb_processor *pc) {
  if (!pc || !pc->candidates) return VLB_ERR_NULL;
  if (pc->n_candidates < 1 || pc->patch_size < 1 || pc->downsample < 1) return VLB_ERR_SHAPE;
  const int32_t s = pc->candidates[0];  // image_size: the first candidate's width
  if (s < pc->patch_size) return VLB_ERR_SHAPE;
  for (int32_t i = 0; i < pc->n_candidates; ++i) {
    const int32_t W = pc->candidates[2 * i], H = pc->candidates[2 * i + 1];
    // step 6 divides the chosen W and H by image_size: whole tiles only
    if (W < 1 || H < 1 || W % s != 0 || H % s != 0) return VLB_ERR_SHAPE;
  }
  return VLB_OK;
}

// Step 2 for one image: scale = min(W / w0, H / h0); the effective area is
// floor(w0 * scale) * floor(h0 * scale), capped at the image's own area; the
// waste is W * H minus it.  Largest effective area, then smallest waste; the
// first candidate on a full tie.
void best_fit(const vlb_processor *pc, int32_t w0, int32_t h0, int32_t *best) {
  int64_t best_eff = -1, best_waste = 0;
  for (int32_t i = 0; i < pc->n_candidates; ++i) {
    const int32_t W = pc->candidates[2 * i], H = pc->candidates[2 * i + 1];
    const double sw = static_cast<double>(W) / w0, sh = static_cast<double>(H) / h0;
    const double scale = sw < sh ? sw : sh;
    const int64_t fw = static_cast<int64_t>(std::floor(w0 * scale));
    const int64_t fh = static_cast<int64_t>(std::floor(h0 * scale));
    const int64_t area = static_cast<int64_t>(w0) * h0;
    const int64_t eff = fw * fh < area ? fw * fh : area;
    const int64_t waste = static_cast<int64_t>(W) * H - eff;
    if (eff > best_eff || (eff == best_eff && waste < best_waste)) {
      best_eff = eff;
      best_waste = waste;
      best[0] = W;
      best[1] = H;
    }
  }
}

}  // namespace

extern "C" {

vlb_status vlb_select_resolution(const vlb_processor *pc, int32_t w0, int32_t h0, int32_t *best) {
  const vlb_status st = check_processor(pc);
  if (st != VLB_OK) return st;
  if (!best) return VLB_ERR_NULL;
  if (w0 < 1 || h0 < 1) return VLB_ERR_SHAPE;
  best_fit(pc, w0, h0, best);
  return VLB_OK;
}

vlb_status vlb_plan_request(const vlb_processor *pc, int32_t n_images, const int32_t *sizes,
                            int32_t *tiles, int64_t *slots) {
  const vlb_status st = check_processor(pc);
  if (st != VLB_OK) return st;
  if (n_images < 0) return VLB_ERR_SHAPE;
  if (n_images == 0) return VLB_OK;
  if (!sizes || !tiles || !slots) return VLB_ERR_NULL;
  for (int32_t i = 0; i < n_images; ++i)
    if (sizes[2 * i] < 1 || sizes[2 * i + 1] < 1) return VLB_ERR_SHAPE;
  const int32_t s = pc->candidates[0];
  const bool crop = n_images <= 2;  // step 1
  // step 7: h' = w' = ceil(floor(image_size / patch_size) / downsample_ratio)
  const int64_t g = s / pc->patch_size;
  const int64_t hp = (g + pc->downsample - 1) / pc->downsample;
  for (int32_t i = 0; i < n_images; ++i) {
    int32_t best[2] = {s, s};
    if (crop) best_fit(pc, sizes[2 * i], sizes[2 * i + 1], best);
    const int64_t tw = best[0] / s, th = best[1] / s;  // step 6, width count first
    tiles[2 * i] = static_cast<int32_t>(tw);
    tiles[2 * i + 1] = static_cast<int32_t>(th);
    // global view with a newline per row, the separator, the local mosaic with a
    // newline per mosaic row
    slots[i] = hp * (hp + 1) + 1 + (th * hp) * (tw * hp + 1);
  }
  return VLB_OK;
}

int64_t vlb_expand_prompt(const int32_t *ids, int64_t n_ids, int32_t image_token_id,
                          int32_t bos_id, const int64_t *slots, int32_t n_images, int32_t *out,
                          int64_t cap) {
  if ((!ids && n_ids > 0) || (!slots && n_images > 0)) return -static_cast<int64_t>(VLB_ERR_NULL);
  if (n_ids < 0 || n_images < 0) return -static_cast<int64_t>(VLB_ERR_SHAPE);
  int64_t n_img = 0, len = 1;  // BOS first
  for (int64_t j = 0; j < n_ids; ++j) {
    if (ids[j] != image_token_id) {
      ++len;
      continue;
    }
    if (n_img >= n_images || slots[n_img] < 0) return -static_cast<int64_t>(VLB_ERR_SHAPE);
    len += slots[n_img++];
  }
  if (n_img != n_images) return -static_cast<int64_t>(VLB_ERR_SHAPE);
  if (!out) return len;
  if (cap < len) return -static_cast<int64_t>(VLB_ERR_SHAPE);
  int64_t o = 0, im = 0;
  out[o++] = bos_id;
  for (int64_t j = 0; j < n_ids; ++j) {
    if (ids[j] != image_token_id) {
      out[o++] = ids[j];
      continue;
    }
    for (int64_t r = 0; r < slots[im]; ++r) out[o++] = image_token_id;
    ++im;
  }
  return len;
}

}  // extern "C"

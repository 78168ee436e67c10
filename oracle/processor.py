"""Oracle of the DeepSeek-VL2 processor's planning steps (pure Python).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only tests/ import it.  It shares no code
with the library's planner (patch_merge_mlp_amd/csrc/vlb_processor.hip); it is
written from mlxcel issue #533 "port DeepSeek-VL2", section "Processor", steps 1,
2, 6 and 7, in the page's order.  The placeholder count uses the fp64 oracle's
closed form (vlb_oracle.c, orc_tiled_placeholders).

Readings where the page leaves a step open (listed in the design notes):
  - candidates that tie on both the effective and the wasted area: the first in
    list order wins;
  - the floating-point steps of the best fit are IEEE double, as the page's own
    arithmetic (Python floats) is;
  - step 1's "at most 2 images" counts the images of the request being planned.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

from oracle import oracle as _o

MAX_CROP_IMAGES = 2  # step 1


def best_resolution(w0: int, h0: int, candidates: Sequence[Tuple[int, int]]) -> Tuple[int, int]:
    """Step 2: for each candidate (W, H), scale = min(W / w0, H / h0); effective =
    min(floor(w0 * scale) * floor(h0 * scale), w0 * h0); wasted = W * H - effective.
    The largest effective area wins, ties go to the smallest waste."""
    best = None
    best_eff, best_waste = -1, None
    for W, H in candidates:
        scale = min(W / w0, H / h0)
        eff = min(math.floor(w0 * scale) * math.floor(h0 * scale), w0 * h0)
        waste = W * H - eff
        if eff > best_eff or (eff == best_eff and waste < best_waste):
            best, best_eff, best_waste = (W, H), eff, waste
    return best


def merged_side(image_size: int, patch_size: int, downsample: int) -> int:
    """Step 7: h' = w' = ceil(floor(image_size / patch_size) / downsample_ratio)."""
    return -(-(image_size // patch_size) // downsample)


def plan_request(sizes: Sequence[Tuple[int, int]], candidates: Sequence[Tuple[int, int]],
                 patch_size: int, downsample: int) -> List[dict]:
    """Steps 1, 2, 6, 7 for every image (w0, h0) of one request: the chosen
    resolution, the [tw, th] tile grid (width count first) and the placeholder
    count of the image."""
    image_size = candidates[0][0]
    crop = len(sizes) <= MAX_CROP_IMAGES
    hp = merged_side(image_size, patch_size, downsample)
    out = []
    for w0, h0 in sizes:
        best = best_resolution(w0, h0, candidates) if crop else (image_size, image_size)
        tw, th = best[0] // image_size, best[1] // image_size
        out.append({"best": best, "tiles": (tw, th),
                    "slots": _o.tiled_placeholders(hp, hp, tw, th)})
    return out


def expand_prompt(ids: Sequence[int], image_token_id: int, slots: Sequence[int],
                  bos_id: int) -> List[int]:
    """Step 7: BOS first, then the prompt with its i-th image token replaced by
    slots[i] copies of the image token.  The prompt must hold one image token
    per image (ValueError otherwise)."""
    if sum(1 for t in ids if t == image_token_id) != len(slots):
        raise ValueError("image tokens in the prompt differ from the number of images")
    out, i = [bos_id], 0
    for t in ids:
        if t == image_token_id:
            out.extend([image_token_id] * slots[i])
            i += 1
        else:
            out.append(t)
    return out

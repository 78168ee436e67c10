"""Seeded synthetic workloads for the vision-to-language bridge.

This module only draws random numbers and lays out buffers; it holds none of
the bridge's arithmetic (no merge, no projector, no token counting).  Both the
HIP path and the CPU oracle read the tensors it produces.  Where a layout needs
the number of placeholder slots of an image, the caller supplies it.

Draw order for one workload, from one CPU torch.Generator seeded with the
workload's seed: layout randomness (per-image grid sides, then the gap cut
points of the placeholder spans), features, LayerNorm gamma, beta, W1, b1, W2,
b2, newline, separator, text embeddings.

Value distributions:
  features, text embeddings, newline, separator: N(0, 1)
  Linear weights: std fan_in**-0.5; biases: std 0.1 (variance 0.01)
  LayerNorm gamma = 1 + 0.1 N(0,1), beta = 0.1 N(0,1)
bf16 workloads draw in float32 and round to bf16 (round-to-nearest-even).

Token ids for the embedded-sequence entry point come from a second generator
(seed 1000 + workload seed, so the draws above are unchanged): the
token-embedding table [VOCAB][out_dim] ~ N(0, 1), then the text ids, uniform
over [0, VOCAB) without the image token; placeholder positions hold
IMAGE_TOKEN_ID.  VOCAB and IMAGE_TOKEN_ID are the VL2 language config's
vocab_size and image_token_index.

The gradient of a training loss with respect to the sequence (seq_grad) comes
from a third generator (seed 2000 + workload seed): N(0, 1) per element.  The middle
Linears of a deeper projector (mid_weights) come from a fourth (seed 3000 +
workload seed), with the Linear weight and bias distributions above.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence, Tuple

import torch


VOCAB = 102400           # VL2 language config vocab_size
IMAGE_TOKEN_ID = 100015  # VL2 image_token_index


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                       # "f32" or "bf16"
    C: int
    k: int
    hidden: int
    out_dim: int
    seq_len: int
    grids: List[Tuple[int, int]]     # per view, storage order
    views_per_image: List[int]
    has_ln: bool = False
    ln_eps: float = 1e-6
    tiled: bool = False
    tiles: List[Tuple[int, int]] = field(default_factory=list)   # (tw, th) per image
    global_tail: bool = False
    fixed_offset: Optional[int] = None  # one contiguous block at this offset
    grid_choices: Optional[Sequence[int]] = None  # ragged: per-image side drawn from these

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def n_images(self) -> int:
        return len(self.views_per_image)


def config(i: int) -> Workload:
    """The five bridge workloads (0: tiny fp32; 1: MoonViT 2x2 + LN; 2: DeepSeek-ViT
    3x3; 3: VL2 tiled views; 4: ragged 3x3)."""
    if i == 0:
        return Workload("tiny-f32-2x2", 0, "f32", C=64, k=2, hidden=256, out_dim=128, seq_len=40,
                        grids=[(8, 8)], views_per_image=[1], fixed_offset=10)
    if i == 1:
        return Workload("moonvit-2x2-ln", 1, "bf16", C=1152, k=2, hidden=4608, out_dim=4096,
                        seq_len=10240, grids=[(64, 64)] * 8, views_per_image=[1] * 8, has_ln=True)
    if i == 2:
        return Workload("deepseek-vit-3x3", 2, "bf16", C=1024, k=3, hidden=5120, out_dim=5120,
                        seq_len=8192, grids=[(96, 96)] * 4, views_per_image=[1] * 4)
    if i == 3:
        # 16 images x (1 global + 2x3 local) 27x27 views.  The sequence is
        # 24,576 long: 16 tiled images need 22,864 slots, more than 16,384.
        return Workload("vl2-tiled-2x3", 3, "bf16", C=1152, k=2, hidden=2560, out_dim=2560,
                        seq_len=24576, grids=[(27, 27)] * (16 * 7), views_per_image=[7] * 16,
                        tiled=True, tiles=[(2, 3)] * 16)
    if i == 4:
        return Workload("ragged-3x3", 4, "bf16", C=1024, k=3, hidden=5120, out_dim=5120,
                        seq_len=32768, grids=[], views_per_image=[1] * 32,
                        grid_choices=list(range(48, 97, 6)))
    raise ValueError(i)


N_CONFIGS = 5


class Generator:
    """Two-phase draw: layout first (grids), then spans and values."""

    def __init__(self, w: Workload):
        self.w = w
        self.g = torch.Generator("cpu").manual_seed(w.seed)
        if w.grid_choices is not None:
            ch = torch.tensor(list(w.grid_choices))
            idx = torch.randint(0, len(ch), (w.n_images,), generator=self.g)
            w.grids = [(int(ch[j]), int(ch[j])) for j in idx]

    def _randn(self, shape, std=1.0, mean=0.0):
        return torch.randn(shape, generator=self.g, dtype=torch.float32) * std + mean

    def placeholder_mask(self, span_lengths: Sequence[int]) -> torch.Tensor:
        """uint8 [seq_len] mask: image spans in image order, separated by gaps that form
        a uniform random composition of the text positions (stars and bars)."""
        w = self.w
        S = w.seq_len
        n = len(span_lengths)
        total = int(sum(span_lengths))
        text = S - total
        if text < 0:
            raise ValueError(f"{w.name}: {total} placeholder slots do not fit {S} positions")
        mask = torch.zeros(S, dtype=torch.uint8)
        if w.fixed_offset is not None:
            pos = w.fixed_offset
            for L in span_lengths:
                mask[pos:pos + L] = 1
                pos += L
            return mask
        cuts = torch.sort(torch.randperm(text + n, generator=self.g)[:n]).values.tolist()
        gaps, prev = [], -1
        for c in cuts:
            gaps.append(c - prev - 1)
            prev = c
        pos = 0
        for L, gap in zip(span_lengths, gaps):
            pos += gap
            mask[pos:pos + L] = 1
            pos += L
        return mask

    def tensors(self, n_pixels: int, K1: int, span_lengths: Sequence[int]) -> dict:
        """All inputs as CPU tensors.  n_pixels = total pixels over views (sum gh*gw),
        K1 = merged width; both are sizes the caller already knows."""
        w = self.w
        dt = w.torch_dtype
        out = {"mask": self.placeholder_mask(span_lengths)}
        out["features"] = self._randn((n_pixels, w.C)).to(dt)
        if w.has_ln:
            out["ln_gamma"] = self._randn((w.C,), 0.1, 1.0).to(dt)
            out["ln_beta"] = self._randn((w.C,), 0.1).to(dt)
        else:
            out["ln_gamma"] = out["ln_beta"] = None
        out["w1"] = self._randn((w.hidden, K1), K1 ** -0.5).to(dt)
        out["b1"] = self._randn((w.hidden,), 0.1).to(dt)
        out["w2"] = self._randn((w.out_dim, w.hidden), w.hidden ** -0.5).to(dt)
        out["b2"] = self._randn((w.out_dim,), 0.1).to(dt)
        if w.tiled:
            out["newline"] = self._randn((w.out_dim,)).to(dt)
            out["separator"] = self._randn((w.out_dim,)).to(dt)
        else:
            out["newline"] = out["separator"] = None
        out["seq"] = self._randn((w.seq_len, w.out_dim)).to(dt)
        return out


def token_inputs(w: Workload, mask: torch.Tensor, vocab: int = VOCAB,
                 image_token_id: int = IMAGE_TOKEN_ID) -> Tuple[torch.Tensor, torch.Tensor]:
    """(ids int32 [seq_len], embedding table [vocab][out_dim] in the workload dtype):
    image_token_id at the mask's positions, uniform text ids elsewhere."""
    g = torch.Generator("cpu").manual_seed(1000 + w.seed)
    table = torch.randn((vocab, w.out_dim), generator=g, dtype=torch.float32).to(w.torch_dtype)
    ids = torch.randint(0, vocab - 1, (w.seq_len,), generator=g, dtype=torch.int64)
    ids = torch.where(ids >= image_token_id, ids + 1, ids)  # skip the image token
    ids = torch.where(mask.bool(), torch.full_like(ids, image_token_id), ids)
    return ids.to(torch.int32), table


def mid_weights(w: Workload, depth: int):
    """Middle Linears of a depth > 2 projector, [(W [hidden][hidden], b [hidden])] * (depth - 2)
    in the workload dtype: W ~ N(0, 1/hidden), b ~ N(0, 0.01), from a generator seeded
    3000 + the workload seed (the other draws are unchanged)."""
    g = torch.Generator("cpu").manual_seed(3000 + w.seed)
    out = []
    for _ in range(depth - 2):
        W = torch.randn((w.hidden, w.hidden), generator=g, dtype=torch.float32) * w.hidden ** -0.5
        b = torch.randn((w.hidden,), generator=g, dtype=torch.float32) * 0.1
        out.append((W.to(w.torch_dtype), b.to(w.torch_dtype)))
    return out


def seq_grad(w: Workload) -> torch.Tensor:
    """Gradient of a loss with respect to the embedded sequence, [seq_len][out_dim]
    in the workload dtype: N(0, 1) from a generator seeded 2000 + the workload seed
    (the other draws are unchanged)."""
    g = torch.Generator("cpu").manual_seed(2000 + w.seed)
    return torch.randn((w.seq_len, w.out_dim), generator=g, dtype=torch.float32).to(w.torch_dtype)


def make(w: Workload, span_fn: Callable[[Workload], Sequence[int]],
         merged_width: Callable[[Workload], int]) -> dict:
    """Draw a whole workload.  span_fn(w) gives the placeholder slots per image and
    merged_width(w) the first Linear's input width, from whichever planner the
    caller trusts."""
    gen = Generator(w)
    n_pixels = sum(gh * gw for gh, gw in w.grids)
    spans = list(span_fn(w))
    t = gen.tensors(n_pixels, merged_width(w), spans)
    t["spans"] = spans
    return t

"""The largest inputs the 32-bit operand offsets allow, on the GPU.

One 1024 x 910 view of 1152 bf16 channels (2,146,959,360 bytes of features, one
column short of the 2^31 - 1 byte limit pinned in test_host_abi), LayerNorm,
2x2 merge, 4608 -> 4608 -> 4096: the merged operand, the hidden activation and
the features all sit just under 2 GiB, so the last row blocks are addressed
with the largest offsets the buffer loads take.  Features are drawn on the GPU
from a seeded generator (the oracle never sees the whole array).  A token row
depends only on its own 2x2 pixels, so each sampled row is checked against the
oracle run on a 2x2 view of exactly those pixels: the first and last rows, rows
at both ends of the last 256-row blocks, and seeded random rows.  Text rows
around the span must come back untouched.
"""
import numpy as np
import pytest
import torch

import common
from oracle import oracle as o
from patch_merge_mlp_amd import vlbridge as v

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

GH, GW, C, K, HID, OUT = 1024, 910, 1152, 2, 4608, 4096
TEXT_HEAD, TEXT_TAIL = 40, 24


def _weights(seed):
    g = torch.Generator("cpu").manual_seed(seed)
    K1 = C * K * K
    bf = torch.bfloat16
    w1 = (torch.randn(HID, K1, generator=g) * K1 ** -0.5).to(bf)
    b1 = (torch.randn(HID, generator=g) * 0.1).to(bf)
    w2 = (torch.randn(OUT, HID, generator=g) * HID ** -0.5).to(bf)
    b2 = (torch.randn(OUT, generator=g) * 0.1).to(bf)
    gamma = (1 + 0.1 * torch.randn(C, generator=g)).to(bf)
    beta = (0.1 * torch.randn(C, generator=g)).to(bf)
    return w1, b1, w2, b2, gamma, beta


def test_largest_features_operand():
    T = (GH // K) * (GW // K)
    assert GH * GW * C * 2 == 2146959360 < 2 ** 31 - 1
    p = v.projector(v.BF16, C, K, HID, OUT, has_ln=True)
    b = v.Batch([(GH, GW)], [1])
    assert v.vlb_num_tokens(p, b) == T
    gdev = torch.Generator(device="cuda").manual_seed(4242)
    feats = torch.randn(GH * GW, C, device=DEV, generator=gdev).to(torch.bfloat16)
    w1, b1, w2, b2, gamma, beta = _weights(4243)
    weights = v.Weights(*(x.to(DEV) for x in (w1, b1, w2, b2, gamma, beta)))
    br = v.Bridge(p, weights)
    S = TEXT_HEAD + T + TEXT_TAIL
    mask = torch.zeros(S, dtype=torch.uint8)
    mask[TEXT_HEAD:TEXT_HEAD + T] = 1
    seq = torch.full((S, OUT), 3.0, dtype=torch.bfloat16, device=DEV)
    print(f"largest operand case: T={T}, seq_len={S}", flush=True)
    ws = br.fused(b, feats, None, None, mask.to(DEV), seq)
    assert v.vlb_check(ws) == v.OK

    last_block = (T - 1) // 256 * 256
    rng = np.random.default_rng(7)
    rows = sorted({0, 255, 256, last_block - 256, last_block - 1, last_block, T - 2, T - 1,
                   *rng.integers(0, T, 24).tolist()})
    wp = GW // K
    f3 = feats.view(GH, GW, C)
    spec = o.Spec(grids=[(K, K)], C=C, k=K, hidden=HID, out_dim=OUT, has_ln=True,
                  views_per_image=[1])
    got, ref = [], []
    for r in rows:
        ty, tx = divmod(r, wp)
        px = f3[K * ty:K * ty + K, K * tx:K * tx + K].reshape(K * K, C).cpu()
        ref.append(o.project_rows(spec, px, gamma, beta, w1, b1, w2, b2)[0])
        got.append(seq[TEXT_HEAD + r].double().cpu().numpy())
    got, ref = np.array(got), np.array(ref)
    err = common.rel_frob(got, ref)
    print(f"sampled rows {len(rows)}, rel err {err:.3e}")
    assert err <= 1e-2
    per_row = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert per_row.max() <= 2e-2, per_row.max()
    text = torch.cat([seq[:TEXT_HEAD], seq[TEXT_HEAD + T:]]).cpu()
    assert torch.equal(text, torch.full_like(text, 3.0))

"""The embedded-sequence entry point (vlb_bridge_embed) against the oracle.

Every row of the sequence is written: text positions take their row of the
token-embedding table (bit for bit), image-token positions take the bridge's
rows (within the bf16 / fp32 tolerance of the fused call's tests, and bit for
bit equal to vlb_bridge_fused's rows).  Device-detected errors write nothing.
"""
import numpy as np
import pytest
import torch

import common
from oracle import oracle as o
from patch_merge_mlp_amd import vlbridge as v
from patch_merge_mlp_amd import workloads as wl
from test_gpu_parity import TOL, _dev, _weights, full, small_workloads

pytestmark = pytest.mark.gpu
IMG = wl.IMAGE_TOKEN_ID


def run_embed(w, t, ids, table, seq0=None):
    p, b = common.lib_projector(w), common.lib_batch(w)
    br = v.Bridge(p, _weights(t))
    g = common.Guards()
    seq = g.like(seq0 if seq0 is not None
                 else torch.zeros(len(ids), w.out_dim, dtype=w.torch_dtype), "seq")
    ws = g.workspace(v.vlb_workspace_bytes(br.p, b, seq.shape[0]))
    v.vlb_bridge_embed(br.p, b, _dev(t["features"]), br.w, _dev(t["newline"]),
                       _dev(t["separator"]), _dev(ids), IMG, _dev(table), seq, ws)
    st = v.vlb_check(ws)
    g.check()
    return st, seq.cpu()


def oracle_embed(w, t, ids, table, rows64):
    spec = common.oracle_spec(w)
    return o.embed_scatter(o.assemble(spec), rows64, t["newline"], t["separator"], ids, IMG,
                           table, w.out_dim)


@pytest.mark.parametrize("w", [small_workloads()[i] for i in (0, 2, 5, 7)], ids=lambda w: w.name)
def test_small_embed_vs_oracle(w):
    t = common.draw(w)
    ids, table = wl.token_inputs(w, t["mask"])
    rows = o.project_rows(common.oracle_spec(w), t["features"], t["ln_gamma"], t["ln_beta"],
                          t["w1"], t["b1"], t["w2"], t["b2"])
    st_ref, ref = oracle_embed(w, t, ids, table, rows)
    assert st_ref == 0
    st, out = run_embed(w, t, ids, table)
    assert st == v.OK
    text = (ids != IMG).numpy()
    got = out.double().numpy()
    assert np.array_equal(got[text], ref[text]), "text rows differ from the table"
    errs, pos, j = [], np.flatnonzero(~text), 0
    for n in t["spans"]:
        errs.append(common.rel_frob(got[pos[j:j + n]], ref[pos[j:j + n]]))
        j += n
    assert max(errs) <= TOL[w.dtype], errs


@pytest.mark.parametrize("i", [1, 3])
def test_full_embed(i):
    """Full-size workloads: text rows are the table's rows (oracle), image-token rows
    are the fused call's rows bit for bit."""
    w, t = full(i)
    ids, table = wl.token_inputs(w, t["mask"])
    st, out = run_embed(w, t, ids, table)
    assert st == v.OK
    # text rows against the oracle (visual rows zero there: only text compared)
    T = v.vlb_num_tokens(common.lib_projector(w), common.lib_batch(w))
    st_ref, ref = oracle_embed(w, t, ids, table, np.zeros((T, w.out_dim)))
    assert st_ref == 0
    text = (ids != IMG).numpy()
    assert np.array_equal(out.double().numpy()[text], ref[text])
    # image-token rows: the fused call's bits
    p, b = common.lib_projector(w), common.lib_batch(w)
    br = v.Bridge(p, _weights(t))
    seq = _dev(t["seq"]).clone()
    br.fused(b, _dev(t["features"]), _dev(t["newline"]), _dev(t["separator"]), _dev(t["mask"]),
             seq)
    img = ~text
    assert torch.equal(out[torch.from_numpy(img)].view(torch.int16),
                       seq.cpu()[torch.from_numpy(img)].view(torch.int16))


@pytest.mark.parametrize("wi", [0, 2, 7])
@pytest.mark.parametrize("fault", ["id_past_vocab", "negative_id", "extra_placeholder",
                                   "missing_placeholder"])
def test_embed_errors_write_nothing(wi, fault):
    w = small_workloads()[wi]
    t = common.draw(w)
    ids, table = wl.token_inputs(w, t["mask"])
    ids = ids.clone()
    text_pos = np.flatnonzero((ids != IMG).numpy())
    img_pos = np.flatnonzero((ids == IMG).numpy())
    if fault == "id_past_vocab":
        ids[text_pos[3]] = wl.VOCAB
    elif fault == "negative_id":
        ids[text_pos[-1]] = -5
    elif fault == "extra_placeholder":
        ids[text_pos[0]] = IMG
    else:
        ids[img_pos[len(img_pos) // 2]] = 7
    seq0 = t["seq"]
    st, out = run_embed(w, t, ids, table, seq0=seq0)
    want = v.ERR_TOKEN_ID if fault in ("id_past_vocab", "negative_id") else v.ERR_MASK_COUNT
    assert st == want
    assert torch.equal(out.view(torch.int16), seq0.view(torch.int16)), "sequence was modified"


def test_embed_text_only():
    """No images: the whole sequence comes from the table."""
    w = small_workloads()[0]
    t = common.draw(w)
    ids, table = wl.token_inputs(w, torch.zeros(w.seq_len, dtype=torch.uint8))
    p = common.lib_projector(w)
    b = v.Batch([], [])
    seq = torch.zeros(w.seq_len, w.out_dim, dtype=w.torch_dtype, device="cuda")
    ws = v.workspace(p, b, w.seq_len)
    v.vlb_bridge_embed(p, b, None, None, None, None, _dev(ids), IMG, _dev(table), seq, ws)
    assert v.vlb_check(ws) == v.OK
    st, ref = o.embed_scatter(np.zeros(0, np.int64), np.zeros((0, w.out_dim)), None, None, ids,
                              IMG, table, w.out_dim)
    assert st == 0 and np.array_equal(seq.cpu().double().numpy(), ref)


def test_planned_request_end_to_end():
    """Processor planning -> prompt expansion -> tiled batch -> the embedded
    sequence, against the oracle's planner and embedded sequence."""
    from oracle import processor as pr
    cands = [(56, 56), (112, 56), (56, 112), (112, 112), (168, 56)]
    pc = v.Processor(cands, 14, 2)
    sizes = [(130, 47), (60, 61)]
    tiles, slots = v.vlb_plan_request(pc, sizes)
    assert [p["tiles"] for p in pr.plan_request(sizes, cands, 14, 2)] == tiles
    b = v.batch_for_request(pc, tiles)
    grids, vpi = b.grids, b.views_per_image
    w = wl.Workload("planned-2img", 31, "bf16", C=64, k=2, hidden=128, out_dim=64,
                    seq_len=sum(slots) + 40, grids=grids, views_per_image=vpi, tiled=True,
                    tiles=tiles)
    t = common.draw(w)
    _, table = wl.token_inputs(w, t["mask"])
    g = torch.Generator().manual_seed(5)
    text = torch.randint(0, IMG, (39,), generator=g).tolist()
    prompt = text[:10] + [IMG] + text[10:25] + [IMG] + text[25:]
    ids = torch.tensor(v.vlb_expand_prompt(prompt, IMG, 1, slots), dtype=torch.int32)
    assert ids.tolist() == pr.expand_prompt(prompt, IMG, slots, 1) and len(ids) == w.seq_len
    st, out = run_embed(w, t, ids, table)
    assert st == v.OK
    rows = o.project_rows(common.oracle_spec(w), t["features"], t["ln_gamma"], t["ln_beta"],
                          t["w1"], t["b1"], t["w2"], t["b2"])
    st_ref, ref = oracle_embed(w, t, ids, table, rows)
    assert st_ref == 0
    text_pos = (ids != IMG).numpy()
    got = out.double().numpy()
    assert np.array_equal(got[text_pos], ref[text_pos])
    assert common.rel_frob(got[~text_pos], ref[~text_pos]) <= TOL["bf16"]

"""The library's request planner (vlb_select_resolution, vlb_plan_request,
vlb_expand_prompt; host only) against the processor oracle, integer for integer.

Candidate lists are synthetic: whole-tile grids (a x b tiles, a*b <= 9) of three
tile sizes, shuffled, some with repeated entries (full ties); image sizes are
uniform over 1..4096 per side plus extreme aspect ratios and exact tile
multiples.  The fp64 best-fit decision is taken identically on both sides.
"""
import random

import pytest

from oracle import processor as pr
from patch_merge_mlp_amd import vlbridge as v


def candidate_lists(seed, n):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        s = rng.choice([384, 336, 448])
        grid = [(a * s, b * s) for a in range(1, 10) for b in range(1, 10) if a * b <= 9]
        c = rng.sample(grid, rng.randint(1, len(grid)))
        if rng.random() < 0.3:  # duplicates: full ties
            c += rng.sample(c, rng.randint(1, len(c)))
            rng.shuffle(c)
        if c[0][0] != s:  # image_size is the first candidate's width
            c.insert(0, (s, s))
        out.append(c)
    return out


def image_sizes(rng, n):
    sizes = [(rng.randint(1, 4096), rng.randint(1, 4096)) for _ in range(n)]
    sizes += [(1, 4096), (4096, 1), (1, 1), (384, 384), (768, 384), (1152, 1152), (737, 738)]
    return sizes


@pytest.mark.parametrize("seed", range(4))
def test_best_fit_matches_oracle(seed):
    rng = random.Random(100 + seed)
    for cands in candidate_lists(seed, 25):
        pc = v.Processor(cands, 14, 2)
        for w0, h0 in image_sizes(rng, 40):
            assert v.vlb_select_resolution(pc, w0, h0) == pr.best_resolution(w0, h0, cands), \
                (cands, w0, h0)


@pytest.mark.parametrize("patch,k", [(14, 2), (16, 2), (14, 3), (16, 1)])
def test_plan_request_matches_oracle(patch, k):
    rng = random.Random(patch * 10 + k)
    for cands in candidate_lists(patch + k, 20):
        pc = v.Processor(cands, patch, k)
        for n_img in (1, 2, 3, 5):
            sizes = [(rng.randint(1, 3000), rng.randint(1, 3000)) for _ in range(n_img)]
            tiles, slots = v.vlb_plan_request(pc, sizes)
            want = pr.plan_request(sizes, cands, patch, k)
            assert tiles == [p["tiles"] for p in want]
            assert slots == [p["slots"] for p in want]
            # the planned batch assembles exactly that many slots
            b = v.batch_for_request(pc, tiles)
            p = v.projector(v.BF16, 64, k, 64, 64)
            assert v.vlb_image_slots(p, b) == slots


def test_page_counts():
    pc = v.Processor([(384, 384), (768, 384), (384, 768)], 14, 2)
    assert v.vlb_plan_request(pc, [(384, 384), (800, 400)]) == ([(1, 1), (2, 1)], [421, 617])
    assert v.vlb_plan_request(v.Processor([(384, 384)], 16, 2), [(640, 480)])[1] == [313]
    # three images: no cropping
    assert v.vlb_plan_request(pc, [(800, 400)] * 3) == ([(1, 1)] * 3, [421] * 3)


def test_expand_prompt_matches_oracle():
    rng = random.Random(7)
    img, bos = 100015, 100000
    for _ in range(50):
        n_img = rng.randint(0, 4)
        slots = [rng.randint(1, 700) for _ in range(n_img)]
        ids = [rng.randint(0, 99999) for _ in range(rng.randint(0, 60))]
        for _ in range(n_img):
            ids.insert(rng.randint(0, len(ids)), img)
        assert v.vlb_expand_prompt(ids, img, bos, slots) == pr.expand_prompt(ids, img, slots, bos)


def test_planner_errors():
    L = v.lib()
    pc = v.Processor([(384, 384), (500, 384)], 14, 2)  # 500 is not a whole tile
    with pytest.raises(v.VlbError) as e:
        v.vlb_select_resolution(pc, 100, 100)
    assert e.value.status == v.ERR_SHAPE
    good = v.Processor([(384, 384)], 14, 2)
    for w0, h0 in ((0, 5), (5, -1)):
        with pytest.raises(v.VlbError):
            v.vlb_select_resolution(good, w0, h0)
    with pytest.raises(v.VlbError):
        v.vlb_select_resolution(v.Processor([(8, 8)], 14, 2), 10, 10)  # tile below one patch
    assert L.vlb_select_resolution(None, 1, 1, None) == v.ERR_NULL
    img = 9
    for ids, slots in (([1, 2], [3]), ([img, img], [3])):
        with pytest.raises(v.VlbError) as e:
            v.vlb_expand_prompt(ids, img, 0, slots)
        assert e.value.status == v.ERR_SHAPE
    import ctypes as ct
    ids = (ct.c_int32 * 2)(img, 5)
    sl = (ct.c_int64 * 1)(4)
    out = (ct.c_int32 * 3)()
    assert L.vlb_expand_prompt(ids, 2, img, 0, sl, 1, out, 3) == -v.ERR_SHAPE  # needs 6
    assert L.vlb_expand_prompt(ids, 2, img, 0, sl, 1, None, 0) == 6

"""Pins of the oracle's layout steps (offsets from splits, routing, gather,
combine): hand-worked cases (tests/golden/route_hand.json, one of them the
offsets of PyTorch issue #152668's reproduction), and invariants on random
routings -- every kept slot lands on exactly one row, an expert's rows hold
its slots in ascending order then padding, sizes are padded as defined, the
offsets equal offsets_from_splits of the counts, and gather followed by an
unweighted topk = 1 combine returns the input.  The gather and the weighted
combine at topk = 2 and 3, with dropped slots and padding rows, are pinned by
hand-worked values (tests/golden/gather_hand.json)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_hand.json")


def cases():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("i", range(3))
def test_route_hand_worked(i):
    c = cases()["route"][i]
    offs, row_slot, slot_row = oracle.route(c["expert_of_slot"], c["num_groups"], c["align"], c["pad_empty"])
    assert offs.tolist() == c["offs"]
    assert row_slot.tolist() == c["row_slot"]
    assert slot_row.tolist() == c["slot_row"]


@pytest.mark.parametrize("i", range(4))
def test_offsets_from_splits_hand_worked(i):
    c = cases()["offsets_from_splits"][i]
    assert oracle.offsets_from_splits(c["splits"], c["align"], c["pad_empty"]).tolist() == c["offs"]


@pytest.mark.parametrize("seed,e,tokens,topk,align,pad_empty", [
    (1, 8, 50, 2, 1, False), (2, 16, 40, 4, 8, True), (3, 5, 30, 3, 16, False), (4, 64, 20, 8, 4, True)])
def test_route_invariants(seed, e, tokens, topk, align, pad_empty):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, e + 1, size=(tokens, topk))        # includes dropped ids -1 and e
    offs, row_slot, slot_row = oracle.route(ids, e, align, pad_empty)
    flat = ids.reshape(-1)
    kept = (flat >= 0) & (flat < e)
    assert np.all(slot_row[~kept] == -1)
    assert sorted(row_slot[row_slot >= 0].tolist()) == np.flatnonzero(kept).tolist()
    for s in np.flatnonzero(kept):
        assert row_slot[slot_row[s]] == s
    counts = np.bincount(flat[kept], minlength=e)
    assert offs.tolist() == oracle.offsets_from_splits(counts, align, pad_empty).tolist()
    start = 0
    for g in range(e):
        seg = row_slot[start:offs[g]]
        mine = np.flatnonzero(flat == g)
        assert seg[:len(mine)].tolist() == mine.tolist()
        assert np.all(seg[len(mine):] == -1)
        size = offs[g] - start
        assert size % align == 0 and (size >= align or not pad_empty)
        start = offs[g]


def test_gather_then_combine_is_identity():
    rng = np.random.default_rng(9)
    tokens, e = 23, 6
    ids = rng.integers(0, e, size=(tokens, 1))
    x = (rng.standard_normal((tokens, 16)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    offs, row_slot, slot_row = oracle.route(ids, e, 8, True)
    g = oracle.gather_rows(x, row_slot, 1)
    assert np.all(g[row_slot < 0] == 0)
    back = oracle.combine_rows(g, slot_row, 1)
    assert np.array_equal(back.value, oracle.decode_bf16(x))


def test_combine_weighted_brute_force():
    y = (np.arange(12, dtype=np.float32).reshape(6, 2) / 4).view(np.uint32) >> 16
    y = y.astype(np.uint16)
    slot_row = np.array([0, 3, -1, 5, 2, 2])
    w = np.array([[0.5, 2.0], [1.0, -1.0], [0.25, 0.25]], dtype=np.float32)
    r = oracle.combine_rows(y, slot_row, 2, w)
    yd = oracle.decode_bf16(y)
    want = np.stack([0.5 * yd[0] + 2.0 * yd[3], -1.0 * yd[5], 0.25 * yd[2] + 0.25 * yd[2]])
    assert np.array_equal(r.value, want)


# ---- gather and combine at topk > 1 (hand-worked) --------------------------------
# A row's token is its slot // topk; a mapping by the slot itself, or by
# slot % topk, gathers other rows (or runs off the source) and fails these.

GATHER_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gather_hand.json")


def gather_cases():
    with open(GATHER_GOLDEN) as f:
        return json.load(f)["cases"]


def _bits(v):
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("i", range(3))
def test_gather_hand_worked(i):
    c = gather_cases()[i]
    offs, row_slot, slot_row = oracle.route(c["expert_of_slot"], c["num_groups"], c["align"], c["pad_empty"])
    assert offs.tolist() == c["offs"]
    assert row_slot.tolist() == c["row_slot"]
    assert slot_row.tolist() == c["slot_row"]
    got = oracle.gather_rows(_bits(c["src"]), row_slot, c["topk"])
    assert np.array_equal(got, _bits(c["gathered"]))


@pytest.mark.parametrize("i", range(3))
def test_combine_hand_worked(i):
    c = gather_cases()[i]
    r = oracle.combine_rows(_bits(c["gathered"]), np.array(c["slot_row"]), c["topk"],
                            np.array(c["weights"], dtype=np.float32))
    assert np.array_equal(r.value, np.array(c["combined"], dtype=np.float64))


@pytest.mark.parametrize("seed,topk", [(11, 2), (12, 3), (13, 8)])
def test_gather_brute_force_distinct_tokens(seed, topk):
    """Every token row is distinct (its first column holds the token index),
    so each gathered row names the token it came from: that must be the
    slot's token for kept slots, and the row is zero for padding."""
    rng = np.random.default_rng(seed)
    tokens, e = 37, 5
    ids = rng.integers(-1, e + 1, size=(tokens, topk))
    src = np.zeros((tokens, 4), dtype=np.float32)
    src[:, 0] = np.arange(tokens) + 1
    src[:, 1:] = rng.standard_normal((tokens, 3))
    offs, row_slot, slot_row = oracle.route(ids, e, 4, True)
    g = oracle.gather_rows(_bits(src), row_slot, topk)
    back = oracle.decode_bf16(g)
    for r, s in enumerate(row_slot):
        if s < 0:
            assert np.all(g[r] == 0)
        else:
            assert back[r, 0] == s // topk + 1
            assert np.array_equal(g[r], _bits(src[s // topk]))

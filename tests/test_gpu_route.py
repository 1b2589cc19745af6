"""GPU parity of the layout steps (gg_offsets_from_splits, gg_route,
gg_gather_rows, gg_combine_rows) against the oracle: integer outputs bit for
bit (offsets, the row of every slot, the slot of every row), gathered rows
bit for bit with untouched rows past the last offset, the combine within the
fp32 tolerance, and a whole routed layer: route -> gather -> grouped forward
-> combine, each stage against the oracle."""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from moe_grouped_gemm_ragged_amd import synth
from gpu_util import device, host, say
from parity import Report, check

pytestmark = pytest.mark.gpu


def routing(seed, tokens, topk, e, dropped=0.0):
    """Top-k distinct experts per token from softmax-skewed scores, with a
    fraction of slots set to an out-of-range id (dropped)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal(e) * 1.5
    p = np.exp(logits) / np.exp(logits).sum()
    ids = np.stack([rng.choice(e, size=topk, replace=False, p=p) for _ in range(tokens)]) if tokens else \
        np.zeros((0, topk), dtype=np.int64)
    if dropped:
        mask = rng.random(ids.shape) < dropped
        ids = np.where(mask, np.where(rng.random(ids.shape) < 0.5, -1, e), ids)
    return ids.astype(np.int32)


CASES = [(1, 4096, 8, 128, 8, True, 0.0), (2, 3000, 6, 64, 16, False, 0.05),
         (3, 1, 1, 2048, 1, False, 0.0), (4, 70000, 2, 256, 8, True, 0.0),
         (5, 0, 4, 16, 8, True, 0.0), (6, 2500, 4, 2048, 4, False, 0.01)]


@pytest.mark.parametrize("seed,tokens,topk,e,align,pad_empty,dropped", CASES)
def test_route_bit_exact(seed, tokens, topk, e, align, pad_empty, dropped):
    dev = device()
    import torch
    ids = routing(seed, tokens, topk, e, dropped)
    say("route", seed, tokens, topk, e, align, pad_empty)
    offs, row_slot, slot_row = gg.route(torch.from_numpy(ids).to(dev), e, align, pad_empty)
    torch.cuda.synchronize()
    ro, rr, rs = oracle.route(ids, e, align, pad_empty)
    assert offs.cpu().numpy().tolist() == ro.tolist()
    used = int(ro[-1])
    assert row_slot[:used].cpu().numpy().tolist() == rr.tolist()
    assert slot_row.cpu().numpy().tolist() == rs.tolist()


@pytest.mark.parametrize("e,align,pad_empty", [(32, 1, False), (2048, 8, True), (100, 16, False)])
def test_offsets_from_splits_bit_exact(e, align, pad_empty):
    dev = device()
    import torch
    rng = np.random.default_rng(e + align)
    splits = rng.integers(-3, 400, size=e)
    splits[rng.choice(e, size=max(1, e // 10), replace=False)] = 0
    say("offsets_from_splits", e, align, pad_empty)
    offs = gg.offsets_from_splits(torch.from_numpy(splits).to(dev), align, pad_empty)
    torch.cuda.synchronize()
    assert offs.cpu().numpy().tolist() == oracle.offsets_from_splits(splits, align, pad_empty).tolist()


@pytest.mark.parametrize("dtype", ["bf16", "u8"])
def test_gather_rows_bit_exact(dtype):
    dev = device()
    import torch
    tokens, topk, e, k = 1500, 4, 40, 272
    ids = routing(7, tokens, topk, e, 0.02)
    offs, row_slot, slot_row = gg.route(torch.from_numpy(ids).to(dev), e, 8, True)
    if dtype == "bf16":
        x = torch.randn((tokens, k), device=dev).to(torch.bfloat16)
        sent = torch.full((row_slot.shape[0], k), -7.0, device=dev).to(torch.bfloat16)
    else:
        x = torch.randint(0, 256, (tokens, k), device=dev, dtype=torch.uint8)
        sent = torch.full((row_slot.shape[0], k), 0xA5, device=dev, dtype=torch.uint8)
    say("gather_rows", dtype)
    gg.gather_rows(x, row_slot, topk, offs, out=sent)
    torch.cuda.synchronize()
    used = int(offs[-1].item())
    xb = x.view(torch.int16) if dtype == "bf16" else x
    got = (sent.view(torch.int16) if dtype == "bf16" else sent).cpu().numpy()
    want = oracle.gather_rows(xb.cpu().numpy(), row_slot[:used].cpu().numpy(), topk)
    assert np.array_equal(got[:used], want)
    rest = got[used:]
    fill = np.int16(np.array([-7.0], dtype=np.float32).view(np.uint32)[0] >> 16) if dtype == "bf16" else 0xA5
    assert np.all(rest == fill), "rows past the last offset were written"


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_combine_rows(out):
    dev = device()
    import torch
    tokens, topk, e, n = 2000, 8, 64, 528
    ids = routing(8, tokens, topk, e, 0.03)
    offs, row_slot, slot_row = gg.route(torch.from_numpy(ids).to(dev), e, 16, False)
    y = torch.randn((row_slot.shape[0], n), device=dev).to(torch.bfloat16)
    w = torch.rand((tokens, topk), device=dev, dtype=torch.float32)
    say("combine_rows", out)
    o = gg.combine_rows(y, slot_row, topk, w, out_dtype={"bf16": torch.bfloat16, "f32": torch.float32}[out])
    torch.cuda.synchronize()
    ref = oracle.combine_rows(synth.bf16_bits(y), slot_row.cpu().numpy(), topk, w.cpu().numpy())
    check(host(o), ref.value, ref.sabs, topk, f"combine {out}")


def test_routed_layer_end_to_end():
    """x -> route (min_alignment 16, empty experts padded) -> gather ->
    grouped forward on the padded offsets -> weighted combine."""
    dev = device()
    import torch
    tokens, topk, e, k, n = 3000, 8, 128, 512, 384
    ids = routing(9, tokens, topk, e, 0.0)
    ids[:, 0] = np.where(ids[:, 0] == 5, 6, ids[:, 0])      # make expert 5 rarer
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    x = torch.randn((tokens, k), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((e, k, n), generator=g, device=dev) * 0.05).to(torch.bfloat16)
    probs = torch.rand((tokens, topk), generator=g, device=dev)
    say("routed layer")
    offs, row_slot, slot_row = gg.route(torch.from_numpy(ids).to(dev), e, 16, True)
    xg = gg.gather_rows(x, row_slot, topk, offs)
    y = gg.forward(xg, w, offs)
    out = gg.combine_rows(y, slot_row, topk, probs)
    torch.cuda.synchronize()
    ro, rr, rs = oracle.route(ids, e, 16, True)
    used = int(ro[-1])
    xg_ref = oracle.gather_rows(synth.bf16_bits(x), rr, topk)
    assert np.array_equal(synth.bf16_bits(xg)[:used], xg_ref)
    ref = oracle.forward(xg_ref, synth.bf16_bits(w), ro.astype(np.int32))
    yb = synth.bf16_bits(y)[:used]
    check(yb, ref.value, ref.sabs, k, "routed forward")
    cref = oracle.combine_rows(yb, rs, topk, probs.cpu().numpy())
    check(synth.bf16_bits(out), cref.value, cref.sabs, topk, "routed combine")


def test_offsets_from_splits_saturate_at_the_row_limit():
    """Counts whose running sum passes 2^31 - 2^16 (the GEMMs' row limit)
    give offsets saturated there, never int32 wrap-around: the oracle's sums
    capped at the limit, bit for bit, and still monotone."""
    dev = device()
    import torch
    cap = (1 << 31) - (1 << 16)
    splits = np.array([5, 1 << 30, (1 << 30) - 7, 1 << 20, 3, 1 << 40, 0, 9], dtype=np.int64)
    say("offsets_from_splits saturation")
    got = gg.offsets_from_splits(torch.from_numpy(splits).to(dev), 8, True)
    torch.cuda.synchronize()
    want = np.minimum(oracle.offsets_from_splits(splits, 8, True), cap)
    g = got.cpu().numpy().astype(np.int64)
    assert g.tolist() == want.tolist()
    assert np.all(np.diff(g) >= 0)

"""gg_route_noalloc (routing with its histograms in the library's fixed
per-GPU scratch array, for callers that cannot allocate) against gg_route
with a caller workspace, through the C ABI: offsets, the slot of every row
and the row of every slot bit for bit, on two calls in a row, the second
with a smaller input (fewer slots and experts), so stale scratch contents
from the first call cannot leak into the second.  Both are also checked
against the oracle's routing."""
import numpy as np
import pytest

import oracle
from moe_grouped_gemm_ragged_amd import binding as gg
from gpu_util import device, say

pytestmark = pytest.mark.gpu


def _ids(seed, tokens, topk, e):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, e, size=(tokens, topk)).astype(np.int32)
    drop = rng.random(ids.shape) < 0.02
    return np.where(drop, -1, ids).astype(np.int32)


def _run(name, ids_d, slots, e, align, pad, cap, ws=None):
    import torch
    dev = ids_d.device
    offs = torch.full((e,), -7, dtype=torch.int32, device=dev)
    row_slot = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    slot_row = torch.full((max(slots, 1),), -7, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    if ws is None:
        rc = gg.call_raw(name, ids_d.data_ptr(), slots, e, align, pad, offs.data_ptr(), row_slot.data_ptr(), cap,
                         slot_row.data_ptr(), st)
    else:
        rc = gg.call_raw(name, ids_d.data_ptr(), slots, e, align, pad, offs.data_ptr(), row_slot.data_ptr(), cap,
                         slot_row.data_ptr(), ws.data_ptr(), st)
    assert rc == 0, (name, rc, gg.last_error())
    return offs, row_slot, slot_row


@pytest.mark.parametrize("first,second", [((21, 8192, 8, 128, 16, 1), (22, 3000, 4, 40, 8, 0))])
def test_route_noalloc_matches_route(first, second):
    import torch
    dev = device()
    for seed, tokens, topk, e, align, pad in (first, second):
        ids = _ids(seed, tokens, topk, e)
        ids_d = torch.from_numpy(ids).to(dev)
        slots = tokens * topk
        cap = gg.route_rows_bound(slots, e, align)
        ws = torch.empty(int(gg.load().gg_route_workspace_bytes(slots, e)), dtype=torch.uint8, device=dev)
        say("route with workspace", seed, tokens, topk, e)
        ref = _run("gg_route", ids_d, slots, e, align, pad, cap, ws)
        say("route_noalloc", seed, tokens, topk, e)
        got = _run("gg_route_noalloc", ids_d, slots, e, align, pad, cap)
        torch.cuda.synchronize()
        ro, rr, rs = oracle.route(ids, e, align, bool(pad))
        used = int(ro[-1])
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        assert got[0].cpu().numpy().tolist() == ro.tolist()
        assert got[1][:used].cpu().numpy().tolist() == rr.tolist()
        assert got[2].cpu().numpy().tolist() == rs.tolist()
        assert torch.all(got[1][used:] == -7), "rows past the last offset were written"

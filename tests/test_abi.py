"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/gg.h declares, and rejects bad arguments with the
documented status before touching the HIP runtime."""
import ctypes
import re

import pytest

from moe_grouped_gemm_ragged_amd import binding as gg

ENTRY = ["gg_forward", "gg_dgrad", "gg_wgrad", "gg_masked_forward", "gg_masked_dgrad", "gg_masked_wgrad"]


@pytest.fixture(scope="module")
def lib():
    return gg.load()


def test_header_declares_the_four_passes():
    syms = gg.header_symbols()
    for name in ENTRY + ["gg_status_str", "gg_last_error", "gg_version"]:
        assert name in syms


def test_library_exports_every_header_symbol(lib):
    for name in gg.header_symbols():
        assert hasattr(lib, name), f"libgg.so does not export {name}"


def test_no_torch_types_in_header():
    with open(gg.header_path()) as f:
        text = f.read()
    assert "torch" not in re.sub(r"/\*.*?\*/", "", text, flags=re.S)


def test_status_strings(lib):
    for code, name in gg.STATUS.items():
        assert lib.gg_status_str(code).decode().startswith(name)
    assert lib.gg_version().decode().startswith("gg ")


# Fake but 16-byte aligned device addresses: every case below must be
# rejected by the host checks, so nothing is ever dereferenced or launched.
A = 0x10000
OK = dict(a=A, b=A + 0x100, g=A + 0x200, c=A + 0x300, dt=0, m=64, k=64, n=64, e=4, s=0)


def call(name, **kw):
    v = dict(OK, **kw)
    return gg.call_raw(name, v["a"], v["b"], v["g"], v["c"], v["dt"], v["m"], v["k"], v["n"],
                       v["e"], v["s"])


@pytest.mark.parametrize("name", ENTRY)
@pytest.mark.parametrize("case,status", [
    (dict(a=0), 1), (dict(b=0), 1), (dict(g=0), 1), (dict(c=0), 1),
    (dict(m=-1), 2), (dict(k=0), 2), (dict(n=0), 2), (dict(k=12), 2), (dict(n=20), 2),
    (dict(k=(1 << 20) + 8), 2), (dict(m=1 << 31), 2), (dict(m=(1 << 31) - (1 << 16)), 2),
    (dict(a=A + 8), 3), (dict(b=A + 2), 3), (dict(c=A + 4), 3), (dict(g=A + 4), 3),
    (dict(dt=2), 4), (dict(dt=-1), 4),
    (dict(e=0), 5), (dict(e=-3), 5), (dict(e=2049), 5),
])
def test_bad_arguments_rejected_before_launch(lib, name, case, status):
    rc = call(name, **case)
    assert rc == status, (name, case, rc, gg.last_error())
    assert gg.last_error() != ""


@pytest.mark.parametrize("name", ["gg_masked_forward", "gg_masked_dgrad", "gg_masked_wgrad"])
def test_masked_row_limit(lib, name):
    rc = call(name, m=1 << 24, e=256)
    assert rc == 2 and "max_m" in gg.last_error()


def test_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(8, 8, dtype=torch.float32)
    w = torch.zeros(1, 8, 8, dtype=torch.bfloat16)
    offs = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(TypeError):
        gg.forward(x, w, offs)
    with pytest.raises(ValueError):
        gg.forward(torch.zeros(8, 16, dtype=torch.bfloat16), w, offs)


EX_ENTRY = [e + "_ex" for e in ENTRY]


def call_ex(name, alpha=1.0, beta=0.0, **kw):
    v = dict(OK, **kw)
    return gg.call_raw(name, v["a"], v["b"], v["g"], v["c"], v["dt"], v["m"], v["k"], v["n"],
                       v["e"], alpha, beta, v["s"])


@pytest.mark.parametrize("name", EX_ENTRY)
@pytest.mark.parametrize("case,status", [
    (dict(a=0), 1), (dict(c=0), 1), (dict(k=12), 2), (dict(n=0), 2), (dict(c=A + 4), 3),
    (dict(dt=5), 4), (dict(e=0), 5), (dict(e=4096), 5),
])
def test_scaled_entry_points_check_like_the_plain_ones(lib, name, case, status):
    rc = call_ex(name, 0.5, 1.0, **case)
    assert rc == status, (name, case, rc, gg.last_error())


@pytest.mark.parametrize("name", ["gg_forward_silu_mul", "gg_masked_forward_silu_mul"])
@pytest.mark.parametrize("case,status", [
    (dict(a=0), 1), (dict(k=12), 2), (dict(n=24), 2), (dict(c=A + 4), 3), (dict(dt=9), 4),
    (dict(e=0), 5),
])
def test_silu_mul_entry_points_check_arguments(lib, name, case, status):
    rc = call(name, **case)
    assert rc == status, (name, case, rc, gg.last_error())


def test_binding_needs_out_to_accumulate():
    torch = pytest.importorskip("torch")
    x = torch.zeros(8, 8, dtype=torch.bfloat16)
    dy = torch.zeros(8, 8, dtype=torch.bfloat16)
    offs = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError):
        gg.wgrad(x, dy, offs, beta=1.0)


# --------------------------------------------------------------------------
# fp8 entry points: host-side checks only
# --------------------------------------------------------------------------

FP8_OK = dict(x=A, xs=A + 0x100, w=A + 0x200, ws=A + 0x300, g=A + 0x400, c=A + 0x500, dt=0,
              m=64, k=256, n=64, e=4, s=0)


def call_fp8(name, **kw):
    v = dict(FP8_OK, **kw)
    return gg.call_raw(name, v["x"], v["xs"], v["w"], v["ws"], v["g"], v["c"], v["dt"], v["m"],
                       v["k"], v["n"], v["e"], v["s"])


@pytest.mark.parametrize("name", ["gg_fp8_forward", "gg_fp8_masked_forward"])
@pytest.mark.parametrize("case,status", [
    (dict(x=0), 1), (dict(xs=0), 1), (dict(w=0), 1), (dict(ws=0), 1), (dict(g=0), 1), (dict(c=0), 1),
    (dict(k=192), 2), (dict(k=64), 2), (dict(n=20), 2), (dict(m=-1), 2),
    (dict(xs=A + 8), 3), (dict(ws=A + 4), 3), (dict(x=A + 8), 3),
    (dict(dt=3), 4), (dict(e=0), 5), (dict(e=2049), 5),
])
def test_fp8_entry_points_check_arguments(lib, name, case, status):
    rc = call_fp8(name, **case)
    assert rc == status, (name, case, rc, gg.last_error())
    assert gg.last_error() != ""


def test_fp8_masked_row_limit(lib):
    rc = call_fp8("gg_fp8_masked_forward", m=1 << 24, e=256)
    assert rc == 2 and "max_m" in gg.last_error()


@pytest.mark.parametrize("layout,rows,k,e,expect", [
    (0, 1000, 768, 8, (4 + 8) * 6 * 256),       # ragged: ceil(1000/256) + E tiles
    (1, 256, 768, 64, 64 * 1 * 6 * 256),         # masked: E * ceil(max_m/256)
    (2, 2048, 768, 64, 64 * 8 * 6 * 256),        # weights: E * ceil(n/256)
    (2, 300, 128, 2, 2 * 2 * 1 * 256),
])
def test_fp8_scale_bytes(lib, layout, rows, k, e, expect):
    assert gg.fp8_scale_bytes(layout, rows, k, e) == expect


@pytest.mark.parametrize("args", [(3, 64, 128, 1), (0, 64, 100, 1), (0, -1, 128, 1), (0, 64, 128, 0),
                                  (0, (1 << 31) - (1 << 16), 128, 1)])
def test_fp8_scale_bytes_rejects(lib, args):
    assert lib.gg_fp8_scale_bytes(*args) == -1


PACK_OK = dict(layout=0, src=A, f32=1, ld=2, g=A + 0x100, rows=64, k=256, e=4, dst=A + 0x200, bad=0, s=0)


def call_pack(**kw):
    v = dict(PACK_OK, **kw)
    return gg.call_raw("gg_fp8_pack_scales", v["layout"], v["src"], v["f32"], v["ld"], v["g"], v["rows"],
                       v["k"], v["e"], v["dst"], v["bad"] or None, v["s"])


@pytest.mark.parametrize("case,status", [
    (dict(src=0), 1), (dict(dst=0), 1), (dict(g=0), 1), (dict(layout=1, g=0), 1),
    (dict(layout=5), 2), (dict(k=200), 2), (dict(ld=1), 2), (dict(rows=-1), 2),
    (dict(rows=(1 << 31) - (1 << 16)), 2),
    (dict(dst=A + 8), 3), (dict(src=A + 2), 3),
    (dict(e=0), 5),
])
def test_fp8_pack_scales_checks_arguments(lib, case, status):
    rc = call_pack(**case)
    assert rc == status, (case, rc, gg.last_error())


NK_ENTRY = ["gg_forward_nk", "gg_dgrad_nk", "gg_wgrad_nk", "gg_masked_forward_nk"]


@pytest.mark.parametrize("name", NK_ENTRY)
@pytest.mark.parametrize("case,status", [
    (dict(a=0), 1), (dict(g=0), 1), (dict(k=12), 2), (dict(n=20), 2), (dict(m=-1), 2),
    (dict(b=A + 2), 3), (dict(dt=2), 4), (dict(e=0), 5),
])
def test_nk_entry_points_check_arguments(lib, name, case, status):
    rc = call(name, **case)
    assert rc == status, (name, case, rc, gg.last_error())
    rc = call_ex(name + "_ex", 0.5, 1.0, **case)
    assert rc == status, (name + "_ex", case, rc, gg.last_error())


BIAS_OK = dict(a=A, b=A + 0x100, g=A + 0x200, bias=A + 0x300, bs=A + 0x400, c=A + 0x500, dt=0,
               m=64, k=64, n=64, e=4, s=0)


def call_bias(name, **kw):
    v = dict(BIAS_OK, **kw)
    return gg.call_raw(name, v["a"], v["b"], v["g"], v["bias"], v["bs"] or None, v["c"], v["dt"], v["m"],
                       v["k"], v["n"], v["e"], 1.0, 0.0, v["s"])


@pytest.mark.parametrize("name", ["gg_forward_bias", "gg_masked_forward_bias"])
@pytest.mark.parametrize("case,status", [
    (dict(a=0), 1), (dict(bias=0), 1), (dict(c=0), 1), (dict(k=12), 2), (dict(m=-1), 2),
    (dict(bias=A + 8), 3), (dict(bs=A + 2), 3), (dict(dt=2), 4), (dict(e=0), 5),
])
def test_bias_entry_points_check_arguments(lib, name, case, status):
    rc = call_bias(name, **case)
    assert rc == status, (name, case, rc, gg.last_error())


def test_route_sizes(lib):
    assert gg.route_rows_bound(100, 8, 16) == 100 + 8 * 16
    assert lib.gg_route_rows_bound(-1, 8, 1) == -1
    assert lib.gg_route_rows_bound(10, 8, 0) == -1
    assert lib.gg_route_workspace_bytes(4096, 16) == 4 * 16 * 4       # 1024 slots per block
    assert lib.gg_route_workspace_bytes(0, 16) == 16 * 4


@pytest.mark.parametrize("case,status", [
    (dict(ids=0), 1), (dict(offs=0), 1), (dict(ws=0), 1), (dict(e=0), 5), (dict(align=0), 2),
    (dict(align=5000), 2), (dict(cap=90), 2), (dict(slots=-1), 2), (dict(ws=A + 8), 3), (dict(offs=A + 2), 3),
    # the rows it may produce must be acceptable to the GEMMs: below 2^31 - 2^16
    (dict(slots=(1 << 31) - (1 << 16) - 4 * 8, cap=1 << 31), 2),
])
def test_route_checks_arguments(lib, case, status):
    v = dict(ids=A, slots=64, e=4, align=8, pad=1, offs=A + 0x100, rs=A + 0x200, cap=64 + 32, sr=A + 0x300,
             ws=A + 0x400, s=0)
    v.update(case)
    rc = gg.call_raw("gg_route", v["ids"] or None, v["slots"], v["e"], v["align"], v["pad"], v["offs"] or None,
                     v["rs"], v["cap"], v["sr"], v["ws"] or None, v["s"])
    assert rc == status, (case, rc, gg.last_error())


@pytest.mark.parametrize("case,status", [
    (dict(src=0), 1), (dict(rb=24), 2), (dict(topk=0), 2), (dict(src=A + 8), 3), (dict(e=0), 5),
    (dict(cap=(1 << 31) - (1 << 16)), 2), (dict(tokens=1 << 30), 2)])
def test_gather_checks_arguments(lib, case, status):
    v = dict(src=A, tokens=10, rb=32, rs=A + 0x100, topk=2, offs=A + 0x200, e=4, cap=40, dst=A + 0x300, s=0)
    v.update(case)
    rc = gg.call_raw("gg_gather_rows", v["src"] or None, v["tokens"], v["rb"], v["rs"], v["topk"], v["offs"],
                     v["e"], v["cap"], v["dst"], v["s"])
    assert rc == status, (case, rc, gg.last_error())


@pytest.mark.parametrize("case,status", [
    (dict(y=0), 1), (dict(n=12), 2), (dict(topk=0), 2), (dict(out=A + 4), 3), (dict(dt=3), 4),
    (dict(cap=(1 << 31) - (1 << 16)), 2), (dict(tokens=1 << 30), 2)])
def test_combine_checks_arguments(lib, case, status):
    v = dict(y=A, n=64, sr=A + 0x100, w=A + 0x200, topk=2, tokens=10, cap=40, out=A + 0x300, dt=0, s=0)
    v.update(case)
    rc = gg.call_raw("gg_combine_rows", v["y"] or None, v["n"], v["sr"], v["w"], v["topk"], v["tokens"], v["cap"],
                     v["out"], v["dt"], v["s"])
    assert rc == status, (case, rc, gg.last_error())


@pytest.mark.parametrize("name", ["gg_bias_grad", "gg_masked_bias_grad", "gg_bias_scale_grad",
                                  "gg_masked_bias_scale_grad"])
@pytest.mark.parametrize("case,status", [
    (dict(dy=0), 1), (dict(g=0), 1), (dict(o=0), 1), (dict(n=12), 2), (dict(m=-1), 2), (dict(dy=A + 8), 3),
    (dict(e=0), 5)])
def test_bias_grad_entry_points_check_arguments(lib, name, case, status):
    v = dict(dy=A, g=A + 0x100, x=A + 0x200, o=A + 0x300, m=64, n=64, e=4, s=0)
    v.update(case)
    rc = gg.call_raw(name, v["dy"] or None, v["g"] or None, v["x"], v["o"] or None, v["m"], v["n"], v["e"], v["s"])
    assert rc == status, (name, case, rc, gg.last_error())


@pytest.mark.parametrize("name", ENTRY)
def test_weight_size_limit(lib, name):
    # one expert's k x n weights must stay under 4 GiB (k * n < 2^31)
    rc = call(name, k=65536, n=32768)
    assert rc == 2 and "k * n" in gg.last_error(), (name, rc, gg.last_error())


@pytest.mark.parametrize("case,status", [
    (dict(ids=0), 1), (dict(offs=0), 1), (dict(e=0), 5), (dict(align=0), 2), (dict(cap=90), 2),
    (dict(slots=-1), 2), (dict(offs=A + 2), 3),
    # histograms beyond the fixed scratch array: rejected before any launch
    (dict(slots=1024 * 1025, e=1024, align=1, cap=1024 * 1025 + 1024), 5),
])
def test_route_noalloc_checks_arguments(lib, case, status):
    v = dict(ids=A, slots=64, e=4, align=8, pad=1, offs=A + 0x100, rs=A + 0x200, cap=64 + 32, sr=A + 0x300, s=0)
    v.update(case)
    rc = gg.call_raw("gg_route_noalloc", v["ids"] or None, v["slots"], v["e"], v["align"], v["pad"],
                     v["offs"] or None, v["rs"], v["cap"], v["sr"], v["s"])
    assert rc == status, (case, rc, gg.last_error())
    if status == 5 and case.get("slots"):
        assert "GG_ROUTE_NOALLOC_SCRATCH_BYTES" in gg.last_error()

"""The C-ABI library on the CPU: it loads, exports every function include/rwnorm.h declares,
rejects invalid arguments before touching a device, and plans launches that cover every row
and column.  No kernel runs here."""
import ctypes
import os

import pytest
import torch

from row_wise_normalization_dyt_amd import _lib
import row_wise_normalization_dyt_amd as rwn

I64 = ctypes.c_int64


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_library_exports_every_declared_function(lib):
    declared = _lib.declared_functions()
    assert {"dyt_fwd", "dyt_bwd", "layernorm_fwd", "layernorm_bwd", "rmsnorm_fwd", "rmsnorm_bwd"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_library_is_built_for_gfx950():
    with open(_lib.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"gfx950" in blob


def test_version(lib):
    assert b"rwnorm" in lib.rwn_version()


def _err(lib):
    return lib.rwn_last_error().decode()


P = ctypes.c_void_p(16)   # a non-NULL, 16-byte-aligned stand-in pointer; never dereferenced


@pytest.mark.parametrize("M,N,code", [(-1, 8, 1), (4, 0, 1), (4, -3, 1), (4, 16385, 2)])
def test_shape_errors(lib, M, N, code):
    assert lib.dyt_fwd(M, N, P, 0, P, P, P, 0, P, None) == code
    assert _err(lib).startswith("dyt_fwd")
    assert lib.layernorm_fwd(M, N, P, 0, P, P, 0, 1e-5, P, None, None, None) == code
    assert lib.rmsnorm_bwd(M, N, P, P, 0, None, P, 0, 1e-6, P, P, P, 1 << 20, None) == code


def test_dtype_errors(lib):
    assert lib.dyt_fwd(4, 8, P, 7, P, P, P, 0, P, None) == 1
    assert lib.dyt_fwd(4, 8, P, 0, P, P, P, 9, P, None) == 1
    assert lib.rmsnorm_fwd(4, 8, P, 0, P, 1, 1e-6, P, None, None) == 2     # f32 x, bf16 weight
    assert "not supported" in _err(lib)
    assert lib.rmsnorm_fwd(4, 8, P, 0, P, 2, 1e-6, P, None, None) == 2     # f32 x, f16 weight
    assert lib.dyt_fwd(4, 8, P, 1, P, P, P, 2, P, None) == 2               # bf16 x, f16 params
    assert lib.dyt_fwd(4, 8, P, 2, P, P, P, 1, P, None) == 2               # f16 x, bf16 params
    assert "float16 x with bfloat16 parameters" in _err(lib)
    assert lib.dyt_fwd(4, 8, P, 3, P, P, P, 0, P, None) == 1               # no dtype code 3
    assert lib.rmsnorm_fwd_form(4, 8, P, 1, P, 1, 1e-6, 3, P, None, None) == 1   # no form 3
    assert "form" in _err(lib)
    assert lib.rmsnorm_bwd_form(4, 8, P, P, 1, None, P, 1, 1e-6, -1, P, P, P, 1 << 20, None) == 1


def test_null_and_eps_errors(lib):
    assert lib.dyt_fwd(4, 8, P, 0, None, P, P, 0, P, None) == 1
    assert lib.dyt_bwd(4, 8, P, P, 0, P, None, 0, P, None, None, None, P, 1 << 20, None) == 1
    assert lib.rmsnorm_fwd(4, 8, P, 1, None, 1, 1e-6, P, None, None) == 1
    for eps in (-1e-5, float("inf"), float("nan")):
        assert lib.layernorm_fwd(4, 8, P, 0, P, P, 0, eps, P, None, None, None) == 1
        assert "eps" in _err(lib)
    # mean without rstd
    assert lib.layernorm_bwd(4, 8, P, P, 0, P, None, P, 0, 1e-5, P, None, None, P, 1 << 20, None) == 1


def test_operand_alignment_errors(lib):
    odd = ctypes.c_void_p(16 + 2)
    # float32 operands must be 4-byte aligned
    assert lib.dyt_fwd(4, 8, odd, 0, P, P, P, 0, P, None) == 1
    # bf16 operands with different addresses modulo 16
    assert lib.dyt_fwd(4, 8, odd, 1, P, P, P, 0, P, None) == 2
    assert "modulo 16" in _err(lib)


def test_empty_forward_is_a_no_op_without_device(lib):
    assert lib.dyt_fwd(0, 8, None, 1, P, P, P, 0, None, None) == 0
    assert lib.layernorm_fwd(0, 8, None, 1, None, None, 0, 1e-5, None, None, None, None) == 0
    assert lib.rmsnorm_fwd(0, 8, None, 1, P, 1, 1e-6, None, None, None) == 0
    # a backward with no gradient requested has nothing to write
    assert lib.rmsnorm_bwd(0, 8, None, None, 1, None, P, 1, 1e-6, None, None, None, 0, None) == 0
    assert _err(lib) == ""


def test_workspace_query_errors(lib):
    out = ctypes.c_size_t(123)
    assert lib.dyt_bwd_workspace_size(0, 8, 0, ctypes.byref(out)) == 0 and out.value == 0
    assert lib.layernorm_bwd_workspace_size(-1, 8, 0, ctypes.byref(out)) == 1
    assert lib.rmsnorm_bwd_workspace_size(5, 8, 0, None) == 1


def test_trace_and_probe_argument_errors(lib):
    assert lib.rwn_trace_begin(0) == 1
    assert lib.rwn_trace_end(None, None, 0) == -1
    assert lib.rwn_stream_probe(None, None, P, 16, 4, 1, 8, None) == 1
    assert lib.rwn_stream_probe(P, None, P, 24, 4, 1, 8, None) == 1
    assert lib.rwn_stream_probe(P, None, P, 32, 3, 1, 8, None) == 1
    assert lib.rwn_stream_probe(P, None, P, 32, 4, 1, 0, None) == 1


# ------------------------------------------------------------------------------ planning

SHAPES = [(1, 1), (7, 24), (4096, 64), (401408, 24), (1048573, 32), (1048573, 128), (1048573, 256),
          (16384, 2048), (8192, 4096), (65536, 1025), (65536, 4096), (65536, 8192), (65536, 16384),
          (3, 7), (257, 17), (7, 129), (4099, 130), (7, 2049), (65537, 255), (5, 1023),
          (9, 3), (1000, 6), (1001, 48), (33, 192), (65, 384)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("backward", [False, True])
@pytest.mark.parametrize("M,N", SHAPES)
def test_plan_covers_rows_and_columns(M, N, dtype, backward):
    esz = 4 if dtype == torch.float32 else 2
    for mis in range(0, 16, esz):
        for layer in ("dyt", "layernorm", "rmsnorm"):
            V = 16 // esz
            if (N % V or mis) and N > 16384 - (V - 1) and layer != "dyt" and esz == 4:
                # documented limit: a misaligned float32 row of this width needs a 4097th chunk slot
                with pytest.raises(rwn.RwnError, match="UNSUPPORTED"):
                    rwn.plan(layer, backward, M, N, dtype, misalign_bytes=mis, cus=256)
                continue
            p = rwn.plan(layer, backward, M, N, dtype, misalign_bytes=mis, cus=256)
            V = p["vec"]
            if p["split"]:
                # split rows: whole aligned chunks (at most N // V of them) in tpr * cpt slots,
                # head and tail (at most 2V - 2 elements) in the first lanes; rows a slot revisits
                # are a multiple of V apart
                assert p["mode"] == 1 and p["ncb"] == 1 and p["rt"] == 1, p
                assert p["tpr"] % 64 == 0 and p["tpr"] * p["cpt"] >= N // V and p["tpr"] >= 2 * V - 2, p
                assert p["block"] == p["tpr"] * p["rpp"] <= 512 and p["strided"] == 1, p
                assert p["ntiles"] * p["rpp"] >= M > (p["ntiles"] - 1) * p["rpp"]
                gt = p["grid"]
                assert 1 <= gt <= max(p["ntiles"], 1) and (gt >= p["ntiles"] or (gt * p["rpp"]) % V == 0), p
                continue
            if p["flat"] == 2:
                # LayerNorm / DyT rows of 12 * 2^k bytes in 12-byte chunks: every lane of a row's
                # power-of-two group live, 4-byte aligned operands, whole waves, a persistent grid
                assert layer in ("layernorm", "dyt") and mis % 4 == 0 and V == 12 // esz, p
                assert N * esz == 12 * p["tpr"] and p["tpr"] <= 64 and p["tpr"] & (p["tpr"] - 1) == 0, p
                assert p["cpt"] == 1 and p["ncb"] == 1 and p["prefetch"] == 0 and p["xcd_remap"] == 0, p
                assert p["rt"] == (1 if backward or p["tpr"] == 1 else 2), p
                assert p["block"] % 64 == 0 and 64 <= p["block"] <= 256 and p["rpp"] * p["tpr"] == p["block"], p
                rows_per_tile = p["rpp"] * p["rt"]
                assert p["ntiles"] * rows_per_tile >= M > (p["ntiles"] - 1) * rows_per_tile, p
                assert p["strided"] == 1 and 1 <= p["grid"] <= p["ntiles"], p
                continue
            # chunks of a row: worst shift is V-1 elements in the shifted mode
            chunks = -(-(N + (V - 1 if p["mode"] == 1 else 0)) // V)
            assert p["tpr"] * p["cpt"] * p["ncb"] >= chunks, p
            assert p["grid"] % p["ncb"] == 0 and (p["ncb"] == 1 or layer == "dyt")
            if p["xcd_remap"]:
                assert p["grid"] % 8 == 0      # the renumbering is a bijection
            packed = layer == "dyt" and p["mode"] == 1 and 64 < p["tpr"] < 512 and p["tpr"] % 64 != 0
            assert p["block"] <= 1024 and (p["block"] % 64 == 0 or p["block"] < 64), p
            assert p["block"] == (-(-p["tpr"] * p["rpp"] // 64) * 64 if packed else p["tpr"] * p["rpp"]), p
            # launch bounds: one chunk per thread (and bf16 with four) at most 512 threads
            if p["rt"] == 1 and (p["cpt"] == 1 or (p["cpt"] == 4 and esz == 2)):
                assert p["block"] <= 512, p
            assert p["tpr"] <= 64 and (p["tpr"] & (p["tpr"] - 1)) == 0 or p["tpr"] % 64 == 0 or packed, p
            if p["mode"] == 0:
                assert N % V == 0 and mis == 0
            if p["mode"] == 1:
                # one slot, or slots that keep their shifts: V apart (blocked), or revisited at a
                # tile stride that is a multiple of V (checked below); narrow rows fill 256 threads
                assert p["rt"] == 1 and (p["rpp"] == 1 or p["rpp"] % V == 0 or packed or p["tpr"] <= 64), p
                if p["tpr"] <= 64 and not p["split"]:
                    assert p["rpp"] * p["tpr"] == p["block"] == max(256, V * p["tpr"]), p
            rows_per_tile = p["rpp"] * p["rt"]
            assert p["ntiles"] * rows_per_tile >= M > (p["ntiles"] - 1) * rows_per_tile
            if p["strided"]:
                gt = p["grid"] // p["ncb"]              # tile stride
                assert 1 <= gt <= max(p["ntiles"], 1)
                if gt < p["ntiles"]:
                    # a thread revisits rows gt * rpp apart: they must share the shift
                    assert (gt * p["rpp"]) % V == 0
            else:
                # blocked: consecutive tiles, every tile covered exactly once
                assert p["grid"] * p["kt"] >= p["ntiles"] > (p["grid"] - 1) * p["kt"]
                if p["mode"] == 1 and p["kt"] > 1:
                    assert p["rpp"] % V == 0, p    # consecutive tiles keep each slot's shift
                if not backward:
                    assert p["kt"] == 1


@pytest.mark.parametrize("layout", [1, 2])
@pytest.mark.parametrize("backward", [False, True])
def test_strided_plans(layout, backward):
    """Strided operands take the general kernels with one row per thread;
    layout 2 (rows of mixed alignment) moves elements (SCALAR), and LayerNorm / RMSNorm take
    it up to 2048 16-bit or 4096 float32 elements, DyT at any width through column blocks."""
    for dtype, esz in ((torch.float32, 4), (torch.bfloat16, 2), (torch.float16, 2)):
        V = 16 // esz
        for N in (1, 7, 24, 128, 129, 1025, 2048, 2049, 4096, 4097, 16384):
            for mis in (range(0, 16, esz) if layout == 1 else (0,)):
                for layer in ("dyt", "layernorm", "rmsnorm"):
                    limit = 4096 if esz == 4 else 2048
                    if layout == 2 and layer != "dyt" and N > limit:
                        with pytest.raises(rwn.RwnError, match="UNSUPPORTED"):
                            rwn.plan(layer, backward, 4099, N, dtype, mis, cus=256, layout=layout)
                        continue
                    if layout == 1 and (N % V or mis) and N > 16384 - (V - 1) and layer != "dyt":
                        # a row that straddles one more chunk than the widest aligned row
                        with pytest.raises(rwn.RwnError, match="UNSUPPORTED"):
                            rwn.plan(layer, backward, 4099, N, dtype, mis, cus=256, layout=layout)
                        continue
                    p = rwn.plan(layer, backward, 4099, N, dtype, mis, cus=256, layout=layout)
                    assert p["rt"] == 1 and p["flat"] == 0 and p["split"] == 0, p
                    # pipelining only where a form exists: two tiles ahead for one vector chunk
                    assert p["prefetch"] <= (2 if p["cpt"] == 1 and p["mode"] != 2 else 1 if p["cpt"] <= 2 else 0), p
                    if layout == 2:
                        assert p["mode"] == 2 and p["vec"] == 1, p
                    else:
                        assert p["mode"] == (0 if (N % V == 0 and mis == 0) else p["mode"]), p
                    chunks = N if p["mode"] == 2 else -(-(N + (V - 1 if p["mode"] == 1 else 0)) // V)
                    assert p["tpr"] * p["cpt"] * p["ncb"] >= chunks, p
                    assert p["cpt"] == 1 or layer != "dyt", p
                    cap = 512 if (p["cpt"] == 1 or (p["cpt"] == 4 and esz == 2)) else 1024
                    assert p["block"] <= cap and p["ntiles"] * p["rpp"] >= 4099 > (p["ntiles"] - 1) * p["rpp"], p


def test_strided_argument_errors(lib):
    """The strided entry points validate leading sizes, strides, spans and output overlap
    before touching a device."""
    A = ctypes.c_int64 * 3
    lead, xs, ys = A(4, 0, 0), A(64, 0, 0), A(64, 0, 0)

    def fwd(nlead=1, lead=lead, N=64, x=P, x_str=xs, y=P, y_str=ys, xdt=0, gstride=1):
        return lib.dyt_fwd_strided(nlead, lead, N, x, x_str, xdt, P, P, gstride, P, 1, 0, y, y_str, None)

    for n in (0, 4):
        assert fwd(nlead=n) == 1 and "nlead" in _err(lib)
    assert fwd(lead=None) == 1
    assert fwd(lead=A(-1, 0, 0)) == 1 and "negative" in _err(lib)
    assert fwd(x_str=A(-64, 0, 0)) == 1 and "negative" in _err(lib)
    assert fwd(x_str=None) == 1 and "strides" in _err(lib)
    assert fwd(gstride=-1) == 1 and "parameter strides" in _err(lib)
    assert fwd(y_str=A(0, 0, 0)) == 1 and "overlap" in _err(lib)           # four rows on one row
    assert fwd(y_str=A(63, 0, 0)) == 1 and "overlap" in _err(lib)          # rows 63 apart, 64 wide
    assert fwd(nlead=2, lead=A(4, 8, 0), y_str=A(8 * 64, 32, 0)) == 1 and "overlap" in _err(lib)
    assert fwd(x_str=A(1 << 40, 0, 0)) == 2 and "spans" in _err(lib)
    assert fwd(nlead=2, lead=A(1 << 16, 1 << 16, 0), x_str=A(0, 0, 0)) == 2 and "rows" in _err(lib)
    assert fwd(x=ctypes.c_void_p(18)) == 1 and "aligned" in _err(lib)      # float32 at 2 mod 4
    assert fwd(N=16385) == 2
    # no rows: nothing to read or write, and no device is needed
    assert fwd(lead=A(0, 0, 0), x=None, y=None) == 0
    assert lib.layernorm_fwd_strided(2, A(0, 5, 0), 8, None, A(8, 40, 0), 1, None, 1, None, 1, 0, 1e-5, None,
                                     A(8, 40, 0), None, None, None) == 0
    bad = A(-1, 0, 0)
    assert lib.layernorm_bwd_strided(1, lead, 64, P, xs, P, bad, 0, None, None, P, 1, 0, 1e-5, P, ys, None, None,
                                     None, 0, None) == 1
    assert lib.rmsnorm_bwd_strided(1, lead, 64, P, xs, P, xs, 0, None, P, 1, 0, 1e-6, 0, P, A(0, 0, 0), None, None,
                                   0, None) == 1
    assert lib.rmsnorm_fwd_strided(1, lead, 64, P, xs, 0, P, -2, 0, 1e-6, 0, P, ys, None, None) == 1


def test_plan_uses_narrow_tiles_for_narrow_rows():
    p = rwn.plan("layernorm", True, 401408, 24, torch.float32, cus=256)
    assert p["mode"] == 0 and p["tpr"] == 8 and p["rpp"] == 32
    p = rwn.plan("dyt", True, 1048573, 32, torch.bfloat16, cus=256)
    assert p["tpr"] == 4 and p["rpp"] == 64
    # grid-stride plans keep at least 8 waves per CU resident
    for bwd in (False, True):
        p = rwn.plan("layernorm", bwd, 401408, 24, torch.float32, cus=256)
        assert p["strided"] and p["grid"] * p["block"] // 64 >= 8 * 256 and p["grid"] % 8 == 0
    # the persistent grid is a whole number of workgroups per CU with 16..28 resident waves,
    # and a perfectly even split wins over one more workgroup per CU only by more than 2%
    p = rwn.plan("layernorm", False, 401408, 24, torch.float32, cus=256)
    waves = p["grid"] * p["block"] // 64 // 256
    assert p["grid"] % 256 == 0 and 16 <= waves <= 28, p
    p = rwn.plan("dyt", False, 1048573, 32, torch.bfloat16, cus=256)
    assert p["ntiles"] % p["grid"] == 0 and p["grid"] == 1024, p
    # short input: the tile count caps the grid (no full grid for one row)
    p = rwn.plan("rmsnorm", False, 1, 128, torch.bfloat16, cus=256)
    assert p["grid"] == 1 and p["ntiles"] == 1


@pytest.mark.parametrize("backward", [False, True])
def test_flat_plans(backward):
    """LayerNorm rows of 12 * 2^k bytes (2^k <= 64) on 4-byte aligned operands take the flat
    kernels with 12-byte chunks (flat 2), and so do such DyT rows in the backward and, where the
    rows are not whole 16-byte chunks, in the forward; other narrow aligned LayerNorm plans with one
    chunk and one row per thread (group sizes 1..64 lanes, no pipelining, at most 256 threads)
    take the 16-byte flat kernels (flat 1); every other plan, and RMSNorm, keeps the general
    kernels."""
    for dtype, V in ((torch.float32, 4), (torch.bfloat16, 8), (torch.float16, 8)):
        esz = 16 // V
        for N in (V, 2 * V, 24 if V == 4 else 32, 24, 3 * V, 6 * V, 48 * V, 16 * V, 64 * V, 64 * V + V, 1025):
            for mis in (0, 2 if V == 8 else 4, 4 if V == 8 else 8):
                for layer in ("dyt", "layernorm", "rmsnorm"):
                    p = rwn.plan(layer, backward, 4099, N, dtype, misalign_bytes=mis, cus=256)
                    lanes = N * esz // 12
                    whole16 = (N * esz) % 16 == 0 and mis % 16 == 0
                    want12 = ((layer == "layernorm" or (layer == "dyt" and (backward or not whole16)))
                              and (N * esz) % 12 == 0 and lanes <= 64
                              and lanes & (lanes - 1) == 0 and mis % 4 == 0)
                    want = (layer == "layernorm" and p["mode"] == 0 and p["cpt"] == 1 and p["rt"] == 1
                            and p["tpr"] <= 64 and p["ncb"] == 1)
                    assert p["flat"] == (2 if want12 else int(want)), (layer, N, mis, p)
                    if p["flat"] == 1:
                        assert N % V == 0 and mis == 0 and p["prefetch"] == 0 and p["block"] <= 256, p
                        assert p["tpr"] in (1, 2, 4, 8, 16, 32, 64) and p["block"] == p["tpr"] * p["rpp"], p
                    if p["flat"] == 2:
                        assert p["tpr"] == lanes and p["vec"] == 12 // esz and p["prefetch"] == 0, p
    p = rwn.plan("layernorm", backward, 401408, 24, torch.float32, cus=256)
    assert p["flat"] == 2 and p["xcd_remap"] == 0 and p["tpr"] == 8


def test_planner_rules_off_grid_rows_and_few_rows():
    """Plan choices that measured rules fix (cus = 256, no occupancy query).  Narrow rows off
    the 16-byte grid move in 16-byte SHIFTED chunks: a power-of-two lane group per row and
    max(256 / tpr, V) row slots, with no pipelining in DyT backwards.  With few rows per CU
    (64 MiB bf16 tensors), 16-bit LayerNorm rows of 512-1024 chunks and RMSNorm / DyT rows of
    1024 chunks take the split-row kernels in both directions; rows of 2048 chunks, narrower
    RMSNorm rows and the same widths with many rows (65536) keep the general backward."""
    bf, f32 = torch.bfloat16, torch.float32
    p = rwn.plan("layernorm", False, 335544, 100, bf, param_dtype=f32, cus=256)
    assert (p["mode"], p["tpr"], p["rpp"], p["split"]) == (1, 16, 16, 0), p
    p = rwn.plan("rmsnorm", True, 1 << 20, 3, bf, cus=256)
    assert (p["mode"], p["tpr"], p["rpp"], p["split"]) == (1, 2, 128, 0), p
    p = rwn.plan("dyt", True, 67108, 500, bf, cus=256)
    assert (p["mode"], p["tpr"], p["rpp"], p["prefetch"]) == (1, 64, 8, 0), p
    for layer, N, few_split in (("layernorm", 4096, 1), ("layernorm", 8192, 1), ("layernorm", 3000, 0),
                                ("layernorm", 16384, 0), ("rmsnorm", 8192, 1), ("rmsnorm", 5120, 0),
                                ("dyt", 8192, 1), ("dyt", 16384, 0)):
        M = (64 << 20) // (2 * N)
        pb = rwn.plan(layer, True, M, N, bf, cus=256)
        assert pb["split"] == few_split, (layer, N, pb)
        if few_split:
            assert rwn.plan(layer, False, M, N, bf, param_dtype=f32, cus=256)["split"] == 1, (layer, N)
        assert rwn.plan(layer, True, 65536, N, bf, cus=256)["split"] == 0, (layer, N)


def test_plan_is_deterministic():
    a = [rwn.plan(l, b, 65536, 1025, torch.bfloat16, 2, cus=256) for l in ("dyt", "rmsnorm") for b in (0, 1)]
    b = [rwn.plan(l, b, 65536, 1025, torch.bfloat16, 2, cus=256) for l in ("dyt", "rmsnorm") for b in (0, 1)]
    assert a == b


_BOUNDS_SCRIPT = r"""
import sys, torch
sys.path.insert(0, {root!r})
import row_wise_normalization_dyt_amd as rwn
bad = []
for layer in ("dyt", "layernorm", "rmsnorm"):
    for dt, esz in ((torch.float32, 4), (torch.bfloat16, 2)):
        for N in (24, 64, 129, 1025, 2048, 4096, 8192, 16384):
            for mis in range(0, 16, esz):
                for bwd in (0, 1):
                    try:
                        p = rwn.plan(layer, bwd, 65537, N, dt, mis, cus=256)
                    except rwn.RwnError:
                        continue
                    cap = 256 if p["rt"] > 1 else (512 if p["cpt"] == 1 or (p["cpt"] == 4 and esz == 2) else 1024)
                    if p["block"] > cap or p["block"] < p["tpr"] * p["rpp"] or p["block"] % 64:
                        bad.append((layer, str(dt), N, mis, bwd, p))
                    if p["prefetch"] and p["cpt"] * p["rt"] > 2 and not p["split"]:   # no pipelined form
                        bad.append(("prefetch", layer, str(dt), N, mis, bwd, p))
                    if p["strided"] and p["grid"] * ((p["block"] + 63) // 64) > 32 * 256:
                        bad.append(("waves", layer, str(dt), N, mis, bwd, p))
                    V = 16 // esz
                    if p["mode"] == 1 and not p["strided"] and p["kt"] > 1 and p["rpp"] % V:
                        bad.append(("shift", layer, str(dt), N, mis, bwd, p))   # a slot's rows change shift
print("BAD", bad)
"""


@pytest.mark.parametrize("env", ["RWN_WIDE_BLOCK=1024", "RWN_WIDE_BLOCK=64", "RWN_FWD_RT=4", "RWN_BWD_RT=2",
                                 "RWN_MIN_WAVES=32", "RWN_WG_PER_CU=3", "RWN_BLOCKED_K=3", "RWN_PREFETCH=1",
                                 "RWN_PREFETCH=0", "RWN_X=0", "RWN_FLAT=0", "RWN_FLAT12=0", "RWN_SPLIT_PF=1",
                                 "RWN_SPLIT_PF=0", "RWN_PACKED_ROWS=0", "RWN_SPLIT=2", "RWN_SPLIT_CPT=4"])
def test_plans_respect_kernel_launch_bounds_under_tuning_overrides(env):
    """Every plan's workgroup fits the launch bound its kernel was compiled for, also with the
    tuning overrides set (a plan over the bound would fail to launch)."""
    import subprocess, sys
    k, v = env.split("=")
    r = subprocess.run([sys.executable, "-c", _BOUNDS_SCRIPT.format(root=os.path.dirname(os.path.dirname(__file__)))],
                       env=dict(os.environ, **{k: v}), capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "BAD []" in r.stdout, r.stdout[-2000:]

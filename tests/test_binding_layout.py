"""Host logic of the binding's strided path (CPU only, no kernel runs): how torch views become the
strided entry points' leading sizes and strides, when the strided path is taken, and the
checks on caller-provided outputs and parameter vectors."""
import pytest
import torch

import row_wise_normalization_dyt_amd as rwn


def _layout(*ts):
    out = rwn._row_layout(list(ts))
    if out is None:
        return None
    n, lead, strides = out
    return list(lead), [list(s) for s in strides]


def test_contiguous_rows_merge_into_one_dimension():
    x = torch.empty(4, 5, 6, 32)
    assert _layout(x, torch.empty_like(x)) == ([120], [[32], [32]])


def test_size_one_dimensions_are_dropped():
    x = torch.empty(1, 7, 1, 3, 16)
    assert _layout(x) == ([21], [[16]])
    single = torch.empty(1, 1, 16)
    assert _layout(single) == ([1], [[0]])


def test_head_major_view_keeps_three_dimensions_with_each_tensors_strides():
    B, S, H, D = 2, 300, 32, 128
    hm = torch.empty(B, H, S, D).permute(0, 2, 1, 3)        # [B, S, H, D] view, head-major memory
    dense = torch.empty(B, S, H, D)
    lead, (s_hm, s_dense) = _layout(hm, dense)
    assert lead == [B, S, H]
    assert s_hm == [H * S * D, D, S * D]
    assert s_dense == [S * H * D, H * D, D]
    # the head-major view alone is a permuted dense tensor: its leading dimensions do not merge in
    # logical order (rows are visited in [B, S, H] order, not in memory order)
    assert _layout(hm)[0] == [B, S, H]


def test_column_slice_has_one_row_stride():
    big = torch.empty(100, 96)
    assert _layout(big[:, 8:72], torch.empty(100, 64)) == ([100], [[96], [64]])


def test_dimensions_merge_only_where_every_tensor_allows():
    a = torch.empty(3, 4, 5, 8)                       # fully mergeable
    b = torch.empty(3, 5, 4, 8).transpose(1, 2)       # dims 1, 2 swapped in memory
    lead, (sa, sb) = _layout(a, b)
    assert lead == [3, 4, 5]                          # b blocks every merge
    assert sa == [160, 40, 8] and sb == [160, 8, 32]
    c = torch.empty(3, 4, 6, 8)[:, :, :5]             # rows of 5 within blocks of 6
    lead, (sa, sc) = _layout(a, c)
    assert lead == [12, 5] and sa == [40, 8] and sc == [48, 8]


def test_more_than_three_unmergeable_dimensions_fall_back():
    x = torch.empty(2, 3, 5, 7, 16).permute(3, 1, 0, 2, 4)
    assert rwn._row_layout([x]) is None


def test_strided_path_is_taken_only_for_views_with_a_contiguous_last_dimension(monkeypatch):
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True))
    dense = torch.empty(8, 64)
    assert not rwn._use_strided([dense], [torch.empty(64)])
    assert rwn._use_strided([dense[:, :32]], [None])                     # a column slice
    assert rwn._use_strided([dense], [torch.empty(128)[::2]])            # a strided parameter
    assert not rwn._use_strided([dense.t()], [None])                     # last dimension strided: copied
    assert not rwn._use_strided([torch.empty(0, 64)], [None])            # no rows
    x4 = torch.empty(2, 3, 4, 16)
    dy4 = torch.empty(2, 4, 3, 16).transpose(1, 2)                      # a head-major gradient
    assert rwn._use_strided([x4, dy4], [None]) and not rwn._use_strided([x4, x4], [None])


def test_parameter_vectors_keep_their_stride():
    src = torch.arange(30.0)[::3]
    v, s = rwn._svec(src, 10, "gamma", torch.device("cpu"))
    assert s == 3 and v.data_ptr() == src.data_ptr()              # read in place, no copy
    v, s = rwn._svec(torch.ones(1, 10), 10, "gamma", torch.device("cpu"))
    assert s == 1 and v.shape == (10,)
    assert rwn._svec(None, 10, "beta", torch.device("cpu")) == (None, 1)
    with pytest.raises(ValueError, match="10 elements"):
        rwn._svec(torch.ones(9), 10, "gamma", torch.device("cpu"))


def test_fresh_outputs_share_the_inputs_phase_modulo_16_bytes():
    base = torch.empty(1000, dtype=torch.bfloat16)
    for off in range(8):
        x = base[off:off + 640].view(10, 64)
        y = rwn._fresh_rows(x)
        assert y.shape == x.shape and y.is_contiguous()
        assert y.data_ptr() % 16 == x.data_ptr() % 16


def test_caller_outputs_are_checked():
    x = torch.empty(10, 64)
    with pytest.raises(ValueError, match="shape"):
        rwn._out_strided(torch.empty(10, 32), x, "y")
    with pytest.raises(ValueError, match="contiguous last dimension"):
        rwn._out_strided(torch.empty(64, 10).t(), x, "y")
    view = torch.empty(10, 96)[:, :64]
    assert rwn._out_strided(view, x, "y") is view


def test_rows12_rule_matches_the_planner():
    """The binding keeps a 4-byte-aligned LayerNorm view exactly where the planner takes the
    12-byte flat kernels for it (every width up to 400, both element sizes)."""
    for dtype in (torch.float32, torch.bfloat16):
        esz = 4 if dtype == torch.float32 else 2
        for N in range(1, 401):
            p = rwn.plan("layernorm", False, 1000, N, dtype, misalign_bytes=4, cus=256)
            assert rwn._rows12(N, esz) == (p["flat"] == 2), (dtype, N, p)


def test_layernorm_rows12_views_are_not_copied(monkeypatch):
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True))
    buf = torch.empty(8 + 100 * 24, dtype=torch.float32)
    base = (16 - buf.data_ptr() % 16) // 4           # element index of a 16-byte boundary
    view = buf[base + 1:base + 1 + 100 * 24].view(100, 24)   # 4 bytes past it
    assert view.data_ptr() % 16 == 4
    assert rwn._as_2d(view, "x", rows12=True).data_ptr() == view.data_ptr()   # taken as it is
    assert rwn._as_2d(view, "x").data_ptr() % 16 == 0                         # other layers: aligned copy
    b16 = torch.empty(16 + 100 * 48, dtype=torch.bfloat16)
    base = (16 - b16.data_ptr() % 16) // 2
    odd = b16[base + 1:base + 1 + 100 * 48].view(100, 48)                      # 2 bytes past: not 4-aligned
    assert rwn._as_2d(odd, "x", rows12=True).data_ptr() % 16 == 0
    even = b16[base + 2:base + 2 + 100 * 48].view(100, 48)                     # 4 bytes past
    assert rwn._as_2d(even, "x", rows12=True).data_ptr() == even.data_ptr()

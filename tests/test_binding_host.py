"""Host-side checks of the Python binding's argument validation (no GPU): the byte spans and
the aliasing rule (the output may be R itself, never a partial overlap or another operand)."""
import pytest
import torch

from decode_skinny_addmm_amd import ops


def test_byte_span_of_views():
    buf = torch.zeros(100, dtype=torch.bfloat16)
    base = buf.data_ptr()
    v = buf[10:70].view(6, 10)
    assert ops._byte_span(v) == (base + 20, base + 140)
    # a column block of a wider matrix: rows 0..2 of width 4 starting at column 3 of a 3 x 10 view
    w = buf[:30].view(3, 10)[:, 3:7]
    assert ops._byte_span(w) == (base + 6, base + 2 * (2 * 10 + 6 + 1))
    lo, hi = ops._byte_span(buf[5:5])
    assert lo == hi                               # an empty tensor touches no byte


def test_overlap_rule():
    buf = torch.zeros(200, dtype=torch.bfloat16)
    X = buf[:40].view(4, 10)
    W = buf[40:100].view(6, 10)
    R = buf[100:124].view(4, 6)
    Y = buf[124:148].view(4, 6)
    ops._check_aliasing((X, W), R, Y)            # disjoint
    ops._check_aliasing((X, W), R, R)            # in place
    with pytest.raises(ValueError):
        ops._check_aliasing((X, W), R, buf[30:54].view(4, 6))   # overlaps X
    with pytest.raises(ValueError):
        ops._check_aliasing((X, W), R, buf[96:120].view(4, 6))  # overlaps W and R
    with pytest.raises(ValueError):
        ops._check_aliasing((X, W), R, buf[101:125].view(4, 6))  # R shifted by one element
    with pytest.raises(ValueError):
        ops._check_aliasing((X, W), R, buf[100:124].view(torch.float32).view(4, 3))  # same bytes, fp32
    # touching spans do not overlap
    assert not ops._overlaps(buf[0:10], buf[10:20])
    assert ops._overlaps(buf[0:11], buf[10:20])

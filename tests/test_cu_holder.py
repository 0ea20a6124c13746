"""ra.CuSeqlens: one host and one device copy of cu_seqlens (no GPU needed)."""
import numpy as np
import pytest


def test_cu_holder_copies_and_checks():
    import torch
    import exact_long_context_ra_amd as ra
    from exact_long_context_ra_amd import api
    c = ra.CuSeqlens([0, 5, 12], "cpu")
    assert c.num_seqs == 2 and c.host.dtype == np.int32 and c.dev.dtype == torch.int32
    assert np.array_equal(c.host, [0, 5, 12]) and c.dev.tolist() == [0, 5, 12]
    # the problem descriptor points at the holder's copies (no new copy)
    h = api._Cu(c, "cpu")
    assert h.host is c.host and h.dev is c.dev and h.n == 2
    # a holder is accepted wherever cu_seqlens is
    assert np.array_equal(ra.layout_positions("zigzag_varlen", 16, 2, 0, ra.CuSeqlens([0, 8, 16], "cpu")),
                          ra.layout_positions("zigzag_varlen", 16, 2, 0, [0, 8, 16]))
    assert ra.CuSeqlens(c, "cpu").host.tolist() == [0, 5, 12]
    with pytest.raises(ValueError):
        ra.CuSeqlens([0], "cpu")
    with pytest.raises(ValueError):
        api._Cu(c, "meta")

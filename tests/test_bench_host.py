"""Host logic of bench.py, on the CPU: the count of rows that an in-place pass moves (its kept
rows at or past row B), against a brute-force count from the oracle's select."""
import numpy as np
import pytest
import torch

import bench
import oracle as O


def _scores(case, U, C):
    rng = np.random.default_rng(3)
    if case == "random":
        return rng.standard_normal((U, C)).astype(np.float32)
    if case == "quantized":  # heavy ties, some of them across row B
        return np.round(rng.standard_normal((U, C)) * 3).astype(np.float32)
    if case == "zeros":  # +0 and -0 only: the first B rows are kept, nothing moves
        return np.where(rng.random((U, C)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    # scores rising with the row: the last B rows are kept
    return np.tile(np.arange(C, dtype=np.float32), (U, 1))


@pytest.mark.parametrize("case", ["random", "quantized", "zeros", "rising"])
def test_moved_row_count_matches_brute_force(case):
    U, C, B = 6, 300, 200
    sc = _scores(case, U, C)
    expect = sum(int(np.sum(O.select_topb(sc[u], B) >= B)) for u in range(U))
    got = int(bench.count_moved_rows(torch, torch.from_numpy(sc), B).item())
    assert got == expect
    if case == "zeros":
        assert got == 0
    if case == "rising":
        assert got == U * (C - B)

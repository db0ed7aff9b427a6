"""The exact-arithmetic inputs of the bit-exact GEMV tests (no GPU): every
row's result is exact in fp32, and a localised decode mistake (one 32-weight
group of one block taking its neighbour's weights, one block's scale or d
misread, two neighbouring nibbles swapped) changes the result of almost every
row, so an exact comparison sees it where the general-input tolerance
(1e-3 * sum |x w|) lets most such rows pass."""
import numpy as np
import pytest

import oracle
from dequant_gemv_amd import synth

N, K = 200, 4096


def _dot(w, x):
    return (w.astype(np.float64) * x[None, :]).sum(axis=1)


def _x_values(fmt, x):
    if synth.x_dtype(fmt) == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1", "f16", "bf16"])
def test_results_are_exact_in_fp32(fmt):
    w = synth.weights_exact(fmt, N, K, 5)
    x = synth.x_ternary(fmt, K, 6)
    y, _ = oracle.gemv(fmt, w, x, N, K)
    assert np.array_equal(y.astype(np.float32).astype(np.float64), y)
    assert np.count_nonzero(y) > 0.9 * N


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1"])
def test_a_group_swap_changes_almost_every_row(fmt):
    w = synth.weights_exact(fmt, N, K, 7)
    x = synth.x_ternary(fmt, K, 8)
    xv = _x_values(fmt, x)
    deq = oracle.dequant(fmt, w, N, K)
    y, _ = oracle.gemv(fmt, w, x, N, K)
    assert np.array_equal(_dot(deq, xv), y)
    bad = deq.copy()
    bad[:, 32:64] = deq[:, 64:96]  # group 1 of block 0 reads group 2's weights
    yb = _dot(bad, xv)
    # ternary weights leave a group's sum unchanged now and then
    assert np.mean(yb != y) > (0.8 if fmt == "tq1" else 0.95)


def test_a_swapped_nibble_pair_changes_most_rows():
    w = synth.weights_exact("q4k", N, K, 9)
    x = synth.x_ternary("q4k", K, 10)
    xv = _x_values("q4k", x)
    deq = oracle.dequant("q4k", w, N, K)
    y, _ = oracle.gemv("q4k", w, x, N, K)
    i = int(np.flatnonzero(xv[:-1] != xv[1:])[0])  # two neighbours with different activations
    bad = deq.copy()
    bad[:, [i, i + 1]] = deq[:, [i + 1, i]]  # their weights exchanged
    # the result moves in every row whose two weights differ
    assert np.array_equal(_dot(bad, xv) != y, deq[:, i] != deq[:, i + 1])
    assert np.mean(deq[:, i] != deq[:, i + 1]) > 0.8

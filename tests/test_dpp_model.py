"""Lane-level model of the cross-lane sequences the kernels use, checked on
the CPU against plain reductions.

A wave has 64 lanes in 4 rows of 16. The DPP controls used:
  row_shr:n    lane l of a row reads lane l - n of the same row; lanes with no
               such source get 0 (bound_ctrl) or keep their old value;
  row_bcast:15 lane 15 of each row is read by every lane of the next row;
  row_bcast:31 lane 31 is read by every lane of rows 2 and 3;
a row mask limits which rows are written (the others keep `old`).
v_permlane16_swap(a, b) swaps the odd rows of a with the even rows of b;
v_permlane32_swap(a, b) swaps the upper half of a with the lower half of b.

The sequences restated here are those of wave_incl_sum (select kernel:
list and fetch-list placement), wave_max / wave_sum (merge kernel) and
max_over_rows (prefill softmax). This pins the lane reasoning, not the
compiled code; the GPU parity tests exercise the kernels themselves.
"""
import numpy as np

LANES, ROW = 64, 16


def dpp(old, src, ctrl, row_mask=0xF, bound_zero=False):
    out = np.array(old, dtype=np.float64, copy=True)
    for l in range(LANES):
        row = l // ROW
        if not (row_mask >> row) & 1:
            continue
        if ctrl[0] == "shr":
            n = ctrl[1]
            if l % ROW >= n:
                out[l] = src[l - n]
            elif bound_zero:
                out[l] = 0.0
        elif ctrl == ("bcast", 15):
            if row >= 1:
                out[l] = src[ROW * row - 1]       # lane 15 of the previous row
            elif bound_zero:
                out[l] = 0.0
        elif ctrl == ("bcast", 31):
            if row >= 2:
                out[l] = src[31]
            elif bound_zero:
                out[l] = 0.0
    return out


def wave_incl_sum(v):
    v = np.array(v, dtype=np.float64)
    for n in (1, 2, 4, 8):
        v = v + dpp(np.zeros(LANES), v, ("shr", n), 0xF, True)
    v = v + dpp(np.zeros(LANES), v, ("bcast", 15), 0xA)
    v = v + dpp(np.zeros(LANES), v, ("bcast", 31), 0xC)
    return v


def wave_max(v):
    v = np.array(v, dtype=np.float64)
    for n in (1, 2, 4, 8):
        v = np.maximum(v, dpp(v, v, ("shr", n), 0xF, False))
    v = np.maximum(v, dpp(v, v, ("bcast", 15), 0xA))
    v = np.maximum(v, dpp(v, v, ("bcast", 31), 0xC))
    return np.full(LANES, v[63])                  # readlane 63


def wave_sum(v):
    return np.full(LANES, wave_incl_sum(v)[63])   # readlane 63


def permlane16_swap(a, b):
    a, b = np.array(a, dtype=np.float64), np.array(b, dtype=np.float64)
    a2, b2 = a.copy(), b.copy()
    for r_odd, r_even in ((1, 0), (3, 2)):
        sa, sb = slice(ROW * r_odd, ROW * r_odd + ROW), slice(ROW * r_even, ROW * r_even + ROW)
        a2[sa], b2[sb] = b[sb], a[sa]
    return a2, b2


def permlane32_swap(a, b):
    a, b = np.array(a, dtype=np.float64), np.array(b, dtype=np.float64)
    a2, b2 = a.copy(), b.copy()
    a2[32:], b2[:32] = b[:32], a[32:]
    return a2, b2


def max_over_rows(v):
    x, y = permlane16_swap(v, v)
    v = np.maximum(x, y)
    x, y = permlane32_swap(v, v)
    return np.maximum(x, y)


def test_incl_sum_is_a_prefix_sum():
    rng = np.random.default_rng(0)
    for _ in range(50):
        v = rng.integers(0, 64, LANES).astype(np.float64)
        np.testing.assert_array_equal(wave_incl_sum(v), np.cumsum(v))


def test_wave_max_and_sum_reach_every_lane():
    rng = np.random.default_rng(1)
    for _ in range(50):
        v = rng.standard_normal(LANES)
        np.testing.assert_array_equal(wave_max(v), np.full(LANES, v.max()))
        np.testing.assert_allclose(wave_sum(v), np.full(LANES, v.sum()), rtol=1e-12)
    # -inf lanes (masked tokens) do not disturb the maximum
    v = np.full(LANES, -np.inf)
    v[37] = 2.5
    assert (wave_max(v) == 2.5).all()


def test_max_over_rows_spans_the_four_rows_of_a_column():
    rng = np.random.default_rng(2)
    for _ in range(50):
        v = rng.standard_normal(LANES)
        got = max_over_rows(v)
        want = np.array([max(v[(l % ROW) + ROW * r] for r in range(4)) for l in range(LANES)])
        np.testing.assert_array_equal(got, want)


def test_swaps_pair_each_lane_with_its_partner():
    v = np.arange(LANES, dtype=np.float64)
    x, y = permlane16_swap(v, v)
    assert all({x[l], y[l]} == {l, l ^ 16} for l in range(LANES))
    x, y = permlane32_swap(v, v)
    assert all({x[l], y[l]} == {l, l ^ 32} for l in range(LANES))

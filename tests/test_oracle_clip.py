"""Pins for the oracle's clip-ratio search (CPU only).

Closed form: for values spread uniformly over [-a, a], the four-level uniform quantiser of
least squared error has levels +-a/4 and +-3a/4 (cell centres), which the min-max scheme
reaches with clip ratio 0.75 (levels -c a, -c a / 3, c a / 3, c a). Rows of 128 evenly
spaced values (2 i + 1) / 128 - 1 have extremes +-127/128, so the optimum sits at
0.75 * 128 / 127 = 0.756, and the 0.01 grid must land on 0.75 or 0.76. Degenerate and
monotone cases check the criterion itself."""

import numpy as np

from oracle import clip, quant

EYE = np.eye(128)


def _uniform_rows(n, seed):
    g = np.random.default_rng(seed)
    x = g.uniform(-1.0, 1.0, (n, 128))
    x[:, 0], x[:, 1] = -1.0, 1.0  # the row extremes at exactly -1 and 1
    return x


def test_uniform_values_give_the_cell_centre_clip():
    g = np.random.default_rng(3)
    spaced = (2 * np.arange(128) + 1) / 128 - 1
    x = np.stack([g.permutation(spaced) for _ in range(16)])
    best, errs = clip.search(x, EYE)
    assert best in (0.75, 0.76), best
    # the error is smallest near the optimum and rises away from it on both sides
    assert errs[0] > errs[25] and errs[-1] > errs[25]


def test_error_matches_a_direct_sum():
    x = _uniform_rows(3, 4) * 2.5
    e = clip.reconstruction_error(x, EYE, 0.8)
    codes, s16, z16, _ = quant.quantize_rows(x, EYE, 0.8)
    lv = z16.astype(np.float64)[:, None] + codes * s16.astype(np.float64)[:, None]
    assert np.isclose(e, np.sum((x - lv) ** 2), rtol=1e-12, atol=0.0)


def test_no_clipping_is_exact_for_four_valued_rows():
    # rows that only take the values -3, -1, 1, 3: c = 1 reconstructs them exactly
    g = np.random.default_rng(5)
    x = g.choice([-3.0, -1.0, 1.0, 3.0], (8, 128))
    x[:, 0], x[:, 1] = -3.0, 3.0
    best, errs = clip.search(x, EYE)
    assert best == 1.0 and errs[-1] == 0.0 and np.all(errs[:-1] > 0)


def test_outliers_pull_the_ratio_down():
    # one large outlier per row: clipping it buys resolution for the bulk of the values
    x = _uniform_rows(32, 6)
    x[:, 2] = 6.0
    best_out, _ = clip.search(x, EYE)
    best_plain, _ = clip.search(_uniform_rows(32, 6), EYE)
    assert best_out < best_plain

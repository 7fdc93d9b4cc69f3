"""Pins for the oracle's mask builder (CPU only).

Each test checks ``oracle.mask`` against something other than itself: the
review's worked toy example (golden fixture), a closed-form count checked
against brute force, the O(n log n) claim, the power-of-two special case,
symmetry and the halving of amortised density per band.
"""

import math
from fractions import Fraction
import os

import numpy as np
import pytest

from oracle import mask as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_toy():
    bands, frame0, counts = [], None, {}
    with open(os.path.join(GOLDEN, "toy_f4_s9.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].split()
            if not line:
                continue
            if line[0] == "band":
                bands.append(tuple(int(x) for x in line[1:]))
            elif line[0] == "frame0_keys":
                frame0 = [int(x) for x in line[1:]]
            else:
                counts[line[0]] = int(line[1])
    return bands, frame0, counts


def test_toy_example_bands():
    bands, _, _ = _read_toy()
    assert len(bands) == 3
    for delta, r, w in bands:
        assert om.band(delta, 9)[:2] == (r, w)


def test_toy_example_frame0_and_row_counts():
    _, frame0, counts = _read_toy()
    f, s = 4, 9
    q = 2 * s + 4
    got = [b for b in range(s) if om.allowed(q, 0 * s + b, s, sink=False)]
    assert got == frame0
    row_nosink = sum(om.allowed(q, k, s, sink=False) for k in range(f * s))
    row_sink = sum(om.allowed(q, k, s, sink=True) for k in range(f * s))
    assert row_nosink == counts["row_count_nosink"]
    assert row_sink == counts["row_count_sink"]
    # the vectorised brute-force mask agrees with the scalar predicate
    m = om.token_mask(f, s, sink=False)
    assert int(m[q].sum()) == counts["row_count_nosink"]


def test_band_index_exact_at_powers_of_two():
    # floor(log2) must not misround at 2**k or 2**k - 1
    for k in range(0, 40):
        assert om.band_index(2 ** k) == k
        if k >= 1:
            assert om.band_index(2 ** k - 1) == k - 1
    assert om.band_index(0) == 0  # max(delta, 1) for the same frame


def test_central_band_is_distance_one():
    # rebuttal "Width of Central Band": the default central band covers
    # |i - j| <= 1, i.e. r == 0 exactly for delta in {0, 1}
    assert [om.band_index(d) for d in range(5)] == [0, 0, 1, 1, 2]


def test_width_halves_per_band():
    # rebuttal "Width Scale Between Consecutive Bands": scale 2
    s = 3600
    ws = [om.band(2 ** r, s)[1] for r in range(8)]
    assert ws == [3600, 1800, 900, 450, 225, 112, 56, 28]


@pytest.mark.parametrize("sink", [False, True])
def test_closed_form_matches_brute_force(sink):
    for f in list(range(1, 13)) + [17, 33, 37]:
        for s in [1, 2, 3, 5, 9, 16]:
            if f * s > 4000:
                continue
            m = om.token_mask(f, s, sink)
            assert int(m.sum()) == om.closed_form_pairs(f, s, sink), (f, s, sink)


def test_toy_total_pairs():
    # 4 frames x 9 tokens: derived totals of the reading (1116 / 1176 of 1296)
    assert om.closed_form_pairs(4, 9, False) == 1116
    assert om.closed_form_pairs(4, 9, True) == 1176
    assert int(om.token_mask(4, 9, True).sum()) == 1176


def test_n_log_n_growth():
    # abstract / review Fig.2: O(n log n) for fixed s and growing f.  The pair
    # count divided by n*s*log2(2f) stays bounded while the dense count n*n
    # divided by the same grows like f / log f.
    s = 16
    ratios = []
    for f in [8, 16, 32, 64, 128, 256, 512]:
        n = f * s
        pairs = om.closed_form_pairs(f, s, sink=False)
        ratios.append(pairs / (n * s * math.log2(2 * f)))
        assert pairs <= 4 * n * s * (1 + math.log2(max(f, 2)))
    assert max(ratios) < 3.0
    dense_ratio = (512 * s) ** 2 / (512 * s * s * math.log2(1024))
    assert dense_ratio > 10 * max(ratios)


def test_density_constant_across_resolution():
    # rebuttal "Complexity with Respect to Spatial Resolution": at a fixed
    # number of frames the mask sparsity does not depend on resolution
    f = 33
    dens = [om.closed_form_pairs(f, s, True) / (f * s) ** 2 for s in [400, 900, 1600, 3600, 8100]]
    assert max(dens) - min(dens) < 0.01


def test_single_token_frames_give_power_of_two_distances():
    # s == 1: every band has w < 1 beyond distance 1, the sampling keeps
    # distance delta iff delta is a power of two (the LLM-style pattern the
    # review's related-work list mentions)
    f = 40
    m = om.token_mask(f, 1, sink=False)
    dists = sorted({abs(i - j) for i in range(f) for j in range(f) if m[i, j]})
    assert dists == [0, 1, 2, 4, 8, 16, 32]


@pytest.mark.parametrize("s", [3, 5, 6, 7])
def test_sampled_bands_keep_the_halving_density(s):
    # review Step 2-C (paper Fig.5 caption): once a band's width falls below
    # one token, only the diagonal is kept, on a subsample of frame pairs
    # chosen so the band's amortised density keeps the decay of the bands
    # above it, 2^-r.  Read off the brute-force mask at sizes where s is not
    # a power of two (so ceil and floor of 2^r / s differ): every frame-pair
    # block of a sampled band is empty or exactly the diagonal, and the mean
    # density over the band's distances lies in (2^-r / 2, 2^-r].  A
    # subsample that keeps too many distances (a floor instead of the
    # ceiling, say) breaks the upper bound; one that keeps too few breaks
    # the lower.
    f = 128 if s <= 5 else 256
    m = om.token_mask(f, s, sink=False)
    eye = np.eye(s, dtype=bool)
    checked = 0
    for r in range(1, 8):
        lo, hi = 2 ** r, 2 ** (r + 1)
        if lo <= s or hi > f:
            continue  # width >= 1 there, or the band does not fit
        dens = []
        for d in range(lo, hi):
            for i, j in ((0, d), (d, 0), (f - 1 - d, f - 1)):
                blk = m[i * s:(i + 1) * s, j * s:(j + 1) * s]
                assert not blk.any() or np.array_equal(blk, eye), (s, d, i, j)
            dens.append(int(m[0:s, d * s:(d + 1) * s].sum()))
        kept = sum(1 for x in dens if x > 0)
        mean = Fraction(kept, s * (hi - lo))  # each kept block holds s of s^2 pairs
        assert Fraction(1, 2 ** (r + 1)) < mean <= Fraction(1, 2 ** r), (s, r, mean)
        checked += 1
    assert checked >= 3


def test_mask_symmetric_without_sink():
    for f, s in [(5, 7), (9, 4), (17, 3)]:
        m = om.token_mask(f, s, sink=False)
        assert np.array_equal(m, m.T)


def test_sink_column_block():
    f, s = 6, 10
    m = om.token_mask(f, s, sink=True)
    assert m[:, :s].all()


@pytest.mark.parametrize("sink", [False, True])
def test_tile_sweep_matches_bruteforce(sink):
    for f, s, T in [(4, 9, 4), (8, 16, 8), (8, 16, 64), (5, 7, 3), (33, 3, 16),
                    (12, 1, 4), (6, 100, 64), (3, 50, 128), (40, 2, 7), (20, 33, 32)]:
        tok = om.token_mask(f, s, sink)
        a = om.kept_tiles(f, s, T, sink)
        b = om.kept_tiles_bruteforce(tok, T)
        assert a.shape == b.shape
        assert np.array_equal(a, b), (f, s, T, sink)


def test_csr_csc_consistent():
    kept = om.kept_tiles(9, 16, 8, True)
    rp, ci = om.csr(kept)
    cp, ri = om.csc(kept)
    assert rp[-1] == cp[-1] == kept.sum()
    for u in range(kept.shape[0]):
        cols = ci[rp[u]:rp[u + 1]]
        assert np.all(np.diff(cols) > 0)
        assert np.array_equal(cols, np.nonzero(kept[u])[0])
    for v in range(kept.shape[1]):
        rows = ri[cp[v]:cp[v + 1]]
        assert np.array_equal(rows, np.nonzero(kept[:, v])[0])


def test_dense_limit_two_frames():
    # f <= 2: both frame distances are in band 0 with full width, so the
    # mask is the dense n x n mask (the reduction to plain attention)
    for s in [1, 5, 64]:
        assert om.token_mask(2, s, sink=False).all()
        assert om.token_mask(1, s, sink=False).all()


def test_tile_pairs_counts_valid_tokens():
    f, s, T = 5, 7, 4
    kept = om.kept_tiles(f, s, T, True)
    eff = om.effective_mask(f, s, T, True)
    assert om.tile_pairs(kept, f * s, T) == int(eff.sum())


# ---- token-exact semantics: full and partial tiles ----------------------------

@pytest.mark.parametrize("sink", [False, True])
def test_full_tiles_match_bruteforce(sink):
    # interval intersection vs AND-reduction of the brute-force token mask,
    # over shapes with ragged tiles, tiles spanning several frames and the
    # below-unit-width branch (s small, far frames)
    for f, s, T in [(4, 9, 4), (8, 16, 8), (8, 16, 64), (5, 7, 3), (33, 3, 16),
                    (12, 1, 4), (6, 100, 64), (3, 50, 128), (40, 2, 7), (20, 33, 32),
                    (20, 5, 7), (9, 37, 16)]:
        tok = om.token_mask(f, s, sink)
        a = om.full_tiles(f, s, T, sink)
        b = om.full_tiles_bruteforce(tok, T)
        assert np.array_equal(a, b), (f, s, T, sink)
        assert not (a & ~om.kept_tiles(f, s, T, sink)).any()  # full implies kept


def test_full_tiles_dense_limit():
    # f <= 2 allows every pair, so every kept (= every) tile is full
    for f, s, T in [(1, 50, 16), (2, 37, 16), (2, 100, 64)]:
        full = om.full_tiles(f, s, T, sink=False)
        assert full.all()


def test_full_tiles_pair_counts():
    # pairs of full tiles are all allowed and the kept tiles hold every
    # allowed pair: full pairs <= allowed pairs (closed form) <= kept pairs
    f, s, T = 12, 40, 16
    n = f * s
    full = om.full_tiles(f, s, T, True)
    kept = om.kept_tiles(f, s, T, True)
    allowed = om.closed_form_pairs(f, s, True)
    assert om.tile_pairs(full, n, T) <= allowed <= om.tile_pairs(kept, n, T)
    assert 0 < full.sum() < kept.sum()


def test_token_mask_rows_matches_token_mask():
    f, s = 9, 16
    tok = om.token_mask(f, s, True)
    rows = np.array([0, 5, 16, 77, 143])
    assert np.array_equal(om.token_mask_rows(f, s, rows, True), tok[rows])
    assert np.array_equal(om.token_mask_rows(f, s, rows, False), om.token_mask(f, s, False)[rows])


@pytest.mark.parametrize("sink", [False, True])
def test_kept_tiles_of_selected_query_tiles(sink):
    # the sweep restricted to some query tiles gives those rows of the map
    for f, s, T in [(4, 9, 4), (8, 16, 8), (5, 7, 3), (33, 3, 16), (9, 100, 64), (40, 20, 64)]:
        full = om.kept_tiles(f, s, T, sink)
        nb = full.shape[0]
        for tiles in ([0], [nb - 1], list(range(0, nb, 3)), [nb - 1, 0, nb // 2]):
            assert np.array_equal(om.kept_tiles(f, s, T, sink, tiles=tiles), full[tiles]), (f, s, T)
        v = om.Variant(decay="harmonic", central=2)
        assert np.array_equal(om.kept_tiles(f, s, T, sink, v, tiles=[nb - 1, 1]),
                              om.kept_tiles(f, s, T, sink, v)[[nb - 1, 1]])

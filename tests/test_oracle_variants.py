"""Pins for the oracle's mask variants (CPU only).

The variants are the knobs of the rebuttal's ablations (central band width,
width scale between consecutive bands, attention sink) and the
harmonic-series decay the review's Appx C.3 comparison uses.  Widths are
measured from the brute-force token mask, not read from the band table, and
checked against what the pages state about each knob; the closed form, the
tile sweep and the full-tile map are checked against brute force for every
variant.
"""

import math

import numpy as np
import pytest

from oracle import mask as om

V = om.Variant


def _measured_width(m, s, i, j):
    """Half width seen by query (frame i, position 0) in key frame j: the
    allowed keys are positions 0 .. w - 1 when w >= 1 (the run |0 - b| < w
    is clipped only on the left)."""
    row = m[i * s, j * s:(j + 1) * s]
    k = int(row.sum())
    assert row[:k].all() and not row[k:].any(), "not a run starting at 0"
    return k


@pytest.mark.parametrize("d", [0, 1, 2, 3, 4])
def test_central_band_definition(d):
    # rebuttal "Width of Central Band": a central band of width d means
    # frames i and j with |i - j| <= d attend each other (in full)
    f, s = 12, 8
    m = om.token_mask(f, s, sink=False, variant=V(central=d))
    for i in range(f):
        for j in range(f):
            block = m[i * s:(i + 1) * s, j * s:(j + 1) * s]
            assert bool(block.all()) == (abs(i - j) <= d), (d, i, j)


@pytest.mark.parametrize("num,den,s,widths", [
    (3, 2, 81, [81, 54, 36, 24, 16]),
    (2, 1, 64, [64, 32, 16, 8, 4]),
    (3, 1, 81, [81, 27, 9, 3, 1]),
    (4, 1, 256, [256, 64, 16, 4, 1]),
])
def test_width_scale_is_ratio_between_consecutive_bands(num, den, s, widths):
    # rebuttal "Width Scale Between Consecutive Bands": consecutive bands'
    # widths differ by the scale (s chosen so every width is exact)
    f = 17
    m = om.token_mask(f, s, sink=False, variant=V(scale=(num, den)))
    got = [_measured_width(m, s, 0, 2 ** r) for r in range(5)]
    assert got == widths
    for a, b in zip(got, got[1:]):
        assert a * den == b * num
    # (reading) bands keep their doubling extent: one width per band
    for r in range(1, 4):
        ws = {_measured_width(m, s, 0, d) for d in range(2 ** r, 2 ** (r + 1))}
        assert ws == {widths[r]}


def test_harmonic_width_inverse_to_distance():
    # review 1.3.2 / Appx C.3: the harmonic-series pattern's diagonal width is
    # inversely proportional to the frame distance (s = 60 divisible by 1..6)
    f, s = 8, 60
    m = om.token_mask(f, s, sink=False, variant=V(decay="harmonic"))
    assert _measured_width(m, s, 0, 0) == s
    for d in range(1, 7):
        assert _measured_width(m, s, 0, d) * d == s, d
    assert _measured_width(m, s, 0, 7) == 60 // 7


def test_scale_two_written_differently_is_the_default():
    f, s = 20, 12
    a = om.token_mask(f, s, True)
    assert np.array_equal(a, om.token_mask(f, s, True, V(scale=(4, 2))))
    assert np.array_equal(a, om.token_mask(f, s, True, V(central=1, decay="radial")))


@pytest.mark.parametrize("num,den", [(3, 2), (3, 1), (4, 1)])
def test_sampled_density_decays_by_scale(num, den):
    # below unit width the kept share of frame distances in band r, times
    # the diagonal density 1/s, follows c**-r (the reading that continues
    # the decay by the width scale c = num / den).  Read off the brute-force
    # mask (no sink): every frame-pair block of a sampled band is empty or
    # exactly the diagonal, and the number of kept distances in
    # [2**r, 2**(r+1)) lies between half of 2**r * s / c**r minus one (a
    # period below 2 c**r / s) and that value plus one (a period of at least
    # c**r / s).  A period that keeps too many distances (floor instead of
    # ceiling, say) breaks the upper bound, one that keeps too few the lower.
    v = V(scale=(num, den))
    checked = 0
    for s in (1, 2, 3):
        f = 512 if s == 1 else 256
        m = om.token_mask(f, s, sink=False, variant=v)
        eye = np.eye(s, dtype=bool)
        for r in range(1, 9):
            lo, hi = 2 ** r, 2 ** (r + 1)
            if hi > f:
                break
            blocks = [m[0:s, d * s:(d + 1) * s] for d in range(lo, hi)]
            if any(b.any() and not np.array_equal(b, eye) for b in blocks):
                assert all(b.sum() > s for b in blocks if b.any()), (num, den, s, r)
                continue  # width >= 1 here: not the sampled regime
            kept = sum(1 for b in blocks if b.any())
            expect = 2 ** r * s * den ** r / num ** r
            assert expect / 2 - 1 <= kept <= expect + 1, (num, den, s, r, kept, expect)
            checked += 1
    assert checked >= 4


VARIANTS = [V(central=0), V(central=2), V(scale=(3, 2)), V(scale=(3, 1)), V(scale=(4, 1)),
            V(decay="harmonic"), V(decay="harmonic", central=2), V(central=3, scale=(5, 2))]


@pytest.mark.parametrize("variant", VARIANTS, ids=str)
@pytest.mark.parametrize("sink", [False, True])
def test_variant_closed_form_matches_brute_force(variant, sink):
    for f in [1, 2, 3, 5, 9, 17, 33]:
        for s in [1, 2, 3, 7, 16]:
            m = om.token_mask(f, s, sink, variant)
            assert int(m.sum()) == om.closed_form_pairs(f, s, sink, variant), (f, s)
            if f * s <= 60:  # the vectorised mask against the scalar predicate
                n = f * s
                ref = [[om.allowed(q, k, s, sink, variant) for k in range(n)] for q in range(n)]
                assert np.array_equal(m, np.array(ref)), (f, s)


@pytest.mark.parametrize("variant", VARIANTS, ids=str)
def test_variant_tiles_and_full_tiles_match_bruteforce(variant):
    for f, s, T, sink in [(8, 16, 8, True), (5, 7, 3, False), (33, 3, 16, True),
                          (12, 20, 32, False), (40, 2, 8, True), (9, 30, 64, True)]:
        m = om.token_mask(f, s, sink, variant)
        kept = om.kept_tiles(f, s, T, sink, variant)
        assert np.array_equal(kept, om.kept_tiles_bruteforce(m, T)), (f, s, T)
        full = om.full_tiles(f, s, T, sink, variant)
        assert np.array_equal(full, om.full_tiles_bruteforce(m, T)), (f, s, T)
        rows = np.array([0, s, f * s // 2, f * s - 1])
        assert np.array_equal(om.token_mask_rows(f, s, rows, sink, variant), m[rows])


def test_harmonic_is_n_log_n():
    # review 1.3.2: the harmonic-series pattern is the other O(n log n) decay
    s = 16
    ratios = []
    for f in [8, 32, 128, 512]:
        n = f * s
        pairs = om.closed_form_pairs(f, s, False, V(decay="harmonic"))
        ratios.append(pairs / (n * s * math.log2(2 * f)))
    assert max(ratios) < 3.0 and min(ratios) > 0.2


def test_ablation_knobs_move_compute_as_the_rebuttal_explains():
    # rebuttal: a wider central band spends more on nearby frames; a larger
    # width scale limits computation on distant frames.  Counted at the
    # 720p shape (33 x 3600), sink on.
    f, s = 33, 3600
    total = [om.closed_form_pairs(f, s, True, V(central=d)) for d in (0, 1, 2)]
    assert total[0] < total[1] < total[2]

    def far_pairs(v):   # pairs between frames at distance >= 4
        tab = om.band_table(f, s, v)
        out = 0
        for d in range(4, f):
            w, q = int(tab[d, 1]), int(tab[d, 2])
            per = s * (2 * w - 1) - w * (w - 1) if w >= 1 else (s if d % q == 0 else 0)
            out += 2 * (f - d) * per
        return out
    far = [far_pairs(V(scale=c)) for c in [(3, 2), (2, 1), (3, 1), (4, 1)]]
    assert far[0] > far[1] > far[2] > far[3]


def test_variant_rejects_bad_parameters():
    for bad in [dict(central=-1), dict(scale=(2, 2)), dict(scale=(1, 2)), dict(decay="linear")]:
        with pytest.raises(ValueError):
            V(**bad)

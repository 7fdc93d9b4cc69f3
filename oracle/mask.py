"""Oracle for the radial static mask (TEST INFRASTRUCTURE ONLY; see package doc).

Token indexing follows the review, Prompt 1.3.1 "Terms and variables": a video
of f frames with s tokens per frame has n = f*s tokens; token q = i*s + a is
position a (row-major inside the frame) of frame i.  The 4-D mask
M~[i, j, a, b] is flattened to the 2-D mask M[i*s + a, j*s + b] (review,
Step 3; paper Eq.4, §4.2).

Readings taken where the extracted text lost the formulas (each is listed
with its reason in the design notes):

* band index   r = floor(log2(max(|i-j|, 1)))            (review toy example,
  parts A-C; paper §4.2 Fig.5a).  Computed with the integer bit length, never
  with a float log2.
* half width   w = floor(s / 2**r)                        (review toy example;
  paper §4.2 Fig.5b "half-diagonal width").
* spatial test |a - b| < w on the row-major in-frame index (review toy
  example part C: k0=4, w=4 admits l=1..7, so the edge is strict).
* width below one (w == 0): keep only the diagonal a == b, and only for frame
  pairs whose distance is a multiple of ceil(2**r / s), so the amortised
  density of that band is about 1/2**r, the same decay as the bands above it
  (review Step 2-C; paper Fig.5 caption, Eq.4; rebuttal "Whether to Reduce
  the Diagonal Frequency when the Width is below 1").  The pages print no
  numbers for this rule: the tests pin the structure (empty or diagonal
  blocks) and the band density within (2^-r / 2, 2^-r] read off the mask,
  but the exact period inside that bound is parity unpinned.
* attention sink: every query may attend every key of frame 0 (review Step 4;
  paper §4.2, Appx A.1 Eq.8).  Column sink only.
* tile semantics: a T x T tile of the n x n mask is kept when at least one
  allowed token pair falls in it, and a kept tile is computed in full (review
  Step 5; paper §4.2: block-wise computation with 128x128 blocks).

Mask variants (the ablations of the rebuttal and the review's Appx C.3
comparison).  The pages name the knobs but not where they enter the
formulas; these readings are used (``Variant``):

* central band d (rebuttal "Width of Central Band": frame pairs with
  |i - j| <= d attend each other in full): the frame distance is shifted,
  e = max(|i - j| - d + 1, 1), and e takes the place of max(|i - j|, 1) in
  the band index and the widths.  d = 1 is the default mask (distances 0
  and 1 share band 0).
* width scale c = num / den (rebuttal "Width Scale Between Consecutive
  Bands": the ratio between the widths of consecutive bands): bands keep
  their doubling extent, r = floor(log2 e), and the half width becomes
  w = floor(s / c**r); below unit width the sampling period is
  ceil(c**r / s), so the band's amortised density keeps decaying by c.
  c = 2 is the default mask.  (Read this way a larger c starves distant
  frames and a smaller c feeds them, as the rebuttal's explanation of the
  ablation says.)
* harmonic-series decay (review 1.3.2, Appx C.3: the diagonal width is
  inversely proportional to the distance): w = floor(s / e), and below unit
  width the period is ceil(e / s).  The width scale does not apply.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Variant:
    """Mask variant (see the module notes); the defaults give the radial mask."""
    decay: str = "radial"          # "radial" or "harmonic"
    central: int = 1               # central band d >= 0
    scale: tuple = (2, 1)          # width scale c = scale[0] / scale[1] > 1

    def __post_init__(self):
        if self.decay not in ("radial", "harmonic"):
            raise ValueError(self.decay)
        num, den = self.scale
        if self.central < 0 or den < 1 or num <= den:
            raise ValueError(self)


DEFAULT = Variant()


# ----------------------------------------------------------------------------
# Band table (review toy example A-C; paper §4.2 Fig.5a/5b; Fig.5 caption)
# ----------------------------------------------------------------------------

def band_index(delta: int) -> int:
    """r = floor(log2(max(delta, 1))) for an integer frame distance delta >= 0."""
    if delta < 0:
        raise ValueError("frame distance must be >= 0")
    return max(int(delta), 1).bit_length() - 1


def band(delta: int, s: int, variant: Variant = DEFAULT) -> tuple[int, int, int]:
    """(r, w, q) for frame distance delta and s tokens per frame.

    r: band index; w = floor(s / 2**r): half width of the kept diagonal;
    q: diagonal sampling period, only meaningful when w == 0, where a frame
    pair at distance delta keeps its diagonal iff delta % q == 0, with
    q = ceil(2**r / s).  For w >= 1 the period is 1 (no sampling).
    A variant replaces max(delta, 1) by the shifted distance e and the base
    2 of the width by its scale, or takes the harmonic width s / e (module
    notes); r is always floor(log2 e).
    """
    if delta < 0:
        raise ValueError("frame distance must be >= 0")
    e = max(int(delta) - variant.central + 1, 1)
    r = band_index(e)
    if variant.decay == "harmonic":
        num, den = e, 1                     # width divisor e
    else:
        num, den = variant.scale[0] ** r, variant.scale[1] ** r   # divisor c**r
    w = (s * den) // num
    if w >= 1:
        q = 1
    else:
        q = -(-num // (s * den))  # ceil(divisor / s) in integers
    return r, w, q


def band_table(f: int, s: int, variant: Variant = DEFAULT) -> np.ndarray:
    """int64 array [f, 3] with (r, w, q) for every frame distance 0..f-1.
    Periods beyond 2**62 are stored as 2**62 (no distance below f reaches
    them, so the sampled diagonal of such a band is empty either way)."""
    cap = 2 ** 62
    rows = [(r, w, min(q, cap)) for r, w, q in (band(d, s, variant) for d in range(f))]
    return np.array(rows, dtype=np.int64).reshape(f, 3)


# ----------------------------------------------------------------------------
# Token predicate and brute-force mask (review Step 2-4; paper Eq.4, Eq.8)
# ----------------------------------------------------------------------------

def allowed(q: int, k: int, s: int, sink: bool = True, variant: Variant = DEFAULT) -> bool:
    """True iff query token q may attend key token k (scalar, plain Python)."""
    i, a = divmod(q, s)
    j, b = divmod(k, s)
    if sink and j == 0:
        return True
    delta = abs(i - j)
    r, w, period = band(delta, s, variant)
    if w >= 1:
        return abs(a - b) < w
    return a == b and delta % period == 0


def token_mask(f: int, s: int, sink: bool = True, variant: Variant = DEFAULT) -> np.ndarray:
    """Brute-force boolean mask [n, n] (n = f*s), True = allowed.

    Evaluates the same predicate as ``allowed`` for every pair at once; meant
    for n up to a few thousand.
    """
    n = f * s
    if n > 16384:
        raise ValueError("token_mask is brute force; n must be <= 16384")
    idx = np.arange(n)
    i, a = np.divmod(idx, s)
    delta = np.abs(i[:, None] - i[None, :])
    tab = band_table(f, s, variant)
    w = tab[delta, 1]
    period = tab[delta, 2]
    sep = np.abs(a[:, None] - a[None, :])
    near = sep < w
    diag = (sep == 0) & (delta % period == 0)
    m = np.where(w >= 1, near, diag)
    if sink:
        m = m | (i[None, :] == 0)
    return m


def closed_form_pairs(f: int, s: int, sink: bool = True, variant: Variant = DEFAULT) -> int:
    """Number of allowed token pairs, counted per frame pair in closed form.

    For a frame pair at distance delta with half width w >= 1, the number of
    (a, b) in [0, s)^2 with |a - b| < w is s*(2w-1) - w*(w-1) (a band of
    2w-1 diagonals minus the two clipped corner triangles; w <= s always).
    With w == 0 it is s when delta is a multiple of the sampling period, else
    0.  There are f frame pairs at distance 0 and 2*(f - delta) at distance
    delta > 0.  The sink adds, for every query frame i != 0, the pairs of
    frame 0 that the band did not already allow.
    """
    def per_pair(delta: int) -> int:
        r, w, period = band(delta, s, variant)
        if w >= 1:
            return s * (2 * w - 1) - w * (w - 1)
        return s if delta % period == 0 else 0

    total = f * per_pair(0)
    for d in range(1, f):
        total += 2 * (f - d) * per_pair(d)
    if sink:
        # each query frame i >= 1 gains the full frame 0 (s*s pairs) minus
        # what band(i) already allowed toward frame 0
        for i in range(1, f):
            total += s * s - per_pair(i)
    return total


# ----------------------------------------------------------------------------
# Tile cover (review Step 5; paper §4.2 "128x128 blocks")
# ----------------------------------------------------------------------------

def n_blocks(n: int, T: int) -> int:
    return -(-n // T)


def kept_tiles(f: int, s: int, T: int, sink: bool = True,
               variant: Variant = DEFAULT, tiles=None) -> np.ndarray:
    """Boolean [nb, nb] tile map: kept[u, v] iff some allowed (q, k) has
    q // T == u and k // T == v.

    Built by sweeping every (query token, key frame) pair: the keys of frame j
    that query q = (i, a) may attend form one contiguous run of positions
    (|a - b| < w, or the single b == a, or all of frame 0 for the sink), so
    they cover a contiguous run of key tiles.  Each run is marked in a
    per-query-tile difference array and a prefix sum gives the union.

    ``tiles``: optional list of query tiles; the sweep then covers only their
    query tokens and the result has one row per listed tile,
    [len(tiles), nb] (for sequences whose full map would not fit in memory).
    """
    n = f * s
    nb = n_blocks(n, T)
    tab = band_table(f, s, variant)
    if tiles is None:
        qtok = np.arange(n, dtype=np.int64)
        qtile = qtok // T
        n_rows = nb
    else:
        tiles = [int(u) for u in tiles]
        qtok = np.concatenate([np.arange(u * T, min(n, (u + 1) * T), dtype=np.int64)
                               for u in tiles])
        qtile = np.concatenate([np.full(min(n, (u + 1) * T) - u * T, r, dtype=np.int64)
                                for r, u in enumerate(tiles)])
        n_rows = len(tiles)
    qi, qa = np.divmod(qtok, s)
    cover = np.zeros((n_rows, nb + 1), dtype=np.int64)
    flat = cover.reshape(-1)
    starts: list[np.ndarray] = []
    ends: list[np.ndarray] = []
    pending = 0
    for j in range(f):
        delta = np.abs(qi - j)
        w = tab[delta, 1]
        period = tab[delta, 2]
        lo = np.where(w >= 1, np.maximum(qa - w + 1, 0), qa)
        hi = np.where(w >= 1, np.minimum(qa + w - 1, s - 1), qa)
        has = (w >= 1) | (delta % period == 0)
        if sink and j == 0:
            lo = np.zeros_like(qa)
            hi = np.full_like(qa, s - 1)
            has = np.ones_like(has)
        klo = (j * s + lo) // T
        khi = (j * s + hi) // T
        rows = qtile[has]
        starts.append(rows * (nb + 1) + klo[has])
        ends.append(rows * (nb + 1) + khi[has] + 1)
        pending += rows.size
        if pending > 8_000_000 or j == f - 1:
            flat += np.bincount(np.concatenate(starts), minlength=flat.size)
            flat -= np.bincount(np.concatenate(ends), minlength=flat.size)
            starts, ends, pending = [], [], 0
    return np.cumsum(cover, axis=1)[:, :nb] > 0


def kept_tiles_bruteforce(mask: np.ndarray, T: int) -> np.ndarray:
    """OR-reduce a token mask [n, n] over T x T tiles (ragged last tile)."""
    n = mask.shape[0]
    nb = n_blocks(n, T)
    pad = nb * T - n
    m = np.pad(mask, ((0, pad), (0, pad)))
    return m.reshape(nb, T, nb, T).any(axis=(1, 3))


def csr(kept: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """CSR of the kept map: per query tile, ascending kept key tiles."""
    counts = kept.sum(axis=1)
    row_ptr = np.zeros(kept.shape[0] + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(kept)[1]
    return row_ptr, col_idx.astype(np.int64)


def csc(kept: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """CSC of the kept map: per key tile, ascending query tiles."""
    return csr(kept.T)


def tile_pairs(kept: np.ndarray, n: int, T: int) -> int:
    """Valid token pairs inside kept tiles (rows and columns clipped to n)."""
    nb = kept.shape[0]
    size = np.full(nb, T, dtype=np.int64)
    size[-1] = n - (nb - 1) * T
    return int(size @ kept.astype(np.int64) @ size)


def effective_mask(f: int, s: int, T: int, sink: bool = True,
                   mode: str = "tile", variant: Variant = DEFAULT) -> np.ndarray:
    """Boolean [n, n] mask the attention uses (small n only).

    mode "tile": every token pair inside a kept tile (tile semantics).
    mode "token": exactly the allowed token pairs.
    """
    tok = token_mask(f, s, sink, variant)
    if mode == "token":
        return tok
    if mode != "tile":
        raise ValueError(mode)
    n = f * s
    kept = kept_tiles_bruteforce(tok, T)
    t = np.arange(n) // T
    return kept[t[:, None], t[None, :]]


# ----------------------------------------------------------------------------
# Token-exact semantics: full and partial tiles (paper Eq.4 at token
# granularity; review Step 3, "4-D mask" flattened).  Under token-exact
# semantics a kept tile is computed with the token predicate applied inside
# it; a tile in which every valid token pair is allowed needs no masking.
# ----------------------------------------------------------------------------

def full_tiles(f: int, s: int, T: int, sink: bool = True,
               variant: Variant = DEFAULT) -> np.ndarray:
    """Boolean [nb, nb] tile map: full[u, v] iff tile (u, v) is kept and every
    token pair (q, k) in it with q, k < n is allowed.

    For a query q = (i, a) the allowed keys of frame j form one contiguous run
    of positions b (see ``kept_tiles``), possibly empty.  The keys of frame j
    that every query of tile u may attend are the intersection of those runs.
    Tile v is full iff, for every frame j its keys fall in, those keys lie
    inside the intersection for frame j.
    """
    n = f * s
    nb = n_blocks(n, T)
    tab = band_table(f, s, variant)
    kept = kept_tiles(f, s, T, sink, variant)
    full = np.zeros_like(kept)
    q = np.arange(n, dtype=np.int64)
    qi, qa = np.divmod(q, s)
    for u in range(nb):
        rows = slice(u * T, min(n, (u + 1) * T))
        i, a = qi[rows], qa[rows]
        common_lo = np.zeros(f, dtype=np.int64)
        common_hi = np.full(f, -1, dtype=np.int64)      # empty by default
        for j in range(f):
            delta = np.abs(i - j)
            w = tab[delta, 1]
            period = tab[delta, 2]
            lo = np.where(w >= 1, np.maximum(a - w + 1, 0), a)
            hi = np.where(w >= 1, np.minimum(a + w - 1, s - 1), a)
            has = (w >= 1) | (delta % period == 0)
            if sink and j == 0:
                lo = np.zeros_like(a)
                hi = np.full_like(a, s - 1)
                has = np.ones_like(has)
            if has.all():
                common_lo[j] = lo.max()
                common_hi[j] = hi.min()
        for v in np.nonzero(kept[u])[0]:
            k0, k1 = v * T, min(n, (v + 1) * T) - 1
            ok = True
            for j in range(k0 // s, k1 // s + 1):
                b0 = max(k0, j * s) - j * s
                b1 = min(k1, (j + 1) * s - 1) - j * s
                if not (common_lo[j] <= b0 and b1 <= common_hi[j]):
                    ok = False
                    break
            full[u, v] = ok
    return full


def full_tiles_bruteforce(mask: np.ndarray, T: int) -> np.ndarray:
    """AND-reduce a token mask [n, n] over T x T tiles, counting only the
    valid pairs of ragged tiles, restricted to kept tiles."""
    n = mask.shape[0]
    nb = n_blocks(n, T)
    pad = nb * T - n
    m = np.pad(mask, ((0, pad), (0, pad)), constant_values=True)
    allowed_all = m.reshape(nb, T, nb, T).all(axis=(1, 3))
    return allowed_all & kept_tiles_bruteforce(mask, T)


def token_mask_rows(f: int, s: int, rows: np.ndarray, sink: bool = True,
                    variant: Variant = DEFAULT) -> np.ndarray:
    """Boolean [len(rows), n]: the token predicate for the given query rows
    against every key (the same predicate as ``allowed``, vectorised)."""
    n = f * s
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.arange(n, dtype=np.int64)
    i, a = np.divmod(rows, s)
    j, b = np.divmod(keys, s)
    delta = np.abs(i[:, None] - j[None, :])
    tab = band_table(f, s, variant)
    w = tab[delta, 1]
    period = tab[delta, 2]
    sep = np.abs(a[:, None] - b[None, :])
    m = np.where(w >= 1, sep < w, (sep == 0) & (delta % period == 0))
    if sink:
        m = m | (j[None, :] == 0)
    return m

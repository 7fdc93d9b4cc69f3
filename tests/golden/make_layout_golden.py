"""Writes tests/golden/layouts.json from the oracle only.

For every workload shape (and a few small ones), and for the mask variants
of the ablations at the 720p shape, it stores the tile count,
the valid token pairs inside kept tiles, SHA-256 digests of the CSR and
CSC arrays as little-endian int32, and digests of the full-tile marks in
CSR and CSC order (one byte per kept tile, 1 = every valid pair allowed), so the C++ mask compiler can be checked
bit-exactly without recomputing the oracle at full size in every test run.

Run from the repository root:  python tests/golden/make_layout_golden.py
"""

import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import mask as om  # noqa: E402

SHAPES = [
    # (frames, tokens_per_frame, tile)
    (8, 256, 64), (33, 3600, 128), (21, 3600, 128), (129, 3600, 128), (66, 3600, 128),
    (4, 9, 4), (66, 256, 128), (2, 300, 128), (40, 1, 8), (600, 3, 16), (17, 100, 64),
]


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()


def digest_u8(a):
    return hashlib.sha256(np.ascontiguousarray(a, dtype=np.uint8).tobytes()).hexdigest()


# mask variants of the ablations, at the 720p shape and a small one (sink on)
VARIANT_SHAPES = [(33, 3600, 128), (8, 256, 64)]
VARIANTS = [om.Variant(central=0), om.Variant(central=2), om.Variant(scale=(3, 2)),
            om.Variant(scale=(3, 1)), om.Variant(scale=(4, 1)), om.Variant(decay="harmonic")]


def entry(f, s, T, sink, v):
    kept = om.kept_tiles(f, s, T, sink, v)
    rp, ci = om.csr(kept)
    cp, ri = om.csc(kept)
    full = om.full_tiles(f, s, T, sink, v)
    return dict(frames=f, tokens_per_frame=s, tile=T, sink=sink,
                variant=dict(decay=v.decay, central=v.central, scale=list(v.scale)),
                n_blocks=int(kept.shape[0]), nnz_tiles=int(kept.sum()),
                nnz_pairs=om.tile_pairs(kept, f * s, T),
                row_ptr=digest(rp), col_idx=digest(ci),
                col_ptr=digest(cp), row_idx=digest(ri),
                n_full=int(full.sum()),
                csr_full=digest_u8(full[kept]),
                csc_full=digest_u8(full.T[kept.T]))


def main():
    out = []
    for f, s, T in SHAPES:
        for sink in (True, False):
            kept = om.kept_tiles(f, s, T, sink)
            rp, ci = om.csr(kept)
            cp, ri = om.csc(kept)
            full = om.full_tiles(f, s, T, sink)
            out.append(dict(frames=f, tokens_per_frame=s, tile=T, sink=sink,
                            n_blocks=int(kept.shape[0]), nnz_tiles=int(kept.sum()),
                            nnz_pairs=om.tile_pairs(kept, f * s, T),
                            row_ptr=digest(rp), col_idx=digest(ci),
                            col_ptr=digest(cp), row_idx=digest(ri),
                            n_full=int(full.sum()),
                            csr_full=digest_u8(full[kept]),
                            csc_full=digest_u8(full.T[kept.T])))
    for f, s, T in VARIANT_SHAPES:
        for v in VARIANTS:
            out.append(entry(f, s, T, True, v))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "layouts.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()

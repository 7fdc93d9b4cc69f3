"""GPU parity of the mask variants against the oracle (needs an MI355X).

The variants (central band d, width scale c, harmonic-series decay) change
the layout the mask compiler emits and, under token-exact semantics, the
predicate the kernels apply inside partial tiles.  Small shapes are compared
element by element (forward and backward) in both modes; the 720p workload
on sampled query tiles for two variants.
"""

import sys

import numpy as np
import pytest
import torch

import static_block_sparse_amd as sba
import workloads
from gpu_util import check_close, check_lse, f64, sample_tiles
from oracle import attention as oa
from oracle import mask as om

pytestmark = pytest.mark.gpu

V = om.Variant


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _layout(f, s, T, v, **kw):
    return sba.Layout(f, s, T, decay=v.decay, central_band=v.central, width_scale=v.scale, **kw)


VARIANTS = [V(central=0), V(central=2), V(scale=(3, 2)), V(scale=(3, 1)), V(scale=(4, 1)),
            V(decay="harmonic"), V(decay="harmonic", central=2), V(central=3, scale=(5, 2))]
SHAPES = [
    # f, s, T, D, sink
    (9, 200, 128, 128, True),    # tiles straddle frames, ragged last tile
    (40, 20, 64, 64, False),     # frames shorter than a chunk, sink off
    (130, 3, 64, 64, True),      # below unit width: sampled diagonals
]


@pytest.mark.parametrize("variant", VARIANTS, ids=str)
@pytest.mark.parametrize("exact", [False, True])
def test_variant_small(variant, exact):
    for f, s, T, D, sink in SHAPES:
        scale = 1.0 / np.sqrt(D)
        _say(f"[variant] {variant} exact={exact} f={f} s={s} T={T} D={D} sink={sink}")
        q, k, v, do = workloads.make_inputs(1, 2, f * s, D, 700 + f, with_dout=True)
        L = _layout(f, s, T, variant, sink=sink, token_exact=exact)
        qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
        o, lse = sba.attn_fwd(qc, kc, vc, L, scale)
        dq, dk, dv = sba.attn_bwd(qc, kc, vc, o, lse, dc, L, scale)
        torch.cuda.synchronize()
        mask = om.effective_mask(f, s, T, sink, "token" if exact else "tile", variant)
        for h in range(2):
            qh, kh, vh, dh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h])
            ro, rl = oa.fwd_masked(qh, kh, vh, mask, scale)
            check_close(f64(o[0, h]), ro, f"O h={h}")
            check_lse(f64(lse[0, h]), rl)
            rq, rk, rv = oa.bwd_masked(qh, kh, vh, dh, mask, scale)
            check_close(f64(dq[0, h]), rq, f"dQ h={h}", normalise=True)
            check_close(f64(dk[0, h]), rk, f"dK h={h}", normalise=True)
            check_close(f64(dv[0, h]), rv, f"dV h={h}", normalise=True)


@pytest.mark.parametrize("variant,exact", [(V(decay="harmonic"), True), (V(scale=(3, 2)), False)],
                         ids=["harmonic-exact", "scale1.5-tile"])
def test_variant_full_size_sampled(variant, exact):
    """720p (33 x 3600, 24 heads) in one launch: forward O/LSE and dQ on
    sampled query tiles of the first and last heads."""
    w = workloads.WORKLOADS["hunyuan_5s_720p"]
    _say(f"[variant-full] {variant} exact={exact}")
    q, k, v, do = workloads.workload_inputs(w, with_dout=True, device="cuda")
    L = _layout(w.frames, w.tokens_per_frame, w.T, variant, token_exact=exact)
    o, lse = sba.attn_fwd(q, k, v, L, w.scale)
    dq, _, _ = sba.attn_bwd(q, k, v, o, lse, do, L, w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(dq.float()).all())
    kept = om.kept_tiles(w.frames, w.tokens_per_frame, w.T, True, variant)
    for h in (0, w.H - 1):
        qh, kh, vh, dh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h])
        for u in sample_tiles(w.N, w.T, w.tokens_per_frame, seed=w.seed)[:4]:
            rows = np.arange(u * w.T, min(w.N, (u + 1) * w.T))
            if exact:
                m = om.token_mask_rows(w.frames, w.tokens_per_frame, rows, True, variant)
            else:
                cols = oa.tile_columns(kept[u], w.N, w.T)
                m = np.zeros((rows.size, w.N), dtype=bool)
                m[:, cols] = True
            ro, rl = oa.fwd_masked(qh[rows], kh, vh, m, w.scale)
            check_close(f64(o[0, h, rows]), ro, f"O h={h} tile={u}")
            check_lse(f64(lse[0, h, rows]), rl, f"lse h={h} tile={u}")
            rq = oa.bwd_masked(qh[rows], kh, vh, dh[rows], m, w.scale)[0]
            check_close(f64(dq[0, h, rows]), rq, f"dQ h={h} tile={u}", normalise=True)

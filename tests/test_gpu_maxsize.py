"""GPU parity at the longest sequence the boundary accepts (needs an MI355X).

One (batch, head) slice of N * D bf16 values must stay below 2^31 bytes.  At
D = 128 the test takes 2047 frames of 4097 tokens, N = 8,386,559 (2,048 short
of the limit, 8,388,607): 65,520 query tiles of 128, the last one 127 rows,
tiles straddling frames, and 340,303,451 kept tiles (about 5,200 per row).
Forward and backward run once on B = H = 1; O, LSE and dQ are compared element by element with the oracle on
sampled query tiles (first, last, the first frame-straddling tile, two
random), the oracle's tile cover swept over those tiles only; dK and dV are
checked through identities that hold at any size (sum_n dV[n] = sum_m dO[m],
sum_n dK[n] = 0).
"""

import sys

import numpy as np
import pytest
import torch

import static_block_sparse_amd as sba
from gpu_util import check_close, check_lse, nan_outputs, sample_tiles
from oracle import attention as oa
from oracle import mask as om

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.timeout(900)
def test_longest_supported_sequence():
    f, s, T, D = 2047, 4097, 128, 128
    N = f * s
    assert N * D * 2 < 2 ** 31 <= (N + s) * D * 2 + s * D * 2
    scale = 1.0 / np.sqrt(D)
    _say(f"[maxsize] building the layout: {f} frames x {s} tokens, N = {N}")
    L = sba.Layout(f, s, T)
    _say(f"[maxsize] {L.nnz_tiles} kept tiles ({L.nnz_tiles / L.n_blocks:.0f} per row)")
    g = torch.Generator("cuda").manual_seed(2047)
    q, k, v, do = (torch.randn((1, 1, N, D), generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(4))
    o, lse, dq, dk, dv = nan_outputs(1, 1, N, D)
    sba.attn_fwd(q, k, v, L, scale, out=o, lse=lse)
    torch.cuda.synchronize()
    _say("[maxsize] forward done")
    sba.attn_bwd(q, k, v, o, lse, do, L, scale, out=(dq, dk, dv))
    torch.cuda.synchronize()
    _say("[maxsize] backward done")
    # the outputs started as NaN: every row was written
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    # identities over the whole sequence (see test_gpu_bwd for the tolerance)
    sdv, sdo = dv.double().sum(dim=2), do.double().sum(dim=2)
    rms = max(float(dv.double().pow(2).mean().sqrt()), float(do.double().pow(2).mean().sqrt()))
    assert float((sdv - sdo).abs().max()) <= 4 * np.sqrt(N) * 2.0 ** -8 * rms
    rms_dk = float(dk.double().pow(2).mean().sqrt())
    assert float(dk.double().sum(dim=2).abs().max()) <= 4 * np.sqrt(N) * 2.0 ** -8 * rms_dk + 1e-6
    # sampled query tiles against the oracle
    tiles = sample_tiles(N, T, s, seed=11)
    kept = om.kept_tiles(f, s, T, True, tiles=tiles)
    qc, kc, vc, dc = (t[0, 0].cpu() for t in (q, k, v, do))
    oc, lc, dqc = o[0, 0].cpu(), lse[0, 0].cpu(), dq[0, 0].cpu()
    for r, u in enumerate(tiles):
        rows = slice(u * T, min(N, (u + 1) * T))
        cols = torch.from_numpy(oa.tile_columns(kept[r], N, T))
        k64, v64 = (x[cols].to(torch.float64).numpy() for x in (kc, vc))
        q64, d64 = (x[rows].to(torch.float64).numpy() for x in (qc, dc))
        ro, rl = oa.fwd_rows(q64, k64, v64, scale)
        check_close(oc[rows].to(torch.float64).numpy(), ro, f"O tile={u}")
        check_lse(lc[rows].to(torch.float64).numpy(), rl, f"LSE tile={u}")
        rq = oa.dq_rows(q64, k64, v64, d64, scale)
        check_close(dqc[rows].to(torch.float64).numpy(), rq, f"dQ tile={u}", normalise=True)
        _say(f"[maxsize] tile {u} ({len(cols)} keys): O, LSE, dQ match")

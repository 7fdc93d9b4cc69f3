"""GPU parity of token-exact mode against the oracle (needs an MI355X).

With ``Layout(..., token_exact=True)`` the kernels apply the token predicate
inside the kept tiles the mask only partly covers, so forward and backward
must equal plain attention under the token mask (oracle ``fwd_masked`` /
``bwd_masked`` with ``token_mask``).  Small shapes are compared element by
element over every head; the full-size 720p workload and the 129-frame one
(where more than half of the kept tiles are partial) on sampled query rows
(forward O/LSE and dQ) and through the gradient identities, and at 720p dK
and dV element by element on sampled key tiles.
"""

import sys

import numpy as np
import pytest
import torch

import static_block_sparse_amd as sba
import workloads
from gpu_util import check_close, check_lse, f64, nan_outputs, sample_tiles
from oracle import attention as oa
from oracle import mask as om

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


SHAPES = [
    # f, s, T, D, B, H
    (8, 256, 64, 64, 1, 2),      # the tiny workload's shape
    (5, 300, 128, 128, 2, 2),    # ragged last tile; tiles straddle frames
    (7, 100, 64, 64, 1, 2),      # ragged; 64-tiles span frames
    (3, 40, 128, 128, 1, 1),     # a single partial tile
    (40, 20, 64, 64, 1, 1),      # narrow bands: most kept tiles partial
    (40, 20, 128, 64, 1, 1),     # head dim 64 with 128-wide tiles
    (300, 2, 64, 64, 1, 1),      # width below one: the sampled diagonal
    (33, 36, 128, 128, 1, 1),    # 3-4 frames per tile
]


def _inputs(f, s, D, B, H, seed):
    return workloads.make_inputs(B, H, f * s, D, seed, with_dout=True)


@pytest.mark.parametrize("f,s,T,D,B,H", SHAPES)
@pytest.mark.parametrize("sink", [True, False])
def test_exact_forward_and_backward_small(f, s, T, D, B, H, sink):
    scale = 1.0 / np.sqrt(D)
    _say(f"[exact] f={f} s={s} T={T} D={D} B={B} H={H} sink={sink}")
    q, k, v, do = _inputs(f, s, D, B, H, 500 + f)
    L = sba.Layout(f, s, T, sink=sink, token_exact=True)
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = sba.attn_fwd(qc, kc, vc, L, scale)
    dq, dk, dv = sba.attn_bwd(qc, kc, vc, o, lse, dc, L, scale)
    torch.cuda.synchronize()
    mask = om.token_mask(f, s, sink)
    for b in range(B):
        for h in range(H):
            qh, kh, vh, dh = f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h])
            ro, rl = oa.fwd_masked(qh, kh, vh, mask, scale)
            check_close(f64(o[b, h]), ro, f"O b={b} h={h}")
            check_lse(f64(lse[b, h]), rl)
            rq, rk, rv = oa.bwd_masked(qh, kh, vh, dh, mask, scale)
            check_close(f64(dq[b, h]), rq, f"dQ b={b} h={h}", normalise=True)
            check_close(f64(dk[b, h]), rk, f"dK b={b} h={h}", normalise=True)
            check_close(f64(dv[b, h]), rv, f"dV b={b} h={h}", normalise=True)


def test_tile_mode_differs_from_the_token_oracle():
    # the shape has partial tiles, so tile semantics must fail the token
    # comparison: the exact-mode test above can tell the two apart
    f, s, T, D = 40, 20, 64, 64
    scale = 1.0 / np.sqrt(D)
    q, k, v, _ = _inputs(f, s, D, 1, 1, 540)
    assert not om.full_tiles(f, s, T)[om.kept_tiles(f, s, T)].all()
    o, lse = sba.attn_fwd(q.cuda(), k.cuda(), v.cuda(), sba.Layout(f, s, T), scale)
    ro, _ = oa.fwd_masked(f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0]), om.token_mask(f, s), scale)
    with pytest.raises(AssertionError):
        check_close(f64(o[0, 0]), ro, "tile-mode O vs token oracle")


def test_all_full_tiles_match_tile_mode():
    # two frames: every pair is allowed, so every kept tile is full and
    # token-exact mode must give what tile mode gives
    f, s, T, D = 2, 700, 128, 128
    q, k, v, do = (t.cuda() for t in _inputs(f, s, D, 1, 2, 550))
    a, b = sba.Layout(f, s, T), sba.Layout(f, s, T, token_exact=True)
    assert all(x.all() for x in b.tile_flags())
    oa_, la = sba.attn_fwd(q, k, v, a)
    ob, lb = sba.attn_fwd(q, k, v, b)
    ga = sba.attn_bwd(q, k, v, oa_, la, do, a)
    gb = sba.attn_bwd(q, k, v, ob, lb, do, b)
    torch.cuda.synchronize()
    assert torch.equal(oa_, ob) and torch.equal(la, lb)
    for x, y in zip(ga, gb):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["hunyuan_5s_720p", "hunyuan_4x_long"])
def test_exact_full_size_sampled_rows(name):
    """720p (33 frames) and 129 frames of 3600 tokens, 24 heads in one launch:
    O, LSE and dQ on sampled query tiles of the first and last heads against
    the token oracle; dK and dV through identities that hold at any size."""
    w = workloads.WORKLOADS[name]
    _say(f"[exact-full] B={w.B} H={w.H} N={w.N} D={w.D}")
    q, k, v, do = workloads.workload_inputs(w, with_dout=True, device="cuda")
    L = sba.Layout(w.frames, w.tokens_per_frame, w.T, token_exact=True)
    o, lse, dq, dk, dv = nan_outputs(w.B, w.H, w.N, w.D)
    sba.attn_fwd(q, k, v, L, w.scale, out=o, lse=lse)
    sba.attn_bwd(q, k, v, o, lse, do, L, w.scale, out=(dq, dk, dv))
    torch.cuda.synchronize()
    # the outputs started as NaN: every row was written
    for t in (o, lse, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    tiles = sample_tiles(w.N, w.T, w.tokens_per_frame, seed=w.seed)
    for h in (0, w.H - 1):
        qh, kh, vh, dh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h])
        for u in tiles:
            rows = np.arange(u * w.T, min(w.N, (u + 1) * w.T))
            m = om.token_mask_rows(w.frames, w.tokens_per_frame, rows)
            ro, rl = oa.fwd_masked(qh[rows], kh, vh, m, w.scale)
            check_close(f64(o[0, h, rows]), ro, f"O h={h} tile={u}")
            check_lse(f64(lse[0, h, rows]), rl, f"lse h={h} tile={u}")
            # a query row's dQ depends only on its own softmax row
            rq = oa.dq_masked(qh[rows], kh, vh, dh[rows], m, w.scale)
            check_close(f64(dq[0, h, rows]), rq, f"dQ h={h} tile={u}", normalise=True)
    # every softmax row sums to one: sum_n dV[n] = sum_m dO[m]; each dS row
    # sums to zero: sum_n dK[n] = 0.  Each of N bf16-rounded terms is off by
    # <= 2^-8 relative, so the sums' errors grow like sqrt(N) * 2^-8 * rms (4x margin).
    sdv, sdo = dv.double().sum(dim=2), do.double().sum(dim=2)
    rms = max(float(dv.double().pow(2).mean().sqrt()), float(do.double().pow(2).mean().sqrt()))
    tol = 4 * np.sqrt(w.N) * 2.0 ** -8 * rms
    assert float((sdv - sdo).abs().max()) <= tol, (float((sdv - sdo).abs().max()), tol)
    rms_dk = float(dk.double().pow(2).mean().sqrt())
    assert float(dk.double().sum(dim=2).abs().max()) <= 4 * np.sqrt(w.N) * 2.0 ** -8 * rms_dk + 1e-6


@pytest.mark.timeout(900)
def test_exact_full_size_dkdv_tiles():
    """720p (33 frames x 3600 tokens, 24 heads in one launch) in token-exact
    mode: dK and dV element by element against the token oracle on key
    tiles 0 (the sink: every query row attends all of its keys), 28
    (straddles frames 0 and 1), the last, partial tile (16 keys) and one
    random tile of the first head, and the last tile of the last head.  Each
    attending row's LSE and Delta come from its own allowed keys (within its
    kept tiles, which hold all of them)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    w = workloads.WORKLOADS["hunyuan_5s_720p"]
    f, s, T, n = w.frames, w.tokens_per_frame, w.T, w.N
    _say(f"[exact-dkdv] B={w.B} H={w.H} N={n} D={w.D}")
    q, k, v, do = workloads.workload_inputs(w, with_dout=True, device="cuda")
    L = sba.Layout(f, s, T, token_exact=True)
    o, lse, dq, dk, dv = nan_outputs(w.B, w.H, n, w.D)
    sba.attn_fwd(q, k, v, L, w.scale, out=o, lse=lse)
    sba.attn_bwd(q, k, v, o, lse, do, L, w.scale, out=(dq, dk, dv))
    torch.cuda.synchronize()
    kept = om.kept_tiles(f, s, T, True)
    nb = kept.shape[0]
    frame0_tiles = -(-s // T)
    rand = int(np.random.default_rng(11).integers(frame0_tiles, nb - 1))
    cases = {0: [0, frame0_tiles - 1, nb - 1, rand], w.H - 1: [nb - 1]}
    key_range = {vt: slice(vt * T, min(n, (vt + 1) * T)) for vt in range(nb)}
    workers = 16
    for h, tiles in cases.items():
        qh, kh, vh, dh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h])
        need = sorted(set(int(u) for vt in tiles for u in np.nonzero(kept[:, vt])[0]))
        _say(f"[exact-dkdv] head {h}: key tiles {tiles}, row terms of {len(need)} query tiles")

        def block_of(u):
            rows = np.arange(u * T, min(n, (u + 1) * T))
            cols = oa.tile_columns(kept[u], n, T)
            m = om.token_mask_rows(f, s, rows)
            lse_u, delta_u = oa.row_stats_masked(qh[rows], kh[cols], vh[cols], dh[rows],
                                                 m[:, cols], w.scale)
            return u, rows, lse_u, delta_u, {vt: m[:, key_range[vt]] for vt in tiles
                                             if kept[u, vt]}

        blocks = {vt: [] for vt in tiles}
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            for u, rows, lse_u, delta_u, allowed in ex.map(block_of, need):
                for vt, a in allowed.items():
                    blocks[vt].append((rows, a, lse_u, delta_u))
        for vt in tiles:
            keys = key_range[vt]
            rk, rv = oa.dkdv_masked_keys(qh, kh, vh, dh, keys, blocks[vt], w.scale)
            sk = check_close(f64(dk[0, h, keys]), rk, f"dK h={h} key tile={vt}", normalise=True)
            sv = check_close(f64(dv[0, h, keys]), rv, f"dV h={h} key tile={vt}", normalise=True)
            _say(f"[exact-dkdv] head {h} key tile {vt} ({len(blocks[vt])} query tiles): "
                 f"dK max {sk['max_abs']:.3g} (rms {sk['rms_ref']:.3g}), "
                 f"dV max {sv['max_abs']:.3g} (rms {sv['rms_ref']:.3g})")

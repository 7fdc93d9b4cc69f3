"""GPU parity of the backward pass against the oracle (needs an MI355X).

Small shapes: dQ, dK, dV compared element by element over every head.
Full-size training workload (66 frames x 3600 tokens, 24 heads): dQ on
sampled query tiles and dK, dV on sampled key tiles (the sink column of the
whole sequence included) element by element against the oracle, plus
identities that hold at any size: sum_n dV[n] = sum_m dO[m] (softmax rows
sum to one) and sum_n dK[n] = 0 (each row of dS sums to zero).
"""

import os
import sys

import numpy as np
import pytest
import torch

import static_block_sparse_amd as sba
import workloads
from gpu_util import PEAKY_REL_MAX, check_close, check_lse, f64, nan_outputs, sample_tiles
from oracle import attention as oa
from oracle import mask as om

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("f,s,T,D,B,H", [
    (8, 256, 64, 64, 1, 2),      # the tiny workload's shape
    (5, 300, 128, 128, 2, 2),    # ragged: last tile 92 rows
    (7, 100, 64, 64, 1, 2),      # ragged: last tile 60 rows
    (3, 40, 128, 128, 1, 1),     # one partial tile
    (66, 256, 128, 128, 1, 1),   # the training workload's frame count at s = 256
    (5, 300, 128, 64, 1, 2),     # head dim 64 with 128-wide tiles
    (9, 100, 128, 64, 2, 1),     # head dim 64 with 128-wide tiles, odd number of tiles
])
def test_backward_small(f, s, T, D, B, H):
    N = f * s
    scale = 1.0 / np.sqrt(D)
    _say(f"[bwd] f={f} s={s} T={T} D={D} B={B} H={H}")
    q, k, v, do = workloads.make_inputs(B, H, N, D, 100 + f, with_dout=True)
    L = sba.Layout(f, s, T)
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = sba.attn_fwd(qc, kc, vc, L, scale)
    dq, dk, dv = sba.attn_bwd(qc, kc, vc, o, lse, dc, L, scale)
    torch.cuda.synchronize()
    kept = om.kept_tiles(f, s, T, True)
    for b in range(B):
        for h in range(H):
            rq, rk, rv = oa.bwd(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h]), kept, T,
                                scale)
            check_close(f64(dq[b, h]), rq, f"dQ b={b} h={h}", normalise=True)
            check_close(f64(dk[b, h]), rk, f"dK b={b} h={h}", normalise=True)
            check_close(f64(dv[b, h]), rv, f"dV b={b} h={h}", normalise=True)


# Columns of 1 .. 9 query chunks (64 rows each): the dK/dV walk has a two-step
# prologue, a loop unrolled over its four chunk buffers and a drain, so every
# column length modulo 4 and the shortest columns take different paths.
# (f, s, chunks per column): single-frame and two-frame layouts are dense.
SHORT_COLUMNS = [(1, 20, 1), (1, 70, 2), (1, 130, 3), (1, 200, 4), (1, 260, 5), (1, 330, 6),
                 (1, 390, 7), (2, 230, 8), (2, 260, 9)]


@pytest.mark.parametrize("f,s,n_chunks", SHORT_COLUMNS)
def test_backward_short_columns(f, s, n_chunks):
    T, D = 128, 128
    N = f * s
    nb = (N + T - 1) // T
    L = sba.Layout(f, s, T)
    col_ptr, row_idx = L.csc()
    col_ptr = np.asarray(col_ptr)
    last = np.asarray(row_idx)[col_ptr[1:] - 1] & 0x7fffffff
    chunks = (np.diff(col_ptr) * 2 - np.where(last == nb - 1, 2 - (N - (nb - 1) * T + 63) // 64, 0))
    _say(f"[bwd short] f={f} s={s} chunks per column {sorted(set(chunks.tolist()))}")
    assert set(chunks.tolist()) == {n_chunks}
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = workloads.make_inputs(1, 1, N, D, 300 + s, with_dout=True)
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = sba.attn_fwd(qc, kc, vc, L, scale)
    dq, dk, dv = sba.attn_bwd(qc, kc, vc, o, lse, dc, L, scale)
    torch.cuda.synchronize()
    kept = om.kept_tiles(f, s, T, True)
    # the forward and dQ walk rows of the same lengths (loops unrolled by two)
    ro, rl = oa.fwd(f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0]), kept, T, scale)
    check_close(f64(o[0, 0]), ro, "O")
    check_lse(f64(lse[0, 0]), rl, "LSE")
    rq, rk, rv = oa.bwd(f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0]), f64(do[0, 0]), kept, T, scale)
    check_close(f64(dq[0, 0]), rq, "dQ", normalise=True)
    check_close(f64(dk[0, 0]), rk, "dK", normalise=True)
    check_close(f64(dv[0, 0]), rv, "dV", normalise=True)


def test_backward_sink_off_and_peaky():
    f, s, T, D = 9, 200, 128, 128
    N = f * s
    scale = 8.0 / np.sqrt(D)
    q, k, v, do = workloads.make_inputs(1, 1, N, D, 201, with_dout=True)
    L = sba.Layout(f, s, T, sink=False)
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = sba.attn_fwd(qc, kc, vc, L, scale)
    dq, dk, dv = sba.attn_bwd(qc, kc, vc, o, lse, dc, L, scale)
    kept = om.kept_tiles(f, s, T, False)
    rq, rk, rv = oa.bwd(f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0]), f64(do[0, 0]), kept, T, scale)
    # Delta from the bf16 O dominates here (see gpu_util): relative bound only
    for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        check_close(f64(got[0, 0]), ref, name, absolute=False, rel_max=PEAKY_REL_MAX)


def test_backward_deterministic():
    f, s, T, D = 6, 300, 128, 128
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(1, 2, f * s, D, 301, with_dout=True))
    L = sba.Layout(f, s, T)
    o, lse = sba.attn_fwd(q, k, v, L)
    a = sba.attn_bwd(q, k, v, o, lse, do, L)
    b = sba.attn_bwd(q, k, v, o, lse, do, L)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.fixture(scope="module",
                params=["train_f66", "hunyuan_5s_720p", "wan21_720p", "hunyuan_4x_long"])
def full_backward(request):
    """A full-size workload (the training step: 66 frames x 3600 tokens, 24
    heads; HunyuanVideo 5 s 720p; Wan2.1 720p, 40 heads; 129 frames, the
    longest; D = 128) run forward
    and backward in bench's launch configuration (every batch and head in one
    launch), into outputs that start as NaN."""
    w = workloads.WORKLOADS[request.param]
    _say(f"[bwd-full] {w.name} B={w.B} H={w.H} N={w.N} D={w.D}")
    q, k, v, do = workloads.workload_inputs(w, with_dout=True, device="cuda")
    L = sba.Layout(w.frames, w.tokens_per_frame, w.T)
    o, lse, dq, dk, dv = nan_outputs(w.B, w.H, w.N, w.D)
    sba.attn_fwd(q, k, v, L, w.scale, out=o, lse=lse)
    sba.attn_bwd(q, k, v, o, lse, do, L, w.scale, out=(dq, dk, dv))
    torch.cuda.synchronize()
    return dict(w=w, q=q, k=k, v=v, do=do, dq=dq, dk=dk, dv=dv)


def test_full_size_backward(full_backward):
    r = full_backward
    w, q, k, v, do, dq, dk, dv = (r[x] for x in ("w", "q", "k", "v", "do", "dq", "dk", "dv"))
    # every gradient row was written
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    # identities over every head
    sdv = dv.double().sum(dim=2)
    sdo = do.double().sum(dim=2)
    rms_dv = float(dv.double().pow(2).mean().sqrt())
    # each of N bf16-rounded terms is off by <= 2^-8 relative (random
    # signs): the sum's error grows like sqrt(N) * 2^-8 * rms; 4x margin
    tol = 4 * np.sqrt(w.N) * 2.0 ** -8 * max(rms_dv, float(do.double().pow(2).mean().sqrt()))
    assert float((sdv - sdo).abs().max()) <= tol, (float((sdv - sdo).abs().max()), tol)
    sdk = dk.double().sum(dim=2)
    rms_dk = float(dk.double().pow(2).mean().sqrt())
    assert float(sdk.abs().max()) <= 4 * np.sqrt(w.N) * 2.0 ** -8 * rms_dk + 1e-6
    # dQ on sampled query tiles of the first and last heads
    kept = om.kept_tiles(w.frames, w.tokens_per_frame, w.T, True)
    for h in (0, w.H - 1):
        qh, kh, vh, dh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h])
        for u in sample_tiles(w.N, w.T, w.tokens_per_frame, seed=w.seed)[:4]:
            rows = slice(u * w.T, min(w.N, (u + 1) * w.T))
            rq = oa.bwd_dq_tile(qh, kh, vh, dh, kept, w.T, w.scale, u)
            check_close(f64(dq[0, h, rows]), rq, f"dQ h={h} tile={u}", normalise=True)


@pytest.mark.timeout(900)
def test_full_size_dkdv_tiles(full_backward):
    """dK and dV element by element at a full-size workload, on key tiles
    whose CSC columns take every path of the dK/dV walk: tile 0 (the sink:
    every query tile of the sequence attends it, 1857 of them in the
    training step, 3629 at 129 frames), tile 28 (straddles frames 0 and 1),
    the last, partial key tile (32, 16, 80 and 16 valid keys) and one
    random tile of the first head, and the last tile of the last head.  The
    oracle takes each row's full softmax over its own kept keys, so the sink
    columns need the row terms of the whole head."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    r = full_backward
    w, q, k, v, do, dk, dv = (r[x] for x in ("w", "q", "k", "v", "do", "dk", "dv"))
    kept = om.kept_tiles(w.frames, w.tokens_per_frame, w.T, True)
    nb = kept.shape[0]
    frame0_tiles = -(-w.tokens_per_frame // w.T)  # 29: tile 28 straddles frames 0 and 1
    rand = int(np.random.default_rng(7).integers(frame0_tiles, nb - 1))
    cases = {0: [0, frame0_tiles - 1, nb - 1, rand], w.H - 1: [nb - 1]}
    workers = min(16, os.cpu_count() or 1)
    for h, tiles in cases.items():
        qh, kh, vh, dh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h])
        need = sorted(set(int(u) for vt in tiles for u in np.nonzero(kept[:, vt])[0]))
        _say(f"[dkdv-full] head {h}: key tiles {tiles}, row terms of {len(need)} query tiles "
             f"on {workers} threads")

        def stats_of(u):
            return u, oa.row_stats(qh, kh, vh, dh, kept, w.T, w.scale, u)

        stats = {}
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            for i, (u, st) in enumerate(ex.map(stats_of, need)):
                stats[u] = st
                if (i + 1) % 400 == 0:
                    _say(f"[dkdv-full]   {i + 1} of {len(need)}")
        for vt in tiles:
            keys = slice(vt * w.T, min(w.N, (vt + 1) * w.T))
            rk, rv = oa.bwd_dkdv_tile(qh, kh, vh, dh, kept, w.T, w.scale, vt, stats=stats)
            sk = check_close(f64(dk[0, h, keys]), rk, f"dK h={h} key tile={vt}", normalise=True)
            sv = check_close(f64(dv[0, h, keys]), rv, f"dV h={h} key tile={vt}", normalise=True)
            _say(f"[dkdv-full] head {h} key tile {vt} (column of {int(kept[:, vt].sum())}): "
                 f"dK max {sk['max_abs']:.3g} (rms {sk['rms_ref']:.3g}), "
                 f"dV max {sv['max_abs']:.3g} (rms {sv['rms_ref']:.3g})")

"""GPU parity at the smallest problems (needs an MI355X): N from 1 token up to
just past one chunk and one tile, in tile and token-exact mode, forward and
backward element by element against the oracle.

With one token the softmax has a single key: P = 1, O = V, and the gradients
are dQ = dK = 0 and dV = dO, which the oracle's textbook formulas give too.
These shapes exercise the partial tail chunk of every kernel with one or a
few valid rows or keys, including the lanes of the upper half of a wave that
hold no valid key at all.
"""

import sys

import numpy as np
import pytest
import torch

import static_block_sparse_amd as sba
import workloads
from gpu_util import check_close, check_lse, f64, nan_outputs
from oracle import attention as oa
from oracle import mask as om

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SHAPES = [
    # f, s, T, D
    (1, 1, 64, 64),      # N = 1
    (2, 1, 64, 64),      # N = 2, two frames of one token
    (3, 1, 128, 128),    # N = 3
    (1, 4, 64, 64),      # one lane group of keys
    (1, 5, 128, 128),    # one key past the lane group
    (1, 63, 64, 64),     # one short of a chunk
    (1, 64, 64, 64),     # exactly one chunk and tile
    (1, 65, 64, 64),     # one key into the second tile
    (5, 13, 128, 128),   # N = 65 over five frames
    (1, 129, 128, 128),  # one key into the second 128-tile
]


@pytest.mark.parametrize("f,s,T,D", SHAPES)
@pytest.mark.parametrize("exact", [False, True])
def test_tiny_problems(f, s, T, D, exact):
    N, B, H = f * s, 1, 2
    scale = 1.0 / np.sqrt(D)
    print(f"[tiny] f={f} s={s} T={T} D={D} exact={exact}", file=sys.stderr, flush=True)
    q, k, v, do = workloads.make_inputs(B, H, N, D, 700 + N, with_dout=True)
    L = sba.Layout(f, s, T, token_exact=exact)
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = sba.attn_fwd(qc, kc, vc, L, scale)
    dq, dk, dv = sba.attn_bwd(qc, kc, vc, o, lse, dc, L, scale)
    torch.cuda.synchronize()
    kept = om.kept_tiles(f, s, T, True)
    mask = om.token_mask(f, s, True)
    for h in range(H):
        qh, kh, vh, dh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h])
        if exact:
            ro, rl = oa.fwd_masked(qh, kh, vh, mask, scale)
            rq, rk, rv = oa.bwd_masked(qh, kh, vh, dh, mask, scale)
        else:
            ro, rl = oa.fwd(qh, kh, vh, kept, T, scale)
            rq, rk, rv = oa.bwd(qh, kh, vh, dh, kept, T, scale)
        check_close(f64(o[0, h]), ro, f"O h={h}")
        check_lse(f64(lse[0, h]), rl)
        check_close(f64(dq[0, h]), rq, f"dQ h={h}", normalise=True)
        check_close(f64(dk[0, h]), rk, f"dK h={h}", normalise=True)
        check_close(f64(dv[0, h]), rv, f"dV h={h}", normalise=True)
    if N == 1:
        # a single key: O is V exactly and dV is dO (both rounded to bf16)
        assert torch.equal(o, v.cuda())
        assert torch.equal(dv, do.cuda())


@pytest.mark.parametrize("exact", [False, True])
def test_many_batch_heads(exact):
    # B * H = 111 (odd, not a multiple of the XCD blocks): every (batch, head)
    # slice lands in its own place; a sample of slices against the oracle
    f, s, T, D, B, H = 5, 60, 64, 64, 3, 37
    N = f * s
    scale = 1.0 / np.sqrt(D)
    print(f"[many-heads] B={B} H={H} exact={exact}", file=sys.stderr, flush=True)
    q, k, v, do = workloads.make_inputs(B, H, N, D, 911, with_dout=True)
    L = sba.Layout(f, s, T, token_exact=exact)
    qc, kc, vc, dc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse, dq, dk, dv = nan_outputs(B, H, N, D)
    sba.attn_fwd(qc, kc, vc, L, scale, out=o, lse=lse)
    sba.attn_bwd(qc, kc, vc, o, lse, dc, L, scale, out=(dq, dk, dv))
    torch.cuda.synchronize()
    kept = om.kept_tiles(f, s, T, True)
    mask = om.token_mask(f, s, True)
    for b, h in [(0, 0), (0, H - 1), (1, 17), (2, 0), (2, H - 1)]:
        qh, kh, vh, dh = f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h])
        if exact:
            ro, rl = oa.fwd_masked(qh, kh, vh, mask, scale)
            rq, rk, rv = oa.bwd_masked(qh, kh, vh, dh, mask, scale)
        else:
            ro, rl = oa.fwd(qh, kh, vh, kept, T, scale)
            rq, rk, rv = oa.bwd(qh, kh, vh, dh, kept, T, scale)
        check_close(f64(o[b, h]), ro, f"O b={b} h={h}")
        check_lse(f64(lse[b, h]), rl)
        check_close(f64(dq[b, h]), rq, f"dQ b={b} h={h}", normalise=True)
        check_close(f64(dk[b, h]), rk, f"dK b={b} h={h}", normalise=True)
        check_close(f64(dv[b, h]), rv, f"dV b={b} h={h}", normalise=True)
    # every row of every slice was written (the outputs started as NaN), and
    # each slice is its own: every output slice differs from its neighbours'
    assert bool(torch.isfinite(lse).all())
    for t in (o, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
        assert not torch.equal(t[0, 0], t[0, 1]) and not torch.equal(t[1, 0], t[2, 0])

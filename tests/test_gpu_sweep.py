"""GPU parity over a seeded sweep of random small configurations (needs an
MI355X).

Each case draws frames, tokens per frame, the supported (head dim, tile)
pair, batch, heads, the sink flag, a mask variant (central band d, width
scale c, radial or harmonic decay) and tile or token-exact semantics from a
fixed seed, then compares forward (O, LSE) and backward (dQ, dK, dV) element
by element with the oracle: tile semantics against ``oracle.attention.fwd``
/ ``bwd`` on the oracle's tile map, token-exact semantics against
``fwd_masked`` / ``bwd_masked`` on its token mask.  The draws cover ragged
last tiles, tiles spanning several short frames, frames longer than a tile,
sampled diagonals below unit width and layouts that are dense, and masks
with one or two tokens per frame, where every query attends the sink keys
and each softmax row holds only a few keys: the gradients of those keys sum
thousands of large rounded terms, so every element gets the term-scaled
allowance (``gpu_util.rounding_sigmas``).
"""

import sys

import numpy as np
import pytest
import torch

import static_block_sparse_amd as sba
import workloads
from gpu_util import check_close, check_lse, f64, rounding_sigmas
from oracle import attention as oa
from oracle import mask as om

pytestmark = pytest.mark.gpu

V = om.Variant
PAIRS = [(64, 64), (64, 128), (128, 128)]  # (head dim, tile)
N_CASES = 120


def _cases():
    rng = np.random.default_rng(20261203)
    out = []
    while len(out) < N_CASES:
        D, T = PAIRS[rng.integers(len(PAIRS))]
        s = int(rng.choice([1, 2, 3, 5, 7, 9, 16, 31, 64, 100, 127, 129, 200, 333]))
        f = int(rng.integers(1, 3000 // s + 1))
        if f * s > 3000 or f * s < 2:
            continue
        decay = "harmonic" if rng.random() < 0.25 else "radial"
        scale = [(2, 1), (3, 2), (3, 1), (4, 1)][rng.integers(4)] if decay == "radial" else (2, 1)
        out.append(dict(f=f, s=s, T=T, D=D, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)),
                        sink=bool(rng.random() < 0.7), exact=bool(rng.random() < 0.4),
                        variant=V(decay=decay, central=int(rng.integers(0, 4)), scale=scale)))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_configuration(case):
    c = CASES[case]
    f, s, T, D, B, H, sink, exact, v = (c[x] for x in ("f", "s", "T", "D", "B", "H", "sink",
                                                      "exact", "variant"))
    N = f * s
    print(f"[sweep {case}] f={f} s={s} N={N} T={T} D={D} B={B} H={H} sink={sink} "
          f"exact={exact} {v}", file=sys.stderr, flush=True)
    scale = 1.0 / np.sqrt(D)
    q, k, vv, do = workloads.make_inputs(B, H, N, D, 5000 + case, with_dout=True)
    L = sba.Layout(f, s, T, sink=sink, token_exact=exact, decay=v.decay, central_band=v.central,
                   width_scale=v.scale)
    qc, kc, vc, dc = (t.cuda() for t in (q, k, vv, do))
    o, lse = sba.attn_fwd(qc, kc, vc, L, scale)
    dq, dk, dv = sba.attn_bwd(qc, kc, vc, o, lse, dc, L, scale)
    torch.cuda.synchronize()
    if exact:
        mask = om.token_mask(f, s, sink, v)
    else:
        kept = om.kept_tiles(f, s, T, sink, v)
        mask = np.repeat(np.repeat(kept, T, axis=0), T, axis=1)[:N, :N]
    for b in range(B):
        for h in range(H):
            args = [f64(x[b, h]) for x in (q, k, vv)]
            if exact:
                ro, rl = oa.fwd_masked(*args, mask, scale)
                rq, rk, rv = oa.bwd_masked(*args, f64(do[b, h]), mask, scale)
            else:
                ro, rl = oa.fwd(*args, kept, T, scale)
                rq, rk, rv = oa.bwd(*args, f64(do[b, h]), kept, T, scale)
            ts = rounding_sigmas(*args, f64(do[b, h]), mask, scale)
            tag = f"case {case} b={b} h={h}"
            check_close(f64(o[b, h]), ro, f"O {tag}", term=ts["o"])
            check_lse(f64(lse[b, h]), rl, f"LSE {tag}")
            check_close(f64(dq[b, h]), rq, f"dQ {tag}", normalise=True, term=ts["dq"])
            check_close(f64(dk[b, h]), rk, f"dK {tag}", normalise=True, term=ts["dk"])
            check_close(f64(dv[b, h]), rv, f"dV {tag}", normalise=True, term=ts["dv"])

"""Pins for the oracle's attention forward/backward (CPU only).

The oracle is checked against library routines it does not use (torch's
float64 scaled_dot_product_attention and autograd), against pure-Python
loops on tiny inputs, finite differences and the V == 1 invariant.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import mask as om


def _rand(shape, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape)


def _sdpa(q, k, v, mask, scale):
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    tm = torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale)
    return o[0, 0].numpy()


def test_dense_limit_equals_sdpa():
    # f = 2 covers every pair: radial attention reduces to plain attention
    f, s, T, d = 2, 40, 16, 8
    n = f * s
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    kept = om.kept_tiles(f, s, T, True)
    assert kept.all()
    o, lse = oa.fwd(q, k, v, kept, T, 0.3)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.3)[0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    ref_lse = torch.logsumexp(0.3 * torch.from_numpy(q) @ torch.from_numpy(k).T, dim=1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("f,s,T", [(5, 7, 4), (8, 16, 16), (6, 9, 8)])
def test_tile_mask_forward_equals_sdpa(f, s, T):
    d = 6
    n = f * s
    q, k, v = _rand((n, d), 4), _rand((n, d), 5), _rand((n, d), 6)
    kept = om.kept_tiles(f, s, T, True)
    eff = om.effective_mask(f, s, T, True)
    o, lse = oa.fwd(q, k, v, kept, T, 0.5)
    np.testing.assert_allclose(o, _sdpa(q, k, v, eff, 0.5), rtol=0, atol=1e-12)
    z = torch.from_numpy(0.5 * (q @ k.T)).masked_fill(~torch.from_numpy(eff), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(z, 1).numpy(), rtol=0, atol=1e-12)


def test_token_mask_forward_equals_sdpa():
    f, s, d = 7, 6, 5
    n = f * s
    q, k, v = _rand((n, d), 7), _rand((n, d), 8), _rand((n, d), 9)
    m = om.token_mask(f, s, True)
    o, _ = oa.fwd_masked(q, k, v, m, 0.7)
    np.testing.assert_allclose(o, _sdpa(q, k, v, m, 0.7), rtol=0, atol=1e-12)


def test_forward_brute_force_loops():
    # pure-Python double loop on a tiny case, one query at a time
    f, s, T, d = 3, 4, 3, 3
    n = f * s
    q, k, v = _rand((n, d), 10), _rand((n, d), 11), _rand((n, d), 12)
    kept = om.kept_tiles(f, s, T, False)
    o, lse = oa.fwd(q, k, v, kept, T, 0.9)
    for qi in range(n):
        keys = [kj for kj in range(n) if kept[qi // T, kj // T]]
        logits = [0.9 * sum(q[qi, x] * k[kj, x] for x in range(d)) for kj in keys]
        mx = max(logits)
        w = [math.exp(z - mx) for z in logits]
        tot = sum(w)
        for x in range(d):
            assert abs(o[qi, x] - sum(wi * v[kj, x] for wi, kj in zip(w, keys)) / tot) < 1e-12
        assert abs(lse[qi] - (mx + math.log(tot))) < 1e-12


def test_v_ones_gives_ones():
    f, s, T, d = 9, 8, 8, 4
    n = f * s
    q, k = _rand((n, d), 13), _rand((n, d), 14)
    kept = om.kept_tiles(f, s, T, True)
    o, _ = oa.fwd(q, k, np.ones((n, d)), kept, T, 1.0)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("f,s,T", [(5, 7, 4), (9, 4, 8), (2, 10, 8)])
def test_backward_equals_autograd(f, s, T):
    d = 5
    n = f * s
    q, k, v, do = (_rand((n, d), 20 + i) for i in range(4))
    kept = om.kept_tiles(f, s, T, True)
    eff = om.effective_mask(f, s, T, True)
    scale = 0.6
    dq, dk, dv = oa.bwd(q, k, v, do, kept, T, scale)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    z = (scale * tq @ tk.T).masked_fill(~torch.from_numpy(eff), -math.inf)
    o = torch.softmax(z, dim=1) @ tv
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    # the token-mask variant agrees with autograd under the token mask
    m = om.token_mask(f, s, True)
    tq2, tk2, tv2 = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    z2 = (scale * tq2 @ tk2.T).masked_fill(~torch.from_numpy(m), -math.inf)
    (torch.softmax(z2, dim=1) @ tv2).backward(torch.from_numpy(do))
    g = oa.bwd_masked(q, k, v, do, m, scale)
    for a, b in zip(g, (tq2.grad, tk2.grad, tv2.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=0, atol=1e-12)
    # dQ of a subset of rows from their mask rows alone equals autograd's
    rows = np.array([0, n // 3, n - 1])
    np.testing.assert_allclose(oa.dq_masked(q[rows], k, v, do[rows], m[rows], scale),
                               tq2.grad.numpy()[rows], rtol=0, atol=1e-12)


def test_backward_finite_differences():
    # two frames (dense) and one with a sparse band: central differences of
    # sum(O * dO) with respect to every input element
    for f, s, T in [(2, 3, 2), (5, 2, 1)]:
        d = 3
        n = f * s
        q, k, v, do = (_rand((n, d), 40 + i) for i in range(4))
        kept = om.kept_tiles(f, s, T, False)
        scale = 0.8
        dq, dk, dv = oa.bwd(q, k, v, do, kept, T, scale)

        def loss(q_, k_, v_):
            o, _ = oa.fwd(q_, k_, v_, kept, T, scale)
            return float((o * do).sum())

        h = 1e-6
        for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            for idx in np.ndindex(arr.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][idx] += h
                up = loss(*args)
                args[which][idx] -= 2 * h
                dn = loss(*args)
                assert abs((up - dn) / (2 * h) - grad[idx]) < 1e-7


def test_dq_tile_matches_full_backward():
    f, s, T, d = 6, 11, 8, 4
    n = f * s
    q, k, v, do = (_rand((n, d), 60 + i) for i in range(4))
    kept = om.kept_tiles(f, s, T, True)
    dq, _, _ = oa.bwd(q, k, v, do, kept, T, 0.7)
    for u in range(kept.shape[0]):
        rows = slice(u * T, min(n, (u + 1) * T))
        np.testing.assert_allclose(oa.bwd_dq_tile(q, k, v, do, kept, T, 0.7, u), dq[rows],
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("f,s,T,sink", [(6, 11, 8, True), (5, 30, 16, False), (9, 7, 4, True),
                                        (3, 40, 64, True)])
def test_dkdv_tile_matches_full_backward(f, s, T, sink):
    # per key tile, from each row's own full softmax (the column's query
    # tiles only), against the whole-head backward and, independently,
    # torch float64 autograd of the masked softmax under the tile map
    n, d = f * s, 5
    q, k, v, do = (_rand((n, d), 70 + i) for i in range(4))
    kept = om.kept_tiles(f, s, T, sink)
    nb = kept.shape[0]
    scale = 0.6
    _, dk, dv = oa.bwd(q, k, v, do, kept, T, scale)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    tok = np.repeat(np.repeat(kept, T, axis=0), T, axis=1)[:n, :n]
    z = scale * tq @ tk.T
    z = z.masked_fill(~torch.from_numpy(tok), float("-inf"))
    (torch.softmax(z, dim=1) @ tv).backward(torch.from_numpy(do))
    stats = {u: oa.row_stats(q, k, v, do, kept, T, scale, u) for u in range(nb)}
    for vt in range(nb):
        keys = slice(vt * T, min(n, (vt + 1) * T))
        gk, gv = oa.bwd_dkdv_tile(q, k, v, do, kept, T, scale, vt)
        np.testing.assert_allclose(gk, dk[keys], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gv, dv[keys], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gk, tk.grad.numpy()[keys], rtol=0, atol=1e-11)
        np.testing.assert_allclose(gv, tv.grad.numpy()[keys], rtol=0, atol=1e-11)
        hk, hv = oa.bwd_dkdv_tile(q, k, v, do, kept, T, scale, vt, stats=stats)
        np.testing.assert_array_equal(hk, gk)
        np.testing.assert_array_equal(hv, gv)


def test_row_stats_are_the_row_terms():
    # LSE from the forward and Delta = rowsum(P * dP), the textbook form
    f, s, T, d = 5, 13, 8, 3
    n = f * s
    q, k, v, do = (_rand((n, d), 80 + i) for i in range(4))
    kept = om.kept_tiles(f, s, T, True)
    _, lse_all = oa.fwd(q, k, v, kept, T, 0.9)
    for u in range(kept.shape[0]):
        rows = slice(u * T, min(n, (u + 1) * T))
        cols = oa.tile_columns(kept[u], n, T)
        z = 0.9 * q[rows] @ k[cols].T
        p = np.exp(z - lse_all[rows, None])
        lse, delta = oa.row_stats(q, k, v, do, kept, T, 0.9, u)
        np.testing.assert_allclose(lse, lse_all[rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(delta, (p * (do[rows] @ v[cols].T)).sum(axis=1),
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("f,s,T,sink", [(6, 11, 8, True), (5, 30, 16, False), (9, 7, 4, True),
                                        (4, 5, 16, True), (3, 40, 64, False)])
def test_dkdv_masked_keys_matches_autograd(f, s, T, sink):
    # per key tile under the token mask, with each row's terms taken over the
    # keys of its kept tiles only (as at full size), against torch float64
    # autograd of the masked softmax over the whole head and the whole-head
    # oracle backward
    n, d = f * s, 6
    q, k, v, do = (_rand((n, d), 90 + i) for i in range(4))
    mask = om.token_mask(f, s, sink)
    kept = om.kept_tiles(f, s, T, sink)
    nb = kept.shape[0]
    scale = 0.7
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    z = (scale * tq @ tk.T).masked_fill(~torch.from_numpy(mask), float("-inf"))
    (torch.softmax(z, dim=1) @ tv).backward(torch.from_numpy(do))
    _, dk_all, dv_all = oa.bwd_masked(q, k, v, do, mask, scale)
    blocks_of = {}
    for u in range(nb):
        rows = slice(u * T, min(n, (u + 1) * T))
        cols = oa.tile_columns(kept[u], n, T)
        lse, delta = oa.row_stats_masked(q[rows], k[cols], v[cols], do[rows],
                                         mask[rows][:, cols], scale)
        blocks_of[u] = (rows, lse, delta)
    for vt in range(nb):
        keys = slice(vt * T, min(n, (vt + 1) * T))
        blocks = [(r, mask[r, keys], lse, delta)
                  for u, (r, lse, delta) in blocks_of.items() if kept[u, vt]]
        gk, gv = oa.dkdv_masked_keys(q, k, v, do, keys, blocks, scale)
        np.testing.assert_allclose(gk, tk.grad.numpy()[keys], rtol=0, atol=1e-11)
        np.testing.assert_allclose(gv, tv.grad.numpy()[keys], rtol=0, atol=1e-11)
        np.testing.assert_allclose(gk, dk_all[keys], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gv, dv_all[keys], rtol=0, atol=1e-12)


def test_dkdv_masked_keys_needs_every_attending_row():
    # leaving out one query tile that attends a key tile changes its
    # gradient: the function sums over exactly the blocks it is given
    f, s, T, d = 5, 13, 8, 4
    n = f * s
    q, k, v, do = (_rand((n, d), 95 + i) for i in range(4))
    mask = om.token_mask(f, s, True)
    scale = 0.8
    keys = slice(0, T)
    blocks = []
    for u in range(-(-n // T)):
        rows = slice(u * T, min(n, (u + 1) * T))
        lse, delta = oa.row_stats_masked(q[rows], k, v, do[rows], mask[rows], scale)
        blocks.append((rows, mask[rows, keys], lse, delta))
    full_k, full_v = oa.dkdv_masked_keys(q, k, v, do, keys, blocks, scale)
    part_k, part_v = oa.dkdv_masked_keys(q, k, v, do, keys, blocks[:-1], scale)
    assert np.abs(full_v - part_v).max() > 1e-3 and np.abs(full_k - part_k).max() > 1e-3

"""GPU parity of the forward pass against the oracle (needs an MI355X).

Every call goes through the C ABI (static_block_sparse_amd -> libradial.so).
Small shapes are compared element by element over every head and row; the
full-size workloads in the launch configuration bench.py times are compared
on sampled query tiles, plus properties that hold at any size.
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


def _run_full_compare(f, s, T, D, B, H, seed, sink=True, scale=None, dense=False, v_ones=False):
    N = f * s
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    _say(f"[fwd] f={f} s={s} T={T} D={D} B={B} H={H} seed={seed} sink={sink} dense={dense}")
    q, k, v = workloads.make_inputs(B, H, N, D, seed)
    if v_ones:
        v = torch.ones_like(v)
    L = sba.Layout(f, s, T, sink=sink, dense=dense)
    o, lse = sba.attn_fwd(q.cuda(), k.cuda(), v.cuda(), L, scale)
    torch.cuda.synchronize()
    kept = np.ones((L.n_blocks,) * 2, bool) if dense else om.kept_tiles(f, s, T, sink)
    go, gl = f64(o), f64(lse)
    stats = []
    for b in range(B):
        for h in range(H):
            ro, rl = oa.fwd(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), kept, T, scale)
            stats.append(check_close(go[b, h], ro, f"O b={b} h={h}"))
            check_lse(gl[b, h], rl)
    return go, stats


def test_tiny_workload_all_heads():
    w = workloads.WORKLOADS["tiny_f8_s256"]
    _run_full_compare(w.frames, w.tokens_per_frame, w.T, w.D, w.B, w.H, w.seed)


@pytest.mark.parametrize("f,s,T,D,B,H", [
    (5, 300, 128, 128, 2, 3),    # N = 1500: 12 tiles, last one 92 rows; tiles straddle frames
    (7, 100, 64, 64, 1, 2),      # N = 700: last tile 60 rows; 64-tiles span frames
    (3, 40, 128, 128, 1, 1),     # a single, partial tile (N = 120 < T)
    (40, 20, 64, 64, 1, 1),      # many frames, narrow bands, rows of very different length
    (5, 300, 128, 64, 1, 2),     # head dim 64 with 128-wide tiles; ragged last tile
    (9, 100, 128, 64, 2, 1),     # head dim 64 with 128-wide tiles; odd number of tiles
    (300, 2, 64, 64, 1, 1),      # tiny frames: the width-below-one sampling fires
])
def test_ragged_shapes(f, s, T, D, B, H):
    _run_full_compare(f, s, T, D, B, H, seed=11 + f)


def test_sink_off():
    _run_full_compare(9, 200, 128, 128, 1, 2, seed=21, sink=False)


def test_v_ones_gives_ones():
    # every softmax row sums to one, so V == 1 must give O == 1
    f, s, T, D = 9, 200, 128, 128
    N = f * s
    q, k, _ = workloads.make_inputs(1, 2, N, D, 31)
    v = torch.ones((1, 2, N, D), dtype=torch.bfloat16)
    o, _ = sba.attn_fwd(q.cuda(), k.cuda(), v.cuda(), sba.Layout(f, s, T))
    err = float((o.double() - 1).abs().max())
    assert err <= 4e-3, err


def test_peaky_softmax():
    # scale x8: logits with std ~8, so a few keys dominate each row
    _run_full_compare(6, 300, 128, 128, 1, 2, seed=41, scale=8.0 / np.sqrt(128))
    _run_full_compare(8, 256, 64, 64, 1, 2, seed=42, scale=8.0 / np.sqrt(64))


@pytest.mark.parametrize("gain", [6.0, 40.0])
@pytest.mark.parametrize("exact", [False, True])
def test_reference_max_moves_late_in_the_walk(gain, exact):
    # Keys of the last frame get `gain` times larger logits.  Rows of the
    # last frames take their reference max from the sink tile, the first of
    # their walk, and meet the large logits in its last chunks: at gain 6
    # (logits up to ~25 in log2 units above the reference) the chunk sum
    # exceeds the bound while finite, at gain 40 (~170 above) the
    # probabilities overflow to inf.  Either way the chunk is redone with its
    # true max, so O and LSE match the oracle.
    f, s, T, D, H = 6, 300, 128, 128, 2
    N = f * s
    _say(f"[fwd-late-max] gain={gain} exact={exact}")
    q, k, v = workloads.make_inputs(1, H, N, D, 61)
    k = k.clone()
    k[:, :, (f - 1) * s:] = (k[:, :, (f - 1) * s:].float() * gain).to(torch.bfloat16)
    L = sba.Layout(f, s, T, token_exact=exact)
    scale = 1.0 / np.sqrt(D)
    o, lse = sba.attn_fwd(q.cuda(), k.cuda(), v.cuda(), L, scale)
    torch.cuda.synchronize()
    go, gl = f64(o), f64(lse)
    kept = om.kept_tiles(f, s, T, True)
    mask = om.token_mask(f, s, True) if exact else None
    for h in range(H):
        qh, kh, vh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h])
        if exact:
            ro, rl = oa.fwd_masked(qh, kh, vh, mask, scale)
        else:
            ro, rl = oa.fwd(qh, kh, vh, kept, T, scale)
        # the last frame's rows really are dominated by the large logits
        assert float(rl[(f - 1) * s:].mean()) > 10.0
        check_close(go[0, h], ro, f"O h={h}")
        check_lse(gl[0, h], rl)


def test_dense_layout_is_plain_attention():
    go, _ = _run_full_compare(4, 300, 128, 128, 1, 2, seed=51, dense=True)
    # and against torch's float64 SDPA on the CPU (a library routine)
    q, k, v = workloads.make_inputs(1, 2, 1200, 128, 51)
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double())
    assert float(np.abs(go - ref.numpy()).max()) <= 2e-2


def test_two_frames_equal_dense_layout_bitwise():
    # f = 2 keeps every tile, so the radial and the dense layouts run the
    # same tiles in the same order
    f, s, T, D = 2, 700, 128, 128
    q, k, v = (t.cuda() for t in workloads.make_inputs(1, 2, f * s, D, 61))
    a, la = sba.attn_fwd(q, k, v, sba.Layout(f, s, T))
    b, lb = sba.attn_fwd(q, k, v, sba.Layout(f, s, T, dense=True))
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("f,s,T,D,exact", [
    (8, 256, 64, 64, False),     # the tiny workload's shape
    (7, 100, 64, 64, True),      # ragged, 64-tiles spanning frames, token-exact
    (5, 300, 128, 128, False),   # ragged last tile, 12 tiles (4 triples)
    (13, 100, 128, 128, True),   # 11 tiles: a last triple of two, token-exact
    (9, 100, 128, 64, False),    # head dim 64 on 128-wide tiles, odd tile count
])
def test_query_tile_groups_agree_bitwise(f, s, T, D, exact):
    # single tiles, pairs and triples: each wave walks its own kept tiles in
    # the same order whatever the group, so the results are the same bits
    q, k, v = (t.cuda() for t in workloads.make_inputs(1, 2, f * s, D, 81))
    L = sba.Layout(f, s, T, token_exact=exact)
    out = {}
    try:
        for cap in (1, 2, 3):
            assert sba.lib().radial_test_set_fwd_group(cap) in (1, 2, 3)
            out[cap] = sba.attn_fwd(q, k, v, L)
    finally:
        sba.lib().radial_test_set_fwd_group(3)
    for cap in (1, 2):
        assert torch.equal(out[cap][0], out[3][0]) and torch.equal(out[cap][1], out[3][1]), cap
    kept = om.kept_tiles(f, s, T, True)
    if not exact:
        ro, rl = oa.fwd(f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0]), kept, T, 1.0 / np.sqrt(D))
        check_close(f64(out[3][0][0, 0]), ro, "O")
        check_lse(f64(out[3][1][0, 0]), rl, "LSE")


def test_deterministic_and_stream_aware():
    f, s, T, D = 6, 300, 128, 128
    q, k, v = (t.cuda() for t in workloads.make_inputs(2, 3, f * s, D, 71))
    L = sba.Layout(f, s, T)
    a, la = sba.attn_fwd(q, k, v, L)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        b, lb = sba.attn_fwd(q, k, v, L)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_rejects_bad_inputs_on_gpu():
    L = sba.Layout(8, 256, 64)
    q = torch.zeros((1, 1, 2048, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sba.RadialError):
        sba.attn_fwd(q, q, q, sba.Layout(8, 255, 64))
    with pytest.raises(sba.RadialError):  # (D, block_size) = (64, 32): not supported
        sba.attn_fwd(q, q, q, sba.Layout(8, 256, 32))
    # misaligned pointer: a view offset by one element
    raw = torch.zeros(2048 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    lib = sba.lib()
    L.upload()
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, 2048), dtype=torch.float32, device="cuda")
    st = lib.radial_attn_fwd(L.handle, 1, 1, 2048, 64, 0.125, raw.data_ptr() + 2, q.data_ptr(),
                             q.data_ptr(), o.data_ptr(), lse.data_ptr(), None)
    assert st == -1


FULL = ["hunyuan_5s_720p", "wan21_720p", "hunyuan_4x_long", "train_f66"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_tiles(name):
    """Full-size workload, all heads in one launch (as bench.py times it);
    oracle check on sampled query tiles of the first and last heads; every
    output row written (the outputs start as NaN)."""
    w = workloads.WORKLOADS[name]
    _say(f"[fwd-full] {name} B={w.B} H={w.H} N={w.N} D={w.D}")
    q, k, v = workloads.workload_inputs(w, with_dout=False, device="cuda")
    L = sba.Layout(w.frames, w.tokens_per_frame, w.T)
    o, lse = nan_outputs(w.B, w.H, w.N, w.D, grads=False)
    sba.attn_fwd(q, k, v, L, w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lse).all())
    assert bool(torch.isfinite(o.float()).all())
    kept = om.kept_tiles(w.frames, w.tokens_per_frame, w.T, True)
    tiles = sample_tiles(w.N, w.T, w.tokens_per_frame, seed=w.seed)
    for h in (0, w.H - 1):
        qh, kh, vh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h])
        for u in tiles:
            rows = slice(u * w.T, min(w.N, (u + 1) * w.T))
            ro, rl = oa.fwd_tile(qh, kh, vh, kept, w.T, w.scale, u)
            check_close(f64(o[0, h, rows]), ro, f"{name} O h={h} tile={u}")
            check_lse(f64(lse[0, h, rows]), rl, f"{name} lse h={h} tile={u}")


def test_dense_layout_full_size_sampled_tiles():
    """The in-repo dense kernel (the same kernel on a layout that keeps every
    tile) at the 4x HunyuanVideo size bench.py compares against, all heads
    in one launch: sampled query tiles of the first and last heads against
    the oracle over all keys; every output row written."""
    w = workloads.WORKLOADS["hunyuan_4x_long"]
    _say(f"[fwd-dense-full] {w.name} B={w.B} H={w.H} N={w.N} D={w.D}")
    q, k, v = workloads.workload_inputs(w, with_dout=False, device="cuda")
    L = sba.Layout(w.frames, w.tokens_per_frame, w.T, dense=True)
    assert L.nnz_tiles == L.n_blocks ** 2
    o, lse = nan_outputs(w.B, w.H, w.N, w.D, grads=False)
    sba.attn_fwd(q, k, v, L, w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lse).all())
    assert bool(torch.isfinite(o.float()).all())
    kept = np.ones((L.n_blocks,) * 2, bool)
    tiles = sample_tiles(w.N, w.T, w.tokens_per_frame, seed=w.seed + 100)
    for h in (0, w.H - 1):
        qh, kh, vh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h])
        for u in tiles:
            rows = slice(u * w.T, min(w.N, (u + 1) * w.T))
            ro, rl = oa.fwd_tile(qh, kh, vh, kept, w.T, w.scale, u)
            check_close(f64(o[0, h, rows]), ro, f"dense O h={h} tile={u}")
            check_lse(f64(lse[0, h, rows]), rl, f"dense lse h={h} tile={u}")

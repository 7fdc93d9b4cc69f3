"""Host-side tests of libradial.so (no GPU needed).

* the library loads and exports every function include/radial.h declares;
* the C++ mask compiler matches the oracle bit-exactly (CSR, CSC, band
  table, token mask, pair count, full/partial tile marks), live on small
  shapes and through stored oracle digests at the full workload shapes;
* argument validation and the allocation-failure hook return the documented
  status codes without touching a GPU.
"""

import ctypes
import hashlib
import json
import os
import re

import numpy as np
import pytest

import static_block_sparse_amd as sba
from oracle import mask as om

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "radial.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(radial_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = sba.lib()
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    # and nm agrees that they are exported C symbols (no C++ mangling)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", sba.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (radial_\w+)", out))
    assert set(names) <= exported


def test_binding_argument_counts_match_header():
    # every prototype's parameter count equals the ctypes argtypes the
    # binding installs (a missing or extra argument shifts every later one)
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = re.findall(r"\b(radial_[a-z_0-9]+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S)
    lib = sba.lib()
    assert len(protos) >= 12
    for name, params in protos:
        params = params.strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        assert len(getattr(lib, name).argtypes) == n, name


SMALL = [(4, 9, 4), (8, 256, 64), (5, 7, 3), (33, 3, 16), (12, 1, 4), (6, 100, 64),
         (3, 50, 128), (40, 2, 7), (20, 33, 32), (66, 256, 128), (17, 100, 64), (1, 5, 2),
         (2, 300, 128), (9, 130, 128)]


@pytest.mark.parametrize("sink", [True, False])
def test_tiles_match_oracle_small(sink):
    for f, s, T in SMALL:
        L = sba.Layout(f, s, T, sink=sink)
        kept = om.kept_tiles(f, s, T, sink)
        rp, ci = om.csr(kept)
        cp, ri = om.csc(kept)
        grp, gci = L.csr()
        gcp, gri = L.csc()
        assert L.n_blocks == kept.shape[0]
        assert L.nnz_tiles == int(kept.sum())
        assert np.array_equal(grp, rp) and np.array_equal(gci, ci), (f, s, T)
        assert np.array_equal(gcp, cp) and np.array_equal(gri, ri), (f, s, T)
        assert L.nnz_pairs == om.tile_pairs(kept, f * s, T)


def test_band_table_matches_oracle():
    for f, s in [(129, 3600), (600, 3), (40, 1), (8, 256)]:
        r, w, p = sba.Layout(f, s, 16).band_table()
        tab = om.band_table(f, s)
        assert np.array_equal(r, tab[:, 0]) and np.array_equal(w, tab[:, 1])
        assert np.array_equal(p, tab[:, 2])


@pytest.mark.parametrize("sink", [True, False])
def test_token_mask_matches_oracle(sink):
    for f, s in [(4, 9), (12, 1), (9, 16), (33, 3), (7, 40)]:
        got = sba.Layout(f, s, 8, sink=sink).token_mask()
        assert np.array_equal(got, om.token_mask(f, s, sink)), (f, s)


def _digest(a):
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()


def _variant_kwargs(g):
    v = g.get("variant")
    if v is None:
        return {}
    return dict(decay=v["decay"], central_band=v["central"], width_scale=tuple(v["scale"]))


def test_tiles_match_oracle_digests_full_size():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "layouts.json")))
    assert sum(1 for g in gold if "variant" in g) >= 12
    for g in gold:
        L = sba.Layout(g["frames"], g["tokens_per_frame"], g["tile"], sink=g["sink"],
                       **_variant_kwargs(g))
        assert L.n_blocks == g["n_blocks"] and L.nnz_tiles == g["nnz_tiles"]
        assert L.nnz_pairs == g["nnz_pairs"]
        rp, ci = L.csr()
        cp, ri = L.csc()
        assert _digest(rp) == g["row_ptr"] and _digest(ci) == g["col_idx"], g
        assert _digest(cp) == g["col_ptr"] and _digest(ri) == g["row_idx"], g


# shapes where the sampled diagonal (w = 0) and frame-straddling tiles occur
FLAG_SHAPES = SMALL + [(600, 3, 16), (40, 1, 8), (129, 20, 16), (70, 5, 9)]


@pytest.mark.parametrize("sink", [True, False])
def test_tile_flags_match_oracle_small(sink):
    for f, s, T in FLAG_SHAPES:
        L = sba.Layout(f, s, T, sink=sink)
        kept = om.kept_tiles(f, s, T, sink)
        full = om.full_tiles(f, s, T, sink)
        a, b = L.tile_flags()
        assert np.array_equal(a, full[kept]), (f, s, T)
        assert np.array_equal(b, full.T[kept.T]), (f, s, T)


def test_tile_flags_match_oracle_digests_full_size():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "layouts.json")))
    u8 = lambda a: hashlib.sha256(np.ascontiguousarray(a, dtype=np.uint8).tobytes()).hexdigest()
    for g in gold:
        L = sba.Layout(g["frames"], g["tokens_per_frame"], g["tile"], sink=g["sink"],
                       token_exact=True, **_variant_kwargs(g))
        a, b = L.tile_flags()
        assert int(a.sum()) == g["n_full"] == int(b.sum()), g
        assert u8(a) == g["csr_full"] and u8(b) == g["csc_full"], g


def test_token_exact_flag_keeps_the_tile_lists():
    # the flag changes only how kept tiles are computed, not which are kept
    for f, s, T in [(8, 256, 64), (33, 3, 16), (12, 1, 4)]:
        a, b = sba.Layout(f, s, T), sba.Layout(f, s, T, token_exact=True)
        assert a.nnz_tiles == b.nnz_tiles and a.nnz_pairs == b.nnz_pairs
        for x, y in zip(a.csr() + a.csc(), b.csr() + b.csc()):
            assert np.array_equal(x, y)
    d = sba.Layout(7, 50, 32, dense=True, token_exact=True)
    assert all(x.all() for x in d.tile_flags())


VARIANTS = [om.Variant(central=0), om.Variant(central=2), om.Variant(scale=(3, 2)),
            om.Variant(scale=(3, 1)), om.Variant(scale=(4, 1)), om.Variant(decay="harmonic"),
            om.Variant(decay="harmonic", central=2), om.Variant(central=3, scale=(5, 2)),
            om.Variant(central=50)]


def _layout(f, s, T, sink, v, **kw):
    return sba.Layout(f, s, T, sink=sink, decay=v.decay, central_band=v.central,
                      width_scale=v.scale, **kw)


@pytest.mark.parametrize("variant", VARIANTS, ids=str)
def test_variants_match_oracle_small(variant):
    cap = 2 ** 31 - 1
    for f, s, T in [(4, 9, 4), (8, 256, 64), (5, 7, 3), (33, 3, 16), (12, 1, 4), (40, 2, 7),
                    (20, 33, 32), (17, 100, 64), (600, 3, 16), (70, 5, 9)]:
        for sink in (True, False):
            L = _layout(f, s, T, sink, variant)
            kept = om.kept_tiles(f, s, T, sink, variant)
            rp, ci = om.csr(kept)
            cp, ri = om.csc(kept)
            assert all(np.array_equal(a, b) for a, b in zip(L.csr() + L.csc(), (rp, ci, cp, ri))), \
                (f, s, T, sink)
            assert L.nnz_pairs == om.tile_pairs(kept, f * s, T)
            full = om.full_tiles(f, s, T, sink, variant)
            a, b = L.tile_flags()
            assert np.array_equal(a, full[kept]) and np.array_equal(b, full.T[kept.T])
            r, w, p = L.band_table()
            tab = om.band_table(f, s, variant)
            assert np.array_equal(r, tab[:, 0]) and np.array_equal(w, tab[:, 1])
            assert np.array_equal(p, np.minimum(tab[:, 2], cap))
            if f * s <= 700:
                assert np.array_equal(L.token_mask(), om.token_mask(f, s, sink, variant))


@pytest.mark.parametrize("prm", [(2, 1, 2, 1), (0, -1, 2, 1), (0, 1, 2, 2), (0, 1, 1, 2),
                                 (0, 1, 17, 1), (0, 1, 10, 5), (0, 1, 2, 0)])
def test_build_ex_rejects_bad_variants(prm):
    P = sba._MaskParams(*prm)
    h = ctypes.c_void_p(123)
    assert sba.lib().radial_mask_build_ex(8, 64, 16, 1, ctypes.byref(P), ctypes.byref(h)) == -1
    assert h.value is None
    # the harmonic decay ignores the scale; NULL params are the defaults
    P = sba._MaskParams(1, 1, 0, 0)
    assert sba.lib().radial_mask_build_ex(8, 64, 16, 1, ctypes.byref(P), ctypes.byref(h)) == 0
    sba.lib().radial_layout_destroy(h)
    assert sba.lib().radial_mask_build_ex(8, 64, 16, 1, None, ctypes.byref(h)) == 0
    sba.lib().radial_layout_destroy(h)
    d = sba._MaskParams(9, 9, 9, 9)
    sba.lib().radial_mask_params_default(ctypes.byref(d))
    assert (d.decay, d.central_band, d.scale_num, d.scale_den) == (0, 1, 2, 1)


def test_dense_flag_keeps_every_tile():
    L = sba.Layout(7, 50, 32, dense=True)
    nb = L.n_blocks
    assert L.nnz_tiles == nb * nb
    assert L.nnz_pairs == L.n * L.n
    assert L.token_mask().all()


def test_sink_flag_off_by_request():
    a, b = sba.Layout(33, 3600, 128, sink=True), sba.Layout(33, 3600, 128, sink=False)
    assert a.nnz_tiles == 389411 and b.nnz_tiles == 371557


@pytest.mark.parametrize("args", [(0, 10, 8, 1), (4, 0, 8, 1), (4, 10, 0, 1), (4, 10, 5000, 1),
                                  (4, 10, 8, 8), (1 << 20, 1 << 12, 128, 1)])
def test_build_rejects_bad_arguments(args):
    h = ctypes.c_void_p(123)
    st = sba.lib().radial_mask_build(*args, ctypes.byref(h))
    assert st == -1
    assert h.value is None
    assert sba.lib().radial_last_error().decode()


def test_compute_calls_validate_before_touching_the_gpu():
    lib = sba.lib()
    L = sba.Layout(8, 256, 64)
    dummy = 4096  # 16-byte aligned fake address, never dereferenced
    args = lambda Lh, B, H, N, D, sc: (Lh, B, H, N, D, sc, dummy, dummy, dummy, dummy, dummy, None)
    assert lib.radial_attn_fwd(*args(None, 1, 1, 2048, 64, 0.125)) == -1
    assert lib.radial_attn_fwd(*args(L.handle, 0, 1, 2048, 64, 0.125)) == -1
    assert lib.radial_attn_fwd(*args(L.handle, 1, 1, 2047, 64, 0.125)) == -3
    assert lib.radial_attn_fwd(*args(L.handle, 1, 1, 2048, 128, 0.125)) == -2
    assert lib.radial_attn_fwd(*args(L.handle, 1, 1, 2048, 64, -1.0)) == -1
    assert lib.radial_attn_fwd(*args(L.handle, 1, 1, 2048, 64, float("nan"))) == -1
    # valid shapes but the layout was never uploaded
    assert lib.radial_attn_fwd(*args(L.handle, 1, 1, 2048, 64, 0.125)) == -6
    assert "upload" in lib.radial_last_error().decode()
    ws = lib.radial_attn_bwd_workspace_bytes(L.handle, 2, 3, 2048, 64)
    assert ws >= 2 * 3 * 2048 * 4 and ws % 256 == 0
    b = (L.handle, 1, 1, 2048, 64, 0.125) + (dummy,) * 10 + (ws, None)
    assert lib.radial_attn_bwd(*b) == -6
    b = (L.handle, 1, 1, 2000, 64, 0.125) + (dummy,) * 10 + (ws, None)
    assert lib.radial_attn_bwd(*b) == -3
    assert lib.radial_status_string(-3) == b"shape mismatch"
    assert lib.radial_status_string(-2) == b"unsupported shape or size"
    # the allocation-free backward validates the same way
    nb_ = (L.handle, 1, 1, 2048, 64, 0.125) + (dummy,) * 9 + (None,)
    assert lib.radial_attn_bwd_noalloc(*nb_) == -6
    nb_ = (None, 1, 1, 2048, 64, 0.125) + (dummy,) * 9 + (None,)
    assert lib.radial_attn_bwd_noalloc(*nb_) == -1
    nb_ = (L.handle, 1, 1, 2048, 64, 0.125) + (dummy,) * 8 + (None, None)
    assert lib.radial_attn_bwd_noalloc(*nb_) in (-1, -6)


def test_compute_calls_reject_slices_of_2_gib_or_more():
    # one (batch, head) slice of N * D bf16 must stay below 2^31 bytes (the
    # kernels address rows inside a slice with 32-bit offsets); the check
    # runs before N is compared with the layout, so a small layout suffices
    lib = sba.lib()
    L = sba.Layout(8, 256, 64)
    dummy = 4096
    for N, D in ((1 << 23, 128), (1 << 24, 64), ((1 << 31) // 256, 128), (1 << 33, 128)):
        fa = (L.handle, 1, 1, N, D, 0.125, dummy, dummy, dummy, dummy, dummy, None)
        assert lib.radial_attn_fwd(*fa) == -2, (N, D)
        assert "2^31" in lib.radial_last_error().decode()
        ba = (L.handle, 1, 1, N, D, 0.125) + (dummy,) * 10 + (1 << 20, None)
        assert lib.radial_attn_bwd(*ba) == -2, (N, D)
    for N in (0, -5):
        fa = (L.handle, 1, 1, N, 64, 0.125, dummy, dummy, dummy, dummy, dummy, None)
        assert lib.radial_attn_fwd(*fa) == -1
    # the largest N below the limit only fails the layout comparison
    N = (1 << 31) // 256 - 1
    fa = (L.handle, 1, 1, N, 128, 0.125, dummy, dummy, dummy, dummy, dummy, None)
    assert lib.radial_attn_fwd(*fa) == -3


def test_forward_group_test_hook():
    lib = sba.lib()
    assert lib.radial_test_set_fwd_group(0) == -1
    assert lib.radial_test_set_fwd_group(4) == -1
    try:
        assert lib.radial_test_set_fwd_group(1) == 3
        assert lib.radial_test_set_fwd_group(2) == 1
    finally:
        assert lib.radial_test_set_fwd_group(3) in (1, 2, 3)


def test_binding_rejects_host_tensors_before_any_launch():
    # a CPU lse or workspace would hand a host pointer to the kernels; the
    # binding refuses them with ValueError before calling the library
    import torch
    if torch.cuda.is_available():
        pytest.skip("checks the CPU-side refusal only")
    L = sba.Layout(8, 256, 64)

    class FakeCuda:
        """Stands in for a GPU bf16 tensor: passes the q/k/v checks only."""
        is_cuda = True
        dtype = torch.bfloat16
        shape = torch.Size((1, 1, 2048, 64))
        device = torch.device("cuda", 0)

        def dim(self):
            return 4

        def is_contiguous(self):
            return True

    class FakeLse(FakeCuda):
        dtype = torch.float32
        shape = torch.Size((1, 1, 2048))

    x = FakeCuda()
    lse_cpu = torch.empty((1, 1, 2048), dtype=torch.float32)
    with pytest.raises(ValueError, match="lse"):
        sba.attn_bwd(x, x, x, x, lse_cpu, x, L)
    ws_cpu = torch.empty(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace"):
        sba.attn_bwd(x, x, x, x, FakeLse(), x, L, workspace=ws_cpu)


def test_allocation_failure_hook():
    lib = sba.lib()
    assert lib.radial_test_set_fail_alloc(2) == -1
    h = ctypes.c_void_p()
    assert lib.radial_test_set_fail_alloc(1) == 0
    try:
        assert lib.radial_mask_build(8, 256, 64, 1, ctypes.byref(h)) == -4
        assert h.value is None
    finally:
        assert lib.radial_test_set_fail_alloc(0) == 1
    assert lib.radial_mask_build(8, 256, 64, 1, ctypes.byref(h)) == 0
    lib.radial_layout_destroy(h)


def test_layout_is_o_n_log_n_at_tile_level_for_long_videos():
    # tile density falls as frames grow at fixed s (the radial mask's whole
    # point); at f = 2 every tile is kept
    dens = []
    for f in [2, 8, 32, 128]:
        L = sba.Layout(f, 3600, 128)
        dens.append(L.nnz_tiles / L.n_blocks ** 2)
    assert dens[0] == 1.0
    assert all(a > b for a, b in zip(dens, dens[1:]))

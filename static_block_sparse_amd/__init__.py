"""Radial block-sparse attention on AMD MI355X (gfx950).

Thin Python binding of ``libradial.so`` (C ABI declared in include/radial.h).
The binding only marshals arguments: every step of the mask compilation and
of the attention runs in the library.  torch provides device memory and the
current HIP stream.

    L = Layout(frames=33, tokens_per_frame=3600, block_size=128)  # sink on
    o, lse = attn_fwd(q, k, v, L)             # q, k, v: bf16 [B, H, N, D] on GPU
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, L)

Raises RuntimeError when the library is not built (there is no fallback).
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np

__all__ = ["Layout", "Schedule", "attn_fwd", "attn_bwd", "attn_bwd_noalloc", "lib", "LIB_PATH", "SINK", "DENSE",
           "TOKEN_EXACT", "DECAYS", "RadialError"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libradial.so")

SINK = 1
DENSE = 2
TOKEN_EXACT = 4
DECAYS = {"radial": 0, "harmonic": 1}


class _MaskParams(ctypes.Structure):
    _fields_ = [("decay", ctypes.c_int32), ("central_band", ctypes.c_int32),
                ("scale_num", ctypes.c_int32), ("scale_den", ctypes.c_int32)]

_STATUS = {0: "RADIAL_OK", -1: "RADIAL_E_INVALID", -2: "RADIAL_E_UNSUPPORTED",
           -3: "RADIAL_E_SHAPE", -4: "RADIAL_E_NOMEM", -5: "RADIAL_E_HIP", -6: "RADIAL_E_STATE"}

_lib = None


class RadialError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


def _declare(L):
    c = ctypes
    vp, i32, i64, u32, f32, sz = c.c_void_p, c.c_int32, c.c_int64, c.c_uint32, c.c_float, c.c_size_t
    P = c.POINTER
    sigs = {
        "radial_mask_build": (c.c_int, [i64, i64, i32, u32, P(vp)]),
        "radial_mask_build_ex": (c.c_int, [i64, i64, i32, u32, P(_MaskParams), P(vp)]),
        "radial_mask_params_default": (None, [P(_MaskParams)]),
        "radial_layout_info": (c.c_int, [vp, P(i64), P(i32), P(i64), P(i64)]),
        "radial_layout_export": (c.c_int, [vp, vp, vp, vp, vp]),
        "radial_layout_tile_flags": (c.c_int, [vp, vp, vp]),
        "radial_layout_band_table": (c.c_int, [vp, vp, vp, vp]),
        "radial_schedule_dense": (c.c_int, [i32, i32, i32, i32]),
        "radial_layout_token_mask": (c.c_int, [vp, vp, i64]),
        "radial_layout_upload": (c.c_int, [vp]),
        "radial_layout_destroy": (None, [vp]),
        "radial_attn_fwd": (c.c_int, [vp, i32, i32, i64, i32, f32, vp, vp, vp, vp, vp, vp]),
        "radial_attn_bwd_workspace_bytes": (sz, [vp, i32, i32, i64, i32]),
        "radial_attn_bwd": (c.c_int, [vp, i32, i32, i64, i32, f32, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, vp, sz, vp]),
        "radial_attn_bwd_noalloc": (c.c_int, [vp, i32, i32, i64, i32, f32, vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp, vp]),
        "radial_test_set_fwd_group": (c.c_int, [i32]),
        "radial_test_set_fail_alloc": (c.c_int, [i32]),
        "radial_status_string": (c.c_char_p, [c.c_int]),
        "radial_last_error": (c.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded library (loaded once).  RuntimeError if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m static_block_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise RadialError(status, lib().radial_last_error().decode())


class Layout:
    """Block-sparse layout of the radial mask (owns a ``radial_layout``).

    ``token_exact=False`` (the default) computes every kept tile in full;
    ``token_exact=True`` masks the tiles the mask only partly covers token by
    token, so the attention follows the token mask exactly.

    Mask variants (include/radial.h, radial_mask_params): ``decay`` "radial"
    or "harmonic", ``central_band`` d (frame pairs with |i - j| <= d attend in
    full) and ``width_scale`` (num, den), the ratio between consecutive
    bands' widths; the defaults give the radial mask."""

    def __init__(self, frames: int, tokens_per_frame: int, block_size: int = 128,
                 sink: bool = True, dense: bool = False, token_exact: bool = False,
                 decay: str = "radial", central_band: int = 1, width_scale=(2, 1)):
        flags = (SINK if sink else 0) | (DENSE if dense else 0) | (TOKEN_EXACT if token_exact else 0)
        if decay not in DECAYS:
            raise ValueError(f"decay must be one of {sorted(DECAYS)}")
        prm = _MaskParams(DECAYS[decay], int(central_band), int(width_scale[0]),
                          int(width_scale[1]))
        h = ctypes.c_void_p()
        _check(lib().radial_mask_build_ex(frames, tokens_per_frame, block_size, flags,
                                          ctypes.byref(prm), ctypes.byref(h)))
        self._h = h
        self.frames = frames
        self.tokens_per_frame = tokens_per_frame
        self.block_size = block_size
        self.sink = sink
        self.dense = dense
        self.token_exact = token_exact
        self.decay = decay
        self.central_band = int(central_band)
        self.width_scale = (int(width_scale[0]), int(width_scale[1]))
        n, nb, nz, pairs = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().radial_layout_info(h, ctypes.byref(n), ctypes.byref(nb), ctypes.byref(nz),
                                        ctypes.byref(pairs)))
        self.n = n.value
        self.n_blocks = nb.value
        self.nnz_tiles = nz.value
        self.nnz_pairs = pairs.value
        self._device = None

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.radial_layout_destroy(h)
            self._h = None

    def csr(self):
        rp = np.empty(self.n_blocks + 1, dtype=np.int32)
        ci = np.empty(self.nnz_tiles, dtype=np.int32)
        _check(lib().radial_layout_export(self._h, rp.ctypes.data, ci.ctypes.data, None, None))
        return rp, ci

    def csc(self):
        cp = np.empty(self.n_blocks + 1, dtype=np.int32)
        ri = np.empty(self.nnz_tiles, dtype=np.int32)
        _check(lib().radial_layout_export(self._h, None, None, cp.ctypes.data, ri.ctypes.data))
        return cp, ri

    def tile_flags(self):
        """(csr_full, csc_full): 1 where a kept tile holds only allowed pairs,
        in the order of ``csr()[1]`` and ``csc()[1]``."""
        a = np.empty(self.nnz_tiles, dtype=np.uint8)
        b = np.empty(self.nnz_tiles, dtype=np.uint8)
        _check(lib().radial_layout_tile_flags(self._h, a.ctypes.data, b.ctypes.data))
        return a.astype(bool), b.astype(bool)

    def band_table(self):
        r = np.empty(self.frames, dtype=np.int32)
        w = np.empty(self.frames, dtype=np.int64)
        p = np.empty(self.frames, dtype=np.int64)
        _check(lib().radial_layout_band_table(self._h, r.ctypes.data, w.ctypes.data, p.ctypes.data))
        return r, w, p

    def token_mask(self):
        out = np.empty((self.n, self.n), dtype=np.uint8)
        _check(lib().radial_layout_token_mask(self._h, out.ctypes.data, out.size))
        return out.astype(bool)

    def upload(self, device=None):
        """Copy the tile lists to a GPU (the current one by default)."""
        import torch
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        if self._device != dev:
            with torch.cuda.device(dev):
                _check(lib().radial_layout_upload(self._h))
            self._device = dev
        return self


class Schedule:
    """Per-call choice between the radial layout and the dense one (the
    first ``dense_layers`` layers, and at inference the first
    ``warmup_steps`` denoising steps, attend in full; radial_schedule_dense
    in include/radial.h).  Both layouts are built once and reused; the
    keyword arguments other than the schedule's go to the radial Layout.

        S = Schedule(33, 3600, dense_layers=2, warmup_steps=12)
        o, lse = S.fwd(q, k, v, layer=l, step=t)      # step=None: training
    """

    def __init__(self, frames: int, tokens_per_frame: int, block_size: int = 128,
                 dense_layers: int = 2, warmup_steps: int = 0, **layout_kwargs):
        if dense_layers < 0 or warmup_steps < 0:
            raise ValueError("dense_layers and warmup_steps must be >= 0")
        self.dense_layers = int(dense_layers)
        self.warmup_steps = int(warmup_steps)
        self.radial = Layout(frames, tokens_per_frame, block_size, **layout_kwargs)
        self.dense = Layout(frames, tokens_per_frame, block_size, dense=True,
                            sink=layout_kwargs.get("sink", True))

    def is_dense(self, layer: int, step: int | None = None) -> bool:
        warm = 0 if step is None else self.warmup_steps
        st = lib().radial_schedule_dense(int(layer), 0 if step is None else int(step),
                                         self.dense_layers, warm)
        if st < 0:
            _check(st)
        return st == 1

    def layout(self, layer: int, step: int | None = None) -> Layout:
        return self.dense if self.is_dense(layer, step) else self.radial

    def fwd(self, q, k, v, layer: int, step: int | None = None, **kw):
        return attn_fwd(q, k, v, self.layout(layer, step), **kw)

    def bwd(self, q, k, v, o, lse, do, layer: int, step: int | None = None, **kw):
        return attn_bwd(q, k, v, o, lse, do, self.layout(layer, step), **kw)

    def pairs(self, n_layers: int, n_steps: int | None = None) -> int:
        """Token pairs computed per batch and head over a whole run of
        n_layers layers x n_steps steps (one pass if n_steps is None)."""
        steps = [None] if n_steps is None else range(n_steps)
        return sum(self.layout(l, t).nnz_pairs for l in range(n_layers) for t in steps)

    def density(self, n_layers: int, n_steps: int | None = None) -> float:
        """Computed share of all token pairs over the run (1.0 = all dense)."""
        units = n_layers * (1 if n_steps is None else n_steps)
        return self.pairs(n_layers, n_steps) / (units * self.radial.n ** 2)


def _check_qkv(name, t, ref=None):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, D]")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ref is not None and (t.shape != ref.shape or t.device != ref.device):
        raise ValueError(f"{name} must match q in shape and device")


def attn_fwd(q, k, v, layout: Layout, scale: float | None = None, out=None, lse=None):
    """Radial attention forward.  Returns (o bf16 [B,H,N,D], lse fp32 [B,H,N])."""
    import torch
    _check_qkv("q", q)
    _check_qkv("k", k, q)
    _check_qkv("v", v, q)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    if out is not None:
        _check_qkv("out", o, q)
    if lse is not None and (l.dtype != torch.float32 or tuple(l.shape) != (B, H, N)
                            or not l.is_contiguous() or l.device != q.device):
        raise ValueError("lse must be contiguous fp32 [B, H, N] on q's device")
    layout.upload(q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        _check(lib().radial_attn_fwd(layout.handle, B, H, N, D, scale, q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), o.data_ptr(), l.data_ptr(), stream))
    return o, l


def attn_bwd(q, k, v, o, lse, do, layout: Layout, scale: float | None = None,
             workspace=None, out=None):
    """Radial attention backward.  Returns (dq, dk, dv), bf16 [B,H,N,D].
    ``out``: optional (dq, dk, dv) tensors to write into."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_qkv(name, t, None if name == "q" else q)
    B, H, N, D = q.shape
    if (not lse.is_cuda or lse.device != q.device or lse.dtype != torch.float32
            or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous fp32 [B, H, N] on q's device")
    if workspace is not None and (not workspace.is_cuda or workspace.device != q.device
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor on q's device")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    else:
        dq, dk, dv = out
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            _check_qkv(name, t, q)
    need = lib().radial_attn_bwd_workspace_bytes(layout.handle, B, H, N, D)
    ws = workspace
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    layout.upload(q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        _check(lib().radial_attn_bwd(layout.handle, B, H, N, D, scale, q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                     ws.numel() * ws.element_size(), stream))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, do, layout: Layout, scale: float | None = None, out=None):
    """``attn_bwd`` through radial_attn_bwd_noalloc: the library keeps the
    backward's row arrays in its static device scratch instead of a
    workspace (nothing is allocated when ``out`` is given).  Same results,
    bit for bit.  Calls that overlap on one device race on the scratch."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_qkv(name, t, None if name == "q" else q)
    B, H, N, D = q.shape
    if (not lse.is_cuda or lse.device != q.device or lse.dtype != torch.float32
            or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous fp32 [B, H, N] on q's device")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    else:
        dq, dk, dv = out
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            _check_qkv(name, t, q)
    layout.upload(q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        _check(lib().radial_attn_bwd_noalloc(layout.handle, B, H, N, D, scale, q.data_ptr(),
                                             k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                             lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                                             dk.data_ptr(), dv.data_ptr(), stream))
    return dq, dk, dv

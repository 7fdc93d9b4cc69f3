"""The gradient tolerance's rounding model against an emulation (CPU only).

The kernels round P and dS to bf16 before the products and form Delta from
the bf16 O they returned.  Emulating exactly those roundings in float64 on
small masks (few keys per row with every query on the sink, and long rows)
gives errors that the allowance built from ``gpu_util.rounding_sigmas`` must
cover, while planted mistakes of the size a kernel bug makes (one key row off
by 5%, a 3% scale, two swapped head-dim columns) must still fail.
"""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import check_close, rounding_sigmas
from oracle import attention as oa
from oracle import mask as om


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _emulated_grads(q, k, v, do, mask, scale):
    z = np.where(mask, scale * (q @ k.T), -np.inf)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = _bf16(p @ v)                                   # the forward's bf16 output
    ds = _bf16(p * (do @ v.T - (do * o).sum(axis=1, keepdims=True)))
    return dict(dq=_bf16(scale * (ds @ k)), dk=_bf16(scale * (ds.T @ q)),
                dv=_bf16(_bf16(p).T @ do))


@pytest.mark.parametrize("f,s,sink,variant", [
    (700, 1, True, om.Variant(central=0, scale=(3, 1))),   # two keys per row, all on the sink
    (300, 2, True, om.Variant(central=2, scale=(4, 1))),
    (12, 100, True, om.Variant()),                          # long rows
    (40, 20, False, om.Variant(decay="harmonic")),
])
def test_rounding_model_covers_the_emulation_and_catches_mistakes(f, s, sink, variant):
    n, D = f * s, 64
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = (t[0, 0].double().numpy()
                   for t in workloads.make_inputs(1, 1, n, D, 4242 + f, with_dout=True))
    mask = om.token_mask(f, s, sink, variant)
    ref = dict(zip(("dq", "dk", "dv"), oa.bwd_masked(q, k, v, do, mask, scale)))
    sig = rounding_sigmas(q, k, v, do, mask, scale)
    emu = _emulated_grads(q, k, v, do, mask, scale)
    for name in ("dq", "dk", "dv"):
        check_close(emu[name], ref[name], name, normalise=True, term=sig[name])
        rms = float(np.sqrt(np.mean(ref[name] ** 2)))
        row = emu[name].copy()
        row[n // 2] = row[n // 2] * 1.05 + 0.05 * rms
        swapped = emu[name][:, [1, 0] + list(range(2, D))]
        for bad in (row, emu[name] * 1.03, swapped):
            with pytest.raises(AssertionError):
                check_close(bad, ref[name], name, normalise=True, term=sig[name])

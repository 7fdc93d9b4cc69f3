"""GPU check of the schedule hook: each call runs the layout the schedule
picks, through the same kernels (bitwise equal to calling that layout
directly)."""

import pytest
import torch

import static_block_sparse_amd as sba
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_schedule_calls_run_the_picked_layout():
    f, s, T, D = 9, 200, 128, 128
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(1, 2, f * s, D, 801, with_dout=True))
    S = sba.Schedule(f, s, T, dense_layers=2, warmup_steps=3)
    ref = {}
    for name, L in (("dense", S.dense), ("radial", S.radial)):
        o, lse = sba.attn_fwd(q, k, v, L)
        ref[name] = (o, lse) + tuple(sba.attn_bwd(q, k, v, o, lse, do, L))
    assert not torch.equal(ref["dense"][0], ref["radial"][0])
    for layer, step, want in [(0, 10, "dense"), (1, None, "dense"), (4, 1, "dense"),
                              (4, 3, "radial"), (7, None, "radial")]:
        o, lse = S.fwd(q, k, v, layer, step)
        g = S.bwd(q, k, v, o, lse, do, layer, step)
        torch.cuda.synchronize()
        for x, y in zip((o, lse) + tuple(g), ref[want]):
            assert torch.equal(x, y), (layer, step, want)

"""Host tests of the layer/step schedule hook (no GPU needed).

The pages keep the first two layers dense in training and inference and run
the first 12 of 50 denoising steps (2 for 4x longer videos) dense at
inference; radial_schedule_dense decides per call, Schedule holds both
layouts.
"""

import pytest

import static_block_sparse_amd as sba


def test_decision_grid():
    lib = sba.lib()
    for layer in range(6):
        for step in range(15):
            for dl, ws in [(2, 12), (0, 0), (2, 0), (0, 2), (3, 1)]:
                want = 1 if (layer < dl or step < ws) else 0
                assert lib.radial_schedule_dense(layer, step, dl, ws) == want


@pytest.mark.parametrize("args", [(-1, 0, 2, 12), (0, -1, 2, 12), (0, 0, -2, 12), (0, 0, 2, -1)])
def test_decision_rejects_negative(args):
    assert sba.lib().radial_schedule_dense(*args) == -1
    assert sba.lib().radial_last_error().decode()


def test_schedule_picks_layouts_and_counts_work():
    S = sba.Schedule(33, 3600, 128, dense_layers=2, warmup_steps=12)
    assert S.layout(0, 30) is S.dense and S.layout(1, 49) is S.dense
    assert S.layout(2, 11) is S.dense and S.layout(2, 12) is S.radial
    assert S.layout(5) is S.radial and S.layout(1) is S.dense      # training: no warm-up
    n2 = S.radial.n ** 2
    assert S.dense.nnz_pairs == n2
    # 60 layers x 50 steps: 2 dense layers for all steps, 12 warm-up steps
    # for the other 58, radial for the remaining 58 x 38
    dense_units = 2 * 50 + 58 * 12
    assert S.pairs(60, 50) == dense_units * n2 + 58 * 38 * S.radial.nnz_pairs
    assert S.density(60, 50) == pytest.approx(S.pairs(60, 50) / (3000 * n2))
    assert S.pairs(60) == 2 * n2 + 58 * S.radial.nnz_pairs


def test_schedule_passes_mask_options():
    S = sba.Schedule(8, 256, 64, dense_layers=1, sink=False, central_band=2, token_exact=True)
    L = S.radial
    assert (L.sink, L.central_band, L.token_exact) == (False, 2, True)
    assert S.dense.dense and not S.dense.sink
    with pytest.raises(ValueError):
        sba.Schedule(8, 256, 64, dense_layers=-1)

"""Guard-padded outputs on the GPU (needs an MI355X).

Every output (O, LSE, dQ, dK, dV) and the backward workspace is a view in the
middle of a larger buffer whose guard zones hold a known bit pattern.  After
the forward and backward the guards must be unchanged, the inputs must be
unchanged, and the outputs must equal (bit for bit) those of a call with plain
tensors.  Ragged shapes (last tile partly past N), both tile sizes,
token-exact mode and a mask variant are covered.
"""

import sys

import pytest
import torch

import static_block_sparse_amd as sba
import workloads

pytestmark = pytest.mark.gpu

GUARD = 4096          # elements on each side (a multiple of 8: keeps 16-byte alignment)
PAT16 = 0x7FA5        # a NaN bit pattern no kernel writes
PAT32 = 0x7FC0A5A5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _guarded(shape, dtype):
    n = 1
    for d in shape:
        n *= d
    itype = torch.int16 if dtype == torch.bfloat16 else torch.int32
    raw = torch.full((n + 2 * GUARD,), PAT16 if itype == torch.int16 else PAT32, dtype=itype,
                     device="cuda")
    view = raw.view(dtype)[GUARD:GUARD + n].view(shape)
    return raw, view


def _guards_intact(raw):
    pat = PAT16 if raw.dtype == torch.int16 else PAT32
    return bool((raw[:GUARD] == pat).all()) and bool((raw[-GUARD:] == pat).all())


@pytest.mark.parametrize("f,s,T,kw", [
    (5, 300, 128, {}),
    (7, 100, 64, {}),
    (40, 20, 64, {"token_exact": True}),
    (9, 200, 128, {"token_exact": True, "decay": "harmonic"}),
    (33, 36, 128, {"central_band": 2, "sink": False}),
], ids=["ragged128", "ragged64", "exact", "exact-harmonic", "d2-nosink"])
def test_outputs_stay_inside_their_buffers(f, s, T, kw):
    D, B, H = T, 1, 2
    N = f * s
    print(f"[guards] f={f} s={s} T={T} {kw}", file=sys.stderr, flush=True)
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(B, H, N, D, 900 + f, with_dout=True))
    inputs = [t.clone() for t in (q, k, v, do)]
    L = sba.Layout(f, s, T, **kw)
    o_ref, lse_ref = sba.attn_fwd(q, k, v, L)
    g_ref = sba.attn_bwd(q, k, v, o_ref, lse_ref, do, L)

    raw_o, o = _guarded((B, H, N, D), torch.bfloat16)
    raw_l, lse = _guarded((B, H, N), torch.float32)
    sba.attn_fwd(q, k, v, L, out=o, lse=lse)
    outs = [_guarded((B, H, N, D), torch.bfloat16) for _ in range(3)]
    need = sba.lib().radial_attn_bwd_workspace_bytes(L.handle, B, H, N, D)
    raw_w = torch.full((need // 4 + 2 * GUARD,), PAT32, dtype=torch.int32, device="cuda")
    ws = raw_w[GUARD:GUARD + need // 4].view(torch.uint8)
    sba.attn_bwd(q, k, v, o, lse, do, L, workspace=ws, out=tuple(t for _, t in outs))
    torch.cuda.synchronize()

    for name, raw in [("O", raw_o), ("LSE", raw_l), ("workspace", raw_w)] + \
                     [(n, r) for n, (r, _) in zip(("dQ", "dK", "dV"), outs)]:
        assert _guards_intact(raw), f"{name}: a guard zone was written"
    for a, b in zip(inputs, (q, k, v, do)):
        assert torch.equal(a, b), "an input was modified"
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    for (_, got), ref in zip(outs, g_ref):
        assert torch.equal(got, ref)

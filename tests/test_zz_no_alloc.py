"""GPU test of the allocation-free backward entry point (needs an MI355X).

radial_attn_bwd_noalloc keeps the backward's row arrays in the library's
static device scratch instead of a caller workspace; it runs the same
kernels as radial_attn_bwd, so its gradients must equal that entry point's
bit for bit.  Two calls in a row, the second on a smaller input (the scratch
keeps the first call's contents), and a size beyond the scratch is refused
before anything is launched.
"""

import ctypes
import sys

import pytest
import torch

import static_block_sparse_amd as sba
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(f, s, T, D, B, H, seed, **kw):
    print(f"[noalloc] f={f} s={s} T={T} D={D} B={B} H={H} {kw}", file=sys.stderr, flush=True)
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(B, H, f * s, D, seed, with_dout=True))
    L = sba.Layout(f, s, T, **kw)
    o, lse = sba.attn_fwd(q, k, v, L)
    return L, q, k, v, o, lse, do


def test_noalloc_backward_matches_workspace_backward_twice():
    # first call: 2 x 3 heads of 7 frames x 300 tokens (ragged tiles); second
    # call: a smaller input, so stale rows of the first call sit in the
    # scratch past the second call's arrays
    cases = [dict(f=7, s=300, T=128, D=128, B=2, H=3, seed=41),
             dict(f=5, s=100, T=64, D=64, B=1, H=2, seed=42, token_exact=True)]
    for c in cases:
        L, q, k, v, o, lse, do = _case(**c)
        ref = sba.attn_bwd(q, k, v, o, lse, do, L)
        got = sba.attn_bwd_noalloc(q, k, v, o, lse, do, L)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), name
            assert bool(torch.isfinite(a.float()).all()), name


def test_noalloc_backward_at_the_training_workload():
    # the training workload's shape (66 frames x 3600 tokens) on 4 of its 24
    # heads; its row arrays (7.6 MB) fit the scratch
    w = workloads.WORKLOADS["train_f66"]
    g = torch.Generator("cuda").manual_seed(77)
    shape = (1, 4, w.N, w.D)
    q, k, v, do = (torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(4))
    L = sba.Layout(w.frames, w.tokens_per_frame, w.T)
    o, lse = sba.attn_fwd(q, k, v, L, w.scale)
    ref = sba.attn_bwd(q, k, v, o, lse, do, L, w.scale)
    got = sba.attn_bwd_noalloc(q, k, v, o, lse, do, L, w.scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name


def test_noalloc_backward_refuses_sizes_beyond_the_scratch():
    # B * H * N = 4100 * 2048 rows: the two row arrays need 67.2 MB, more than
    # the 64 MiB scratch.  Real (uninitialised) tensors back every pointer,
    # although the call must return before launching anything.
    L = sba.Layout(8, 256, 64).upload()
    B, H, N, D = 1, 4100, 2048, 64
    need = sba.lib().radial_attn_bwd_workspace_bytes(L.handle, B, H, N, D)
    assert need > (64 << 20)
    t = [torch.empty((B, H, N, D), dtype=torch.bfloat16, device="cuda") for _ in range(8)]
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    q, k, v, o, do, dq, dk, dv = t
    st = sba.lib().radial_attn_bwd_noalloc(
        L.handle, B, H, N, D, 0.125, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
        lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -2, st
    assert "scratch" in sba.lib().radial_last_error().decode()
    torch.cuda.synchronize()


def test_noalloc_backward_under_graph_capture():
    # the callers the entry point is for: the forward and the allocation-free
    # backward captured in one graph (layout uploaded and outputs allocated
    # beforehand), replayed three times with eager work and a synchronisation
    # between replays; every replay must give the eager result bit for bit
    f, s, T, D, B, H = 6, 300, 128, 128, 1, 2
    L = sba.Layout(f, s, T).upload()
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(B, H, f * s, D, 77, with_dout=True))
    o_ref, lse_ref = sba.attn_fwd(q, k, v, L)
    ref = sba.attn_bwd(q, k, v, o_ref, lse_ref, do, L)
    o, lse = torch.empty_like(q), torch.empty_like(lse_ref)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        sba.attn_fwd(q, k, v, L, out=o, lse=lse)
        sba.attn_bwd_noalloc(q, k, v, o, lse, do, L, out=grads)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sba.attn_fwd(q, k, v, L, out=o, lse=lse)
        sba.attn_bwd_noalloc(q, k, v, o, lse, do, L, out=grads)
    for rep in range(3):
        for t in (o, lse) + grads:
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), rep
        for name, a, b in zip(("dq", "dk", "dv"), grads, ref):
            assert torch.equal(a, b), (rep, name)

"""The library's launches inside a captured HIP graph (torch.cuda.CUDAGraph):
the entry points only enqueue kernels on the caller's stream -- no
allocation, no synchronisation, no memset -- so a capture of fa_fwd_ex,
fa_decode_splitk and fa_bwd with preallocated outputs and workspaces replays
correctly; so does fa_decode_splitk_mq, and fa_decode_splitk_static,
whose partial states live in the library's own device scratch (the entry
point made for capture: the caller passes no workspace).  Each replay
follows fresh inputs written eagerly into the captured buffers, with eager
library work and a synchronisation in between, and must equal the eager
calls on the same inputs bit for bit (same kernels, same launch
parameters)."""

import pytest
import torch

import workloads
from tests.parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_05_amd as fa

    fa.lib()
    return torch.device("cuda:0")


def test_graph_capture_and_replay(dev):
    import online_softmax_05_amd as fa

    B, H, N, d = 2, 4, 300, 128
    q = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    k, v, g = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    bws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N) // 4, dtype=torch.float32, device=dev)
    Bd, Hd, Nkd = 4, 8, 1500
    qd = torch.empty((Bd, Hd, d), dtype=torch.bfloat16, device=dev)
    kc = torch.empty((Bd, Hd, Nkd, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    kl = torch.empty((Bd,), dtype=torch.int32, device=dev)
    od, ld = torch.empty((Bd, Hd, d), dtype=torch.bfloat16, device=dev), torch.empty((Bd, Hd), device=dev)
    dws = torch.empty(fa.fa_decode_splitk_workspace_bytes(Bd, Hd, Nkd, d, 512) // 4, dtype=torch.float32, device=dev)
    nqm = 4
    qm = torch.empty((Bd, Hd, nqm, d), dtype=torch.bfloat16, device=dev)
    om, lm = torch.empty_like(qm), torch.empty((Bd, Hd, nqm), device=dev)
    mws = torch.empty(fa.fa_decode_splitk_mq_workspace_bytes(Bd, Hd, nqm, Nkd, d, 256) // 4, dtype=torch.float32,
                      device=dev)
    os_, ls_ = torch.empty_like(od), torch.empty_like(ld)

    def fill(seed):
        gen = torch.Generator().manual_seed(seed)
        for t in (q, k, v, g, qd, kc, vc, qm):
            t.copy_(torch.randn(t.shape, generator=gen).to(t.dtype))
        kl.copy_(torch.randint(1, Nkd + 1, (Bd,), generator=gen, dtype=torch.int32))

    def calls():
        fa.fa_fwd_ex(q, k, v, causal=True, window_left=100, keep_256=230, seed=7, out=o, lse=lse)
        fa.fa_bwd_ex(q, k, v, o, g, lse, causal=True, window_left=100, keep_256=230, seed=7, dq=dq, dk=dk, dv=dv,
                     workspace=bws)
        fa.fa_decode_splitk(qd, kc, vc, kl, chunk=512, out=od, lse=ld, workspace=dws)
        fa.fa_decode_splitk_mq(qm, kc, vc, kl, causal=True, chunk=256, out=om, lse=lm, workspace=mws)
        fa.fa_decode_splitk_static(qd, kc, vc, kl, out=os_, lse=ls_, chunk=64)

    fill(1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on a side stream, as torch's capture recipe asks
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("capturing fa_fwd_ex + fa_bwd_ex + fa_decode_splitk + fa_decode_splitk_mq + fa_decode_splitk_static")
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    outs = (o, lse, dq, dk, dv, od, ld, om, lm, os_, ls_)
    for rep, seed in enumerate((11, 12, 13)):
        fill(seed)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        calls()  # eager work between replays, on the same inputs
        torch.cuda.synchronize()
        say(f"graph replay {rep}: comparing {len(outs)} outputs with the eager calls")
        names = ("o", "lse", "dq", "dk", "dv", "o_dec", "lse_dec", "o_mq", "lse_mq", "o_static", "lse_static")
        for name, a, b in zip(names, got, outs):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"

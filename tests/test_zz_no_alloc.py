"""The decode entry point that allocates nothing (fa_decode_splitk_static)
against the one that takes a workspace (fa_decode_splitk).

Both run the same kernels; only where the partial states live differs (a
static device array of the library instead of a caller buffer).  Two calls
in a row, the second on a smaller input, so that the second call runs over
the first call's leftover states in the shared array: each output must equal
fa_decode_splitk's bit for bit, and both must match the float64 oracle at
the usual tolerances (bf16: o 2e-2, lse 1e-3; fp32: 1e-5; k_len = 0 gives
o = 0, lse = -inf exactly).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.parity_util import compare, f64, say, scale32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_05_amd as fa

    fa.lib()
    return torch.device("cuda:0")


def _case(seed, B, H, Nk, d, dt, k_len):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, d, generator=g).to(dt)
    k = torch.randn(B, H, Nk, d, generator=g).to(dt)
    v = torch.randn(B, H, Nk, d, generator=g).to(dt)
    return q, k, v, torch.tensor(k_len, dtype=torch.int32)


def _oracle(q, k, v, kl):
    B, H, d = q.shape
    o = np.zeros((B, H, v.shape[3]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = int(kl[b])
        for h in range(H):
            ob, lb = oracle.attention_head(f64(q[b, h])[None], f64(k[b, h, :n]), f64(v[b, h, :n]),
                                           scale=scale32(1 / np.sqrt(d)), nq=1)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_static_decode_matches_workspace_decode(dev, dt):
    import online_softmax_05_amd as fa

    calls = [
        (1000, 6, 8, 2600, 128, [2600, 1, 1537, 0, 700, 2048]),   # 6 chunks per sequence-head
        (1001, 3, 4, 1100, 128, [513, 1100, 64]),                 # smaller: over the first call's states
    ]
    for seed, B, H, Nk, d, kl in calls:
        q, k, v, k_len = _case(seed, B, H, Nk, d, dt, kl)
        say(f"static decode {dt}: B {B} H {H} Nk {Nk} d {d} k_len {kl}")
        qd, kd, vd, kld = q.to(dev), k.to(dev), v.to(dev), k_len.to(dev)
        o_ws, l_ws = fa.fa_decode_splitk(qd, kd, vd, kld, chunk=512)
        o_st = torch.empty_like(o_ws)
        l_st = torch.empty_like(l_ws)
        fa.fa_decode_splitk_static(qd, kd, vd, kld, out=o_st, lse=l_st, chunk=512)
        torch.cuda.synchronize()
        assert torch.equal(o_ws, o_st), "static-scratch output differs from the workspace call"
        assert torch.equal(l_ws, l_st), "static-scratch lse differs from the workspace call"
        o_ref, lse_ref = _oracle(q, k, v, kl)
        compare(o_st, l_st, o_ref, lse_ref, dt, f"static decode {dt} B {B} H {H}")


def test_static_decode_rejects_oversized(dev):
    import online_softmax_05_amd as fa

    # 64 x 64 sequence-heads of 8192 keys in 512-key chunks need 34 MB of states
    q = torch.zeros(64, 64, 128, dtype=torch.bfloat16, device=dev)
    k = torch.empty(64, 64, 8192, 128, dtype=torch.bfloat16, device=dev)  # never read: rejected on the host
    k_len = torch.full((64,), 8192, dtype=torch.int32, device=dev)
    out = torch.empty(64, 64, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(fa.FaError) as e:
        fa.fa_decode_splitk_static(q, k, k, k_len, out=out, chunk=512)
    assert e.value.status == 4

"""GPU parity of the multi-query split-KV path (fa_decode_splitk_mq) against
the float64 oracle.

The Nq query rows of sequence b are its last Nq positions; with the causal
flag row i sees keys j <= i + k_len[b] - Nq ([GS] section 6, bottom-right
alignment taken against the sequence's own length).  The oracle is therefore
the dense definition applied to the cache truncated to k_len[b] keys
(bottom-right causal over Nk = k_len[b]).  Tolerances as for the forward
pass: fp32 1e-5 for o and lse; bf16 2e-2 for o and 1e-3 for lse; rows with no
allowed key exactly o = 0 and lse = -inf.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import compare, compare_every_head, f64, say, scale32

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_05_amd as fa

    fa.lib()
    return torch.device("cuda:0")


def oracle_mq(q, k, v, k_len, scale, causal):
    B, H, Nq, _ = q.shape
    dv = v.shape[3]
    o = np.zeros((B, H, Nq, dv))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        n = int(k_len[b])
        for h in range(H):
            ob, lb = oracle.attention_head(f64(q[b, h]), f64(k[b, h, :n]), f64(v[b, h, :n]), scale=scale32(scale),
                                           nq=Nq, causal=causal)
            o[b, h], lse[b, h] = ob, lb
    return o, lse


CASES = [
    # (B, H, Nq, Nk_max, dk, dv, causal, chunk)
    (3, 2, 4, 700, 128, 128, True, 512),    # matrix-core path
    (2, 3, 16, 1300, 128, 128, True, 256),
    (2, 2, 1, 900, 128, 128, False, 512),
    (2, 2, 7, 333, 128, 128, False, 64),
    (2, 2, 5, 500, 64, 64, True, 128),      # general path
    (1, 3, 3, 200, 40, 24, True, 64),
    (2, 2, 3, 8400, 128, 128, True, 64),    # more than 64 chunks per row (the merge's chunk groups)
    (2, 1, 2, 4300, 64, 24, False, 64),
    (2, 2, 4, 4500, 128, 128, True, 2048),  # matrix-core path, the largest chunk, a ragged last chunk
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_mq_parity(dev, case, dt):
    import online_softmax_05_amd as fa

    B, H, Nq, Nk, dk, dv, causal, chunk = CASES[case]
    dtype = DT[dt]
    inp = workloads.seeded_case(400 + case, B, H, Nq, Nk, dk, dv, dtype)
    g = torch.Generator().manual_seed(500 + case)
    # lengths: the full cache, a few keys (fewer than Nq: empty causal rows), empty, random
    k_len = torch.randint(1, Nk + 1, (B,), generator=g, dtype=torch.int32)
    k_len[0] = Nk
    if B > 1:
        k_len[1] = max(0, min(Nk, Nq // 2))
    if B > 2:
        k_len[2] = 0
    say(f"decode mq case {case} {dt}: B {B} H {H} Nq {Nq} Nk {Nk} d {dk}/{dv} causal {causal} chunk {chunk} "
        f"k_len {k_len.tolist()}")
    d = workloads.to_device(inp, dev)
    o, lse = fa.fa_decode_splitk_mq(d["q"], d["k"], d["v"], k_len.to(dev), causal=causal, scale=inp["scale"],
                                    chunk=chunk)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_mq(inp["q"], inp["k"], inp["v"], k_len, inp["scale"], causal)
    compare(o, lse, o_ref, lse_ref, dtype, f"decode mq case {case} {dt}")


def test_decode_mq_single_row_matches_decode(dev):
    """With Nq = 1 the multi-query path computes what fa_decode_splitk does."""
    import online_softmax_05_amd as fa

    inp = workloads.seeded_case(450, 4, 2, 1, 1500, 128, 128, torch.bfloat16)
    k_len = torch.tensor([1500, 1, 777, 1024], dtype=torch.int32, device=dev)
    d = workloads.to_device(inp, dev)
    o1, l1 = fa.fa_decode_splitk(d["q"][:, :, 0].contiguous(), d["k"], d["v"], k_len, scale=inp["scale"])
    o2, l2 = fa.fa_decode_splitk_mq(d["q"], d["k"], d["v"], k_len, causal=True, scale=inp["scale"])
    torch.cuda.synchronize()
    assert float((o1.float() - o2[:, :, 0].float()).abs().max()) <= 2e-2
    assert float((l1 - l2[:, :, 0]).abs().max()) <= 1e-3


def test_decode_mq_full_size_every_row(dev):
    """The multi-query decode workload (64x32 sequences x 4 causal rows, caches
    of 8192 keys, lengths U{1..8192}, d128 bf16, 2048-key chunks) in the launch
    configuration the benchmark times: every row of every (sequence, head)
    against the oracle over the cache truncated to the sequence's length."""
    import online_softmax_05_amd as fa

    inp = workloads.decode_mq(dev)
    kl = inp["k_len_host"]
    say(f"decode mq full size 64x32x4, kv 8192, lengths {int(kl.min())}..{int(kl.max())}")
    o, lse = fa.fa_decode_splitk_mq(inp["q"], inp["k"], inp["v"], inp["k_len"], causal=True, scale=inp["scale"],
                                    chunk=inp["chunk"])
    torch.cuda.synchronize()
    compare_every_head(o, lse, inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True, k_len_host=kl,
                       what="decode mq full size")

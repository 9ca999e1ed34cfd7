"""Caches whose single head spans more than 2^31 bytes.

The decode entry points address a head's K and V through 64-bit base
offsets (each wave or chunk builds a buffer descriptor of a few kilobytes
at its own rows), so one head's cache may exceed what a single 32-bit
descriptor could cover.  One sequence and head with 9e6 keys of d = 128
(2.3 GB each for K and V), the key length 3 keys short of the end, through
the single-query and the multi-query split-K decodes.  The reference merges
the oracle's per-block states (m, l, u) of 1e6-key blocks, which the merge
rule makes exact ([GS] section 4; [OA] "Updating the Exponential Sum and
Weighted Sum Together"); tolerances as everywhere for bf16 (o 2e-2, lse
1e-3).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import compare, f64, say, scale32

pytestmark = pytest.mark.gpu

BLOCK = 1_000_000


@pytest.fixture(scope="module")
def big(dev):
    say("large cache: drawing 1 x 1 x 9e6 x 128 bf16 K and V on the device")
    inp = workloads.long_cache(dev)
    host = {n: inp[n][0, 0].to("cpu") for n in ("q", "k", "v")}
    return inp, host


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_05_amd as fa

    fa.lib()
    return torch.device("cuda:0")


def reference(host, scale, ends):
    """o [len(ends), dv], lse: row i attends to keys [0, ends[i]) of the
    cache, merged from 1e6-key block states."""
    q = f64(host["q"])
    out_o, out_l = [], []
    states = [None] * len(ends)
    for lo in range(0, max(ends), BLOCK):
        hi = min(lo + BLOCK, max(ends))
        kb = f64(host["k"][lo:hi])
        vb = f64(host["v"][lo:hi])
        x = (kb @ q.T) * scale  # [rows, nq]
        for i, end in enumerate(ends):
            n = min(hi, end) - lo
            if n > 0:
                states[i] = oracle.merge_states(states[i], oracle.block_state(x[:n, i], vb[:n]))
    for m, l, u in states:
        out_o.append(u / l)
        out_l.append(m + np.log(l))
    return np.stack(out_o), np.array(out_l)


def test_decode_head_past_2gib(dev, big):
    import online_softmax_05_amd as fa

    inp, host = big
    klen = int(inp["k_len"][0])
    say(f"large cache: fa_decode_splitk over {klen} keys")
    o, lse = fa.fa_decode_splitk(inp["q"][:, :, 0], inp["k"], inp["v"], inp["k_len"].to(dev), scale=inp["scale"])
    torch.cuda.synchronize()
    host1 = dict(host, q=host["q"][:1])
    o_ref, lse_ref = reference(host1, scale32(inp["scale"]), [klen])
    compare(o[0, 0][None], lse[0, 0][None], o_ref, lse_ref, torch.bfloat16, "decode, head past 2^31 bytes")


def test_decode_mq_head_past_2gib(dev, big):
    import online_softmax_05_amd as fa

    inp, host = big
    klen = int(inp["k_len"][0])
    nq = inp["q"].shape[2]
    say(f"large cache: fa_decode_splitk_mq, {nq} causal rows over {klen} keys")
    o, lse = fa.fa_decode_splitk_mq(inp["q"], inp["k"], inp["v"], inp["k_len"].to(dev), causal=True,
                                    scale=inp["scale"], chunk=2048)
    torch.cuda.synchronize()
    # bottom-right causal: row i of the last nq positions sees klen - (nq - 1 - i) keys
    o_ref, lse_ref = reference(host, scale32(inp["scale"]), [klen - (nq - 1 - i) for i in range(nq)])
    compare(o[0, 0], lse[0, 0], o_ref, lse_ref, torch.bfloat16, "multi-query decode, head past 2^31 bytes")

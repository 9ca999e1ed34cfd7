"""GPU parity of the mask variants (fa_fwd_ex): top-left causal alignment and
sliding windows measured from the aligned position ([GS] section 6), against
the float64 oracle on the same seeded inputs.

Tolerances as for the plain forward: fp32 1e-5 and bf16 2e-2 (o) / 1e-3
(lse) in max abs; rows left with no visible key must be exactly o = 0 and
lse = -inf.  The small cases span several 128-row blocks and 64-key tiles with
ragged tails, so that tiles are skipped at both ends, masked at both edges and
left whole in between; the full-size case is the prefill shape with a
1024-key causal window, compared on sampled rows of two heads.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import compare, compare_every_head, f64, oracle_full, say

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_05_amd as fa

    fa.lib()
    return torch.device("cuda:0")


def run_ex(inp, dev, block_n=0):
    import online_softmax_05_amd as fa

    d = workloads.to_device(inp, dev)
    o, lse = fa.fa_fwd_ex(d["q"], d["k"], d["v"], bias=d.get("bias"), k_len=d.get("k_len"), scale=inp["scale"],
                          causal=inp["causal"], align=inp["align"], window_left=inp["window_left"],
                          window_right=inp["window_right"], block_n=block_n)
    torch.cuda.synchronize()
    return o, lse


# (Nq, Nk, dk, dv, causal, align, wl, wr, bias, k_len)
CASES = [
    (200, 333, 64, 64, True, "top_left", None, None, False, None),
    (333, 200, 64, 64, True, "top_left", None, None, False, None),
    (300, 300, 128, 128, True, "top_left", None, None, True, "random"),
    (700, 700, 128, 128, True, "bottom_right", 63, None, False, None),
    (517, 700, 128, 128, True, "bottom_right", 200, None, False, "random"),
    (700, 517, 64, 128, True, "top_left", 130, None, True, None),
    (300, 517, 128, 64, False, "top_left", 100, 37, True, "random"),
    (400, 150, 64, 64, True, "bottom_right", 10, None, False, None),   # rows 0..249 empty
    (300, 300, 128, 128, True, "bottom_right", 20, None, False, [60, 300]),  # rows past 80 see nothing in b=0
    (257, 257, 128, 128, False, "bottom_right", 0, 0, False, None),   # one key per row
    (130, 390, 128, 128, False, "top_left", None, 5, False, None),    # right edge only
    (190, 190, 64, 64, True, "bottom_right", 1000, None, False, None),  # window wider than the sequence
]


def _case_id(c):
    nq, nk, dk, dv, causal, align, wl, wr, bias, kl = c
    return (f"{nq}x{nk}_d{dk}-{dv}_{'c' if causal else 'nc'}_{align}_wl{wl}_wr{wr}" + ("_bias" if bias else "")
            + ("" if kl is None else "_klen"))


def make_case(c, dtype, seed):
    nq, nk, dk, dv, causal, align, wl, wr, bias, kl = c
    B = 2 if kl is not None else 1
    inp = workloads.seeded_case(seed, B, 2, nq, nk, dk, dv, dtype, causal=causal, bias=bias, k_len=kl)
    inp.update(align=align, window_left=wl, window_right=wr)
    return inp


@pytest.mark.parametrize("case", CASES, ids=_case_id)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_mask_variants(dev, case, dt):
    inp = make_case(case, DT[dt], 4000 + CASES.index(case))
    o_ref, lse_ref = oracle_full(inp)
    for bn in (32, 64, 128):
        say(f"mask variant {_case_id(case)} {dt} block_n={bn}")
        o, lse = run_ex(inp, dev, block_n=bn)
        compare(o, lse, o_ref, lse_ref, DT[dt], f"{_case_id(case)} {dt} bn={bn}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_window_zero_picks_aligned_key(dev, dt):
    """Causal with a left width 0: each row sees only the key at its aligned
    position, so o_i = v_{pos_i} exactly and lse_i = s_{i,pos_i}."""
    for align, nq, nk in (("bottom_right", 150, 230), ("top_left", 230, 150)):
        inp = make_case((nq, nk, 64, 64, True, align, 0, None, False, None), DT[dt], 4100)
        say(f"window 0 {align} {dt}")
        o, lse = run_ex(inp, dev)
        off = nk - nq if align == "bottom_right" else 0
        v = f64(inp["v"])
        oo = f64(o)
        for i in range(nq):
            p = i + off
            if 0 <= p < nk:
                assert np.array_equal(oo[0, :, i], v[0, :, p]), (align, i)
            else:
                assert np.all(oo[0, :, i] == 0.0) and np.all(np.isneginf(f64(lse)[0, :, i]))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_plain_masks_match_fa_fwd(dev, dt):
    """fa_fwd_ex without a window and with bottom-right alignment is fa_fwd,
    bit for bit (the same kernel runs); top-left alignment with Nq == Nk is
    the same mask and agrees to rounding."""
    import online_softmax_05_amd as fa

    inp = workloads.seeded_case(4200, 2, 3, 320, 320, 128, 128, DT[dt], causal=True)
    d = workloads.to_device(inp, dev)
    say(f"plain masks vs fa_fwd {dt}")
    o1, l1 = fa.fa_fwd(d["q"], d["k"], d["v"], causal=True)
    o2, l2 = fa.fa_fwd_ex(d["q"], d["k"], d["v"], causal=True)
    o3, l3 = fa.fa_fwd_ex(d["q"], d["k"], d["v"], causal=True, align="top_left")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle_full(inp)
    compare(o3, l3, o_ref, lse_ref, DT[dt], f"top-left Nq == Nk {dt}")


def test_full_size_sliding_window(dev):
    """The prefill shape (4x32x4096, d128, bf16) with a causal 1024-key window,
    in the launch configuration the benchmark times: every row of every head
    against the oracle."""
    import online_softmax_05_amd as fa

    inp = workloads.prefill(dev)
    wl = 1023
    say("full-size sliding window 4x32x4096 d128 bf16, window 1024")
    o, lse = fa.fa_fwd_ex(inp["q"], inp["k"], inp["v"], causal=True, window_left=wl, scale=inp["scale"])
    torch.cuda.synchronize()
    compare_every_head(o, lse, inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True, window=(wl, None),
                       what="full-size window 1024")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_huge_windows_are_no_mask(dev, dt):
    """Window widths near 2^31 (the row-range arithmetic is 64-bit) select
    every key: the result equals the unwindowed call bit for bit, for both
    alignments and with and without causal."""
    import online_softmax_05_amd as fa

    big = 2**31 - 1
    inp = workloads.seeded_case(4300, 2, 2, 190, 270, 128, 128, DT[dt], causal=False, bias=True, k_len="random")
    d = workloads.to_device(inp, dev)
    for causal in (False, True):
        for align in ("bottom_right", "top_left"):
            say(f"huge windows {dt} causal={causal} {align}")
            kw = dict(bias=d["bias"], k_len=d["k_len"], scale=inp["scale"], causal=causal, align=align)
            a = fa.fa_fwd_ex(d["q"], d["k"], d["v"], **kw)
            b = fa.fa_fwd_ex(d["q"], d["k"], d["v"], window_left=big, window_right=big, **kw)
            torch.cuda.synchronize()
            assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), (causal, align)

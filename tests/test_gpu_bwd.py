"""GPU parity of the backward by recomputation (fa_bwd) against the float64
oracle ([GS] section 7; [VW] Step 8).

The GPU backward consumes the GPU forward's O and lse, so the oracle is given
those same arrays (``o=``, ``lse=``): both sides then rebuild the same
probabilities, and the comparison isolates the backward.  A second check runs
the oracle end to end (its own forward) at the forward's tolerance added in.

Tolerances, relative to the largest reference magnitude of each gradient
(a gradient is a sum of many signed terms, so an absolute bound would depend
on the shape), or to the size of one term, scale * |g| * |v| * max(|q|, |k|),
where a gradient cancels to zero:

* fp32 inputs: 2e-5.  Every product and sum is fp32 (relative rounding
  6e-8 per operation); a sum over n terms carries about sqrt(n) * 6e-8 of its
  largest terms, and the exponential adds about 1e-7 per probability: well
  under 1e-5 for n <= 4096.
* bf16 inputs: 2e-2.  P and D are rounded to bf16 (2^-9 relative) before
  they multiply G, Q or K; the errors of independent terms add in quadrature,
  so each gradient carries a few times 2^-9 = 2e-3 of its largest entries.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import bwd_every_head, f64, say, scale32

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
TOL = {torch.float32: 2e-5, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_05_amd as fa

    fa.lib()
    return torch.device("cuda:0")


def run_case(inp, g, dev):
    import online_softmax_05_amd as fa

    d = workloads.to_device(inp, dev)
    gd = g.to(dev)
    o, lse = fa.fa_fwd(d["q"], d["k"], d["v"], bias=d.get("bias"), k_len=d.get("k_len"), scale=inp["scale"],
                       causal=inp["causal"])
    dq, dk, dv = fa.fa_bwd(d["q"], d["k"], d["v"], o, gd, lse, bias=d.get("bias"), k_len=d.get("k_len"),
                           scale=inp["scale"], causal=inp["causal"])
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def oracle_bwd(inp, g, o=None, lse=None):
    k_len = None if inp.get("k_len") is None else inp["k_len"].cpu().numpy()
    return oracle.attention_bwd_ref(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(g), scale=scale32(inp["scale"]),
                                    causal=inp["causal"], k_len=k_len, bias=f64(inp.get("bias")),
                                    o=None if o is None else f64(o), lse=None if lse is None else f64(lse))


def term_size(inp, g):
    """Size of one term of the gradient sums, scale * |g| * |v| * max(|q|, |k|):
    the magnitude rounding errors are relative to when a gradient cancels to
    (near) zero, e.g. a row that sees a single key."""
    mx = lambda t: float(t.abs().max()) if t.numel() else 0.0  # noqa: E731
    return abs(scale32(inp["scale"])) * mx(g.float()) * mx(inp["v"].float()) * max(mx(inp["q"].float()),
                                                                                mx(inp["k"].float()))


def rel_err(got, ref, floor=1e-30):
    got = f64(got)
    assert not np.isnan(got).any(), "NaN in gradient"
    if not ref.size:
        return 0.0
    return float(np.max(np.abs(got - ref))) / max(float(np.max(np.abs(ref))), floor)


def check(inp, g, dev, what, tol_extra=0.0):
    dtype = inp["q"].dtype
    say(f"bwd {what}: q {tuple(inp['q'].shape)} k {tuple(inp['k'].shape)} v {tuple(inp['v'].shape)} {dtype}")
    o, lse, dq, dk, dv = run_case(inp, g, dev)
    ref = oracle_bwd(inp, g, o=o, lse=lse)
    tol = TOL[dtype] + tol_extra
    floor = term_size(inp, g)
    errs = [rel_err(x, r, floor) for x, r in zip((dq, dk, dv), ref)]
    say(f"bwd {what}: rel err dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e} (tol {tol:.0e})")
    for name, e in zip(("dQ", "dK", "dV"), errs):
        assert e <= tol, f"{what}: {name} relative error {e:.3e} > {tol}"
    return o, lse, (dq, dk, dv), ref


CASES = [
    # (B, H, Nq, Nk, dk, dv, causal, bias, k_len)
    (1, 1, 64, 64, 64, 64, False, False, None),
    (2, 2, 130, 97, 64, 64, True, False, None),        # Nq > Nk: empty top rows
    (2, 3, 77, 200, 128, 128, True, True, [200, 31]),  # ragged tails, bias, key lengths
    (1, 2, 48, 48, 40, 24, True, False, None),         # head dims off the fast sizes
    (2, 1, 33, 65, 128, 64, False, True, [0, 50]),     # an all-empty sequence
    (1, 1, 1, 1, 16, 8, False, False, None),
    (1, 1, 5, 300, 32, 96, True, False, "random"),
    # bf16: several 256-row dQ and 128-key dK/dV work-groups, both axes ragged
    (2, 2, 600, 700, 128, 128, True, False, "random"),
    (1, 3, 513, 390, 64, 128, False, False, [389]),   # one row past two dQ work-groups; keys end mid-group
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_bwd_parity(dev, case, dt):
    B, H, Nq, Nk, dk, dv, causal, bias, k_len = CASES[case]
    inp = workloads.seeded_case(300 + case, B, H, Nq, Nk, dk, dv, DT[dt], causal=causal, bias=bias, k_len=k_len)
    g = workloads.seeded_upstream(300 + case, B, H, Nq, dv, DT[dt])
    check(inp, g, dev, f"case {case} {dt}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_bwd_end_to_end(dev, dt):
    """Forward and backward on the GPU against the oracle's own forward and
    backward: the forward's rounding of O and lse enters as well."""
    inp = workloads.seeded_case(320, 2, 2, 150, 150, 64, 64, DT[dt], causal=True, bias=True, k_len=[150, 90])
    g = workloads.seeded_upstream(320, 2, 2, 150, 64, DT[dt])
    o, lse, grads, _ = check(inp, g, dev, f"end-to-end {dt}")
    ref = oracle_bwd(inp, g)
    tol = {torch.float32: 1e-4, torch.bfloat16: 3e-2}[DT[dt]]
    for name, x, r in zip(("dQ", "dK", "dV"), grads, ref):
        e = rel_err(x, r, term_size(inp, g))
        say(f"end-to-end {dt} {name}: rel err {e:.2e} (tol {tol:.0e})")
        assert e <= tol


def test_bwd_empty_rows_and_keys(dev):
    """Rows with no allowed key have dQ = 0 exactly; keys no row can see get
    dK = dV = 0 exactly."""
    inp = workloads.seeded_case(330, 2, 1, 40, 24, 32, 32, torch.float32, causal=True, k_len=[24, 10])
    g = workloads.seeded_upstream(330, 2, 1, 40, 32, torch.float32)
    o, lse, dq, dk, dv = run_case(inp, g, dev)
    dq, dk, dv = f64(dq), f64(dk), f64(dv)
    assert np.all(dq[:, :, :16] == 0.0)       # rows i < Nq - Nk see no key
    assert np.all(dk[1, :, 10:] == 0.0) and np.all(dv[1, :, 10:] == 0.0)


def test_bwd_deterministic(dev):
    """No atomics: two runs give bitwise identical gradients."""
    inp = workloads.seeded_case(340, 2, 2, 200, 180, 64, 64, torch.bfloat16, causal=True, bias=True)
    g = workloads.seeded_upstream(340, 2, 2, 200, 64, torch.bfloat16)
    a = run_case(inp, g, dev)[2:]
    b = run_case(inp, g, dev)[2:]
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_full_size_every_head(dev):
    """The benchmark's backward workload (causal bf16 4x32x4096^2, d = 128),
    in the launch configuration the benchmark times: every element of dQ, dK
    and dV of all 128 (batch, head) pairs against the oracle, which rebuilds
    P from the GPU forward's O and lse."""
    import online_softmax_05_amd as fa

    say("bwd full size: drawing the backward workload")
    inp = workloads.backward(dev)
    o, lse = fa.fa_fwd(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True)
    grads = fa.fa_bwd(inp["q"], inp["k"], inp["v"], o, inp["g"], lse, scale=inp["scale"], causal=True)
    torch.cuda.synchronize()
    bwd_every_head(inp["q"], inp["k"], inp["v"], inp["g"], o, lse, grads, scale=inp["scale"], causal=True,
                   tol=TOL[torch.bfloat16], what="bwd full size", floor=True)

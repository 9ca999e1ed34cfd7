"""Seeded random sweep of fa_fwd_ex and fa_bwd_ex against the float64 oracle:
alignment, left/right windows, dropout, bias, key lengths, head dims, tile
widths and dtypes drawn together, so that combinations the targeted tests do
not list are exercised too ([GS] section 6 masks and dropout).

Bounds as in the targeted tests: forward O within the dtype's bound times
r = 256/keep (lse undropped, unscaled bound), empty rows exact; gradients
within 2e-5 (fp32) / 2e-2 (bf16) of the largest reference entry or of r times
one term's size.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import TOL, f64, oracle_full, say, scale32

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
BWD_TOL = {torch.float32: 2e-5, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_05_amd as fa

    fa.lib()
    return torch.device("cuda:0")


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    dims = [(128, 128), (64, 64), (128, 64), (64, 128), (32, 48), (96, 128), (8, 8)]
    out = []
    for i in range(n):
        dk, dv = dims[int(rng.integers(0, len(dims)))]
        nq = int(rng.choice([1, 17, 64, 100, 129, 200, 257]))
        nk = int(rng.choice([1, 33, 64, 97, 128, 190, 300]))
        out.append(dict(
            i=i, B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), nq=nq, nk=nk, dk=dk, dv=dv,
            dt=["f32", "bf16"][int(rng.integers(0, 2))], causal=bool(rng.integers(0, 2)),
            align=["bottom_right", "top_left"][int(rng.integers(0, 2))],
            wl=[None, None, 0, 5, 40, 150][int(rng.integers(0, 6))],
            wr=[None, None, None, 0, 7, 60][int(rng.integers(0, 6))],
            keep=[256, 256, 230, 128, 40][int(rng.integers(0, 5))],
            bias=bool(rng.integers(0, 2)), kl=[None, "random"][int(rng.integers(0, 2))],
            bn=[0, 32, 64, 128][int(rng.integers(0, 4))], seed=int(rng.integers(0, 2**63))))
    return out


def _inputs(c):
    inp = workloads.seeded_case(9000 + c["i"], c["B"], c["H"], c["nq"], c["nk"], c["dk"], c["dv"], DT[c["dt"]],
                                causal=c["causal"], bias=c["bias"], k_len=c["kl"])
    inp.update(align=c["align"], window_left=c["wl"], window_right=c["wr"],
               dropout=None if c["keep"] == 256 else (c["keep"], c["seed"]))
    return inp


def _run_fwd(inp, c, dev):
    import online_softmax_05_amd as fa

    d = workloads.to_device(inp, dev)
    o, lse = fa.fa_fwd_ex(d["q"], d["k"], d["v"], bias=d.get("bias"), k_len=d.get("k_len"), scale=inp["scale"],
                          causal=c["causal"], align=c["align"], window_left=c["wl"], window_right=c["wr"],
                          keep_256=c["keep"], seed=c["seed"], block_n=c["bn"])
    torch.cuda.synchronize()
    return d, o, lse


FWD = _cases(40, 2026)


@pytest.mark.parametrize("c", FWD, ids=lambda c: f"f{c['i']}")
def test_fwd_ex_sweep(dev, c):
    inp = _inputs(c)
    say(f"fwd_ex sweep {c}")
    _, o, lse = _run_fwd(inp, c, dev)
    o_ref, lse_ref = oracle_full(inp)
    r = 256.0 / c["keep"]
    tol = TOL[DT[c["dt"]]]
    og, lg = f64(o), f64(lse)
    assert not np.isnan(og).any() and not np.isnan(lg).any()
    emp = np.isneginf(lse_ref)
    assert np.all(og[emp] == 0.0) and np.all(np.isneginf(lg[emp])), "empty rows"
    ne = ~emp
    if ne.any():
        e_o = float(np.max(np.abs(og[ne] - o_ref[ne])))
        e_l = float(np.max(np.abs(lg[ne] - lse_ref[ne])))
        say(f"  max|do| {e_o:.2e} (tol {tol['o'] * r:.1e}) max|dlse| {e_l:.2e}")
        assert e_o <= tol["o"] * r and e_l <= tol["lse"], (e_o, e_l)


def _fast_cases(n, seed):
    """Cases the fast bf16 kernel takes (head dims 64/128, default tile
    width), several query tiles of 128 rows and ragged lengths, so that
    masked edge tiles, tiles that one wave sees whole while another does not,
    and unmasked runs all occur."""
    rng = np.random.default_rng(seed)
    dims = [(128, 128), (64, 64), (128, 64), (64, 128)]
    out = []
    for i in range(n):
        dk, dv = dims[int(rng.integers(0, len(dims)))]
        out.append(dict(
            i=100 + i, B=1, H=int(rng.integers(1, 3)), nq=int(rng.choice([300, 511, 700, 1000])),
            nk=int(rng.choice([256, 513, 800, 1000])), dk=dk, dv=dv, dt="bf16", causal=bool(rng.integers(0, 2)),
            align=["bottom_right", "top_left"][int(rng.integers(0, 2))],
            wl=[None, None, 31, 100, 257][int(rng.integers(0, 5))],
            wr=[None, None, None, 0, 33][int(rng.integers(0, 5))],
            keep=[256, 256, 230][int(rng.integers(0, 3))],
            bias=bool(rng.integers(0, 2)), kl=[None, "random"][int(rng.integers(0, 2))],
            bn=[0, 64][int(rng.integers(0, 2))], seed=int(rng.integers(0, 2**63))))
    return out


FWD_FAST = _fast_cases(16, 77)


@pytest.mark.parametrize("c", FWD_FAST, ids=lambda c: f"fast{c['i']}")
def test_fwd_ex_sweep_fast_kernel(dev, c):
    test_fwd_ex_sweep(dev, c)


BWD = _cases(24, 4052)


@pytest.mark.parametrize("c", BWD, ids=lambda c: f"b{c['i']}")
def test_bwd_ex_sweep(dev, c):
    import online_softmax_05_amd as fa

    dtype = DT[c["dt"]]
    inp = _inputs(c)
    g = workloads.seeded_upstream(9500 + c["i"], c["B"], c["H"], c["nq"], c["dv"], dtype)
    say(f"bwd_ex sweep {c}")
    d, o, lse = _run_fwd(inp, c, dev)
    grads = fa.fa_bwd_ex(d["q"], d["k"], d["v"], o, g.to(dev), lse, bias=d.get("bias"), k_len=d.get("k_len"),
                         scale=inp["scale"], causal=c["causal"], align=c["align"], window_left=c["wl"],
                         window_right=c["wr"], keep_256=c["keep"], seed=c["seed"])
    torch.cuda.synchronize()
    k_len = None if inp.get("k_len") is None else inp["k_len"].cpu().numpy()
    ref = oracle.attention_bwd_ref(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(g), scale=scale32(inp["scale"]),
                                   causal=c["causal"], k_len=k_len, bias=f64(inp.get("bias")), o=f64(o), lse=f64(lse),
                                   align=c["align"], window=(c["wl"], c["wr"]), dropout=inp.get("dropout"))
    mx = lambda t: float(t.abs().max()) if t.numel() else 0.0  # noqa: E731
    term = (256.0 / c["keep"]) * abs(scale32(inp["scale"])) * mx(g.float()) * mx(inp["v"].float()) * max(
        mx(inp["q"].float()), mx(inp["k"].float()))
    for name, x, rf in zip(("dQ", "dK", "dV"), grads, ref):
        got = f64(x)
        assert not np.isnan(got).any(), name
        e = float(np.max(np.abs(got - rf))) / max(float(np.max(np.abs(rf))) if rf.size else 0.0, term, 1e-30)
        say(f"  {name} rel err {e:.2e}")
        assert e <= BWD_TOL[dtype], (name, e)

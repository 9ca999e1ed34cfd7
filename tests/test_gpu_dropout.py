"""GPU parity of dropout (fa_fwd_ex / fa_bwd_ex with keep_256 < 256) and of the
backward under the mask variants, against the float64 oracle on the same
seeded inputs ([GS] section 6: the backward replays the forward's random
mask and scaling).

* The keep/drop decision is an integer decision from the same generator on
  both sides, so it must agree bit for bit: with V the identity (Nk = dv), row
  i of O is r z_ij p_ij, and O_ij = 0 exactly where the element was dropped.
* Outputs: the plain forward tolerances (fp32 1e-5, bf16 O 2e-2 / lse 1e-3)
  times r = 256/keep for O -- the dropped output is r times a partial sum of
  the same terms, so its rounding error scales with r; lse is undropped.
* Gradients: the backward tolerances (fp32 2e-5, bf16 2e-2) relative to the
  largest reference entry or to one term's size, the term size times r.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import bwd_every_head, TOL, compare, compare_every_head, f64, oracle_full, say, scale32

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


def fwd(inp, dev, block_n=0):
    import online_softmax_05_amd as fa

    d = workloads.to_device(inp, dev)
    keep, seed = inp.get("dropout") or (256, 0)
    o, lse = fa.fa_fwd_ex(d["q"], d["k"], d["v"], bias=d.get("bias"), k_len=d.get("k_len"), scale=inp["scale"],
                          causal=inp["causal"], align=inp.get("align", "bottom_right"),
                          window_left=inp.get("window_left"), window_right=inp.get("window_right"), keep_256=keep,
                          seed=seed, block_n=block_n)
    torch.cuda.synchronize()
    return o, lse


def compare_dropped(o, lse, o_ref, lse_ref, dtype, keep, what):
    r = 256.0 / keep
    tol = dict(TOL[dtype])
    o64, l64 = f64(o), f64(lse)
    emp = np.isneginf(lse_ref)
    assert not np.isnan(o64).any() and not np.isnan(l64).any(), f"{what}: NaN"
    assert np.all(o64[emp] == 0.0) and np.all(np.isneginf(l64[emp])), f"{what}: empty rows"
    ne = ~emp
    err_o = float(np.max(np.abs(o64[ne] - o_ref[ne]))) if ne.any() else 0.0
    err_l = float(np.max(np.abs(l64[ne] - lse_ref[ne]))) if ne.any() else 0.0
    say(f"{what}: max|do| = {err_o:.3e} (tol {tol['o'] * r:.1e}), max|dlse| = {err_l:.3e} (tol {tol['lse']:.0e})")
    assert err_o <= tol["o"] * r, what
    assert err_l <= tol["lse"], what


# (B, H, Nq, Nk, dk, dv, causal, bias, k_len, align, wl, wr, keep)
FWD_CASES = [
    (1, 2, 200, 333, 64, 64, True, False, None, "bottom_right", None, None, 230),
    (2, 2, 300, 300, 128, 128, True, True, "random", "bottom_right", None, None, 128),
    (1, 3, 257, 190, 128, 64, True, False, None, "top_left", 100, None, 200),
    (2, 1, 129, 400, 96, 40, False, True, [400, 77], "bottom_right", 60, 20, 16),
    (1, 1, 70, 70, 32, 32, False, False, None, "bottom_right", None, None, 255),
]


def _fid(c):
    return f"{c[2]}x{c[3]}_d{c[4]}-{c[5]}_{'c' if c[6] else 'nc'}_{c[9]}_wl{c[10]}_keep{c[12]}"


@pytest.mark.parametrize("case", FWD_CASES, ids=_fid)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_dropout_forward(dev, case, dt):
    B, H, nq, nk, dk, dv, causal, bias, kl, align, wl, wr, keep = case
    inp = workloads.seeded_case(7000 + nq + nk, B, H, nq, nk, dk, dv, DT[dt], causal=causal, bias=bias, k_len=kl)
    inp.update(align=align, window_left=wl, window_right=wr, dropout=(keep, 0x5EED0000 + nq))
    o_ref, lse_ref = oracle_full(inp)
    for bn in (0, 32, 128):
        say(f"dropout fwd {_fid(case)} {dt} block_n={bn}")
        o, lse = fwd(inp, dev, block_n=bn)
        compare_dropped(o, lse, o_ref, lse_ref, DT[dt], keep, f"{_fid(case)} {dt} bn={bn}")


@pytest.mark.parametrize("dt,d,nq,nk,bn", [("f32", 64, 150, 64, 0), ("bf16", 64, 150, 64, 0),
                                          ("bf16", 128, 300, 128, 0), ("bf16", 128, 130, 128, 32),
                                          ("f32", 128, 70, 128, 128)])
def test_dropout_mask_bits(dev, dt, d, nq, nk, bn):
    """V = I makes O_ij = r z_ij p_ij: the set of dropped elements must equal
    the oracle's mask exactly (every p_ij > 0 here), and the kept fraction is
    about keep/256."""
    keep, seed = 180, 0x0123456789ABCDEF
    B, H = 2, 3
    g = torch.Generator().manual_seed(7100 + d + nq)
    q = (0.1 * torch.randn((B, H, nq, d), generator=g)).to(DT[dt])
    k = (0.1 * torch.randn((B, H, nk, d), generator=g)).to(DT[dt])
    v = torch.eye(nk, dtype=torch.float32)[None, None].repeat(B, H, 1, 1).to(DT[dt])
    inp = dict(q=q, k=k, v=v, bias=None, k_len=None, causal=False, scale=1.0 / 8, dropout=(keep, seed))
    say(f"dropout mask bits {dt} d={d} {nq}x{nk} block_n={bn}")
    o, _ = fwd(inp, dev, block_n=bn)
    got_kept = f64(o) != 0.0
    for b in range(B):
        for h in range(H):
            want = oracle.keep_mask(b * H + h, np.arange(nq), nk, seed, keep)
            bad = np.argwhere(got_kept[b, h] != want)
            assert bad.size == 0, f"mask differs at (b={b}, h={h}) rows/keys {bad[:5].tolist()}"
    frac = float(got_kept.mean())
    sigma = (keep / 256 * (1 - keep / 256) / got_kept.size) ** 0.5
    assert abs(frac - keep / 256) < 6 * sigma, frac


def test_dropout_reproducible_and_seeded(dev):
    import online_softmax_05_amd as fa

    inp = workloads.seeded_case(7200, 2, 4, 256, 256, 128, 128, torch.bfloat16, causal=True)
    d = workloads.to_device(inp, dev)
    say("dropout reproducibility")
    a = fa.fa_fwd_ex(d["q"], d["k"], d["v"], causal=True, dropout_p=0.1, seed=42)[0].clone()
    b = fa.fa_fwd_ex(d["q"], d["k"], d["v"], causal=True, dropout_p=0.1, seed=42)[0].clone()
    c = fa.fa_fwd_ex(d["q"], d["k"], d["v"], causal=True, dropout_p=0.1, seed=43)[0].clone()
    n = fa.fa_fwd_ex(d["q"], d["k"], d["v"], causal=True, dropout_p=0.0, seed=42)[0].clone()
    p = fa.fa_fwd(d["q"], d["k"], d["v"], causal=True)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert torch.equal(n, p), "keep 256 must be fa_fwd bit for bit"


def test_dropout_full_size_every_row(dev):
    """The prefill shape (4x32x4096, d128, bf16, causal) with dropout p = 0.1
    (keep 230): every row of every head against the oracle (same mask)."""
    import online_softmax_05_amd as fa

    inp = workloads.prefill(dev)
    keep, seed = 230, 2024
    say("dropout full size 4x32x4096 d128 bf16 keep 230")
    o, lse = fa.fa_fwd_ex(inp["q"], inp["k"], inp["v"], causal=True, keep_256=keep, seed=seed, scale=inp["scale"])
    torch.cuda.synchronize()
    compare_every_head(o, lse, inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True, dropout=(keep, seed),
                       o_tol_factor=256.0 / keep, what="full-size dropout")


# ---------------------------------------------------------------------------
# backward with dropout and the mask variants
# ---------------------------------------------------------------------------

def _bwd_run(inp, g, dev):
    import online_softmax_05_amd as fa

    d = workloads.to_device(inp, dev)
    keep, seed = inp.get("dropout") or (256, 0)
    kw = dict(bias=d.get("bias"), k_len=d.get("k_len"), scale=inp["scale"], causal=inp["causal"],
              align=inp.get("align", "bottom_right"), window_left=inp.get("window_left"),
              window_right=inp.get("window_right"), keep_256=keep, seed=seed)
    o, lse = fa.fa_fwd_ex(d["q"], d["k"], d["v"], **kw)
    grads = fa.fa_bwd_ex(d["q"], d["k"], d["v"], o, g.to(dev), lse, **kw)
    torch.cuda.synchronize()
    return o, lse, grads


def _bwd_oracle(inp, g, o, lse):
    k_len = None if inp.get("k_len") is None else inp["k_len"].cpu().numpy()
    return oracle.attention_bwd_ref(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(g), scale=scale32(inp["scale"]),
                                    causal=inp["causal"], k_len=k_len, bias=f64(inp.get("bias")), o=f64(o),
                                    lse=f64(lse), align=inp.get("align", "bottom_right"),
                                    window=(inp.get("window_left"), inp.get("window_right")),
                                    dropout=inp.get("dropout"))


def _term(inp, g, keep):
    mx = lambda t: float(t.abs().max()) if t.numel() else 0.0  # noqa: E731
    return (256.0 / keep) * abs(scale32(inp["scale"])) * mx(g.float()) * mx(inp["v"].float()) * max(
        mx(inp["q"].float()), mx(inp["k"].float()))


# (B, H, Nq, Nk, dk, dv, causal, bias, k_len, align, wl, wr, keep)
BWD_CASES = [
    (1, 2, 130, 200, 64, 64, True, False, None, "bottom_right", None, None, 230),
    (2, 2, 200, 200, 128, 128, True, True, "random", "bottom_right", 70, None, 256),
    (1, 2, 190, 130, 128, 128, True, False, None, "top_left", None, None, 256),
    (2, 1, 150, 260, 128, 64, True, False, [260, 90], "top_left", 40, None, 200),
    (1, 2, 96, 160, 64, 128, False, True, None, "bottom_right", 30, 25, 128),
    (1, 1, 77, 100, 40, 24, True, False, None, "bottom_right", 20, None, 180),   # general kernels
    # no bias, no dropout, several 64-row query tiles: the dK/dV kernel's
    # unmasked run of query tiles lies between masked ones
    (1, 2, 700, 900, 128, 128, True, False, None, "bottom_right", 200, None, 256),
    (2, 2, 640, 640, 128, 128, True, False, [640, 333], "top_left", 150, None, 256),
    (1, 2, 520, 800, 64, 64, False, False, None, "bottom_right", 130, 70, 256),
    (1, 1, 1000, 1000, 128, 128, True, False, None, "bottom_right", None, None, 256),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=_fid)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_masks_and_dropout(dev, case, dt):
    B, H, nq, nk, dk, dv, causal, bias, kl, align, wl, wr, keep = case
    dtype = DT[dt]
    inp = workloads.seeded_case(7300 + nq + nk, B, H, nq, nk, dk, dv, dtype, causal=causal, bias=bias, k_len=kl)
    inp.update(align=align, window_left=wl, window_right=wr, dropout=None if keep == 256 else (keep, 991 + nq))
    g = workloads.seeded_upstream(7300 + nq, B, H, nq, dv, dtype)
    say(f"bwd masks/dropout {_fid(case)} {dt}")
    o, lse, grads = _bwd_run(inp, g, dev)
    ref = _bwd_oracle(inp, g, o, lse)
    floor = _term(inp, g, keep)
    errs = []
    for x, r in zip(grads, ref):
        got = f64(x)
        assert not np.isnan(got).any()
        errs.append(float(np.max(np.abs(got - r))) / max(float(np.max(np.abs(r))) if r.size else 0.0, floor))
    say(f"bwd {_fid(case)} {dt}: rel err dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}")
    for name, e in zip(("dQ", "dK", "dV"), errs):
        assert e <= BWD_TOL[dtype], f"{name} relative error {e:.3e}"


def test_backward_ex_defaults_match_fa_bwd(dev):
    import online_softmax_05_amd as fa

    inp = workloads.seeded_case(7400, 2, 2, 200, 200, 128, 128, torch.bfloat16, causal=True)
    g = workloads.seeded_upstream(7400, 2, 2, 200, 128, torch.bfloat16).to(dev)
    d = workloads.to_device(inp, dev)
    say("fa_bwd_ex defaults vs fa_bwd")
    o, lse = fa.fa_fwd(d["q"], d["k"], d["v"], causal=True)
    a = fa.fa_bwd(d["q"], d["k"], d["v"], o, g, lse, causal=True)
    b = fa.fa_bwd_ex(d["q"], d["k"], d["v"], o, g, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_dropout_full_size_every_head(dev):
    """The prefill shape with dropout p = 0.1 through fa_fwd_ex and fa_bwd_ex:
    every element of dQ, dK and dV of all 128 heads against the oracle (given
    the GPU's O and lse)."""
    import online_softmax_05_amd as fa

    inp = workloads.backward(dev)
    keep, seed = 230, 77
    say("bwd dropout full size 4x32x4096 d128 bf16 keep 230")
    o, lse = fa.fa_fwd_ex(inp["q"], inp["k"], inp["v"], causal=True, keep_256=keep, seed=seed, scale=inp["scale"])
    grads = fa.fa_bwd_ex(inp["q"], inp["k"], inp["v"], o, inp["g"], lse, causal=True, keep_256=keep, seed=seed,
                         scale=inp["scale"])
    torch.cuda.synchronize()
    bwd_every_head(inp["q"], inp["k"], inp["v"], inp["g"], o, lse, grads, scale=inp["scale"], causal=True,
                   tol=BWD_TOL[torch.bfloat16], what="full-size dropout bwd", dropout=(keep, seed))

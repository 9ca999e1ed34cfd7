"""Helpers for the GPU parity tests: run the oracle on the exact inputs the
GPU receives and compare element by element."""

import sys

import numpy as np
import torch

import oracle

# tolerances (max abs, over all elements, after upcasting to float64)
TOL = {
    torch.float32: dict(o=1e-5, lse=1e-5),
    torch.bfloat16: dict(o=2e-2, lse=1e-3),
}


def say(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def f64(t):
    return None if t is None else t.detach().to("cpu").double().numpy()


def scale32(scale):
    """The float32 scale the GPU receives, as a float64."""
    return float(np.float32(scale))


def oracle_full(inp):
    """Dense oracle over a whole (small) workload dict of CPU or device tensors."""
    k_len = None if inp.get("k_len") is None else inp["k_len"].cpu().numpy()
    return oracle.attention_ref(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale=scale32(inp["scale"]),
                                causal=inp["causal"], k_len=k_len, bias=f64(inp.get("bias")),
                                align=inp.get("align", "bottom_right"),
                                window=(inp.get("window_left"), inp.get("window_right")),
                                dropout=inp.get("dropout"))


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what, empty=None, logit_scale=1.0):
    """Max-abs comparison at the dtype's tolerance; rows with lse_ref = -inf
    (empty rows) must match exactly: o = 0 and lse = -inf.

    ``logit_scale`` >= 1 widens the fp32 bounds for logits larger than the
    standard scaling gives: fp32 represents a logit of size |s| only to about
    |s| * 6e-8, so both fp32 bounds grow in proportion."""
    tol = dict(TOL[dtype])
    if dtype == torch.float32 and logit_scale > 1.0:
        tol = dict(o=tol["o"] * logit_scale, lse=tol["lse"] * logit_scale)
    o = f64(o_gpu)
    lse = f64(lse_gpu)
    assert o.shape == o_ref.shape, (what, o.shape, o_ref.shape)
    assert not np.isnan(o).any(), f"{what}: NaN in o"
    assert not np.isnan(lse).any(), f"{what}: NaN in lse"
    emp = np.isneginf(lse_ref) if empty is None else empty
    if emp.any():
        assert np.all(o[emp] == 0.0), f"{what}: empty rows must give o = 0"
        assert np.all(np.isneginf(lse[emp])), f"{what}: empty rows must give lse = -inf"
    ne = ~emp
    err_o = float(np.max(np.abs(o[ne] - o_ref[ne]))) if ne.any() else 0.0
    err_l = float(np.max(np.abs(lse[ne] - lse_ref[ne]))) if ne.any() else 0.0
    say(f"{what}: max|do| = {err_o:.3e} (tol {tol['o']:.0e}), max|dlse| = {err_l:.3e} (tol {tol['lse']:.0e})")
    assert err_o <= tol["o"], f"{what}: max |o - o_ref| = {err_o:.3e} > {tol['o']}"
    assert err_l <= tol["lse"], f"{what}: max |lse - lse_ref| = {err_l:.3e} > {tol['lse']}"
    return err_o, err_l


def oracle_rows(q, k, v, rows, *, scale, causal, k_len=None, bias=None, align="bottom_right",
                window=(None, None), dropout=None):
    """Oracle on sampled rows of device tensors: rows is a list of (b, h, i).
    Only the needed slices are copied to the host.  Returns (o [n, dv], lse [n])."""
    B, H, Nq, _ = q.shape
    Nk, dv = k.shape[2], v.shape[3]
    o = np.zeros((len(rows), dv))
    lse = np.zeros(len(rows))
    by_head = {}
    for n, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((n, i))
    kl = None if k_len is None else k_len.cpu().numpy()
    for (b, h), items in by_head.items():
        idx = [i for _, i in items]
        qi = f64(q[b, h, idx])
        kk, vv = f64(k[b, h]), f64(v[b, h])
        bb = None if bias is None else f64(bias[b, h, idx])
        ob, lb = oracle.attention_head(qi, kk, vv, scale=scale32(scale), nq=Nq, causal=causal,
                                       k_len_b=None if kl is None else int(kl[b]), bias=bb, row_ids=idx,
                                       align=align, window=window, dropout=dropout, bh=b * H + h)
        for j, (n, _) in enumerate(items):
            o[n] = ob[j]
            lse[n] = lb[j]
    return o, lse

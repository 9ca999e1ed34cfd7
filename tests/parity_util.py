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


def _blas_limit(n):
    try:
        from threadpoolctl import threadpool_limits

        return threadpool_limits(limits=n, user_api="blas")
    except Exception:  # noqa: BLE001
        import contextlib

        return contextlib.nullcontext()


def compare_every_head(o_gpu, lse_gpu, q, k, v, *, scale, causal, k_len_host=None, nq_rows=None, what,
                       dtype=torch.bfloat16, workers=8, row_block=2048, window=(None, None), dropout=None,
                       o_tol_factor=1.0):
    """Every output element of a full-size launch against the oracle.

    o_gpu [B,H,Nq,dv], lse_gpu [B,H,Nq] (device or host); q, k, v the exact
    inputs (device or host).  The oracle runs head by head (complete rows of
    S in blocks of ``row_block`` rows), ``workers`` heads at a time on host
    threads (numpy releases the interpreter lock inside its large array
    operations; BLAS is limited to one thread per worker).  With
    ``k_len_host`` the keys of sequence b are truncated to k_len[b] before the
    call, for the decode entry points whose causal alignment is against the
    sequence's own length.  Max-abs errors over all elements at the dtype's
    tolerance (the o bound times ``o_tol_factor``: the dropout tests' 256/keep);
    ``window`` and ``dropout`` as for the oracle; rows with lse_ref = -inf
    must be exactly o = 0, lse = -inf.
    Returns (max |do|, max |dlse|, number of rows compared)."""
    import concurrent.futures

    qh = q.detach().to("cpu")
    kh = k.detach().to("cpu")
    vh = v.detach().to("cpu")
    og = o_gpu.detach().to("cpu").double().numpy()
    lg = lse_gpu.detach().to("cpu").double().numpy()
    B, H, Nq = qh.shape[0], qh.shape[1], qh.shape[2]
    tol = dict(TOL[dtype])
    tol["o"] *= o_tol_factor
    sc = scale32(scale)

    def head(bh):
        b, h = divmod(bh, H)
        n = kh.shape[2] if k_len_host is None else int(k_len_host[b])
        qq = qh[b, h].double().numpy()
        kk = kh[b, h, :n].double().numpy()
        vv = vh[b, h, :n].double().numpy()
        e_o = e_l = 0.0
        for r0 in range(0, Nq, row_block):
            r1 = min(Nq, r0 + row_block)
            o_ref, l_ref = oracle.attention_head(qq[r0:r1], kk, vv, scale=sc, nq=Nq, causal=causal,
                                                 row_ids=np.arange(r0, r1), window=window, dropout=dropout,
                                                 bh=bh)
            o, lse = og[b, h, r0:r1], lg[b, h, r0:r1]
            emp = np.isneginf(l_ref)
            if emp.any():
                assert np.all(o[emp] == 0.0) and np.all(np.isneginf(lse[emp])), \
                    f"{what}: empty rows of ({b}, {h}) must give o = 0, lse = -inf"
            ne = ~emp
            assert not np.isnan(o).any() and not np.isnan(lse).any(), f"{what}: NaN in ({b}, {h})"
            if ne.any():
                e_o = max(e_o, float(np.max(np.abs(o[ne] - o_ref[ne]))))
                e_l = max(e_l, float(np.max(np.abs(lse[ne] - l_ref[ne]))))
        return e_o, e_l

    err_o = err_l = 0.0
    with _blas_limit(1), concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for e_o, e_l in ex.map(head, range(B * H)):
            err_o, err_l = max(err_o, e_o), max(err_l, e_l)
    say(f"{what}: every element of {B * H} heads x {Nq} rows: max|do| = {err_o:.3e} (tol {tol['o']:.0e}), "
        f"max|dlse| = {err_l:.3e} (tol {tol['lse']:.0e})")
    assert err_o <= tol["o"], f"{what}: max |o - o_ref| = {err_o:.3e} > {tol['o']}"
    assert err_l <= tol["lse"], f"{what}: max |lse - lse_ref| = {err_l:.3e} > {tol['lse']}"
    return err_o, err_l, B * H * Nq


def bwd_every_head(q, k, v, g, o, lse, grads, *, scale, causal, tol, what, dropout=None, floor=False,
                   workers=8):
    """Every element of dQ, dK and dV of a full-size backward against the oracle.

    The oracle rebuilds P of each (batch, head) from the GPU forward's o and
    lse (the backward's own inputs) and returns the head's three gradients;
    heads run ``workers`` at a time on host threads with one BLAS thread each.
    A head's error in a gradient is max |got - ref| over the head, relative
    to max |ref| over the head (or, with ``floor``, to at least one term of
    the gradient sums, scale * |g| * |v| * max(|q|, |k|), for gradients that
    cancel to near zero).  Asserts the worst head of each gradient against
    ``tol`` and returns the three worst relative errors."""
    import concurrent.futures

    host = [t.detach().to("cpu") for t in (q, k, v, g, o, lse, *grads)]
    qh, kh, vh, gh, oh, lh, dqh, dkh, dvh = host
    B, H, Nq = qh.shape[0], qh.shape[1], qh.shape[2]
    sc = scale32(scale)

    def head(bh):
        b, h = divmod(bh, H)
        qq, kk, vv, gg = (t[b, h].double().numpy() for t in (qh, kh, vh, gh))
        ref = oracle.attention_bwd_head(qq, kk, vv, gg, scale=sc, nq=Nq, causal=causal, o=oh[b, h].double().numpy(),
                                        lse=lh[b, h].double().numpy(), dropout=dropout, bh=bh)
        fl = abs(sc) * np.abs(gg).max() * np.abs(vv).max() * max(np.abs(qq).max(), np.abs(kk).max()) if floor else 0.0
        errs = []
        for got_t, r in zip((dqh, dkh, dvh), ref):
            got = got_t[b, h].double().numpy()
            assert not np.isnan(got).any(), f"{what}: NaN in a gradient of ({b}, {h})"
            errs.append(float(np.max(np.abs(got - r))) / max(float(np.max(np.abs(r))), fl, 1e-30))
        return errs

    worst = [0.0, 0.0, 0.0]
    with _blas_limit(1), concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for i, errs in enumerate(ex.map(head, range(B * H))):
            worst = [max(a, e) for a, e in zip(worst, errs)]
            if (i + 1) % 16 == 0 or i + 1 == B * H:
                say(f"{what}: {i + 1} of {B * H} heads, worst rel err dQ {worst[0]:.2e} dK {worst[1]:.2e} "
                    f"dV {worst[2]:.2e} (tol {tol:.0e})")
    for name, e in zip(("dQ", "dK", "dV"), worst):
        assert e <= tol, f"{what}: {name} relative error {e:.3e} > {tol}"
    return worst

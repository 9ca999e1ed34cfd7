"""Float64 gradients of masked attention by recomputation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[GS] section 7 ("Why training need not save the full probability matrix";
also [VW] Step 8, "Backward pass: the recompute trade"): the forward pass keeps
only each row's output o_i and log-sum-exp L_i.  Given the original Q, K, V,
the fixed mask and the fixed bias, the probabilities are rebuilt from the
scores, and for an upstream gradient G (row g_i = dLoss/do_i):

    s_ij  = scale * (q_i . k_j) + b_ij                 on the allowed set J_i
    p_ij  = exp(s_ij - L_i)  on J_i, 0 elsewhere
    c_i   = g_i . o_i        (the softmax Jacobian's row reduction: the sum
                              sum_j p_ij (g_i . v_j) with sum and dot product
                              exchanged)
    D_ij  = p_ij (g_i . v_j - c_i)     gradient w.r.t. the scaled logit s_ij
    dV    = P^T G
    dQ    = scale * D K
    dK    = scale * D^T Q

The Q and K gradients carry the original scale ([GS] section 7).  The bias is
fixed (no gradient).  With dropout ([GS] section 6: the backward must replay
the forward's random mask and scaling) the forward used P~ = (Z o P) * r,
Z the kept elements and r = 256/keep_256 (``oracle.dropout``), so

    dV    = P~^T G
    D_ij  = p_ij (z_ij r (g_i . v_j) - c_i),   c_i = g_i . o_i

(c_i = sum_j p_ij z_ij r (g_i . v_j) = g_i . o_i still holds because o_i is
the dropped output); dQ and dK follow from D as above.  Readings where the
pages stop short:

* A row with no allowed key (empty J_i) has the convention o_i = 0 and
  lse_i = -inf ([GS] section 6).  [GS] section 7 says not to read that
  convention as the derivative of softmax on an empty set, and derives the
  gradients for non-empty rows only; the plainest reading that the rest
  supports is that an empty row contributes nothing to any gradient (its
  output does not depend on Q, K or V), so its p_ij and D_ij are zero and
  dQ_i = 0.
* ``o`` and ``lse`` default to the oracle's own forward values.  The GPU path
  receives the forward kernel's stored O and lse instead (that is the point
  of recomputation); callers may pass those here to reproduce exactly what
  the kernel consumes.

Inputs are converted to float64 exactly; ``scale`` is used as given.
"""

import numpy as np

from .dense import allowed_mask, attention_head
from .dropout import keep_mask, keep_scale


def attention_bwd_head(q, k, v, g, *, scale, nq, causal=False, k_len_b=None,
                       bias=None, row_ids=None, o=None, lse=None, align="bottom_right",
                       window=(None, None), dropout=None, bh=0):
    """Gradients for selected query rows of one (batch, head).

    q: [R, dk] rows ``row_ids`` (default 0..R-1) of a query axis of length
    ``nq``; k: [Nk, dk]; v: [Nk, dv]; g: [R, dv] upstream gradient of those
    rows' outputs; bias: [R, Nk] or None.  Returns (dq [R, dk], dk [Nk, dk],
    dv [Nk, dv]): dk and dv are the contributions of these rows only (the
    full gradients when all rows of the head are passed).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    rows = q.shape[0]
    nk = k.shape[0]
    if row_ids is None:
        row_ids = np.arange(rows)
    row_ids = np.asarray(row_ids, dtype=np.int64)

    if o is None or lse is None:
        o_f, lse_f = attention_head(q, k, v, scale=scale, nq=nq, causal=causal,
                                    k_len_b=k_len_b, bias=bias, row_ids=row_ids, align=align,
                                    window=window, dropout=dropout, bh=bh)
        o = o_f if o is None else o
        lse = lse_f if lse is None else lse
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)

    ok = allowed_mask(row_ids, nq, nk, causal, k_len_b, align=align, window=window)
    nonempty = ok.any(axis=1) & np.isfinite(lse)
    s = (q @ k.T) * float(scale)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)
    lse_safe = np.where(nonempty, lse, 0.0)
    p = np.where(ok & nonempty[:, None], np.exp(np.where(ok, s, 0.0) - lse_safe[:, None]), 0.0)

    c = np.sum(g * o, axis=1)                      # c_i = g_i . o_i
    if dropout is None:
        zr = 1.0                                   # no dropout: z = 1, r = 1
    else:
        keep_256, seed = dropout
        zr = np.where(keep_mask(bh, row_ids, nk, seed, keep_256), keep_scale(keep_256), 0.0)
    d = p * (zr * (g @ v.T) - c[:, None])          # dLoss / ds_ij
    dv = (p * zr).T @ g
    dq = float(scale) * (d @ k)
    dk = float(scale) * (d.T @ q)
    return dq, dk, dv


def attention_bwd_ref(q, k, v, g, *, scale, causal=False, k_len=None, bias=None,
                      o=None, lse=None, align="bottom_right", window=(None, None), dropout=None):
    """Gradients over a whole batch: q [B,H,Nq,dk], k [B,H,Nk,dk],
    v [B,H,Nk,dv], g [B,H,Nq,dv]; optional k_len [B], bias [B,H,Nq,Nk], and
    the forward's o [B,H,Nq,dv] / lse [B,H,Nq] to use in place of the
    oracle's own; ``align``, ``window`` and ``dropout`` as for the forward.
    Returns (dq, dk, dv) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    bsz, heads, nq, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(bsz):
        klb = None if k_len is None else int(k_len[b])
        for h in range(heads):
            res = attention_bwd_head(
                q[b, h], k[b, h], v[b, h], g[b, h], scale=scale, nq=nq, causal=causal,
                k_len_b=klb, bias=None if bias is None else bias[b, h],
                o=None if o is None else o[b, h], lse=None if lse is None else lse[b, h],
                align=align, window=window, dropout=dropout, bh=b * heads + h)
            dq[b, h], dk[b, h], dv[b, h] = res
    return dq, dk, dv

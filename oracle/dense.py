"""Dense float64 definition of masked attention: S and P are materialised.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the operator itself, written out plainly ([GS] section 1; [VW] Step 1;
[OA] "Computing the Value Weighted Sum First"): for each query row i of one
(batch, head),

    s_ij  = scale * (q_i . k_j) + b_ij                       for j in J_i
    m_i   = max_{j in J_i} s_ij                              ([VW] Step 3)
    e_ij  = exp(s_ij - m_i) on J_i, 0 elsewhere
    l_i   = sum_j e_ij
    P_ij  = e_ij / l_i
    o_i   = sum_j P_ij v_j
    lse_i = m_i + ln l_i                                     ([GS] section 7)

and a row whose allowed set J_i is empty gets o_i = 0, lse_i = -inf, P_i = 0
([GS] section 6: the softmax of an empty set is undefined, so the output is a
stated convention).  The max subtraction does not change the result; it only
keeps every exponential <= 1 ([VW] Step 3).

The allowed set ([GS] sections 1 and 6) is the intersection of

* the key-length (padding) mask  j < clamp(k_len[b], 0, Nk), and
* the bottom-right causal mask   j <= i + Nk - Nq  (zero-based indices, the
  two sequences' ends aligned; rows with i + Nk - Nq < 0 are empty).

The causal offset uses the tensor extents Nq and Nk, not k_len: padding is a
separate key mask ([GS] section 6 treats it as its own mask).

Mask variants ([GS] section 6: top-left alignment as the alternative
convention; sliding windows need the same alignment audit).  Query row i sits
at key position pos_i = i + Nk - Nq (bottom-right, the default) or pos_i = i
(top-left); causal keeps j <= pos_i; a window (wl, wr) keeps
pos_i - wl <= j (wl given) and j <= pos_i + wr (wr given).  Reading: the
window is measured from the aligned position, exactly like the causal
limit, and combines with the other masks by intersection.

Inputs are converted to float64 exactly (bf16 and fp32 values are exactly
representable); ``scale`` is used as given -- callers pass the float32 value
the GPU receives.
"""

import numpy as np

from .dropout import keep_mask, keep_scale

_ROW_BLOCK = 2048  # rows of S materialised at once; every row is complete


def allowed_mask(row_ids, nq, nk, causal, k_len_b, align="bottom_right", window=(None, None)):
    """Boolean [len(row_ids), nk]: True where key j is visible to query row i.

    [GS] section 6: global zero-based positions, bottom-right alignment (or
    top-left), a key-length mask that may empty whole rows or whole tiles,
    and an optional window (wl, wr) around the aligned position.
    """
    row_ids = np.asarray(row_ids, dtype=np.int64).reshape(-1)
    j = np.arange(nk, dtype=np.int64)[None, :]
    limit = nk if k_len_b is None else min(max(int(k_len_b), 0), nk)
    ok = np.broadcast_to(j < limit, (row_ids.size, nk)).copy()
    if align not in ("bottom_right", "top_left"):
        raise ValueError(f"unknown alignment {align!r}")
    pos = row_ids[:, None] + ((nk - nq) if align == "bottom_right" else 0)
    if causal:
        ok &= j <= pos
    wl, wr = window
    if wl is not None:
        ok &= j >= pos - int(wl)
    if wr is not None:
        ok &= j <= pos + int(wr)
    return ok


def attention_head(q, k, v, *, scale, nq, causal=False, k_len_b=None,
                   bias=None, row_ids=None, return_p=False, align="bottom_right",
                   window=(None, None), dropout=None, bh=0):
    """Dense attention for selected query rows of one (batch, head).

    q: [R, dk] the query rows whose global indices are ``row_ids`` (default
    0..R-1) on a query axis of length ``nq``; k: [Nk, dk]; v: [Nk, dv];
    bias: [R, Nk] or None, added after scaling ([GS] section 1).
    dropout: None or (keep_256, seed): the probabilities are dropped with the
    counter-based mask of head ``bh`` = b*H + h and the kept ones scaled by
    256/keep_256 before the product with V; lse is the undropped one
    (``oracle.dropout``).
    Returns (o [R, dv], lse [R]) and, if ``return_p``, also P [R, Nk] (the
    undropped probabilities).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = q.shape[0]
    nk, dv = k.shape[0], v.shape[1]
    if row_ids is None:
        row_ids = np.arange(rows)
    row_ids = np.asarray(row_ids, dtype=np.int64)

    ok = allowed_mask(row_ids, nq, nk, causal, k_len_b, align=align, window=window)
    s = (q @ k.T) * float(scale)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)
    s = np.where(ok, s, -np.inf)

    nonempty = ok.any(axis=1)
    m = np.where(nonempty, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(ok, np.exp(s - m[:, None]), 0.0)
    ell = e.sum(axis=1)
    safe_ell = np.where(nonempty, ell, 1.0)
    p = e / safe_ell[:, None]
    if dropout is None:
        o = p @ v
    else:
        keep_256, seed = dropout
        z = keep_mask(bh, row_ids, nk, seed, keep_256)
        o = (np.where(z, p, 0.0) * keep_scale(keep_256)) @ v
    lse = np.where(nonempty, m + np.log(safe_ell), -np.inf)
    o[~nonempty] = 0.0
    p[~nonempty] = 0.0
    if return_p:
        return o, lse, p
    return o, lse


def attention_ref(q, k, v, *, scale, causal=False, k_len=None, bias=None,
                  return_p=False, align="bottom_right", window=(None, None), dropout=None):
    """Dense attention over a whole batch: q [B,H,Nq,dk], k [B,H,Nk,dk],
    v [B,H,Nk,dv], k_len [B] or None, bias [B,H,Nq,Nk] or None.

    Returns o [B,H,Nq,dv] and lse [B,H,Nq] in float64 (and P [B,H,Nq,Nk] when
    ``return_p``; only for small shapes).  Rows are processed in blocks so
    that S never holds more than a block of complete rows at once.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, heads, nq, _ = q.shape
    nk, dv = k.shape[2], v.shape[3]
    o = np.zeros((bsz, heads, nq, dv))
    lse = np.full((bsz, heads, nq), -np.inf)
    p_all = np.zeros((bsz, heads, nq, nk)) if return_p else None
    for b in range(bsz):
        klb = None if k_len is None else int(k_len[b])
        for h in range(heads):
            for r0 in range(0, nq, _ROW_BLOCK):
                r1 = min(nq, r0 + _ROW_BLOCK)
                bb = None if bias is None else bias[b, h, r0:r1]
                res = attention_head(q[b, h, r0:r1], k[b, h], v[b, h],
                                     scale=scale, nq=nq, causal=causal,
                                     k_len_b=klb, bias=bb,
                                     row_ids=np.arange(r0, r1),
                                     return_p=return_p, align=align, window=window,
                                     dropout=dropout, bh=b * heads + h)
                o[b, h, r0:r1] = res[0]
                lse[b, h, r0:r1] = res[1]
                if return_p:
                    p_all[b, h, r0:r1] = res[2]
    if return_p:
        return o, lse, p_all
    return o, lse

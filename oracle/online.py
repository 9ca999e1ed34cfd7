"""The pages' tile recurrence, in float64, for tiny shapes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is not the definition of the operator (``dense`` is); it is the method
the pages derive, written from their description so that the recurrence itself
can be pinned against their printed intermediate states and against the dense
definition under any key partition and visiting order.

* Per-block state ([VW] Step 4; [GS] section 3): for a nonempty set A of
  allowed keys with logits x_j,
      m_A = max x_j,   l_A = sum_{j in A} exp(x_j - m_A),
      u_A = sum_{j in A} exp(x_j - m_A) v_j      (length dv; not normalised).
* Merge of two disjoint blocks ([GS] section 4; [VW] Step 5; [OA] "Updating
  the Exponential Sum and Weighted Sum Together"): with m = max(m_A, m_B),
  both l and u of each block are rebased by exp(m_X - m):
      l = exp(m_A - m) l_A + exp(m_B - m) l_B,
      u = exp(m_A - m) u_A + exp(m_B - m) u_B.
  An empty block is skipped, never evaluated as exp(-inf - (-inf)) ([GS]
  section 6).
* Sequential form ([GS] section 5; [VW] Step 5): because the merge is exact
  and associative, a row's state after the key tiles visited so far is the
  merge of those tiles' block states, taken one tile at a time in visiting
  order from the empty state.  A tile in which the row has no allowed key
  contributes no block.  The row's output is u / l of its final state and
  lse = m + ln l; a row that never received a block is empty: o = 0,
  lse = -inf ([GS] sections 5-7).
"""

import numpy as np

from .dense import allowed_mask


def block_state(x, vals):
    """(m, l, u) of one nonempty block of logits ``x`` [n] with values [n, dv]."""
    x = np.asarray(x, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    if x.size == 0:
        raise ValueError("block_state needs a nonempty block")
    m = x.max()
    e = np.exp(x - m)
    return m, e.sum(), e @ vals


def merge_states(a, b):
    """Merge two states of disjoint key sets; ``None`` is the empty state."""
    if a is None:
        return b
    if b is None:
        return a
    m_a, l_a, u_a = a
    m_b, l_b, u_b = b
    m = max(m_a, m_b)
    alpha_a = np.exp(m_a - m)
    alpha_b = np.exp(m_b - m)
    return m, alpha_a * l_a + alpha_b * l_b, alpha_a * u_a + alpha_b * u_b


def _check_partition(tiles, n):
    """Key tiles must cover [0, n) once each: a repeated key would be counted
    twice in both l and u ([GS] section 4)."""
    seen = np.zeros(n, dtype=np.int64)
    for lo, hi in tiles:
        if not (0 <= lo <= hi <= n):
            raise ValueError(f"tile ({lo}, {hi}) outside [0, {n}]")
        seen[lo:hi] += 1
    if np.any(seen != 1):
        raise ValueError("tiles must partition the key axis exactly once")


def even_tiles(n, size):
    """Contiguous tiles of ``size`` keys (the last one ragged)."""
    return [(lo, min(n, lo + size)) for lo in range(0, n, size)] or [(0, 0)]


def online_ref(q, k, v, *, scale, causal=False, k_len_b=None, bias=None,
               key_tiles=None, query_tiles=None, order=None, trace=None):
    """Tile-by-tile forward for one (batch, head).

    q [Nq, dk], k [Nk, dk], v [Nk, dv], bias [Nq, Nk] or None.
    ``key_tiles``: list of (lo, hi) key ranges forming a partition of the key
    axis (irregular and empty tiles allowed); ``order``: visiting order of the
    key tiles; ``query_tiles``: list of (lo, hi) query ranges.  If ``trace``
    is a list, one record per (query tile, key tile) is appended holding the
    per-row (m, l, u, alpha) after that tile.
    Returns (o [Nq, dv], lse [Nq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk, dv = q.shape[0], k.shape[0], v.shape[1]
    if key_tiles is None:
        key_tiles = even_tiles(nk, max(nk, 1))
    _check_partition(key_tiles, nk)
    if query_tiles is None:
        query_tiles = even_tiles(nq, max(nq, 1))
    if order is None:
        order = range(len(key_tiles))
    if sorted(order) != list(range(len(key_tiles))):
        raise ValueError("order must visit every key tile once")

    o = np.zeros((nq, dv))
    lse = np.full(nq, -np.inf)
    for qa, qb in query_tiles:
        states = [None] * (qb - qa)  # per row of the query tile; None = empty
        for t in order:
            ka, kb = key_tiles[t]
            # scaled scores and the mask by global position ([GS] section 6)
            s = (q[qa:qb] @ k[ka:kb].T) * float(scale)
            if bias is not None:
                s = s + np.asarray(bias, dtype=np.float64)[qa:qb, ka:kb]
            ok = allowed_mask(np.arange(qa, qb), nq, nk, causal, k_len_b)[:, ka:kb]
            alphas = np.ones(qb - qa)
            for r in range(qb - qa):
                if not ok[r].any():
                    continue  # no allowed key in this tile: no block to merge
                old = states[r]
                states[r] = merge_states(old, block_state(s[r, ok[r]], v[ka:kb][ok[r]]))
                # the factor the merge applied to the state held before
                alphas[r] = 0.0 if old is None else np.exp(old[0] - states[r][0])
            if trace is not None:
                trace.append({"query_tile": (qa, qb), "key_tile": (ka, kb),
                              "m": np.array([-np.inf if x is None else x[0] for x in states]),
                              "l": np.array([0.0 if x is None else x[1] for x in states]),
                              "u": np.array([np.zeros(dv) if x is None else x[2] for x in states]),
                              "alpha": alphas})
        for r, st in enumerate(states):
            if st is not None:
                m, ell, u = st
                o[qa + r] = u / ell
                lse[qa + r] = m + np.log(ell)
    return o, lse

"""Pins for the float64 oracle: each takes the oracle package as an argument.

The same suite runs against the real oracle (tests/test_oracle.py) and
against deliberately mutated copies of it (tests/test_oracle_mutants.py), so
that every plausible mistake in the oracle -- a dropped term, a wrong sign, a
wrong index or alignment, a transposed operand -- is shown to fail at least
one pin.

What pins the oracle (none of it is the oracle's own formula retyped):

* the values the pages print for their worked examples (tests/golden/*.json,
  each with its citation), at the printed precision;
* closed forms: equal logits give the plain mean, a single allowed key gives
  that key's value, an empty key axis gives O = 0 and lse = -inf;
* invariants: rows of P sum to one, masked weight is zero,
  max s <= lse <= max s + ln |J|, a common logit shift leaves O unchanged and
  moves lse by the shift, the tile recurrence is independent of tile size and
  visiting order;
* an independent library routine: torch's CPU scaled_dot_product_attention
  in float64 under an explicit additive mask (rows with at least one allowed
  key), and scipy's logsumexp for lse;
* for the backward ([GS] section 7): torch autograd of the plain operator in
  float64, central finite differences of the forward definition, and the
  identities the recomputed gradients satisfy (identical keys, row sums of P
  and of D, empty rows, a single visible key).
"""

import itertools
import json
import math
import pathlib

import numpy as np

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"

_SYMBOLS = {"ln3": math.log(3.0), "1/sqrt2": 1.0 / math.sqrt(2.0)}


def _num(x):
    if isinstance(x, str):
        return _SYMBOLS[x]
    if isinstance(x, list):
        return [_num(e) for e in x]
    return x


def load_golden(name):
    with open(GOLDEN / name) as f:
        fx = json.load(f)
    for key in ("q", "k", "v", "scale"):
        if key in fx:
            fx[key] = _num(fx[key])
    return fx


def _close(got, want, tol, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    err = np.max(np.abs(got - want)) if got.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}\n got {got}\n want {want}"


def _dense1(orc, q, k, v, scale, **kw):
    """Dense oracle on a single (batch, head) given as 2-D lists."""
    q = np.asarray(q, dtype=np.float64)[None, None]
    k = np.asarray(k, dtype=np.float64)[None, None]
    v = np.asarray(v, dtype=np.float64)[None, None]
    o, lse, p = orc.attention_ref(q, k, v, scale=scale, return_p=True, **kw)
    return o[0, 0], lse[0, 0], p[0, 0]


def _accept(x, y, abs_tol, rel_tol):
    """Element-wise acceptance rule of the pages' CPU checks (section 9 of
    "How Does FlashAttention Preserve Global Softmax Across Tiles?")."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    both_inf = np.isinf(x) & np.isinf(y) & (np.sign(x) == np.sign(y))
    fin = ~both_inf
    bound = abs_tol + rel_tol * np.maximum(np.abs(x[fin]), np.abs(y[fin]))
    return bool(np.all(np.abs(x[fin] - y[fin]) <= bound)) and not np.any(np.isnan(x) | np.isnan(y))


# --------------------------------------------------------------------------
# worked examples printed on the pages
# --------------------------------------------------------------------------

def pin_gs_sec2_tile_local_counterexample(orc):
    fx = load_golden("gs_sec2_tile_local_counterexample.json")
    ex, tol = fx["expected"], fx["tolerance"]
    o, lse, p = _dense1(orc, fx["q"], fx["k"], fx["v"], fx["scale"])
    _close(p[0], ex["weights"], tol, "global weights")
    _close(o[0], ex["o"], tol, "dense output")
    _close(lse[0], math.log(4.0), tol, "lse = ln(1 + 3)")
    for order in ([0, 1], [1, 0]):
        oo, _ = orc.online_ref(fx["q"], fx["k"], fx["v"], scale=fx["scale"],
                               key_tiles=fx["key_tiles"], order=order)
        _close(oo[0], ex["o"], tol, f"online output, order {order}")
    # the two wrong answers the page names must differ from the oracle's
    assert abs(o[0, 0] - ex["tile_local_sum"]) > 0.2
    assert abs(o[0, 0] - ex["tile_local_average"]) > 0.2


def pin_gs_sec4_rescale_both(orc):
    fx = load_golden("gs_sec4_rescale_both.json")
    ex, tol = fx["expected"], fx["tolerance"]
    o, _, _ = _dense1(orc, fx["q"], fx["k"], fx["v"], fx["scale"])
    _close(o[0], ex["o"], tol, "dense output")
    trace = []
    oo, _ = orc.online_ref(fx["q"], fx["k"], fx["v"], scale=fx["scale"],
                           key_tiles=fx["key_tiles"], trace=trace)
    _close(oo[0], ex["o"], tol, "online output")
    _close(trace[1]["alpha"][0], ex["alpha_second_tile"], tol, "alpha at tile 2")
    assert abs(oo[0, 0] - ex["denominator_only_rescale"]) > 0.2


def pin_vw_step6_row0(orc):
    fx = load_golden("vw_step6_row0.json")
    ex, tol = fx["expected"], fx["tolerance"]
    q, k, v, scale = (np.asarray(fx[x], dtype=np.float64) for x in ("q", "k", "v", "scale"))
    scale = float(scale)
    o, _, _ = _dense1(orc, q, k, v, scale)
    _close(o[0], ex["o"], tol, "dense row 0")
    tiles = fx["key_tiles"]
    states = []
    for t, (lo, hi) in enumerate(tiles):
        x = (q[0] @ k[lo:hi].T) * scale
        _close(x, ex["tile_scores"][t], tol, f"tile {t} scores")
        m, ell, u = orc.block_state(x, v[lo:hi])
        _close(m, ex["tile_m"][t], tol, f"tile {t} m")
        _close(np.exp(x - m), ex["tile_exponents"][t], tol, f"tile {t} exponents")
        _close(ell, ex["tile_l"][t], tol, f"tile {t} l")
        _close(u, ex["tile_u"][t], tol, f"tile {t} u")
        states.append((m, ell, u))
    m, ell, u = orc.merge_states(states[0], states[1])
    _close(ell, ex["merged_l"], tol, "merged l")
    _close(u, ex["merged_u"], tol, "merged u")
    _close(u / ell, ex["o"], tol, "merged output")
    trace = []
    oo, _ = orc.online_ref(q, k, v, scale=scale, key_tiles=tiles, trace=trace)
    _close(oo[0], ex["o"], tol, "online row 0")
    _close(trace[-1]["l"][0], ex["merged_l"], tol, "online final l")
    _close(trace[-1]["u"][0], ex["merged_u"], tol, "online final u")


def pin_oa_fig1(orc):
    fx = load_golden("oa_fig1_weighted_sum_first.json")
    ex, tol = fx["expected"], fx["tolerance"]
    o, _, p = _dense1(orc, fx["q"], fx["k"], fx["v"], fx["scale"])
    _close(p[0], ex["probabilities"], tol, "probabilities")
    _close(o[0], ex["o"], tol, "output")
    x = np.asarray(fx["q"]) @ np.asarray(fx["k"]).T
    m, ell, u = orc.block_state(x[0], fx["v"])
    _close(np.exp(x[0] - m), ex["exponentials"], tol, "exponentials")
    _close(ell, ex["l"], tol, "exponential sum")
    _close(u, ex["u"], tol, "weighted sum before division")
    _close(u / ell, ex["o"], tol, "divided once")


def pin_oa_fig2_chunk_states(orc):
    fx = load_golden("oa_fig2_chunk_states.json")
    ex, tol = fx["expected"], fx["tolerance"]
    trace = []
    o, _ = orc.online_ref(fx["q"], fx["k"], fx["v"], scale=fx["scale"],
                          key_tiles=fx["key_tiles"], trace=trace)
    assert len(trace) == 3
    for t, want in enumerate(ex["states"]):
        _close(trace[t]["m"][0], want["m"], tol, f"m after chunk {t + 1}")
        _close(trace[t]["l"][0], want["l"], tol, f"l after chunk {t + 1}")
        _close(trace[t]["u"][0], want["u"], tol, f"a after chunk {t + 1}")
        if want["alpha"] is not None:
            _close(trace[t]["alpha"][0], want["alpha"], tol, f"alpha at chunk {t + 1}")
    alpha3 = trace[2]["alpha"][0]
    _close(alpha3 * trace[1]["l"][0], ex["chunk3_rescaled_l"], tol, "rescaled l")
    _close(alpha3 * trace[1]["u"][0], ex["chunk3_rescaled_u"], tol, "rescaled a")
    # chunk contributions against the chunk's own block state, rebased to m
    v = np.asarray(fx["v"], dtype=np.float64)
    x = (np.asarray(fx["q"]) @ np.asarray(fx["k"]).T)[0]
    for c, lo, m_ref in ((2, 2, 2.0), (3, 4, 3.0)):
        mb, lb, ub = orc.block_state(x[lo:lo + 2], v[lo:lo + 2])
        f = math.exp(mb - m_ref)
        _close(np.exp(x[lo:lo + 2] - m_ref), ex[f"chunk{c}_exponentials"], tol, f"chunk {c} exponentials")
        _close(f * lb, ex[f"chunk{c}_mass"], tol, f"chunk {c} mass")
        _close(f * ub, ex[f"chunk{c}_contribution"], tol, f"chunk {c} contribution")
    _close(o[0], ex["o"], tol, "online output")
    od, _, _ = _dense1(orc, fx["q"], fx["k"], fx["v"], fx["scale"])
    _close(od[0], ex["o"], tol, "dense output")
    # merging the three chunks' own states in any order and grouping gives
    # the printed final state (merge is associative and commutative,
    # "How Does FlashAttention Preserve Global Softmax Across Tiles?" section 4)
    blocks = [orc.block_state(x[lo:hi], v[lo:hi]) for lo, hi in fx["key_tiles"]]
    final = ex["states"][-1]
    for perm in itertools.permutations(range(3)):
        a, b, c = (blocks[i] for i in perm)
        for st in (orc.merge_states(orc.merge_states(a, b), c),
                   orc.merge_states(a, orc.merge_states(b, c)),
                   orc.merge_states(None, orc.merge_states(orc.merge_states(a, None), orc.merge_states(b, c)))):
            _close(st[0], final["m"], tol, f"merged m {perm}")
            _close(st[1], final["l"], tol, f"merged l {perm}")
            _close(st[2], final["u"], tol, f"merged a {perm}")


def pin_oa_fig3_two_queries(orc):
    fx = load_golden("oa_fig3_two_queries.json")
    ex, tol = fx["expected"], fx["tolerance"]
    q, k = np.asarray(fx["q"]), np.asarray(fx["k"])
    for t, (lo, hi) in enumerate(fx["key_tiles"]):
        _close(q @ k[lo:hi].T, ex["tile_scores"][t], tol, f"tile {t} scores")
    trace = []
    o, _ = orc.online_ref(fx["q"], fx["k"], fx["v"], scale=fx["scale"],
                          key_tiles=fx["key_tiles"], trace=trace)
    _close(trace[0]["l"], ex["tile1_l"], tol, "tile-1 sums")
    _close(trace[0]["u"], ex["tile1_u"], tol, "tile-1 weighted sums")
    _close(np.exp(q @ k[0:2].T - trace[0]["m"][:, None]), ex["tile1_exponentials"], tol,
           "tile-1 exponentials")
    _close(trace[1]["alpha"], ex["tile2_alpha"], tol, "per-row rescale at tile 2")
    _close(trace[1]["l"], ex["final_l"], tol, "final sums")
    _close(trace[1]["u"], ex["final_u"], tol, "final weighted sums")
    _close(o, ex["o"], tol, "online outputs")
    od, _, _ = _dense1(orc, fx["q"], fx["k"], fx["v"], fx["scale"])
    _close(od, ex["o"], tol, "dense outputs")


def pin_gs_sec6_alignment(orc):
    fx = load_golden("gs_sec6_alignment.json")
    for case in fx["cases"]:
        nq, nk = case["nq"], case["nk"]
        ok = orc.allowed_mask(np.arange(nq), nq, nk, True, None)
        assert list(ok.sum(axis=1)) == case["allowed_counts"], (case, ok)
        # the visible keys are always a prefix (keys 0 .. count-1)
        for i, cnt in enumerate(case["allowed_counts"]):
            assert ok[i, :cnt].all() and not ok[i, cnt:].any()
        if "top_left_counts" in case:
            assert case["top_left_counts"] != case["allowed_counts"]
            tl = orc.allowed_mask(np.arange(nq), nq, nk, True, None, align="top_left")
            assert list(tl.sum(axis=1)) == case["top_left_counts"], (case, tl)
        # the dense output of an empty row is exactly zero, its lse -inf
        rng = np.random.default_rng(nq * 10 + nk)
        q = rng.standard_normal((nq, 3))
        k = rng.standard_normal((nk, 3))
        v = rng.standard_normal((nk, 2))
        o, lse, p = _dense1(orc, q, k, v, 0.5, causal=True)
        for i, cnt in enumerate(case["allowed_counts"]):
            if cnt == 0:
                assert np.all(o[i] == 0.0) and lse[i] == -np.inf
            assert np.all(p[i, cnt:] == 0.0)
    # the key-length mask: keys at or beyond k_len are invisible; k_len is
    # clamped to [0, Nk]
    ok = orc.allowed_mask(np.arange(3), 3, 6, False, 4)
    assert list(ok.sum(axis=1)) == [4, 4, 4]
    assert list(orc.allowed_mask(np.arange(2), 2, 5, False, 99).sum(axis=1)) == [5, 5]
    assert list(orc.allowed_mask(np.arange(2), 2, 5, False, -3).sum(axis=1)) == [0, 0]
    # both masks together intersect; the causal offset uses Nq and Nk
    ok = orc.allowed_mask(np.arange(4), 4, 6, True, 4)
    assert list(ok.sum(axis=1)) == [3, 4, 4, 4]


def pin_mask_variants(orc):
    """Top-left alignment and windows ([GS] section 6), against bands built
    independently with torch's tril/triu (a key j is visible from row i when
    pos_i - wl <= j <= pos_i (+ wr)), closed forms, and torch SDPA under that
    band."""
    import torch

    rng = np.random.default_rng(61)
    for (nq, nk, align, wl, wr, causal, k_len) in (
            (7, 11, "bottom_right", 3, None, True, None), (7, 11, "top_left", 3, None, True, None),
            (9, 6, "bottom_right", 2, None, True, 5), (6, 9, "top_left", None, None, True, 8),
            (8, 8, "bottom_right", 2, 1, False, None), (5, 12, "top_left", 0, 4, False, 10),
            (10, 10, "bottom_right", 0, None, True, None)):
        off = (nk - nq) if align == "bottom_right" else 0
        band = torch.ones(nq, nk, dtype=torch.bool)
        if causal:
            band = band.tril(diagonal=off)
        if wr is not None:
            band = band.tril(diagonal=off + wr)
        if wl is not None:
            band = band.triu(diagonal=off - wl)
        if k_len is not None:
            band[:, min(max(k_len, 0), nk):] = False
        ok = orc.allowed_mask(np.arange(nq), nq, nk, causal, k_len, align=align, window=(wl, wr))
        assert np.array_equal(ok, band.numpy()), (nq, nk, align, wl, wr, causal, k_len)
        q = rng.standard_normal((1, 1, nq, 4))
        k = rng.standard_normal((1, 1, nk, 4))
        v = rng.standard_normal((1, 1, nk, 3))
        o, lse = orc.attention_ref(q, k, v, scale=0.7, causal=causal, k_len=None if k_len is None else [k_len],
                                   align=align, window=(wl, wr))
        rows = band.any(dim=1).numpy()
        add = np.where(band.numpy(), 0.0, -np.inf)[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=torch.from_numpy(add),
            scale=0.7).numpy()
        _close(o[0, 0, rows], ref[0, 0, rows], 1e-12, "window vs SDPA")
        assert np.all(o[0, 0, ~rows] == 0.0) and np.all(lse[0, 0, ~rows] == -np.inf)
        if causal and wl == 0:  # a row sees exactly the key at its aligned position
            for i in range(nq):
                if 0 <= i + off < nk:
                    _close(o[0, 0, i], v[0, 0, i + off], 1e-14, "window 0 picks the aligned key")


# --------------------------------------------------------------------------
# the CPU check families of the pages' section 9, dense vs online
# --------------------------------------------------------------------------

def _random_partition(rng, n, max_tiles=4):
    """Irregular contiguous tiles, empty ones allowed."""
    cuts = sorted(rng.integers(0, n + 1, size=rng.integers(0, max_tiles)))
    bounds = [0, *cuts, n]
    return [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:])]


def pin_gs_sec9_families(orc):
    fx = load_golden("gs_sec9_check_families.json")
    at, rt = fx["acceptance"]["abs"], fx["acceptance"]["rel"]
    rng = np.random.default_rng(9)
    n_cmp = 0
    for fam in fx["families"]:
        for nq, nk, dk, dv in fam["shapes"]:
            q = rng.standard_normal((nq, dk))
            k = rng.standard_normal((nk, dk))
            v = rng.standard_normal((nk, dv))
            scale = 1.0 / math.sqrt(dk)
            bias = None
            if fam.get("shift"):
                # a wide span of finite logits ([GS] section 9, "common logit
                # shifts and wide span")
                bias = np.tile(np.array([0.0, 40.0, -40.0, 39.5, 1.0])[:nk], (nq, 1))
            k_lens = [None]
            if fam.get("padding"):
                k_lens = [0, 1, nk - 1, nk]
            for klen in k_lens:
                od, ld, _ = _dense1(orc, q, k, v, scale, causal=fam["causal"],
                                    k_len=None if klen is None else [klen],
                                    bias=None if bias is None else bias[None, None])
                if fam.get("all_orders"):
                    parts = [[(0, 2), (2, 4), (4, 6)]]
                else:
                    parts = [_random_partition(rng, nk) for _ in range(3)]
                    parts.append(orc.even_tiles(nk, 2))
                for tiles in parts:
                    orders = [list(range(len(tiles)))]
                    if fam.get("all_orders"):
                        orders = [list(p) for p in itertools.permutations(range(3))]
                    for order in orders:
                        for qt in (orc.even_tiles(nq, 2), orc.even_tiles(nq, max(nq, 1))):
                            oo, lo = orc.online_ref(q, k, v, scale=scale, causal=fam["causal"],
                                                    k_len_b=klen, bias=bias, key_tiles=tiles,
                                                    query_tiles=qt, order=order)
                            assert _accept(od, oo, at, rt), (fam["name"], tiles, order, od, oo)
                            assert _accept(ld, lo, at, rt), (fam["name"], tiles, order, ld, lo)
                            n_cmp += 2
    assert n_cmp > 59


def pin_seeded_shapes_dense_vs_online(orc):
    """Sixteen seeded shapes of our own in place of the page's unlisted ones,
    with bias and both masks, random irregular tiles and random order."""
    rng = np.random.default_rng(16)
    for _ in range(16):
        nq, nk = int(rng.integers(1, 9)), int(rng.integers(0, 11))
        dk, dv = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        q = rng.standard_normal((nq, dk))
        k = rng.standard_normal((nk, dk))
        v = rng.standard_normal((nk, dv))
        bias = rng.standard_normal((nq, nk))
        causal = bool(rng.integers(0, 2))
        klen = int(rng.integers(-1, nk + 2))
        od, ld, _ = _dense1(orc, q, k, v, 0.7, causal=causal, k_len=[klen], bias=bias[None, None])
        tiles = _random_partition(rng, nk)
        order = list(rng.permutation(len(tiles)))
        oo, lo = orc.online_ref(q, k, v, scale=0.7, causal=causal, k_len_b=klen, bias=bias,
                                key_tiles=tiles, query_tiles=orc.even_tiles(nq, 3), order=order)
        assert _accept(od, oo, 2e-12, 2e-12), (nq, nk, tiles, order)
        assert _accept(ld, lo, 2e-12, 2e-12), (nq, nk, tiles, order)


def pin_duplicate_keys_rejected(orc):
    """A key counted twice inflates both l and u ([GS] section 4), so the
    recurrence refuses a key partition with a repeated key."""
    q, k, v = [[1.0]], [[0.0], [1.0]], [[1.0], [2.0]]
    for tiles in ([(0, 2), (1, 2)], [(0, 1)]):
        try:
            orc.online_ref(q, k, v, scale=1.0, key_tiles=tiles)
        except ValueError:
            continue
        raise AssertionError(f"partition {tiles} was accepted")


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def pin_closed_forms(orc):
    rng = np.random.default_rng(5)
    # equal logits give the plain mean of the allowed values ([VW] Step 7)
    nq, nk, dk, dv = 6, 9, 4, 3
    q = np.zeros((nq, dk))
    k = rng.standard_normal((nk, dk))
    v = rng.standard_normal((nk, dv))
    o, lse, _ = _dense1(orc, q, k, v, 0.5, causal=True, k_len=[7])
    for i in range(nq):
        cnt = min(i + nk - nq + 1, 7)
        _close(o[i], v[:cnt].mean(axis=0), 1e-13, f"equal logits row {i}")
        _close(lse[i], math.log(cnt), 1e-13, f"equal logits lse row {i}")
    # a single allowed key: o = v_j and lse = s_j
    q = rng.standard_normal((1, dk))
    bias = rng.standard_normal((1, nk))
    o, lse, _ = _dense1(orc, q, k, v, 0.3, k_len=[1], bias=bias[None, None])
    _close(o[0], v[0], 1e-14, "single key output")
    _close(lse[0], 0.3 * float(q[0] @ k[0]) + bias[0, 0], 1e-14, "single key lse")
    # one dominating score: the output collapses to that key's value
    bias = np.zeros((1, nk))
    bias[0, 4] = 60.0
    o, _, _ = _dense1(orc, np.zeros((1, dk)), k, v, 1.0, bias=bias[None, None])
    _close(o[0], v[4], 1e-12, "dominating score")
    # empty key axis: o = 0, lse = -inf, never NaN ([GS] section 9 family)
    o, lse, _ = _dense1(orc, rng.standard_normal((2, 3)), np.zeros((0, 3)),
                        np.zeros((0, 2)), 0.5)
    assert o.shape == (2, 2) and np.all(o == 0.0) and np.all(lse == -np.inf)
    oo, lo = orc.online_ref(rng.standard_normal((2, 3)), np.zeros((0, 3)), np.zeros((0, 2)),
                            scale=0.5)
    assert np.all(oo == 0.0) and np.all(lo == -np.inf)
    # a padded-away sequence (k_len = 0): every row empty, no NaN
    o, lse, p = _dense1(orc, rng.standard_normal((3, 2)), rng.standard_normal((4, 2)),
                        rng.standard_normal((4, 5)), 1.0, causal=True, k_len=[0])
    assert np.all(o == 0.0) and np.all(lse == -np.inf) and np.all(p == 0.0)
    # two keys with logit gap g and scalar values (0, 1): o = 1 / (1 + e^-g)
    for gap in (0.0, 1.0, 7.5, -3.0):
        o, lse, _ = _dense1(orc, [[1.0]], [[0.0], [gap]], [[0.0], [1.0]], 1.0)
        _close(o[0, 0], 1.0 / (1.0 + math.exp(-gap)), 1e-15, f"two-key gap {gap}")
        _close(lse[0], max(0.0, gap) + math.log1p(math.exp(-abs(gap))), 1e-14, "two-key lse")


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def pin_invariants(orc):
    rng = np.random.default_rng(7)
    bsz, heads, nq, nk, dk, dv = 2, 3, 11, 13, 6, 5
    q = rng.standard_normal((bsz, heads, nq, dk))
    k = rng.standard_normal((bsz, heads, nk, dk))
    v = rng.standard_normal((bsz, heads, nk, dv))
    bias = rng.standard_normal((bsz, heads, nq, nk))
    k_len = [9, 13]
    o, lse, p = orc.attention_ref(q, k, v, scale=0.4, causal=True, k_len=k_len, bias=bias,
                                  return_p=True)
    for b in range(bsz):
        ok = orc.allowed_mask(np.arange(nq), nq, nk, True, k_len[b])
        cnt = ok.sum(axis=1)
        for h in range(heads):
            assert np.all(p[b, h][~ok] == 0.0), "masked weight must be zero"
            nonempty = cnt > 0
            _close(p[b, h][nonempty].sum(axis=1), np.ones(nonempty.sum()), 1e-14, "rows sum to one")
            assert np.all(p[b, h] >= 0.0)
            s = 0.4 * q[b, h] @ k[b, h].T + bias[b, h]
            smax = np.where(ok, s, -np.inf).max(axis=1)
            assert np.all(lse[b, h][nonempty] >= smax[nonempty] - 1e-12)
            assert np.all(lse[b, h][nonempty] <= smax[nonempty] + np.log(cnt[nonempty]) + 1e-12)
    # a common shift c of one row's logits leaves o unchanged, moves lse by c
    shift = np.zeros_like(bias)
    shift[:, :, 4, :] = 123.25
    shift[:, :, 7, :] = -50.5
    o2, lse2 = orc.attention_ref(q, k, v, scale=0.4, causal=True, k_len=k_len, bias=bias + shift)
    _close(o2, o, 1e-12, "shifted output")
    fin = np.isfinite(lse)
    _close((lse2 - lse)[fin], shift[..., 0][fin], 1e-11, "shifted lse")
    # the output is a convex combination of the allowed values (per coordinate)
    for b in range(bsz):
        ok = orc.allowed_mask(np.arange(nq), nq, nk, True, k_len[b])
        for h in range(heads):
            for i in range(nq):
                if ok[i].any():
                    vv = v[b, h][ok[i]]
                    assert np.all(o[b, h, i] <= vv.max(axis=0) + 1e-12)
                    assert np.all(o[b, h, i] >= vv.min(axis=0) - 1e-12)
    # batch entries and heads are independent: permuting heads permutes outputs
    perm = [2, 0, 1]
    o3, _ = orc.attention_ref(q[:, perm], k[:, perm], v[:, perm], scale=0.4, causal=True,
                              k_len=k_len, bias=bias[:, perm])
    _close(o3, o[:, perm], 0.0, "head permutation")
    # 1 <= l <= n for every nonempty row ([GS] section 3), read off the trace
    trace = []
    orc.online_ref(q[1, 0], k[1, 0], v[1, 0], scale=0.4, causal=True, k_len_b=13,
                   bias=bias[1, 0], key_tiles=orc.even_tiles(nk, 4), trace=trace)
    ok = orc.allowed_mask(np.arange(nq), nq, nk, True, 13)
    ell = trace[-1]["l"]
    assert np.all(ell >= 1.0 - 1e-12) and np.all(ell <= ok.sum(axis=1) + 1e-12)


def pin_tile_size_invariance(orc):
    """Changing the tile size must not change the output beyond rounding
    ([GS] section 9, diagnosis of tile-size dependence)."""
    rng = np.random.default_rng(11)
    nq, nk, dk, dv = 9, 17, 4, 3
    q, k = rng.standard_normal((nq, dk)) * 3, rng.standard_normal((nk, dk)) * 3
    v = rng.standard_normal((nk, dv))
    outs = []
    for ts in (1, 2, 3, 5, 8, 17):
        for qs in (1, 4, 9):
            outs.append(orc.online_ref(q, k, v, scale=0.5, causal=True, k_len_b=15,
                                       key_tiles=orc.even_tiles(nk, ts),
                                       query_tiles=orc.even_tiles(nq, qs)))
    for o, lse in outs[1:]:
        assert _accept(o, outs[0][0], 2e-12, 2e-12)
        assert _accept(lse, outs[0][1], 2e-12, 2e-12)


# --------------------------------------------------------------------------
# independent library routines
# --------------------------------------------------------------------------

def pin_library_sdpa(orc):
    """torch's CPU scaled_dot_product_attention (float64, explicit additive
    mask) computes the same operator; scipy's logsumexp gives lse."""
    import torch
    from scipy.special import logsumexp

    rng = np.random.default_rng(3)
    for (bsz, heads, nq, nk, dk, dv, causal, k_len, use_bias, scale) in (
            (2, 3, 7, 9, 5, 3, True, [9, 6], True, 0.37),
            (1, 2, 9, 4, 2, 6, False, [3], False, 1.0),
            (2, 1, 5, 12, 8, 8, True, [12, 12], True, 1.0 / math.sqrt(8)),
            (1, 1, 16, 16, 3, 1, True, None, False, 0.9),
    ):
        q = rng.standard_normal((bsz, heads, nq, dk))
        k = rng.standard_normal((bsz, heads, nk, dk))
        v = rng.standard_normal((bsz, heads, nk, dv))
        bias = rng.standard_normal((bsz, heads, nq, nk)) if use_bias else np.zeros((bsz, heads, nq, nk))
        o, lse = orc.attention_ref(q, k, v, scale=scale, causal=causal, k_len=k_len,
                                   bias=bias if use_bias else None)
        ok = np.zeros((bsz, heads, nq, nk), dtype=bool)
        for b in range(bsz):
            ok[b, :] = orc.allowed_mask(np.arange(nq), nq, nk, causal,
                                        None if k_len is None else k_len[b])
        # the mask is checked independently: bottom-right prefix lengths
        for b in range(bsz):
            lim = nk if k_len is None else min(max(k_len[b], 0), nk)
            for i in range(nq):
                cnt = min(lim, i + nk - nq + 1) if causal else lim
                assert ok[b, 0, i].sum() == max(cnt, 0)
        add = np.where(ok, bias, -np.inf)
        rows = ok.any(axis=-1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=torch.from_numpy(add), scale=scale).numpy()
        _close(o[rows], ref[rows], 1e-12, "vs torch SDPA")
        lib_lse = logsumexp(np.where(ok, scale * np.einsum("bhid,bhjd->bhij", q, k) + bias, -np.inf),
                            axis=-1)
        _close(lse[rows], lib_lse[rows], 1e-12, "vs scipy logsumexp")
        assert np.all(o[~rows] == 0.0) and np.all(lse[~rows] == -np.inf)


def pin_sampled_rows(orc):
    """Rows evaluated one by one (how full-size outputs are spot-checked)
    agree with the whole-matrix evaluation and with the equal-logit closed
    form at the rows' global positions."""
    rng = np.random.default_rng(21)
    nq, nk, dk, dv = 12, 20, 4, 3
    q = rng.standard_normal((nq, dk))
    k = rng.standard_normal((nk, dk))
    v = rng.standard_normal((nk, dv))
    bias = rng.standard_normal((nq, nk))
    o, lse, _ = _dense1(orc, q, k, v, 0.6, causal=True, k_len=[17], bias=bias[None, None])
    rows = np.array([11, 0, 5, 7])
    os_, ls_ = orc.attention_head(q[rows], k, v, scale=0.6, nq=nq, causal=True, k_len_b=17,
                                  bias=bias[rows], row_ids=rows)
    _close(os_, o[rows], 1e-14, "sampled rows")
    _close(ls_, lse[rows], 1e-14, "sampled lse")
    # zero query rows sampled at their global positions: mean of the visible prefix
    qz = np.zeros((3, dk))
    rows = np.array([0, 4, 10])
    oz, lz = orc.attention_head(qz, k, v, scale=0.6, nq=nq, causal=True, k_len_b=17,
                                row_ids=rows)
    for n, i in enumerate(rows):
        cnt = min(i + nk - nq + 1, 17)
        _close(oz[n], v[:cnt].mean(axis=0), 1e-13, f"sampled equal-logit row {i}")
        _close(lz[n], math.log(cnt), 1e-13, f"sampled equal-logit lse row {i}")


# --------------------------------------------------------------------------
# backward by recomputation ([GS] section 7, [VW] Step 8)
# --------------------------------------------------------------------------

def _bwd_case(rng, bsz, heads, nq, nk, dk, dv, scale_g=1.0):
    q = rng.standard_normal((bsz, heads, nq, dk))
    k = rng.standard_normal((bsz, heads, nk, dk))
    v = rng.standard_normal((bsz, heads, nk, dv))
    g = rng.standard_normal((bsz, heads, nq, dv)) * scale_g
    return q, k, v, g


def pin_bwd_autograd(orc):
    """torch autograd (float64, CPU) of the plain operator gives the same
    dQ, dK, dV: an independent differentiation of the definition.  Only rows
    with an allowed key enter the autograd graph (softmax over an empty set
    has no derivative); the oracle must give those rows' dQ = 0."""
    import torch

    rng = np.random.default_rng(41)
    for (bsz, heads, nq, nk, dk, dv, causal, k_len, use_bias, scale) in (
            (2, 2, 7, 9, 5, 3, True, [9, 6], True, 0.37),
            (1, 2, 9, 4, 2, 6, False, [3], False, 1.0),
            (2, 1, 5, 12, 8, 8, True, [12, 0], True, 1.0 / math.sqrt(8)),
            (1, 1, 12, 5, 3, 4, True, None, False, 0.9),   # Nq > Nk: empty top rows
    ):
        q, k, v, g = _bwd_case(rng, bsz, heads, nq, nk, dk, dv)
        bias = rng.standard_normal((bsz, heads, nq, nk)) if use_bias else None
        dq, dk_, dv_ = orc.attention_bwd_ref(q, k, v, g, scale=scale, causal=causal, k_len=k_len, bias=bias)
        for b in range(bsz):
            lim = nk if k_len is None else min(max(k_len[b], 0), nk)
            for h in range(heads):
                rows = [i for i in range(nq) if (min(lim, i + nk - nq + 1) if causal else lim) > 0]
                if not rows:  # every row empty: nothing depends on Q, K or V
                    assert np.all(dq[b, h] == 0.0) and np.all(dk_[b, h] == 0.0) and np.all(dv_[b, h] == 0.0)
                    continue
                tq = torch.from_numpy(q[b, h]).clone().requires_grad_(True)
                tk = torch.from_numpy(k[b, h]).clone().requires_grad_(True)
                tv = torch.from_numpy(v[b, h]).clone().requires_grad_(True)
                loss = torch.zeros((), dtype=torch.float64)
                for i in rows:
                    cnt = min(lim, i + nk - nq + 1) if causal else lim
                    logit = (tk[:cnt] @ tq[i]) * scale
                    if bias is not None:
                        logit = logit + torch.from_numpy(bias[b, h, i, :cnt])
                    o_i = torch.softmax(logit, dim=0) @ tv[:cnt]
                    loss = loss + (o_i * torch.from_numpy(g[b, h, i])).sum()
                gq, gk, gv = torch.autograd.grad(loss, (tq, tk, tv), allow_unused=False)
                _close(dq[b, h], gq.numpy(), 1e-12, "dQ vs autograd")
                _close(dk_[b, h], gk.numpy(), 1e-12, "dK vs autograd")
                _close(dv_[b, h], gv.numpy(), 1e-12, "dV vs autograd")
                empty = [i for i in range(nq) if i not in rows]
                assert np.all(dq[b, h, empty] == 0.0), "empty rows must give dQ = 0"


def pin_bwd_finite_differences(orc):
    """Central differences of the loss sum(G * O), O from the oracle's
    forward definition, match the backward on a tiny masked, biased case."""
    rng = np.random.default_rng(43)
    nq, nk, dk, dv, scale = 4, 5, 3, 2, 0.7
    q, k, v, g = _bwd_case(rng, 1, 1, nq, nk, dk, dv)
    bias = rng.standard_normal((1, 1, nq, nk))
    kw = dict(scale=scale, causal=True, k_len=[4], bias=bias)

    def loss(qq, kk, vv):
        o, _ = orc.attention_ref(qq, kk, vv, **kw)
        return float(np.sum(o * g))

    dq, dk_, dv_ = orc.attention_bwd_ref(q, k, v, g, **kw)
    eps = 1e-6
    for x, gx, name in ((q, dq, "dQ"), (k, dk_, "dK"), (v, dv_, "dV")):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        _close(gx, num, 1e-7, f"{name} vs central differences")


def pin_bwd_invariants(orc):
    """Identities of the recomputed gradients: with identical keys dQ = 0;
    each non-empty row's probabilities sum to one, so the keys' dV sum to the
    sum of the non-empty rows' G; each row of D sums to zero, so the keys'
    dK sum to zero; an empty row contributes nothing; passing the forward's
    O and lse explicitly changes nothing."""
    rng = np.random.default_rng(47)
    nq, nk, dk, dv = 6, 7, 4, 3
    q, k, v, g = _bwd_case(rng, 1, 1, nq, nk, dk, dv)
    kk = np.repeat(k[:, :, :1], nk, axis=2)
    dq, _, _ = orc.attention_bwd_ref(q, kk, v, g, scale=0.8, causal=True)
    _close(dq, np.zeros_like(dq), 1e-13, "identical keys give dQ = 0")
    bias = rng.standard_normal((1, 1, nq, nk))
    for k_len in ([7], [3], [0]):
        dq, dk_, dv_ = orc.attention_bwd_ref(q, k, v, g, scale=0.8, causal=True, k_len=k_len, bias=bias)
        ok = orc.allowed_mask(np.arange(nq), nq, nk, True, k_len[0])
        rows = ok.any(axis=1)
        _close(dv_[0, 0].sum(axis=0), g[0, 0, rows].sum(axis=0), 1e-12, "sum_j dV_j = sum of G")
        _close(dk_[0, 0].sum(axis=0), np.zeros(dk), 1e-12, "sum_j dK_j = 0")
        assert np.all(dq[0, 0, ~rows] == 0.0)
        assert np.all(dk_[0, 0, k_len[0]:] == 0.0) and np.all(dv_[0, 0, k_len[0]:] == 0.0), \
            "keys past k_len get no gradient"
        o, lse = orc.attention_ref(q, k, v, scale=0.8, causal=True, k_len=k_len, bias=bias)
        e = orc.attention_bwd_ref(q, k, v, g, scale=0.8, causal=True, k_len=k_len, bias=bias, o=o, lse=lse)
        for a, b_ in zip(e, (dq, dk_, dv_)):
            _close(a, b_, 1e-14, "explicit O and lse")
    # an extra empty row (Nq > Nk under bottom-right causal) with any G
    q2 = np.concatenate([rng.standard_normal((1, 1, 1, dk)), q], axis=2)
    g2 = np.concatenate([rng.standard_normal((1, 1, 1, dv)) * 100, g], axis=2)
    k2, v2 = k[:, :, :nq], v[:, :, :nq]
    a = orc.attention_bwd_ref(q[:, :, :], k2, v2, g, scale=0.8, causal=True)
    b_ = orc.attention_bwd_ref(q2, k2, v2, g2, scale=0.8, causal=True)
    _close(b_[1], a[1], 1e-13, "empty row leaves dK unchanged")
    _close(b_[2], a[2], 1e-13, "empty row leaves dV unchanged")
    assert np.all(b_[0][0, 0, 0] == 0.0)


def pin_bwd_single_key(orc):
    """Closed form: a row that sees one key has p = 1 and o = v, so its D row
    is zero (dQ_i = 0) and it passes g_i straight to that key's dV; with a
    1x1 problem dK = 0 and dV = g."""
    rng = np.random.default_rng(53)
    q, k, v, g = _bwd_case(rng, 1, 1, 1, 1, 3, 2)
    dq, dk_, dv_ = orc.attention_bwd_ref(q, k, v, g, scale=1.3)
    _close(dq, np.zeros_like(dq), 1e-15, "1x1 dQ")
    _close(dk_, np.zeros_like(dk_), 1e-15, "1x1 dK")
    _close(dv_, g, 1e-15, "1x1 dV")
    q, k, v, g = _bwd_case(rng, 1, 1, 4, 4, 3, 2)
    dq, _, dv_ = orc.attention_bwd_ref(q, k, v, g, scale=1.3, causal=True)
    _close(dq[0, 0, 0], np.zeros(3), 1e-15, "row 0 under causal sees key 0 only")


# --------------------------------------------------------------------------
# dropout with a counter-based mask ([GS] section 6: the backward replays the
# forward's mask and scaling)
# --------------------------------------------------------------------------

def pin_philox_known_answers(orc):
    """The generator reproduces the published known-answer vectors of
    Philox4x32-10 (tests/golden/philox4x32_10_kat.json)."""
    with open(GOLDEN / "philox4x32_10_kat.json") as f:
        fx = json.load(f)
    for vec in fx["vectors"]:
        ctr = np.array([int(x, 16) for x in vec["counter"]], dtype=np.uint32)
        key = np.array([int(x, 16) for x in vec["key"]], dtype=np.uint32)
        want = [int(x, 16) for x in vec["output"]]
        got = [int(x) for x in orc.philox4x32_10(ctr, key)]
        assert got == want, (vec, [f"{x:08x}" for x in got])


def pin_philox_statistics(orc):
    """Bytes of consecutive counters are uniform (chi-square over 256 bins),
    and flipping any one counter or key bit flips about half of the 128
    output bits (avalanche)."""
    n = 1 << 16
    ctr = np.zeros((n, 4), dtype=np.uint32)
    ctr[:, 0] = np.arange(n, dtype=np.uint32)
    ctr[:, 2] = 7
    words = orc.philox4x32_10(ctr, np.array([12345, 678], dtype=np.uint32))
    by = np.frombuffer(words.astype("<u4").tobytes(), dtype=np.uint8)
    hist = np.bincount(by, minlength=256).astype(np.float64)
    exp = by.size / 256.0
    chi2 = float(np.sum((hist - exp) ** 2 / exp))
    assert 170.0 < chi2 < 350.0, f"byte chi-square {chi2:.1f} over 255 degrees of freedom"
    rng = np.random.default_rng(5)
    base_c = rng.integers(0, 1 << 32, (256, 4), dtype=np.uint64).astype(np.uint32)
    base_k = rng.integers(0, 1 << 32, (256, 2), dtype=np.uint64).astype(np.uint32)
    out0 = orc.philox4x32_10(base_c, base_k)

    def flipped(a, b):
        x = (a ^ b).astype(np.uint64)
        return sum(int(bin(int(w)).count("1")) for w in x.reshape(-1)) / a.shape[0]

    for word in range(4):
        for bit in (0, 13, 31):
            c = base_c.copy()
            c[:, word] ^= np.uint32(1 << bit)
            mean = flipped(out0, orc.philox4x32_10(c, base_k))
            assert abs(mean - 64.0) < 3.0, (word, bit, mean)
    for word in range(2):
        k = base_k.copy()
        k[:, word] ^= np.uint32(1 << 17)
        assert abs(flipped(out0, orc.philox4x32_10(base_c, k)) - 64.0) < 3.0


def pin_dropout_mask_layout(orc):
    """The vectorised mask follows the stated layout element by element
    (counter (i, j div 64, b*H+h, (j div 4) mod 4), byte j mod 4 of word
    (j div 16) mod 4), keeps about keep_256/256 of the elements, and
    keep_256 = 256 keeps everything."""
    seed, bh, rows, nk = 0x1234_5678_9ABC_DEF0, 5, [0, 3, 70, 129], 200
    got = orc.dropout_bytes(bh, rows, nk, seed)
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)
    for a, i in enumerate(rows):
        for j in range(nk):
            ctr = np.array([i, j // 64, bh, (j // 4) % 4], dtype=np.uint32)
            word = int(orc.philox4x32_10(ctr, key)[(j // 16) % 4])
            assert int(got[a, j]) == (word >> (8 * (j % 4))) & 0xFF, (i, j)
    z = orc.keep_mask(3, np.arange(256), 512, 99, 230)
    rate, n = float(z.mean()), z.size
    sigma = math.sqrt(230 / 256 * (26 / 256) / n)
    assert abs(rate - 230 / 256) < 5 * sigma, rate
    assert orc.keep_mask(0, np.arange(8), 64, 1, 256).all()
    assert orc.keep_scale(230) == 256.0 / 230.0
    # different heads, rows and seeds draw different masks
    assert not np.array_equal(orc.dropout_bytes(0, [0], 64, 1), orc.dropout_bytes(1, [0], 64, 1))
    assert not np.array_equal(orc.dropout_bytes(0, [0], 64, 1), orc.dropout_bytes(0, [1], 64, 1))
    assert not np.array_equal(orc.dropout_bytes(0, [0], 64, 1), orc.dropout_bytes(0, [0], 64, 2))


def pin_dropout_forward(orc):
    """Forward with dropout: equals torch float64 attention with the mask
    applied to softmax(S) and the kept values scaled by 256/T; lse is the
    undropped one; T = 256 is no dropout, bit for bit; averaged over many
    seeds the dropped output approaches the undropped one."""
    import torch

    rng = np.random.default_rng(71)
    bsz, heads, nq, nk, dk, dv = 2, 2, 5, 70, 4, 3
    q = rng.standard_normal((bsz, heads, nq, dk))
    k = rng.standard_normal((bsz, heads, nk, dk))
    v = rng.standard_normal((bsz, heads, nk, dv))
    kw = dict(scale=0.6, causal=True, k_len=[70, 40])
    o0, l0 = orc.attention_ref(q, k, v, **kw)
    o_t, l_t = orc.attention_ref(q, k, v, dropout=(256, 77), **kw)
    assert np.array_equal(o0, o_t) and np.array_equal(l0, l_t)
    t, seed = 200, 0xABCDEF
    o, lse = orc.attention_ref(q, k, v, dropout=(t, seed), **kw)
    assert np.array_equal(lse, l0), "dropout must not change lse"
    for b in range(bsz):
        lim = kw["k_len"][b]
        for h in range(heads):
            s = torch.from_numpy(q[b, h]) @ torch.from_numpy(k[b, h]).T * 0.6
            i = torch.arange(nq)[:, None]
            j = torch.arange(nk)[None, :]
            allowed = (j <= i + nk - nq) & (j < lim)
            p = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=1)
            p = torch.nan_to_num(p, nan=0.0)
            z = torch.from_numpy(orc.keep_mask(b * heads + h, np.arange(nq), nk, seed, t))
            ref = (p * z * (256.0 / t)) @ torch.from_numpy(v[b, h])
            _close(o[b, h], ref.numpy(), 1e-12, "dropout forward vs torch")
    samples = np.stack([orc.attention_ref(q, k, v, dropout=(t, sd), **kw)[0] for sd in range(300)])
    mean, err = samples.mean(axis=0), samples.std(axis=0) / math.sqrt(300)
    assert np.all(np.abs(mean - o0) <= 5 * err + 1e-12), float(np.max(np.abs(mean - o0) / (err + 1e-300)))


def pin_dropout_backward(orc):
    """Backward with dropout: torch autograd (float64) of softmax, the fixed
    dropout mask and its scaling gives the oracle's dQ, dK, dV; the oracle is
    given its own dropped forward output."""
    import torch

    rng = np.random.default_rng(73)
    bsz, heads, nq, nk, dk, dv = 1, 2, 6, 70, 4, 5
    q, k, v, g = _bwd_case(rng, bsz, heads, nq, nk, dk, dv)
    t, seed, scale = 180, 31337, 0.45
    dq, dk_, dv_ = orc.attention_bwd_ref(q, k, v, g, scale=scale, causal=True, dropout=(t, seed))
    for h in range(heads):
        tq = torch.from_numpy(q[0, h]).clone().requires_grad_(True)
        tk = torch.from_numpy(k[0, h]).clone().requires_grad_(True)
        tv = torch.from_numpy(v[0, h]).clone().requires_grad_(True)
        i = torch.arange(nq)[:, None]
        j = torch.arange(nk)[None, :]
        allowed = j <= i + nk - nq
        s = (tq @ tk.T) * scale
        p = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=1)
        z = torch.from_numpy(orc.keep_mask(h, np.arange(nq), nk, seed, t))
        o = (p * z * (256.0 / t)) @ tv
        loss = (o * torch.from_numpy(g[0, h])).sum()
        gq, gk, gv = torch.autograd.grad(loss, (tq, tk, tv))
        _close(dq[0, h], gq.numpy(), 1e-12, "dropout dQ vs autograd")
        _close(dk_[0, h], gk.numpy(), 1e-12, "dropout dK vs autograd")
        _close(dv_[0, h], gv.numpy(), 1e-12, "dropout dV vs autograd")


PINS = [
    pin_gs_sec2_tile_local_counterexample,
    pin_gs_sec4_rescale_both,
    pin_vw_step6_row0,
    pin_oa_fig1,
    pin_oa_fig2_chunk_states,
    pin_oa_fig3_two_queries,
    pin_gs_sec6_alignment,
    pin_gs_sec9_families,
    pin_seeded_shapes_dense_vs_online,
    pin_duplicate_keys_rejected,
    pin_closed_forms,
    pin_invariants,
    pin_tile_size_invariance,
    pin_library_sdpa,
    pin_sampled_rows,
    pin_mask_variants,
    pin_bwd_autograd,
    pin_philox_known_answers,
    pin_philox_statistics,
    pin_dropout_mask_layout,
    pin_dropout_forward,
    pin_dropout_backward,
    pin_bwd_finite_differences,
    pin_bwd_invariants,
    pin_bwd_single_key,
]


def failing_pins(orc):
    """Names of the pins that fail (or raise) for the given oracle."""
    import warnings

    failed = []
    for pin in PINS:
        try:
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                with np.errstate(all="ignore"):
                    pin(orc)
        except Exception as exc:  # noqa: BLE001 -- any failure counts
            failed.append((pin.__name__, f"{type(exc).__name__}: {str(exc)[:160]}"))
    return failed

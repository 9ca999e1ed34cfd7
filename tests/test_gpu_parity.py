"""GPU parity: the HIP library (through the C ABI binding) against the float64
oracle, element by element, on the same seeded inputs.

Tolerances (max abs over all compared elements): fp32 inputs 1e-5 for o and
lse; bf16 inputs 2e-2 for o and 1e-3 for lse; empty rows exactly o = 0 and
lse = -inf.  Every workload is compared in full: the full-size prefill,
long-context and decode workloads too, in the launch configuration the
benchmark times (the oracle runs head by head on host threads).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import pins
from tests.parity_util import TOL, compare, compare_every_head, f64, oracle_full, say, scale32

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_05_amd as fa

    fa.lib()
    return torch.device("cuda:0")


def run_fwd(inp, dev, block_n=None):
    import online_softmax_05_amd as fa

    d = workloads.to_device(inp, dev)
    o, lse = fa.fa_fwd(d["q"], d["k"], d["v"], bias=d.get("bias"), k_len=d.get("k_len"), scale=inp["scale"],
                       causal=inp["causal"], block_n=inp.get("block_n", 0) if block_n is None else block_n)
    torch.cuda.synchronize()
    return o, lse


# ---------------------------------------------------------------------------
# the pages' worked examples, through the GPU
# ---------------------------------------------------------------------------

GOLDEN_CASES = ["gs_sec2_tile_local_counterexample.json", "gs_sec4_rescale_both.json", "vw_step6_row0.json",
                "oa_fig1_weighted_sum_first.json", "oa_fig2_chunk_states.json", "oa_fig3_two_queries.json"]


@pytest.mark.parametrize("name", GOLDEN_CASES)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_worked_examples(dev, name, dt):
    fx = pins.load_golden(name)
    dtype = DT[dt]
    q = torch.tensor(fx["q"], dtype=torch.float32)[None, None].to(dtype)
    k = torch.tensor(fx["k"], dtype=torch.float32)[None, None].to(dtype)
    v = torch.tensor(fx["v"], dtype=torch.float32)[None, None].to(dtype)
    inp = dict(q=q, k=k, v=v, bias=None, k_len=None, causal=False, scale=float(fx["scale"]))
    say(f"worked example {name} {dt}")
    for bn in (32, 64, 128):
        o, lse = run_fwd(inp, dev, block_n=bn)
        o_ref, lse_ref = oracle_full(inp)
        compare(o, lse, o_ref, lse_ref, dtype, f"{name} {dt} block_n={bn}")
    if dt == "f32":
        # the page's printed output, at the printed precision
        want = np.asarray(fx["expected"]["o"], dtype=np.float64).reshape(o_ref.shape[2:])
        assert np.max(np.abs(f64(o)[0, 0] - want)) <= fx["tolerance"] + 1e-5


# ---------------------------------------------------------------------------
# the pages' CPU-check shape families, run on the GPU
# ---------------------------------------------------------------------------

FAMILY_CASES = [
    # (Nq, Nk, dk, dv, causal, k_len)
    (5, 9, 4, 3, False, None),
    (7, 7, 5, 2, True, None),
    (2, 6, 1, 1, True, None),
    (5, 2, 1, 1, True, None),     # Nq > Nk: rows 0-2 empty
    (2, 4, 3, 2, True, [1]),
    (4, 7, 3, 4, True, [0]),      # padded-away sequence: every row empty
    (4, 7, 3, 4, False, [5]),
    (2, 0, 3, 2, False, None),    # empty key axis
    (1, 5, 1, 1, False, None),
    (1, 5, 1, 2, False, None),
    (3, 6, 4, 3, False, None),
]


@pytest.mark.parametrize("case", FAMILY_CASES, ids=lambda c: "x".join(map(str, c[:4])) + ("c" if c[4] else ""))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_page_families(dev, case, dt):
    nq, nk, dk, dv, causal, k_len = case
    inp = workloads.seeded_case(1000 + nq * 100 + nk, 1, 1, nq, nk, dk, dv, DT[dt], causal=causal,
                                bias=False, k_len=k_len)
    say(f"family {case} {dt}")
    o, lse = run_fwd(inp, dev)
    o_ref, lse_ref = oracle_full(inp)
    compare(o, lse, o_ref, lse_ref, DT[dt], f"family {case} {dt}")


def test_wide_logit_span(dev):
    """Large common shifts and a wide span of finite logits, through the bias."""
    bias = torch.tensor([0.0, 40.0, -40.0, 39.5, 1.0], dtype=torch.float32).repeat(3, 1)
    bias[1] += 1000.0
    bias[2] -= 2000.0
    for dt in ("f32", "bf16"):
        inp = workloads.seeded_case(77, 1, 1, 3, 5, 2, 2, DT[dt])
        inp["bias"] = bias[None, None].clone()
        say(f"wide logit span {dt}")
        o, lse = run_fwd(inp, dev)
        o_ref, lse_ref = oracle_full(inp)
        tol_lse = 1e-5 if dt == "f32" else 1e-3
        # lse is ~2000 in magnitude here: compare it relative to its size
        assert np.max(np.abs(f64(lse) - lse_ref) / np.maximum(1.0, np.abs(lse_ref))) <= tol_lse
        assert np.max(np.abs(f64(o) - o_ref)) <= TOL[DT[dt]]["o"]


# ---------------------------------------------------------------------------
# the small and masks workloads, compared in full
# ---------------------------------------------------------------------------

def test_small_workload_all_tiles(dev):
    inp = workloads.small()
    o_ref, lse_ref = oracle_full(inp)
    outs = []
    for bn in (64, 32, 128):
        say(f"small workload fp32 block_n={bn}")
        o, lse = run_fwd(inp, dev, block_n=bn)
        compare(o, lse, o_ref, lse_ref, torch.float32, f"small block_n={bn}")
        outs.append((f64(o), f64(lse)))
    # tile-size invariance beyond the oracle check
    for o, lse in outs[1:]:
        assert np.max(np.abs(o - outs[0][0])) <= 2e-6
        assert np.max(np.abs(lse - outs[0][1])) <= 2e-6


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_masks_workload(dev, dt):
    inp = workloads.masks(DT[dt])
    say(f"masks workload {dt}, k_len={inp['k_len'].tolist()}")
    o_ref, lse_ref = oracle_full(inp)
    assert np.all(np.isneginf(lse_ref[0])), "sequence 0 (k_len = 0) must be all empty rows"
    for bn in (0, 32, 128):
        o, lse = run_fwd(inp, dev, block_n=bn)
        compare(o, lse, o_ref, lse_ref, DT[dt], f"masks {dt} block_n={bn}")
    # equal-logit rows: the plain mean of the visible values ([VW] Step 7)
    v = f64(inp["v"])
    klen = inp["k_len"].tolist()
    nq = nk = workloads.SHAPES["masks"]["Nq"]
    og = f64(o)
    for b in range(2):
        for i in inp["equal_rows"].tolist():
            cnt = min(klen[b], i + nk - nq + 1)
            for h in range(4):
                if cnt <= 0:
                    assert np.all(og[b, h, i] == 0.0)
                else:
                    mean = v[b, h, :cnt].mean(axis=0)
                    assert np.max(np.abs(og[b, h, i] - mean)) <= TOL[DT[dt]]["o"]


# ---------------------------------------------------------------------------
# seeded sweep over ragged shapes, head dims, masks and dtypes
# ---------------------------------------------------------------------------

def _sweep_cases():
    rng = np.random.default_rng(2024)
    cases = []
    dims = [(128, 128), (64, 64), (128, 64), (64, 128), (32, 32), (8, 16), (100, 72), (1, 1), (3, 5), (96, 128)]
    for n in range(30):
        dk, dv = dims[n % len(dims)]
        nq = int(rng.choice([1, 7, 31, 32, 33, 127, 128, 129, 200, 300, 513]))
        nk = int(rng.choice([0, 1, 5, 63, 64, 65, 130, 257, 400, 700]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        causal = bool(rng.integers(0, 2))
        bias = bool(rng.integers(0, 2))
        kl = [None, "random"][int(rng.integers(0, 2))]
        dt = ["f32", "bf16"][n % 2]
        bn = [0, 32, 64, 128][int(rng.integers(0, 4))]
        cases.append((n, B, H, nq, nk, dk, dv, dt, causal, bias, kl, bn))
    return cases


GENERAL_MULTI_TILE = [
    # (Nq, Nk, dk, dv, causal, block_n): no bias, several key tiles, block
    # widths the fast bf16 kernel does not take, so the general kernels run
    (200, 200, 64, 64, True, 32), (200, 200, 64, 64, False, 32), (64, 200, 64, 64, False, 128),
    (333, 517, 128, 128, True, 128), (517, 333, 128, 96, True, 32), (130, 700, 32, 64, False, 32),
]


@pytest.mark.parametrize("case", GENERAL_MULTI_TILE, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_general_kernels_no_bias_multi_tile(dev, case, dt):
    """Regression: the no-bias general kernels over several key tiles, with
    masked elements in the first accumulator slot of a tile."""
    nq, nk, dk, dv, causal, bn = case
    inp = workloads.seeded_case(6000 + nq + nk, 2, 2, nq, nk, dk, dv, DT[dt], causal=causal)
    say(f"general no-bias multi-tile {case} {dt}")
    o, lse = run_fwd(inp, dev, block_n=bn)
    o_ref, lse_ref = oracle_full(inp)
    compare(o, lse, o_ref, lse_ref, DT[dt], f"general no-bias {case} {dt}")


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: f"s{c[0]}")
def test_seeded_sweep(dev, case):
    n, B, H, nq, nk, dk, dv, dt, causal, bias, kl, bn = case
    inp = workloads.seeded_case(5000 + n, B, H, nq, nk, dk, dv, DT[dt], causal=causal, bias=bias, k_len=kl)
    say(f"sweep {case} k_len={None if inp['k_len'] is None else inp['k_len'].tolist()}")
    o, lse = run_fwd(inp, dev, block_n=bn)
    o_ref, lse_ref = oracle_full(inp)
    compare(o, lse, o_ref, lse_ref, DT[dt], f"sweep {n}")


# (B, H, Nq, Nk, causal): grids of the fast bf16 kernel whose (batch, head)
# count is not a multiple of 8 or of the tile group (4 for causal grids of
# 64 or more blocks, else 2; 1 above 2 MiB of K/V per block), so that the
# last group holds 1, 2 or 3 blocks
FAST_GRIDS = [
    (1, 3, 600, 4200, True),   # 3 blocks of 2.05 MiB K/V: one block at a time
    (13, 5, 300, 300, True),   # 65 blocks, groups of 4, last group 1
    (3, 22, 520, 520, True),   # 66 blocks, groups of 4, last group 2
    (1, 67, 129, 129, True),   # 67 blocks, groups of 4, last group 3
    (7, 9, 200, 333, True),    # 63 blocks, pairs, last group 1
    (5, 13, 257, 600, False),  # 65 blocks, pairs (no causal mask), last group 1
]


@pytest.mark.parametrize("case", FAST_GRIDS, ids=lambda c: "x".join(map(str, c)))
def test_fast_kernel_odd_grids(dev, case):
    """Every (batch, head, query tile) of the fast kernel's grid is computed
    once, whatever the grouping of its blocks."""
    B, H, nq, nk, causal = case
    inp = workloads.seeded_case(7000 + B * H + nq, B, H, nq, nk, 128, 128, torch.bfloat16, causal=causal,
                                k_len="random")
    say(f"fast kernel grid {case}")
    o, lse = run_fwd(inp, dev)
    o_ref, lse_ref = oracle_full(inp)
    compare(o, lse, o_ref, lse_ref, torch.bfloat16, f"fast grid {case}")


# (B, H, Nq, Nk, dk, dv, causal, align): launches the fast bf16 kernel runs
# with eight waves (256 query rows) per work-group -- no left window, no
# bias, no dropout and at least 512 such work-groups -- with ragged query
# and key counts, random key lengths, both head dims and both causal
# alignments (top-left through fa_fwd_ex)
EIGHT_WAVE_CASES = [
    (2, 256, 300, 300, 128, 128, True, None),      # 2 query tiles per head, the second ragged
    (1, 512, 257, 400, 64, 128, False, None),      # one row past the first tile
    (4, 128, 200, 520, 128, 64, True, None),       # 512 work-groups of 200 rows
    (2, 256, 300, 260, 64, 64, True, "top_left"),  # Nq > Nk, top-left causal
]


@pytest.mark.parametrize("case", EIGHT_WAVE_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"_{c[6]}_{c[7]}")
def test_fast_kernel_eight_waves(dev, case):
    import online_softmax_05_amd as fa

    B, H, nq, nk, dk, dv, causal, align = case
    inp = workloads.seeded_case(7100 + H + nq + dk, B, H, nq, nk, dk, dv, torch.bfloat16, causal=causal,
                                k_len="random")
    say(f"fast kernel, eight waves {case}")
    d = workloads.to_device(inp, dev)
    if align is None:
        o, lse = fa.fa_fwd(d["q"], d["k"], d["v"], k_len=d["k_len"], scale=inp["scale"], causal=causal)
    else:
        o, lse = fa.fa_fwd_ex(d["q"], d["k"], d["v"], k_len=d["k_len"], scale=inp["scale"], causal=causal,
                              align=align, window_left=None, window_right=None)
        inp.update(align=align, window_left=None, window_right=None)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(inp)
    compare(o, lse, o_ref, lse_ref, torch.bfloat16, f"eight waves {case}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 1e-3, 3.0])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_scale_values(dev, scale, dt):
    """Negative, zero, tiny and large logit scales (the kernels keep their
    exponent scale positive by flipping the sign of Q)."""
    for use_bias in (False, True):
        inp = workloads.seeded_case(int(abs(scale) * 1000) + 3, 2, 2, 150, 140, 64, 64, DT[dt], causal=True,
                                    bias=use_bias, k_len=[140, 77])
        inp["scale"] = scale
        say(f"scale={scale} {dt} bias={use_bias}")
        o, lse = run_fwd(inp, dev)
        o_ref, lse_ref = oracle_full(inp)
        # logits here are up to |scale| sqrt(dk) times the standard scaling's
        compare(o, lse, o_ref, lse_ref, DT[dt], f"scale={scale} {dt} bias={use_bias}",
                logit_scale=max(1.0, abs(scale) * math.sqrt(64)))


def test_k_len_clamped(dev):
    """k_len outside [0, Nk] is clamped by the kernels."""
    inp = workloads.seeded_case(31, 3, 2, 40, 50, 64, 64, torch.bfloat16, causal=False, k_len=[-5, 77, 20])
    say("k_len clamp")
    o, lse = run_fwd(inp, dev)
    ref = dict(inp)
    ref["k_len"] = torch.tensor([0, 50, 20], dtype=torch.int32)
    o_ref, lse_ref = oracle_full(ref)
    compare(o, lse, o_ref, lse_ref, torch.bfloat16, "k_len clamp")


def test_run_to_run_bitwise(dev):
    inp = workloads.seeded_case(4242, 2, 3, 300, 333, 128, 128, torch.bfloat16, causal=True, bias=True,
                                k_len="random")
    say("determinism")
    o1, l1 = run_fwd(inp, dev)
    o2, l2 = run_fwd(inp, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_lse_optional_and_out_reuse(dev):
    import online_softmax_05_amd as fa

    inp = workloads.seeded_case(99, 1, 2, 65, 70, 64, 64, torch.float32, causal=True)
    d = workloads.to_device(inp, dev)
    say("lse optional")
    o1, _ = fa.fa_fwd(d["q"], d["k"], d["v"], causal=True, want_lse=False)
    out = torch.full_like(o1, float("nan"))
    o2, l2 = fa.fa_fwd(d["q"], d["k"], d["v"], causal=True, out=out)
    torch.cuda.synchronize()
    assert o2.data_ptr() == out.data_ptr()
    assert torch.equal(o1, o2)


# ---------------------------------------------------------------------------
# full-size prefill and long-context workloads: every output element
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["prefill", "long"])
def test_full_size_every_row(dev, name):
    import online_softmax_05_amd as fa

    say(f"{name}: drawing inputs on the device")
    inp = getattr(workloads, name)(dev)
    say(f"{name}: fa_fwd (the benchmark's launch configuration)")
    o, lse = fa.fa_fwd(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True, block_n=inp["block_n"])
    torch.cuda.synchronize()
    say(f"{name}: oracle on every row of every head")
    compare_every_head(o, lse, inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True,
                       what=f"{name} full size")
    # row 0 sees exactly key 0 (bottom-right causal, Nq == Nk): o = v_0, lse = s_00
    v0 = inp["v"][:, :, 0, :].float()
    assert torch.max(torch.abs(o[:, :, 0, :].float() - v0)).item() <= 1e-2
    s00 = (inp["q"][:, :, 0, :].float() * inp["k"][:, :, 0, :].float()).sum(-1) * scale32(inp["scale"])
    assert torch.max(torch.abs(lse[:, :, 0] - s00)).item() <= 1e-3
    del inp, o, lse
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# split-K decode
# ---------------------------------------------------------------------------

def _decode_oracle(q, k, v, k_len_host, pairs, scale):
    o = np.zeros((len(pairs), v.shape[3]))
    lse = np.zeros(len(pairs))
    for n, (b, h) in enumerate(pairs):
        kl = int(k_len_host[b])
        ob, lb = oracle.attention_head(f64(q[b, h][None]), f64(k[b, h, :kl]), f64(v[b, h, :kl]),
                                       scale=scale32(scale), nq=1, causal=False)
        o[n], lse[n] = ob[0], lb[0]
    return o, lse


def test_decode_full_size_every_row(dev):
    import online_softmax_05_amd as fa

    say("decode: drawing inputs on the device")
    inp = workloads.decode(dev)
    say("decode: fa_decode_splitk (the benchmark's launch configuration)")
    o, lse = fa.fa_decode_splitk(inp["q"], inp["k"], inp["v"], inp["k_len"], scale=inp["scale"],
                                 chunk=inp["chunk"])
    torch.cuda.synchronize()
    say("decode: oracle on every (sequence, head)")
    compare_every_head(o[:, :, None], lse[:, :, None], inp["q"][:, :, None], inp["k"], inp["v"],
                       scale=inp["scale"], causal=False, k_len_host=inp["k_len_host"], what="decode full size")
    del inp, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [64, 512, 2048])
def test_decode_small_full(dev, dt, chunk):
    import online_softmax_05_amd as fa

    g = torch.Generator().manual_seed(chunk)
    B, H, Nk, dk, dv = 5, 3, 1500, 128, 64
    q = torch.randn(B, H, dk, generator=g).to(DT[dt])
    k = torch.randn(B, H, Nk, dk, generator=g).to(DT[dt])
    v = torch.randn(B, H, Nk, dv, generator=g).to(DT[dt])
    k_len = torch.tensor([0, 1, 700, 1500, 9999], dtype=torch.int32)
    scale = 1.0 / math.sqrt(dk)
    say(f"decode small {dt} chunk={chunk}")
    o, lse = fa.fa_decode_splitk(q.to(dev), k.to(dev), v.to(dev), k_len.to(dev), scale=scale, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(f64(q)[:, :, None], f64(k), f64(v), scale=scale32(scale),
                                          k_len=np.clip(k_len.numpy(), 0, Nk))
    compare(o[:, :, None], lse[:, :, None], o_ref, lse_ref, DT[dt], f"decode {dt} chunk={chunk}")


@pytest.mark.parametrize("chunk", [64, 512, 2048])
def test_decode_fast_path_lengths(dev, chunk):
    """dk = dv = 128 bf16 (the single-pass partial kernel): lengths at and
    around the 16-row steps, the 4-wave quarters and the chunk edges."""
    import online_softmax_05_amd as fa

    g = torch.Generator().manual_seed(900 + chunk)
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1000, 2047, 2048, 2049, 2500]
    B, H, Nk, d = len(lens), 2, 2500, 128
    q = torch.randn(B, H, d, generator=g).to(torch.bfloat16)
    k = (torch.randn(B, H, Nk, d, generator=g) * 2.0).to(torch.bfloat16)
    v = torch.randn(B, H, Nk, d, generator=g).to(torch.bfloat16)
    k_len = torch.tensor(lens, dtype=torch.int32)
    scale = 1.0 / math.sqrt(d)
    say(f"decode fast path chunk={chunk}")
    o, lse = fa.fa_decode_splitk(q.to(dev), k.to(dev), v.to(dev), k_len.to(dev), scale=scale, chunk=chunk)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(f64(q)[:, :, None], f64(k), f64(v), scale=scale32(scale),
                                          k_len=k_len.numpy())
    compare(o[:, :, None], lse[:, :, None], o_ref, lse_ref, torch.bfloat16, f"decode fast chunk={chunk}")


@pytest.mark.parametrize("dt,dims", [("bf16", (128, 128)), ("f32", (64, 24)), ("bf16", (40, 1))])
def test_decode_many_chunks(dev, dt, dims):
    """More than 64 chunk states per row (the merge takes them 64 at a time)
    and head dims below the wave width."""
    import online_softmax_05_amd as fa

    dk, dv = dims
    g = torch.Generator().manual_seed(4000 + dk + dv)
    lens = [4095, 4096, 4097, 4160, 8191]
    B, H, Nk = len(lens), 2, 8191
    q = torch.randn(B, H, dk, generator=g).to(DT[dt])
    k = torch.randn(B, H, Nk, dk, generator=g).to(DT[dt])
    v = torch.randn(B, H, Nk, dv, generator=g).to(DT[dt])
    k_len = torch.tensor(lens, dtype=torch.int32)
    scale = 1.0 / math.sqrt(dk)
    say(f"decode many chunks {dt} dims={dims}")
    o, lse = fa.fa_decode_splitk(q.to(dev), k.to(dev), v.to(dev), k_len.to(dev), scale=scale, chunk=64)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(f64(q)[:, :, None], f64(k), f64(v), scale=scale32(scale),
                                          k_len=k_len.numpy())
    compare(o[:, :, None], lse[:, :, None], o_ref, lse_ref, DT[dt], f"decode many chunks {dt} dims={dims}")


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (40, 24), (1, 1)])
def test_decode_matches_fwd_nq1(dev, dims):
    """Decode equals the prefill kernel with one query row (causal is a no-op
    there) and both equal the oracle."""
    import online_softmax_05_amd as fa

    dk, dv = dims
    g = torch.Generator().manual_seed(dk * 1000 + dv)
    B, H, Nk = 3, 2, 777
    q = torch.randn(B, H, 1, dk, generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, Nk, dk, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, Nk, dv, generator=g).to(torch.bfloat16)
    k_len = torch.tensor([777, 300, 64], dtype=torch.int32)
    say(f"decode vs fwd dims={dims}")
    qd, kd, vd, kl = q.to(dev), k.to(dev), v.to(dev), k_len.to(dev)
    od, ld = fa.fa_decode_splitk(qd[:, :, 0].contiguous(), kd, vd, kl, chunk=128)
    of, lf = fa.fa_fwd(qd, kd, vd, k_len=kl, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(f64(q), f64(k), f64(v), scale=scale32(1 / math.sqrt(dk)),
                                          k_len=k_len.numpy())
    compare(od[:, :, None], ld[:, :, None], o_ref, lse_ref, torch.bfloat16, f"decode dims={dims}")
    compare(of, lf, o_ref, lse_ref, torch.bfloat16, f"fwd Nq=1 dims={dims}")


def test_decode_empty_and_degenerate(dev):
    import online_softmax_05_amd as fa

    say("decode degenerate")
    q = torch.randn(2, 2, 64, device=dev).to(torch.bfloat16)
    k = torch.randn(2, 2, 0, 64, device=dev).to(torch.bfloat16)
    o, lse = fa.fa_decode_splitk(q, k, k, torch.tensor([0, 5], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # Nk = 0 prefill: o = 0, lse = -inf
    qq = torch.randn(1, 2, 9, 16, device=dev)
    kk = torch.randn(1, 2, 0, 16, device=dev)
    o, lse = fa.fa_fwd(qq, kk, kk)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))

"""Key rows at or past a sequence's key length are never read.

Every entry point that takes key lengths promises that rows j >= k_len[b] of
K and V are not read: a KV cache (or a padded key tensor) may hold anything
there.  Each test fills those rows with NaN (K) and with +inf, -inf and NaN
(V), and checks that

* the result equals, bit for bit, the same call on the same inputs with
  finite values in those rows (a masked key has weight exactly zero, and a
  row that is never read cannot contribute 0 * NaN), and
* the result matches the float64 oracle on the finite inputs at the usual
  tolerances (fp32: 1e-5; bf16: o 2e-2, lse 1e-3; empty rows exactly
  o = 0, lse = -inf).

The masked keys drop out of the softmax ([GS] section 6, key and padding
masks by global position; [VW] Step 7, a masked score contributes nothing).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity_util import compare, f64, oracle_full, say, scale32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_softmax_05_amd as fa

    fa.lib()
    return torch.device("cuda:0")


def poison(k, v, k_len):
    """Copies of k and v whose rows j >= k_len[b] hold NaN (k) and a cycle of
    +inf, -inf, NaN (v)."""
    kp, vp = k.clone(), v.clone()
    bad = torch.tensor([float("inf"), float("-inf"), float("nan")], dtype=torch.float32)
    for b, n in enumerate(k_len.tolist()):
        n = max(0, min(int(n), k.shape[2]))
        kp[b, :, n:] = float("nan")
        rows = vp.shape[2] - n
        if rows > 0:
            pat = bad[torch.arange(rows) % 3].to(vp.dtype)
            vp[b, :, n:] = pat[None, :, None].expand(vp.shape[1], rows, vp.shape[3])
    return kp, vp


FWD_CASES = [
    # (dtype, B, H, Nq, Nk, dk, dv, causal, block_n, k_len)
    (torch.bfloat16, 3, 2, 200, 330, 128, 128, True, 0, [330, 150, 7]),     # fast bf16 kernel
    (torch.bfloat16, 2, 2, 130, 260, 64, 128, False, 0, [100, 0]),          # fast bf16 kernel, d 64/128
    (torch.bfloat16, 2, 2, 130, 200, 128, 128, True, 32, [199, 61]),        # general bf16 kernel
    (torch.float32, 2, 2, 96, 150, 64, 64, False, 0, [150, 37]),            # fp32 kernel
]


@pytest.mark.parametrize("case", range(len(FWD_CASES)))
def test_fwd_tail_never_read(dev, case):
    import online_softmax_05_amd as fa

    dtype, B, H, Nq, Nk, dk, dv, causal, block_n, kl = FWD_CASES[case]
    inp = workloads.seeded_case(900 + case, B, H, Nq, Nk, dk, dv, dtype, causal=causal, k_len=kl)
    kp, vp = poison(inp["k"], inp["v"], inp["k_len"])
    say(f"fwd tail case {case}: {dtype} B {B} H {H} Nq {Nq} Nk {Nk} d {dk}/{dv} causal {causal} "
        f"block_n {block_n} k_len {kl}")
    d = workloads.to_device(inp, dev)
    kl_d = inp["k_len"].to(dev)
    o_c, l_c = fa.fa_fwd(d["q"], d["k"], d["v"], k_len=kl_d, scale=inp["scale"], causal=causal, block_n=block_n)
    o_p, l_p = fa.fa_fwd(d["q"], kp.to(dev), vp.to(dev), k_len=kl_d, scale=inp["scale"], causal=causal,
                         block_n=block_n)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_p) and torch.equal(l_c, l_p), "rows past k_len changed the result"
    o_ref, lse_ref = oracle_full(inp)
    compare(o_p, l_p, o_ref, lse_ref, dtype, f"fwd tail case {case}")


BWD_CASES = [
    (torch.bfloat16, 2, 2, 192, 256, 128, 128, True, [256, 97]),   # matrix-core backward
    (torch.float32, 2, 2, 70, 90, 64, 32, False, [41, 90]),        # general backward
]


@pytest.mark.parametrize("case", range(len(BWD_CASES)))
def test_bwd_tail_never_read(dev, case):
    import online_softmax_05_amd as fa

    dtype, B, H, Nq, Nk, dk, dv, causal, kl = BWD_CASES[case]
    inp = workloads.seeded_case(950 + case, B, H, Nq, Nk, dk, dv, dtype, causal=causal, k_len=kl)
    g = workloads.seeded_upstream(960 + case, B, H, Nq, dv, dtype)
    kp, vp = poison(inp["k"], inp["v"], inp["k_len"])
    say(f"bwd tail case {case}: {dtype} B {B} H {H} Nq {Nq} Nk {Nk} d {dk}/{dv} causal {causal} k_len {kl}")
    d = workloads.to_device(inp, dev)
    kl_d = inp["k_len"].to(dev)
    gd = g.to(dev)
    o, lse = fa.fa_fwd(d["q"], d["k"], d["v"], k_len=kl_d, scale=inp["scale"], causal=causal)
    clean = fa.fa_bwd(d["q"], d["k"], d["v"], o, gd, lse, k_len=kl_d, scale=inp["scale"], causal=causal)
    pois = fa.fa_bwd(d["q"], kp.to(dev), vp.to(dev), o, gd, lse, k_len=kl_d, scale=inp["scale"], causal=causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), clean, pois):
        assert not torch.isnan(b).any(), f"{name}: NaN from rows past k_len"
        assert torch.equal(a, b), f"{name}: rows past k_len changed the result"
    for b_, n in enumerate(kl):
        assert torch.all(pois[1][b_, :, n:] == 0) and torch.all(pois[2][b_, :, n:] == 0), \
            "dK, dV rows past k_len must be zero"
    # the oracle rebuilds P from the GPU forward's o and lse, as in the
    # backward parity tests; bounds relative to each gradient's largest
    # entry (fp32 2e-5, bf16 2e-2)
    ref = oracle.attention_bwd_ref(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(g),
                                   scale=scale32(inp["scale"]), causal=causal, k_len=inp["k_len"].numpy(),
                                   o=f64(o), lse=f64(lse))
    tol = 2e-2 if dtype == torch.bfloat16 else 2e-5
    for name, got, want in zip(("dq", "dk", "dv"), pois, ref):
        err = float(np.max(np.abs(f64(got) - want))) / max(float(np.max(np.abs(want))), 1e-30)
        say(f"bwd tail case {case} {name}: rel err {err:.3e} (tol {tol:.0e})")
        assert err <= tol, (name, err)


def _oracle_decode(q, k, v, k_len, scale, nq, causal):
    B, H = q.shape[:2]
    dv = v.shape[3]
    o = np.zeros((B, H, nq, dv))
    lse = np.full((B, H, nq), -np.inf)
    for b in range(B):
        n = int(k_len[b])
        for h in range(H):
            qb = f64(q[b, h]).reshape(nq, -1)
            ob, lb = oracle.attention_head(qb, f64(k[b, h, :n]), f64(v[b, h, :n]), scale=scale32(scale), nq=nq,
                                           causal=causal)
            o[b, h], lse[b, h] = ob, lb
    return o, lse


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_decode_tail_never_read(dev, dt):
    import online_softmax_05_amd as fa

    B, H, Nk, d = 4, 2, 1100, 128
    g = torch.Generator().manual_seed(970)
    q = torch.randn(B, H, d, generator=g).to(dt)
    k = torch.randn(B, H, Nk, d, generator=g).to(dt)
    v = torch.randn(B, H, Nk, d, generator=g).to(dt)
    kl = torch.tensor([1, 513, 0, 1037], dtype=torch.int32)
    kp, vp = poison(k, v, kl)
    say(f"decode tail {dt}: B {B} H {H} Nk {Nk} d {d} k_len {kl.tolist()}")
    o_c, l_c = fa.fa_decode_splitk(q.to(dev), k.to(dev), v.to(dev), kl.to(dev), chunk=512)
    o_p, l_p = fa.fa_decode_splitk(q.to(dev), kp.to(dev), vp.to(dev), kl.to(dev), chunk=512)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_p) and torch.equal(l_c, l_p), "cache rows past k_len changed the result"
    o_ref, lse_ref = _oracle_decode(q[:, :, None], k, v, kl.numpy(), 1 / np.sqrt(d), 1, False)
    compare(o_p, l_p, o_ref[:, :, 0], lse_ref[:, :, 0], dt, f"decode tail {dt}")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_decode_mq_tail_never_read(dev, dt):
    import online_softmax_05_amd as fa

    B, H, Nq, Nk, d = 4, 2, 4, 1100, 128
    g = torch.Generator().manual_seed(980)
    q = torch.randn(B, H, Nq, d, generator=g).to(dt)
    k = torch.randn(B, H, Nk, d, generator=g).to(dt)
    v = torch.randn(B, H, Nk, d, generator=g).to(dt)
    kl = torch.tensor([3, 517, 0, 1029], dtype=torch.int32)  # 517: mid-tile and past a chunk edge
    kp, vp = poison(k, v, kl)
    say(f"decode mq tail {dt}: B {B} H {H} Nq {Nq} Nk {Nk} d {d} k_len {kl.tolist()}")
    o_c, l_c = fa.fa_decode_splitk_mq(q.to(dev), k.to(dev), v.to(dev), kl.to(dev), causal=True, chunk=512)
    o_p, l_p = fa.fa_decode_splitk_mq(q.to(dev), kp.to(dev), vp.to(dev), kl.to(dev), causal=True, chunk=512)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_p) and torch.equal(l_c, l_p), "cache rows past k_len changed the result"
    o_ref, lse_ref = _oracle_decode(q, k, v, kl.numpy(), 1 / np.sqrt(d), Nq, True)
    compare(o_p, l_p, o_ref, lse_ref, dt, f"decode mq tail {dt}")

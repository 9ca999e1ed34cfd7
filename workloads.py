"""Seeded synthetic inputs for the attention workloads.

This module only draws inputs; it holds none of the attention arithmetic and
imports neither the oracle nor the HIP library, so both sides can be fed the
very same values.  Every workload is a fixed recipe (shapes, distributions,
seeds); the pages measure nothing on a public dataset, so nothing stands in
for one.

Workloads (sizes as [B, H, N, d]):

* ``small``       1x1, Nq=Nk=256, d=64, fp32 N(0,1), no mask, no bias,
                  scale 1/8, key tile 64.
* ``masks``       2x4, Nq=Nk=1024, dk=128, dv=64, fp32 or bf16; bottom-right
                  causal; k_len = [0, x] with x ~ U{0..1024} redrawn until
                  x % 64 != 0 (the boundary falls inside a key tile); bias
                  fp32 N(0,1); for every (b, h) the rows i = 0 mod 128 get a
                  zero query and a zero bias row, so all their logits are equal.
* ``prefill``     4x32, Nq=Nk=4096, d=128, bf16 N(0,1), causal, 1/sqrt(128).
* ``long``        1x16, Nq=Nk=16384, d=128, bf16, causal, Q and K ~ N(0, 4^2)
                  (logit std about 16, the running max rises often), V ~ N(0,1).
* ``decode``      64x32, one query token, Nk_max=8192, k_len ~ U{1..8192} per
                  sequence, d=128, bf16 N(0,1), split into 512-key chunks.
* ``decode_mq``   the decode caches and lengths with 4 query rows per
                  sequence (its last 4 positions, causal), q from seed 305,
                  split into 2048-key chunks (the fastest measured split for
                  this kernel: fewer end-of-chunk merges).
* ``backward``    the prefill Q, K, V plus an upstream gradient dLoss/dO
                  ~ N(0,1) from seed 203.
* ``window``      the prefill Q, K, V with a causal sliding window of 1024
                  keys (each row sees its own position and the 1023 before).
* ``dropout``     the prefill Q, K, V with dropout p = 0.1 (keep 230 of 256
                  byte values), mask seed 0x5EED.
* ``dropout_bwd`` the backward workload under that same dropout.

Workload k draws Q/K/V from seed k; bias, k_len and the special rows come
from a second generator seeded 100 + k.  Small workloads are drawn on the CPU
(torch's CPU generator) and copied to the device; the three large ones are
drawn directly on the device with torch's device generator, one batch entry
at a time, and any slice the CPU needs is copied back from the device.
"""

import math

import torch

SEEDS = {"small": 1, "masks": 2, "prefill": 3, "long": 4, "decode": 5}

SHAPES = {
    "small": dict(B=1, H=1, Nq=256, Nk=256, dk=64, dv=64),
    "masks": dict(B=2, H=4, Nq=1024, Nk=1024, dk=128, dv=64),
    "prefill": dict(B=4, H=32, Nq=4096, Nk=4096, dk=128, dv=128),
    "long": dict(B=1, H=16, Nq=16384, Nk=16384, dk=128, dv=128),
    "decode": dict(B=64, H=32, Nq=1, Nk=8192, dk=128, dv=128),
    "backward": dict(B=4, H=32, Nq=4096, Nk=4096, dk=128, dv=128),
    "decode_mq": dict(B=64, H=32, Nq=4, Nk=8192, dk=128, dv=128),
    "window": dict(B=4, H=32, Nq=4096, Nk=4096, dk=128, dv=128),
    "dropout": dict(B=4, H=32, Nq=4096, Nk=4096, dk=128, dv=128),
    "dropout_bwd": dict(B=4, H=32, Nq=4096, Nk=4096, dk=128, dv=128),
}

DESCRIPTIONS = {
    "small": "attention fwd 1x1x256x256 d64 fp32, no mask",
    "masks": "attention fwd 2x4x1024x1024 dk128 dv64, causal + key lengths + bias + equal-logit rows",
    "prefill": "attention fwd prefill 4x32x4096x4096 d128 bf16 causal",
    "long": "attention fwd long context 1x16x16384x16384 d128 bf16 causal, Q,K ~ N(0,16)",
    "decode": "split-K decode 64x32 queries, KV lengths U[1,8192], d128 bf16, 512-key chunks",
    "backward": "attention bwd (dQ, dK, dV by recomputation) 4x32x4096x4096 d128 bf16 causal, upstream gradient N(0,1)",
    "decode_mq": "split-K multi-query decode 64x32 sequences x 4 query rows (causal), KV lengths U[1,8192], d128 bf16, "
                 "2048-key chunks",
    "window": "attention fwd prefill 4x32x4096x4096 d128 bf16 causal, sliding window of 1024 keys",
    "dropout": "attention fwd prefill 4x32x4096x4096 d128 bf16 causal, dropout p=0.1 (keep 230/256)",
    "dropout_bwd": "attention bwd 4x32x4096x4096 d128 bf16 causal, dropout p=0.1 (keep 230/256) replayed",
}

DROPOUT = (230, 0x5EED)  # (keep_256, seed) of the dropout workloads


def _randn_cpu(gen, shape, std=1.0):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x * std if std != 1.0 else x


def _randn_dev(gen, shape, device, dtype, std=1.0):
    """Draw one batch entry at a time on the device (bounded fp32 temporaries)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    for b in range(shape[0]):
        x = torch.randn(shape[1:], generator=gen, dtype=torch.float32, device=device)
        if std != 1.0:
            x.mul_(std)
        out[b].copy_(x)
    return out


def small(dtype=torch.float32):
    s = SHAPES["small"]
    g = torch.Generator().manual_seed(SEEDS["small"])
    q = _randn_cpu(g, (s["B"], s["H"], s["Nq"], s["dk"])).to(dtype)
    k = _randn_cpu(g, (s["B"], s["H"], s["Nk"], s["dk"])).to(dtype)
    v = _randn_cpu(g, (s["B"], s["H"], s["Nk"], s["dv"])).to(dtype)
    return dict(q=q, k=k, v=v, bias=None, k_len=None, causal=False, scale=1.0 / 8.0, block_n=64)


def masks(dtype=torch.float32):
    s = SHAPES["masks"]
    B, H, Nq, Nk, dk, dv = (s[x] for x in ("B", "H", "Nq", "Nk", "dk", "dv"))
    g = torch.Generator().manual_seed(SEEDS["masks"])
    g2 = torch.Generator().manual_seed(100 + SEEDS["masks"])
    q = _randn_cpu(g, (B, H, Nq, dk))
    k = _randn_cpu(g, (B, H, Nk, dk))
    v = _randn_cpu(g, (B, H, Nk, dv))
    bias = _randn_cpu(g2, (B, H, Nq, Nk))
    while True:
        x = int(torch.randint(0, Nk + 1, (1,), generator=g2))
        if x % 64 != 0:
            break
    k_len = torch.tensor([0, x], dtype=torch.int32)
    eq_rows = torch.arange(0, Nq, 128)
    q[:, :, eq_rows, :] = 0.0
    bias[:, :, eq_rows, :] = 0.0
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), bias=bias, k_len=k_len, causal=True,
                scale=1.0 / math.sqrt(dk), block_n=0, equal_rows=eq_rows)


def prefill(device):
    s = SHAPES["prefill"]
    g = torch.Generator(device=device).manual_seed(SEEDS["prefill"])
    shp_q = (s["B"], s["H"], s["Nq"], s["dk"])
    q = _randn_dev(g, shp_q, device, torch.bfloat16)
    k = _randn_dev(g, (s["B"], s["H"], s["Nk"], s["dk"]), device, torch.bfloat16)
    v = _randn_dev(g, (s["B"], s["H"], s["Nk"], s["dv"]), device, torch.bfloat16)
    return dict(q=q, k=k, v=v, bias=None, k_len=None, causal=True, scale=1.0 / math.sqrt(128), block_n=0)


def window(device):
    """The prefill workload's Q, K, V (same seed, same draws) under a causal
    sliding window of 1024 keys (left width 1023)."""
    inp = prefill(device)
    inp["window_left"] = 1023
    return inp


def dropout(device):
    """The prefill workload's Q, K, V (same seed, same draws) with dropout
    (keep_256, seed) = DROPOUT."""
    inp = prefill(device)
    inp["dropout"] = DROPOUT
    return inp


def dropout_bwd(device):
    """The backward workload under the dropout workload's mask."""
    inp = backward(device)
    inp["dropout"] = DROPOUT
    return inp


def backward(device):
    """The prefill workload's Q, K, V (same seed, same draws) plus an upstream
    gradient dLoss/dO ~ N(0, 1) from a second generator (seed 200 + the
    prefill seed)."""
    inp = prefill(device)
    s = SHAPES["backward"]
    g = torch.Generator(device=device).manual_seed(200 + SEEDS["prefill"])
    inp["g"] = _randn_dev(g, (s["B"], s["H"], s["Nq"], s["dv"]), device, torch.bfloat16)
    return inp


def long(device):
    s = SHAPES["long"]
    g = torch.Generator(device=device).manual_seed(SEEDS["long"])
    q = _randn_dev(g, (s["B"], s["H"], s["Nq"], s["dk"]), device, torch.bfloat16, std=4.0)
    k = _randn_dev(g, (s["B"], s["H"], s["Nk"], s["dk"]), device, torch.bfloat16, std=4.0)
    v = _randn_dev(g, (s["B"], s["H"], s["Nk"], s["dv"]), device, torch.bfloat16)
    return dict(q=q, k=k, v=v, bias=None, k_len=None, causal=True, scale=1.0 / math.sqrt(128), block_n=0)


def decode(device):
    s = SHAPES["decode"]
    B, H, Nk, dk, dv = (s[x] for x in ("B", "H", "Nk", "dk", "dv"))
    g = torch.Generator(device=device).manual_seed(SEEDS["decode"])
    g2 = torch.Generator().manual_seed(100 + SEEDS["decode"])
    q = _randn_dev(g, (B, H, dk), device, torch.bfloat16)
    k = _randn_dev(g, (B, H, Nk, dk), device, torch.bfloat16)
    v = _randn_dev(g, (B, H, Nk, dv), device, torch.bfloat16)
    k_len = torch.randint(1, Nk + 1, (B,), generator=g2, dtype=torch.int64).to(torch.int32)
    return dict(q=q, k=k, v=v, k_len=k_len.to(device), k_len_host=k_len, scale=1.0 / math.sqrt(dk),
                chunk=512)


def decode_mq(device):
    """The decode workload's caches and lengths (same seeds, same draws) with
    4 query rows per sequence from a second device generator (seed
    300 + the decode seed), split into 2048-key chunks."""
    inp = decode(device)
    s = SHAPES["decode_mq"]
    g = torch.Generator(device=device).manual_seed(300 + SEEDS["decode"])
    inp["q"] = _randn_dev(g, (s["B"], s["H"], s["Nq"], s["dk"]), device, torch.bfloat16)
    inp["chunk"] = 2048
    return inp


def long_cache(device, Nk=9_000_000, nq=4, seed=17):
    """One sequence and head whose K and V caches each span more than 2^31
    bytes (9e6 keys of d = 128 in bf16: 2.3 GB each), drawn on the device:
    q [1,1,nq,128] and caches [1,1,Nk,128] ~ N(0, 1), the key length 3 keys
    short of Nk."""
    g = torch.Generator(device=device).manual_seed(seed)
    q = _randn_dev(g, (1, 1, nq, 128), device, torch.bfloat16)
    k = _randn_dev(g, (1, 1, Nk, 128), device, torch.bfloat16)
    v = _randn_dev(g, (1, 1, Nk, 128), device, torch.bfloat16)
    k_len = torch.tensor([Nk - 3], dtype=torch.int32)
    return dict(q=q, k=k, v=v, k_len=k_len, scale=1.0 / math.sqrt(128))


def to_device(inputs, device):
    """Copy every tensor of a CPU-drawn workload to ``device``."""
    out = {}
    for key, val in inputs.items():
        out[key] = val.to(device) if isinstance(val, torch.Tensor) and key != "equal_rows" else val
    return out


def seeded_upstream(seed, B, H, Nq, dv, dtype):
    """A seeded upstream gradient dLoss/dO ~ N(0, 1) of shape [B,H,Nq,dv] (CPU),
    from its own generator (seed 200 + seed)."""
    g = torch.Generator().manual_seed(200 + seed)
    return _randn_cpu(g, (B, H, Nq, dv)).to(dtype)


def seeded_case(seed, B, H, Nq, Nk, dk, dv, dtype, *, causal=False, bias=False, k_len=None, q_std=1.0,
                k_std=1.0):
    """A small seeded case of arbitrary shape (CPU), for parity sweeps.
    ``k_len``: None, a list, or "random" (U{0..Nk} per sequence)."""
    g = torch.Generator().manual_seed(seed)
    q = _randn_cpu(g, (B, H, Nq, dk), q_std).to(dtype)
    k = _randn_cpu(g, (B, H, Nk, dk), k_std).to(dtype)
    v = _randn_cpu(g, (B, H, Nk, dv)).to(dtype)
    bt = _randn_cpu(g, (B, H, Nq, Nk)) if bias else None
    if isinstance(k_len, str) and k_len == "random":
        k_len = torch.randint(0, Nk + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    elif k_len is not None:
        k_len = torch.tensor(k_len, dtype=torch.int32)
    return dict(q=q, k=k, v=v, bias=bt, k_len=k_len, causal=causal, scale=1.0 / math.sqrt(dk), block_n=0)

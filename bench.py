"""Benchmark of the attention forward library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload prefill|long|decode|decode_mq|backward|window|dropout|dropout_bwd|
                                small|masks_f32|masks_bf16]
                    [--no-cpu-baseline] [--only] [--copy-calibration]

A step is one pass of the hot path over one batch of synthetic input that is
already resident in device memory: one fa_fwd call for the prefill and
long-context workloads, one fa_fwd_ex call for the sliding-window prefill, one fa_decode_splitk call (partial + merge kernels)
for decode, one fa_decode_splitk_mq call for the multi-query decode, one
fa_bwd call (dQ then dK/dV kernels; O and lse from one untimed fa_fwd) for
the backward workload, one fa_fwd call for the small (1x1x256^2 fp32) and
masks (2x4x1024^2 with key lengths, bias and causal, fp32 and bf16)
workloads.  W untimed steps, then exactly K timed steps between device
synchronisations; the JSON line on stdout reports the main workload
(default: causal bf16 prefill 4x32x4096^2, d=128) and, under "secondary",
every other workload measured the same way.

Algorithmic work (what the method must do, not what a kernel happens to do):
* prefill / long / window: FLOPs = 2 (dk + dv) x (number of allowed
  query-key pairs, under the window for the sliding-window workload);
  exponentials and maxima are not counted;
* backward: FLOPs = 2 (3 dk + 2 dv) x (allowed pairs): the five products
  S = QK^T, dP = G V^T, dV = P^T G, dK = D^T Q, dQ = D K ([GS] section 7);
  recomputing S and dP in both the dK/dV and the dQ kernel is not counted;
* decode: bytes = the K/V rows actually read (sum over sequences of
  H * k_len * (dk + dv) * 2) + q + o (2 bytes each) + lse (4 bytes); the
  split-K workspace is not counted; the multi-query decode counts the same
  K/V bytes plus Nq rows of q, o and lse;
* small / masks: FLOPs = 2 (dk + dv) x (allowed pairs, counted exactly from
  the causal and key-length masks) and bytes = Q + K + V + bias + O + lse;
  both are far too small to fill the GPU (launch latency dominates), and the
  roofline names the larger of the two ideal times (the bias read for masks);

roofline.achieved divides that work per launch by the kernel's mean duration
measured with HIP events recorded on the launch stream around every timed
launch (the minimum and median launch durations are reported beside it).
roofline.traffic comes from a stored rocprofv3 counter summary
(profiles/<workload>_traffic.json), and roofline.clock_ghz, frac_at_clock and
mfma_busy from another (profiles/<workload>_counters.json: GRBM_GUI_ACTIVE per
XCD over the dispatch duration, SQ_VALU_MFMA_BUSY_CYCLES over
GRBM_GUI_ACTIVE x 1024 SIMDs); each is reported only while the kernel
sources (their code: comments and whitespace are not hashed) still hash to
the value recorded with it.  frac_at_clock is achieved
over the dense peak at that measured clock (256 CU x 4096 FLOP/clk x clock).

cpu_baseline times the float64 oracle (test infrastructure, used here only
for this leg) on a bounded sample of the same workload on the host cores;
max_abs_err compares the GPU outputs of the timed launches with the oracle on
that same sample (o and lse max-abs; gradients max-abs over the largest
reference entry).  The oracle samples run after every workload has been
timed, so that no host work overlaps a timed region.
"""

import argparse
import hashlib
import json
import math
import os
import pathlib
import platform
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk (dense bf16 MFMA) x 2.4 GHz (published 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0      # HBM3E, published 8 TB/s
PEAK_F32_MFMA_TFLOPS = 157.3  # dense fp32 matrix, published
METRIC = "attn fwd TFLOP/s (% bf16 MFMA peak) prefill; decode HBM GB/s (% peak)"
# sources of the kernel each workload's roofline describes (stored counter
# summaries are only reported while these still hash to the recorded value)
KERNEL_SOURCES = {
    "prefill": ["online_softmax_05_amd/csrc/fa_fwd_bf16_fast.hip", "online_softmax_05_amd/csrc/fa_common.h",
                "online_softmax_05_amd/csrc/fa_mask.h", "online_softmax_05_amd/csrc/fa_dropout.h"],
    "long": ["online_softmax_05_amd/csrc/fa_fwd_bf16_fast.hip", "online_softmax_05_amd/csrc/fa_common.h",
             "online_softmax_05_amd/csrc/fa_mask.h", "online_softmax_05_amd/csrc/fa_dropout.h"],
    "window": ["online_softmax_05_amd/csrc/fa_fwd_bf16_fast.hip", "online_softmax_05_amd/csrc/fa_common.h",
               "online_softmax_05_amd/csrc/fa_mask.h", "online_softmax_05_amd/csrc/fa_dropout.h"],
    "dropout": ["online_softmax_05_amd/csrc/fa_fwd_bf16_fast.hip", "online_softmax_05_amd/csrc/fa_common.h",
                "online_softmax_05_amd/csrc/fa_mask.h", "online_softmax_05_amd/csrc/fa_dropout.h"],
    "dropout_bwd": ["online_softmax_05_amd/csrc/fa_bwd.hip", "online_softmax_05_amd/csrc/fa_bwd_bf16.hip",
                    "online_softmax_05_amd/csrc/fa_tiles.h", "online_softmax_05_amd/csrc/fa_common.h",
                    "online_softmax_05_amd/csrc/fa_mask.h", "online_softmax_05_amd/csrc/fa_dropout.h"],
    "decode": ["online_softmax_05_amd/csrc/fa_decode.hip", "online_softmax_05_amd/csrc/fa_common.h",
               "online_softmax_05_amd/csrc/fa_merge.h"],
    "backward": ["online_softmax_05_amd/csrc/fa_bwd.hip", "online_softmax_05_amd/csrc/fa_bwd_bf16.hip",
                 "online_softmax_05_amd/csrc/fa_tiles.h", "online_softmax_05_amd/csrc/fa_common.h",
                 "online_softmax_05_amd/csrc/fa_mask.h", "online_softmax_05_amd/csrc/fa_dropout.h"],
    "decode_mq": ["online_softmax_05_amd/csrc/fa_decode_mq.hip", "online_softmax_05_amd/csrc/fa_tiles.h",
                  "online_softmax_05_amd/csrc/fa_common.h", "online_softmax_05_amd/csrc/fa_merge.h"],
}
# (the last template argument of the fast forward and of the dK/dV kernel is
# its waves per work-group)
KERNEL_NAMES = {"prefill": "fwd_bf16_fast_kernel<128, 128, false, false, 8>",
                "long": "fwd_bf16_fast_kernel<128, 128, false, false, 8>",
                "window": "fwd_bf16_fast_kernel<128, 128, false, false, 4>",
                "dropout": "fwd_bf16_fast_kernel<128, 128, false, true, 4>",
                "dropout_bwd": "bwd_dq_bf16_kernel<128, 128, false, true, 4> + bwd_dkdv_bf16_kernel<128, 128, false, true, 4>",
                "decode": "decode_partial_fast_kernel + decode_merge_kernel",
                "backward": "bwd_dq_bf16_kernel<128, 128, false, false, 8> + bwd_dkdv_bf16_kernel<128, 128, false, false, 8>",
                "decode_mq": "mq_partial_bf16_kernel + mq_merge_kernel"}


ALL_WORKLOADS = ("prefill", "long", "decode", "decode_mq", "backward", "window", "dropout", "dropout_bwd", "small",
                 "masks_f32", "masks_bf16")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _code_only(text):
    """C++ source with comments removed and whitespace runs collapsed, so
    that a stored record stays tied to the code, not to its comments."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":  # string or character literal: copied whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(name):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[name]:
        h.update(_code_only((ROOT / rel).read_text()).encode())
    return h.hexdigest()[:16]


def causal_pairs(nq, nk, window_left=None):
    """Allowed (query, key) pairs of one head under bottom-right causal,
    optionally limited to a left window of ``window_left`` keys before the
    row's own position."""
    total = 0
    for i in range(nq):
        end = max(0, min(nk, i + nk - nq + 1))
        lo = 0 if window_left is None else max(0, i + nk - nq - window_left)
        total += max(0, end - lo)
    return total


def _stored(name, kind):
    p = ROOT / "profiles" / f"{name}_{kind}.json"
    if not p.exists() or name not in KERNEL_SOURCES:
        return None
    rec = json.loads(p.read_text())
    if rec.get("kernel_source_hash") != kernel_source_hash(name):
        return None
    return rec


def stored_traffic(name):
    rec = _stored(name, "traffic")
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def traffic_source(name):
    """Where roofline.traffic comes from: it is not measured in this run."""
    if stored_traffic(name) is None:
        return None
    return (f"profiles/{name}_traffic.json: FETCH_SIZE + WRITE_SIZE of separate rocprofv3 --pmc runs of this "
            f"workload, scaled by a plain copy's readings; used because the kernel sources still hash to the "
            f"value recorded with it")


def clock_fields(name, achieved_tflops):
    """Measured shader clock and MFMA busy fraction from the stored counter
    record, and the fraction of the dense bf16 peak at that clock."""
    rec = _stored(name, "counters")
    if rec is None:
        return dict(clock_ghz=None, frac_at_clock=None, mfma_busy=None)
    ghz = rec["clock_ghz"]
    return dict(clock_ghz=ghz, frac_at_clock=achieved_tflops / (256 * 4096 * ghz * 1e-3),
                mfma_busy=rec.get("mfma_busy"))


def cpu_model():
    """The host CPU's model name, read from /proc/cpuinfo (no subprocess)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


def causal_pairs_klen(nq, nk, k_len):
    """Allowed pairs of one head under bottom-right causal and a key length."""
    total = 0
    for i in range(nq):
        total += max(0, min(k_len, i + nk - nq + 1))
    return total


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def time_launches(fn, steps, warmup):
    """W untimed calls, then K timed calls between synchronisations; events on
    the current stream around each call give the per-launch duration."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = sorted(s.elapsed_time(e) for s, e in ev)
    return dict(ms_per_step=wall * 1e3 / steps, launch_ms_mean=sum(durs) / len(durs),
                launch_ms_median=durs[len(durs) // 2], launch_ms_min=durs[0], launch_ms_max=durs[-1])


def launch_fields(t):
    return dict(launch_ms_mean=t["launch_ms_mean"], launch_ms_median=t["launch_ms_median"],
                launch_ms_min=t["launch_ms_min"], launch_ms_max=t["launch_ms_max"])


# ---------------------------------------------------------------------------
# CPU baseline (the oracle, on a bounded sample)
# ---------------------------------------------------------------------------

def blas_name():
    """The BLAS library numpy calls (threadpoolctl's view), e.g. "openblas 0.3.27"."""
    try:
        import numpy  # noqa: F401  (loads the BLAS library threadpoolctl looks for)
        from threadpoolctl import threadpool_info

        libs = [f"{d.get('internal_api')} {d.get('version')}" for d in threadpool_info() if d.get("user_api") == "blas"]
        return ", ".join(libs) if libs else None
    except Exception:  # noqa: BLE001
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def _err_acc():
    return dict(o=0.0, lse=0.0, rows=0)


def _err_update(acc, o_gpu, lse_gpu, o_ref, lse_ref):
    """Max-abs errors over nonempty rows; empty rows (lse_ref = -inf) must be
    exactly o = 0, lse = -inf, else the error is reported as infinite."""
    import numpy as np

    emp = np.isneginf(lse_ref)
    if emp.any() and not (np.all(o_gpu[emp] == 0.0) and np.all(np.isneginf(lse_gpu[emp]))):
        acc["o"] = acc["lse"] = float("inf")
    ne = ~emp
    if ne.any():
        acc["o"] = max(acc["o"], float(np.max(np.abs(o_gpu[ne] - o_ref[ne]))))
        acc["lse"] = max(acc["lse"], float(np.max(np.abs(lse_gpu[ne] - lse_ref[ne]))))
    acc["rows"] += int(o_ref.shape[0])


def cpu_baseline_prefill(inp, name, budget_s, out, lse):
    import numpy as np

    import oracle

    q, k, v = inp["q"], inp["k"], inp["v"]
    B, H, N, dk = q.shape
    dv = v.shape[3]
    scale = float(np.float32(inp["scale"]))
    wl = inp.get("window_left")
    flops = 0.0
    heads = 0
    err = _err_acc()
    elapsed = 0.0  # oracle time only; device-to-host copies of the inputs are excluded
    for bh in range(B * H):
        b, h = divmod(bh, H)
        qh = q[b, h].double().cpu().numpy()
        kh = k[b, h].double().cpu().numpy()
        vh = v[b, h].double().cpu().numpy()
        og = out[b, h].double().cpu().numpy()
        lg = lse[b, h].double().cpu().numpy()
        for r0 in range(0, N, 2048):
            r1 = min(N, r0 + 2048)
            ts = time.perf_counter()
            o_ref, l_ref = oracle.attention_head(qh[r0:r1], kh, vh, scale=scale, nq=N, causal=True,
                                                 row_ids=np.arange(r0, r1), window=(wl, None),
                                                 dropout=inp.get("dropout"), bh=bh)
            elapsed += time.perf_counter() - ts
            _err_update(err, og[r0:r1], lg[r0:r1], o_ref, l_ref)
        flops += 2.0 * (dk + dv) * causal_pairs(N, N, wl)
        heads += 1
        if elapsed >= budget_s:
            break
    return dict(value=flops / elapsed / 1e12, unit="TFLOP/s", cores=blas_threads(), blas=blas_name(), kind="oracle",
                sample=f"{heads} of {B * H} heads of the {name} workload, every query row, dense float64 "
                       f"numpy oracle, {elapsed:.1f} s of oracle time (input copies excluded)",
                seconds=elapsed, cpu=cpu_model()), err


def cpu_baseline_decode(inp, budget_s, out, lse, nq=1, name="decode"):
    import numpy as np

    import oracle

    q, k, v, kl = inp["q"], inp["k"], inp["v"], inp["k_len_host"]
    B, H = q.shape[0], q.shape[1]
    dk = q.shape[-1]
    dv = v.shape[3]
    scale = float(np.float32(inp["scale"]))
    nbytes = 0.0
    pairs = 0
    err = _err_acc()
    elapsed = 0.0  # oracle time only; device-to-host copies of the inputs are excluded
    for b in range(B):
        n = int(kl[b])
        kb = k[b, :, :n].double().cpu().numpy()
        vb = v[b, :, :n].double().cpu().numpy()
        qb = q[b].double().cpu().numpy().reshape(H, nq, dk)
        ob = out[b].double().cpu().numpy().reshape(H, nq, dv)
        lb = lse[b].double().cpu().numpy().reshape(H, nq)
        for h in range(H):
            ts = time.perf_counter()
            o_ref, l_ref = oracle.attention_head(qb[h], kb[h], vb[h], scale=scale, nq=nq, causal=nq > 1)
            elapsed += time.perf_counter() - ts
            _err_update(err, ob[h], lb[h], o_ref, l_ref)
            nbytes += n * (dk + dv) * 2 + nq * (dk * 2 + dv * 2 + 4)
            pairs += 1
        if elapsed >= budget_s:
            break
    return dict(value=nbytes / elapsed / 1e9, unit="GB/s", cores=blas_threads(), blas=blas_name(), kind="oracle",
                sample=f"{pairs} of {B * H} (sequence, head) pairs ({nq} query row{'s' if nq > 1 else ''} each) of "
                       f"the {name} workload, dense float64 numpy oracle, {elapsed:.1f} s of oracle time "
                       f"(input copies excluded)",
                seconds=elapsed, cpu=cpu_model()), err


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def _err_fields(err):
    return None if err is None else dict(o=err["o"], lse=err["lse"], rows_compared=err["rows"])


def run_prefill(name, args, dev):
    import torch

    import online_softmax_05_amd as fa
    import workloads

    log(f"{name}: drawing inputs on the device")
    inp = getattr(workloads, name)(dev)
    s = workloads.SHAPES[name]
    B, H, N, dk, dv = s["B"], s["H"], s["Nq"], s["dk"], s["dv"]
    out = torch.empty((B, H, N, dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

    wl = inp.get("window_left")
    keep, seed = inp.get("dropout") or (256, 0)

    def step():
        if wl is None and keep == 256:
            fa.fa_fwd(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True, block_n=inp["block_n"],
                      out=out, lse=lse)
        else:
            fa.fa_fwd_ex(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True, window_left=wl,
                         keep_256=keep, seed=seed, block_n=inp["block_n"], out=out, lse=lse)

    log(f"{name}: timing {args.warmup} + {args.steps} steps")
    t = time_launches(step, args.steps, args.warmup)
    pairs = B * H * causal_pairs(N, N, wl)
    flops = 2.0 * (dk + dv) * pairs
    value = flops / (t["ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (t["launch_ms_mean"] * 1e-3) / 1e12
    traffic = stored_traffic(name)
    res = dict(
        workload=workloads.DESCRIPTIONS[name], value=value, unit="TFLOP/s", ms_per_step=t["ms_per_step"],
        frac_of_peak=value / PEAK_BF16_TFLOPS,
        roofline=dict(bound="mfma", achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=achieved / PEAK_BF16_TFLOPS, traffic=traffic, traffic_source=traffic_source(name),
                      kernel=KERNEL_NAMES[name], **launch_fields(t), **clock_fields(name, achieved),
                      algorithmic_flops_per_launch=flops,
                      algorithmic_bytes_per_launch=2 * B * H * N * (2 * dk + dv) + 2 * B * H * N * dv
                      + 4 * B * H * N),
        config=dict(workload=workloads.DESCRIPTIONS[name], B=B, H=H, Nq=N, Nk=N, dk=dk, dv=dv, causal=True,
                    dtype="bf16", block_n=64 if inp["block_n"] == 0 else inp["block_n"],
                    allowed_pairs=pairs, **({} if wl is None else {"window_left": wl}),
                    **({} if keep == 256 else {"dropout_keep_256": keep, "dropout_seed": seed})),
    )
    def finish():
        if not args.no_cpu_baseline:
            log(f"{name}: timing the oracle on a bounded sample")
            res["cpu_baseline"], err = cpu_baseline_prefill(inp, name, args.cpu_budget, out, lse)
            res["cpu_baseline"]["value_same_unit_as_gpu"] = True
            res["max_abs_err"] = _err_fields(err)

    return res, finish


def cpu_baseline_backward(inp, budget_s, grads, name="backward"):
    import numpy as np

    import oracle

    q, k, v, g = inp["q"], inp["k"], inp["v"], inp["g"]
    B, H, N, dk = q.shape
    dv = v.shape[3]
    scale = float(np.float32(inp["scale"]))
    flops = 0.0
    heads = 0
    err = dict(dq=0.0, dk=0.0, dv=0.0)
    elapsed = 0.0  # oracle time only (it rebuilds its own forward); input copies excluded
    for bh in range(B * H):
        b, h = divmod(bh, H)
        qh, kh, vh, gh = (t[b, h].double().cpu().numpy() for t in (q, k, v, g))
        ts = time.perf_counter()
        ref = oracle.attention_bwd_head(qh, kh, vh, gh, scale=scale, nq=N, causal=True, dropout=inp.get("dropout"),
                                        bh=bh)
        elapsed += time.perf_counter() - ts
        for key, got, want in zip(("dq", "dk", "dv"), grads, ref):
            gg = got[b, h].double().cpu().numpy()
            err[key] = max(err[key], float(np.max(np.abs(gg - want))) / max(float(np.max(np.abs(want))), 1e-30))
        flops += 2.0 * (3 * dk + 2 * dv) * causal_pairs(N, N)
        heads += 1
        if elapsed >= budget_s:
            break
    return dict(value=flops / elapsed / 1e12, unit="TFLOP/s", cores=blas_threads(), blas=blas_name(), kind="oracle",
                sample=f"{heads} of {B * H} heads of the {name} workload, dense float64 numpy oracle "
                       f"(forward included), {elapsed:.1f} s of oracle time (input copies excluded)",
                seconds=elapsed, cpu=cpu_model()), dict(err, heads_compared=heads, kind="max abs / max |ref|")


def run_backward(args, dev, name="backward"):
    import torch

    import online_softmax_05_amd as fa
    import workloads

    log(f"{name}: drawing inputs on the device")
    inp = getattr(workloads, name)(dev)
    s = workloads.SHAPES[name]
    B, H, N, dk, dv = s["B"], s["H"], s["Nq"], s["dk"], s["dv"]
    keep, seed = inp.get("dropout") or (256, 0)
    o, lse = fa.fa_fwd_ex(inp["q"], inp["k"], inp["v"], scale=inp["scale"], causal=True, keep_256=keep, seed=seed)
    dq, dk_, dv_ = torch.empty_like(inp["q"]), torch.empty_like(inp["k"]), torch.empty_like(inp["v"])
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N) // 4, dtype=torch.float32, device=dev)

    def step():
        if keep == 256:
            fa.fa_bwd(inp["q"], inp["k"], inp["v"], o, inp["g"], lse, scale=inp["scale"], causal=True, dq=dq,
                      dk=dk_, dv=dv_, workspace=ws)
        else:
            fa.fa_bwd_ex(inp["q"], inp["k"], inp["v"], o, inp["g"], lse, scale=inp["scale"], causal=True,
                         keep_256=keep, seed=seed, dq=dq, dk=dk_, dv=dv_, workspace=ws)

    log(f"{name}: timing {args.warmup} + {args.steps} steps")
    t = time_launches(step, args.steps, args.warmup)
    pairs = B * H * causal_pairs(N, N)
    flops = 2.0 * (3 * dk + 2 * dv) * pairs
    value = flops / (t["ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (t["launch_ms_mean"] * 1e-3) / 1e12
    res = dict(
        workload=workloads.DESCRIPTIONS[name], value=value, unit="TFLOP/s", ms_per_step=t["ms_per_step"],
        frac_of_peak=value / PEAK_BF16_TFLOPS,
        roofline=dict(bound="mfma", achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=achieved / PEAK_BF16_TFLOPS, traffic=stored_traffic(name), traffic_source=traffic_source(name),
                      kernel=KERNEL_NAMES[name], **launch_fields(t), **clock_fields(name, achieved),
                      algorithmic_flops_per_launch=flops),
        config=dict(workload=workloads.DESCRIPTIONS[name], B=B, H=H, Nq=N, Nk=N, dk=dk, dv=dv, causal=True,
                    dtype="bf16", allowed_pairs=pairs,
                    **({} if keep == 256 else {"dropout_keep_256": keep, "dropout_seed": seed})),
    )
    def finish():
        if not args.no_cpu_baseline:
            log(f"{name}: timing the oracle on a bounded sample")
            res["cpu_baseline"], res["max_abs_err"] = cpu_baseline_backward(inp, args.cpu_budget, (dq, dk_, dv_),
                                                                            name)

    return res, finish


def run_decode_mq(args, dev):
    import torch

    import online_softmax_05_amd as fa
    import workloads

    log("decode_mq: drawing inputs on the device")
    inp = workloads.decode_mq(dev)
    s = workloads.SHAPES["decode_mq"]
    B, H, Nq, Nk, dk, dv = s["B"], s["H"], s["Nq"], s["Nk"], s["dk"], s["dv"]
    chunk = inp["chunk"]
    ws = torch.empty(fa.fa_decode_splitk_mq_workspace_bytes(B, H, Nq, Nk, dv, chunk) // 4, dtype=torch.float32,
                     device=dev)
    out = torch.empty((B, H, Nq, dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)

    def step():
        fa.fa_decode_splitk_mq(inp["q"], inp["k"], inp["v"], inp["k_len"], causal=True, scale=inp["scale"],
                               chunk=chunk, out=out, lse=lse, workspace=ws)

    log(f"decode_mq: timing {args.warmup} + {args.steps} steps")
    t = time_launches(step, args.steps, args.warmup)
    kl = inp["k_len_host"].long()
    nbytes = float(H * kl.sum().item() * (dk + dv) * 2 + B * H * Nq * (dk * 2 + dv * 2 + 4))
    value = nbytes / (t["ms_per_step"] * 1e-3) / 1e9
    achieved = nbytes / (t["launch_ms_mean"] * 1e-3) / 1e9
    res = dict(
        workload=workloads.DESCRIPTIONS["decode_mq"], value=value, unit="GB/s", ms_per_step=t["ms_per_step"],
        frac_of_peak=value / PEAK_HBM_GBS,
        roofline=dict(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s", frac=achieved / PEAK_HBM_GBS,
                      traffic=stored_traffic("decode_mq"), traffic_source=traffic_source("decode_mq"), kernel=KERNEL_NAMES["decode_mq"], **launch_fields(t),
                      algorithmic_bytes_per_launch=nbytes),
        config=dict(workload=workloads.DESCRIPTIONS["decode_mq"], B=B, H=H, Nq=Nq, Nk_max=Nk, dk=dk, dv=dv,
                    chunk=chunk, causal=True, dtype="bf16", k_len_sum=int(kl.sum().item())),
    )
    def finish():
        if not args.no_cpu_baseline:
            log("decode_mq: timing the oracle on a bounded sample")
            res["cpu_baseline"], err = cpu_baseline_decode(inp, args.cpu_budget, out, lse, nq=Nq, name="decode_mq")
            res["max_abs_err"] = _err_fields(err)

    return res, finish


def run_decode(args, dev):
    import torch

    import online_softmax_05_amd as fa
    import workloads

    log("decode: drawing inputs on the device")
    inp = workloads.decode(dev)
    s = workloads.SHAPES["decode"]
    B, H, Nk, dk, dv = s["B"], s["H"], s["Nk"], s["dk"], s["dv"]
    chunk = inp["chunk"]
    ws = torch.empty(fa.fa_decode_splitk_workspace_bytes(B, H, Nk, dv, chunk) // 4, dtype=torch.float32,
                     device=dev)
    out = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)

    def step():
        fa.fa_decode_splitk(inp["q"], inp["k"], inp["v"], inp["k_len"], scale=inp["scale"], chunk=chunk,
                            out=out, lse=lse, workspace=ws)

    log(f"decode: timing {args.warmup} + {args.steps} steps")
    t = time_launches(step, args.steps, args.warmup)
    kl = inp["k_len_host"].long()
    nbytes = float(H * kl.sum().item() * (dk + dv) * 2 + B * H * (dk * 2 + dv * 2 + 4))
    value = nbytes / (t["ms_per_step"] * 1e-3) / 1e9
    achieved = nbytes / (t["launch_ms_mean"] * 1e-3) / 1e9
    res = dict(
        workload=workloads.DESCRIPTIONS["decode"], value=value, unit="GB/s", ms_per_step=t["ms_per_step"],
        frac_of_peak=value / PEAK_HBM_GBS,
        roofline=dict(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s", frac=achieved / PEAK_HBM_GBS,
                      traffic=stored_traffic("decode"), traffic_source=traffic_source("decode"), kernel=KERNEL_NAMES["decode"], **launch_fields(t),
                      algorithmic_bytes_per_launch=nbytes),
        config=dict(workload=workloads.DESCRIPTIONS["decode"], B=B, H=H, Nk_max=Nk, dk=dk, dv=dv, chunk=chunk,
                    dtype="bf16", k_len_sum=int(kl.sum().item())),
    )
    def finish():
        if not args.no_cpu_baseline:
            log("decode: timing the oracle on a bounded sample")
            res["cpu_baseline"], err = cpu_baseline_decode(inp, args.cpu_budget, out, lse)
            res["max_abs_err"] = _err_fields(err)

    return res, finish


def run_small(name, args, dev):
    """The small workloads: 1x1x256^2 d64 fp32 without masks (key tile 64),
    and the masks workload 2x4x1024^2, dk 128, dv 64, causal with key
    lengths [0, x], an fp32 bias and equal-logit rows, in fp32 or bf16.  The
    whole workload is compared with the oracle."""
    import numpy as np
    import torch

    import online_softmax_05_amd as fa
    import oracle
    import workloads

    base = "small" if name == "small" else "masks"
    dtype = torch.bfloat16 if name == "masks_bf16" else torch.float32
    inp = workloads.small() if base == "small" else workloads.masks(dtype)
    d = workloads.to_device(inp, dev)
    s = workloads.SHAPES[base]
    B, H, Nq, Nk, dk, dv = (s[x] for x in ("B", "H", "Nq", "Nk", "dk", "dv"))
    out = torch.empty((B, H, Nq, dv), dtype=dtype, device=dev)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)

    def step():
        fa.fa_fwd(d["q"], d["k"], d["v"], bias=d.get("bias"), k_len=d.get("k_len"), scale=inp["scale"],
                  causal=inp["causal"], block_n=inp["block_n"], out=out, lse=lse)

    log(f"{name}: timing {args.warmup} + {args.steps} steps")
    t = time_launches(step, args.steps, args.warmup)
    if inp["k_len"] is None:
        pairs = B * H * (causal_pairs(Nq, Nk) if inp["causal"] else Nq * Nk)
    else:
        pairs = H * sum(causal_pairs_klen(Nq, Nk, max(0, min(Nk, int(x)))) for x in inp["k_len"].tolist())
    flops = 2.0 * (dk + dv) * pairs
    esz = 2 if dtype == torch.bfloat16 else 4
    nbytes = float(esz * B * H * (Nq * dk + Nk * dk + Nk * dv + Nq * dv) + 4 * B * H * Nq
                   + (0 if inp["bias"] is None else 4 * B * H * Nq * Nk))
    mfma_peak = PEAK_BF16_TFLOPS if dtype == torch.bfloat16 else PEAK_F32_MFMA_TFLOPS
    t_mfma = flops / (mfma_peak * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    sec = t["launch_ms_mean"] * 1e-3
    if t_hbm >= t_mfma:
        roof = dict(bound="hbm", achieved=nbytes / sec / 1e9, peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=nbytes / sec / 1e9 / PEAK_HBM_GBS)
    else:
        roof = dict(bound="mfma", achieved=flops / sec / 1e12, peak=mfma_peak, unit="TFLOP/s",
                    frac=flops / sec / 1e12 / mfma_peak)
    kern = {"small": "fwd_f32_kernel (fp32 matrix cores)", "masks_f32": "fwd_f32_kernel (fp32 matrix cores)",
            "masks_bf16": "fwd_bf16_fast_kernel<128, 64, true, false, 4>"}[name]
    res = dict(
        workload=workloads.DESCRIPTIONS[base] + ("" if base == "small" else f", {'bf16' if esz == 2 else 'fp32'}"),
        value=flops / (t["ms_per_step"] * 1e-3) / 1e12, unit="TFLOP/s", ms_per_step=t["ms_per_step"],
        roofline=dict(roof, traffic=None, kernel=kern, **launch_fields(t), algorithmic_flops_per_launch=flops,
                      algorithmic_bytes_per_launch=nbytes,
                      note="far below one launch's worth of work for 256 CUs: launch latency bound"),
        config=dict(workload=workloads.DESCRIPTIONS[base], B=B, H=H, Nq=Nq, Nk=Nk, dk=dk, dv=dv,
                    causal=inp["causal"], dtype="bf16" if esz == 2 else "f32", block_n=inp["block_n"] or 64,
                    allowed_pairs=pairs, **({} if inp["k_len"] is None else {"k_len": inp["k_len"].tolist()}),
                    bias=inp["bias"] is not None),
    )

    def finish():
        if args.no_cpu_baseline:
            return
        log(f"{name}: timing the oracle on the whole workload")
        kl = None if inp["k_len"] is None else inp["k_len"].numpy()
        args64 = [inp[x].double().numpy() for x in ("q", "k", "v")]
        bias64 = None if inp["bias"] is None else inp["bias"].double().numpy()
        scale = float(np.float32(inp["scale"]))
        reps, elapsed = 0, 0.0
        while elapsed < min(args.cpu_budget, 3.0) or reps == 0:
            ts = time.perf_counter()
            o_ref, l_ref = oracle.attention_ref(*args64, scale=scale, causal=inp["causal"], k_len=kl, bias=bias64)
            elapsed += time.perf_counter() - ts
            reps += 1
        res["cpu_baseline"] = dict(value=reps * flops / elapsed / 1e12, unit="TFLOP/s", cores=blas_threads(), blas=blas_name(),
                                   kind="oracle", sample=f"the whole {name} workload, {reps} runs of the dense "
                                                         f"float64 numpy oracle, {elapsed:.2f} s",
                                   seconds=elapsed, cpu=cpu_model())
        err = _err_acc()
        og = out.double().cpu().numpy().reshape(-1, dv)
        lg = lse.double().cpu().numpy().reshape(-1)
        _err_update(err, og, lg, o_ref.reshape(-1, dv), l_ref.reshape(-1))
        res["max_abs_err"] = _err_fields(err)

    return res, finish


def copy_calibration(dev, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, to scale the HBM byte counters."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written": nbytes,
                      "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=list(ALL_WORKLOADS), default="prefill")
    ap.add_argument("--only", action="store_true", help="measure only the main workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work per workload")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the per-GPU kernel is the unit of work; sharding is a design note).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import online_softmax_05_amd as fa

    fa.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return

    order = [args.workload] + ([] if args.only else [w for w in ALL_WORKLOADS if w != args.workload])
    runners = {"decode": run_decode, "decode_mq": run_decode_mq, "backward": run_backward,
               "dropout_bwd": lambda a, d: run_backward(a, d, "dropout_bwd"),
               "small": lambda a, d: run_small("small", a, d), "masks_f32": lambda a, d: run_small("masks_f32", a, d),
               "masks_bf16": lambda a, d: run_small("masks_bf16", a, d)}
    # Every workload is timed first; the oracle samples (CPU baselines and
    # error figures) run afterwards, on the outputs each timed run left, so
    # that no host-side work -- nor the BLAS worker threads it leaves
    # spinning -- overlaps any GPU timing.
    results, pending = {}, []
    for w in order:
        results[w], finish = runners[w](args, dev) if w in runners else run_prefill(w, args, dev)
        pending.append(finish)
    for finish in pending:
        finish()
    pending.clear()

    main_res = results[args.workload]
    line = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": main_res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, drawn on the device; no dataset)",
        "config": main_res["config"],
        "frac_of_peak": main_res["frac_of_peak"],
        "roofline": main_res["roofline"],
        "cpu_baseline": main_res.get("cpu_baseline"),
        "max_abs_err": main_res.get("max_abs_err"),
        "secondary": [dict(results[w]) for w in order[1:]],
        "kernel_source_hash": {w: kernel_source_hash(w) for w in order if w in KERNEL_SOURCES},
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

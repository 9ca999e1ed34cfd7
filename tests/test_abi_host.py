"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and validates arguments on the host (no GPU needed: only the
fa_check_* validators and argument errors that are rejected before any
launch are exercised here)."""

import math
import pathlib
import re
import shutil
import subprocess

import pytest

import online_softmax_05_amd as fa

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "fa.h"

OK, NULL, SHAPE, UNSUP, WS, HIPERR = 0, 1, 2, 3, 4, 5
P = 0x10000  # a fake, 16-byte aligned "device address" (never dereferenced)


def header_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_library_built():
    assert fa.lib_path().exists(), "libfa.so is not built (python -m online_softmax_05_amd.build)"


def test_exports_every_declared_symbol():
    names = header_functions()
    assert {"fa_fwd", "fa_decode_splitk", "fa_decode_splitk_workspace_bytes", "fa_check_fwd",
            "fa_check_decode", "fa_bwd", "fa_bwd_workspace_bytes", "fa_check_bwd", "fa_status_str",
            "fa_abi_version", "fa_decode_splitk_mq", "fa_decode_splitk_mq_workspace_bytes",
            "fa_check_decode_mq", "fa_fwd_ex", "fa_check_fwd_ex", "fa_bwd_ex", "fa_check_bwd_ex"} <= set(names)
    lib = fa.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in fa.h but not exported"
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", str(fa.lib_path())], capture_output=True,
                             text=True).stdout
        exported = set(re.findall(r"\b(fa_[a-z0-9_]+)\b", out))
        assert set(names) <= exported
        # nothing else with the public prefix leaks out
        assert exported <= set(names)


def test_header_is_plain_c():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = '#include "fa.h"\nint main(void) { return (int)sizeof(fa_status) + FA_BF16; }\n'
    res = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
                          f"-I{HEADER.parent}", "-x", "c", "-"], input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_abi_version_and_status_strings():
    assert fa.fa_abi_version() == 105
    for st in range(6):
        assert isinstance(fa.fa_status_str(st), str) and fa.fa_status_str(st)
    assert fa.fa_status_str(0) == "ok"
    assert "unknown" in fa.fa_status_str(99)


def fwd_args(**kw):
    a = dict(q=P, k=P, v=P, bias=None, k_len=None, o=P, lse=P, B=2, H=3, Nq=17, Nk=33, dk=64, dv=32,
             dtype=fa.FA_BF16, scale=0.125, causal=1, block_n=0)
    a.update(kw)
    return a


def check_fwd(**kw):
    a = fwd_args(**kw)
    return fa.fa_check_fwd(a["q"], a["k"], a["v"], a["bias"], a["k_len"], a["o"], a["lse"], a["B"], a["H"],
                           a["Nq"], a["Nk"], a["dk"], a["dv"], a["dtype"], a["scale"], a["causal"],
                           a["block_n"])


@pytest.mark.parametrize("kw,want", [
    ({}, OK),
    ({"dtype": fa.FA_F32}, OK),
    ({"bias": P, "k_len": P}, OK),
    ({"lse": None}, OK),
    ({"block_n": 32}, OK), ({"block_n": 64}, OK), ({"block_n": 128}, OK),
    ({"block_n": 16}, UNSUP), ({"block_n": 256}, UNSUP), ({"block_n": -1}, UNSUP),
    ({"q": None}, NULL), ({"o": None}, NULL), ({"k": None}, NULL), ({"v": None}, NULL),
    ({"Nk": 0, "k": None, "v": None}, OK),           # empty key axis: o = 0, lse = -inf
    ({"Nq": 0, "q": None, "o": None}, OK),           # nothing to compute
    ({"B": 0, "q": None, "k": None, "v": None, "o": None}, OK),
    ({"H": 0}, OK),
    ({"B": -1}, SHAPE), ({"H": -2}, SHAPE), ({"Nq": -1}, SHAPE), ({"Nk": -5}, SHAPE),
    ({"dk": 0}, SHAPE), ({"dv": 0}, SHAPE),
    ({"dk": 129}, UNSUP), ({"dv": 200}, UNSUP), ({"dk": 1, "dv": 1}, OK), ({"dk": 128, "dv": 128}, OK),
    ({"dtype": 2}, UNSUP), ({"dtype": -1}, UNSUP),
    ({"causal": 2}, UNSUP),
    ({"scale": math.inf}, UNSUP), ({"scale": math.nan}, UNSUP), ({"scale": -0.5}, OK),
    ({"B": 1 << 16, "H": 1 << 16, "Nq": 1 << 10}, SHAPE),  # grid would not fit 32 bits
    ({"Nq": 2**31 - 1, "Nk": 2}, SHAPE),
])
def test_check_fwd(kw, want):
    assert check_fwd(**kw) == want


def check_fwd_ex(align=fa.FA_ALIGN_BOTTOM_RIGHT, wl=-1, wr=-1, keep=256, seed=0, **kw):
    a = fwd_args(**kw)
    return fa.fa_check_fwd_ex(a["q"], a["k"], a["v"], a["bias"], a["k_len"], a["o"], a["lse"], a["B"],
                              a["H"], a["Nq"], a["Nk"], a["dk"], a["dv"], a["dtype"], a["scale"], a["causal"],
                              align, wl, wr, keep, seed, a["block_n"])


@pytest.mark.parametrize("kw,want", [
    ({}, OK), ({"align": fa.FA_ALIGN_TOP_LEFT}, OK), ({"align": 2}, UNSUP), ({"align": -1}, UNSUP),
    ({"wl": 0}, OK), ({"wr": 0}, OK), ({"wl": 127, "wr": 3, "causal": 0}, OK), ({"wl": 2**31 - 1}, OK),
    ({"wl": -2}, UNSUP), ({"wr": -7}, UNSUP),
    ({"wl": 4, "dk": 300}, UNSUP), ({"wl": 4, "q": None}, NULL), ({"wl": 4, "causal": 3}, UNSUP),
    ({"wl": 4, "Nq": 0, "q": None, "o": None}, OK),
    ({"keep": 230, "seed": 2**64 - 1}, OK), ({"keep": 1}, OK), ({"keep": 0}, UNSUP), ({"keep": 257}, UNSUP),
    ({"keep": -3}, UNSUP), ({"keep": 200, "wl": 7, "align": fa.FA_ALIGN_TOP_LEFT, "dtype": fa.FA_F32}, OK),
])
def test_check_fwd_ex(kw, want):
    assert check_fwd_ex(**kw) == want


def test_fwd_ex_rejects_before_launch():
    f = fa.lib().fa_fwd_ex
    assert f(P, P, P, None, None, P, P, 1, 1, 4, 4, 8, 8, fa.FA_BF16, 1.0, 1, 5, -1, -1, 256, 0, 0, None) == UNSUP
    assert f(P, P, P, None, None, P, P, 1, 1, 4, 4, 8, 8, fa.FA_BF16, 1.0, 1, 0, -3, -1, 256, 0, 0, None) == UNSUP
    assert f(P, P, P, None, None, P, P, 1, 1, 4, 4, 8, 8, fa.FA_BF16, 1.0, 1, 0, -1, -1, 0, 7, 0, None) == UNSUP
    assert f(None, None, None, None, None, None, None, 0, 4, 4, 4, 8, 8, fa.FA_F32, 1.0, 0, 1, 3, 3, 100, 9, 0,
             None) == OK


def test_keep_256_for():
    assert fa.keep_256_for(0.0) == 256 and fa.keep_256_for(0.1) == 230 and fa.keep_256_for(0.5) == 128
    assert fa.keep_256_for(0.999) == 1
    for bad in (-0.1, 1.0, 2.0):
        with pytest.raises(fa.FaError):
            fa.keep_256_for(bad)


def check_bwd_ex(align=fa.FA_ALIGN_BOTTOM_RIGHT, wl=-1, wr=-1, keep=256, **kw):
    a = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, bias=None, k_len=None, dq=P, dk=P, dv=P, B=2, H=3, Nq=40, Nk=70,
             d_k=64, d_v=64, dtype=fa.FA_BF16, scale=0.125, causal=1)
    a.update(kw)
    ws = fa.fa_bwd_workspace_bytes(a["B"], a["H"], a["Nq"])
    return fa.fa_check_bwd_ex(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["bias"], a["k_len"], a["dq"],
                              a["dk"], a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["d_k"], a["d_v"], a["dtype"],
                              a["scale"], a["causal"], align, wl, wr, keep, 5, P, ws)


@pytest.mark.parametrize("kw,want", [
    ({}, OK), ({"align": fa.FA_ALIGN_TOP_LEFT, "wl": 3}, OK), ({"keep": 100}, OK), ({"keep": 0}, UNSUP),
    ({"keep": 300}, UNSUP), ({"align": 7}, UNSUP), ({"wr": -2}, UNSUP), ({"q": None}, NULL), ({"causal": 5}, UNSUP),
    ({"d_k": 200}, UNSUP),
    ({"B": 65535, "H": 1, "Nq": 1 << 20, "Nk": 64}, OK),
    ({"B": 65535, "H": 1, "Nq": 1 << 22, "Nk": 64}, SHAPE),  # 1-D tile grid would exceed 2^31
    ({"B": 256, "H": 257, "Nq": 64, "Nk": 64}, SHAPE),       # B*H above the 2-D grid limit
])
def test_check_bwd_ex(kw, want):
    assert check_bwd_ex(**kw) == want


def test_fwd_rejects_before_launch():
    # invalid arguments come back as an error code without any GPU work
    a = fwd_args(dk=300)
    st = fa.lib().fa_fwd(a["q"], a["k"], a["v"], None, None, a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                         a["Nk"], a["dk"], a["dv"], a["dtype"], a["scale"], a["causal"], a["block_n"], None)
    assert st == UNSUP
    st = fa.lib().fa_fwd(None, P, P, None, None, P, None, 1, 1, 4, 4, 8, 8, fa.FA_F32, 1.0, 0, 0, None)
    assert st == NULL
    # an empty problem is a successful no-op
    st = fa.lib().fa_fwd(None, None, None, None, None, None, None, 0, 4, 4, 4, 8, 8, fa.FA_F32, 1.0, 0, 0, None)
    assert st == OK


def test_workspace_bytes():
    f = fa.fa_decode_splitk_workspace_bytes
    assert f(64, 32, 8192, 128, 512) == 64 * 32 * 16 * 130 * 4
    assert f(2, 3, 1000, 64, 512) == 2 * 3 * 2 * 66 * 4
    assert f(2, 3, 0, 64, 512) == 0
    assert f(1, 1, 1, 1, 64) == 1 * 1 * 1 * 3 * 4
    assert f(1, 1, 100, 8, 100) == 0     # chunk not a multiple of 64
    assert f(-1, 1, 100, 8, 64) == 0
    assert f(1, 1, 100, 0, 64) == 0


def check_dec(**kw):
    a = dict(q=P, k=P, v=P, k_len=P, o=P, lse=P, B=4, H=2, Nk=1000, dk=128, dv=64, chunk=512,
             dtype=fa.FA_BF16, scale=0.1, ws=P, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = fa.fa_decode_splitk_workspace_bytes(a["B"], a["H"], a["Nk"], a["dv"], a["chunk"])
    return fa.fa_check_decode(a["q"], a["k"], a["v"], a["k_len"], a["o"], a["lse"], a["B"], a["H"], a["Nk"],
                              a["dk"], a["dv"], a["chunk"], a["dtype"], a["scale"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("kw,want", [
    ({}, OK), ({"dtype": fa.FA_F32}, OK), ({"lse": None}, OK),
    ({"k_len": None}, NULL), ({"q": None}, NULL), ({"o": None}, NULL), ({"k": None}, NULL),
    ({"ws": None}, WS), ({"ws_bytes": 100}, WS), ({"ws": P + 4}, WS),
    ({"chunk": 100}, UNSUP), ({"chunk": 0}, UNSUP), ({"chunk": 4096}, UNSUP), ({"chunk": 64}, OK),
    ({"chunk": 2048}, OK),
    ({"dk": 129}, UNSUP), ({"dv": 0}, SHAPE), ({"B": -1}, SHAPE), ({"Nk": -1}, SHAPE),
    ({"Nk": 0, "k": None, "v": None, "ws": None, "ws_bytes": 0}, OK),
    ({"B": 0, "q": None, "o": None, "k_len": None}, OK),
    ({"scale": math.nan}, UNSUP), ({"dtype": 7}, UNSUP),
])
def test_check_decode(kw, want):
    assert check_dec(**kw) == want


def check_bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, bias=None, k_len=None, dq=P, dk=P, dv=P, B=2, H=3, Nq=100,
             Nk=120, d_k=64, d_v=32, dtype=fa.FA_BF16, scale=0.125, causal=1, ws=P, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = fa.fa_bwd_workspace_bytes(a["B"], a["H"], a["Nq"])
    return fa.fa_check_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["bias"], a["k_len"],
                           a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["d_k"], a["d_v"],
                           a["dtype"], a["scale"], a["causal"], a["ws"], a["ws_bytes"])


def test_bwd_workspace_bytes():
    f = fa.fa_bwd_workspace_bytes
    assert f(2, 3, 100) == 2 * 3 * 100 * 4
    assert f(0, 3, 100) == 0 and f(-1, 3, 100) == 0 and f(1, 1, -5) == 0


@pytest.mark.parametrize("kw,want", [
    ({}, OK), ({"dtype": fa.FA_F32}, OK), ({"bias": P, "k_len": P}, OK), ({"causal": 0}, OK),
    ({"lse": None}, NULL), ({"q": None}, NULL), ({"o": None}, NULL), ({"dout": None}, NULL),
    ({"dq": None}, NULL), ({"dk": None}, NULL), ({"dv": None}, NULL), ({"k": None}, NULL), ({"v": None}, NULL),
    ({"ws": None}, WS), ({"ws_bytes": 100}, WS), ({"ws": P + 4}, WS),
    ({"d_k": 129}, UNSUP), ({"d_v": 0}, SHAPE), ({"B": -1}, SHAPE), ({"Nk": -1}, SHAPE), ({"Nq": -3}, SHAPE),
    ({"causal": 2}, UNSUP), ({"scale": math.inf}, UNSUP), ({"dtype": 3}, UNSUP),
    ({"B": 256, "H": 256}, SHAPE),                                   # B*H beyond the 16-bit grid axis
    ({"Nq": 0, "q": None, "o": None, "dout": None, "lse": None, "dq": None, "ws": None, "ws_bytes": 0}, OK),
    ({"Nk": 0, "k": None, "v": None, "dk": None, "dv": None}, OK),
    ({"B": 0, "q": None, "k": None, "v": None, "o": None, "dout": None, "lse": None, "dq": None, "dk": None,
      "dv": None, "ws": None, "ws_bytes": 0}, OK),
])
def test_check_bwd(kw, want):
    assert check_bwd(**kw) == want


def check_mq(**kw):
    a = dict(q=P, k=P, v=P, k_len=P, o=P, lse=P, B=4, H=2, Nq=4, Nk=1000, dk=128, dv=64, chunk=512,
             dtype=fa.FA_BF16, scale=0.1, causal=1, ws=P, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = fa.fa_decode_splitk_mq_workspace_bytes(a["B"], a["H"], a["Nq"], a["Nk"], a["dv"], a["chunk"])
    return fa.fa_check_decode_mq(a["q"], a["k"], a["v"], a["k_len"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                                 a["Nk"], a["dk"], a["dv"], a["chunk"], a["dtype"], a["scale"], a["causal"],
                                 a["ws"], a["ws_bytes"])


def test_mq_workspace_bytes():
    f = fa.fa_decode_splitk_mq_workspace_bytes
    assert f(2, 3, 4, 1000, 64, 512) == 2 * 3 * 2 * 4 * 66 * 4
    assert f(1, 1, 17, 100, 8, 64) == 0 and f(1, 1, 0, 100, 8, 64) == 0   # Nq outside 1..16
    assert f(1, 1, 2, 100, 8, 100) == 0                                   # chunk not a multiple of 64


@pytest.mark.parametrize("kw,want", [
    ({}, OK), ({"dtype": fa.FA_F32}, OK), ({"lse": None}, OK), ({"causal": 0}, OK), ({"Nq": 1}, OK),
    ({"Nq": 16}, OK), ({"Nq": 17}, UNSUP), ({"Nq": 0}, UNSUP), ({"causal": 3}, UNSUP),
    ({"k_len": None}, NULL), ({"q": None}, NULL), ({"o": None}, NULL), ({"k": None}, NULL),
    ({"ws": None}, WS), ({"ws_bytes": 100}, WS), ({"ws": P + 8}, WS),
    ({"chunk": 100}, UNSUP), ({"chunk": 4096}, UNSUP), ({"chunk": 64}, OK),
    ({"dk": 129}, UNSUP), ({"dv": 0}, SHAPE), ({"B": -1}, SHAPE), ({"Nk": -1}, SHAPE),
    ({"Nk": 0, "k": None, "v": None, "ws": None, "ws_bytes": 0}, OK),
    ({"B": 0, "q": None, "o": None, "k_len": None}, OK),
    ({"scale": math.nan}, UNSUP), ({"dtype": 2}, UNSUP),
])
def test_check_decode_mq(kw, want):
    assert check_mq(**kw) == want


def test_binding_fails_loudly_without_a_device():
    import torch

    q = torch.zeros(1, 1, 4, 8)
    with pytest.raises(fa.FaError):
        fa.fa_fwd(q, q, q)


def static_decode(**kw):
    """fa_decode_splitk_static with fake pointers: every case here is rejected
    (or is a no-op) on the host, before the scratch lookup or any launch."""
    a = dict(q=P, k=P, v=P, k_len=P, o=P, lse=P, B=4, H=8, Nk=1000, dk=128, dv=128, chunk=512,
             dtype=fa.FA_BF16, scale=0.125)
    a.update(kw)
    return fa.lib().fa_decode_splitk_static(a["q"], a["k"], a["v"], a["k_len"], a["o"], a["lse"], a["B"], a["H"],
                                           a["Nk"], a["dk"], a["dv"], a["chunk"], a["dtype"], a["scale"], None)


@pytest.mark.parametrize("kw,want", [
    # partial states beyond the static scratch: 64 x 64 sequence-heads x 16 chunks x 130 floats = 34 MB
    ({"B": 64, "H": 64, "Nk": 8192}, WS),
    ({"B": 64, "H": 128, "Nk": 8192, "chunk": 1024}, WS),   # 8192 x 8 x 130 x 4 = 34 MB
    ({"chunk": 100}, UNSUP), ({"dk": 129}, UNSUP), ({"dtype": 7}, UNSUP),
    ({"q": None}, NULL), ({"k_len": None}, NULL), ({"o": None}, NULL),
    ({"B": -1}, SHAPE),
    ({"B": 0, "q": None, "o": None}, OK),     # nothing to compute: no scratch lookup, no launch
])
def test_static_decode_host_checks(kw, want):
    assert fa.FA_STATIC_SCRATCH_BYTES == 32 * 1024 * 1024
    assert static_decode(**kw) == want


def test_static_decode_limit_matches_workspace_size():
    # the decode workload (64 x 32 sequence-heads, 8192 keys, 512-key chunks,
    # dv 128) fits; twice its heads do not
    assert fa.fa_decode_splitk_workspace_bytes(64, 32, 8192, 128, 512) <= fa.FA_STATIC_SCRATCH_BYTES
    assert fa.fa_decode_splitk_workspace_bytes(64, 64, 8192, 128, 512) > fa.FA_STATIC_SCRATCH_BYTES

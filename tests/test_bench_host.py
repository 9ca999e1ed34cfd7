"""Host-side checks of bench.py (no GPU): the multi-GPU refusal, the
algorithmic pair counts its FLOP figures rest on, and the source hashing
that decides whether a stored rocprofv3 record still describes the kernels."""

import json
import pathlib
import subprocess
import sys

import bench

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_causal_pairs_closed_forms():
    # bottom-right causal, Nq = Nk = n: row i sees i + 1 keys
    for n in (1, 7, 64, 300):
        assert bench.causal_pairs(n, n) == n * (n + 1) // 2
    # Nq < Nk: row i sees i + Nk - Nq + 1 keys
    assert bench.causal_pairs(3, 10) == 8 + 9 + 10
    # a left window of w keys before the row's own: min(i + 1, w + 1) keys
    n, w = 300, 40
    assert bench.causal_pairs(n, n, w) == sum(min(i + 1, w + 1) for i in range(n))
    # the sliding-window workload's count
    assert bench.causal_pairs(4096, 4096, 1023) == 1024 * 1025 // 2 + (4096 - 1024) * 1024


def test_code_only_drops_comments_and_whitespace_keeps_literals():
    src = 'int a; // note\n/* block\n comment */ int  b = "x//y /* z */";\nchar c = \'"\';  // end\n'
    assert bench._code_only(src) == 'int a; int b = "x//y /* z */"; char c = \'"\';'
    assert bench._code_only("a  /*x*/b") == "a b"


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    f = tmp_path / "k.hip"
    f.write_text("__global__ void k(int* p) { p[0] = 1; }  // first\n")
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    monkeypatch.setitem(bench.KERNEL_SOURCES, "probe", ["k.hip"])
    h0 = bench.kernel_source_hash("probe")
    f.write_text("// reworded comment\n__global__ void k(int* p) {\n  p[0] = 1;\n}\n")
    assert bench.kernel_source_hash("probe") == h0
    f.write_text("__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.kernel_source_hash("probe") != h0


def test_stored_records_match_the_current_kernels():
    """Every committed counter or traffic record was taken with the kernels
    as they are now (else bench.py would silently drop it)."""
    recs = sorted((ROOT / "profiles").glob("*.json"))
    assert recs, "no stored records"
    for p in recs:
        rec = json.loads(p.read_text())
        assert rec["kernel_source_hash"] == bench.kernel_source_hash(rec["workload"]), p.name

"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pin suite rejects every one of them.

Each mutation is an exact text replacement in one oracle source file; the
mutated package is written to a temporary directory and imported under a
fresh name.  A mutation whose anchor text is missing fails the test, so the
list cannot silently drift away from the oracle's source.
"""

import importlib.util
import pathlib
import shutil
import sys
import uuid

import pytest

from tests import pins

ORACLE_DIR = pathlib.Path(__file__).resolve().parent.parent / "oracle"

# (id, file, anchor text, replacement)
MUTANTS = [
    # --- dense definition -------------------------------------------------
    ("top_left_causal", "dense.py",
     "ok &= j <= pos\n", "ok &= j <= row_ids[:, None]\n"),
    ("strict_causal", "dense.py",
     "ok &= j <= pos\n", "ok &= j < pos\n"),
    ("causal_offset_sign", "dense.py",
     "((nk - nq) if align", "((nq - nk) if align"),
    ("klen_off_by_one", "dense.py",
     "ok = np.broadcast_to(j < limit,", "ok = np.broadcast_to(j <= limit,"),
    ("klen_ignored", "dense.py",
     "limit = nk if k_len_b is None else min(max(int(k_len_b), 0), nk)", "limit = nk"),
    ("scale_dropped", "dense.py",
     "s = (q @ k.T) * float(scale)", "s = (q @ k.T)"),
    ("scale_squared", "dense.py",
     "s = (q @ k.T) * float(scale)", "s = (q @ k.T) * float(scale) ** 2"),
    ("bias_sign", "dense.py",
     "s = s + np.asarray(bias, dtype=np.float64)", "s = s - np.asarray(bias, dtype=np.float64)"),
    ("bias_scaled", "dense.py",
     "s = s + np.asarray(bias, dtype=np.float64)",
     "s = s + float(scale) * np.asarray(bias, dtype=np.float64)"),
    ("bias_dropped", "dense.py",
     "s = s + np.asarray(bias, dtype=np.float64)", "s = s"),
    ("max_shift_sign", "dense.py",
     "e = np.where(ok, np.exp(s - m[:, None]), 0.0)", "e = np.where(ok, np.exp(s + m[:, None]), 0.0)"),
    ("mask_not_applied_to_exp", "dense.py",
     "e = np.where(ok, np.exp(s - m[:, None]), 0.0)",
     "e = np.exp(np.where(ok, s, np.where(np.isfinite(s), s, 0.0) * 0.0) - m[:, None])"),
    ("no_normalisation", "dense.py",
     "p = e / safe_ell[:, None]", "p = e"),
    ("normalise_by_count", "dense.py",
     "p = e / safe_ell[:, None]", "p = e / np.maximum(ok.sum(axis=1), 1)[:, None]"),
    ("lse_drops_max", "dense.py",
     "lse = np.where(nonempty, m + np.log(safe_ell), -np.inf)",
     "lse = np.where(nonempty, np.log(safe_ell), -np.inf)"),
    ("lse_log2", "dense.py",
     "lse = np.where(nonempty, m + np.log(safe_ell), -np.inf)",
     "lse = np.where(nonempty, m + np.log2(safe_ell), -np.inf)"),
    ("empty_lse_zero", "dense.py",
     "lse = np.where(nonempty, m + np.log(safe_ell), -np.inf)",
     "lse = np.where(nonempty, m + np.log(safe_ell), 0.0)"),
    ("empty_row_nan", "dense.py",
     "o[~nonempty] = 0.0", "o[~nonempty] = np.nan"),
    ("values_transposed_rows", "dense.py",
     "o = p @ v", "o = p @ v[::-1]"),
    ("keys_reversed", "dense.py",
     "s = (q @ k.T) * float(scale)", "s = (q @ k[::-1].T) * float(scale)"),
    ("row_ids_ignored", "dense.py",
     "ok = allowed_mask(row_ids, nq, nk, causal, k_len_b,",
     "ok = allowed_mask(np.arange(rows), nq, nk, causal, k_len_b,"),
    # --- tile recurrence and merge ------------------------------------------
    ("rescale_l_only", "online.py",
     "alpha_a * u_a + alpha_b * u_b", "u_a + alpha_b * u_b"),
    ("rescale_u_only", "online.py",
     "alpha_a * l_a + alpha_b * l_b", "l_a + alpha_b * l_b"),
    ("alpha_inverted", "online.py",
     "alpha_a = np.exp(m_a - m)", "alpha_a = np.exp(m - m_a)"),
    ("merge_without_rebase", "online.py",
     "states[r] = merge_states(old, block_state(s[r, ok[r]], v[ka:kb][ok[r]]))",
     "blk = block_state(s[r, ok[r]], v[ka:kb][ok[r]])\n"
     "                states[r] = blk if old is None else (max(old[0], blk[0]), old[1] + blk[1], old[2] + blk[2])"),
    ("tile_local_positions", "online.py",
     "ok = allowed_mask(np.arange(qa, qb), nq, nk, causal, k_len_b)[:, ka:kb]",
     "ok = allowed_mask(np.arange(qb - qa), qb - qa, kb - ka, causal, k_len_b)"),
    ("bias_tile_misaligned", "online.py",
     "s = s + np.asarray(bias, dtype=np.float64)[qa:qb, ka:kb]",
     "s = s + np.asarray(bias, dtype=np.float64)[qa:qb, :kb - ka]"),
    ("empty_tile_not_skipped", "online.py",
     "if not ok[r].any():\n                    continue", "if False:\n                    continue"),
    ("duplicates_allowed", "online.py",
     "if np.any(seen != 1):", "if np.any(seen < 1):"),
    ("lse_drops_max_online", "online.py",
     "lse[qa + r] = m + np.log(ell)", "lse[qa + r] = np.log(ell)"),
    ("merge_rescale_dropped", "online.py",
     "return m, alpha_a * l_a + alpha_b * l_b, alpha_a * u_a + alpha_b * u_b",
     "return m, alpha_a * l_a + alpha_b * l_b, u_a + u_b"),
    ("merge_alpha_sign", "online.py",
     "alpha_b = np.exp(m_b - m)", "alpha_b = np.exp(m - m_b)"),
    ("block_state_unshifted", "online.py",
     "e = np.exp(x - m)\n    return m, e.sum(), e @ vals", "e = np.exp(x)\n    return m, e.sum(), e @ vals"),
    ("block_state_normalised", "online.py",
     "return m, e.sum(), e @ vals", "return m, e.sum(), (e @ vals) / e.sum()"),
    # --- mask variants ------------------------------------------------------
    ("top_left_offset", "dense.py",
     "pos = row_ids[:, None] + ((nk - nq) if align == \"bottom_right\" else 0)",
     "pos = row_ids[:, None] + (nk - nq)"),
    ("window_left_off_by_one", "dense.py",
     "ok &= j >= pos - int(wl)", "ok &= j > pos - int(wl)"),
    ("window_left_sign", "dense.py",
     "ok &= j >= pos - int(wl)", "ok &= j >= pos + int(wl)"),
    ("window_right_ignored", "dense.py",
     "ok &= j <= pos + int(wr)", "ok &= j <= pos + nk"),
    # --- backward by recomputation ------------------------------------------
    ("bwd_c_dropped", "backward.py",
     "d = p * (zr * (g @ v.T) - c[:, None])", "d = p * (zr * (g @ v.T))"),
    ("bwd_c_sign", "backward.py",
     "d = p * (zr * (g @ v.T) - c[:, None])", "d = p * (zr * (g @ v.T) + c[:, None])"),
    ("bwd_c_from_v", "backward.py",
     "c = np.sum(g * o, axis=1)", "c = np.sum(g, axis=1) * 0.5"),
    ("bwd_dq_unscaled", "backward.py",
     "dq = float(scale) * (d @ k)", "dq = (d @ k)"),
    ("bwd_dk_unscaled", "backward.py",
     "dk = float(scale) * (d.T @ q)", "dk = (d.T @ q)"),
    ("bwd_dk_uses_p", "backward.py",
     "dk = float(scale) * (d.T @ q)", "dk = float(scale) * (p.T @ q)"),
    ("bwd_dq_uses_v", "backward.py",
     "dq = float(scale) * (d @ k)", "dq = float(scale) * (d @ v[:, :1].repeat(k.shape[1], axis=1))"),
    ("bwd_dv_uses_d", "backward.py",
     "dv = (p * zr).T @ g", "dv = (d * zr).T @ g"),
    ("bwd_dv_rows_reversed", "backward.py",
     "dv = (p * zr).T @ g", "dv = (p * zr).T @ g[::-1]"),
    ("bwd_lse_sign", "backward.py",
     "np.exp(np.where(ok, s, 0.0) - lse_safe[:, None])", "np.exp(np.where(ok, s, 0.0) + lse_safe[:, None])"),
    ("bwd_mask_ignored", "backward.py",
     "p = np.where(ok & nonempty[:, None],", "p = np.where(nonempty[:, None] | True,"),
    ("bwd_bias_ignored", "backward.py",
     "s = s + np.asarray(bias, dtype=np.float64)", "s = s"),
    ("bwd_scale_dropped_in_logits", "backward.py",
     "s = (q @ k.T) * float(scale)", "s = (q @ k.T)"),
    # --- dropout -------------------------------------------------------------
    ("philox_no_key_bump", "dropout.py", "if rnd < 9:", "if rnd < 0:"),
    ("philox_nine_rounds", "dropout.py", "for rnd in range(10):", "for rnd in range(9):"),
    ("philox_multipliers_swapped", "dropout.py",
     "p0 = c0.astype(np.uint64) * _M0", "p0 = c0.astype(np.uint64) * _M1"),
    ("philox_output_order", "dropout.py",
     "c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0", "c0, c1, c2, c3 = hi0 ^ c1 ^ k0, lo1, hi1 ^ c3 ^ k1, lo0"),
    ("dropout_head_ignored", "dropout.py", "ctr[..., 2] = int(bh)", "ctr[..., 2] = 0"),
    ("dropout_word_index", "dropout.py", "((j >> 4) & 3)[None, :, None]", "((j >> 2) & 3)[None, :, None]"),
    ("dropout_byte_shift", "dropout.py", "(8 * (j & 3))", "(8 * ((j >> 4) & 3))"),
    ("dropout_keep_le", "dropout.py",
     "return dropout_bytes(bh, row_ids, nk, seed).astype(np.int64) < t",
     "return dropout_bytes(bh, row_ids, nk, seed).astype(np.int64) <= t"),
    ("dropout_scale_255", "dropout.py", "return 256.0 / float(keep_256)", "return 255.0 / float(keep_256)"),
    ("dropout_fwd_unscaled", "dense.py",
     "o = (np.where(z, p, 0.0) * keep_scale(keep_256)) @ v", "o = np.where(z, p, 0.0) @ v"),
    ("dropout_fwd_mask_inverted", "dense.py",
     "o = (np.where(z, p, 0.0) * keep_scale(keep_256)) @ v", "o = (np.where(z, 0.0, p) * keep_scale(keep_256)) @ v"),
    ("dropout_bwd_ignored_in_d", "backward.py",
     "d = p * (zr * (g @ v.T) - c[:, None])", "d = p * ((g @ v.T) - c[:, None])"),
    ("dropout_bwd_ignored_in_dv", "backward.py", "dv = (p * zr).T @ g", "dv = p.T @ g"),
]


def _load_mutant(tmp_path, fname, anchor, repl):
    pkg_name = f"oracle_mut_{uuid.uuid4().hex[:8]}"
    dst = tmp_path / pkg_name
    shutil.copytree(ORACLE_DIR, dst, ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.o"))
    src = (dst / fname).read_text()
    assert src.count(anchor) == 1, f"anchor not found exactly once in {fname}: {anchor!r}"
    (dst / fname).write_text(src.replace(anchor, repl))
    spec = importlib.util.spec_from_file_location(pkg_name, dst / "__init__.py",
                                                  submodule_search_locations=[str(dst)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[pkg_name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("mid,fname,anchor,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_rejected(tmp_path, mid, fname, anchor, repl):
    mod = _load_mutant(tmp_path, fname, anchor, repl)
    failed = pins.failing_pins(mod)
    assert failed, f"mutant {mid} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    mod = _load_mutant(tmp_path, "dense.py", "import numpy as np", "import numpy as np")
    assert pins.failing_pins(mod) == []

"""Mutation check of the oracle's pins.

Each entry of MUTANTS is a plausible mistake (a dropped factor, an off-by-one mask, a wrong
log base, a swapped index, a transposed operand, a wrong sign or rounding rule).  It is planted
in a temporary copy of ``oracle/`` on the CPU, the three pin suites run against that copy in a
subprocess, and at least one pin must fail.  An unmodified copy must pass them all, so the
harness itself is checked too.  Nothing here touches the GPU path.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["test_oracle_pins.py", "test_oracle_bwd_pins.py", "test_oracle_fp8_pins.py"]

# (name, oracle file, text to replace (must occur exactly once), replacement)
MUTANTS = [
    # forward definition
    ("scale_dropped", "attention.py",
     "s = scale * (q_rows @ k.T)", "s = q_rows @ k.T"),
    ("scores_against_values", "attention.py",
     "s = scale * (q_rows @ k.T)", "s = scale * (q_rows @ v.T)"),
    ("causal_diagonal_excluded", "attention.py",
     "return np.minimum(rows + 1, L)", "return np.minimum(np.maximum(rows, 1), L)"),
    ("causal_one_key_too_many", "attention.py",
     "return np.minimum(rows + 1, L)", "return np.minimum(rows + 2, L)"),
    ("mask_keeps_first_hidden_key", "attention.py",
     "invisible = np.arange(L)[None, :] >= counts[:, None]",
     "invisible = np.arange(L)[None, :] > counts[:, None]"),
    ("no_normalisation", "attention.py", "p = e / l[:, None]", "p = e"),
    ("lse_base_2", "attention.py", "lse = m + np.log(l)", "lse = m + np.log2(l)"),
    ("lse_without_maximum", "attention.py", "lse = m + np.log(l)", "lse = np.log(l)"),
    ("gqa_heads_interleaved", "attention.py",
     "            g = h // group\n            ob, lb, pb",
     "            g = h % Hkv\n            ob, lb, pb"),
    ("padding_rows_attend", "attention.py",
     "valid = rows < L                      # padded",
     "valid = rows < N                      # padded"),
    # paged forms
    ("paged_block_and_slot_swapped", "paged.py",
     "[t // bs]\n", "[t % bs]\n"),
    ("paged_decode_lse_base_2", "paged.py",
     "lse[b, h] = m + np.log(l)", "lse[b, h] = m + np.log2(l)"),
    ("paged_decode_scale_dropped", "paged.py",
     "s = float(scale) * (kb[:, g, :] @ q[b, h])", "s = kb[:, g, :] @ q[b, h]"),
    ("chunk_offset_dropped", "paged.py",
     "counts = (L - Q) + sel[valid] + 1", "counts = sel[valid] + 1"),
    ("chunk_rows_past_chunk_attend", "paged.py",
     "valid = sel < Q\n", "valid = sel < L\n"),
    # backward
    ("bwd_row_term_sign", "backward.py",
     "            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))\n            dq[b, h, :L]",
     "            ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))\n            dq[b, h, :L]"),
    ("bwd_dv_untransposed", "backward.py", "dv[b, g, :L] += p.T @ dob", "dv[b, g, :L] += p @ dob"),
    ("bwd_dk_scale_dropped", "backward.py",
     "dk[b, g, :L] += scale * (ds.T @ qb)", "dk[b, g, :L] += ds.T @ qb"),
    ("bwd_dq_uses_values", "backward.py",
     "dq[b, h, :L] = scale * (ds @ kb)", "dq[b, h, :L] = scale * (ds @ vb)"),
    ("bwd_row_subset_drops_row_term", "backward.py",
     "            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))\n            dq[b, h, valid]",
     "            ds = p * dp\n            dq[b, h, valid]"),
    ("bwd_key_subset_row_term_sign", "backward.py",
     "dsj = pj * (dpj - drow[:, None])", "dsj = pj * (dpj + drow[:, None])"),
    ("bwd_key_subset_dk_scale_dropped", "backward.py",
     "dk[b, g, valid] += scale * (dsj.T @ q[b, h, rows])", "dk[b, g, valid] += dsj.T @ q[b, h, rows]"),
    ("bwd_key_subset_row_term_from_values", "backward.py",
     "drow = (dob * o).sum(axis=1)", "drow = (dob * vb[rows]).sum(axis=1)"),
    ("bwd_key_subset_dv_from_scores", "backward.py",
     "dv[b, g, valid] += pj.T @ dob", "dv[b, g, valid] += dsj.T @ dob"),
    # FP8 form
    ("e4m3_ties_away_from_zero", "fp8.py",
     "up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1))", "up = frac >= 0.5"),
    ("e4m3_subnormal_exponent", "fp8.py",
     "np.ldexp(m / 8.0, 1 - _BIAS)", "np.ldexp(m / 8.0, -_BIAS)"),
    ("fp8_output_not_rescaled", "fp8.py",
     "acc = alpha[:, None] * acc + pq @ vb[j0:j0 + block]", "acc = acc + pq @ vb[j0:j0 + block]"),
    ("fp8_row_sum_not_rescaled", "fp8.py",
     "l = alpha * l + p.sum(axis=1)", "l = l + p.sum(axis=1)"),
]


def _run(name, fname, old, new):
    """Copy oracle/ and the pin suites to a scratch tree, plant the mutant (if any) and run the
    pins there.  Returns (pytest exit status, tail of its output)."""
    with tempfile.TemporaryDirectory(prefix="oracle_mutant_") as tmp:
        shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(tmp, "oracle"),
                        ignore=shutil.ignore_patterns("__pycache__"))
        os.makedirs(os.path.join(tmp, "tests"))
        for f in PIN_FILES + ["conftest.py"]:
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(tmp, "tests", f))
        shutil.copy(os.path.join(ROOT, "pytest.ini"), os.path.join(tmp, "pytest.ini"))
        if fname is not None:
            path = os.path.join(tmp, "oracle", fname)
            with open(path) as f:
                src = f.read()
            assert src.count(old) == 1, f"{name}: the mutated text must occur exactly once"
            with open(path, "w") as f:
                f.write(src.replace(old, new))
        env = {k: v for k, v in os.environ.items() if k != "PYTHONPATH"}
        env["PYTHONDONTWRITEBYTECODE"] = "1"
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            *[os.path.join("tests", f) for f in PIN_FILES]],
                           cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
        return r.returncode, (r.stdout + r.stderr)[-1500:]


@pytest.fixture(scope="module")
def outcomes():
    jobs = [("control", None, None, None)] + MUTANTS
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {j[0]: ex.submit(_run, *j) for j in jobs}
        return {k: f.result() for k, f in futs.items()}


def test_unmodified_copy_passes_every_pin(outcomes):
    code, out = outcomes["control"]
    assert code == 0, out


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_mutant_is_caught_by_a_pin(outcomes, name):
    code, out = outcomes[name]
    # 1 = some test failed (0 would mean every pin accepted the mistake; 2-4 = harness error)
    assert code == 1, f"mutant {name}: pytest exit status {code}\n{out}"

"""Plausible mistakes planted in a copy of the oracle must each fail a pin.

Every case copies ``oracle/`` into a temporary directory, replaces one
snippet of its source with a plausible mistake (a dropped term, a wrong
sign, a transposed index, another rounding rule), and runs the pin tests
against that copy in a child process.  The pins pass on the real oracle
(the other test files) and must fail on every mutant.  CPU only.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    # (file, original snippet, mistake, pin test file); the first is the
    # control: an unchanged copy, which must pass
    ("hadamard.py", "", "", "*"),
    ("hadamard.py", "bin(i & j)", "bin(i | j)", "test_oracle_hadamard.py"),
    ("hadamard.py", ">> (c & 31)", ">> (31 - (c & 31))", "test_oracle_hadamard.py"),
    ("hadamard.py", "((d[sl][None, :] * x[:, sl]) @ h.T)", "(d[sl][None, :] * (x[:, sl] @ h.T))",
     "test_oracle_hadamard.py"),
    ("hadamard.py", "@ h.T) / np.sqrt(float(block))", "@ h.T) / float(block)", "test_oracle_hadamard.py"),
    ("rtn.py", "lo = np.minimum(v.min(axis=2), 0.0)", "lo = v.min(axis=2)", "test_oracle_rtn.py"),
    ("rtn.py", "s = s16.astype(np.float64)", "s = np.where(s16 == 1, 1.0, (hi - lo) / qmax)", "test_oracle_rtn.py"),
    ("rtn.py", "np.rint(v / s[:, :, None]", "np.floor(0.5 + v / s[:, :, None]", "test_oracle_rtn.py"),
    ("rtn.py", "np.rint(-lo / s)", "np.ceil(-lo / s)", "test_oracle_rtn.py"),
    ("rtn.py", "wp.astype(np.float32)", "wp.astype(np.float16).astype(np.float32)", "test_oracle_rtn.py"),
    ("pack.py", "acc |= c << (bits * j)", "acc |= c << (bits * (per_run - 1 - j))", "test_oracle_pack.py"),
    ("pack.py", "out.append((acc >> (32 * w)) & 0xFFFFFFFF)",
     "out.append((acc >> (32 * (wpr - 1 - w))) & 0xFFFFFFFF)", "test_oracle_pack.py"),
    ("pack.py", "off.append(off[-1] + MIXED_ROWS * words_per_row(int(b), k))",
     "off.append(off[-1] + MIXED_ROWS * words_per_row(6, k))", "test_oracle_pack.py"),
    ("linear.py", "gidx = np.arange(k) // group", "gidx = np.arange(k) % (k // group)", "test_oracle_linear.py"),
    ("linear.py", "(q.astype(np.float64) - z64) * s64", "(q.astype(np.float64) + z64) * s64", "test_oracle_linear.py"),
    ("linear.py", "(q.astype(np.float64) - z64) * s64", "q.astype(np.float64) * s64 - z64", "test_oracle_linear.py"),
    ("linear.py", "xr = rht(x64, sign_bits)", "xr = x64", "test_oracle_linear.py"),
    ("contract.c", "acc += w[j * k + t] * x[i * k + t];", "acc += w[j * k + t] * x[t];", "test_oracle_linear.py"),
    ("contract.c", "for (int64_t t = 0; t < k; ++t)", "for (int64_t t = 1; t < k; ++t)", "test_oracle_linear.py"),
    ("embed.py", "return out.astype(out_dtype)", "return out.astype(np.float32).astype(out_dtype)",
     "test_oracle_embed.py"),
    ("embed.py", "if 0 <= r < n:", "if r < n:", "test_oracle_embed.py"),
    ("embed.py", "out[i] = dequant(q[r:r + 1]", "out[i] = dequant(q[r - 1:r]", "test_oracle_embed.py"),
]


@pytest.mark.parametrize("fname,orig,bad,pins", MUTANTS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTANTS)])
def test_mutant_is_caught(tmp_path, fname, orig, bad, pins):
    dst = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp*"))
    if orig:
        src = (dst / fname).read_text()
        assert src.count(orig) >= 1, f"snippet not found in {fname}: {orig}"
        (dst / fname).write_text(src.replace(orig, bad))
    shutil.copytree(os.path.join(ROOT, "tests"), tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py", "test_gpu*", "test_abi*"))
    shutil.copytree(os.path.join(ROOT, "workloads"), tmp_path / "workloads",
                    ignore=shutil.ignore_patterns("__pycache__"))
    env = dict(os.environ, PYTHONPATH=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    targets = [str(tmp_path / "tests" / p) for p in
               (["test_oracle_hadamard.py", "test_oracle_rtn.py", "test_oracle_pack.py",
                 "test_oracle_linear.py"] if pins == "*" else [pins])]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + targets,
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=300)
    if not orig:
        assert r.returncode == 0, r.stdout[-3000:]
        return
    assert r.returncode != 0, f"mutant survived: {fname}: {orig!r} -> {bad!r}\n{r.stdout[-2000:]}"

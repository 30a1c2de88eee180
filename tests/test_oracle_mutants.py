"""The oracle's pins catch plausible mistakes: each mutant below plants one mistake
in a copy of oracle/ref.py (a source-text replacement), and the pin suite
tests/test_oracle.py must fail against that copy. CPU only; the mutants never
leave a temporary directory."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REF = os.path.join(ROOT, "oracle", "ref.py")

# (name, original text, mutated text): each original occurs exactly once in ref.py
MUTANTS = [
    ("zero-point dropped from the codes", "q = np.clip(t + z[:, :, None].astype(np.float32), 0, qmax)",
     "q = np.clip(t + 0 * z[:, :, None].astype(np.float32), 0, qmax)"),
    ("zero-point sign flipped in dequantization", "return ((qg - zf) * sf).reshape(N, K)",
     "return ((qg + zf) * sf).reshape(N, K)"),
    ("floor instead of round-to-nearest", "t = np.rint(Wg / s[:, :, None]).astype(np.float32)",
     "t = np.floor(Wg / s[:, :, None]).astype(np.float32)"),
    ("half away from zero instead of half to even", "t = np.rint(Wg / s[:, :, None]).astype(np.float32)",
     "t = (np.sign(Wg / s[:, :, None]) * np.floor(np.abs(Wg / s[:, :, None]) + 0.5)).astype(np.float32)"),
    ("range divided by qmax + 1", "d = (rng / np.float32(qmax)).astype(np.float32)",
     "d = (rng / np.float32(qmax + 1)).astype(np.float32)"),
    ("codes computed with the unrounded scale", "s = s16.astype(np.float32)", "s = d"),
    ("no floor on the step", "d = np.maximum(d, FP16_MIN_NORMAL)", "d = d"),
    ("codes clamped one short", "q = np.clip(t + z[:, :, None].astype(np.float32), 0, qmax)",
     "q = np.clip(t + z[:, :, None].astype(np.float32), 0, qmax - 1)"),
    ("range forced to include 0", "mn = Wg.min(axis=2)", "mn = np.minimum(Wg.min(axis=2), 0)"),
    ("zero-point from the maximum", "zf = np.rint((-mn) / s).astype(np.float32)",
     "zf = np.rint((mx - mn) / s - mx / s).astype(np.float32) + 1"),
    ("4-bit nibbles in reverse order", "out |= q8[:, :, i] << np.uint32(4 * i)",
     "out |= q8[:, :, i] << np.uint32(4 * (7 - i))"),
    ("3-bit pair halves swapped",
     "out[:, :, w] |= (u[:, :, lo] << np.uint32(3 * i)) | (u[:, :, hi] << np.uint32(16 + 3 * i))",
     "out[:, :, w] |= (u[:, :, hi] << np.uint32(3 * i)) | (u[:, :, lo] << np.uint32(16 + 3 * i))"),
    ("3-bit split pair in the wrong bits",
     "out[:, :, b] |= (((u[:, :, lo] >> np.uint32(b)) & np.uint32(1)) << np.uint32(15)) | \\",
     "out[:, :, 2 - b] |= (((u[:, :, lo] >> np.uint32(b)) & np.uint32(1)) << np.uint32(15)) | \\"),
    ("split ties to the higher flat index", "chosen = np.sort(np.concatenate([above, ties[:need]]))",
     "chosen = np.sort(np.concatenate([above, ties[ties.size - need:]]))"),
    ("split leaves the value in the dense part", "Wd.reshape(-1)[chosen] = np.float32(0.0)", "pass"),
    ("sparse term drops the last entry of each row", "prod = x64[:, col] * v[None, :]           # [M, nnz]",
     "prod = x64[:, col] * v[None, :]; prod[:, np.maximum(row_ptr[1:].astype(np.int64) - 1, 0)] = 0"),
    ("dequantization with the neighbouring group's metadata",
     "zf = np.asarray(z).astype(np.float64)[:, :, None]",
     "zf = np.roll(np.asarray(z).astype(np.float64), 1, axis=1)[:, :, None]"),
    ("act-order groups by contiguous channels", "S = np.asarray(s).astype(np.float64)[:, g_idx]",
     "S = np.asarray(s).astype(np.float64)[:, np.arange(len(g_idx)) * (int(np.max(g_idx)) + 1) // len(g_idx)]"),
    ("INT8 scale over all channels, outliers included",
     "amax = np.abs(xf[:, keep]).max(axis=1) if keep.any() else np.zeros(M, np.float32)",
     "amax = np.abs(xf).max(axis=1)"),
    ("INT8 scale of amax / 128", "s = np.where(amax > 0, amax / np.float32(QX), np.float32(1.0)).astype(np.float32)",
     "s = np.where(amax > 0, amax / np.float32(QX + 1), np.float32(1.0)).astype(np.float32)"),
    ("W4A8 product without the row scale",
     "y = sx.astype(np.float64)[:, None] * (xq.astype(np.float64) @ W_hat.T)",
     "y = (xq.astype(np.float64) @ W_hat.T)"),
    ("low-rank components in reverse order", "return (x64 @ L1.T) @ L2.T", "return (x64 @ L1[::-1].T) @ L2.T"),
]


def test_every_mutant_applies_once():
    src = open(REF).read()
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, name


def _run_pins(tmp_path, old=None, new=None):
    """Run tests/test_oracle.py against a copy of the oracle package in tmp_path
    (first on the import path), with `old` replaced by `new` in its ref.py; the copy
    marks itself, so the run can show that it imported the copy."""
    pkg = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg, ignore=shutil.ignore_patterns("__pycache__"))
    src = (pkg / "ref.py").read_text()
    if old is not None:
        assert src.count(old) == 1
        src = src.replace(old, new)
    (pkg / "ref.py").write_text(src + "\nMUTANT_COPY = True\n")
    probe = tmp_path / "test_probe_copy.py"
    probe.write_text("import oracle.ref\n\ndef test_copy_is_imported():\n    assert oracle.ref.MUTANT_COPY\n")
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]))
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", str(probe),
                           os.path.join(ROOT, "tests", "test_oracle.py")], cwd=str(tmp_path), env=env,
                          capture_output=True, text=True, timeout=600)


@pytest.mark.slow
def test_unmutated_copy_passes(tmp_path):
    """Control: the harness imports the copy and the pins pass on it unchanged."""
    r = _run_pins(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, name, old, new):
    """The pin suite fails on this mutant of the oracle (and only the pins fail: the
    copy itself is imported)."""
    r = _run_pins(tmp_path, old, new)
    assert "test_probe_copy.py ." in r.stdout or "1 failed" not in r.stdout or r.returncode != 0
    assert r.returncode != 0, f"no pin fails for the mutant: {name}\n{r.stdout[-2000:]}"
    assert "test_copy_is_imported" not in r.stdout.split("short test summary")[-1], r.stdout[-2000:]

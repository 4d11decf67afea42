"""Planted mistakes in a copy of the oracle must each fail a pin.

Each mutant is the oracle's source with one plausible error (a dropped term,
a wrong sign or exponent, a transposed operand, a wrong rounding direction),
written to a temporary package and run against the unchanged pin tests in a
child process.  The unmutated copy must pass, so a failure is the mutant's."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ttq_oracle.py")
PINS = [os.path.join(ROOT, "tests", f) for f in (
    "test_oracle_colstats.py", "test_oracle_quantize.py", "test_oracle_pack.py",
    "test_oracle_lowrank.py", "test_oracle_linear.py", "test_oracle_refresh.py")]

MUTANTS = {
    "sum_not_mean": ("mean = powed.sum(axis=0) / T", "mean = powed.sum(axis=0)"),
    "lambda_outside_power": ("return (mean + lam) ** alpha", "return mean ** alpha + lam"),
    "root_of_norm": ("return (mean + lam) ** alpha", "return (mean ** (1.0 / p) + lam) ** alpha"),
    "scale_by_inverse_root": ("sq = np.sqrt(D32)", "sq = np.float32(1.0) / np.sqrt(D32)"),
    "no_zero_in_range": ("mn = np.minimum(grp.min(axis=2), zero32)", "mn = grp.min(axis=2)"),
    "scale_rounded_to_nearest": ("s16[low] = np.nextafter(s16[low], np.float16(np.inf))", "pass"),
    "zero_point_sign": ("z = np.clip(np.rint(-mn / s), zero32, N)", "z = np.clip(np.rint(mn / s), zero32, N)"),
    "floor_not_rint": ("codes = np.clip(np.rint(grp / s[:, :, None])", "codes = np.clip(np.floor(grp / s[:, :, None])"),
    "pack_big_endian": ("bit = q * k\n        w, off = divmod(bit, 32)\n        words", "bit = q * (31 - k)\n        w, off = divmod(bit, 32)\n        words"),
    "unscaled_input": ("Y = (X64 * rs[None, :]) @ Vh.T", "Y = X64 @ Vh.T"),
    "transposed_A": ("A = root[:, None] * Vt[:r, :]", "A = root[:, None] * Vt[:, :r].T"),
    "residual_sign": ("W16.astype(np.float64) - B.astype(np.float64) @ A.astype(np.float64)).astype(np.float16)",
                      "W16.astype(np.float64) + B.astype(np.float64) @ A.astype(np.float64)).astype(np.float16)"),
    "lowrank_term_dropped": ("Y = Y + (X64 @ A64.T) @ B64.T", "Y = Y"),
    "slot_order_inverted": ("SLOT_CODE8 = (0, 2, 4, 6, 1, 3, 5, 7)", "SLOT_CODE8 = (0, 4, 1, 5, 2, 6, 3, 7)"),
    "refresh_weight_by_d": ("    M = W64 * sq[None, :]\n    P = M.T", "    M = W64 * (sq * sq)[None, :]\n    P = M.T"),
    "refresh_no_unweighting": ("    A = Vn.T / sq[None, :]", "    A = Vn.T.copy()"),
    "refresh_unweighted_B": ("    B = M @ Vn\n", "    B = W64 @ Vn\n"),
    "refresh_not_orthonormalised": ("    Vn = Q * sign[None, :]", "    Vn = P / np.linalg.norm(P, axis=0)[None, :]"),
    "refresh_one_sided": ("    P = M.T @ (M @ V64)", "    P = M.T @ M[:, :V64.shape[1]]"),
}


def _run(tmp_path, source):
    pkg = tmp_path / "oracle"
    pkg.mkdir(exist_ok=True)
    (pkg / "ttq_oracle.py").write_text(source)
    (pkg / "__init__.py").write_text(open(os.path.join(ROOT, "oracle", "__init__.py")).read())
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([str(tmp_path), ROOT])
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "--rootdir", str(tmp_path), "-c", os.devnull, *PINS],
                          cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=600)
    return proc.returncode, proc.stdout[-2000:]


def test_unmutated_copy_passes(tmp_path):
    rc, out = _run(tmp_path, open(SRC).read())
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} no longer in the oracle"
    rc, out = _run(tmp_path, src.replace(old, new, 1))
    assert rc != 0, f"mutant {name} survived every pin:\n{out}"

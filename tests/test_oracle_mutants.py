"""The oracle's pins must catch plausible mistakes in the oracle.

Each case below plants one slip in a scratch copy of oracle/ref.py (a
transposed operand, a dropped term, a wrong sign, index or order) and runs
the oracle's pin files against that copy in a child process; the pins must
fail.  A control run with no change must pass.  Only the oracle is mutated,
on the CPU; the pins and the input generator are copied unchanged.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in oracle/ref.py, replacement)
MUTANTS = [
    ("int4 gate/up swapped",
     "return swiglu_ffn(a, W13[:, :I], W13[:, I:], W2)",
     "return swiglu_ffn(a, W13[:, I:], W13[:, :I], W2)"),
    ("fp16 gate/up swapped",
     "return swiglu_ffn(a, w13f[:I].T, w13f[I:].T, w2.astype(dtype).T)",
     "return swiglu_ffn(a, w13f[I:].T, w13f[:I].T, w2.astype(dtype).T)"),
    ("int4 down projection rows reversed",
     "W2 = dequant_gptq(*q2, dtype=dtype, bits=bits)     # [I, H]",
     "W2 = dequant_gptq(*q2, dtype=dtype, bits=bits)[::-1]     # [I, H]"),
    ("code order inside a word reversed",
     "q[i::per, :] = (qw >> np.uint32(bits * i)) & mask",
     "q[per - 1 - i::per, :] = (qw >> np.uint32(bits * i)) & mask"),
    ("zero order inside a word reversed",
     "z[:, i::per] = (qz >> np.uint32(bits * i)) & mask",
     "z[:, per - 1 - i::per] = (qz >> np.uint32(bits * i)) & mask"),
    ("group size 256 instead of 128",
     "g = np.arange(q.shape[0]) // GROUP",
     "g = np.arange(q.shape[0]) // (2 * GROUP)"),
    ("scale of group 0 used everywhere",
     "return (q.astype(dtype) - z[g, :].astype(dtype)) * s[g, :]",
     "return (q.astype(dtype) - z[g, :].astype(dtype)) * s[0 * g, :]"),
    ("silu sign flipped",
     "return a / (1.0 + np.exp(-a))",
     "return a / (1.0 + np.exp(a))"),
    ("ties to the higher expert index",
     "order = np.lexsort((np.arange(E), -L32[t].astype(np.float64)))",
     "order = np.lexsort((-np.arange(E), -L32[t].astype(np.float64)))"),
    ("always renormalised",
     "    if renormalize:\n        wts = wts / wts.sum(axis=1, keepdims=True)",
     "    if True:\n        wts = wts / wts.sum(axis=1, keepdims=True)"),
    ("butterfly rounds in reverse order",
     "for d in (32, 16, 8, 4, 2, 1):",
     "for d in (1, 2, 4, 8, 16, 32):"),
    ("chunks of 4 hidden elements per lane",
     "CHUNK = 8 ",
     "CHUNK = 4 "),
    ("gather not stable",
     "for p in range(n):                      # increasing p: stability",
     "for p in reversed(range(n)):"),
    ("sorted token taken modulo k",
     "sorted_token[:rows] = sorted_pair[:rows] // k",
     "sorted_token[:rows] = sorted_pair[:rows] % k"),
    ("ELB counts into layer 0",
     "out[layer, e] += 1",
     "out[0, e] += 1"),
    ("combine weights of the slots reversed",
     "out[t] += np.float64(weights[t, j]) * y_sorted[r].astype(dtype)",
     "out[t] += np.float64(weights[t, k - 1 - j]) * y_sorted[r].astype(dtype)"),
    ("shared gate ignored",
     "c = 1.0 if shared_scale is None else float(shared_scale[t])",
     "c = 1.0"),
    ("shared gate sign flipped",
     "gate = 1.0 / (1.0 + np.exp(-g32))",
     "gate = 1.0 / (1.0 + np.exp(g32))"),
    ("shared expert dropped from the layer",
     "sh = expert_ffn_f16(x, shared[\"w13\"], shared[\"w2\"], dtype)",
     "sh = 0 * expert_ffn_f16(x, shared[\"w13\"], shared[\"w2\"], dtype)"),
    ("AWQ factors multiplied instead of divided",
     "xa = np.asarray(xr).astype(dtype) / np.asarray(a13).astype(dtype)",
     "xa = np.asarray(xr).astype(dtype) * np.asarray(a13).astype(dtype)"),
    ("AWQ down-input factors dropped",
     "return (h / np.asarray(a2).astype(dtype)) @ W2",
     "return h @ W2"),
    ("rms eps outside the root",
     "return a / np.sqrt(np.mean(a * a, axis=-1, keepdims=True) + eps)",
     "return a / (np.sqrt(np.mean(a * a, axis=-1, keepdims=True)) + eps)"),
]


def _tree(tmp, src_text):
    os.makedirs(os.path.join(tmp, "oracle"))
    os.makedirs(os.path.join(tmp, "tests", "golden"))
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(tmp, "oracle"))
    with open(os.path.join(tmp, "oracle", "ref.py"), "w") as f:
        f.write(src_text)
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(tmp, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    for p in glob.glob(os.path.join(ROOT, "tests", "golden", "*")):
        shutil.copy(p, os.path.join(tmp, "tests", "golden"))
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    pins = [p for p in pins if not p.endswith("test_oracle_mutants.py")]
    for p in pins + [os.path.join(ROOT, "tests", "conftest.py")]:
        shutil.copy(p, os.path.join(tmp, "tests"))
    return [os.path.join(tmp, "tests", os.path.basename(p)) for p in pins]


def _run_pins(tmp, files):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "--rootdir", tmp, *files], cwd=tmp, env=env, capture_output=True,
                       text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def oracle_source():
    with open(os.path.join(ROOT, "oracle", "ref.py")) as f:
        return f.read()


def test_control_copy_passes(tmp_path, oracle_source):
    files = _tree(str(tmp_path), oracle_source)
    rc, out = _run_pins(str(tmp_path), files)
    assert rc == 0, out


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, oracle_source, name, old, new):
    assert oracle_source.count(old) == 1, f"mutation site for '{name}' not found once"
    files = _tree(str(tmp_path), oracle_source.replace(old, new))
    rc, out = _run_pins(str(tmp_path), files)
    assert rc != 0, f"'{name}' passed every pin:\n{out}"

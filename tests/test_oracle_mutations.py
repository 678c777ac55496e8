"""The oracle's pins catch plausible mistakes: each case plants one mistake in a copy of
the oracle (on the CPU) and checks that the pin tests then fail."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle_logprob.py", "tests/test_oracle_diagnostics.py",
             "tests/test_oracle_lmhead.py", "tests/test_oracle_training.py",
             "tests/test_oracle_sharding.py"]

MUTATIONS = [
    ("logprob.py", "lpt = xt - lt", "lpt = lt - xt"),                          # sign
    ("logprob.py", "return m + math.log(", "return math.log("),                 # dropped term
    ("logprob.py", "xt = float(train_row[y])", "xt = float(train_row[y - 1])"),  # index
    ("logprob.py", "lpt - lpr, bool(bad)", "lpr - lpt, bool(bad)"),             # drift sign
    ("logprob.py", "<< np.uint32(16)", "<< np.uint32(15)"),                      # widening
    ("logprob.py", "return att & act", "return att | act"),                      # active rule
    ("logprob.py", 'layout == "right" and (not a2[b, t]) and a2[b, t + 1]',
     'layout == "right" and a2[b, t] and (not a2[b, t + 1])'),                   # padding side
    ("logprob.py", "(ids < 0) | (ids >= V)", "(ids < 0) | (ids > V)"),           # OOV bound
    ("diagnostics.py", "k = (q_num * n + q_den - 1) // q_den", "k = (q_num * n) // q_den"),
    ("diagnostics.py", "a[nearest_rank(n, 99, 100) - 1]", "a[nearest_rank(n, 95, 100) - 1]"),
    ("diagnostics.py", "lo_edge = 1.0 - eps_low", "lo_edge = 1.0 - eps_high"),
    ("diagnostics.py", "math.expm1(v) - v for v", "math.expm1(v) + v for v"),
    ("diagnostics.py", "math.fsum(abs(v) for v in vals) / n", "math.fsum(vals) / n"),
    ("diagnostics.py", "math.fsum(math.exp(v) for v in vals) / n",
     "math.fsum(math.exp(v) for v in vals) / (n + 1)"),
    ("diagnostics.py", 'out["argmax_row"] = int(r)\n            break',
     'out["argmax_row"] = int(r)'),                                              # last tie
    ("logprob.py", "            x = x * v", "            x = x / v"),                 # scale
    ("logprob.py", "x = v * np.tanh(x / v)", "x = np.tanh(x / v)"),               # soft cap
    ("logprob.py", "        V = int(vocab_real)", "        pass"),                      # mask
    ("training.py", "-math.fsum((p[nz] * (x[nz] - lse)).tolist())",
     "-math.fsum((p[nz] * x[nz]).tolist())"),                                   # entropy
    ("training.py", "g[int(y)] += 1.0", "g[int(y)] -= 1.0"),                      # dlogits
    ("training.py", "d = d * (1.0 - t * t)", "d = d * (1.0 - t)"),                # cap slope
    ("training.py", "            d = d / v", "            d = d * v"),              # temp slope
    ("training.py", "g = dlogits_row(z, y) * chain_derivative(x, transform)",
     "g = dlogits_row(z, y)"),                                                   # chain rule
    ("training.py", "out[r, :Vr] = np.nan", "out[r, :Vr] = 0.0"),                 # bad id
    ("diagnostics.py", "math.fsum(-v for v in vals) / n", "math.fsum(vals) / n"),  # kl sign
    ("diagnostics.py", 'st["argmax_row"] += lo', 'st["argmax_row"] += 0'),         # local row
    ("diagnostics.py", "if not 0 <= lo <= hi <= N:", "if not 0 <= lo <= N:"),       # bounds
    ("sharding.py", "z * math.exp(m - M) for m, z in live", "z for m, z in live"),   # rescale
    ("sharding.py", "if boundaries[s] <= y < boundaries[s + 1]:",
     "if boundaries[s] <= y <= boundaries[s + 1]:"),                              # owner
    ("sharding.py", "return M + math.log(", "return math.log("),                  # max term
    ("lmhead.py", "z[i, int(ids[r])]", "z[i, int(ids[i])]"),
    ("lmhead.py", "z = apply_transforms(h @ weight_f64, transforms)",
     "z = apply_transforms(h[:, ::-1] @ weight_f64, transforms)"),               # reversed K
    ("lmhead.py", "z = apply_transforms(h @ weight_f64, transforms)",
     "z = h @ weight_f64"),                                                      # chain dropped
]


def _run_mutation(tmp_root, idx, fname, old, new):
    tmp_path = os.path.join(tmp_root, f"m{idx}")
    os.makedirs(tmp_path)
    dst = os.path.join(tmp_path, "oracle")
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("__pycache__"))
    path = os.path.join(dst, fname)
    src = open(path).read()
    if src.count(old) != 1:
        return f"mutation anchor not found once: {old!r}"
    open(path, "w").write(src.replace(old, new))
    for t in PIN_TESTS:
        shutil.copy(os.path.join(ROOT, t), os.path.join(tmp_path, os.path.basename(t)))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp_path, "golden"))
    env = dict(os.environ, PYTHONPATH=f"{tmp_path}{os.pathsep}{ROOT}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "--rootdir", tmp_path] +
                       [os.path.join(tmp_path, os.path.basename(t)) for t in PIN_TESTS],
                       cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)
    if r.returncode == 0:
        return f"planted mistake survived the pins: {new!r}\n{r.stdout[-2000:]}"
    return None


@pytest.fixture(scope="module")
def mutation_results(tmp_path_factory):
    from concurrent.futures import ThreadPoolExecutor
    root = str(tmp_path_factory.mktemp("mutations"))
    with ThreadPoolExecutor(max_workers=6) as ex:
        futs = [ex.submit(_run_mutation, root, i, *m) for i, m in enumerate(MUTATIONS)]
        return [f.result() for f in futs]


@pytest.mark.parametrize("idx", range(len(MUTATIONS)),
                         ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_pins_catch_planted_mistake(mutation_results, idx):
    err = mutation_results[idx]
    assert err is None, err

"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutation below plants one mistake in a copy of oracle/sol_oracle.py in a
temporary directory and runs tests/test_oracle_pins.py against that copy in a
subprocess: the run must fail. An unmutated copy must pass, so a failure can
only come from the planted mistake. Nothing here touches the HIP library.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "sol_oracle.py")).read()

# name: (exact text in the oracle, replacement)
MUTATIONS = {
    # the correction (virtual tokens of unselected blocks)
    "multiplicity_64_dropped": ("w = BLOCK * np.exp(", "w = 1.0 * np.exp("),
    "block_sum_for_mean_value": ("num += w @ vbar[dropped]", "num += w @ (BLOCK * vbar[dropped])"),
    "virtual_term_only_in_denominator": ("num += w @ vbar[dropped]", "pass"),
    "row_logit_unscaled": ("virt = (qi @ kbar_rows[dropped].T) / math.sqrt(d)",
                           "virt = (qi @ kbar_rows[dropped].T)"),
    # routing
    "tau_sign": ("return mu + mu.dtype.type(beta) * sigma", "return mu - mu.dtype.type(beta) * sigma"),
    "variance_for_std": ("sigma = np.sqrt((dev * dev).mean(axis=1))", "sigma = (dev * dev).mean(axis=1)"),
    "sample_std": ("sigma = np.sqrt((dev * dev).mean(axis=1))",
                   "sigma = np.sqrt((dev * dev).sum(axis=1) / (dev.shape[1] - 1))"),
    "proxy_unscaled": ("return (qbar @ kbar.T) * scale", "return (qbar @ kbar.T)"),
    "proxy_transposed": ("return (qbar @ kbar.T) * scale",
                         "return ((kbar @ qbar.T) * scale) if qbar.shape[0] == kbar.shape[0] else (qbar @ kbar.T) * scale"),
    "non_strict_test": ("return s_hat > tau[:, None]", "return s_hat >= tau[:, None]"),
    "covariance_uncentred": ("c = kbar - m[None, :]", "c = kbar"),
    # exact attention
    "exact_logits_unscaled": ("logits = (qi @ k_kept.T) / math.sqrt(d)", "logits = (qi @ k_kept.T)"),
    # routing baselines
    "topk_ties_to_higher_index": ("        order = sorted(range(nb), key=lambda j: (-float(s_hat[i, j]), j))\n"
                                  "        keep[i, order[:k]] = True",
                                  "        order = sorted(range(nb), key=lambda j: (-float(s_hat[i, j]), -j))\n"
                                  "        keep[i, order[:k]] = True"),
    "topp_block_reaching_p_dropped": ("            keep[i, j] = True\n            acc += prob[j]\n"
                                      "            if acc >= p:\n                break",
                                      "            acc += prob[j]\n            if acc >= p:\n                break\n"
                                      "            keep[i, j] = True"),
    # joint attention text segment
    "text_columns_off_by_one": ("mask[:, t0:] = True", "mask[:, t0 + 1:] = True"),
    "text_rows_off_by_one": ("mask[qb >= t0, :] = True", "mask[qb > t0, :] = True"),
}


def _run_pins(tmp, src: str) -> subprocess.CompletedProcess:
    os.makedirs(os.path.join(tmp, "oracle"))
    with open(os.path.join(tmp, "oracle", "sol_oracle.py"), "w") as f:
        f.write(src)
    open(os.path.join(tmp, "oracle", "__init__.py"), "w").close()
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp, "tests", "golden"))
    for name in ("test_oracle_pins.py", "conftest.py", "__init__.py"):
        shutil.copy(os.path.join(ROOT, "tests", name), os.path.join(tmp, "tests", name))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    env.pop("PYTHONPATH", None)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "tests/test_oracle_pins.py"], cwd=tmp, env=env, capture_output=True,
                          text=True, timeout=600)


def test_unmutated_copy_passes(tmp_path):
    r = _run_pins(str(tmp_path), SRC)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_fails_a_pin(name, tmp_path):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, f"mutation {name}: anchor text not found once in the oracle"
    r = _run_pins(str(tmp_path), SRC.replace(old, new))
    assert r.returncode != 0, f"mutation {name} passed every pin:\n{r.stdout[-1500:]}"

"""The oracle's pins must catch plausible mistakes.

Each case copies oracle.c, plants one mistake (a wrong index, a transposed
operand, an off-by-one expert boundary, a dropped term, truncation instead
of rounding, a flipped sign), builds the copy on the CPU and runs the pin
suite against it in a fresh process: the suite has to fail.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "fwd_wrong_weight_index": ("const uint16_t *w = W + ((int64_t)e * N + n) * K;",
                               "const uint16_t *w = W + ((int64_t)e * N + n) * K + 1;"),
    "dgrad_transposed_weight": ("bf16_value(w[n * K + k])", "bf16_value(w[k * N + n])"),
    "wgrad_range_off_by_one": ("for (int64_t t = o[e]; t < (int64_t)o[e + 1]; ++t)",
                               "for (int64_t t = o[e] + 1; t < (int64_t)o[e + 1]; ++t)"),
    "expert_boundary": ("if (t < (int64_t)o[e + 1])", "if (t <= (int64_t)o[e + 1])"),
    "router_dropped_term": ("s += xh * wh + xh * wl + xl * wh;", "s += xh * wh + xh * wl;"),
    "bf16_truncation": ("r = rint(x / spacing) * spacing;", "r = trunc(x / spacing) * spacing;"),
    "wgrad_sign": ("double p = bf16_value(G[t * N + n]) * bf16_value(X[t * K + k]);",
                   "double p = -bf16_value(G[t * N + n]) * bf16_value(X[t * K + k]);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert before in src, "mutation site moved; update the mutation table"
    for d in ("oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    (tmp_path / "oracle" / "oracle.c").write_text(src.replace(before, after))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0, f"planted mistake {name} went unnoticed:\n{r.stdout[-2000:]}"

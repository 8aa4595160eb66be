"""Plants plausible mistakes in copies of the CPU oracle (on the CPU) and
checks that at least one pin catches each of them.  This is what makes the
pins trustworthy: a dropped term, a wrong sign or index, swapped weights or a
reciprocal in place of a division all fail a pin."""
import ctypes
import os
import subprocess
import sys

import pytest

import oracle
from oracle import build as oracle_build
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.LIB_PATH), "dl_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("sum_drops_running_term", "sum[j] = sum[j] + c;", "sum[j] = c;"),
    ("first_fold_adds_to_stale", "if (first)\n            sum[j] = c;\n        else\n            sum[j] = sum[j] + c;",
     "sum[j] = sum[j] + c;"),
    ("mean_reciprocal_multiply", "float g = sum[j] / N;", "float g = sum[j] * (1.0f / N);"),
    ("mean_wrong_count", "float N = (float)count;", "float N = (float)(count + 1);"),
    ("ema_weights_swapped", "ema[j] = beta * ema[j] + one_minus_beta * g;",
     "ema[j] = one_minus_beta * ema[j] + beta * g;"),
    ("ema_constant_0p1", "float one_minus_beta = 1.0f - beta;\n#pragma omp parallel for schedule(static)\n    for (int64_t j = 0; j < n; ++j) {\n        float g",
     "float one_minus_beta = 0.1f;\n#pragma omp parallel for schedule(static)\n    for (int64_t j = 0; j < n; ++j) {\n        float g"),
    ("standalone_ema_swapped", "ema[j] = beta * ema[j] + one_minus_beta * g[j];",
     "ema[j] = beta * g[j] + one_minus_beta * ema[j];"),
    ("delta_sign_flipped", "float d = theta[j] - oracle_ckpt_value(ckpt, dtype, j);",
     "float d = oracle_ckpt_value(ckpt, dtype, j) - theta[j];"),
    ("delta_unweighted", "float w = (float)tokens;", "float w = 1.0f;"),
    ("delta_first_not_copied", "if (first)\n            acc[j] = p;\n        else\n            acc[j] = acc[j] + p;",
     "acc[j] = acc[j] + p;"),
    ("nesterov_old_momentum", "float u = dbar + mu * m_new;", "float u = dbar + mu * m[j];"),
    ("nesterov_drops_gradient", "float u = dbar + mu * m_new;", "float u = mu * m_new;"),
    ("nesterov_heavy_ball", "float u = dbar + mu * m_new;", "float u = m_new;"),
    ("nesterov_dampened", "float m_new = mu * m[j] + dbar;",
     "float m_new = mu * m[j] + (1.0f - mu) * dbar;"),
    ("nesterov_step_sign", "float theta_new = theta[j] - lr * u;",
     "float theta_new = theta[j] + lr * u;"),
    ("nesterov_wrong_total", "float W = (float)total_tokens;", "float W = (float)(total_tokens - 1);"),
    ("nesterov_ema_of_old_global",
     "theta[j] = theta_new;\n        if (ema)\n            ema[j] = beta * ema[j] + one_minus_beta * theta_new;",
     "if (ema)\n            ema[j] = beta * ema[j] + one_minus_beta * theta[j];\n        theta[j] = theta_new;"),
    ("nesterov_momentum_not_stored", "m[j] = m_new;", "m[j] = m[j];"),
    ("bf16_wrong_shift", "((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    ("adopt_sign_flipped", "float shift = g[j] - oracle_ckpt_value(pushed, dtype, j);",
     "float shift = oracle_ckpt_value(pushed, dtype, j) - g[j];"),
    ("adopt_replaces", "theta[j] = theta[j] + shift;", "theta[j] = g[j];"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutant {name}: original text not found in the oracle"
    mutated = src.replace(old, new, 1)
    c = tmp_path / f"{name}.c"
    c.write_text(mutated)
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, "-Wno-unused-variable",
                    "-Wno-unused-but-set-variable",
                    "-Wno-unused-parameter", "-o", str(so), str(c)], check=True)
    return oracle.Oracle(str(so))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    orc = _build_mutant(tmp_path, name, old, new)
    caught = None
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught = pin.__name__
            break
    assert caught, f"no pin catches the planted mistake {name}"

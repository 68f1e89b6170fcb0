"""Plants plausible mistakes in a temporary copy of the oracle (on the CPU
only) and checks that the pins in test_oracle_pins.py, test_oracle_multi.py
and test_oracle_quant.py catch every one."""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "min instead of max per channel": ("terms[d] = a > c ? a : c;", "terms[d] = a < c ? a : c;"),
    "sign slip on the min row": ("double a = qd * bf16_value(lo[d]);", "double a = -qd * bf16_value(lo[d]);"),
    "last channel dropped": ("double u = orc_exact_sum(terms, D, &st);", "double u = orc_exact_sum(terms, D - 1, &st);"),
    "first head instead of group max": ("if (u > best) best = u;", "if (h == g * G) best = u;"),
    "ties to the highest id": ("return (a->id > b->id) - (a->id < b->id);", "return (a->id < b->id) - (a->id > b->id);"),
    "local window one page short": ("for (int64_t j = P - pol->n_local_pages; j < P; j++)",
                                    "for (int64_t j = P - pol->n_local_pages + 1; j < P; j++)"),
    "one sink page too many": ("j < P && j < pol->n_sink_pages; j++) flags[j] = 1;",
                               "j < P && j <= pol->n_sink_pages; j++) flags[j] = 1;"),
    "value layout transposed": ("return bf16_value(v_pool[(ph * lay->head_dim_v + dv) * lay->page_size + t]);",
                                "return bf16_value(v_pool[(ph * lay->page_size + t) * lay->head_dim_v + dv]);"),
    "token past the end attended": ("int use = pos < L && ", "int use = pos <= L && "),
    "scale dropped": ("s_buf[n] = scale * dot;", "s_buf[n] = dot;"),
    "summary over the whole page": ("for (int32_t t = 1; t < valid; t++) {", "for (int32_t t = 1; t < ps; t++) {"),
    "round half up": ("if (round_bit && (sticky || (M & 1ULL))) {", "if (round_bit) {"),
    "window one token longer": ("if (a < sink_end || e > win_begin) flags[j] = 1;",
                                "if (a < sink_end || e >= win_begin) flags[j] = 1;"),
    "static mask ignores the sink": ("(!st || pos < sink_end || pos >= win_begin)", "(!st || pos >= win_begin)"),
    # multi-query step
    "drafts scored by the last one only": ("for (int32_t r = 0; r < nq * G; r++) {",
                                           "for (int32_t r = (nq - 1) * G; r < nq * G; r++) {"),
    "every draft stops at the first draft": ("int64_t L = (int64_t)bat->seq_lens[b] - nq + 1 + i;",
                                             "int64_t L = (int64_t)bat->seq_lens[b] - nq + 1;"),
    "draft sees the next draft": ("int64_t L = (int64_t)bat->seq_lens[b] - nq + 1 + i;",
                                  "int64_t L = (int64_t)bat->seq_lens[b] - nq + 2 + i - (i == nq - 1);"),
    "static union not widened": ("wide.window_tokens = pol->window_tokens + nq - 1;",
                                 "wide.window_tokens = pol->window_tokens;"),
    "empty window widened": ("if (pol->window_tokens > 0) wide.window_tokens",
                             "if (pol->window_tokens >= 0) wide.window_tokens"),
    # quantised pages
    "step over four levels": ("float st = d / 3.0f;", "float st = d / 4.0f;"),
    "codes truncated": ("c = nearbyintf(r);", "c = truncf(r);"),
    "quantised region one page too long": ("num_pages(bat->seq_lens[b], ps) - qz->residual_pages : 0;",
                                           "num_pages(bat->seq_lens[b], ps) - qz->residual_pages + 1 : 0;"),
    "binary16 rounds toward zero": ("double n = nearbyint(ldexp(a, 10 - E));", "double n = trunc(ldexp(a, 10 - E));"),
    "zero point at the maximum": ("uint16_t m16 = half_bits(mn), s16 = half_bits(st);",
                                  "uint16_t m16 = half_bits(mx), s16 = half_bits(st);"),
}
PIN_FILES = ["test_oracle_pins.py", "test_oracle_multi.py", "test_oracle_quant.py"]


def _run_mutant(item):
    name, (old, new) = item
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) == 1, "mutation anchor not unique: " + name
    d = tempfile.mkdtemp(prefix="orc_mut_")
    try:
        shutil.copy(os.path.join(ROOT, "oracle", "oracle.h"), d)
        with open(os.path.join(d, "oracle.c"), "w") as f:
            f.write(src.replace(old, new))
        so = os.path.join(d, "liboracle_mut.so")
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-shared",
                               "-fPIC", os.path.join(d, "oracle.c"), "-o", so, "-lm"])
        env = dict(os.environ, QASP_ORACLE_LIB=so)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] +
                           [os.path.join(ROOT, "tests", f) for f in PIN_FILES],
                           env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
        # caught = a pin test failed (not a crash, import error or collection error)
        caught = r.returncode == 1 and " failed" in r.stdout and "error" not in r.stdout.split("\n")[-2]
        return name, caught
    finally:
        shutil.rmtree(d, ignore_errors=True)


def test_every_planted_mistake_is_caught():
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = dict(ex.map(_run_mutant, MUTANTS.items()))
    survivors = [n for n, caught in results.items() if not caught]
    assert not survivors, "pins missed: %s" % survivors

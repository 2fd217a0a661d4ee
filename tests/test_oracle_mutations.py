"""The oracle's pins have teeth: each planted mistake - a plausible slip in the C
oracle's mask, scale, head mapping, slot mapping, format decoding or softmax - makes
the pin suite fail.  Every mutant is applied to a temporary copy of
oracle/kvattn_oracle.c, built with the oracle's own build step, and the pin tests
run against it in a subprocess (CPU only; the library is not involved)."""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvattn_oracle.c")
PINS = ["tests/test_oracle.py", "tests/test_tree_oracle.py"]

# (name, exact text in the oracle, what it becomes)
MUTANTS = [
    ("window off by one", "(p >= P - window + 1)", "(p >= P - window)"),
    ("no 1/sqrt(d) scale", "w[j] = s * scale;", "w[j] = s;"),
    ("GQA heads interleaved", "const int kvh = h / g;", "const int kvh = h % pr->num_kv_heads;"),
    ("row position one early", "int64_t P = T - q_len + i;", "int64_t P = T - q_len + i - 1;"),
    ("ring rolls over the whole capacity",
     "n_sink + (p - n_sink) % (capacity - n_sink)", "n_sink + (p - n_sink) % capacity"),
    ("page table ignored", "int64_t phys = block_table[(int64_t)b * blocks_per_seq + page];",
     "int64_t phys = (int64_t)b * blocks_per_seq + page;"),
    ("binary16 exponent bias", "ldexp((double)(m + 1024), e - 25)",
     "ldexp((double)(m + 1024), e - 24)"),
    ("no max subtraction", "w[j] = exp(w[j] - m);", "w[j] = exp(w[j]);"),
    ("E4M3 exponent bias", "ldexp((double)(m + 8), e - 10)", "ldexp((double)(m + 8), e - 11)"),
    ("tree prefix off by one", "if (p < P0) return 1;", "if (p <= P0) return 1;"),
    ("V scale dropped", "(load_elem(vc, kvt, vbase + d) * vs)", "load_elem(vc, kvt, vbase + d)"),
]


def _run_pins_against(name, old, new, tmp):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutant {name!r}: its text must occur once in the oracle"
    src = os.path.join(tmp, f"m{abs(hash(name)) % 10**8}.c")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    lib = obuild.build(src=src, lib=src[:-2] + ".so")
    env = dict(os.environ, KVATTN_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True)
    return name, r.returncode, r.stdout[-600:]


def test_every_planted_mistake_fails_a_pin():
    # the control: an unchanged copy, built and loaded the same way, passes every pin
    control = ("unchanged copy", "int oracle_max_threads(void) {", "int oracle_max_threads(void) {")
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(4) as ex:
            results = list(ex.map(lambda m: _run_pins_against(*m, tmp), [control] + MUTANTS))
    assert results[0][1] == 0, "the unchanged copy fails the pins:\n" + results[0][2]
    survivors = [(n, out) for n, rc, out in results[1:] if rc != 1]
    # pytest exits 1 when a test failed; anything else (0: all passed, 2+: errors) is a miss
    assert not survivors, "mutants the pins did not catch:\n" + "\n".join(
        f"--- {n}\n{out}" for n, out in survivors)

"""The pins catch plausible mistakes in the oracle.

Each case compiles a copy of oracle/oracle.c with one mistake planted (a
dropped scale, a transposed layout index, a wrong GQA map, an off-by-one, a
wrong rounding tie, a merge without its rescale, a wrong free-list end, ...)
and runs the oracle pins against that build in a child process: every mutant
must fail at least one pin.  An unplanted copy built the same way must pass,
which shows that the child really ran the pins on the copy.  Everything here
runs on the CPU; nothing is planted in the library under test.
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("k_scale dropped",
     "p->BS, X)) * p->k_scale;", "p->BS, X));"),
    ("v_scale dropped",
     "p->D, p->BS)) * p->v_scale;", "p->D, p->BS));"),
    ("score scale dropped",
     "sc[t - t0] = p->scale * acc;", "sc[t - t0] = acc;"),
    ("GQA map interleaved (h mod Hkv)",
     "int G = p->Hq / p->Hkv, g = h / G;", "int G = p->Hq / p->Hkv, g = h % p->Hkv;"),
    ("K tile token-major instead of [D/X][BS][X]",
     "return (((b * H + h) * (D / X) + d / X) * BS + o) * X + d % X;",
     "return (((b * H + h) * BS + o) * (D / X) + d / X) * X + d % X;"),
    ("V tile [BS][D] instead of [D][BS]",
     "return ((b * H + h) * D + d) * BS + o;", "return ((b * H + h) * BS + o) * D + d;"),
    ("normaliser skips the last token",
     "for (int t = 0; t < L; ++t) sum += exp(sc[t] - m);",
     "for (int t = 0; t + 1 < L; ++t) sum += exp(sc[t] - m);"),
    ("block offset from the wrong index",
     "int64_t o = t % p->BS;\n", "int64_t o = (t / p->BS) % p->BS;\n"),
    ("E4M3 exponent bias 8",
     "mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("E4M3 ties to odd",
     "(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)"),
    ("bf16 ties away from zero",
     "return (((lo >> 16) & 1) == 0) ? (uint16_t)(lo >> 16) : (uint16_t)(hi >> 16);",
     "return (uint16_t)(hi >> 16);"),
    ("fp8 cache write multiplies by the scale",
     "float q = x / scale;", "float q = x * scale;"),
    ("cache write offset from the block index",
     "int64_t b = slot / block_size, o = slot % block_size;",
     "int64_t b = slot / block_size, o = (slot / block_size) % block_size;"),
    ("split merge without the partition rescale",
     "Lam += lp[part] * exp(mp[part] - M);", "Lam += lp[part];"),
    ("freed block returned to the head of the free list",
     "bm->fifo[(bm->head + bm->count) % bm->num_blocks] = blk;",
     "bm->head = (bm->head + bm->num_blocks - 1) % bm->num_blocks;\n"
     "      bm->fifo[bm->head] = blk;"),
]


def run_pins(lib_path):
    env = dict(os.environ, PKV_ORACLE_LIB=lib_path, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_oracle_pins.py")]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def build_copy(tmp_path, name, text, repl):
    src = open(O.SRC).read()
    if text is not None:
        assert src.count(text) == 1, f"{name}: the text to replace is not unique in oracle.c"
        src = src.replace(text, repl)
    path = os.path.join(str(tmp_path), "oracle_copy.c")
    with open(path, "w") as f:
        f.write(src)
    return O.compile_to(path, os.path.join(str(tmp_path), "liboracle_copy.so"))


def test_unplanted_copy_passes_the_pins(tmp_path):
    r = run_pins(build_copy(tmp_path, "unplanted", None, None))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,text,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, name, text, repl):
    r = run_pins(build_copy(tmp_path, name, text, repl))
    assert r.returncode != 0, f"mistake not caught by any pin: {name}\n" + r.stdout[-2000:]

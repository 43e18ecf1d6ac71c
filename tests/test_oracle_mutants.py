"""The pins catch plausible mistakes in the oracle.

Each case compiles a copy of oracle/oracle.c with one mistake planted (a
dropped scale, a transposed layout index, a wrong GQA map, an off-by-one, a
wrong rounding tie, a merge without its rescale, a wrong free-list end, ...)
and runs the oracle pins against that build in a child process: every mutant
must fail at least one pin.  An unplanted copy built the same way must pass,
which shows that the child really ran the pins on the copy.  The Python
oracles (prefix caching, the batching simulation) get the same treatment:
a planted copy of the module replaces it in a child that runs only their
pins (not the library-against-oracle comparisons).  Everything here runs on
the CPU; nothing is planted in the library under test.
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
    ("prefill: a query row skips its own token",
     "    const int n = pos + 1;\n", "    const int n = pos > 0 ? pos : 1;\n"),
    ("prefill: query position counted from the chunk start",
     "const int pos = context_lens[s] - C + (int)(i - query_start[s]);",
     "const int pos = (int)(i - query_start[s]);"),
    ("prefill: k_scale dropped",
     "X)) *\n                    p.k_scale;", "X));"),
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


# (module, name, text in oracle/<module>.py, replacement, pin selection)
PREFIX_PINS = "not matches_oracle"
SIM_PINS = "not matches_oracle and not native"
PY_MUTANTS = [
    ("prefix_cache", "LRU evicts the newest released block",
     "victim = next(iter(self.lru))", "victim = next(reversed(self.lru))", PREFIX_PINS),
    ("prefix_cache", "eviction keeps the evicted block's descendants",
     "        for c in self.children.pop(b, []):\n            self._uncache(c)",
     "        self.children.pop(b, [])", PREFIX_PINS),
    ("prefix_cache", "a prompt reuses the block holding its last token",
     "for i in range((n - 1) // self.BS if n > 0 else 0):", "for i in range(n // self.BS):",
     PREFIX_PINS),
    ("prefix_cache", "a released cached block goes straight to the free list",
     "            if b in self.key_of:\n                self.lru[b] = None",
     "            if False:\n                self.lru[b] = None", PREFIX_PINS),
    ("batching_sim", "preemption takes the earliest admitted request",
     "victim = [x for x in running if alive[x]][-1]",
     "victim = [x for x in running if alive[x]][0]", SIM_PINS),
    ("batching_sim", "static reservation one block too many",
     "mb = -(-max_model_len // BS)", "mb = -(-max_model_len // BS) + 1", SIM_PINS),
    ("batching_sim", "admission up to max_num_seqs + 1",
     "while waiting and len(running) < max_num_seqs:",
     "while waiting and len(running) <= max_num_seqs:", SIM_PINS),
]

TEST_FILE = {"prefix_cache": "test_prefix_cache.py", "batching_sim": "test_batching_sim.py"}


def run_py_pins(mod, path, select):
    """Child process: the planted module replaces oracle.<mod>, then pytest
    runs the module's pins."""
    boot = (
        "import sys, importlib.util\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import oracle\n"
        f"spec = importlib.util.spec_from_file_location('oracle.{mod}', {path!r})\n"
        "m = importlib.util.module_from_spec(spec)\n"
        f"sys.modules['oracle.{mod}'] = m\n"
        "spec.loader.exec_module(m)\n"
        f"oracle.{mod} = m\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', '-m', 'not gpu', '-k', "
        f"{select!r}, {os.path.join(ROOT, 'tests', TEST_FILE[mod])!r}]))\n")
    return subprocess.run([sys.executable, "-c", boot], cwd=ROOT, capture_output=True, text=True,
                          timeout=600)


def py_copy(tmp_path, mod, text, repl):
    src = open(os.path.join(ROOT, "oracle", mod + ".py")).read()
    if text is not None:
        assert src.count(text) == 1, f"{mod}: the text to replace is not unique"
        src = src.replace(text, repl)
    path = os.path.join(str(tmp_path), mod + "_copy.py")
    with open(path, "w") as f:
        f.write(src)
    return path


@pytest.mark.parametrize("mod", ["prefix_cache", "batching_sim"])
def test_unplanted_python_oracle_passes_its_pins(tmp_path, mod):
    select = PREFIX_PINS if mod == "prefix_cache" else SIM_PINS
    r = run_py_pins(mod, py_copy(tmp_path, mod, None, None), select)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]


@pytest.mark.parametrize("mod,name,text,repl,select", PY_MUTANTS, ids=[m[1] for m in PY_MUTANTS])
def test_planted_python_oracle_mistake_fails_a_pin(tmp_path, mod, name, text, repl, select):
    r = run_py_pins(mod, py_copy(tmp_path, mod, text, repl), select)
    assert r.returncode == 1, f"mistake not caught by a pin: {name}\n" + r.stdout[-2000:] + r.stderr[-1000:]

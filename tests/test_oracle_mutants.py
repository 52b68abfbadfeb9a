"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pin suite rejects every one of them.  A mutant that passes all pins would
mean the pins do not cover that part of the oracle."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
sys.path.insert(0, os.path.join(ROOT, "oracle"))
import build as oracle_build  # noqa: E402  (oracle/build.py: the gcc flags)

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("ceil_to_floor", "if (rotate_bytes % num_bytes != 0)\n        k += 1;", "if (0)\n        k += 1;"),
    ("no_negative_fold", "if (r < 0)\n        r += kk;", "if (0)\n        r += kk;"),
    ("stride_unrounded", "return (num_bytes + 255u) / 256u * 256u;", "return num_bytes;"),
    ("pattern_mult", "* 517u) % 383u + 31u)", "* 571u) % 383u + 31u)"),
    ("pattern_mod", "(((i % 383u) * 517u)", "(((i % 384u) * 517u)"),
    ("pattern_offset", "% 383u + 31u)", "% 383u + 13u)"),
    ("pattern_scale", "* (uint64_t)(buffer_idx + 1);", "* (uint64_t)(buffer_idx + 2);"),
    ("pattern_float_index", "uint64_t v = (((i % 383u)", "uint64_t v = ((((uint64_t)(float)i % 383u)"),
    ("mix_shift", "z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;", "z = (z ^ (z >> 28)) * 0x94D049BB133111EBULL;"),
    ("weyl_index", "key + (j + 1u) * 0x9E3779B97F4A7C15ULL", "key + j * 0x9E3779B97F4A7C15ULL"),
    ("value_bits", ">> 40) - 8388608;", ">> 41) - 8388608;"),
    ("value_sign", ">> 40) - 8388608;", ">> 40) - 0;"),
    ("zero_32B_as_16B", "{0, 1, 2, 4, 32}", "{0, 1, 2, 4, 16}"),
    ("keys_swapped", "uint64_t value_key = seed ^ (uint64_t)(2 * buffer_idx);",
     "uint64_t value_key = seed ^ (uint64_t)(2 * buffer_idx + 1);"),
    ("category_order", "if (draw < upper) {", "if (draw <= upper) {"),
    ("drop_last_source", "for (int k = 2; k <= nsrc; k++) {", "for (int k = 2; k < nsrc; k++) {"),
    ("start_from_zero", "memcpy(dst, srcs[0], (size_t)(n * 4u));\n    for (int k = 2;",
     "memset(dst, 0, (size_t)(n * 4u));\n    for (int k = 1;"),
    ("reverse_order",
     "memcpy(dst, srcs[0], (size_t)(n * 4u));\n    for (int k = 2; k <= nsrc; k++) {\n        const float *next = srcs[k - 1];",
     "memcpy(dst, srcs[nsrc - 1], (size_t)(n * 4u));\n    for (int k = 2; k <= nsrc; k++) {\n        const float *next = srcs[nsrc - k];"),
    ("accumulate_in_double",
     "memcpy(dst, srcs[0], (size_t)(n * 4u));\n    for (int k = 2; k <= nsrc; k++) {\n        const float *next = srcs[k - 1];\n        for (uint64_t i = 0; i < n; i++)\n            dst[i] = dst[i] + next[i];\n    }",
     "for (uint64_t i = 0; i < n; i++) {\n        double acc = srcs[0][i];\n        for (int k = 2; k <= nsrc; k++)\n            acc += srcs[k - 1][i];\n        dst[i] = (float)acc;\n    }"),
    ("pattern_index_shift", "out[i] = pattern[i % pattern_len];", "out[i] = pattern[(i + 1) % pattern_len];"),
    ("memset_ignored", "memset(dst, (int)(memset_byte & 0xFFu), (size_t)(n * 4u));", "memset(dst, 0, (size_t)(n * 4u));"),
    ("batch_swapped_offsets", "memcpy(pool + dst_off, src_image + src_off, (size_t)bytes);",
     "memcpy(pool + src_off, src_image + dst_off, (size_t)bytes);"),
    ("batch_short", "memcpy(pool + dst_off, src_image + src_off, (size_t)bytes);",
     "memcpy(pool + dst_off, src_image + src_off, (size_t)(bytes ? bytes - 1 : 0));"),
    ("mismatch_byte_index", "return (int64_t)(i / elem_size);", "return (int64_t)i;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new, tmp_path):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(text.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, "-Wno-error", str(mutated), "-o", str(lib)], check=True)
    env = dict(os.environ, TB_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout[-2000:]}"

"""The CPU oracle against what pins it from outside (CPU only).

Every pin in ``oracle_pins.py`` runs against the oracle as built from
``oracle/oracle.c``.  Then each of a set of plausible mistakes is planted in a
copy of ``oracle.c`` (a dropped term, a wrong sign or index, a transposed
operand, fp32 accumulation, ...), built, and run against the same pins in a
child process: each planted mistake must make at least one pin fail.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import oracle_pins as P

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_thread_count_invariance(orc):
    import gemm_inputs as gi
    rng = gi.rng_for(91)
    m, n, k = 70, 45, 130
    A = gi.colmajor(gi.draw(rng, m * k, "u", np.float32), m, k, m, np.nan)
    B = gi.colmajor(gi.draw(rng, k * n, "u", np.float32), k, n, k, np.nan)
    before = orc.num_threads()
    try:
        orc.set_num_threads(1)
        R1 = orc.gemm(m, n, k, 1.0, A, m, B, k, 0.0, None, m)
        orc.set_num_threads(4)
        R4 = orc.gemm(m, n, k, 1.0, A, m, B, k, 0.0, None, m)
    finally:
        orc.set_num_threads(before)
    assert np.array_equal(R1, R4)


def test_argument_checks(orc):
    with pytest.raises(ValueError):
        orc.gemm(4, 4, 4, 1.0, np.zeros(3, np.float32), 4, np.zeros(16, np.float32), 4,
                 0.0, None, 4)
    with pytest.raises(ValueError):
        orc.gemm_entries(4, 4, 4, 1.0, np.zeros(16, np.float32), 4,
                         np.zeros(16, np.float32), 4, 0.0, None, 4, [4], [0])


# (name, text in oracle.c, replacement).  Each replacement is applied to the
# first occurrence only, which is in the function named by the first word.
MUTANTS = [
    ("f32_accumulate_in_float",
     "acc[i] += (double)a_col[i] * b;",
     "acc[i] = (float)(acc[i] + (double)a_col[i] * b);"),
    ("f32_drop_beta_term",
     "if (beta != 0.0) r += beta * (double)C0[(size_t)i + (size_t)j * ldc];",
     "if (beta != 0.0) r += 0.0;"),
    ("f32_beta_sign",
     "if (beta != 0.0) r += beta * (double)C0[(size_t)i + (size_t)j * ldc];",
     "if (beta != 0.0) r -= beta * (double)C0[(size_t)i + (size_t)j * ldc];"),
    ("f32_alpha_scales_c",
     "if (beta != 0.0) r += beta * (double)C0[(size_t)i + (size_t)j * ldc];",
     "if (beta != 0.0) r += alpha * beta * (double)C0[(size_t)i + (size_t)j * ldc];"),
    ("f32_skip_first_k",
     "for (int p = 0; p < k; ++p) {\n                    double b = (double)B",
     "for (int p = 1; p < k; ++p) {\n                    double b = (double)B"),
    ("f32_lda_as_m",
     "const float *a_col = A + (size_t)p * lda;",
     "const float *a_col = A + (size_t)p * m;"),
    ("f32_b_transposed",
     "double b = (double)B[(size_t)p + (size_t)j * ldb];",
     "double b = (double)B[(size_t)j + (size_t)p * ldb];"),
    ("f32_write_ldr_as_ldc",
     "R[(size_t)i + (size_t)j * ldr] = r;",
     "R[(size_t)i + (size_t)j * (ldr > 1 ? ldr - 1 : 1)] = r;"),
    ("f32_entries_b_transposed",
     "s += (double)A[i + (size_t)p * lda] * (double)B[(size_t)p + j * ldb];",
     "s += (double)A[i + (size_t)p * lda] * (double)B[j + (size_t)p * ldb];"),
    ("f64_drop_last_k",
     "for (int p = 0; p < k; ++p) {\n                    double b = B[",
     "for (int p = 0; p < k - 1; ++p) {\n                    double b = B["),
    ("f64_alpha_ignored",
     "double r = use_ab ? alpha * acc[i] : 0.0;\n                if (beta != 0.0) r += beta * C0[",
     "double r = use_ab ? acc[i] : 0.0;\n                if (beta != 0.0) r += beta * C0["),
    ("rowmajor_b_stride_lda",
     "const double *b_row = B + (size_t)p * ldb;",
     "const double *b_row = B + (size_t)p * lda;"),
    ("rowmajor_a_colmajor",
     "double a = A[(size_t)i * lda + p];",
     "double a = A[(size_t)p * lda + i];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert old in src, "mutation target not found: %s" % name
    bad = src.replace(old, new, 1)
    assert bad != src
    csrc = tmp_path / ("mutant_%s.c" % name)
    csrc.write_text(bad)
    so = str(tmp_path / ("libmutant_%s.so" % name))
    oracle.compile_source(str(csrc), so)
    proc = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), so],
                          capture_output=True, text=True, timeout=600,
                          env={**os.environ, "OMP_NUM_THREADS": "2"})
    # A named pin must fail; a later crash from a wild index does not count
    # on its own.
    tripped = [ln.split()[1] for ln in proc.stdout.splitlines()
               if ln.startswith("PIN-FAILED ")]
    assert proc.returncode != 0 and tripped, (
        "planted mistake %s tripped no pin (exit %d):\n%s" % (
            name, proc.returncode, proc.stdout[-2000:]))

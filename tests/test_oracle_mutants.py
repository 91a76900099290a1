"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each one.

Each mutant is one textual change to oracle.c (a dropped term, a wrong sign or index, a
transposed operand, another rounding), compiled to a temporary library and run against
test_oracle_pins.py in a child process.  A mutant that every pin lets through would mean
the pins do not constrain that part of the oracle."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")

MUTANTS = [
    ("half-away rounding of W/alpha", "float r = rintf(q);", "float r = roundf(q);"),
    ("dropped abs in absmean", "s += fabs((double)w[i]);", "s += (double)w[i];"),
    ("mean divides by count-1", "return (float)(s / (double)count);", "return (float)(s / (double)(count - 1));"),
    ("transposed division W/alpha", "float q = w / alpha;", "float q = alpha / w;"),
    ("dropped upper clip of codes", "if (r > 1.0f) r = 1.0f;", ""),
    ("reversed bit order in quantize_weights", "byte |= (unsigned)(c + 1) << (2 * i);",
     "byte |= (unsigned)(c + 1) << (6 - 2 * i);"),
    ("reversed bit order in pack", "byte |= (unsigned)(w + 1) << (2 * i);",
     "byte |= (unsigned)(w + 1) << (6 - 2 * i);"),
    ("wrong code offset in unpack", "codes[n * k + 4 * b + i] = (int8_t)((int)c - 1);",
     "codes[n * k + 4 * b + i] = (int8_t)((int)c);"),
    ("dropped abs in activation max", "if (a > mx) mx = a;", "if (a > mx) mx = row[j];"),
    ("dropped 1e-8 guard", "float b = mx + 1e-8f;", "float b = mx;"),
    ("reciprocal instead of division", "float t = (row[j] * 127.0f) / b;", "float t = row[j] * (127.0f / b);"),
    ("reciprocal in ternarization", "float q = w / alpha;", "float q = w * (1.0f / alpha);"),
    ("half-away rounding of activations", "float r = rintf(t);", "float r = roundf(t);"),
    ("sign flip on +1 weights", "if (c == 1) s += xq[m * k + j];", "if (c == 1) s -= xq[m * k + j];"),
    ("dropped token index", "else if (c == -1) s -= xq[m * k + j];", "else if (c == -1) s -= xq[j];"),
    ("fp32 dequant scale", "return (float)((double)alpha * (double)beta / 127.0);",
     "return alpha * beta / 127.0f;"),
    ("transposed acc in dequant", "float v = (float)acc[m * n_rows + n] * s;",
     "float v = (float)acc[n * m_rows + m] * s;"),
    ("bias subtracted", "if (bias) v = v + bias[n];", "if (bias) v = v - bias[n];"),
    ("per-row alpha indexed by token", "float a = alpha_rows ? alpha_rows[n] : alpha;",
     "float a = alpha_rows ? alpha_rows[m] : alpha;"),
    ("reversed butterfly difference", "v[j + h] = a - b;", "v[j + h] = b - a;"),
    ("descending butterfly strides", "for (int64_t h = 1; h < block; h *= 2) {",
     "for (int64_t h = block / 2; h >= 1; h /= 2) {"),
    ("rotation scaled by 1/B", "const float scale = (float)(1.0 / sqrt((double)block));",
     "const float scale = (float)(1.0 / (double)block);"),
    ("rotation signs ignored", "o[j] = (signs && signs[j] < 0) ? -row[j] : row[j];", "o[j] = row[j];"),
    ("rotation block offset dropped", "float* v = o + b0;", "float* v = o;"),
    ("block alpha from the wrong row", "alpha[n * kb + b] = oracle_absmean(w + n * k + b * ORACLE_BLOCK, ORACLE_BLOCK);",
     "alpha[n * kb + b] = oracle_absmean(w + b * ORACLE_BLOCK, ORACLE_BLOCK);"),
    ("block code uses a neighbouring block", "alpha[n * kb + j / ORACLE_BLOCK]", "alpha[n * kb + (j + 64) / ORACLE_BLOCK % kb]"),
    ("block sums over half a block", "for (int64_t j = b * ORACLE_BLOCK; j < (b + 1) * ORACLE_BLOCK; ++j) {",
     "for (int64_t j = b * ORACLE_BLOCK; j < b * ORACLE_BLOCK + ORACLE_BLOCK / 2; ++j) {"),
    ("block dequant in fp32", "const double t = (double)beta[m] / 127.0;", "const double t = (double)(beta[m] / 127.0f);"),
    ("block dequant drops alpha", "s += (double)alpha[n * kb + b] * (double)acc[(m * n_rows + n) * kb + b];",
     "s += (double)acc[(m * n_rows + n) * kb + b];"),
    ("gelu with sqrt 2 for 1/sqrt 2", "erfc(-v * 0.70710678118654752440)", "erfc(-v * 1.41421356237309504880)"),
    ("gelu without the half", "g[i] = (float)(0.5 * v * erfc(", "g[i] = (float)(v * erfc("),
    ("gelu with erfc(+h / sqrt 2)", "erfc(-v * 0.7071", "erfc(v * 0.7071"),
    ("gelu as 1 + erf (cancels for h < -5)", "erfc(-v * 0.70710678118654752440)", "(1.0 + erf(v * 0.70710678118654752440))"),
    ("gelu flushed to 0 below -6", "g[i] = (float)(0.5 * v * erfc(-v * 0.70710678118654752440));",
     "g[i] = v < -6.0 ? 0.0f : (float)(0.5 * v * erfc(-v * 0.70710678118654752440));"),
    ("t5 radix 4", "for (int i = 0; i < 5; ++i, p3 *= 3) {", "for (int i = 0; i < 5; ++i, p3 *= 4) {"),
    ("t5 padding as weight -1", "int c = 1;                                     /* past K: weight 0 */",
     "int c = 0;"),
    ("t5 trit order reversed on unpack", "for (int i = 0; i < (int)(j % 5); ++i) v /= 3;",
     "for (int i = 0; i < 4 - (int)(j % 5); ++i) v /= 3;"),
    ("t5 rows of 16 ceil(K/64) bytes", "int64_t oracle_t5_row_bytes(int64_t k) { return 16 * ((k + 79) / 80); }",
     "int64_t oracle_t5_row_bytes(int64_t k) { return 16 * ((k + 63) / 64); }"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_kill_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique/found: {old!r}"
    mut = tmp_path / "oracle_mutant.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    r = subprocess.run([sys.executable, os.path.join(HERE, "_mutant_runner.py"), str(mut), str(so)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant '{name}' survived every pin:\n{r.stdout[-2000:]}"

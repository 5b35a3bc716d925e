"""The oracle's pins are strong enough to catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle source (a dropped
or flipped term, a wrong index, a wrong rounding), builds it with gcc on the
CPU, and runs the oracle pin suite against it in a subprocess: the suite must
fail.  Nothing here touches the real oracle build or the GPU.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "wq_oracle.c")
PINS = ["tests/test_oracle_formats.py", "tests/test_oracle_packing.py",
        "tests/test_oracle_dequant.py", "tests/test_oracle_linear.py", "tests/test_oracle_swiglu.py",
        "tests/test_oracle_hadamard.py"]

MUTANTS = {
    "zero_sign": ("e = s * ((double)q - z);", "e = s * ((double)q + z);"),
    "sym_zero": ("z = (double)(1 << (L->bits - 1));", "z = (double)(1 << L->bits);"),
    "group_index": ("return k / L->group_size;", "return (L->K - 1 - k) / L->group_size;"),
    "scale_transposed": ("double s = wqo_f16_to_f64(L->scales[(size_t)g * L->N + n]);",
                         "double s = wqo_f16_to_f64(L->scales[(size_t)n * L->G + g]);"),
    "round_half_away": ("double r = rint(a / quantum);", "double r = round(a / quantum);"),
    "round_truncate": ("double r = rint(a / quantum);", "double r = floor(a / quantum);"),
    "no_subnormal_quantum": ("if (e < emin) e = emin;", ";"),
    "lut_index": ("e = s * wqo_f16_to_f64(L->lut[q]);",
                  "e = s * wqo_f16_to_f64(L->lut[(q + 1) & ((1u << L->bits) - 1u)]);"),
    "reduction_index": ("for (int k = 0; k < K; ++k) acc += xr[k] * wcol[k];",
                        "for (int k = 0; k < K; ++k) acc += xr[k] * wcol[K - 1 - k];"),
    "dropped_last_term": ("for (int k = 0; k < K; ++k) acc += xr[k] * wcol[k];",
                          "for (int k = 0; k < K - 1; ++k) acc += xr[k] * wcol[k];"),
    "code_order": ("  long bit = (long)bits * idx;\n  long r = bit / 32;\n  int sh = (int)(bit % 32);\n  uint64_t two",
                   "  long bit = (long)bits * (idx ^ 1);\n  long r = bit / 32;\n  int sh = (int)(bit % 32);\n  uint64_t two"),
    "fp16_zero_from_scale": ("z = wqo_f16_to_f64(((const uint16_t*)L->zeros)[(size_t)g * L->N + n]);",
                             "z = wqo_f16_to_f64(((const uint16_t*)L->zeros)[(size_t)g * L->N + (n ^ 1)]);"),
    "packed_zero_row": ("z = (double)stream_code((const uint32_t*)L->zeros + (size_t)g * wpr, 1, n, L->bits);",
                        "z = (double)stream_code((const uint32_t*)L->zeros, 1, n, L->bits);"),
    "silu_sign": ("double wqo_silu(double v) { return v / (1.0 + exp(-v)); }",
                  "double wqo_silu(double v) { return v / (1.0 + exp(v)); }"),
    "swiglu_dropped_up": ("for (size_t i = 0; i < n; ++i) h[i] = wqo_silu(g[i]) * u[i];",
                          "for (size_t i = 0; i < n; ++i) h[i] = wqo_silu(g[i]);"),
    "hadamard_or_for_and": ("  unsigned v = i & j;", "  unsigned v = i | j;"),
    "hadamard_norm": ("const double norm = 1.0 / sqrt((double)b);", "const double norm = 1.0 / (double)b;"),
    "hadamard_block_offset": ("const double* xb = x + (size_t)m * K + k0;", "const double* xb = x + (size_t)m * K;"),
    "fine_zero_by_scale_group": ("z = wqo_f16_to_f64(((const uint16_t*)L->zeros)[(size_t)(k / fine_zero_group(L->mode)) * L->N + n]);",
                                 "z = wqo_f16_to_f64(((const uint16_t*)L->zeros)[(size_t)g * L->N + n]);"),
    "fine_zero_group_size": ("return mode == WQO_ZERO_F16_G8 ? 8 :", "return mode == WQO_ZERO_F16_G8 ? 16 :"),
    "bf16_as_f16": ("return dtype == WQO_BF16 ? wqo_f64_to_bf16(v) : wqo_f64_to_f16(v);",
                    "return wqo_f64_to_f16(v);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "mutant.c")
        so = os.path.join(td, "libmutant.so")
        open(c, "w").write(src.replace(before, after))
        subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", c, "-o", so, "-lm"],
                       check=True, capture_output=True)
        env = dict(os.environ, WQ_ORACLE_LIB=so, OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"


def test_control_unmodified_copy_passes():
    """The same harness on an unmodified copy passes, so the failures above come
    from the planted mistakes and not from the harness."""
    with tempfile.TemporaryDirectory() as td:
        so = os.path.join(td, "libcontrol.so")
        subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", SRC, "-o", so, "-lm"],
                       check=True, capture_output=True)
        env = dict(os.environ, WQ_ORACLE_LIB=so, OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PINS],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-2000:]

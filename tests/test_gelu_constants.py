"""The fast GELU's constants in csrc/common.hpp against their generator, csrc/fit_gelu.py.

The kernels decide GELU's fp32 rounding from an fp64 approximation whose error is assumed to
stay below 6e-14 relative over v >= -4 (the rounding test's tolerance).  This test refits the
polynomial, requires the constants compiled into the kernels to be the ones the fit prints, bit
for bit, and measures the approximation's error against long-double erfcl on a sample.
No GPU; the oracle is not involved.
"""
import importlib.util
import os
import re
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bitlinear_matmul_absmean_amd", "csrc")


def _fit_module():
    # loaded without writing bytecode next to the kernel sources
    spec = importlib.util.spec_from_file_location("fit_gelu", os.path.join(CSRC, "fit_gelu.py"))
    mod = importlib.util.module_from_spec(spec)
    keep = sys.dont_write_bytecode
    sys.dont_write_bytecode = True
    try:
        spec.loader.exec_module(mod)
    finally:
        sys.dont_write_bytecode = keep
    return mod


def _kernel_constants():
    src = open(os.path.join(CSRC, "common.hpp")).read()
    ns = src[src.index("namespace gelu_poly {"):src.index("}  // namespace gelu_poly")]
    s2 = re.search(r"kS2 = 2\.0 \* ([-0-9.e]+), kO = ([-0-9.e]+);", ns)
    body = ns[ns.index("kC[17] = {") + len("kC[17] = {"):ns.index("};")]
    coef = [float(t) for t in body.replace("\n", " ").split(",") if t.strip()]
    return np.array(coef), float(s2.group(1)), float(s2.group(2))


def test_kernel_constants_are_the_fit():
    fit = _fit_module()
    coef, s, o = fit.fit()
    kc, ks, ko = _kernel_constants()
    assert kc.size == 17
    assert np.array_equal(kc.view(np.uint64), coef.astype(np.float64).view(np.uint64))
    assert ks == s and ko == o


def test_fast_path_error_bound():
    fit = _fit_module()
    coef, s, o = fit.fit()
    rng = np.random.default_rng(7)
    v = np.concatenate([np.linspace(-4.0, 12.0, 20_001), rng.uniform(-4.0, 6.0, 20_000),
                        rng.normal(0.0, 1.0, 10_000)]).astype(np.float32)
    v = v[(v >= -4.0) & (v != 0.0)]
    exact = fit.gelu_ld(v)
    got = fit.gelu_fast(v, coef, s, o).astype(np.longdouble)
    rel = np.abs((got - exact) / exact).astype(np.float64)
    # the rounding test's tolerance is 6e-14; the fit stays well inside it
    assert rel.max() < 3e-14, rel.max()

"""The polynomial exponential of the merge variant (pq_attn_reduce_polyexp),
pinned on the CPU: the coefficients the kernel holds (read from its source)
against numpy's exp2, with the kernel's fp32 Horner form and range
reduction, inside the bound the header states; and the fit script
reproduces them."""
import os
import re
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_product_amd", "csrc")
BOUND = 8.4e-8 * 1.02      # the header's "8.4e-8 at most", with the last digit's slack


def kernel_coefficients():
    text = open(os.path.join(CSRC, "decode_kernel.hpp")).read()
    body = text[text.index("poly_exp2(float x)"):]
    body = body[:body.index("return __builtin_ldexpf")]
    vals = dict(re.findall(r"(c\d) = ([-+0-9.e]+)f", body))
    return np.array([np.float32(vals[f"c{k}"]) for k in range(7)], np.float32)


def poly_exp2_f32(x):
    """The kernel's arithmetic: n = floor(x), f = x - n, Horner in fp32
    (fma rounded once per step), times 2^n."""
    c = kernel_coefficients()
    x = np.asarray(x, np.float32)
    n = np.floor(x)
    f = (x - n).astype(np.float32)
    p = np.full_like(f, c[6])
    for k in range(5, -1, -1):
        p = (p.astype(np.float64) * f + c[k]).astype(np.float32)   # one rounding, as fma
    out = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    return np.where(x >= -126.0, out, np.float32(0.0))


def test_fraction_part_within_bound():
    f = np.linspace(0.0, 1.0, 1 << 20, dtype=np.float32, endpoint=False)
    rel = np.abs(poly_exp2_f32(f).astype(np.float64) / np.exp2(f.astype(np.float64)) - 1.0)
    assert rel.max() <= BOUND


def test_merge_weight_range_within_bound():
    """Merge weights are 2^x for x <= 0 (m_c - m* in base 2)."""
    x = -np.concatenate([np.linspace(0.0, 1.0, 4096), np.linspace(1.0, 125.9, 1 << 18)]).astype(np.float32)
    rel = np.abs(poly_exp2_f32(x).astype(np.float64) / np.exp2(x.astype(np.float64)) - 1.0)
    assert rel.max() <= BOUND
    assert poly_exp2_f32(np.float32(0.0)) == 1.0
    assert poly_exp2_f32(np.float32(-np.inf)) == 0.0 and poly_exp2_f32(np.float32(-200.0)) == 0.0


def test_fit_script_reproduces_the_coefficients():
    out = subprocess.run([sys.executable, os.path.join(CSRC, "exp2_poly_fit.py")], capture_output=True,
                         text=True, check=True).stdout
    got = np.array([np.float32(v) for v in re.findall(r"c\d = ([-+0-9.e]+)f", out)], np.float32)
    np.testing.assert_array_equal(got, kernel_coefficients())
    assert float(re.search(r"\): ([0-9.e-]+)", out).group(1)) <= BOUND

"""The constants of the kernels' fp64 exponential (CPU only).

The draw weights and the resolve's merges evaluate 2^(s/1024) as a table entry
2^(j/1024) times a degree-3 Taylor polynomial of 2^(r/1024), |r| <= 1/2, scaled
by ldexp.  These tests pin the committed constants to the mathematics: the
table header is what its generator writes, every entry is the double nearest
2^(j/1024) (checked with 50-digit decimal arithmetic, independently of the
generator), the polynomial coefficients in the device source are
(ln 2)^i / i! / 1024^i rounded to double, and the truncation bound of the
degree-3 series on |r| <= 1/2 stays below 1e-15.
"""

import math
import re
import subprocess
import sys
from decimal import Decimal, getcontext
from pathlib import Path

CSRC = Path(__file__).resolve().parents[1] / "lossless_rejection_sampling_sampler_amd" / "csrc"


def _table_values():
    text = (CSRC / "sv_exp2_table.h").read_text()
    m = re.search(r"kExp2Table\[(\d+)\]\s*=\s*\{(.*?)\};", text, re.S)
    assert m, "table declaration not found"
    vals = [float(v) for v in m.group(2).replace("\n", " ").split(",") if v.strip()]
    return int(m.group(1)), vals


def test_header_is_generator_output():
    out = subprocess.run([sys.executable, "gen_exp2_table.py"], cwd=CSRC, capture_output=True, text=True,
                         check=True).stdout
    assert out == (CSRC / "sv_exp2_table.h").read_text()


def test_entries_are_nearest_doubles():
    n, vals = _table_values()
    src = (CSRC / "sv_device.h").read_text()
    assert f"constexpr int kExp2TableSize = {n};" in src
    assert f"constexpr int kExp2Shift = {n.bit_length() - 1};" in src and n & (n - 1) == 0
    assert len(vals) == n
    getcontext().prec = 50
    ln2 = Decimal(2).ln()
    for j, v in enumerate(vals):
        exact = (Decimal(j) / n * ln2).exp()
        err = abs(Decimal(v) - exact)
        # within half an ulp of the exact value (entries lie in [1, 2): ulp 2^-52)
        assert err <= Decimal(2) ** -53, (j, v)


def test_polynomial_coefficients_and_clamp():
    src = (CSRC / "sv_device.h").read_text()
    body = src[src.index("__device__ __forceinline__ double exp2_tab("):]
    body = body[:body.index("\n}\n")]
    coefs = [float(c) for c in re.findall(r"fma\(r, (?:p|[0-9.e+-]+), ([0-9.e+-]+)\)", body)]
    lead = float(re.search(r"fma\(r, ([0-9.e+-]+), ", body).group(1))
    # Horner order: c3 (lead), c2, c1, c0
    n, _ = _table_values()
    getcontext().prec = 50
    ln2 = Decimal(2).ln()
    want = [float(ln2 ** i / math.factorial(i) / Decimal(n) ** i) for i in range(4)]
    assert [lead] + coefs == [want[3], want[2], want[1], want[0]]
    # the clamp is n * -1080: its power of two, 2^-1080, is below the smallest double
    assert f"fmax(s, {-1080.0 * n!r})" in body
    assert 2.0 ** -1080 == 0.0
    # truncation of the degree-3 series at |r| = 1/2: x^4 / 24 e^x with x = ln2 / (2n)
    x = math.log(2) / (2 * n)
    assert x ** 4 / 24 * math.exp(x) < 1e-15

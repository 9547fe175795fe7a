"""Fixed-order fp64 evaluation rules for the selector.

Test infrastructure only (see the package docstring).

The selector turns floating-point statistics into integers (ranks, tier
counts, event masks).  For two independent implementations to reach the same
integers on the same inputs, every floating-point result that feeds a
decision must be evaluated in the same precision and order.  The page fixes
only the formulas (Sec. 2.4, Eqs. (9)-(14)); the evaluation rules below are
this implementation's reading, stated once and followed on both sides:

* precision: IEEE binary64; only correctly rounded +, -, *, / and sqrt; no
  fused multiply-add.  Python floats satisfy this.
* csum(x): the sum of a sequence x[0..n) is taken as 64 interleaved running
  sums p_l = (((0 + x[l]) + x[l+64]) + x[l+128]) + ...  for l < 64, combined
  pairwise: for w = 32, 16, 8, 4, 2, 1: p_l <- p_l + p_{l+w} for l < w;
  the result is p_0.
* exp2(x): x is first clamped to [-2000, 1000] (a NaN x becomes 1000, as
  fmin / fmax treat it); n = round-half-even(x),
  f = x - n (exact),
  y = f * LN2 with LN2 the binary64 value nearest ln 2; the Taylor polynomial
  sum_{i=0}^{14} y^i / i! is evaluated by Horner's rule from i = 14 down
  (p = p * y + c_i, each coefficient the binary64 value nearest 1/i!);
  the result is ldexp(p, n).  Accurate to about 1 ulp.
* powi(r, n): binary powering from the least significant bit:
  res = 1; base = r; while n: if n & 1: res = res * base; base = base * base;
  n >>= 1.
"""
from __future__ import annotations

import math

LN2 = 0.6931471805599453          # binary64 nearest ln 2 (0x3FE62E42FEFA39EF)
_EXP_COEF = [1.0 / math.factorial(i) for i in range(15)]


def csum(xs) -> float:
    """Sum in the fixed 64-lane interleaved + pairwise-tree order."""
    xs = [float(x) for x in xs]
    n = len(xs)
    p = [0.0] * 64
    for i in range(n):
        p[i & 63] = p[i & 63] + xs[i]
    w = 32
    while w >= 1:
        for lane in range(w):
            p[lane] = p[lane] + p[lane + w]
        w >>= 1
    return p[0]


def exp2(x: float) -> float:
    """2**x in the fixed evaluation order described in the module docstring."""
    x = max(-2000.0, min(1000.0, float(x)))
    n = round(x)                       # Python rounds half to even
    f = x - n
    y = f * LN2
    p = _EXP_COEF[14]
    for i in range(13, -1, -1):
        p = p * y + _EXP_COEF[i]
    return math.ldexp(p, int(n))


def powi(r: float, n: int) -> float:
    """r**n for integer n >= 0 by binary powering (least significant bit first)."""
    res = 1.0
    base = float(r)
    n = int(n)
    while n:
        if n & 1:
            res = res * base
        base = base * base
        n >>= 1
    return res

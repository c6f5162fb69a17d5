"""Pins of the oracle's sigma32 (the fp32 router sigmoid).

The page ("InternLumina-U2中256个专家的路由秘密…", §二 step 1) fixes a per-expert
logistic sigmoid evaluated in fp32; sigma32 is this build's specification of
its rounding.  These tests pin it to mathematics that does not go through it:
an independent long-double evaluation of 1/(1+exp(-z)), exact special values,
monotonicity, the reflection identity, and the spec's constants recomputed in
high-precision decimal arithmetic.
"""
import math
import os
import struct
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle


def _bits(f):
    return struct.unpack("<I", struct.pack("<f", f))[0]


def test_special_values():
    z = np.array([0.0, -0.0, np.inf, -np.inf, 200.0, -200.0, 40.5, -104.5], np.float32)
    s = oracle.sigmoid32(z)
    assert s[0] == 0.5 and s[1] == 0.5
    assert s[2] == 1.0 and s[3] == 0.0
    assert s[4] == 1.0 and s[5] == 0.0
    assert s[6] == 1.0
    assert s[7] == 0.0
    assert np.isnan(oracle.sigmoid32(np.array([np.nan], np.float32))[0])


def test_textbook_values():
    # 1/(1+e^-z) from Python's own exp, rounded once to fp32
    for z in [1.0, -1.0, 0.5, 2.0, -3.0, 10.0, -20.0, -87.5, -95.0, -103.0]:
        ref = np.float32(1.0 / (1.0 + math.exp(-z)))
        got = oracle.sigmoid32(np.array([z], np.float32))[0]
        assert abs(int(_bits(got)) - int(_bits(ref))) <= 1, (z, got, ref)


def test_subnormal_results():
    # sigma(z) ~ e^z below fp32's normal range: results must be subnormal, not flushed
    z = np.array([-90.0, -100.0, -103.0], np.float32)
    s = oracle.sigmoid32(z)
    assert np.all(s > 0) and np.all(s < np.finfo(np.float32).tiny)


def test_reflection():
    rng = np.random.default_rng(5)
    z = rng.normal(0, 4, 20000).astype(np.float32)
    a = oracle.sigmoid32(z).astype(np.float64)
    b = oracle.sigmoid32(-z).astype(np.float64)
    # each side is within one fp32 ulp of the exact value, so the sum is within 2^-23 of 1
    assert np.max(np.abs(a + b - 1.0)) <= 2.0 ** -23


def test_spec_constants():
    getcontext().prec = 80
    ln2 = Decimal(2).ln()
    l1 = float(ln2)
    l2 = float(ln2 - Decimal(l1))
    log2e = float(1 / ln2)
    assert l1 == float.fromhex("0x1.62e42fefa39efp-1")
    assert l2 == float.fromhex("0x1.abc9e3b39803fp-56")
    assert log2e == float.fromhex("0x1.71547652b82fep+0")
    # the spec's constants as written in oracle.c
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    for c in ["0x1.62e42fefa39efp-1", "0x1.abc9e3b39803fp-56", "0x1.71547652b82fep+0"]:
        assert c in src


@pytest.mark.parametrize("stride", [257])
def test_accuracy_and_monotonicity_sampled(stride):
    """Every 257th fp32 bit pattern (16.7M inputs, both signs): within 1 ulp
    of RN32 of a long-double evaluation, and monotone."""
    checked, not_rn, over1, nonmono = oracle.sigmoid32_scan(0, 2 ** 32, stride)
    assert checked == (2 ** 32 + stride - 1) // stride
    assert over1 == 0
    assert nonmono == 0
    # correctly rounded except in rare double-rounding cases
    assert not_rn <= checked // 100000


def test_monotone_dense_near_zero():
    """Consecutive fp32 values around the region where scores are compared."""
    for lo, hi in [(0x00000000, 0x00000000 + 4_000_000), (0x3F000000, 0x3F000000 + 4_000_000),
                   (0xBF000000, 0xBF000000 + 4_000_000), (0x40800000, 0x40800000 + 4_000_000)]:
        checked, not_rn, over1, nonmono = oracle.sigmoid32_scan(lo, hi, 1)
        assert over1 == 0 and nonmono == 0


@pytest.mark.slow
def test_accuracy_exhaustive():
    checked, not_rn, over1, nonmono = oracle.sigmoid32_scan(0, 2 ** 32, 1)
    assert checked == 2 ** 32
    assert over1 == 0 and nonmono == 0

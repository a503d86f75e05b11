"""Pins for the oracle's rotary coefficients, rotation and softmax scale.

Each test checks the oracle against something other than its own code: a
constant the pages print (tests/golden/page_constants.txt), a closed form
evaluated in 50-digit decimal arithmetic, the defining property of a
quantity, or a textbook routine (complex multiplication)."""

import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import workloads
from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.txt")


def golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                vals[k] = float(v)
    return vals


KIMI = workloads.YARN_KIMI
getcontext().prec = 50
PI = Decimal("3.14159265358979323846264338327950288419716939937510")


def _dec_ln(x):
    return Decimal(x).ln()


def test_yarn_class_defaults_mscale():
    # With the YaRN class defaults (mscale 1, mscale_all_dim 0) the table
    # multiplier is g(f,1)/1; with mscale = mscale_all_dim it is exactly 1.
    g = golden()
    spec = workloads.RopeSpec(kind="yarn", base=g["yarn_default_base"], factor=32.0,
                              original_max_pos=int(g["yarn_default_original_max_position_embeddings"]),
                              beta_fast=g["yarn_default_beta_fast"], beta_slow=g["yarn_default_beta_slow"],
                              mscale=g["yarn_default_mscale"], mscale_all_dim=g["yarn_default_mscale_all_dim"])
    expect = float(1 + Decimal(str(g["mscale_log_coefficient"])) * _dec_ln(32))
    assert O.rope_table_mscale(spec) == pytest.approx(expect, rel=1e-15)
    assert O.rope_table_mscale(KIMI) == 1.0
    # no scaling -> no correction
    assert O.yarn_get_mscale(1.0, 5.0) == 1.0
    assert O.yarn_get_mscale(0.5, 5.0) == 1.0


def test_correction_dim_defining_property():
    # cd(n) is the (fractional) pair-dimension whose wavelength 2*pi*base^(2d/D)
    # fits n times into the original context: L / lambda(d) = n.
    for (dim, base, L) in [(64, 50000.0, 4096), (64, 10000.0, 4096), (16, 10000.0, 2048)]:
        for n in [32.0, 1.0, 4.0]:
            d = O.yarn_correction_dim(n, dim, base, L)
            wavelength = 2 * math.pi * base ** (2 * d / dim)
            assert L / wavelength == pytest.approx(n, rel=1e-12)


def test_correction_range_kimi_closed_form():
    # 50-digit closed form of the two correction dims for D=64, base 5e4, L=4096.
    def cd(n):
        return Decimal(64) * _dec_ln(Decimal(4096) / (Decimal(n) * 2 * PI)) / (2 * _dec_ln(50000))
    assert float(cd(32)) == pytest.approx(O.yarn_correction_dim(32, 64, 50000.0, 4096), rel=1e-14)
    assert float(cd(1)) == pytest.approx(O.yarn_correction_dim(1, 64, 50000.0, 4096), rel=1e-14)
    lo, hi = O.yarn_correction_range(32, 1, 64, 50000.0, 4096)
    assert (lo, hi) == (math.floor(cd(32)), math.ceil(cd(1))) == (8, 20)
    # clamping: a huge beta_fast drives the low bound negative -> 0; a tiny
    # beta_slow drives the high bound past dim-1 -> dim-1
    lo, hi = O.yarn_correction_range(1e9, 1e-30, 64, 50000.0, 4096)
    assert lo == 0 and hi == 63


def test_yarn_inv_freq_band_edges():
    inv = O.rope_inv_freq(KIMI, 64)
    assert inv.shape == (32,)
    theta = [float(Decimal(1) / (Decimal(50000) ** (Decimal(2 * i) / Decimal(64)))) for i in range(32)]
    # below the band: pure extrapolation (unscaled frequency)
    for i in range(0, 9):
        assert inv[i] == pytest.approx(theta[i], rel=1e-14)
    # above the band: pure interpolation (frequency / factor)
    for i in range(20, 32):
        assert inv[i] == pytest.approx(theta[i] / 32.0, rel=1e-14)
    # middle of the band (i=14, ramp 0.5): average of the two
    assert inv[14] == pytest.approx(0.5 * theta[14] + 0.5 * theta[14] / 32.0, rel=1e-14)
    # strictly between inside the band
    for i in range(9, 20):
        assert theta[i] / 32.0 < inv[i] < theta[i]
    assert inv[0] == 1.0


def test_default_rope_is_yarn_at_factor_one():
    d = workloads.RopeSpec(kind="default", base=10000.0)
    y = workloads.RopeSpec(kind="yarn", base=10000.0, factor=1.0, mscale=1.0, mscale_all_dim=0.0)
    np.testing.assert_allclose(O.rope_inv_freq(d, 64), O.rope_inv_freq(y, 64), rtol=1e-15)
    assert O.rope_table_mscale(y) == 1.0
    c1, s1 = O.rope_table(d, 64, 50)
    c2, s2 = O.rope_table(y, 64, 50)
    np.testing.assert_allclose(c1, c2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-15)


def test_degenerate_ramp_widened():
    r = O.yarn_linear_ramp(3, 3, 8)
    g = golden()["ramp_singularity_widening"]
    expect = np.clip((np.arange(8) - 3) / g, 0, 1)
    np.testing.assert_array_equal(r, expect)


def test_unknown_rope_kind_raises():
    bad = workloads.RopeSpec(kind="ntk-by-parts", base=10000.0)
    with pytest.raises(ValueError):
        O.rope_inv_freq(bad, 64)


def test_table_shape_and_position_zero():
    g = golden()
    cos, sin = O.rope_table(KIMI, 64, 1001)
    assert cos[1000:1001].shape == (1, int(g["kimi_k2_decode_table_pairs"]))
    m = O.rope_table_mscale(KIMI)
    np.testing.assert_array_equal(cos[0], np.full(32, m))
    np.testing.assert_array_equal(sin[0], np.zeros(32))


def test_rotation_is_complex_multiplication():
    # half pairing: (x_i + j x_{i+D/2}) * exp(j p theta_i), by numpy complex arithmetic
    rng = np.random.default_rng(0)
    for spec, D in [(KIMI, 64), (workloads.RopeSpec(kind="default", base=10000.0), 16)]:
        cos, sin = O.rope_table(spec, D, 300)
        m = O.rope_table_mscale(spec)
        inv = O.rope_inv_freq(spec, D)
        x = rng.standard_normal((300, D))
        y = O.rotate(x, cos, sin, "half")
        z = (x[:, :D // 2] + 1j * x[:, D // 2:]) * (m * np.exp(1j * np.arange(300)[:, None] * inv[None]))
        np.testing.assert_allclose(y[:, :D // 2], z.real, atol=1e-12)
        np.testing.assert_allclose(y[:, D // 2:], z.imag, atol=1e-12)
        # interleaved pairing: (x_2i + j x_2i+1) * exp(j p theta_i)
        yi = O.rotate(x, cos, sin, "interleaved")
        zi = (x[:, 0::2] + 1j * x[:, 1::2]) * (m * np.exp(1j * np.arange(300)[:, None] * inv[None]))
        np.testing.assert_allclose(yi[:, 0::2], zi.real, atol=1e-12)
        np.testing.assert_allclose(yi[:, 1::2], zi.imag, atol=1e-12)


def test_rotation_invariants():
    rng = np.random.default_rng(1)
    spec = workloads.RopeSpec(kind="default", base=10000.0)
    D = 64
    cos, sin = O.rope_table(spec, D, 2000)
    x = rng.standard_normal((5, D))
    k = rng.standard_normal((5, D))
    for pairing in ("half", "interleaved"):
        # identity at position 0
        np.testing.assert_array_equal(O.rotate(x, cos[0], sin[0], pairing), x)
        # pairwise norm preservation
        y = O.rotate(x, cos[777], sin[777], pairing)
        np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
        # relative position: <R(p+d) q, R(p'+d) k> = <R(p) q, R(p') k>
        for (p, pp, d) in [(5, 3, 100), (900, 17, 512)]:
            a = np.sum(O.rotate(x, cos[p + d], sin[p + d], pairing) * O.rotate(k, cos[pp + d], sin[pp + d], pairing), 1)
            b = np.sum(O.rotate(x, cos[p], sin[p], pairing) * O.rotate(k, cos[pp], sin[pp], pairing), 1)
            np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)


def test_interleaved_is_permuted_half():
    rng = np.random.default_rng(2)
    D = 16
    cos, sin = O.rope_table(workloads.RopeSpec(kind="default", base=10000.0), D, 40)
    x = rng.standard_normal((40, D))
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])  # de-interleave
    inv = np.argsort(perm)
    a = O.rotate(x, cos, sin, "interleaved")
    b = O.rotate(x[:, perm], cos, sin, "half")[:, inv]
    np.testing.assert_allclose(a, b, atol=1e-14)


def test_softmax_scales():
    g = golden()
    W = workloads.WORKLOADS
    # GLM-5: 1/sqrt(256) exactly, no correction under default RoPE
    assert O.softmax_scale(W["glm5_4k"].rope, W["glm5_4k"].Dqk) == 1.0 / math.sqrt(g["glm5_softmax_scale_inverse_square"])
    assert W["glm5_4k"].Dqk == 256
    # Kimi-K2: 1/sqrt(192) * (1 + 0.1 ln 32)^2 (50-digit closed form)
    gk = 1 + Decimal("0.1") * _dec_ln(32)
    expect = float(gk * gk / Decimal(int(g["kimi_k2_softmax_scale_inverse_square"])).sqrt())
    for name in ("kimi_k2_1k", "kimi_k2_8k", "kimi_k2_decode"):
        assert O.softmax_scale(W[name].rope, W[name].Dqk) == pytest.approx(expect, rel=1e-15)
    # tiny: 1/sqrt(48)
    assert O.softmax_scale(W["tiny"].rope, 48) == pytest.approx(float(1 / Decimal(48).sqrt()), rel=1e-15)
    # YaRN with mscale_all_dim = 0: no correction
    s = workloads.RopeSpec(kind="yarn", base=1e4, factor=40.0, mscale=1.0, mscale_all_dim=0.0)
    assert O.softmax_scale(s, 192) == 192 ** -0.5

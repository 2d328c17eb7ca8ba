"""Property-based pins of the oracle's quantizers (hypothesis), on the inputs that break
quantizers: exact half-way quotients, all-equal groups, subnormals and the bf16 extremes.

Each property is a closed form, an invariant or a brute-force search, never the oracle's
own formula typed again:
  INT4 ("Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers", 技术细节 1 step 3: scale
  absmax/7 per 64-channel group, round half to even, clamp) -- exact halves round to the
  even code; an all-equal group is all sevens; sign symmetry; power-of-two equivariance;
  every code is the nearest grid point (exhaustive search) and within half a step.
  NVFP4 (same page, 技术细节 3) -- the block scale is the E4M3 value nearest to the block's
  amax / (6 S) by exhaustive search over all 127 positive codes; every code is the E2M1
  value nearest to v / (scale S) (exhaustive over the 8 magnitudes, ties to the even code).
  AWQ ("Diffusers Natively Integrates Nunchaku Lite ...", third paragraph: 4-bit weights,
  group-64 scales and zero points) -- codes and zero points in [0, 15]; every in-range
  element reconstructs within half a scale step; a constant group keeps its value exactly
  when the value is an integer.
"""
import math

import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import oracle  # noqa: E402

SETTINGS = dict(max_examples=120, deadline=None, derandomize=True, database=None)
F32_MIN_NORMAL = 2.0 ** -126


def f32(x):
    return np.asarray(x, dtype=np.float32)


def codes_of(vals):
    c, s = oracle.quant_rows_int4(f32(vals).reshape(1, -1))
    return oracle.unpack_int4(c)[0].astype(np.int64), s[0]


# ---- strategies
finite_f32 = st.floats(width=32, allow_nan=False, allow_infinity=False, allow_subnormal=True)
bf16_extreme = st.sampled_from([3.3895313892515355e38, -3.3895313892515355e38,   # bf16 max
                                F32_MIN_NORMAL, 2.0 ** -133, -(2.0 ** -133)])          # bf16 subnormal min


@st.composite
def group_values(draw):
    """64 fp32 values: a mix of ordinary, subnormal, extreme and repeated magnitudes."""
    kind = draw(st.sampled_from(["any", "subnormal", "extreme", "scaled"]))
    if kind == "any":
        v = draw(st.lists(finite_f32, min_size=64, max_size=64))
    elif kind == "subnormal":
        v = draw(st.lists(st.floats(min_value=-F32_MIN_NORMAL, max_value=F32_MIN_NORMAL, width=32, allow_subnormal=True),
                          min_size=64, max_size=64))
    elif kind == "extreme":
        v = draw(st.lists(st.one_of(bf16_extreme, finite_f32), min_size=64, max_size=64))
    else:
        e = draw(st.integers(-140, 120))
        ints = draw(st.lists(st.integers(-1000, 1000), min_size=64, max_size=64))
        v = [math.ldexp(i, e) for i in ints]
    return f32(v)


# ---- INT4
@settings(**SETTINGS)
@given(e=st.integers(-140, 100), ks=st.lists(st.integers(-7, 6), min_size=63, max_size=63),
       neg=st.booleans())
def test_int4_exact_halves_round_to_even(e, ks, neg):
    # one element +-7 * 2^e makes the scale exactly 2^e; the others are (k + 1/2) 2^e, so
    # every quotient is an exact half and must go to the even neighbour
    anchor = -7.0 if neg else 7.0
    vals = [math.ldexp(anchor, e)] + [math.ldexp(k + 0.5, e) for k in ks]
    assert all(float(f32(v)) == v for v in vals)
    q, s = codes_of(vals)
    assert s[0] == np.float32(math.ldexp(1.0, e))
    expect = [int(anchor)] + [round(k + 0.5) for k in ks]   # Python rounds halves to even
    assert q.tolist() == expect
    assert all(c % 2 == 0 for c in q[1:])


@settings(**SETTINGS)
@given(v=st.floats(min_value=2.0 ** -120, max_value=3.3895313892515355e38, width=32),
       neg=st.booleans())
def test_int4_all_equal_group_is_all_sevens(v, neg):
    v = -v if neg else v
    q, s = codes_of([v] * 64)
    assert np.all(q == (-7 if neg else 7))
    assert s[0] > 0


@settings(**SETTINGS)
@given(vals=group_values())
def test_int4_nearest_grid_point_sign_symmetry(vals):
    q, s = codes_of(vals)
    s0 = float(s[0])
    assert -7 <= q.min() and q.max() <= 7
    if s0 == 0.0:   # absmax / 7 underflowed (or the group is zero): all codes zero
        assert np.all(q == 0)
        return
    x = vals.astype(np.float64)
    # nearest point of the grid {c * s}: no other code is strictly closer (up to the
    # fp32 quotient's own rounding, one part in 2^23 of the step)
    grid = np.arange(-8, 8)[None, :] * s0
    d = np.abs(x[:, None] - grid)
    best = d.min(axis=1)
    mine = np.abs(x - q * s0)
    assert np.all(mine <= best + s0 * 2.0 ** -22 + 1e-300)
    assert np.all(mine <= 0.5 * s0 * (1 + 2.0 ** -21) + 1e-300)
    qn, sn = codes_of(-vals)
    assert sn[0] == s[0] and np.array_equal(qn, -q)


@settings(**SETTINGS)
@given(vals=group_values(), p=st.integers(-20, 20))
def test_int4_power_of_two_equivariance(vals, p):
    # exact only while every value and the scale stay normal and finite
    a = float(np.max(np.abs(vals)))
    if a == 0.0 or a / 7 < F32_MIN_NORMAL * 2.0 ** 24 or a * 2.0 ** p > 3e38 or a * 2.0 ** p / 7 < F32_MIN_NORMAL * 2.0 ** 24:
        return
    nz = np.abs(vals[vals != 0])
    if nz.size and (nz.min() < F32_MIN_NORMAL or nz.min() * 2.0 ** p < F32_MIN_NORMAL):
        return
    q, s = codes_of(vals)
    q2, s2 = codes_of(vals * np.float32(2.0 ** p))
    assert np.array_equal(q2, q)
    assert s2[0] == s[0] * np.float32(2.0 ** p)


# ---- NVFP4
def e4m3_positive_table():
    vals = oracle.e4m3_decode(np.arange(1, 127, dtype=np.uint8))   # 0x7f is NaN in E4M3 FN
    return np.asarray(vals, np.float64)


E4M3 = e4m3_positive_table()
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


@settings(**SETTINGS)
@given(vals=st.lists(st.floats(min_value=-1048576.0, max_value=1048576.0, width=32, allow_subnormal=True),
                     min_size=16, max_size=16),
       S=st.sampled_from([2.0 ** -20, 1e-3, 0.0123, 0.5, 1.0, 7.0, 300.0]))
def test_nvfp4_scale_and_codes_nearest_by_search(vals, S):
    v = f32(vals)
    S = np.float32(S)
    c, sb = oracle.quant_rows_nvfp4(v.reshape(1, 16), S)
    sbv = float(oracle.e4m3_decode(sb.reshape(-1))[0])
    a = float(np.max(np.abs(v)))
    target = float(np.float32(a) / np.float32(np.float32(6.0) * S))
    # the block scale: the E4M3 value nearest to the (saturated) target, ties to even code
    t = min(target, 448.0)
    if t > 0:
        d = np.abs(E4M3 - t)
        cand = np.flatnonzero(d == d.min()) + 1
        near_zero = t <= 2.0 ** -10    # half the smallest subnormal: may round to zero
        assert (sbv in E4M3[cand - 1]) or (near_zero and sbv == 0.0)
        if len(cand) > 1 and sbv != 0.0:
            code = int(np.flatnonzero(E4M3 == sbv)[0]) + 1
            assert code % 2 == 0
    else:
        assert sbv == 0.0
    u = oracle.unpack_u4(c)[0]
    if sbv == 0.0:
        assert np.all(u & 7 == 0)
        return
    dd = float(np.float32(np.float32(sbv) * S))
    for x, code in zip(v, u):
        y = abs(float(np.float32(x / np.float32(dd))))
        dist = np.abs(E2M1 - y)
        cand = np.flatnonzero(dist == dist.min())
        assert (code & 7) in cand
        if len(cand) > 1:
            assert (code & 7) % 2 == 0
        assert bool(code & 8) == bool(np.signbit(x))


# ---- AWQ
@settings(**SETTINGS)
@given(vals=st.lists(st.floats(min_value=-8192.0, max_value=8192.0, width=32, allow_subnormal=True),
                     min_size=64, max_size=64))
def test_awq_codes_in_range_and_reconstruct(vals):
    w = f32(vals).reshape(1, 64)
    q, sc, z = oracle.awq_quant_weight(w)
    qq = oracle.unpack_u4(q)[0].astype(np.int64)
    s = float(oracle.bf16_to_f64(sc.reshape(-1))[0])
    zz = float(oracle.bf16_to_f64(z.reshape(-1))[0])
    assert s > 0 and 0 <= zz <= 15 and zz == int(zz)
    assert qq.min() >= 0 and qq.max() <= 15
    rec = (qq - zz) * s
    lo, hi = -zz * s, (15 - zz) * s     # the representable range of this group
    inside = (w[0] >= lo) & (w[0] <= hi)
    err = np.abs(rec - w[0].astype(np.float64))
    # half a step, plus the fp32 quotient's rounding
    assert np.all(err[inside] <= 0.5 * s * (1 + 2.0 ** -20) + 1e-30)
    # outside the range the code saturates at the nearer end
    assert np.all(qq[w[0] < lo] == 0) and np.all(qq[w[0] > hi] == 15)


@settings(**SETTINGS)
@given(n=st.integers(-7, 15))
def test_awq_constant_integer_group_is_exact(n):
    # range 0: the scale falls back to 1 and an integer value in [-15, 15] round-trips
    w = np.full((1, 64), np.float32(n))
    q, sc, z = oracle.awq_quant_weight(w)
    qq = oracle.unpack_u4(q)[0].astype(np.int64)
    s = float(oracle.bf16_to_f64(sc.reshape(-1))[0])
    zz = float(oracle.bf16_to_f64(z.reshape(-1))[0])
    assert s == 1.0
    assert np.all((qq - zz) * s == n)

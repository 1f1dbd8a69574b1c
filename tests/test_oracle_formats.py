"""Pins of the oracle's number formats: bf16, E4M3, E2M1, E8M0.

Each test checks the oracle against something other than its own formulas:
torch's float8 / bfloat16 casts and decoders (library routines), the golden
landmark tables (the format definitions), brute-force nearest search over the
whole code table, and defining inequalities of the scale rule.
"""

import math
import struct
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 0), float(v)))
    return rows


def _same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return both_nan | eq


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def torch_e4m3_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def nearest_code(table_pos, v):
    """Brute force: index of the nearest entry of the ascending table of
    non-negative finite values, ties to the even index, saturating at the end."""
    a = np.abs(np.asarray(v, np.float64))
    n = len(table_pos)
    hi = np.searchsorted(table_pos, a, side="left")
    over = hi >= n
    hi = np.clip(hi, 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    dlo = a - table_pos[lo]
    dhi = table_pos[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return np.where(over, n - 1, idx)


# ---------------------------------------------------------------- bf16

def test_bf16_widen_exhaustive(orc):
    ref = _all_bf16_values()
    got = np.array([orc.lib().orc_bf16_to_f64(h) for h in range(65536)])
    assert _same(got, ref).all()


def test_bf16_rne_matches_torch_on_fp32(orc):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    special = np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.3895314e38, 3.4e38,
                        1e-40, -1e-45, 2.0**-126, 2.0**-133], np.float32)
    f = np.concatenate([f, special])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_rne(float(v)) for v in f], np.uint16)
    assert (got == ref).all()


def test_bf16_rne_nan_is_canonical(orc):
    # a NaN in the bf16 intermediate carries no sign or payload: whatever NaN
    # fp64 arithmetic made (x86 makes Inf * 0 a negative one), the result is
    # the canonical quiet NaN
    with np.errstate(invalid="ignore"):
        inf_times_zero = np.float64(np.inf) * np.float64(0.0)
    neg_nan = -np.float64(np.nan)
    assert np.isnan(inf_times_zero) and np.signbit(neg_nan)
    for v in (float("nan"), float(neg_nan), float(inf_times_zero),
              struct.unpack("<d", struct.pack("<Q", 0x7FF0000000000001))[0],   # signalling
              struct.unpack("<d", struct.pack("<Q", 0xFFF8DEADBEEF0000))[0]):  # payload, negative
        assert math.isnan(v)
        assert orc.bf16_rne(v) == 0x7FC0
    # infinities and zeros keep their signs
    assert orc.bf16_rne(math.inf) == 0x7F80 and orc.bf16_rne(-math.inf) == 0xFF80
    assert orc.bf16_rne(0.0) == 0x0000 and orc.bf16_rne(-0.0) == 0x8000


def test_bf16_rne_ties_from_fp64(orc):
    # midpoints between neighbouring bf16 values go to the even one; a hair
    # above or below a midpoint goes to the nearer one (single rounding from fp64)
    rng = np.random.default_rng(12)
    for h in rng.integers(0x0080, 0x7F7F, size=3000):
        h = int(h)
        a = orc.lib().orc_bf16_to_f64(h)
        b = orc.lib().orc_bf16_to_f64(h + 1)
        mid = (a + b) / 2
        even = h if h % 2 == 0 else h + 1
        assert orc.bf16_rne(mid) == even
        assert orc.bf16_rne(math.nextafter(mid, math.inf)) == h + 1
        assert orc.bf16_rne(math.nextafter(mid, -math.inf)) == h
        assert orc.bf16_rne(-mid) == 0x8000 | even


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_matches_torch_exhaustive(orc):
    ref = torch_e4m3_table()
    got = orc.decode_table("e4m3")
    assert _same(got, ref).all()


def test_e4m3_golden_points(orc):
    for c, v in _read_table("e4m3_points.txt"):
        got = orc.decode("e4m3", c)
        assert _same([got], [v]).all(), (hex(c), got, v)


def test_e4m3_round_trip_all_codes(orc):
    tab = torch_e4m3_table()
    finite = [c for c in range(256) if not math.isnan(tab[c])]
    assert len(finite) == 254  # exactly one NaN pattern per sign
    for rnd in ("rne", "sr"):
        for r in (0, 1, 0x80000000, 0xFFFFFFFF):
            got = orc.encode_array("e4m3", rnd, tab[finite], np.full(len(finite), r))
            assert (got == np.array(finite)).all()


def test_e4m3_rne_brute_force_bf16_times_scales(orc):
    tab = torch_e4m3_table()
    pos = tab[:127]  # codes 0x00..0x7E, ascending, finite
    assert np.all(np.diff(pos) > 0)
    vals = _all_bf16_values()
    vals = vals[np.isfinite(vals)]
    for k in range(-20, 21, 1):
        v = np.ldexp(vals, k)
        got = orc.encode_array("e4m3", "rne", v)
        want = nearest_code(pos, v).astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (k, v[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3_rne_brute_force_fp64_ties(orc):
    tab = torch_e4m3_table()
    pos = tab[:127]
    mids = (pos[:-1] + pos[1:]) / 2
    v = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                        [448.0, 450.0, 464.0, 479.9, 480.0, 511.9, 1e9, 2.0**-10, 2.0**-11]])
    v = np.concatenate([v, -v])
    got = orc.encode_array("e4m3", "rne", v)
    want = nearest_code(pos, v).astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    assert (got == want).all()


def test_e4m3_rne_matches_torch_cast_in_range(orc):
    rng = np.random.default_rng(13)
    f = np.concatenate([
        rng.uniform(-448, 448, 100_000),
        rng.standard_normal(100_000) * 0.01,
        np.ldexp(rng.uniform(1, 2, 50_000), rng.integers(-14, 9, 50_000)),
    ]).astype(np.float32)
    f = np.clip(f, -448, 448)
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.encode_array("e4m3", "rne", f.astype(np.float64))
    assert (got == ref).all()


def test_e4m3_signed_zero_kept(orc):
    assert orc.encode("e4m3", "rne", -0.0) == 0x80
    assert orc.encode("e4m3", "rne", -1e-30) == 0x80
    assert orc.encode("e4m3", "rne", 1e-30) == 0x00
    assert orc.encode("e4m3", "sr", -1e-30, 0) == 0x80


# ---------------------------------------------------------------- E2M1

def test_e2m1_decode_golden(orc):
    tab = _read_table("e2m1_values.txt")
    assert len(tab) == 16
    got = orc.decode_table("e2m1")
    assert _same(got, [v for _, v in tab]).all()


def test_e2m1_round_trip_and_brute_force(orc):
    tab = np.array([v for _, v in _read_table("e2m1_values.txt")])
    for rnd in ("rne", "sr"):
        got = orc.encode_array("e2m1", rnd, tab, np.full(16, 0x12345678))
        assert (got == np.arange(16)).all()
    pos = tab[:8]
    # documented ties: .25->0, .75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, w in ties.items():
        c = orc.encode("e2m1", "rne", v)
        assert orc.decode("e2m1", c) == w
    vals = _all_bf16_values()
    vals = vals[np.isfinite(vals)]
    for k in range(-6, 7):
        v = np.ldexp(vals, k)
        got = orc.encode_array("e2m1", "rne", v)
        want = nearest_code(pos, v).astype(np.uint8) | np.where(np.signbit(v), 8, 0).astype(np.uint8)
        assert (got == want).all(), k


# ---------------------------------------------------------------- E8M0

@pytest.mark.parametrize("elem,emax", [("e4m3", 8), ("e2m1", 2)])
def test_e8m0_scale_defining_inequalities(orc, elem, emax):
    vals = _all_bf16_values()
    vals = vals[np.isfinite(vals) & (vals > 0)]
    rng = np.random.default_rng(14)
    extra = np.ldexp(rng.uniform(1, 2, 20000), rng.integers(-160, 128, 20000))
    extra = np.concatenate([extra, np.ldexp(1.0, np.arange(-149, 128)),
                            np.nextafter(np.ldexp(1.0, np.arange(-148, 128)), 0)])
    for a in np.concatenate([vals, extra]):
        code = orc.e8m0_scale(elem, float(a))
        assert 0 <= code <= 254
        s = code - 127
        if code == 0 and a < math.ldexp(1.0, emax - 126):
            continue  # clamped at 2^-127: a is below the lowest binade the scale can anchor
        r = math.ldexp(float(a), -(s + emax))
        assert 1.0 <= r < 2.0, (a, code)


def test_e8m0_special_cases(orc):
    for elem in ("e4m3", "e2m1"):
        assert orc.e8m0_scale(elem, 0.0) == 0
        assert orc.e8m0_scale(elem, float("nan")) == 0xFF
        assert orc.e8m0_scale(elem, float("inf")) == 0xFF
    # the scale never lets the block absmax overflow after rounding: a / 2^s < 2^(emax+1)
    assert orc.e8m0_scale("e4m3", 448.0) == 127
    assert orc.e8m0_scale("e4m3", 511.0) == 127
    assert orc.e8m0_scale("e4m3", 512.0) == 128
    assert orc.e8m0_scale("e2m1", 6.0) == 127
    assert orc.e8m0_scale("e2m1", 8.0) == 128


@pytest.mark.parametrize("elem,maxval", [("e4m3", 448.0), ("e2m1", 6.0)])
def test_e8m0_ceil_rule_smallest_non_saturating_scale(orc, elem, maxval):
    """Round-up rule: the smallest power of two that brings the block absmax
    within the element maximum, checked against a search over every byte."""
    vals = _all_bf16_values()
    vals = vals[np.isfinite(vals) & (vals > 0)]
    rng = np.random.default_rng(15)
    extra = np.ldexp(rng.uniform(1, 2, 20000), rng.integers(-160, 128, 20000))
    extra = np.concatenate([extra, np.ldexp(maxval, np.arange(-140, 128)),
                            np.nextafter(np.ldexp(maxval, np.arange(-140, 128)), np.inf)])
    a = np.concatenate([vals, extra])
    got = np.array([orc.e8m0_scale(elem, float(v), rule="ceil") for v in a])
    cand = np.arange(-127, 128)
    ok = a[:, None] <= np.ldexp(maxval, cand)[None, :]
    want = np.where(ok.any(1), np.argmax(ok, axis=1), 254)
    assert (got == want).all()
    floor = np.array([orc.e8m0_scale(elem, float(v)) for v in a])
    assert set(np.unique(got - floor)) <= {0, 1}


def test_e8m0_ceil_rule_golden_points(orc):
    for elem in ("e4m3", "e2m1"):
        assert orc.e8m0_scale(elem, 0.0, rule="ceil") == 0
        assert orc.e8m0_scale(elem, float("nan"), rule="ceil") == 0xFF
        assert orc.e8m0_scale(elem, float("inf"), rule="ceil") == 0xFF
    assert orc.e8m0_scale("e4m3", 448.0, rule="ceil") == 127
    assert orc.e8m0_scale("e4m3", 449.0, rule="ceil") == 128
    assert orc.e8m0_scale("e4m3", 896.0, rule="ceil") == 128
    assert orc.e8m0_scale("e4m3", 897.0, rule="ceil") == 129
    assert orc.e8m0_scale("e4m3", 256.0, rule="ceil") == 127   # floor rule gives 127 too
    assert orc.e8m0_scale("e4m3", 224.0, rule="ceil") == 126   # 224 = 448 / 2
    assert orc.e8m0_scale("e2m1", 6.0, rule="ceil") == 127
    assert orc.e8m0_scale("e2m1", 6.5, rule="ceil") == 128
    assert orc.e8m0_scale("e2m1", 3.0, rule="ceil") == 126
    assert orc.e8m0_scale("e2m1", 4.0, rule="ceil") == 127     # floor rule gives 127


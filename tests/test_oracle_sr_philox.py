"""Pins of the oracle's stochastic rounding and its Philox stream.

Stochastic rounding is defined on the aibr.jp stochastic-rounding explainer
(core-technique paragraph): one of the two neighbouring representable values is
chosen with a probability set by the distance, so the expected value equals the
input. The Philox4x32-10 stream is pinned against two independent
implementations: numpy's Philox4x64-10 (same round structure and key schedule,
one shared body in the oracle) and rocRAND's Philox4x32-10 engine, built here
from its header as a host program.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from test_oracle_formats import nearest_code, torch_e4m3_table

HELPER = os.path.join(os.path.dirname(__file__), "helpers", "rocrand_philox_words.cpp")


# ---------------------------------------------------------------- Philox

def test_philox4x64_matches_numpy(orc):
    rng = np.random.default_rng(21)
    for trial in range(40):
        key = int(rng.integers(0, 2**63)) << 65 | int(rng.integers(0, 2**63))
        key &= (1 << 128) - 1
        ctr = int(rng.integers(0, 2**63)) * (trial % 5)
        if trial == 3:
            ctr = (1 << 64) - 1          # carry into the second word
        bg = np.random.Philox(key=key, counter=ctr)
        raw = bg.random_raw(4)
        c = ctr + 1                      # numpy encrypts the incremented counter
        words = [(c >> (64 * i)) & (2**64 - 1) for i in range(4)]
        got = orc.philox4x64(words, [key & (2**64 - 1), key >> 64])
        assert [int(v) for v in got] == [int(v) for v in raw]


@pytest.fixture(scope="module")
def rocrand_words(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND helper")
    exe = str(tmp_path_factory.mktemp("rocrand") / "rp")
    subprocess.check_call([hipcc, "-O1", "-o", exe, HELPER], cwd="/tmp")

    def run(seed, sub, off, n):
        out = subprocess.check_output([exe, str(seed), str(sub), str(off), str(n)], text=True)
        return np.array([int(v) for v in out.split()], dtype=np.uint64)
    return run


def test_philox4x32_stream_matches_rocrand(orc, rocrand_words):
    # the stochastic-rounding word of element n under (seed, offset) is word
    # n of rocRAND's engine seeded with `seed` at subsequence `offset`
    cases = [(0x5EED, 0, 0, 4096), (0, 0, 0, 64), (0xFFFFFFFFFFFFFFFF, 7, 123, 257),
             (0x123456789ABCDEF0, 1 << 40, (1 << 34) + 5, 300), (42, 3, (1 << 32) - 2, 64)]
    for seed, offset, n0, count in cases:
        want = rocrand_words(seed, offset, n0, count)
        got = orc.sr_words(seed, offset, n0, count).astype(np.uint64)
        assert (got == want).all(), (seed, offset, n0)


def test_philox4x32_uniformity(orc):
    w = orc.sr_words(0x5EED, 0, 0, 1 << 18)
    for shift in (0, 8, 16, 24):
        byte = (w >> shift) & 0xFF
        counts = np.bincount(byte, minlength=256)
        expect = w.size / 256
        chi2 = ((counts - expect) ** 2 / expect).sum()
        assert chi2 < 255 + 8 * np.sqrt(2 * 255)  # ~8 sigma band for 255 dof
    bits = np.unpackbits(w.view(np.uint8))
    assert abs(bits.mean() - 0.5) < 5 * 0.5 / np.sqrt(bits.size)


# ---------------------------------------------------------------- SR

def _neighbours(pos, v):
    """Round-down and round-up neighbours of |v| on the finite grid (brute force)."""
    a = np.abs(v)
    hi = np.searchsorted(pos, a, side="left")
    hi = np.clip(hi, 0, len(pos) - 1)
    exact = pos[hi] == a
    lo = np.where(exact, hi, np.clip(hi - 1, 0, len(pos) - 1))
    return lo, hi


def test_sr_result_is_a_neighbour(orc):
    tab = torch_e4m3_table()
    pos = tab[:127]
    rng = np.random.default_rng(22)
    v = np.ldexp(rng.uniform(1, 2, 200_000), rng.integers(-12, 9, 200_000))
    v = np.clip(v, 0, 448) * np.where(rng.random(v.size) < 0.5, -1, 1)
    r = orc.sr_words(7, 0, 0, v.size)
    got = orc.encode_array("e4m3", "sr", v, r)
    lo, hi = _neighbours(pos, v)
    mag = got & 0x7F
    assert np.all((mag == lo) | (mag == hi))
    assert np.all((got >> 7) == np.signbit(v))


def test_sr_exact_on_grid(orc):
    tab = torch_e4m3_table()
    fin = np.array([c for c in range(256) if not np.isnan(tab[c])])
    for r in (0, 1, 12345, 0xFFFFFFFF):
        got = orc.encode_array("e4m3", "sr", tab[fin], np.full(fin.size, r))
        assert (got == fin).all()


@pytest.mark.parametrize("elem", ["e4m3", "e2m1"])
@pytest.mark.parametrize("frac", [0.001, 0.1, 0.25, 0.5, 0.75, 0.9])
def test_sr_probability_follows_distance(orc, elem, frac):
    # value between two neighbours at fractional distance `frac`; P(up) must be frac
    if elem == "e4m3":
        lo, hi = 1.25, 1.375
    else:
        lo, hi = 1.0, 1.5
    v = lo + frac * (hi - lo)
    n = 200_000
    r = orc.sr_words(0xABC, 1, 0, n)
    got = orc.encode_array(elem, "sr", np.full(n, v), r)
    up = orc.encode(elem, "rne", hi)
    down = orc.encode(elem, "rne", lo)
    assert set(np.unique(got)) <= {up, down}
    p_hat = (got == up).mean()
    sigma = np.sqrt(frac * (1 - frac) / n)
    assert abs(p_hat - frac) < 5 * sigma + 1e-9


def test_sr_is_unbiased(orc):
    tab = torch_e4m3_table()
    rng = np.random.default_rng(23)
    n = 1_000_000
    v = np.ldexp(rng.uniform(1, 2, n), rng.integers(-9, 8, n))
    r = orc.sr_words(0x5EED, 0, 0, n)
    got = tab[orc.encode_array("e4m3", "sr", v, r)]
    # error in units of the local quantum (2^(floor(log2 v) - 3), min 2^-9)
    q = np.ldexp(1.0, np.maximum(np.floor(np.log2(v)).astype(int), -6) - 3)
    e = (got - v) / q
    assert np.all(np.abs(e) < 1)
    assert abs(e.mean()) < 5 * e.std() / np.sqrt(n)
    # RNE on the same values is biased only by ties; SR spreads both ways
    assert (e > 0).mean() > 0.3 and (e < 0).mean() > 0.3


def test_sr_saturates(orc):
    r = np.array([0, 1 << 31, 0xFFFFFFFF], np.uint32)
    got = orc.encode_array("e4m3", "sr", np.full(3, 470.0), r)
    assert (got == 0x7E).all()
    got = orc.encode_array("e2m1", "sr", np.full(3, -7.5), r)
    assert (got == 0xF).all()


# ---------------------------------------------------------------- the B-bit decision, exactly

def _e2m1_table():
    path = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")
    tab = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            c, v = line.split()
            tab[int(c, 0)] = float(v)
    return np.array([tab[c] for c in range(16)])


def _sr_by_definition(elem, v, r, table):
    """Stochastic rounding written out with exact rationals: q = |v| in units of
    the local quantum (binade of |v|, at least the smallest normal), n = floor(q),
    f = q - n; round up iff r < 2^(32-B) * floor(f * 2^B), B the fp32 mantissa
    bits the format drops (20 for E4M3, 22 for E2M1); saturate at the largest
    value; then the code whose table value is the result, with v's sign."""
    from fractions import Fraction
    mbits, emin, maxval = (3, -6, 448.0) if elem == "e4m3" else (1, 0, 6.0)
    B = 23 - mbits
    a = Fraction(abs(v))
    neg = np.signbit(v)
    if a == 0:
        mag = Fraction(0)
    else:
        e = a.numerator.bit_length() - a.denominator.bit_length()
        if Fraction(2) ** e > a:
            e -= 1
        e = max(e, emin)
        quantum = Fraction(2) ** (e - mbits)
        q = a / quantum
        n = q.numerator // q.denominator
        f = q - n
        thr = (f * 2 ** B).numerator // (f * 2 ** B).denominator * 2 ** (32 - B)
        mag = min((n + (1 if r < thr else 0)) * quantum, Fraction(maxval))
    half = len(table) // 2
    pos = [c for c in range(half) if table[c] == float(mag)]
    assert len(pos) == 1, (v, mag)
    return pos[0] | (half if neg else 0)


@pytest.mark.parametrize("elem", ["e4m3", "e2m1"])
def test_sr_decision_is_the_b_bit_rule(orc, elem):
    # random values over every binade that reaches subnormal targets and far
    # below them, random words and words at the B-bit threshold +- 1 and +- one
    # step of the dropped low bits
    table = torch_e4m3_table() if elem == "e4m3" else _e2m1_table()
    mbits, emin, top = (3, -6, 8) if elem == "e4m3" else (1, 0, 2)
    B = 23 - mbits
    rng = np.random.default_rng(31 if elem == "e4m3" else 32)
    n = 3000
    e = rng.integers(-40, top + 1, n)
    v = np.ldexp(rng.uniform(1, 2, n), e).astype(np.float32).astype(np.float64)
    v = np.minimum(v, 448.0 if elem == "e4m3" else 6.0) * np.where(rng.random(n) < 0.5, -1, 1)
    a = np.abs(v)
    ee = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1))), emin)
    q = np.ldexp(a, (-(ee - mbits)).astype(np.int64))
    thr = np.ldexp(np.floor(np.ldexp(q - np.floor(q), B)), 32 - B)
    step = 2.0 ** (32 - B)
    words = [rng.integers(0, 1 << 32, n, dtype=np.uint64)]
    for d in (-step - 1, -1, 0, step - 1, step):
        words.append(np.clip(thr + d, 0, 2 ** 32 - 1).astype(np.uint64))
    for r in words:
        r = r.astype(np.uint32)
        got = orc.encode_array(elem, "sr", v, r)
        want = [_sr_by_definition(elem, float(v[i]), int(r[i]), table) for i in range(n)]
        assert (got == np.array(want)).all()


def test_sr_b_bit_rule_differs_from_a_full_word_rule_only_below_the_dropped_bits(orc):
    # Mutation guard on the rule itself: a value whose fraction (in units of the
    # quantum) has bits only below the top B rounds down under the B-bit rule
    # for every word, where a 32-bit comparison would round up for small words.
    # A subnormal E4M3 target (quantum 2^-9) and an fp64 value at a normal one.
    for v, lo, hi in ((2.0 ** -8 + 2.0 ** -30, 2.0 ** -8, 3 * 2.0 ** -9),
                      (1.25 + 2.0 ** -30, 1.25, 1.375)):
        quantum = hi - lo
        f = (v - lo) / quantum                  # exact: power-of-two quantum
        assert 0 < f < 2.0 ** -20
        full = int(np.floor(np.ldexp(f, 32)))
        assert full >= 1
        r = np.array([0, full - 1, full, 0xFFFFFFFF], np.uint32)
        got = orc.encode_array("e4m3", "sr", np.full(4, v), r)
        assert (got == orc.encode("e4m3", "rne", lo)).all(), (v, got)
    # and at a fraction with bits at the top B, the threshold is 2^12 floor(f 2^20)
    v = 1.25 + 2.0 ** -20                   # f = 2^-17: floor(f 2^20) = 8
    got = orc.encode_array("e4m3", "sr", np.full(2, v), np.array([8 * 4096 - 1, 8 * 4096], np.uint32))
    assert list(got) == [orc.encode("e4m3", "rne", 1.375), orc.encode("e4m3", "rne", 1.25)]

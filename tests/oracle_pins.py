"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function takes a loaded ``oracle.Oracle`` and raises
AssertionError when the oracle disagrees with what mathematics or the format
definition fixes.  ``tests/test_oracle_pins.py`` runs them on the real oracle;
``tests/test_oracle_mutants.py`` runs them on deliberately broken copies of the
oracle's C source and requires every copy to fail at least one pin.

What pins what:
  * f16 decode    : all 65,536 patterns vs numpy and vs Python's struct codec.
  * f16 encode    : random doubles, exact ties, subnormals and overflow vs
                    numpy's correctly rounded conversion.
  * matmul        : exact rational brute force (fractions) on tiny shapes with
                    every code value, within the f64 summation error bound and
                    bit-exact where the exact sum is representable; closed
                    forms (constant codes); one-hot x across word and group
                    boundaries; linearity identities.
  * SiLU / FFN    : silu(0)=0, silu(ln 3)=(3/4)ln 3, silu(-g)=silu(g)-g, the
                    gate (not up) is the one gated.
  * argmax        : planted maximum, ties go to the lowest index.
  * attention     : one position returns its V row, equal scores the mean of
                    V, a dominant key its V row, grouped-query heads, page
                    order invariance; the softmax weights in closed form at
                    known score gaps and several temperatures (base e, one
                    scaling), and the magnitude sum sum_t p_t |V_t| with V of
                    both signs.
  * RoPE          : a hand example (pairing and frequency), identity at 0,
                    norm preservation, q.k depends on the position difference
                    only, only q and k heads of the fused QKV rotate; the
                    rotary-pair layout decoded in the opposite direction.
  * add + RMSNorm : a hand example (x = (3, 4)), the residual against numpy's
                    f16 addition, constant inputs (+-1, and 1/sqrt(2) with
                    eps = mean square), scale invariance, exact gamma scaling.
  * int3          : one-hot x at every position (codes crossing word
                    boundaries included) against codes written through a
                    Python integer stream; constant codes 0, 4, 7; the device
                    layout read back destination by destination.
  * int8 KV       : a hand-quantised row away from ties, the +-127 maximum
                    (placed at every index of the row, the last included),
                    reconstruction within half a step, power-of-two scaling,
                    the zero row; the append's bytes against blocks located in
                    Python; int8 attention equal bit for bit to the f16
                    attention over the exactly dequantised cache.
  * device layout : hand-derived geometry table (tests/golden), a byte-level
                    hand example, and a decoder written in the opposite
                    direction (destination -> logical) over random shapes.
"""
from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

import numpy as np

import seeded_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

U64 = 2.0 ** -53   # unit roundoff of f64


def half_fraction(bits: int) -> Fraction:
    """Exact value of an f16 pattern via Python's own binary16 codec."""
    return Fraction(struct.unpack("<e", struct.pack("<H", int(bits)))[0])


def exact_gemv(codes: np.ndarray, scales: np.ndarray, x: np.ndarray):
    """Exact rational y and sum|terms| for codes [n][k] (integers 0..15)."""
    n, k = codes.shape
    xs = [half_fraction(b) for b in x]
    ys, as_ = [], []
    for r in range(n):
        s_row = [half_fraction(b) for b in scales[r]]
        tot = Fraction(0)
        mag = Fraction(0)
        for kk in range(k):
            t = xs[kk] * (int(codes[r, kk]) - 8) * s_row[kk // 32]
            tot += t
            mag += abs(t)
        ys.append(tot)
        as_.append(mag)
    return ys, as_


# ---------------------------------------------------------------- f16 codec
def pin_half_decode_all_patterns(orc, quick=False):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = orc.halves_to_doubles(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros and the struct codec as a second reference
    assert math.copysign(1.0, orc.half_to_double(0x8000)) == -1.0
    step = 97 if quick else 7
    for b in range(0, 65536, step):
        if (b & 0x7C00) != 0x7C00:
            assert orc.half_to_double(b) == float(half_fraction(b)), hex(b)


def pin_half_encode_rne(orc, quick=False):
    rng = np.random.default_rng(1234)
    cnt = 20000 if quick else 300000
    parts = [
        rng.standard_normal(cnt // 4) * 10.0 ** rng.integers(-9, 6, cnt // 4),
        rng.uniform(-70000, 70000, cnt // 8),
        rng.uniform(-1e-4, 1e-4, cnt // 8),      # around the subnormal range
    ]
    # exact midpoints between neighbouring f16 values: ties must go to even
    b = rng.integers(0, 0x7bff, cnt // 4, dtype=np.int64).astype(np.uint16)
    lo = b.view(np.float16).astype(np.float64)
    hi = (b + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (lo + hi) / 2.0
    parts += [mids, -mids,
              np.array([65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25,
                        2.0 ** -25 * 3, 2.0 ** -24 * 1.5, 0.0, -0.0,
                        2.0 ** -14 - 2.0 ** -25, 6.1e-5])]
    v = np.concatenate(parts)
    ref = v.astype(np.float16).view(np.uint16)
    got = orc.doubles_to_halves(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(v[i], hex(ref[i]), hex(got[i])) for i in bad[:5]]
    assert orc.double_to_half(float("inf")) == 0x7C00
    assert orc.double_to_half(float("-inf")) == 0xFC00
    assert (orc.double_to_half(float("nan")) & 0x7C00) == 0x7C00


# ------------------------------------------------------------------ matmul
def _tiny_cases(quick):
    shapes = [(1, 32), (2, 64), (3, 96), (17, 32)] if not quick else \
             [(1, 32), (3, 96), (17, 32)]
    rng = np.random.default_rng(77)
    for n, k in shapes:
        codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
        codes.ravel()[:16] = np.arange(16)          # every code value appears
        scales = si.f16_bits(rng.uniform(-0.05, 0.05, (n, k // 32)))
        x = si.f16_bits(rng.standard_normal(k) * 2.0)
        yield codes, scales, x


def pin_gemv_rational(orc, quick=False):
    for codes, scales, x in _tiny_cases(quick):
        words = si.pack_codes(codes)
        y, a = orc.gemv(words, scales, x)
        ey, ea = exact_gemv(codes, scales, x)
        k = codes.shape[1]
        for r in range(codes.shape[0]):
            bound = (k * U64 / (1 - k * U64)) * float(ea[r])
            assert abs(Fraction(y[r]) - ey[r]) <= Fraction(bound), (r, y[r], float(ey[r]))
            assert abs(Fraction(a[r]) - ea[r]) <= Fraction(bound), (r, a[r], float(ea[r]))


def pin_gemv_exactly_representable(orc, quick=False):
    """x in {-4..4}/4, scales in {2^-7, 2^-8}: every term and partial sum is a
    multiple of 2^-10 well inside 53 bits, so f64 must be exact."""
    rng = np.random.default_rng(5)
    n, k = (5, 256) if quick else (9, 1024)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scales = si.f16_bits(2.0 ** -rng.integers(7, 9, (n, k // 32)))
    x = si.f16_bits(rng.integers(-4, 5, k) / 4.0)
    y, a = orc.gemv(si.pack_codes(codes), scales, x)
    ey, ea = exact_gemv(codes, scales, x)
    assert [Fraction(v) for v in y] == ey
    assert [Fraction(v) for v in a] == ea


def pin_gemv_closed_forms(orc, quick=False):
    k = 3072
    x = si.f16_bits(np.ones(k))
    # c = 15, s = 2^-6, x = 1: y = 7 * 2^-6 * 3072 = 336 exactly
    words = si.pack_codes(np.full((2, k), 15, np.uint8))
    scales = si.f16_bits(np.full((2, k // 32), 2.0 ** -6))
    y, a = orc.gemv(words, scales, x)
    assert list(y) == [336.0, 336.0] and list(a) == [336.0, 336.0]
    # constant code c, scale s, random x: y = (c - 8) * s * sum(x), exactly
    rng = np.random.default_rng(9)
    xr = si.f16_bits(rng.standard_normal(256))
    sx = sum(half_fraction(b) for b in xr)
    for c in (0, 3, 8, 12, 15):
        words = si.pack_codes(np.full((1, 256), c, np.uint8))
        s = si.f16_bits(np.full((1, 8), 0.0126953125))
        y, _ = orc.gemv(words, s, xr)
        exact = (c - 8) * Fraction(0.0126953125) * sx
        mag = abs(c - 8) * Fraction(0.0126953125) * sum(abs(half_fraction(b)) for b in xr)
        assert abs(Fraction(y[0]) - exact) <= Fraction(2 * 256 * U64) * mag, \
            (c, y[0], float(exact))
        if c == 8:
            assert y[0] == 0.0 and math.copysign(1.0, y[0]) == 1.0


def pin_gemv_one_hot(orc, quick=False):
    rng = np.random.default_rng(11)
    n, k = 7, 128
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scales = si.f16_bits(rng.uniform(0.005, 0.02, (n, k // 32)))
    words = si.pack_codes(codes)
    positions = [0, 1, 7, 8, 15, 31, 32, 33, 63, 64, 95, 100, 127]
    for kk in positions:
        x = np.zeros(k, np.uint16)
        x[kk] = 0x3C00          # 1.0
        y, _ = orc.gemv(words, scales, x)
        for r in range(n):
            want = (int(codes[r, kk]) - 8) * half_fraction(scales[r, kk // 32])
            assert Fraction(y[r]) == want, (kk, r)


def pin_gemv_linearity(orc, quick=False):
    rng = np.random.default_rng(13)
    w, s = si.draw_weight(rng, 6, 96)
    x = si.draw_x(rng, 96)
    y, a = orc.gemv(w, s, x)
    x2 = si.f16_bits(x.view(np.float16).astype(np.float64) * 2.0)
    xn = x ^ np.uint16(0x8000)
    y2, a2 = orc.gemv(w, s, x2)
    yn, an = orc.gemv(w, s, xn)
    assert np.array_equal(y2, 2.0 * y) and np.array_equal(a2, 2.0 * a)
    assert np.array_equal(yn, -y) and np.array_equal(an, a)


def pin_gemm_rows(orc, quick=False):
    """each row of the batched form is the single-vector form; and a closed
    form: X row i all (i+1)/4, constant code 12, scale 2^-5 -> 4*(i+1)/4*2^-5*k."""
    rng = np.random.default_rng(17)
    w, s = si.draw_weight(rng, 5, 64)
    X = si.draw_X(rng, 3, 64)
    Y, A = orc.gemm(w, s, X)
    for i in range(3):
        y, a = orc.gemv(w, s, X[i])
        assert np.array_equal(Y[i], y) and np.array_equal(A[i], a)
    k = 96
    words = si.pack_codes(np.full((4, k), 12, np.uint8))
    scales = si.f16_bits(np.full((4, k // 32), 2.0 ** -5))
    X = si.f16_bits(np.repeat((np.arange(3)[:, None] + 1) / 4.0, k, axis=1))
    Y, _ = orc.gemm(words, scales, X)
    for i in range(3):
        assert np.all(Y[i] == 4 * (i + 1) / 4.0 * 2.0 ** -5 * k)


# -------------------------------------------------------------- SiLU / FFN
def pin_silu(orc, quick=False):
    assert orc.silu(0.0) == 0.0
    ln3 = math.log(3.0)
    assert abs(orc.silu(ln3) - 0.75 * ln3) <= 4 * U64 * ln3
    for g in (0.1, 0.5, 1.0, 2.5, 7.0, 20.0):
        assert abs(orc.silu(-g) - (orc.silu(g) - g)) <= 8 * U64 * max(1.0, g)
    assert orc.silu(40.0) == 40.0
    assert -1e-12 < orc.silu(-40.0) < 0.0


def pin_ffn(orc, quick=False):
    """gate codes c_g, up codes c_u, x = 1: g = (c_g-8) s_g k, u = (c_u-8) s_u k;
    h = g * sigmoid(g) * u.  Gate 8 -> h = 0; up 8 -> h = 0; the gate is the
    gated half (silu applied to g, not to u)."""
    k, n = 64, 3
    x = si.f16_bits(np.ones(k))
    def w_const(c, s):
        return (si.pack_codes(np.full((n, k), c, np.uint8)),
                si.f16_bits(np.full((n, k // 32), s)))
    for cg, cu, sg, su in ((10, 13, 2.0 ** -5, 2.0 ** -6), (5, 14, 2.0 ** -4, 2.0 ** -3),
                           (8, 13, 2.0 ** -5, 2.0 ** -6), (12, 8, 2.0 ** -5, 2.0 ** -6)):
        gw, gs = w_const(cg, sg)
        uw, us = w_const(cu, su)
        out = orc.ffn_gate_up_silu(gw, gs, uw, us, x)
        g = (cg - 8) * sg * k
        u = (cu - 8) * su * k
        want = g / (1.0 + math.exp(-g)) * u
        assert np.all(np.abs(out["h"] - want) <= 8 * U64 * abs(want)), (cg, cu, out["h"], want)
        assert np.all(out["g"] == g) and np.all(out["u"] == u)
        assert np.all(out["ag"] == abs(g)) and np.all(out["au"] == abs(u))


# ------------------------------------------------------------------ argmax
def pin_argmax(orc, quick=False):
    assert orc.argmax(np.array([1.0, 3.0, 2.0])) == 1
    assert orc.argmax(np.array([5.0, 5.0, 5.0])) == 0
    assert orc.argmax(np.array([-3.0, -1.0, -1.0, -2.0])) == 1
    v = np.random.default_rng(3).standard_normal(1000)
    v[417] = 10.0
    v[901] = 10.0
    assert orc.argmax(v) == 417


def pin_lmhead(orc, quick=False):
    """planted winner (all codes 15, x = 1) and a planted exact tie (two equal
    rows) resolve to the lowest index; logits are the matmul."""
    rng = np.random.default_rng(23)
    n, k = 40, 96
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    codes[29] = 15
    codes[33] = 15
    scales = si.f16_bits(rng.uniform(0.005, 0.02, (n, k // 32)))
    scales[33] = scales[29]
    words = si.pack_codes(codes)
    x = si.f16_bits(np.ones(k))
    logits, a, idx = orc.lmhead(words, scales, x)
    y, _ = orc.gemv(words, scales, x)
    assert np.array_equal(logits, y) and idx == 29


# ----------------------------------------------------------- device layout
def pin_add_rmsnorm(orc, quick=False):
    """Residual add + RMSNorm: a hand example, the residual against numpy's
    f16 addition, closed forms and exact invariances."""
    f16 = si.f16_bits
    one = f16(np.ones(2))
    # hand example: x = (3, 4), k = 2, eps = 0: mean of squares 12.5, root
    # 3.5355339...; 3 / 3.5355339 = 0.8485281 lies 1737.79 f16 steps of 2^-11
    # above 0 -> 1738 * 2^-11 = 0.8486328125; 4 / 3.5355339 = 1.1313708 is
    # 1158.52 steps of 2^-10 -> 1159 * 2^-10 = 1.1318359375
    h, xn = orc.add_rmsnorm(f16(np.array([3.0, 4.0])), None, one, 0.0)
    assert np.array_equal(h, f16(np.array([3.0, 4.0])))
    assert np.array_equal(xn, f16(np.array([0.8486328125, 1.1318359375])))
    # the residual is f16(x + r), as numpy's correctly rounded f16 addition
    rng = np.random.default_rng(31)
    k = 256 if quick else 3072
    x = rng.normal(0, 1, k).astype(np.float16)
    r = rng.normal(0, 4, k).astype(np.float16)
    g = rng.uniform(0.5, 2.0, k).astype(np.float16)
    h, xn = orc.add_rmsnorm(x.view(np.uint16), r.view(np.uint16), g.view(np.uint16), 1e-5)
    assert np.array_equal(h, (x + r).view(np.uint16))
    # adding first is the same as normalising the stored residual
    h2, xn2 = orc.add_rmsnorm(h, None, g.view(np.uint16), 1e-5)
    assert np.array_equal(h2, h) and np.array_equal(xn2, xn)
    # constant input: each element is +-1 exactly (mean over k, not the sum)
    for c in (2.0, -0.375):
        _, xn = orc.add_rmsnorm(f16(np.full(k, c)), None, f16(np.ones(k)), 0.0)
        assert np.array_equal(xn, f16(np.full(k, math.copysign(1.0, c))))
        # eps = c^2 doubles the mean square: 1 / sqrt(2) -> 1448 * 2^-11
        _, xn = orc.add_rmsnorm(f16(np.full(k, c)), None, f16(np.ones(k)), c * c)
        assert np.array_equal(xn, f16(np.full(k, math.copysign(0.70703125, c))))
    # eps = 0: scaling x by 2 changes nothing; gamma scales the output exactly
    _, a = orc.add_rmsnorm(x.view(np.uint16), None, g.view(np.uint16), 0.0)
    _, b = orc.add_rmsnorm((x * np.float16(2)).view(np.uint16), None, g.view(np.uint16), 0.0)
    assert np.array_equal(a, b)
    _, c2 = orc.add_rmsnorm(x.view(np.uint16), None, (g * np.float16(2)).view(np.uint16), 0.0)
    av = a.view(np.float16).astype(np.float64)
    normal = np.abs(av) >= 2.0 ** -13
    assert np.array_equal(c2.view(np.float16).astype(np.float64)[normal], 2 * av[normal])
    # against the plain formula evaluated in numpy f64 (one rounding to f16)
    hv = (x + r).astype(np.float64)
    want = (hv * g.astype(np.float64) / np.sqrt(np.mean(hv * hv) + 1e-5)).astype(np.float16)
    _, xn = orc.add_rmsnorm(x.view(np.uint16), r.view(np.uint16), g.view(np.uint16), 1e-5)
    assert np.array_equal(xn, want.view(np.uint16))


def pin_rope(orc, quick=False):
    """RoPE: a hand example (which dims pair, which frequency), identity at
    position 0, norm preservation, the relative-position property of q.k, and
    which heads of the fused QKV output rotate."""
    base = 10000.0
    # head of 4 dims, position 1: pair (0, 2) turns by 1 rad, pair (1, 3) by
    # 10000^(-2/4) = 0.01 rad; a unit vector on dim 0 lands on (cos 1, sin 1)
    assert orc.rope_pair(1.0, 0.0, 0, 4, 1, base) == (math.cos(1.0), math.sin(1.0))
    oi, oj = orc.rope_pair(0.0, 1.0, 1, 4, 1, base)
    assert abs(oi + math.sin(0.01)) < 1e-15 and abs(oj - math.cos(0.01)) < 1e-15
    rng = np.random.default_rng(37)
    for _ in range(20):
        yi, yj = rng.normal(size=2)
        i, pos = int(rng.integers(0, 48)), int(rng.integers(0, 4096))
        assert orc.rope_pair(yi, yj, i, 96, 0, base) == (yi, yj)
        oi, oj = orc.rope_pair(yi, yj, i, 96, pos, base)
        assert abs((oi * oi + oj * oj) - (yi * yi + yj * yj)) <= 1e-12 * (yi * yi + yj * yj)

    def rot(v, pos):
        out = np.empty_like(v)
        for i in range(48):
            out[i], out[i + 48] = orc.rope_pair(v[i], v[i + 48], i, 96, pos, base)
        return out

    q, kk = rng.normal(size=96), rng.normal(size=96)
    for p1, p2, t in ((5, 3, 100), (0, 77, 1000), (2000, 1999, 17)):
        d0 = float(rot(q, p1) @ rot(kk, p2))
        d1 = float(rot(q, p1 + t) @ rot(kk, p2 + t))
        assert abs(d0 - d1) <= 1e-9 * (abs(d0) + 1.0)
    # fused QKV: 2 q heads, 1 k head, 1 v head of 8 dims; position 0 is the
    # plain matmul; elsewhere v is untouched and q, k are the rotated rows
    d, nq = 8, 2
    n, k = 4 * d, 64
    w, s = si.draw_weight(rng, n, k)
    x = si.draw_x(rng, k)
    y_plain, a_plain = orc.gemv(w, s, x)
    y0, a0 = orc.qkv_rope(w, s, x, d, nq, 0, base)
    assert np.array_equal(y0, y_plain) and np.array_equal(a0, a_plain)
    y5, _ = orc.qkv_rope(w, s, x, d, nq, 5, base)
    assert np.array_equal(y5[3 * d:], y_plain[3 * d:])
    for h in range(3):
        for i in range(d // 2):
            want = orc.rope_pair(y_plain[h * d + i], y_plain[h * d + i + d // 2], i, d, 5, base)
            assert (y5[h * d + i], y5[h * d + i + d // 2]) == want


def pin_rope_layout(orc, quick=False):
    """Rotary-pair layout: decoded in the opposite direction, logical row
    2p + u holds dim p % (d/2) + u d/2 of head p / (d/2)."""
    rng = np.random.default_rng(41)
    for n, k, d in ((96, 64, 96), (48, 3072, 8), (24, 96, 12)):
        w, s = si.draw_weight(rng, n, k)
        geo = orc.layout_geometry(n, k)
        dw, ds = decode_layout(orc.encode_rope(w, s, d), n, k, **geo)
        src = np.array([(r // 2 // (d // 2)) * d + (r // 2) % (d // 2) + (r % 2) * (d // 2)
                        for r in range(n)])
        assert np.array_equal(dw[:n, :k // 8], w[src]) and np.array_equal(ds[:n, :k // 32], s[src])


def _cache(rng, pages, nkv, d, scale=1.0):
    return si.f16_bits(rng.normal(0.0, scale, (pages, 2, nkv, 16, d)))


def pin_attention(orc, quick=False):
    """Paged-attention decode: one position returns its V row, equal scores
    return the mean of V, a dominant key selects its V row, the grouped-query
    head mapping, and the physical page order does not matter."""
    rng = np.random.default_rng(43)
    nq, nkv, d = 4, 2, 32
    pages = 4
    cache = _cache(rng, pages, nkv, d)
    q = si.f16_bits(rng.normal(0.0, 1.0, (nq, d)))
    table = np.array([2, 0, 3, 1], np.int32)
    V = lambda t, g: cache[table[t // 16], 1, g, t % 16].view(np.float16).astype(np.float64)
    # a single position: its V row, exactly
    out, _ = orc.attention_decode(q, cache, table, 1, nq, nkv, d, 0.125)
    for h in range(nq):
        assert np.array_equal(out[h], V(0, h // 2))
    # scale 0 (and equal keys): every weight 1/ctx -> the mean of V
    ctx = 37
    out, _ = orc.attention_decode(q, cache, table, ctx, nq, nkv, d, 0.0)
    for h in range(nq):
        want = np.mean([V(t, h // 2) for t in range(ctx)], axis=0)
        assert np.allclose(out[h], want, rtol=1e-12, atol=1e-12)
    eq = cache.copy()
    eq[:, 0] = eq[0, 0, 0, 0]         # every key the same row
    out, _ = orc.attention_decode(q, eq, table, ctx, nq, nkv, d, 0.3)
    for h in range(nq):
        want = np.mean([eq[table[t // 16], 1, h // 2, t % 16].view(np.float16).astype(np.float64)
                        for t in range(ctx)], axis=0)
        assert np.allclose(out[h], want, rtol=1e-12, atol=1e-12)
    # a dominant key: position 21 of kv head 1 matches query heads 2 and 3
    big = cache.copy()
    big[table[21 // 16], 0, 1, 21 % 16] = si.f16_bits(np.full(d, 4.0))
    qq = si.f16_bits(np.full((nq, d), 4.0))
    out, _ = orc.attention_decode(qq, big, table, ctx, nq, nkv, d, 1.0)
    for h in (2, 3):
        assert np.allclose(out[h], V(21, 1), rtol=0, atol=1e-12)
    # grouped heads: constant V per kv head -> each query head returns its group's value
    grp = cache.copy()
    for g in range(nkv):
        grp[:, 1, g] = si.f16_bits(np.full(d, g + 1.5))
    out, _ = orc.attention_decode(q, grp, table, ctx, nq, nkv, d, 0.2)
    for h in range(nq):
        assert np.allclose(out[h], h // 2 + 1.5, rtol=1e-14)
    # the physical page order does not matter
    perm = np.array([1, 3, 0, 2])
    moved = np.empty_like(cache)
    moved[perm] = cache
    a1, _ = orc.attention_decode(q, cache, table, ctx, nq, nkv, d, 0.17)
    a2, _ = orc.attention_decode(q, moved, perm[table].astype(np.int32), ctx, nq, nkv, d, 0.17)
    assert np.array_equal(a1, a2)


def pin_attention_softmax(orc, quick=False):
    """The softmax weighting and its temperature in closed form, and the
    magnitude sum a = sum_t p_t |V_t| that sizes every attention tolerance.

    One query head, q = 1 at dimension 0 and 0 elsewhere; key t holds c_t at
    dimension 0 and 0 elsewhere, so the raw score of position t is exactly
    c_t and the scaled one is scale * c_t (power-of-two scales: exact).  With
    position 0 at score 0 the weights are e^(scale c_t) / sum_u e^(scale c_u),
    which fixes the exponent base (e, not 2), that the score is scaled once by
    `scale` (no hidden 1/sqrt(d)), the normalisation, and, with V of mixed
    signs, a = sum_t p_t |V_t| (not the un-normalised sum, not |out|)."""
    nkv, nq = 1, 1
    for d in (32, 96):
        for scale, cs in ((0.5, (0.0, 2.0)), (0.125, (0.0, 2.0)), (0.25, (0.0, 3.0, -1.5))):
            ctx = len(cs)
            pages = 1
            cache = np.zeros((pages, 2, nkv, 16, d), np.uint16)
            q = np.zeros((nq, d), np.uint16)
            q[0, 0] = si.f16_bits([1.0])[0]
            vals = []
            for t, c in enumerate(cs):
                cache[0, 0, 0, t, 0] = si.f16_bits([c])[0]
                # V rows of both signs, element by element: +/- (t + 1) * 0.75, alternating
                v = np.array([(t + 1) * 0.75 * (1 if (i + t) % 2 == 0 else -1) for i in range(d)])
                cache[0, 1, 0, t] = si.f16_bits(v)
                vals.append(v)
            table = np.array([0], np.int32)
            out, a = orc.attention_decode(q, cache, table, ctx, nq, nkv, d, scale)
            w = np.array([math.exp(scale * c) for c in cs])
            p = w / w.sum()
            want = sum(p[t] * vals[t] for t in range(ctx))
            want_a = sum(p[t] * np.abs(vals[t]) for t in range(ctx))
            assert np.allclose(out[0], want, rtol=1e-13, atol=0), (d, scale, out[0][:4], want[:4])
            assert np.allclose(a[0], want_a, rtol=1e-13, atol=0), (d, scale, a[0][:4], want_a[:4])
            # the two-position form the weights reduce to: (V0 + e^D V1) / (1 + e^D)
            if ctx == 2:
                D = scale * cs[1]
                two = (vals[0] + math.exp(D) * vals[1]) / (1.0 + math.exp(D))
                assert np.allclose(out[0], two, rtol=1e-13, atol=0)


def load_geometry_golden():
    rows = []
    with open(os.path.join(GOLDEN, "layout_geometry.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(t) for t in line.split()])
    return rows


def pin_layout_geometry(orc, quick=False):
    for rows, k, L, CG, P, TR, tiles, tb in load_geometry_golden():
        got = orc.layout_geometry(rows, k)
        assert got == dict(L=L, CG=CG, P=P, TR=TR, tiles=tiles, tile_bytes=tb), \
            (rows, k, got)
        assert orc.layout_bytes(rows, k) == tiles * tb


def pin_layout_hand_example(orc, quick=False):
    """rows = 1, k = 32: one tile of 2304 bytes with L = 1, CG = 1.  Logical row r
    sits in lane r // 2, half r % 2; only (row 0, group 0) is real data."""
    words = np.array([[0x76543210, 0xFEDCBA98, 0x01234567, 0x89ABCDEF]], np.uint32)
    scales = np.array([[0x2A3B]], np.uint16)
    got = orc.encode_rows(words, scales)
    want = bytearray()
    for u in range(2):
        for lane in range(64):
            if (lane, u) == (0, 0):
                want += words[0].tobytes()
            else:
                want += b"\x88" * 16
    for lane in range(64):
        for u in range(2):
            want += scales[0].tobytes() if (lane, u) == (0, 0) else b"\x00\x00"
    assert got.tobytes() == bytes(want)


def decode_layout(buf: np.ndarray, rows: int, k: int, L, CG, P, TR, tiles, tile_bytes):
    """Walk the device buffer unit by unit (destination -> logical) and rebuild
    words, scales; also return the padding units seen."""
    G = k // 32
    words = np.zeros((tiles * TR, P * L * CG * 4), np.uint32)
    scales = np.zeros((tiles * TR, P * L * CG), np.uint16)
    for t in range(tiles):
        for p in range(P):
            base = t * tile_bytes + p * CG * 2304
            for lane in range(64):
                s, c = divmod(lane, L)
                for u in range(2):
                    r = t * TR + 2 * s + u
                    for j in range(CG):
                        g = p * L * CG + c * CG + j
                        off = base + (u * CG + j) * 1024 + lane * 16
                        words[r, 4 * g:4 * g + 4] = buf[off:off + 16].view(np.uint32)
                        soff = base + 2 * CG * 1024 + lane * 4 * CG + (u * CG + j) * 2
                        scales[r, g] = buf[soff:soff + 2].view(np.uint16)[0]
    return words, scales


def pin_layout_roundtrip(orc, quick=False):
    rng = np.random.default_rng(29)
    shapes = [(5, 96), (3, 8192 + 32 * 5), (130, 64)] if quick else \
             [(5, 96), (3, 8192 + 32 * 5), (130, 64), (9, 3072), (4, 16384 + 32 * 3), (33, 32 * 7)]
    for n, k in shapes:
        w, s = si.draw_weight(rng, n, k)
        geo = orc.layout_geometry(n, k)
        buf = orc.encode_rows(w, s)
        dw, ds = decode_layout(buf, n, k, **geo)
        G = k // 32
        assert np.array_equal(dw[:n, :k // 8], w) and np.array_equal(ds[:n, :G], s)
        assert np.all(dw[n:] == 0x88888888) and np.all(dw[:, k // 8:] == 0x88888888)
        assert np.all(ds[n:] == 0) and np.all(ds[:, G:] == 0)
    # gate/up: logical row 2i is gate i, 2i + 1 is up i
    n, k = 7, 96
    gw, gs = si.draw_weight(rng, n, k)
    uw, us = si.draw_weight(rng, n, k)
    buf = orc.encode_gate_up(gw, gs, uw, us)
    geo = orc.layout_geometry(2 * n, k)
    dw, ds = decode_layout(buf, 2 * n, k, **geo)
    assert np.array_equal(dw[0:2 * n:2, :k // 8], gw) and np.array_equal(dw[1:2 * n:2, :k // 8], uw)
    assert np.array_equal(ds[0:2 * n:2, :3], gs) and np.array_equal(ds[1:2 * n:2, :3], us)


def _stream_words3(codes) -> np.ndarray:
    """codes [n][k] in 0..7 -> canonical words3 [n][3k/32], through one Python
    integer per row holding sum_k codes[k] * 8^k (the stream read LSB first)."""
    codes = np.asarray(codes)
    n, k = codes.shape
    out = np.zeros((n, 3 * k // 32), np.uint32)
    for r in range(n):
        v = 0
        for kk in reversed(range(k)):
            v = v * 8 + int(codes[r, kk])
        for j in range(3 * k // 32):
            out[r, j] = (v >> (32 * j)) & 0xFFFFFFFF
    return out


def pin_int3(orc, quick=False):
    """int3 matmul: one-hot x reads back (q - 4) * s for every position (codes
    that cross a word boundary included), constant codes give closed forms,
    and the stream is read per row."""
    rng = np.random.default_rng(31)
    n, k = 3, 64
    codes = rng.integers(0, 8, size=(n, k))
    codes[:, 10] = 5      # stream bits 30..32: crosses from word 0 into word 1
    codes[:, 21] = 6      # bits 63..65: word 1 into word 2
    codes[:, 42] = 3      # bits 126..128, second group: word 3 into word 4
    words3 = _stream_words3(codes)
    scales = si.f16_bits(rng.uniform(0.25, 2.0, size=(n, k // 32)))
    sv = scales.view(np.float16).astype(np.float64)
    for kk in range(k):
        x = np.zeros(k, np.uint16)
        x[kk] = si.f16_bits(1.0)
        y, a = orc.gemv3(words3, scales, x)
        want = (codes[:, kk] - 4) * sv[:, kk // 32]
        assert np.array_equal(y, want), (kk, y, want)
        assert np.array_equal(a, np.abs(want))
    # constant codes: y = (c - 4) * sum over groups of s_g * (sum of x in g)
    x = si.draw_x(rng, k)
    xv = x.view(np.float16).astype(np.float64)
    gsum = xv.reshape(k // 32, 32).sum(axis=1)
    for c in (0, 4, 7):
        wc = _stream_words3(np.full((n, k), c))
        y, _ = orc.gemv3(wc, scales, x)
        want = (c - 4) * (sv * gsum).sum(axis=1)
        assert np.allclose(y, want, rtol=1e-13, atol=0), (c, y, want)
        if c == 4:
            assert np.all(y == 0.0)


def _decode3_device(buf: np.ndarray, n: int, k: int, g6):
    """Read an int3 device layout back into codes [n][k] and scales [n][k/32],
    and the padding slots' codes and scales, walking destinations."""
    L, CG, P, TR, T = g6["L"], g6["CG"], g6["P"], g6["TR"], g6["tiles"]
    PB = CG * 1792
    G = k // 32
    codes = np.full((n, k), -1)
    scales = np.zeros((n, G), np.uint16)
    pad_codes, pad_scales = set(), set()
    w32 = buf.view(np.uint32)
    for t in range(T):
        for p in range(P):
            base = (t * P + p) * PB
            for uj in range(2 * CG):
                u, j = divmod(uj, CG)
                for lane in range(64):
                    s_, c = divmod(lane, L)
                    r = t * TR + 2 * s_ + u
                    g = p * L * CG + c * CG + j
                    off = base + uj * 768 + lane * 12
                    w = [int(w32[off // 4 + i]) for i in range(3)]
                    grp = [0] * 32
                    for i in range(3):
                        for m in range(5):
                            grp[10 * i + m] = (w[i] >> (3 * m)) & 7
                            grp[10 * i + 5 + m] = (w[i] >> (16 + 3 * m)) & 7
                        grp[30] |= ((w[i] >> 15) & 1) << i
                        grp[31] |= ((w[i] >> 31) & 1) << i
                    so = base + 2 * CG * 768 + lane * 4 * CG + uj * 2
                    sc = int(buf[so]) | (int(buf[so + 1]) << 8)
                    if r < n and g < G:
                        codes[r, 32 * g:32 * g + 32] = grp
                        scales[r, g] = sc
                    else:
                        pad_codes.update(grp)
                        pad_scales.add(sc)
    return codes, scales, pad_codes, pad_scales


def pin_int3_layout(orc, quick=False):
    """The int3 device layout read back destination by destination: every
    (row, group) lands once with its 32 codes and scale; padding holds code 4
    (a zero weight) with scale 0; the size is tiles * P * CG * 1792 (one and
    two passes)."""
    rng = np.random.default_rng(37)
    shapes = [(5, 64), (3, 3072)] if quick else [(5, 64), (3, 3072), (70, 96), (2, 8192), (2, 8224),
                                                 (3, 16384)]
    for n, k in shapes:
        codes = rng.integers(0, 8, size=(n, k))
        words3 = _stream_words3(codes)
        scales = si.f16_bits(rng.uniform(0.005, 0.02, size=(n, k // 32)))
        buf = orc.encode3(words3, scales)
        g6 = orc.layout_geometry(n, k)
        assert buf.size == g6["tiles"] * g6["P"] * g6["CG"] * 1792
        dc, ds, pc, ps = _decode3_device(buf, n, k, g6)
        assert np.array_equal(dc, codes), (n, k)
        assert np.array_equal(ds, scales)
        assert pc <= {4} and ps <= {0}
    # gate/up: 2n logical rows, even rows the gate, odd rows the up matrix
    n, k = 5, 96
    gc, uc = rng.integers(0, 8, size=(n, k)), rng.integers(0, 8, size=(n, k))
    gs = si.f16_bits(rng.uniform(0.005, 0.02, size=(n, k // 32)))
    us = si.f16_bits(rng.uniform(0.005, 0.02, size=(n, k // 32)))
    buf = orc.encode3_gate_up(_stream_words3(gc), gs, _stream_words3(uc), us)
    g6 = orc.layout_geometry(2 * n, k)
    dc, ds, pc, ps = _decode3_device(buf, 2 * n, k, g6)
    assert np.array_equal(dc[0::2], gc) and np.array_equal(dc[1::2], uc)
    assert np.array_equal(ds[0::2], gs) and np.array_equal(ds[1::2], us)
    assert pc <= {4} and ps <= {0}


def pin_int3_gemm(orc, quick=False):
    """int3 GEMM: row r of Y is the int3 GEMV of row r of X, exactly."""
    rng = np.random.default_rng(59)
    m, n, k = 5, 7, 96
    w3, s3 = si.draw_weight3(rng, n, k)
    X = si.f16_bits(rng.normal(0, 1, (m, k)))
    Y, A = orc.gemm3(w3, s3, X)
    for r in range(m):
        y, a = orc.gemv3(w3, s3, X[r])
        assert np.array_equal(Y[r], y) and np.array_equal(A[r], a), r


def pin_int3_ffn(orc, quick=False):
    """int3 FFN: the gate (not the up) is the gated half; constant codes give
    h = silu(cg * S) * cu * S in closed form."""
    rng = np.random.default_rng(53)
    n, k = 3, 64
    x = si.draw_x(rng, k)
    xv = x.view(np.float16).astype(np.float64)
    s = si.f16_bits(np.full((n, k // 32), 0.0625))
    S = 0.0625 * xv.sum()
    for cg, cu in ((7, 5), (1, 6), (4, 7)):
        gw, uw = _stream_words3(np.full((n, k), cg)), _stream_words3(np.full((n, k), cu))
        r = orc.ffn_gate_up_silu3(gw, s, uw, s, x)
        gv, uv = (cg - 4) * S, (cu - 4) * S
        want = gv / (1.0 + math.exp(-gv)) * uv
        assert np.allclose(r["h"], want, rtol=1e-12, atol=1e-15), (cg, cu, r["h"], want)
        assert np.allclose(r["g"], gv, rtol=1e-13) and np.allclose(r["u"], uv, rtol=1e-13)


def pin_kv_quant(orc, quick=False):
    """int8 KV rows: a hand example away from rounding ties, |q| <= 127 with
    the largest element at +-127, the reconstruction within half a step,
    power-of-two scaling of the row, and the zero row."""
    q, sc = orc.kv_quant_row(si.f16_bits([2.0, -1.5, 0.25, 0.0]))
    # scale = 2/127; x / scale = 127, -95.25, 15.875, 0
    assert np.array_equal(q, np.array([127, -95, 16, 0], np.int8)), q
    assert sc == np.float32(2.0) / np.float32(127.0)
    rng = np.random.default_rng(41)
    for d in (32, 96, 256):
        x = si.f16_bits(rng.normal(0, 1.5, d))
        q, sc = orc.kv_quant_row(x)
        xv = x.view(np.float16).astype(np.float64)
        assert np.abs(q.astype(np.int64)).max() == 127
        assert np.abs(q[np.argmax(np.abs(xv))]) == 127
        assert np.all(np.abs(q.astype(np.float64) * float(sc) - xv) <= float(sc) * (0.5 + 1e-6))
        q2, sc2 = orc.kv_quant_row(si.f16_bits(xv * 4.0))
        assert np.array_equal(q2, q) and sc2 == np.float32(sc) * np.float32(4.0)
    q, sc = orc.kv_quant_row(np.zeros(64, np.uint16))
    assert sc == 0 and np.all(q == 0)
    # the row maximum at every index, the first and the last included: the
    # element of largest magnitude (3 or -3, every other |x| < 1) becomes
    # +-127 and fixes the scale 3/127 (f32)
    for d in ((32, 96) if quick else (32, 96, 256)):
        base = rng.uniform(-0.99, 0.99, d)
        for j in range(d):
            for sign in (1.0, -1.0):
                xv = base.copy()
                xv[j] = 3.0 * sign
                q, sc = orc.kv_quant_row(si.f16_bits(xv))
                assert sc == np.float32(3.0) / np.float32(127.0), (d, j, sc)
                assert int(q[j]) == int(127 * sign), (d, j, q[j])
                assert np.abs(q.astype(np.int64)).max() == 127


def _kv8_block(orc, nkv, d, page, kv, g):
    """byte offset of the (page, K|V, kv head) block of an int8 cache"""
    return page * 2 * nkv * (16 * d + 64) + (kv * nkv + g) * (16 * d + 64)


def pin_kv_append_int8(orc, quick=False):
    """The int8 append writes each k / v head's quantised row into its block's
    slot and its scale into the block's scale array, nothing else; an absent
    page writes nothing."""
    rng = np.random.default_rng(43)
    nq, nkv, d = 4, 2, 32
    pages = 3
    pb = orc.kv8_page_bytes(nkv, d)
    assert pb == 2 * nkv * (16 * d + 64)
    table = np.array([2, 0], np.int32)
    qkv = si.f16_bits(rng.normal(0, 1, (nq + 2 * nkv) * d))
    for pos in (0, 5, 21):
        cache = np.full((pages, pb), 0xA5, np.uint8)
        orc.kv_append_int8(qkv, nq, nkv, d, pos, cache, table)
        flat = cache.reshape(-1)
        want = np.full(flat.size, 0xA5, np.uint8)
        for kv in (0, 1):
            for g in range(nkv):
                row = qkv[(nq + kv * nkv + g) * d:(nq + kv * nkv + g + 1) * d]
                q, sc = orc.kv_quant_row(row)
                o = _kv8_block(orc, nkv, d, table[pos // 16], kv, g)
                want[o + (pos % 16) * d:o + (pos % 16 + 1) * d] = q.view(np.uint8)
                so = o + 16 * d + 4 * (pos % 16)
                want[so:so + 4] = np.array([sc], np.float32).view(np.uint8)
        assert np.array_equal(flat, want), pos
    cache = np.full((pages, pb), 0xA5, np.uint8)
    orc.kv_append_int8(qkv, nq, nkv, d, 3, cache, np.array([7], np.int32))
    assert np.all(cache == 0xA5)


def pin_attention_int8(orc, quick=False):
    """Attention over an int8 cache equals the (pinned) f16 attention over the
    cache of its dequantised values, bit for bit, when those values are exact
    in f16 (power-of-two scales): pins the block layout, the slot, the scale
    placement and K vs V."""
    rng = np.random.default_rng(47)
    nq, nkv, d = 4, 2, 64
    ctx = 45
    pages = 4
    table = np.array([3, 1, 0], np.int32)
    pb = orc.kv8_page_bytes(nkv, d)
    cache8 = np.zeros((pages, pb), np.uint8)
    cache16 = np.zeros((pages, 2, nkv, 16, d), np.uint16)
    for p in range(pages):
        for kv in (0, 1):
            for g in range(nkv):
                codes = rng.integers(-127, 128, (16, d)).astype(np.int8)
                scales = (2.0 ** -rng.integers(5, 9, 16)).astype(np.float32)
                o = _kv8_block(orc, nkv, d, p, kv, g) - p * pb
                cache8[p, o:o + 16 * d] = codes.view(np.uint8).reshape(-1)
                cache8[p, o + 16 * d:o + 16 * d + 64] = scales.view(np.uint8)
                cache16[p, kv, g] = si.f16_bits(codes.astype(np.float64) * scales[:, None])
    q = si.f16_bits(rng.normal(0, 1, (nq, d)))
    out8, a8 = orc.attention_decode_int8(q, cache8, table, ctx, nq, nkv, d, 0.11)
    out16, a16 = orc.attention_decode(q, cache16, table, ctx, nq, nkv, d, 0.11)
    assert np.array_equal(out8, out16) and np.array_equal(a8, a16)


ALL_PINS = [
    pin_half_decode_all_patterns, pin_half_encode_rne,
    pin_gemv_rational, pin_gemv_exactly_representable, pin_gemv_closed_forms,
    pin_gemv_one_hot, pin_gemv_linearity, pin_gemm_rows,
    pin_silu, pin_ffn, pin_argmax, pin_lmhead, pin_add_rmsnorm, pin_rope, pin_attention,
    pin_attention_softmax, pin_layout_geometry, pin_layout_hand_example, pin_layout_roundtrip, pin_rope_layout,
    pin_int3, pin_int3_layout, pin_int3_gemm, pin_int3_ffn, pin_kv_quant, pin_kv_append_int8, pin_attention_int8,
]

"""q4_gemv on the GPU against the oracle: random parity at the decode shapes
and at ragged/edge shapes, bit-exact pins where the exact result is
representable, determinism and sign symmetry."""
import numpy as np
import pytest

import seeded_inputs as si
from parity import (assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16,
                    tol_f16)

pytestmark = pytest.mark.gpu


def run_gemv(q4, w, s, x):
    pw = q4.pack(dev_u32(w), dev_u16(s))
    return q4.gemv(pw, dev_f16(x)), pw


def test_gemv_3072_parity(q4, orc):
    inp = si.workload(si.GEMV_3072, seed=0)
    y, _ = run_gemv(q4, inp["words"], inp["scales"], inp["x"])
    ref, a = orc.gemv(inp["words"], inp["scales"], inp["x"])
    ratio = assert_within(host_f16_as_f64(y), ref, tol_f16(ref, a), "gemv 3072x3072")
    print(f"max err/tol {ratio:.3g}")


@pytest.mark.parametrize("key", list(si.LAYER_SHAPES))
def test_layer_set_parity(q4, orc, key):
    inp = si.workload(si.LAYER_SET, seed=0)
    w, s = inp[key]
    x = inp["x8192"] if key == "down" else inp["x3072"]
    y, _ = run_gemv(q4, w, s, x)
    ref, a = orc.gemv(w, s, x)
    ratio = assert_within(host_f16_as_f64(y), ref, tol_f16(ref, a), key)
    print(f"{key}: max err/tol {ratio:.3g}")


# includes the long-k split kernel with several tiles per block and an odd
# last tile (3001 x 8192) and with padded groups (777 x 7168: 224 of 256
# group slots real)
RAGGED = [(1, 32), (2, 32), (17, 96), (130, 64), (33, 224), (7, 160), (6, 192), (1, 768),
          (3, 3200), (5, 16384), (3, 8352), (4, 16480), (1001, 3072), (9, 8192), (64, 4096),
          (3, 3072), (3001, 8192), (777, 7168)]


@pytest.mark.parametrize("n,k", RAGGED)
def test_gemv_ragged_shapes(q4, orc, n, k):
    rng = np.random.default_rng(1000 + n * 31 + k)
    x = si.draw_x(rng, k)
    w, s = si.draw_weight(rng, n, k)
    y, _ = run_gemv(q4, w, s, x)
    ref, a = orc.gemv(w, s, x)
    assert_within(host_f16_as_f64(y), ref, tol_f16(ref, a), f"gemv {n}x{k}")


@pytest.mark.parametrize("n,k", [(3072, 3072), (3072, 8192), (37, 16480)])
def test_gemv_one_hot_bit_exact(q4, orc, n, k):
    """x = e_k: y_n = (q - 8) * s exactly in f32; the f16 output must be its
    round-to-nearest-even, bit for bit (pins row stride, group, nibble)."""
    rng = np.random.default_rng(3)
    w, s = si.draw_weight(rng, n, k)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    for kk in [0, 1, 4, 7, 8, 31, 32, 33, 100, k // 2 + 5, k - 33, k - 1]:
        x = np.zeros(k, np.uint16)
        x[kk] = 0x3C00
        y = host_u16(q4.gemv(pw, dev_f16(x)))
        ref, _ = orc.gemv(w, s, x)
        want = orc.doubles_to_halves(ref)
        bad = np.nonzero(y != want)[0]
        assert bad.size == 0, f"k={kk}: rows {bad[:5].tolist()} got {y[bad[:5]]} want {want[bad[:5]]}"


def test_gemv_closed_forms_bit_exact(q4):
    k = 3072
    x = si.f16_bits(np.ones(k))
    # every code 15, scale 2^-6: y = 7 * 2^-6 * 3072 = 336 in every row
    w = si.pack_codes(np.full((130, k), 15, np.uint8))
    s = si.f16_bits(np.full((130, k // 32), 2.0 ** -6))
    y, _ = run_gemv(q4, w, s, x)
    assert np.all(host_u16(y) == si.f16_bits(336.0))
    # code 8 means weight 0: y must be +0 exactly, whatever x is
    rng = np.random.default_rng(8)
    w8 = si.pack_codes(np.full((64, k), 8, np.uint8))
    s8 = si.f16_bits(rng.uniform(0.005, 0.02, (64, k // 32)))
    y, _ = run_gemv(q4, w8, s8, si.draw_x(rng, k))
    assert np.all(host_u16(y) == 0)


@pytest.mark.parametrize("n,k", [(3072, 3072), (3072, 8192), (16384, 3072), (101, 16480)])
def test_gemv_exactly_representable_bit_exact(q4, orc, n, k):
    """x in {-4..4}/4, scales in {2^-7, 2^-8}: every product and partial sum is
    exact in f32 in any order, so y must be the RNE of the exact sum."""
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    w = si.pack_codes(codes)
    s = si.f16_bits(2.0 ** -rng.integers(7, 9, (n, k // 32)))
    x = si.f16_bits(rng.integers(-4, 5, k) / 4.0)
    y, _ = run_gemv(q4, w, s, x)
    ref, _ = orc.gemv(w, s, x)
    want = orc.doubles_to_halves(ref)
    got = host_u16(y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5].tolist()}"


def test_gemv_deterministic(q4):
    """Run-to-run bitwise identical (fixed reduction order, no atomics)."""
    inp = si.workload(si.GEMV_3072, seed=4)
    pw = q4.pack(dev_u32(inp["words"]), dev_u16(inp["scales"]))
    x = dev_f16(inp["x"])
    ys = [host_u16(q4.gemv(pw, x)) for _ in range(3)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])

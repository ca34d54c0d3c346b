"""q4_gemm / q4_gemm_path on the GPU against the oracle: the VALU kernel
(forced, or m = 1 with Y 2-byte aligned; exact dequant) and the MFMA kernels
(m >= 2, f16 dequant), full
checks at moderate sizes and sampled checks at the full prefill shape."""
import numpy as np
import pytest

import seeded_inputs as si
from parity import assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16, tol_f16

pytestmark = pytest.mark.gpu

PATHS = {"auto": 0, "valu": 1, "mfma": 2}


def run(q4, w, s, X, path=0):
    pw = q4.pack(dev_u32(w), dev_u16(s))
    return q4.gemm(pw, dev_f16(X), path=path), pw


@pytest.mark.parametrize("m", [1, 2, 5, 8, 9, 15, 16, 17, 31, 33, 64, 65, 97, 128, 129])
def test_gemm_parity_auto(q4, orc, m):
    rng = np.random.default_rng(100 + m)
    n, k = 1000, 3072
    w, s = si.draw_weight(rng, n, k)
    X = si.draw_X(rng, m, k)
    Y, _ = run(q4, w, s, X)
    ref, a = orc.gemm(w, s, X)
    assert_within(host_f16_as_f64(Y), ref, tol_f16(ref, a), f"gemm m={m}")


@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("m", [1, 3, 16, 24, 40])
def test_gemm_forced_paths(q4, orc, path, m):
    rng = np.random.default_rng(7 * m + len(path))
    n, k = 777, 8192
    w, s = si.draw_weight(rng, n, k)
    X = si.draw_X(rng, m, k)
    Y, _ = run(q4, w, s, X, PATHS[path])
    ref, a = orc.gemm(w, s, X)
    assert_within(host_f16_as_f64(Y), ref, tol_f16(ref, a), f"gemm {path} m={m}")


@pytest.mark.parametrize("n,k", [(33, 96), (130, 224), (9, 3200), (70, 8352), (5, 16480), (64, 256)])
@pytest.mark.parametrize("m", [1, 6, 16, 20])
def test_gemm_ragged_shapes(q4, orc, n, k, m):
    rng = np.random.default_rng(n * k + m)
    w, s = si.draw_weight(rng, n, k)
    X = si.draw_X(rng, m, k)
    for path in (0, 2):
        Y, _ = run(q4, w, s, X, path)
        ref, a = orc.gemm(w, s, X)
        assert_within(host_f16_as_f64(Y), ref, tol_f16(ref, a), f"gemm {n}x{k} m={m} path={path}")


@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("m", [3, 16, 64])
def test_gemm_exactly_representable_bit_exact(q4, orc, path, m):
    """x in {-4..4}/4, scales in {2^-7, 2^-8}: products and every partial sum
    are exact in f32 (and (q - 8) * s is exact in f16), so both kernels must
    give the round-to-nearest-even of the exact result."""
    rng = np.random.default_rng(m)
    n, k = 512, 3072
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    w = si.pack_codes(codes)
    s = si.f16_bits(2.0 ** -rng.integers(7, 9, (n, k // 32)))
    X = si.f16_bits(rng.integers(-4, 5, (m, k)) / 4.0)
    Y, _ = run(q4, w, s, X, PATHS[path])
    ref, _ = orc.gemm(w, s, X)
    want = orc.doubles_to_halves(ref.ravel()).reshape(ref.shape)
    got = host_u16(Y)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} entries differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_gemm_one_hot_rows(q4, orc, path):
    """row i of X is e_{k_i}: Y[i][r] = (q[r][k_i] - 8) * s exactly (one f16
    rounding); pins the k order and the output layout of both kernels."""
    rng = np.random.default_rng(21)
    n, k = 300, 3072
    w, s = si.draw_weight(rng, n, k)
    ks = [0, 1, 4, 7, 8, 31, 32, 255, 256, 1000, 2047, 3071, 100, 5, 6, 3, 2, 1536]
    X = np.zeros((len(ks), k), np.uint16)
    for i, kk in enumerate(ks):
        X[i, kk] = 0x3C00
    Y, _ = run(q4, w, s, X, PATHS[path])
    ref, _ = orc.gemm(w, s, X)
    want = orc.doubles_to_halves(ref.ravel()).reshape(ref.shape)
    assert np.array_equal(host_u16(Y), want)


@pytest.mark.parametrize("m", [16, 24, 64, 100, 128, 256])
def test_gemm_prefill_full_shape_sampled(q4, orc, m):
    """The full prefill shape (W 16384 x 3072): every output computed on the
    GPU, 96 weight rows x all m rows checked against the oracle."""
    inp = si.workload(si.GEMM, seed=0, m=m)
    w, s, X = inp["words"], inp["scales"], inp["X"]
    Y, _ = run(q4, w, s, X)
    Yh = host_f16_as_f64(Y)
    rows = np.sort(np.random.default_rng(m).choice(16384, 96, replace=False))
    ref, a = orc.gemm(np.ascontiguousarray(w[rows]), np.ascontiguousarray(s[rows]), X)
    assert_within(Yh[:, rows], ref, tol_f16(ref, a), f"prefill m={m}")
    assert np.all(np.isfinite(Yh))


def test_gemm_mfma_matches_valu_within_tolerance(q4, orc):
    """the two kernels on the same inputs both sit within the bound of the
    oracle, and differ from each other by less than twice that bound"""
    rng = np.random.default_rng(5)
    n, k, m = 640, 3072, 24
    w, s = si.draw_weight(rng, n, k)
    X = si.draw_X(rng, m, k)
    Yv, pw = run(q4, w, s, X, 1)
    Ym = q4.gemm(pw, dev_f16(X), path=2)
    ref, a = orc.gemm(w, s, X)
    t = tol_f16(ref, a)
    assert_within(host_f16_as_f64(Yv), ref, t, "valu")
    assert_within(host_f16_as_f64(Ym), ref, t, "mfma")
    assert_within(host_f16_as_f64(Ym), host_f16_as_f64(Yv), 2 * t, "mfma vs valu")


@pytest.mark.parametrize("int3", [False, True])
def test_gemm_one_row_is_the_gemv(q4, orc, int3):
    """m = 1 on the default path runs the GEMV kernels: the output equals
    q4_gemv's bit for bit and sits within the oracle's bound.  With Y only
    2-byte aligned it takes the VALU GEMM kernel instead, also within the
    bound."""
    import torch
    rng = np.random.default_rng(77 + int3)
    n, k = 1001, 3072
    if int3:
        w, s = si.draw_weight3(rng, n, k)
        pw = q4.pack_int3(dev_u32(w), dev_u16(s))
        ref, a = orc.gemm3(w, s, si.draw_X(np.random.default_rng(5), 1, k))
    else:
        w, s = si.draw_weight(rng, n, k)
        pw = q4.pack(dev_u32(w), dev_u16(s))
        ref, a = orc.gemm(w, s, si.draw_X(np.random.default_rng(5), 1, k))
    X = si.draw_X(np.random.default_rng(5), 1, k)
    Y = q4.gemm(pw, dev_f16(X))
    y = q4.gemv(pw, dev_f16(X[0]))
    assert np.array_equal(host_u16(Y).reshape(-1), host_u16(y))
    assert_within(host_f16_as_f64(Y), ref, tol_f16(ref, a), "gemm m=1 (gemv kernels)")
    buf = torch.empty(n + 1, dtype=torch.float16, device="cuda")
    Ym = buf[1:].view(1, n)
    q4.gemm(pw, dev_f16(X), out=Ym)
    assert_within(host_f16_as_f64(Ym), ref, tol_f16(ref, a), "gemm m=1, Y 2-byte aligned (VALU kernel)")


@pytest.mark.parametrize("n,k", [(777, 8192), (130, 224), (70, 1568), (64, 512), (1000, 4096)])
@pytest.mark.parametrize("m", [33, 64, 65, 100, 128, 129, 200])
def test_gemm_k_split_tiles(q4, orc, n, k, m):
    """the K-split MFMA kernel's tiles (64 weight rows for m <= 64, 128 above;
    32 / 64 / 128 activation rows) and the k > 4096 fallbacks (64-row tiles
    up to m = 128, the weight-direct kernel above), on layouts from L = 8 to
    64 (steps that run past a row's pairs, several M blocks, ragged n)"""
    rng = np.random.default_rng(n + 3 * k + 7 * m)
    w, s = si.draw_weight(rng, n, k)
    X = si.draw_X(rng, m, k)
    Y, _ = run(q4, w, s, X)
    ref, a = orc.gemm(w, s, X)
    assert_within(host_f16_as_f64(Y), ref, tol_f16(ref, a), f"gemm {n}x{k} m={m}")


@pytest.mark.parametrize("m", [5, 64, 200])
def test_gemm_repeat_bit_identical(q4, orc, m):
    """the K-split kernel adds its wavefronts' partial tiles in a fixed order:
    three calls on the same inputs give the same bits (and sit within the
    oracle's bound)"""
    rng = np.random.default_rng(900 + m)
    n, k = 700, 3072
    w, s = si.draw_weight(rng, n, k)
    X = si.draw_X(rng, m, k)
    Y0, pw = run(q4, w, s, X)
    Xd = dev_f16(X)
    for _ in range(2):
        assert np.array_equal(host_u16(q4.gemm(pw, Xd)), host_u16(Y0))
    ref, a = orc.gemm(w, s, X)
    assert_within(host_f16_as_f64(Y0), ref, tol_f16(ref, a), f"gemm m={m}")

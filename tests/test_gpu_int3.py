"""The int3 variant of the matmul on the GPU against the oracle: the packed
layouts (plain and gate/up) byte for byte, the unpack round trip, GEMV parity
at the decode shapes and at ragged/edge shapes (f16 output bound as for
int4), bit-exact one-hot reads (codes that cross a word boundary included),
exactly representable sums, closed forms and determinism, at one and at
several passes (k > 8192); the fused FFN and the f32 LM head with argmax over
int3 weights; the int3 GEMM on the VALU and
MFMA paths (full parity, forced paths, ragged shapes, bit-exact cases, and
sampled rows at the full prefill shape)."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import (argmax_ok, assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16,
                    tol_f16, tol_f32, tol_ffn)

pytestmark = pytest.mark.gpu


def stream_words3(codes) -> np.ndarray:
    """codes [n][k] in 0..7 -> canonical words3 [n][3k/32] (code k at stream
    bits 3k .. 3k+2, LSB first), bit by bit."""
    codes = np.asarray(codes, dtype=np.uint64)
    n, k = codes.shape
    bits = np.zeros((n, 3 * k), np.uint64)
    for t in range(3):
        bits[:, t::3] = (codes >> np.uint64(t)) & np.uint64(1)
    bits = bits.reshape(n, 3 * k // 32, 32)
    return (bits << np.arange(32, dtype=np.uint64)).sum(axis=2).astype(np.uint32)


def run(q4, w3, s, x):
    pw = q4.pack_int3(dev_u32(w3), dev_u16(s))
    return q4.gemv(pw, dev_f16(x)), pw


@pytest.mark.parametrize("n,k", [(3072, 3072), (1, 32), (17, 96), (130, 64), (33, 224),
                                 (999, 544), (5, 8192), (70, 7168), (64, 8224), (3, 16384),
                                 (130, 24608)])
def test_pack_int3_byte_exact_and_roundtrip(q4, orc, n, k):
    rng = np.random.default_rng(n * 7 + k)
    w3, s = si.draw_weight3(rng, n, k)
    pw = q4.pack_int3(dev_u32(w3), dev_u16(s))
    assert pw.layout == q4.LAYOUT_INT3
    assert np.array_equal(pw.buf.cpu().numpy(), orc.encode3(w3, s))
    uw, us = q4.unpack(pw)
    assert np.array_equal(uw.cpu().numpy().view(np.uint32), w3)
    assert np.array_equal(us.cpu().numpy().view(np.uint16), s)


@pytest.mark.parametrize("n,k", [(3072, 3072), (9216, 3072), (16384, 3072), (3072, 8192)])
def test_gemv_int3_decode_shapes(q4, orc, n, k):
    rng = np.random.default_rng(n + 3 * k)
    w3, s = si.draw_weight3(rng, n, k)
    x = si.draw_x(rng, k)
    y, _ = run(q4, w3, s, x)
    ref, a = orc.gemv3(w3, s, x)
    ratio = assert_within(host_f16_as_f64(y), ref, tol_f16(ref, a), f"int3 gemv {n}x{k}")
    print(f"{n}x{k}: max err/tol {ratio:.3g}")


RAGGED = [(1, 32), (2, 32), (17, 96), (130, 64), (33, 224), (7, 160), (6, 192), (1, 768),
          (1001, 3072), (9, 8192), (64, 4096), (3001, 8192), (777, 7168), (3, 3200),
          (3072, 16384), (130, 8224), (17, 24608), (1, 16384), (999, 8448)]


@pytest.mark.parametrize("n,k", RAGGED)
def test_gemv_int3_ragged(q4, orc, n, k):
    rng = np.random.default_rng(5000 + n * 31 + k)
    w3, s = si.draw_weight3(rng, n, k)
    x = si.draw_x(rng, k)
    y, _ = run(q4, w3, s, x)
    ref, a = orc.gemv3(w3, s, x)
    assert_within(host_f16_as_f64(y), ref, tol_f16(ref, a), f"int3 gemv {n}x{k}")


@pytest.mark.parametrize("n,k", [(3072, 3072), (130, 8192), (130, 16384)])
def test_gemv_int3_one_hot_bit_exact(q4, orc, n, k):
    """x = e_k: y_n = (q - 4) * s exactly; the f16 output is its RNE, bit for
    bit, at positions that cover every code slot of the device words (10 and
    21 cross canonical word boundaries; 30 and 31 are the bit-sliced codes)."""
    rng = np.random.default_rng(17)
    w3, s = si.draw_weight3(rng, n, k)
    pw = q4.pack_int3(dev_u32(w3), dev_u16(s))
    for kk in list(range(32)) + [32 + 10, 32 + 21, 32 + 30, k // 2 + 7, k - 33, k - 2, k - 1]:
        x = np.zeros(k, np.uint16)
        x[kk] = 0x3C00
        got = host_u16(q4.gemv(pw, dev_f16(x)))
        ref, _ = orc.gemv3(w3, s, x)
        want = orc.doubles_to_halves(ref)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"k={kk}: rows {bad[:5].tolist()} got {got[bad[:5]]} want {want[bad[:5]]}"


@pytest.mark.parametrize("n,k", [(3072, 3072), (9216, 3072), (101, 8192), (101, 16384)])
def test_gemv_int3_exactly_representable(q4, orc, n, k):
    """x in {-4..4}/4, scales in {2^-7, 2^-8}: exact in f32 in any order, so y
    is the RNE of the exact sum."""
    rng = np.random.default_rng(n + k + 1)
    codes = rng.integers(0, 8, (n, k))
    w3 = stream_words3(codes)
    s = si.f16_bits(2.0 ** -rng.integers(7, 9, (n, k // 32)))
    x = si.f16_bits(rng.integers(-4, 5, k) / 4.0)
    y, _ = run(q4, w3, s, x)
    ref, _ = orc.gemv3(w3, s, x)
    want = orc.doubles_to_halves(ref)
    bad = np.nonzero(host_u16(y) != want)[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5].tolist()}"


def test_gemv_int3_closed_forms(q4):
    k = 3072
    x = si.f16_bits(np.ones(k))
    # every code 7, scale 2^-6: y = 3 * 2^-6 * 3072 = 144 in every row
    w = stream_words3(np.full((130, k), 7))
    s = si.f16_bits(np.full((130, k // 32), 2.0 ** -6))
    y, _ = run(q4, w, s, x)
    assert np.all(host_u16(y) == si.f16_bits(144.0))
    # every code 0: y = -4 * 2^-6 * 3072 = -192
    y, _ = run(q4, stream_words3(np.zeros((130, k), np.int64)), s, x)
    assert np.all(host_u16(y) == si.f16_bits(-192.0))
    # code 4 is the zero weight: y = +0 whatever x is
    rng = np.random.default_rng(4)
    s4 = si.f16_bits(rng.uniform(0.005, 0.02, (64, k // 32)))
    y, _ = run(q4, stream_words3(np.full((64, k), 4)), s4, si.draw_x(rng, k))
    assert np.all(host_u16(y) == 0)


def test_gemv_int3_deterministic(q4):
    rng = np.random.default_rng(9)
    w3, s = si.draw_weight3(rng, 9216, 3072)
    pw = q4.pack_int3(dev_u32(w3), dev_u16(s))
    x = dev_f16(si.draw_x(rng, 3072))
    outs = [host_u16(q4.gemv(pw, x)) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("n,k", [(8192, 3072), (64, 3072), (17, 96), (130, 64), (999, 544),
                                 (40, 8192), (40, 8224), (256, 16384)])
def test_pack_int3_gate_up_and_ffn(q4, orc, n, k):
    rng = np.random.default_rng(7 * n + k)
    gw, gs = si.draw_weight3(rng, n, k)
    uw, us = si.draw_weight3(rng, n, k)
    x = si.draw_x(rng, k)
    pw = q4.pack_int3_gate_up(dev_u32(gw), dev_u16(gs), dev_u32(uw), dev_u16(us))
    assert pw.layout == q4.LAYOUT_INT3_GATE_UP
    if n * k <= 3072 * 1024:
        assert np.array_equal(pw.buf.cpu().numpy(), orc.encode3_gate_up(gw, gs, uw, us))
        ww, ss = q4.unpack(pw)
        ww, ss = ww.cpu().numpy().view(np.uint32), ss.cpu().numpy().view(np.uint16)
        assert np.array_equal(ww[0::2], gw) and np.array_equal(ww[1::2], uw)
        assert np.array_equal(ss[0::2], gs) and np.array_equal(ss[1::2], us)
    h = q4.ffn_gate_up_silu(pw, dev_f16(x))
    ref = orc.ffn_gate_up_silu3(gw, gs, uw, us, x)
    r = assert_within(host_f16_as_f64(h), ref["h"], tol_ffn(ref), f"int3 ffn {n}x{k}")
    print(f"max err/tol {r:.3g}")


@pytest.mark.parametrize("n,k", [(32064, 3072), (1001, 3072), (7, 160), (1001, 8192), (3, 8192),
                                 (1001, 16384), (5, 8224)])
def test_lmhead_int3(q4, orc, n, k):
    rng = np.random.default_rng(11 * n + k)
    w3, s3 = si.draw_weight3(rng, n, k)
    x = si.draw_x(rng, k)
    pw = q4.pack_int3(dev_u32(w3), dev_u16(s3))
    for _ in range(2):   # the workspace is reused
        logits, idx = q4.lmhead_f32(pw, dev_f16(x))
    ref, a = orc.gemv3(w3, s3, x)
    got = logits.cpu().numpy().astype(np.float64)
    assert_within(got, ref, tol_f32(a), f"int3 lm head {n}x{k}")
    assert argmax_ok(int(idx.item()), ref, a, orc.argmax(ref))
    assert int(idx.item()) == int(np.argmax(got))



GEMM_PATHS = {"auto": 0, "valu": 1, "mfma": 2}


def run_gemm3(q4, w3, s, X, path=0):
    pw = q4.pack_int3(dev_u32(w3), dev_u16(s))
    return q4.gemm(pw, dev_f16(X), path=path), pw


@pytest.mark.parametrize("m", [1, 2, 5, 8, 9, 15, 16, 17, 31, 33, 64, 65, 97, 128, 129])
def test_gemm_int3_parity_auto(q4, orc, m):
    rng = np.random.default_rng(300 + m)
    n, k = 1001, 3072
    w3, s = si.draw_weight3(rng, n, k)
    X = si.draw_X(rng, m, k)
    Y, _ = run_gemm3(q4, w3, s, X)
    ref, a = orc.gemm3(w3, s, X)
    assert_within(host_f16_as_f64(Y), ref, tol_f16(ref, a), f"int3 gemm m={m}")


@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("m", [1, 3, 16, 24, 40])
def test_gemm_int3_forced_paths(q4, orc, path, m):
    rng = np.random.default_rng(11 * m + len(path))
    n, k = 777, 8192
    w3, s = si.draw_weight3(rng, n, k)
    X = si.draw_X(rng, m, k)
    Y, _ = run_gemm3(q4, w3, s, X, GEMM_PATHS[path])
    ref, a = orc.gemm3(w3, s, X)
    assert_within(host_f16_as_f64(Y), ref, tol_f16(ref, a), f"int3 gemm {path} m={m}")


@pytest.mark.parametrize("n,k", [(33, 96), (130, 224), (9, 3200), (70, 8160), (1, 32), (64, 256),
                                 (70, 8224), (33, 16384)])
@pytest.mark.parametrize("m", [1, 6, 16, 20])
def test_gemm_int3_ragged_shapes(q4, orc, n, k, m):
    rng = np.random.default_rng(7 * n * k + m)
    w3, s = si.draw_weight3(rng, n, k)
    X = si.draw_X(rng, m, k)
    ref, a = orc.gemm3(w3, s, X)
    for path in (0, 1, 2):
        Y, _ = run_gemm3(q4, w3, s, X, path)
        assert_within(host_f16_as_f64(Y), ref, tol_f16(ref, a), f"int3 gemm {n}x{k} m={m} path={path}")


@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("m", [3, 16, 64])
def test_gemm_int3_exactly_representable_bit_exact(q4, orc, path, m):
    """x in {-4..4}/4, scales in {2^-7, 2^-8}: every product and partial sum
    is exact in f32 and (q - 4) * s is exact in f16, so both kernels must give
    the round-to-nearest-even of the exact result."""
    rng = np.random.default_rng(40 + m)
    n, k = 512, 3072
    w3 = stream_words3(rng.integers(0, 8, (n, k)))
    s = si.f16_bits(2.0 ** -rng.integers(7, 9, (n, k // 32)))
    X = si.f16_bits(rng.integers(-4, 5, (m, k)) / 4.0)
    Y, _ = run_gemm3(q4, w3, s, X, GEMM_PATHS[path])
    ref, _ = orc.gemm3(w3, s, X)
    want = orc.doubles_to_halves(ref.ravel()).reshape(ref.shape)
    bad = np.argwhere(host_u16(Y) != want)
    assert bad.size == 0, f"{len(bad)} entries differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_gemm_int3_one_hot_rows(q4, orc, path):
    """row i of X is e_{k_i}: Y[i][r] = (q[r][k_i] - 4) * s exactly (one f16
    rounding); the positions cover every code slot of a 32-group (10 and 21
    cross canonical word boundaries, 30 and 31 are the bit-sliced codes) and
    pin the k order and output layout of both kernels."""
    rng = np.random.default_rng(23)
    n, k = 300, 3072
    w3, s = si.draw_weight3(rng, n, k)
    ks = list(range(32)) + [32, 42, 53, 62, 63, 255, 256, 1000, 2047, 3061, 3070, 3071, 1536]
    X = np.zeros((len(ks), k), np.uint16)
    for i, kk in enumerate(ks):
        X[i, kk] = 0x3C00
    Y, _ = run_gemm3(q4, w3, s, X, GEMM_PATHS[path])
    ref, _ = orc.gemm3(w3, s, X)
    want = orc.doubles_to_halves(ref.ravel()).reshape(ref.shape)
    assert np.array_equal(host_u16(Y), want)


@pytest.mark.parametrize("m", [4, 16, 24, 64, 128, 256])
def test_gemm_int3_prefill_full_shape_sampled(q4, orc, m):
    """The full prefill shape (W 16384 x 3072, int3): every output computed on
    the GPU, 96 weight rows x all m rows checked against the oracle."""
    rng = np.random.default_rng(900 + m)
    w3, s = si.draw_weight3(rng, 16384, 3072)
    X = si.draw_X(rng, m, 3072)
    Y, _ = run_gemm3(q4, w3, s, X)
    Yh = host_f16_as_f64(Y)
    rows = np.sort(np.random.default_rng(m).choice(16384, 96, replace=False))
    ref, a = orc.gemm3(np.ascontiguousarray(w3[rows]), np.ascontiguousarray(s[rows]), X)
    assert_within(Yh[:, rows], ref, tol_f16(ref, a), f"int3 prefill m={m}")
    assert np.all(np.isfinite(Yh))


def test_gemm_int3_row_matches_gemv(q4, orc):
    """m = 1 through the GEMM and the GEMV read the same packed buffer and both
    sit within the bound of the oracle."""
    rng = np.random.default_rng(61)
    n, k = 3072, 3072
    w3, s = si.draw_weight3(rng, n, k)
    X = si.draw_X(rng, 1, k)
    Y, pw = run_gemm3(q4, w3, s, X, 1)
    y = q4.gemv(pw, dev_f16(X[0]))
    ref, a = orc.gemm3(w3, s, X)
    t = tol_f16(ref, a)
    assert_within(host_f16_as_f64(Y), ref, t, "gemm m=1")
    assert_within(host_f16_as_f64(y)[None, :], ref, t, "gemv")

"""The fused QKV step on the GPU (rotary-paired layout, RoPE on the q and k
heads, K/V appended to a paged cache) against the oracle.  Tolerance of a
rotated element: y_i' = y_i cos - y_j sin mixes two matmul rows, so the bound
adds their magnitude sums: 2e-3 |y'| + 1e-3 (a_i + a_j) + 1e-5; v rows keep
the plain f16 bound."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import (assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16,
                    tol_f16)

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A


def pair_tol(y_ref, a, d, nq, nkv):
    a2 = a.copy()
    half = d // 2
    for h in range(nq + nkv):
        lo, hi = h * d, h * d + half
        s = a[lo:lo + half] + a[hi:hi + half]
        a2[lo:lo + half] = s
        a2[hi:hi + half] = s
    return tol_f16(y_ref, a2)


def run_case(q4, orc, n, k, d, nq, pos, seed, norm=False):
    nkv = (n // d - nq) // 2
    rng = np.random.default_rng(seed)
    w, s = si.draw_weight(rng, n, k)
    x = si.draw_x(rng, k)
    pw = q4.pack_rope(dev_u32(w), dev_u16(s), d)
    pages = pos // 16 + 3
    table = rng.permutation(pages).astype(np.int32)
    cache = torch.full((pages, 2, nkv, 16, d), SENTINEL, dtype=torch.int16, device="cuda")
    pt = torch.from_numpy(table).cuda()
    if norm:
        r = si.f16_bits(rng.normal(0.0, 2.0, k))
        gamma = si.f16_bits(rng.uniform(0.5, 1.5, k))
        h_ref, xn = orc.add_rmsnorm(x, r, gamma, 1e-5)
        hout = dev_f16(np.zeros(k, np.uint16))
        y = q4.qkv_rope_append(pw, dev_f16(x), nq, pos, 10000.0, cache, pt,
                               norm=(dev_f16(r), dev_f16(gamma), 1e-5, hout))
        assert np.array_equal(host_u16(hout), h_ref)
        x_eff = xn
    else:
        y = q4.qkv_rope_append(pw, dev_f16(x), nq, pos, 10000.0, cache, pt)
        x_eff = x
    y_ref, a = orc.qkv_rope(w, s, x_eff, d, nq, pos, 10000.0)
    yb = host_u16(y)
    assert_within(host_f16_as_f64(y), y_ref, pair_tol(y_ref, a, d, nq, nkv),
                  f"qkv rope n={n} k={k} pos={pos}")
    # the cache: exactly the k and v heads of y, at the page and slot of pos
    c = cache.cpu().numpy().view(np.uint16)
    page, slot = table[pos // 16], pos % 16
    kpart = yb[nq * d:(nq + nkv) * d].reshape(nkv, d)
    vpart = yb[(nq + nkv) * d:].reshape(nkv, d)
    assert np.array_equal(c[page, 0, :, slot], kpart)
    assert np.array_equal(c[page, 1, :, slot], vpart)
    mask = np.ones(c.shape, bool)
    mask[page, :, :, slot] = False
    assert np.all(c[mask] == SENTINEL)
    return pw, x, y


def test_pack_rope_byte_exact_and_roundtrip(q4, orc):
    rng = np.random.default_rng(3)
    for n, k, d in ((9216, 3072, 96), (96, 64, 8), (384, 8192, 96)):
        w, s = si.draw_weight(rng, n, k)
        pw = q4.pack_rope(dev_u32(w), dev_u16(s), d)
        assert np.array_equal(pw.buf.cpu().numpy(), orc.encode_rope(w, s, d))
        uw, us = q4.unpack(pw)
        assert np.array_equal(uw.cpu().numpy().view(np.uint32), w)
        assert np.array_equal(us.cpu().numpy().view(np.uint16), s)


@pytest.mark.parametrize("pos", [0, 37, 4095])
def test_qkv_rope_phi3(q4, orc, pos):
    """Phi-3-mini: 32 q, 32 k, 32 v heads of 96 over k = 3072."""
    run_case(q4, orc, 9216, 3072, 96, 32, pos, seed=pos)


@pytest.mark.parametrize("n,k,d,nq,pos", [
    (512, 1024, 64, 4, 100),      # grouped-query shape: 4 q heads, 2 k/v heads
    (384, 8192, 96, 2, 19),       # long k: the split kernel
    (96, 16480, 8, 4, 5),         # k > 8192: the multi-pass kernel
    (48, 96, 16, 1, 3),           # one q head, one k/v pair, tiny k
])
def test_qkv_rope_shapes(q4, orc, n, k, d, nq, pos):
    run_case(q4, orc, n, k, d, nq, pos, seed=n + k)


def test_qkv_rope_with_norm_prologue(q4, orc):
    run_case(q4, orc, 9216, 3072, 96, 32, 21, seed=9, norm=True)


def test_qkv_rope_position_zero_is_the_plain_gemv(q4):
    """At position 0 every angle is 0: the output is the plain matmul of the
    same weight bit for bit (same per-row arithmetic in another row order)."""
    rng = np.random.default_rng(4)
    w, s = si.draw_weight(rng, 9216, 3072)
    x = si.draw_x(rng, 3072)
    y = q4.qkv_rope_append(q4.pack_rope(dev_u32(w), dev_u16(s), 96), dev_f16(x), 32, 0, 10000.0)
    y_plain = q4.gemv(q4.pack(dev_u32(w), dev_u16(s)), dev_f16(x))
    assert np.array_equal(host_u16(y), host_u16(y_plain))


def test_qkv_rope_invalid_page_appends_nothing(q4, orc):
    rng = np.random.default_rng(6)
    n, k, d, nq = 9216, 3072, 96, 32
    w, s = si.draw_weight(rng, n, k)
    x = si.draw_x(rng, k)
    pw = q4.pack_rope(dev_u32(w), dev_u16(s), d)
    cache = torch.full((2, 2, 32, 16, d), SENTINEL, dtype=torch.int16, device="cuda")
    pt = torch.tensor([1, 7, -1], dtype=torch.int32, device="cuda")
    for pos in (20, 33):   # page entries 7 and -1: outside the 2 pages
        y = q4.qkv_rope_append(pw, dev_f16(x), nq, pos, 10000.0, cache, pt)
        assert np.all(cache.cpu().numpy().view(np.uint16) == SENTINEL)
        y_ref, a = orc.qkv_rope(w, s, x, d, nq, pos, 10000.0)
        assert_within(host_f16_as_f64(y), y_ref, pair_tol(y_ref, a, d, nq, 32), "qkv no append")

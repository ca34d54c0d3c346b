"""Residual add + RMSNorm fused into the GEMV / gate-up matmul on the GPU,
against the oracle (add_rmsnorm, then the matmul on the oracle's normalised
vector): the residual output bit for bit, y within the f16 bound.  The GPU
normalises in f32, so an element of its normalised vector may sit one f16 ulp
from the oracle's; that moves y by at most 2^-11 * sum |x_k w_k|, inside the
1e-3 * sum |x_k w_k| term of the bound."""
import numpy as np
import pytest

import seeded_inputs as si
from parity import (assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16,
                    tol_f16, tol_ffn)

pytestmark = pytest.mark.gpu


def draw_norm_inputs(rng, k, with_residual):
    x = si.draw_x(rng, k)
    x[:: 97] = 0x8000          # a few -0.0: the residual output must keep them
    r = si.f16_bits(rng.normal(0.0, 2.0, k)) if with_residual else None
    gamma = si.f16_bits(rng.uniform(0.5, 1.5, k))
    return x, r, gamma


# block kernel (QKV shape, small k), long-k split kernel, multi-pass kernel
SHAPES = [(9216, 3072), (3000, 8192), (5, 16480), (130, 96), (7, 64)]


@pytest.mark.parametrize("with_residual", [True, False])
@pytest.mark.parametrize("n,k", SHAPES)
def test_add_rmsnorm_gemv_parity(q4, orc, n, k, with_residual):
    rng = np.random.default_rng(n * 7 + k + with_residual)
    x, r, gamma = draw_norm_inputs(rng, k, with_residual)
    w, s = si.draw_weight(rng, n, k)
    eps = 1e-5
    h_ref, xn_ref = orc.add_rmsnorm(x, r, gamma, eps)
    y_ref, a = orc.gemv(w, s, xn_ref)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    hout = dev_f16(np.zeros(k, np.uint16))
    y = q4.add_rmsnorm_gemv(pw, dev_f16(x), None if r is None else dev_f16(r), dev_f16(gamma),
                            eps, residual_out=hout)
    assert np.array_equal(host_u16(hout), h_ref)
    ratio = assert_within(host_f16_as_f64(y), y_ref, tol_f16(y_ref, a), f"norm gemv {n}x{k}")
    print(f"max err/tol {ratio:.3g}")
    # without a residual output, the same y bit for bit
    y2 = q4.add_rmsnorm_gemv(pw, dev_f16(x), None if r is None else dev_f16(r), dev_f16(gamma), eps)
    assert np.array_equal(host_u16(y2), host_u16(y))


@pytest.mark.parametrize("n,k", [(8192, 3072), (129, 8192), (3, 16416)])
def test_add_rmsnorm_ffn_parity(q4, orc, n, k):
    rng = np.random.default_rng(n + 5 * k)
    x, r, gamma = draw_norm_inputs(rng, k, True)
    gate = si.draw_weight(rng, n, k)
    up = si.draw_weight(rng, n, k)
    eps = 1e-6
    h_ref, xn_ref = orc.add_rmsnorm(x, r, gamma, eps)
    ref = orc.ffn_gate_up_silu(*gate, *up, xn_ref)
    pgu = q4.pack_gate_up(dev_u32(gate[0]), dev_u16(gate[1]), dev_u32(up[0]), dev_u16(up[1]))
    hout = dev_f16(np.zeros(k, np.uint16))
    h = q4.add_rmsnorm_ffn_gate_up_silu(pgu, dev_f16(x), dev_f16(r), dev_f16(gamma), eps,
                                        residual_out=hout)
    assert np.array_equal(host_u16(hout), h_ref)
    assert_within(host_f16_as_f64(h), ref["h"], tol_ffn(ref), f"norm ffn {n}x{k}")


@pytest.mark.parametrize("n,k", [(3072, 3072), (777, 8192), (3, 16480)])
@pytest.mark.parametrize("c", [2.0, -0.5])
def test_add_rmsnorm_constant_input_is_plain_gemv_of_ones(q4, n, k, c):
    """x = c everywhere, gamma = 1, eps = 0: the normalised vector is sign(c)
    exactly (1 / sqrt(c^2) is exact for these c), so y must equal q4_gemv of
    that vector bit for bit."""
    rng = np.random.default_rng(k)
    w, s = si.draw_weight(rng, n, k)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    x = si.f16_bits(np.full(k, c))
    ones = si.f16_bits(np.ones(k))
    y = q4.add_rmsnorm_gemv(pw, dev_f16(x), None, dev_f16(ones), 0.0)
    y_plain = q4.gemv(pw, dev_f16(si.f16_bits(np.full(k, np.sign(c)))))
    assert np.array_equal(host_u16(y), host_u16(y_plain))


def test_add_rmsnorm_deterministic(q4):
    rng = np.random.default_rng(5)
    x, r, gamma = draw_norm_inputs(rng, 3072, True)
    w, s = si.draw_weight(rng, 9216, 3072)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    ys = [host_u16(q4.add_rmsnorm_gemv(pw, dev_f16(x), dev_f16(r), dev_f16(gamma), 1e-5))
          for _ in range(3)]
    assert all(np.array_equal(ys[0], v) for v in ys[1:])

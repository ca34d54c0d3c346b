"""q4_ffn_gate_up_silu on the GPU against the oracle (fused gate/up + SiLU),
then the down projection on the oracle's own f16 h and end to end."""
import numpy as np
import pytest

import seeded_inputs as si
from parity import (assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16,
                    tol_f16, tol_ffn)

pytestmark = pytest.mark.gpu


def pack_gu(q4, gate, up):
    return q4.pack_gate_up(dev_u32(gate[0]), dev_u16(gate[1]), dev_u32(up[0]), dev_u16(up[1]))


def test_ffn_phi3_parity_and_down(q4, orc):
    inp = si.workload(si.FFN, seed=0)
    pw = pack_gu(q4, inp["gate"], inp["up"])
    h = q4.ffn_gate_up_silu(pw, dev_f16(inp["x"]))
    ref = orc.ffn_gate_up_silu(*inp["gate"], *inp["up"], inp["x"])
    ratio = assert_within(host_f16_as_f64(h), ref["h"], tol_ffn(ref), "ffn h")
    print(f"h: max err/tol {ratio:.3g}")
    # stage-wise down projection on the oracle's own h (rounded by the oracle)
    dw, ds = inp["down"]
    h_ref16 = orc.doubles_to_halves(ref["h"])
    pd = q4.pack(dev_u32(dw), dev_u16(ds))
    y = q4.gemv(pd, dev_f16(h_ref16))
    yref, a = orc.gemv(dw, ds, h_ref16)
    assert_within(host_f16_as_f64(y), yref, tol_f16(yref, a), "down on oracle h")
    # end to end: the GPU's h feeds the GPU's down.  Bound: the down tolerance
    # plus sum_k |w[n][k]| * |h_gpu[k] - h_ref16[k]| (how far the GPU's h moved)
    hh = host_u16(h)
    y2 = host_f16_as_f64(q4.gemv(pd, h))
    dh = np.abs(orc.halves_to_doubles(hh) - orc.halves_to_doubles(h_ref16))
    wabs = _abs_weight_times(orc, dw, ds, dh)
    assert_within(y2, yref, 1.01 * tol_f16(yref, a) + wabs * (1 + 1e-3), "down end to end")


def _abs_weight_times(orc, words, scales, v):
    """sum_k |w[n][k]| * v[k] through the oracle: a_ref of x = v with the
    weights' own magnitudes (v >= 0 rounded up to f16)."""
    vb = orc.doubles_to_halves(v * (1 + 2.0 ** -10))
    _, a = orc.gemv(words, scales, vb)
    return a


def test_ffn_closed_forms(q4):
    """gate codes 8 -> g = 0 -> h = +0; up codes 8 -> u = 0 -> h = 0."""
    k, n = 3072, 300
    rng = np.random.default_rng(2)
    x = si.draw_x(rng, k)
    s = si.f16_bits(rng.uniform(0.005, 0.02, (n, k // 32)))
    w8 = si.pack_codes(np.full((n, k), 8, np.uint8))
    wr, sr = si.draw_weight(rng, n, k)
    h = host_u16(q4.ffn_gate_up_silu(pack_gu(q4, (w8, s), (wr, sr)), dev_f16(x)))
    assert np.all((h & 0x7FFF) == 0)
    h = host_u16(q4.ffn_gate_up_silu(pack_gu(q4, (wr, sr), (w8, s)), dev_f16(x)))
    assert np.all((h & 0x7FFF) == 0)


@pytest.mark.parametrize("n,k", [(1, 32), (7, 96), (129, 3072), (300, 8192 + 32 * 3),
                                 (129, 8192), (1000, 7168)])
def test_ffn_ragged(q4, orc, n, k):
    rng = np.random.default_rng(n + 3 * k)
    x = si.draw_x(rng, k)
    gate = si.draw_weight(rng, n, k)
    up = si.draw_weight(rng, n, k)
    h = q4.ffn_gate_up_silu(pack_gu(q4, gate, up), dev_f16(x))
    ref = orc.ffn_gate_up_silu(*gate, *up, x)
    assert_within(host_f16_as_f64(h), ref["h"], tol_ffn(ref), f"ffn {n}x{k}")

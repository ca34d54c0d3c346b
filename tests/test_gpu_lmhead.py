"""q4_lmhead_f32 on the GPU: f32 logits against the oracle, and the greedy
argmax (exact index, or within the tolerance gap when several are right)."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import argmax_ok, assert_within, dev_f16, dev_u16, dev_u32, tol_f32

pytestmark = pytest.mark.gpu


def test_lmhead_phi3_parity(q4, orc):
    inp = si.workload(si.LM_HEAD, seed=0)
    pw = q4.pack(dev_u32(inp["words"]), dev_u16(inp["scales"]))
    logits, idx = q4.lmhead_f32(pw, dev_f16(inp["x"]))
    ref, a, idx_ref = orc.lmhead(inp["words"], inp["scales"], inp["x"])
    got = logits.cpu().numpy().astype(np.float64)
    ratio = assert_within(got, ref, tol_f32(a), "lm head logits")
    print(f"logits max err/tol {ratio:.3g}; argmax {int(idx.item())} oracle {idx_ref}")
    assert argmax_ok(int(idx.item()), ref, a, idx_ref)
    # the kernel's argmax is exactly the argmax of its own f32 logits
    assert int(idx.item()) == int(np.argmax(got))


@pytest.mark.parametrize("n,k", [(32064, 3072), (1001, 3072), (5, 3072), (1, 3072),
                                 (1001, 8192), (5003, 8192)])
def test_lmhead_planted_argmax_and_ties(q4, orc, n, k):
    """A planted winner (codes 15, x = 1) and an exact tie with a later copy of
    the same row: the lowest index wins, across blocks; repeated calls with
    different n reuse the same workspace.  k = 8192 takes the long-k split
    kernel (1001 rows) and the block kernel with 4 groups per lane (5003)."""
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    scales = si.f16_bits(rng.uniform(0.005, 0.02, (n, k // 32)))
    win = (n * 5) // 7
    codes[win] = 15
    scales[win] = si.f16_bits(0.02)
    if n > 1:
        twin = n - 1 if win != n - 1 else 0
        lo, hi = sorted((win, twin))
        codes[twin] = codes[win]
        scales[twin] = scales[win]
    else:
        lo = win
    w = si.pack_codes(codes)
    x = si.f16_bits(np.ones(k))
    pw = q4.pack(dev_u32(w), dev_u16(scales))
    for _ in range(3):
        logits, idx = q4.lmhead_f32(pw, dev_f16(x))
        assert int(idx.item()) == lo
    ref, a, idx_ref = orc.lmhead(w, scales, x)
    assert idx_ref == lo
    assert_within(logits.cpu().numpy(), ref, tol_f32(a), "planted logits")


def test_lmhead_without_argmax_and_scaling(q4):
    """Same logits with and without the argmax; doubling x doubles every f32
    logit bit for bit (a power-of-two scale commutes with every rounding,
    including the directed rounding of v_dot2_f32_f16)."""
    inp = si.workload(si.LM_HEAD, seed=3, scale=0.1)
    pw = q4.pack(dev_u32(inp["words"]), dev_u16(inp["scales"]))
    x = dev_f16(inp["x"])
    l1, none = q4.lmhead_f32(pw, x, with_argmax=False)
    assert none is None
    l2, _ = q4.lmhead_f32(pw, x)
    assert torch.equal(l1, l2)
    x2 = si.f16_bits(inp["x"].view(np.float16).astype(np.float64) * 2)
    l4, _ = q4.lmhead_f32(pw, dev_f16(x2))
    assert torch.equal(l4, 2 * l1)


def test_lmhead_odd_symmetry_exact_inputs(q4):
    """With exactly representable inputs every sum is exact, so negating x
    negates every logit bit for bit.  (With general inputs this does not hold:
    v_dot2_f32_f16 rounds its f32 result toward -inf, not to nearest even.)"""
    n, k = 4100, 3072
    rng = np.random.default_rng(6)
    w = si.pack_codes(rng.integers(0, 16, (n, k), dtype=np.uint8))
    s = si.f16_bits(2.0 ** -rng.integers(7, 9, (n, k // 32)))
    x = si.f16_bits(rng.integers(-4, 5, k) / 4.0)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    l1, _ = q4.lmhead_f32(pw, dev_f16(x))
    ln, _ = q4.lmhead_f32(pw, dev_f16(x ^ np.uint16(0x8000)))
    assert torch.equal(ln, -l1)

"""q4_pack / q4_pack_gate_up / q4_unpack on the GPU: bytes must equal the
oracle's independent encoder of the device layout (exact), and unpack must
return the canonical input (exact)."""
import numpy as np
import pytest

import seeded_inputs as si
from parity import dev_u16, dev_u32

pytestmark = pytest.mark.gpu

SHAPES = [(3072, 3072), (3072, 8192), (32064, 3072), (1, 32), (17, 96), (130, 64),
          (33, 224), (7, 160), (6, 192), (3, 3200), (5, 16384), (3, 8352), (4, 16480),
          (1000, 3072)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_pack_bytes_equal_oracle_encoder(q4, orc, n, k):
    rng = np.random.default_rng(n * 7919 + k)
    w, s = si.draw_weight(rng, n, k)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    got = pw.buf.cpu().numpy()
    want = orc.encode_rows(w, s)
    assert got.size == want.size == q4.packed_bytes(n, k)
    assert q4.layout_geometry(n, k) == orc.layout_geometry(n, k)
    diff = np.nonzero(got != want)[0]
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:8].tolist()}"
    words, scales = q4.unpack(pw)
    assert np.array_equal(words.cpu().numpy().view(np.uint32), w)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), s)


@pytest.mark.parametrize("n,k", [(8192, 3072), (7, 96), (1, 32), (100, 8192 + 32 * 3)])
def test_pack_gate_up_bytes_equal_oracle_encoder(q4, orc, n, k):
    rng = np.random.default_rng(n + k)
    gw, gs = si.draw_weight(rng, n, k)
    uw, us = si.draw_weight(rng, n, k)
    pw = q4.pack_gate_up(dev_u32(gw), dev_u16(gs), dev_u32(uw), dev_u16(us))
    got = pw.buf.cpu().numpy()
    want = orc.encode_gate_up(gw, gs, uw, us)
    assert got.size == want.size == q4.packed_bytes(n, k, q4.LAYOUT_GATE_UP)
    assert np.array_equal(got, want)
    words, scales = q4.unpack(pw)
    words = words.cpu().numpy().view(np.uint32)
    scales = scales.cpu().numpy().view(np.uint16)
    assert np.array_equal(words[0::2], gw) and np.array_equal(words[1::2], uw)
    assert np.array_equal(scales[0::2], gs) and np.array_equal(scales[1::2], us)


def test_every_code_value_and_nibble_survives(q4):
    # each word holds 8 distinct codes; all 16 values at every nibble position
    n, k = 16, 256
    codes = (np.arange(n)[:, None] + np.arange(k)[None, :]) % 16
    w = si.pack_codes(codes.astype(np.uint8))
    s = np.arange(n * k // 32, dtype=np.uint16).reshape(n, k // 32)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    words, scales = q4.unpack(pw)
    assert np.array_equal(words.cpu().numpy().view(np.uint32), w)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), s)

"""The allocation-free LM head (q4_lmhead_f32_noalloc, argmax candidates in
the library's static scratch) against q4_lmhead_f32 with a caller workspace,
through the C ABI: the same logits bit for bit and the same argmax index, on
two calls in a row (the second on a smaller weight, so it runs fewer blocks
over the scratch the first one left behind), int4 and int3."""
import ctypes

import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import argmax_ok, dev_f16, dev_u16, dev_u32

pytestmark = pytest.mark.gpu


def _noalloc(q4, pw, x):
    logits = torch.full((pw.n,), float("nan"), dtype=torch.float32, device="cuda")
    am = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    rc = q4.lib.q4_lmhead_f32_noalloc(ctypes.byref(pw.desc), x.data_ptr(), logits.data_ptr(),
                                      am.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, q4.lib.q4_strerror(rc)
    return logits, am


def _with_ws(q4, pw, x):
    logits = torch.empty(pw.n, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    need = int(q4.lib.q4_workspace_bytes(q4.OP_LMHEAD, 1, pw.n, pw.k))
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    q4.lmhead_f32(pw, x, logits, am, ws=ws)
    return logits, am


@pytest.mark.parametrize("fmt", [4, 3])
def test_noalloc_lmhead_matches_workspace_call(q4, orc, fmt):
    rng = np.random.default_rng(31 + fmt)
    for n, k in ((32064, 3072), (777, 1024)):    # the second call is smaller
        x = si.draw_x(rng, k)
        if fmt == 4:
            w, s = si.draw_weight(rng, n, k)
            pw = q4.pack(dev_u32(w), dev_u16(s))
            ref, a = orc.gemv(w, s, x)
        else:
            w, s = si.draw_weight3(rng, n, k)
            pw = q4.pack_int3(dev_u32(w), dev_u16(s))
            ref, a = orc.gemv3(w, s, x)
        xd = dev_f16(x)
        l1, i1 = _noalloc(q4, pw, xd)
        l2, i2 = _with_ws(q4, pw, xd)
        torch.cuda.synchronize()
        assert torch.equal(l1, l2), (n, k)
        assert int(i1.item()) == int(i2.item()), (n, k)
        assert argmax_ok(int(i1.item()), ref, a, orc.argmax(ref)), (n, k)


def test_noalloc_lmhead_without_argmax(q4):
    rng = np.random.default_rng(37)
    w, s = si.draw_weight(rng, 300, 3072)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    xd = dev_f16(si.draw_x(rng, 3072))
    logits = torch.empty(300, dtype=torch.float32, device="cuda")
    rc = q4.lib.q4_lmhead_f32_noalloc(ctypes.byref(pw.desc), xd.data_ptr(), logits.data_ptr(), None,
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    l2, _ = _with_ws(q4, pw, xd)
    torch.cuda.synchronize()
    assert torch.equal(logits, l2)

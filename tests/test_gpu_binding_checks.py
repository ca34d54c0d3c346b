"""The binding refuses caller mistakes with a Python error before anything
is launched: a host cache, a cache whose heads or dims do not match the
weight, a page table too short for the position or context."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import dev_f16, dev_u16, dev_u32

pytestmark = pytest.mark.gpu


def test_qkv_rope_append_checks(q4):
    rng = np.random.default_rng(3)
    d, nq, nkv, k = 64, 4, 2, 256
    n = (nq + 2 * nkv) * d
    w, s = si.draw_weight(rng, n, k)
    pw = q4.pack_rope(dev_u32(w), dev_u16(s), d)
    x = dev_f16(si.draw_x(rng, k))
    cache = torch.zeros((3, 2, nkv, 16, d), dtype=torch.float16, device="cuda")
    pt = torch.arange(3, dtype=torch.int32, device="cuda")
    q4.qkv_rope_append(pw, x, nq, 40, 10000.0, cache, pt)     # a valid call
    torch.cuda.synchronize()
    with pytest.raises(TypeError):
        q4.qkv_rope_append(pw, x, nq, 40, 10000.0, cache.cpu(), pt)
    with pytest.raises(ValueError):   # kv heads do not match the weight
        q4.qkv_rope_append(pw, x, nq, 40, 10000.0,
                           torch.zeros((3, 2, nkv + 1, 16, d), dtype=torch.float16, device="cuda"), pt)
    with pytest.raises(ValueError):   # head dim does not match
        q4.qkv_rope_append(pw, x, nq, 40, 10000.0,
                           torch.zeros((3, 2, nkv, 16, d // 2), dtype=torch.float16, device="cuda"), pt)
    with pytest.raises(ValueError):   # q heads that leave an odd k/v split
        q4.qkv_rope_append(pw, x, nq + 1, 40, 10000.0, cache, pt)
    with pytest.raises(ValueError):   # position 48 needs 4 page-table entries
        q4.qkv_rope_append(pw, x, nq, 48, 10000.0, cache, pt)


def test_attention_checks(q4):
    rng = np.random.default_rng(4)
    nq, nkv, d = 4, 2, 64
    cache = dev_f16(si.f16_bits(rng.normal(0, 1, (4, 2, nkv, 16, d))))
    pt = torch.arange(4, dtype=torch.int32, device="cuda")
    q = dev_f16(si.f16_bits(rng.normal(0, 1, nq * d)))
    q4.attention_decode(q, cache, pt, 64, nq, 0.125)
    torch.cuda.synchronize()
    with pytest.raises(TypeError):
        q4.attention_decode(q, cache.cpu(), pt, 64, nq, 0.125)
    with pytest.raises(ValueError):   # 65 positions need 5 entries
        q4.attention_decode(q, cache, pt, 65, nq, 0.125)
    pb = q4.kv_int8_page_bytes(nkv, d)
    cache8 = torch.zeros((4, pb), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        q4.attention_decode_int8(q, cache8, pt, 65, nq, nkv, d, 0.125)
    qkv = dev_f16(si.f16_bits(rng.normal(0, 1, (nq + 2 * nkv) * d)))
    with pytest.raises(ValueError):
        q4.kv_append_int8(qkv, nq, nkv, d, 64, cache8, pt)


def test_workspace_is_never_freed(q4):
    a = q4.workspace(torch.device("cuda", 0), 1 << 12)
    ptr = a.data_ptr()
    b = q4.workspace(torch.device("cuda", 0), 1 << 22)
    assert b.numel() >= 1 << 22
    # the outgrown buffer is still owned by the module (graphs may hold it)
    assert any(t.data_ptr() == ptr for t in q4._retired) or b.data_ptr() == ptr

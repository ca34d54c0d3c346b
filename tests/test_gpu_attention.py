"""Paged-attention decode on the GPU against the oracle.  Bound per output
element: 2e-3 |o| + 1e-3 sum_t p_t |v_t| + 1e-5 (f32 scores and softmax, one
f16 rounding of the output; the second term sizes the f32 accumulation)."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16

pytestmark = pytest.mark.gpu

NAN16 = 0x7E00


def tol_attn(o, a):
    return 2e-3 * np.abs(o) + 1e-3 * a + 1e-5


def make(rng, ctx, nq, nkv, d, spare_pages=2):
    pages = (ctx + 15) // 16 + spare_pages
    cache = si.f16_bits(rng.normal(0.0, 1.0, (pages, 2, nkv, 16, d)))
    table = rng.permutation(pages)[: (ctx + 15) // 16].astype(np.int32)
    # every slot the context does not cover holds NaN: it must never leak in
    used = np.zeros((pages, 16), bool)
    for t in range(ctx):
        used[table[t // 16], t % 16] = True
    for kv in (0, 1):
        for g in range(nkv):
            cache[:, kv, g][~used] = NAN16
    q = si.f16_bits(rng.normal(0.0, 1.0, (nq, d)))
    return cache, table, q


def run(q4, cache, table, q, ctx, nq, scale):
    c = torch.from_numpy(cache.view(np.float16)).cuda()
    return q4.attention_decode(dev_f16(q.reshape(-1)), c, torch.from_numpy(table).cuda(), ctx,
                               nq, scale)


@pytest.mark.parametrize("ctx", [1, 15, 16, 17, 255, 256, 257, 1000, 4096])
def test_attention_phi3(q4, orc, ctx):
    rng = np.random.default_rng(ctx)
    nq = nkv = 32
    d = 96
    cache, table, q = make(rng, ctx, nq, nkv, d)
    scale = 1.0 / np.sqrt(d)
    out = run(q4, cache, table, q, ctx, nq, scale)
    ref, a = orc.attention_decode(q, cache, table, ctx, nq, nkv, d, scale)
    r = assert_within(host_f16_as_f64(out), ref, tol_attn(ref, a), f"attention ctx={ctx}")
    print(f"max err/tol {r:.3g}")


@pytest.mark.parametrize("nq,nkv,d,ctx", [(8, 2, 64, 300), (4, 1, 128, 70), (2, 2, 256, 33),
                                          (6, 3, 32, 513)])
def test_attention_shapes(q4, orc, nq, nkv, d, ctx):
    rng = np.random.default_rng(nq * 100 + d + ctx)
    cache, table, q = make(rng, ctx, nq, nkv, d)
    scale = 0.7 / np.sqrt(d)
    out = run(q4, cache, table, q, ctx, nq, scale)
    ref, a = orc.attention_decode(q, cache, table, ctx, nq, nkv, d, scale)
    assert_within(host_f16_as_f64(out), ref, tol_attn(ref, a), f"attention {nq}/{nkv}x{d} ctx={ctx}")


def test_attention_absent_page(q4, orc):
    """A table entry outside the cache drops its 16 positions: the same as
    attending over the remaining positions only."""
    rng = np.random.default_rng(77)
    nq = nkv = 4
    d, ctx = 64, 40
    cache, table, q = make(rng, ctx, nq, nkv, d)
    holed = table.copy()
    holed[1] = -1
    out = run(q4, cache, holed, q, ctx, nq, 0.125)
    # positions 0..15 (page table[0]) and 32..39 (slots 0..7 of page table[2])
    ref, a = orc.attention_decode(q, cache, np.array([table[0], table[2]], np.int32), 24, nq, nkv,
                                  d, 0.125)
    assert_within(host_f16_as_f64(out), ref, tol_attn(ref, a), "attention absent page")


def test_attention_deterministic(q4):
    rng = np.random.default_rng(5)
    cache, table, q = make(rng, 3000, 32, 32, 96)
    outs = [host_u16(run(q4, cache, table, q, 3000, 32, 0.1)) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_attention_many_chunks(q4, orc):
    """Contexts split into many chunks per head (a single head, grouped
    heads, long contexts) through one shared workspace, called in a row with
    different shapes."""
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda").fill_(0xFF)
    for i, (nq, nkv, d, ctx) in enumerate([(1, 1, 64, 5000), (4, 2, 128, 20000), (32, 32, 96, 1000),
                                           (1, 1, 64, 300), (4, 2, 128, 20000)]):
        rng = np.random.default_rng(900 + i)
        need = q4.lib.q4_workspace_bytes(q4.OP_ATTENTION, ctx, nq, d)
        assert 0 < need <= ws.numel()
        cache, table, q = make(rng, ctx, nq, nkv, d)
        c = torch.from_numpy(cache.view(np.float16)).cuda()
        out = q4.attention_decode(dev_f16(q.reshape(-1)), c, torch.from_numpy(table).cuda(), ctx,
                                  nq, 0.09, ws=ws)
        ref, a = orc.attention_decode(q, cache, table, ctx, nq, nkv, d, 0.09)
        assert_within(host_f16_as_f64(out), ref, tol_attn(ref, a), f"attention {nq}x{d} ctx={ctx}")


def test_attention_long_context_many_chunks(q4, orc):
    """70,000 positions over 2 query heads on one kv head: 137 chunks per
    head, so the combine kernel merges its records in several batches of 16
    (the last one partial)."""
    rng = np.random.default_rng(70000)
    nq, nkv, d, ctx = 2, 1, 128, 70000
    assert q4.lib.q4_workspace_bytes(q4.OP_ATTENTION, ctx, nq, d) > nq * 32 * (d + 2) * 4
    cache, table, q = make(rng, ctx, nq, nkv, d)
    out = run(q4, cache, table, q, ctx, nq, 0.08)
    ref, a = orc.attention_decode(q, cache, table, ctx, nq, nkv, d, 0.08)
    assert_within(host_f16_as_f64(out), ref, tol_attn(ref, a), "attention ctx 70000")


def test_decode_steps_then_attention(q4, orc):
    """The decode pipeline: 40 fused QKV steps fill the cache through a page
    table; attention of the last step's q over the 40 positions matches the
    oracle on the cache as written."""
    rng = np.random.default_rng(11)
    nq = nkv = 4
    d, k = 64, 256
    n = (nq + 2 * nkv) * d
    w, s = si.draw_weight(rng, n, k)
    pw = q4.pack_rope(dev_u32(w), dev_u16(s), d)
    pages = 5
    table = np.array([3, 0, 4], np.int32)
    cache = torch.zeros((pages, 2, nkv, 16, d), dtype=torch.float16, device="cuda")
    pt = torch.from_numpy(table).cuda()
    steps = 40
    for pos in range(steps):
        x = si.draw_x(rng, k)
        y = q4.qkv_rope_append(pw, dev_f16(x), nq, pos, 10000.0, cache, pt)
    qh = host_u16(y)[: nq * d].reshape(nq, d)
    out = q4.attention_decode(y[: nq * d], cache, pt, steps, nq, 0.125)
    cb = cache.cpu().numpy().view(np.uint16)
    ref, a = orc.attention_decode(qh, cb, table, steps, nq, nkv, d, 0.125)
    assert_within(host_f16_as_f64(out), ref, tol_attn(ref, a), "decode then attention")

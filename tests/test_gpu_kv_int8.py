"""The int8 KV cache on the GPU against the oracle: the quantise-and-append
bytes bit for bit (codes and scales are decided in f32 on both sides), and
attention over int8 caches within the attention bound
(2e-3 |o| + 1e-3 sum_t p_t |v_t| + 1e-5), alone and after 40 decode steps
that fill the cache through the fused QKV step."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16

pytestmark = pytest.mark.gpu


def tol_attn(o, a):
    return 2e-3 * np.abs(o) + 1e-3 * a + 1e-5


def block_offset(nkv, d, page, kv, g):
    return page * 2 * nkv * (16 * d + 64) + (kv * nkv + g) * (16 * d + 64)


def make_cache8(rng, ctx, nkv, d, spare_pages=2):
    """int8 pages with random codes and scales for the slots the context
    covers; every other slot has a NaN scale, so a read outside the context
    shows up as NaN."""
    pages = (ctx + 15) // 16 + spare_pages
    pb = 2 * nkv * (16 * d + 64)
    table = rng.permutation(pages)[: (ctx + 15) // 16].astype(np.int32)
    cache = np.zeros((pages, pb), np.uint8)
    flat = cache.reshape(-1)
    flat[:] = rng.integers(0, 256, flat.size, dtype=np.uint8)
    used = np.zeros((pages, 16), bool)
    for t in range(ctx):
        used[table[t // 16], t % 16] = True
    for p in range(pages):
        for kv in (0, 1):
            for g in range(nkv):
                so = block_offset(nkv, d, p, kv, g) + 16 * d
                sc = rng.uniform(0.002, 0.03, 16).astype(np.float32)
                sc[~used[p]] = np.nan
                flat[so:so + 64] = sc.view(np.uint8)
    return cache, table


def run8(q4, cache, table, q, ctx, nq, nkv, d, scale, ws=None):
    return q4.attention_decode_int8(dev_f16(q.reshape(-1)), torch.from_numpy(cache).cuda(),
                                    torch.from_numpy(table).cuda(), ctx, nq, nkv, d, scale, ws=ws)


@pytest.mark.parametrize("nq,nkv,d,ctx", [(32, 32, 96, 1), (32, 32, 96, 17), (32, 32, 96, 1000),
                                          (32, 32, 96, 4096), (8, 2, 64, 300), (4, 1, 128, 70),
                                          (2, 2, 256, 33), (6, 3, 32, 513), (1, 1, 64, 5000)])
def test_attention_int8_parity(q4, orc, nq, nkv, d, ctx):
    rng = np.random.default_rng(nq * 1000 + d + ctx)
    cache, table = make_cache8(rng, ctx, nkv, d)
    q = si.f16_bits(rng.normal(0.0, 1.0, (nq, d)))
    scale = 1.0 / np.sqrt(d)
    out = run8(q4, cache, table, q, ctx, nq, nkv, d, scale)
    ref, a = orc.attention_decode_int8(q, cache, table, ctx, nq, nkv, d, scale)
    r = assert_within(host_f16_as_f64(out), ref, tol_attn(ref, a), f"int8 attention {nq}/{nkv}x{d} ctx={ctx}")
    print(f"max err/tol {r:.3g}")


def test_attention_int8_long_context(q4, orc):
    """70,000 positions, 2 query heads: many chunks through the combine kernel."""
    rng = np.random.default_rng(70001)
    nq, nkv, d, ctx = 2, 1, 128, 70000
    cache, table = make_cache8(rng, ctx, nkv, d)
    q = si.f16_bits(rng.normal(0.0, 1.0, (nq, d)))
    out = run8(q4, cache, table, q, ctx, nq, nkv, d, 0.08)
    ref, a = orc.attention_decode_int8(q, cache, table, ctx, nq, nkv, d, 0.08)
    assert_within(host_f16_as_f64(out), ref, tol_attn(ref, a), "int8 attention ctx 70000")


def test_kv_append_int8_bit_exact(q4, orc):
    rng = np.random.default_rng(61)
    nq, nkv, d = 32, 32, 96
    pages = 4
    pb = q4.kv_int8_page_bytes(nkv, d)
    table = np.array([2, 0, 3], np.int32)
    gpu = torch.full((pages, pb), 0xA5, dtype=torch.uint8, device="cuda")
    ref = np.full((pages, pb), 0xA5, np.uint8)
    pt = torch.from_numpy(table).cuda()
    for pos in (0, 1, 15, 16, 31, 40, 47):
        vals = rng.normal(0.0, 1.0, (nq + 2 * nkv) * d)
        if pos == 1:
            vals[(nq + 3) * d:(nq + 4) * d] = 0.0            # a zero row: scale 0, codes 0
        if pos == 15:
            vals[(nq + nkv + 5) * d + 7] = 3000.0            # one dominant value
        qkv = si.f16_bits(vals)
        q4.kv_append_int8(dev_f16(qkv), nq, nkv, d, pos, gpu, pt)
        orc.kv_append_int8(qkv, nq, nkv, d, pos, ref, table)
    got = gpu.cpu().numpy()
    bad = np.nonzero(got.reshape(-1) != ref.reshape(-1))[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:5].tolist()}"
    # a table entry outside the cache appends nothing
    before = gpu.clone()
    q4.kv_append_int8(dev_f16(qkv), nq, nkv, d, 3, gpu, torch.tensor([9], dtype=torch.int32, device="cuda"))
    assert torch.equal(before, gpu)


def test_decode_steps_then_int8_attention(q4, orc):
    """40 fused QKV steps (no f16 cache), each followed by the int8 append,
    then int8 attention of the last step's q over the 40 positions."""
    rng = np.random.default_rng(12)
    nq, nkv, d, k = 4, 2, 64, 256
    n = (nq + 2 * nkv) * d
    w, s = si.draw_weight(rng, n, k)
    pw = q4.pack_rope(dev_u32(w), dev_u16(s), d)
    table = np.array([3, 0, 4], np.int32)
    pt = torch.from_numpy(table).cuda()
    pb = q4.kv_int8_page_bytes(nkv, d)
    cache = torch.zeros((5, pb), dtype=torch.uint8, device="cuda")
    ref = np.zeros((5, pb), np.uint8)
    steps = 40
    for pos in range(steps):
        y = q4.qkv_rope_append(pw, dev_f16(si.draw_x(rng, k)), nq, pos, 10000.0)
        q4.kv_append_int8(y, nq, nkv, d, pos, cache, pt)
        orc.kv_append_int8(host_u16(y), nq, nkv, d, pos, ref, table)
    got = cache.cpu().numpy()
    assert np.array_equal(got, ref)
    qh = host_u16(y)[: nq * d].reshape(nq, d)
    out = q4.attention_decode_int8(y[: nq * d], cache, pt, steps, nq, nkv, d, 0.125)
    r, a = orc.attention_decode_int8(qh, got, table, steps, nq, nkv, d, 0.125)
    assert_within(host_f16_as_f64(out), r, tol_attn(r, a), "decode then int8 attention")


def test_attention_int8_deterministic(q4):
    rng = np.random.default_rng(6)
    cache, table = make_cache8(rng, 3000, 32, 96)
    q = si.f16_bits(rng.normal(0.0, 1.0, (32, 96)))
    outs = [host_u16(run8(q4, cache, table, q, 3000, 32, 32, 96, 0.1)) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])

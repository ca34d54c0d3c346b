"""Attention + O-projection with the context-chunk merge inside the
projection's x staging (q4_attention_oproj): bit for bit the same y as
q4_attention_decode (f16 or int8 cache) followed by q4_gemv, including the
shapes where the projection runs the split kernel and the library falls back
to the separate merge; and within the composed bound of the oracle's
attention and matmul."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16, tol_f16

pytestmark = pytest.mark.gpu

NAN16 = 0x7E00


def make_cache(rng, ctx, nkv, d):
    pages = (ctx + 15) // 16 + 2
    cache = si.f16_bits(rng.normal(0.0, 1.0, (pages, 2, nkv, 16, d)))
    table = rng.permutation(pages)[: (ctx + 15) // 16].astype(np.int32)
    used = np.zeros((pages, 16), bool)
    for t in range(ctx):
        used[table[t // 16], t % 16] = True
    for kv in (0, 1):
        for g in range(nkv):
            cache[:, kv, g][~used] = NAN16
    return cache, table


def make_cache8(rng, ctx, nkv, d):
    pages = (ctx + 15) // 16 + 2
    pb = 2 * nkv * (16 * d + 64)
    table = rng.permutation(pages)[: (ctx + 15) // 16].astype(np.int32)
    cache = rng.integers(0, 256, (pages, pb), dtype=np.uint8)
    sc = cache.reshape(pages, 2, nkv, 16 * d + 64)[:, :, :, 16 * d:]
    sc[:] = rng.uniform(0.002, 0.03, (pages, 2, nkv, 16)).astype(np.float32).view(np.uint8).reshape(
        pages, 2, nkv, 64)
    return cache, table


CASES = [(32, 32, 96, 3072, 1), (32, 32, 96, 3072, 40), (32, 32, 96, 3072, 1000),
         (32, 32, 96, 3072, 4096), (8, 2, 64, 256, 300), (4, 4, 32, 96, 17),
         (32, 8, 256, 512, 700)]   # the last: k = 8192 with few tiles -> split kernel, separate merge


@pytest.mark.parametrize("nq,nkv,d,n,ctx", CASES)
def test_attention_oproj_equals_unfused_f16(q4, nq, nkv, d, n, ctx):
    rng = np.random.default_rng(nq * 7 + d + n + ctx)
    cache, table = make_cache(rng, ctx, nkv, d)
    q = dev_f16(si.f16_bits(rng.normal(0.0, 1.0, nq * d)))
    w, s = si.draw_weight(rng, n, nq * d)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    c = torch.from_numpy(cache.view(np.float16)).cuda()
    pt = torch.from_numpy(table).cuda()
    y = q4.attention_oproj(q, c, pt, ctx, nq, d ** -0.5, pw)
    att = q4.attention_decode(q, c, pt, ctx, nq, d ** -0.5)
    y_ref = q4.gemv(pw, att.reshape(-1))
    assert np.array_equal(host_u16(y), host_u16(y_ref)), f"fused differs from unfused ({nq}x{d}, ctx {ctx})"


@pytest.mark.parametrize("nq,nkv,d,n,ctx", CASES[1:])
def test_attention_oproj_equals_unfused_int8(q4, nq, nkv, d, n, ctx):
    rng = np.random.default_rng(nq * 11 + d + n + ctx)
    cache, table = make_cache8(rng, ctx, nkv, d)
    q = dev_f16(si.f16_bits(rng.normal(0.0, 1.0, nq * d)))
    w, s = si.draw_weight(rng, n, nq * d)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    c = torch.from_numpy(cache).cuda()
    pt = torch.from_numpy(table).cuda()
    y = q4.attention_oproj(q, c, pt, ctx, nq, d ** -0.5, pw, kv_int8=True, n_kv_heads=nkv, head_dim=d)
    att = q4.attention_decode_int8(q, c, pt, ctx, nq, nkv, d, d ** -0.5)
    y_ref = q4.gemv(pw, att.reshape(-1))
    assert np.array_equal(host_u16(y), host_u16(y_ref)), f"fused differs from unfused ({nq}x{d}, ctx {ctx})"


def test_attention_oproj_against_oracle(q4, orc):
    """y against the oracle's attention rounded to f16 and its matmul: the
    matmul bound plus the attention bound (and one f16 step of x) carried
    through |W|."""
    rng = np.random.default_rng(77)
    nq = nkv = 32
    d, n, ctx = 96, 3072, 777
    cache, table = make_cache(rng, ctx, nkv, d)
    qh = si.f16_bits(rng.normal(0.0, 1.0, (nq, d)))
    w, s = si.draw_weight(rng, n, nq * d)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    y = q4.attention_oproj(dev_f16(qh.reshape(-1)), torch.from_numpy(cache.view(np.float16)).cuda(),
                           torch.from_numpy(table).cuda(), ctx, nq, d ** -0.5, pw)
    att, a_att = orc.attention_decode(qh, cache, table, ctx, nq, nkv, d, d ** -0.5)
    x16 = orc.doubles_to_halves(att.reshape(-1))
    y_ref, a_ref = orc.gemv(w, s, x16)
    t_x = 2e-3 * np.abs(att) + 1e-3 * a_att + 1e-5 + 2.0 ** -10 * np.abs(att)
    _, carried = orc.gemv(w, s, si.f16_bits(t_x.reshape(-1) * 1.01))
    assert_within(host_f16_as_f64(y), y_ref, tol_f16(y_ref, a_ref) + carried, "attention + O-proj")

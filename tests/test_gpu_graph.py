"""Replaying the ops from a HIP graph: every replay must equal the eager
result bit for bit, with eager work and synchronisation between replays
(including the LM-head argmax's second launch); the GEMV family, the decode
step's ops, and the GEMM kernels and int3 ops."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import dev_f16, dev_u16, dev_u32

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(q4):
    rng = np.random.default_rng(12)
    x = dev_f16(si.draw_x(rng, 3072))
    w = q4.pack(*[f(a) for f, a in zip((dev_u32, dev_u16), si.draw_weight(rng, 9216, 3072))])
    g, u = si.draw_weight(rng, 8192, 3072), si.draw_weight(rng, 8192, 3072)
    gu = q4.pack_gate_up(dev_u32(g[0]), dev_u16(g[1]), dev_u32(u[0]), dev_u16(u[1]))
    d = q4.pack(*[f(a) for f, a in zip((dev_u32, dev_u16), si.draw_weight(rng, 3072, 8192))])
    lm = q4.pack(*[f(a) for f, a in zip((dev_u32, dev_u16), si.draw_weight(rng, 32064, 3072))])
    y = torch.empty(9216, dtype=torch.float16, device="cuda")
    h = torch.empty(8192, dtype=torch.float16, device="cuda")
    yd = torch.empty(3072, dtype=torch.float16, device="cuda")
    logits = torch.empty(32064, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(q4.lib.q4_workspace_bytes(q4.OP_LMHEAD, 1, 32064, 3072), dtype=torch.uint8,
                     device="cuda")

    def run():
        q4.gemv(w, x, y)
        q4.ffn_gate_up_silu(gu, x, h)
        q4.gemv(d, h, yd)
        q4.lmhead_f32(lm, x, logits, am, ws=ws)

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y, h, yd, logits, am)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(4):
        for t in (y, h, yd, logits, am):
            t.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "h", "down", "logits", "argmax"), eager, (y, h, yd, logits, am)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from eager"


def test_graph_replays_decode_layer_ops(q4):
    """The decode-step ops around the matmul replayed from one graph: add +
    RMSNorm + QKV + RoPE + f16 append, the int8 append, attention over both
    caches (two launches each), an int3 GEMV; every replay equal to eager,
    with the caches reset between replays."""
    rng = np.random.default_rng(13)
    nq = nkv = 32
    d, k, ctx = 96, 3072, 700
    n = (nq + 2 * nkv) * d
    w, s = si.draw_weight(rng, n, k)
    pw = q4.pack_rope(dev_u32(w), dev_u16(s), d)
    w3, s3 = si.draw_weight3(rng, 3072, 3072)
    p3 = q4.pack_int3(dev_u32(w3), dev_u16(s3))
    x = dev_f16(si.draw_x(rng, k))
    r = dev_f16(si.draw_x(rng, k))
    gamma = dev_f16(si.f16_bits(rng.uniform(0.5, 1.5, k)))
    pages = (ctx + 15) // 16 + 1
    pt = torch.from_numpy(rng.permutation(pages)[: pages - 1].astype(np.int32)).cuda()
    cache0 = torch.randn((pages, 2, nkv, 16, d), device="cuda").to(torch.float16)
    pb8 = q4.kv_int8_page_bytes(nkv, d)
    cache80 = torch.randint(0, 256, (pages, pb8), dtype=torch.uint8, device="cuda")
    cache80.view(pages, 2, nkv, 16 * d + 64)[:, :, :, 16 * d:].copy_(
        torch.full((pages, 2, nkv, 16), 0.01, device="cuda").view(torch.uint8))
    cache, cache8 = cache0.clone(), cache80.clone()
    qkv = torch.empty(n, dtype=torch.float16, device="cuda")
    hres = torch.empty(k, dtype=torch.float16, device="cuda")
    att = torch.empty((nq, d), dtype=torch.float16, device="cuda")
    att8 = torch.empty((nq, d), dtype=torch.float16, device="cuda")
    y3 = torch.empty(3072, dtype=torch.float16, device="cuda")
    ws = torch.zeros(q4.lib.q4_workspace_bytes(q4.OP_ATTENTION, ctx, nq, d), dtype=torch.uint8,
                     device="cuda")
    ws8 = torch.zeros_like(ws)
    pos = ctx - 1

    def run():
        q4.qkv_rope_append(pw, x, nq, pos, 10000.0, cache, pt, out=qkv,
                           norm=(r, gamma, 1e-5, hres))
        q4.kv_append_int8(qkv, nq, nkv, d, pos, cache8, pt)
        q4.attention_decode(qkv[: nq * d], cache, pt, ctx, nq, d ** -0.5, out=att, ws=ws)
        q4.attention_decode_int8(qkv[: nq * d], cache8, pt, ctx, nq, nkv, d, d ** -0.5, out=att8,
                                 ws=ws8)
        q4.gemv(p3, x, y3)

    outs = (qkv, hres, att, att8, y3, cache, cache8)
    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    cache.copy_(cache0)
    cache8.copy_(cache80)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    names = ("qkv", "residual", "attention", "attention int8", "int3 gemv", "cache", "int8 cache")
    for rep in range(4):
        for t in outs[:5]:
            t.zero_()                      # eager work between replays
        cache.copy_(cache0)
        cache8.copy_(cache80)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, eager, outs):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from eager"


def test_graph_replays_gemm_and_int3(q4):
    """The GEMM on each of its kernels (GEMV at m = 1, VALU at m = 3, small
    and tiled MFMA at m = 8, 100, 256), int4 and int3, and the int3 FFN, LM
    head (two launches) and multi-pass GEMV, replayed from one graph: every
    replay equal to eager."""
    rng = np.random.default_rng(14)
    k = 3072
    w, s = si.draw_weight(rng, 4096, k)
    pw = q4.pack(dev_u32(w), dev_u16(s))
    w3, s3 = si.draw_weight3(rng, 4096, k)
    p3 = q4.pack_int3(dev_u32(w3), dev_u16(s3))
    g3, gs3 = si.draw_weight3(rng, 2048, k)
    u3, us3 = si.draw_weight3(rng, 2048, k)
    gu3 = q4.pack_int3_gate_up(dev_u32(g3), dev_u16(gs3), dev_u32(u3), dev_u16(us3))
    l3, ls3 = si.draw_weight3(rng, 5003, k)
    lm3 = q4.pack_int3(dev_u32(l3), dev_u16(ls3))
    mp3w, mp3s = si.draw_weight3(rng, 777, 16384)
    mp3 = q4.pack_int3(dev_u32(mp3w), dev_u16(mp3s))
    X = dev_f16(si.draw_X(rng, 256, k))
    x = X[0].contiguous()
    xl = dev_f16(si.draw_x(rng, 16384))
    ms = (1, 3, 8, 100, 256)
    Ys = {(m, f): torch.empty((m, 4096), dtype=torch.float16, device="cuda") for m in ms for f in (4, 3)}
    h3 = torch.empty(2048, dtype=torch.float16, device="cuda")
    logits = torch.empty(5003, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(q4.lib.q4_workspace_bytes(q4.OP_LMHEAD, 1, 5003, k), dtype=torch.uint8,
                     device="cuda")
    ymp = torch.empty(777, dtype=torch.float16, device="cuda")

    def run():
        for m in ms:
            q4.gemm(pw, X[:m], Ys[(m, 4)])
            q4.gemm(p3, X[:m], Ys[(m, 3)])
        q4.ffn_gate_up_silu(gu3, x, h3)
        q4.lmhead_f32(lm3, x, logits, am, ws=ws)
        q4.gemv(mp3, xl, ymp)

    outs = list(Ys.values()) + [h3, logits, am, ymp]
    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    names = [f"gemm m={m} int{f}" for (m, f) in Ys] + ["int3 ffn", "int3 logits", "int3 argmax",
                                                      "int3 multi-pass gemv"]
    for rep in range(4):
        for t in outs:
            t.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, eager, outs):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from eager"

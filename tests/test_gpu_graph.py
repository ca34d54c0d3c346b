"""Replaying the ops from a HIP graph: every replay must equal the eager
result bit for bit, with eager work and synchronisation between replays
(including the LM-head argmax's second launch)."""
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

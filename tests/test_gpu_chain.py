"""q4_chain (several GEMV stages in one persistent launch) against the
oracle: each stage's output is checked on the inputs that stage actually
read (stage-wise), so a dependent stage is judged on the GPU's own output of
the stage it reads.  Also: repeated calls on one workspace (the per-block
launch counter), HIP-graph replays, every geometry the chain kernel has, and
the stage-only waits ("after")."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from parity import (assert_within, dev_f16, dev_u16, dev_u32, host_f16_as_f64, host_u16,
                    tol_f16, tol_ffn)

pytestmark = pytest.mark.gpu


def pack(q4, w):
    return q4.pack(dev_u32(w[0]), dev_u16(w[1]))


def test_chain_layer_set(q4, orc):
    """The layer set's four GEMVs in one launch, gate_up after O-proj and
    down after gate_up; each against the oracle and equal to q4_gemv where
    the chain computes a tile the way the block kernel does."""
    inp = si.workload(si.LAYER_SET, seed=0)
    W = {key: pack(q4, inp[key]) for key in si.LAYER_SHAPES}
    x3, x8 = dev_f16(inp["x3072"]), dev_f16(inp["x8192"])
    xin = {"qkv": x3, "o_proj": x3, "gate_up": x3, "down": x8}
    xh = {"qkv": inp["x3072"], "o_proj": inp["x3072"], "gate_up": inp["x3072"], "down": inp["x8192"]}
    stages = [q4.Stage(W["qkv"], x=x3), q4.Stage(W["o_proj"], x=x3),
              q4.Stage(W["gate_up"], x=x3, after=1), q4.Stage(W["down"], x=x8, after=2)]
    outs = q4.chain(stages)
    torch.cuda.synchronize()
    assert q4.chain_error() == 0
    for key, y in zip(si.LAYER_SHAPES, outs):
        ref, a = orc.gemv(*inp[key], xh[key])
        assert_within(host_f16_as_f64(y), ref, tol_f16(ref, a), f"chain {key}")
        if key != "down":   # k = 3072: the block kernel's tile arithmetic
            assert np.array_equal(host_u16(y), host_u16(q4.gemv(W[key], xin[key]))), key


def test_chain_decode_mlp(q4, orc):
    """O-proj -> residual add + RMSNorm -> gate/up + SiLU -> down, each stage
    reading the previous one's output (src), stage-wise against the oracle."""
    rng = np.random.default_rng(21)
    o_w, down_w = si.draw_weight(rng, 3072, 3072), si.draw_weight(rng, 3072, 8192)
    g, u = si.draw_weight(rng, 8192, 3072), si.draw_weight(rng, 8192, 3072)
    x = si.draw_x(rng, 3072)
    r = si.f16_bits(rng.normal(0.0, 2.0, 3072))
    gamma = si.f16_bits(rng.uniform(0.5, 1.5, 3072))
    gu = q4.pack_gate_up(dev_u32(g[0]), dev_u16(g[1]), dev_u32(u[0]), dev_u16(u[1]))
    hres = torch.empty(3072, dtype=torch.float16, device="cuda")
    stages = [q4.Stage(pack(q4, o_w), x=dev_f16(x)),
              q4.Stage(gu, src=0, residual=dev_f16(r), gamma=dev_f16(gamma), eps=1e-5, residual_out=hres),
              q4.Stage(pack(q4, down_w), src=1)]
    o, h, y = q4.chain(stages)
    torch.cuda.synchronize()
    assert q4.chain_error() == 0
    o_ref, a = orc.gemv(*o_w, x)
    assert_within(host_f16_as_f64(o), o_ref, tol_f16(o_ref, a), "o")
    h_ref, xn = orc.add_rmsnorm(host_u16(o), r, gamma, 1e-5)
    assert np.array_equal(host_u16(hres), h_ref), "residual out"
    ref = orc.ffn_gate_up_silu(*g, *u, xn)
    assert_within(host_f16_as_f64(h), ref["h"], tol_ffn(ref), "gate/up SiLU")
    y_ref, a = orc.gemv(*down_w, host_u16(h))
    assert_within(host_f16_as_f64(y), y_ref, tol_f16(y_ref, a), "down")


def test_chain_repeats_and_graph(q4):
    """Calls on one workspace (the launch counter advances) give the same
    bits, eagerly and from HIP-graph replays with eager work between them."""
    rng = np.random.default_rng(22)
    x = dev_f16(si.draw_x(rng, 3072))
    w1, w2 = pack(q4, si.draw_weight(rng, 3072, 3072)), pack(q4, si.draw_weight(rng, 4992, 3072))
    w3 = pack(q4, si.draw_weight(rng, 777, 4992))
    stages = [q4.Stage(w1, x=x), q4.Stage(w2, src=0), q4.Stage(w3, src=1)]
    first = [t.clone() for t in q4.chain(stages)]
    for _ in range(6):
        q4.chain(stages)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b.out) for a, b in zip(first, stages))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q4.chain(stages)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        q4.chain(stages)
        q4.chain(stages)
    for rep in range(4):
        for st in stages:
            st.out.zero_()
        q4.chain(stages)                  # an eager call between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, st) in enumerate(zip(first, stages)):
            assert torch.equal(a, st.out), f"replay {rep}, stage {i}"
    assert q4.chain_error() == 0


@pytest.mark.parametrize("k", [1568, 2048, 3072, 4096, 5120, 6176, 8192])
def test_chain_geometries(q4, orc, k):
    """Every geometry of the chain kernel, with ragged row counts, a given x,
    a dependent x (k rows feeding the next stage) and a stage-only wait."""
    rng = np.random.default_rng(k)
    x = si.draw_x(rng, k)
    wa = si.draw_weight(rng, k, k)          # k rows: its output is the next x
    wb = si.draw_weight(rng, 131, k)
    wc = si.draw_weight(rng, 70, k)
    stages = [q4.Stage(pack(q4, wa), x=dev_f16(x)), q4.Stage(pack(q4, wb), src=0),
              q4.Stage(pack(q4, wc), x=dev_f16(x), after=1)]
    ya, yb, yc = q4.chain(stages)
    torch.cuda.synchronize()
    assert q4.chain_error() == 0
    ref, a = orc.gemv(*wa, x)
    assert_within(host_f16_as_f64(ya), ref, tol_f16(ref, a), f"k={k} stage 0")
    ref, a = orc.gemv(*wb, host_u16(ya))
    assert_within(host_f16_as_f64(yb), ref, tol_f16(ref, a), f"k={k} stage 1")
    ref, a = orc.gemv(*wc, x)
    assert_within(host_f16_as_f64(yc), ref, tol_f16(ref, a), f"k={k} stage 2")


def test_chain_rejects_before_launch(q4):
    rng = np.random.default_rng(23)
    x = dev_f16(si.draw_x(rng, 3072))
    w = pack(q4, si.draw_weight(rng, 64, 3072))
    small = pack(q4, si.draw_weight(rng, 64, 1024))   # k = 1024: no chain geometry
    with pytest.raises(q4.Q4Error):
        q4.chain([q4.Stage(small, x=dev_f16(si.draw_x(rng, 1024)))])
    with pytest.raises(q4.Q4Error):   # src must name an earlier stage whose n equals k
        q4.chain([q4.Stage(w, x=x), q4.Stage(w, src=0)])
    with pytest.raises(q4.Q4Error):   # a stage cannot wait for itself
        q4.chain([q4.Stage(w, x=x, after=0)])

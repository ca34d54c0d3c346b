"""The C ABI on the CPU (no GPU needed, nothing is launched): the library
loads and exports every function include/q4.h declares; the host geometry
agrees with the oracle's; every documented error code comes back, from the
host-side validation, before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")


@pytest.fixture(scope="module")
def q4():
    import int4_quantized_decode_q4_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(q4_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(q4):
    names = declared_functions()
    assert len(names) >= 12, names
    lib = ctypes.CDLL(q4.LIBRARY)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


SHAPES = [(3072, 3072), (3072, 8192), (32064, 3072), (1, 32), (17, 96), (130, 64), (33, 224),
          (7, 160), (6, 192), (3, 3200), (5, 16384), (3, 8352), (4, 16480), (999, 544),
          (2, 2048), (10, 12288), (1, 65536)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_host_geometry_matches_oracle(q4, orc, n, k):
    assert q4.layout_geometry(n, k) == orc.layout_geometry(n, k)
    assert q4.packed_bytes(n, k) == orc.layout_bytes(n, k)
    assert q4.packed_bytes(n, k, q4.LAYOUT_GATE_UP) == orc.layout_bytes(2 * n, k)


@pytest.mark.parametrize("n,k", [(3072, 3072), (3072, 8192), (1, 32), (17, 96), (130, 64),
                                 (33, 224), (999, 544), (5, 7168), (64, 8224), (3, 16384),
                                 (5, 24608)])
def test_int3_packed_bytes_matches_oracle(q4, orc, n, k):
    assert q4.packed_bytes(n, k, q4.LAYOUT_INT3) == orc.lib.q4o_layout3_bytes(n, k)


def test_int3_errors(q4, orc):
    lib = q4.lib
    out = q4.q4_weight()
    r = ctypes.byref(out)
    W, S, D = A, A + 0x10000, A + 0x100000
    nb = q4.packed_bytes(64, 96, q4.LAYOUT_INT3)
    nb2 = q4.packed_bytes(64, 8224, q4.LAYOUT_INT3)   # two passes
    assert nb > 0 and nb2 == orc.lib.q4o_layout3_bytes(64, 8224) > nb
    f = lib.q4_pack_int3
    assert f(None, S, 64, 96, D, nb, r, None) == q4.ERR_NULL
    assert f(W, S, 64, 96, D, nb, None, None) == q4.ERR_NULL
    assert f(W, S, 64, 100, D, nb, r, None) == q4.ERR_SHAPE
    assert f(W, S, 64, 8224, D, nb2 - 1, r, None) == q4.ERR_SIZE
    assert f(W + 2, S, 64, 96, D, nb, r, None) == q4.ERR_ALIGN
    assert f(W, S + 1, 64, 96, D, nb, r, None) == q4.ERR_ALIGN
    assert f(W, S, 64, 96, D + 16, nb, r, None) == q4.ERR_ALIGN
    assert f(W, S, 64, 96, D, nb - 1, r, None) == q4.ERR_SIZE
    assert f(W, S, 64, 96, W, nb, r, None) == q4.ERR_ALIAS
    assert out.data is None
    X, Y = A + 0x200000, A + 0x300000
    w3 = weight(q4, layout=q4.LAYOUT_INT3)
    assert lib.q4_gemv(ctypes.byref(weight(q4, layout=q4.LAYOUT_INT3, k=8224, nbytes=nb2 - 1)),
                       X, Y, None) == q4.ERR_SIZE
    assert lib.q4_gemv(ctypes.byref(weight(q4, layout=q4.LAYOUT_INT3, nbytes=nb - 1)), X, Y,
                       None) == q4.ERR_SIZE
    assert lib.q4_gemv(ctypes.byref(w3), X + 8, Y, None) == q4.ERR_ALIGN
    assert lib.q4_gemv(ctypes.byref(w3), X, X, None) == q4.ERR_ALIAS
    # the LM head and the GEMM take int3 rows (validated like int4); the FFN
    # and the norm / RoPE ops refuse them, and the gate/up layout is only for
    # the FFN
    assert lib.q4_lmhead_f32(ctypes.byref(w3), X, Y, A + 0x600000, None, 0, None) == q4.ERR_WORKSPACE
    assert lib.q4_lmhead_f32(ctypes.byref(w3), X, Y + 4, None, None, 0, None) == q4.ERR_ALIGN
    assert lib.q4_gemm(ctypes.byref(w3), X, 0, Y, None, 0, None) == q4.ERR_SHAPE
    assert lib.q4_gemm(ctypes.byref(w3), X + 8, 4, Y, None, 0, None) == q4.ERR_ALIGN
    assert lib.q4_gemm(ctypes.byref(weight(q4, layout=q4.LAYOUT_INT3, k=8224, nbytes=nb2 - 1)), X, 4, Y,
                       None, 0, None) == q4.ERR_SIZE
    assert lib.q4_add_rmsnorm_gemv(ctypes.byref(w3), X, None, A + 0x700000, 1e-5, None, Y,
                                   None) == q4.ERR_LAYOUT
    assert lib.q4_ffn_gate_up_silu(ctypes.byref(w3), X, Y, None) == q4.ERR_LAYOUT
    assert lib.q4_unpack(ctypes.byref(w3), W + 2, S, None) == q4.ERR_ALIGN
    g3 = weight(q4, layout=q4.LAYOUT_INT3_GATE_UP)
    assert g3.bytes == q4.packed_bytes(64, 96, q4.LAYOUT_INT3_GATE_UP) == orc.lib.q4o_layout3_bytes(128, 96)
    assert lib.q4_gemv(ctypes.byref(g3), X, Y, None) == q4.ERR_LAYOUT
    assert lib.q4_lmhead_f32(ctypes.byref(g3), X, Y, None, None, 0, None) == q4.ERR_LAYOUT
    assert lib.q4_ffn_gate_up_silu(ctypes.byref(g3), X + 8, Y, None) == q4.ERR_ALIGN
    assert lib.q4_ffn_gate_up_silu(ctypes.byref(weight(q4, layout=q4.LAYOUT_INT3_GATE_UP,
                                                        nbytes=g3.bytes - 1)), X, Y, None) == q4.ERR_SIZE
    fg = lib.q4_pack_int3_gate_up
    nbg = g3.bytes
    assert fg(W, S, None, S, 64, 96, D, nbg, r, None) == q4.ERR_NULL
    assert fg(W, S, W, S, 64, 8224, D, q4.packed_bytes(64, 8224, q4.LAYOUT_INT3_GATE_UP) - 1, r,
              None) == q4.ERR_SIZE
    assert fg(W, S, W + 2, S, 64, 96, D, nbg, r, None) == q4.ERR_ALIGN
    assert fg(W, S, W, S, 64, 96, D, nbg - 1, r, None) == q4.ERR_SIZE
    assert fg(W, S, D, S, 64, 96, D, nbg, r, None) == q4.ERR_ALIAS
    assert out.data is None


def test_packed_bytes_invalid(q4):
    assert q4.packed_bytes(0, 32) == 0
    assert q4.packed_bytes(1, 48) == 0
    assert q4.packed_bytes(1, 16) == 0
    assert q4.packed_bytes(-5, 64) == 0
    assert q4.packed_bytes(4, 64, 7) == 0


# fake device addresses: validation rejects the call before anything uses them
A = 0x7f0000000000


def weight(q4, n=64, k=96, layout=1, version=1, data=A + 0x100000, nbytes=None):
    w = q4.q4_weight()
    w.n, w.k, w.layout, w.version = n, k, layout, version
    w.data = data
    w.bytes = q4.packed_bytes(n, k, layout) if nbytes is None else nbytes
    return w


def test_pack_errors(q4):
    lib = q4.lib
    out = q4.q4_weight()
    nb = q4.packed_bytes(64, 96)
    r = ctypes.byref(out)
    W, S, D = A, A + 0x10000, A + 0x100000
    assert lib.q4_pack(None, S, 64, 96, D, nb, r, None) == q4.ERR_NULL
    assert lib.q4_pack(W, S, 64, 96, D, nb, None, None) == q4.ERR_NULL
    assert lib.q4_pack(W, S, 0, 96, D, nb, r, None) == q4.ERR_SHAPE
    assert lib.q4_pack(W, S, 64, 100, D, nb, r, None) == q4.ERR_SHAPE
    assert lib.q4_pack(W, S, 64, 16, D, nb, r, None) == q4.ERR_SHAPE
    assert lib.q4_pack(W + 4, S, 64, 96, D, nb, r, None) == q4.ERR_ALIGN
    assert lib.q4_pack(W, S + 1, 64, 96, D, nb, r, None) == q4.ERR_ALIGN
    assert lib.q4_pack(W, S, 64, 96, D + 16, nb, r, None) == q4.ERR_ALIGN
    assert lib.q4_pack(W, S, 64, 96, D, nb - 1, r, None) == q4.ERR_SIZE
    assert lib.q4_pack(W, S, 64, 96, W, nb, r, None) == q4.ERR_ALIAS
    assert lib.q4_pack_gate_up(W, S, None, S, 64, 96, D, 10 ** 9, r, None) == q4.ERR_NULL
    nb3 = q4.packed_bytes(64, 3072)
    assert lib.q4_pack_gate_up(W, S, W, S, 64, 3072, D, nb3, r, None) == q4.ERR_SIZE
    assert out.data is None   # nothing was written to the descriptor


def test_gemv_family_errors(q4):
    lib = q4.lib
    X, Y = A + 0x200000, A + 0x300000
    w = weight(q4)
    r = ctypes.byref(w)
    assert lib.q4_gemv(None, X, Y, None) == q4.ERR_NULL
    assert lib.q4_gemv(r, None, Y, None) == q4.ERR_NULL
    assert lib.q4_gemv(r, X, None, None) == q4.ERR_NULL
    assert lib.q4_gemv(ctypes.byref(weight(q4, data=None)), X, Y, None) == q4.ERR_NULL
    assert lib.q4_gemv(ctypes.byref(weight(q4, k=100)), X, Y, None) == q4.ERR_SHAPE
    assert lib.q4_gemv(ctypes.byref(weight(q4, n=0)), X, Y, None) == q4.ERR_SHAPE
    assert lib.q4_gemv(ctypes.byref(weight(q4, layout=2)), X, Y, None) == q4.ERR_LAYOUT
    assert lib.q4_gemv(ctypes.byref(weight(q4, version=2)), X, Y, None) == q4.ERR_LAYOUT
    assert lib.q4_gemv(ctypes.byref(weight(q4, data=A + 0x100010)), X, Y, None) == q4.ERR_ALIGN
    assert lib.q4_gemv(ctypes.byref(weight(q4, nbytes=100)), X, Y, None) == q4.ERR_SIZE
    assert lib.q4_gemv(r, X + 8, Y, None) == q4.ERR_ALIGN
    assert lib.q4_gemv(r, X, Y + 2, None) == q4.ERR_ALIGN
    assert lib.q4_gemv(r, X, X + 64, None) == q4.ERR_ALIAS
    assert lib.q4_gemv(r, X, A + 0x100000 + 512, None) == q4.ERR_ALIAS
    # gemm
    assert lib.q4_gemm(r, X, 0, Y, None, 0, None) == q4.ERR_SHAPE
    assert lib.q4_gemm(r, X, 4, X + 256, None, 0, None) == q4.ERR_ALIAS
    assert lib.q4_gemm(r, X + 2, 4, Y, None, 0, None) == q4.ERR_ALIGN
    # fused FFN wants the gate/up layout
    assert lib.q4_ffn_gate_up_silu(r, X, Y, None) == q4.ERR_LAYOUT
    gu = weight(q4, layout=2)
    assert lib.q4_ffn_gate_up_silu(ctypes.byref(gu), X, X, None) == q4.ERR_ALIAS
    assert lib.q4_ffn_gate_up_silu(ctypes.byref(gu), X, Y + 1, None) == q4.ERR_ALIGN


def test_add_rmsnorm_errors(q4):
    lib = q4.lib
    X, R, Gm, H, Y = A + 0x200000, A + 0x210000, A + 0x220000, A + 0x230000, A + 0x300000
    w = weight(q4)
    r = ctypes.byref(w)
    f = lib.q4_add_rmsnorm_gemv
    assert f(None, X, R, Gm, 1e-5, H, Y, None) == q4.ERR_NULL
    assert f(r, None, R, Gm, 1e-5, H, Y, None) == q4.ERR_NULL
    assert f(r, X, R, None, 1e-5, H, Y, None) == q4.ERR_NULL
    assert f(r, X, R, Gm, 1e-5, H, None, None) == q4.ERR_NULL
    assert f(r, X, R, Gm, -1.0, H, Y, None) == q4.ERR_SHAPE
    assert f(r, X, R, Gm, float("nan"), H, Y, None) == q4.ERR_SHAPE
    assert f(r, X, R, Gm, float("inf"), H, Y, None) == q4.ERR_SHAPE
    assert f(r, X + 8, R, Gm, 1e-5, H, Y, None) == q4.ERR_ALIGN
    assert f(r, X, R + 8, Gm, 1e-5, H, Y, None) == q4.ERR_ALIGN
    assert f(r, X, R, Gm + 2, 1e-5, H, Y, None) == q4.ERR_ALIGN
    assert f(r, X, R, Gm, 1e-5, H + 8, Y, None) == q4.ERR_ALIGN
    assert f(r, X, R, Gm, 1e-5, H, Y + 2, None) == q4.ERR_ALIGN
    assert f(r, X, R, Gm, 1e-5, R, Y, None) == q4.ERR_ALIAS        # residual updated in place
    assert f(r, X, R, Gm, 1e-5, H, Gm + 64, None) == q4.ERR_ALIAS  # y over gamma
    assert f(r, X, R, Gm, 1e-5, H, H + 64, None) == q4.ERR_ALIAS   # the two outputs
    assert f(r, X, R, Gm, 1e-5, X + 32, Y, None) == q4.ERR_ALIAS   # residual_out over x
    assert f(ctypes.byref(weight(q4, layout=2)), X, R, Gm, 1e-5, H, Y, None) == q4.ERR_LAYOUT
    g = lib.q4_add_rmsnorm_ffn_gate_up_silu
    gu = ctypes.byref(weight(q4, layout=2))
    assert g(r, X, R, Gm, 1e-5, H, Y, None) == q4.ERR_LAYOUT
    assert g(gu, X, R, Gm, -0.5, H, Y, None) == q4.ERR_SHAPE
    assert g(gu, X, R, Gm, 1e-5, H, Y + 1, None) == q4.ERR_ALIGN
    assert g(gu, X, R, Gm, 1e-5, H, X, None) == q4.ERR_ALIAS


def rope_weight(q4, n=96, k=96, head_dim=8, **kw):
    w = weight(q4, n=n, k=k, layout=3, **kw)
    w.head_dim = head_dim
    return w


def test_rope_errors(q4):
    lib = q4.lib
    X, Y, C, T = A + 0x200000, A + 0x300000, A + 0x400000, A + 0x500000
    W0, S0, D = A + 0x600000, A + 0x700000, A + 0x800000
    out = q4.q4_weight()
    pr = lib.q4_pack_rope
    nb = q4.packed_bytes(96, 96, q4.LAYOUT_ROPE)
    assert nb == q4.packed_bytes(96, 96)
    assert pr(W0, S0, 96, 96, 7, D, nb, ctypes.byref(out), None) == q4.ERR_SHAPE   # odd
    assert pr(W0, S0, 96, 96, 0, D, nb, ctypes.byref(out), None) == q4.ERR_SHAPE
    assert pr(W0, S0, 96, 96, 64, D, nb, ctypes.byref(out), None) == q4.ERR_SHAPE  # 64 !| 96
    assert pr(None, S0, 96, 96, 8, D, nb, ctypes.byref(out), None) == q4.ERR_NULL
    assert pr(W0, S0, 96, 96, 8, D, nb - 1, ctypes.byref(out), None) == q4.ERR_SIZE
    w = rope_weight(q4)
    r = ctypes.byref(w)
    f = lib.q4_qkv_rope_append
    # 96 rows = 12 heads of 8: 4 q + 4 k + 4 v
    assert f(ctypes.byref(weight(q4, n=96)), X, 4, 0, 1e4, Y, C, T, 2, None) == q4.ERR_LAYOUT
    assert f(ctypes.byref(rope_weight(q4, head_dim=7)), X, 4, 0, 1e4, Y, C, T, 2, None) == q4.ERR_SHAPE
    assert f(ctypes.byref(rope_weight(q4, head_dim=64)), X, 4, 0, 1e4, Y, C, T, 2, None) == q4.ERR_SHAPE
    assert f(r, X, 5, 0, 1e4, Y, C, T, 2, None) == q4.ERR_SHAPE      # 7 k/v heads: odd
    assert f(r, X, 13, 0, 1e4, Y, C, T, 2, None) == q4.ERR_SHAPE     # more q heads than heads
    assert f(r, X, -1, 0, 1e4, Y, C, T, 2, None) == q4.ERR_SHAPE
    assert f(r, X, 4, -1, 1e4, Y, C, T, 2, None) == q4.ERR_SHAPE
    assert f(r, X, 4, 0, 0.0, Y, C, T, 2, None) == q4.ERR_SHAPE
    assert f(r, X, 4, 0, float("nan"), Y, C, T, 2, None) == q4.ERR_SHAPE
    assert f(r, X, 4, 0, 1e4, Y, C, T, 0, None) == q4.ERR_SHAPE      # a cache of no pages
    assert f(r, X, 4, 0, 1e4, Y, C, None, 2, None) == q4.ERR_NULL    # a cache needs a table
    assert f(r, None, 4, 0, 1e4, Y, C, T, 2, None) == q4.ERR_NULL
    assert f(r, X, 4, 0, 1e4, None, C, T, 2, None) == q4.ERR_NULL
    assert f(r, X + 8, 4, 0, 1e4, Y, C, T, 2, None) == q4.ERR_ALIGN
    assert f(r, X, 4, 0, 1e4, Y + 2, C, T, 2, None) == q4.ERR_ALIGN
    assert f(r, X, 4, 0, 1e4, Y, C + 2, T, 2, None) == q4.ERR_ALIGN
    assert f(r, X, 4, 0, 1e4, X + 64, C, T, 2, None) == q4.ERR_ALIAS     # qkv over x
    assert f(r, X, 4, 0, 1e4, Y, Y + 64, T, 2, None) == q4.ERR_ALIAS     # cache over qkv
    assert f(r, X, 4, 0, 1e4, Y, C, C + 64, 2, None) == q4.ERR_ALIAS     # table inside cache
    g = lib.q4_add_rmsnorm_qkv_rope_append
    Gm = A + 0x220000
    assert g(r, X, None, None, 1e-5, None, 4, 0, 1e4, Y, C, T, 2, None) == q4.ERR_NULL
    assert g(r, X, None, Gm, -1.0, None, 4, 0, 1e4, Y, C, T, 2, None) == q4.ERR_SHAPE
    assert g(r, X, None, Gm, 1e-5, None, 4, 0, 1e4, Y, Gm + 32, T, 2, None) == q4.ERR_ALIAS
    # the other ops refuse the rotary-paired layout
    assert lib.q4_gemv(r, X, Y, None) == q4.ERR_LAYOUT


def test_attention_errors(q4):
    lib = q4.lib
    Q, C, T, O, Wk = A + 0x200000, A + 0x1000000, A + 0x300000, A + 0x400000, A + 0x500000
    f = lib.q4_attention_decode
    need = lib.q4_workspace_bytes(q4.OP_ATTENTION, 4096, 32, 96)
    # one (max, sum, d sums) f32 record per head and chunk, chunks of >= 64 positions
    assert need > 0 and need % (32 * (96 + 2) * 4) == 0 and need <= 32 * 64 * (96 + 2) * 4
    assert lib.q4_workspace_bytes(q4.OP_ATTENTION, 64, 32, 96) == 0    # one chunk: none
    ok = (Q, C, T, 300, 4096, 32, 32, 96, 0.1, O, Wk, need, None)
    def call(**kw):
        names = ("q", "c", "t", "pages", "ctx", "nq", "nkv", "d", "scale", "o", "ws", "wsb", "s")
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])
    assert call(q=None) == q4.ERR_NULL
    assert call(c=None) == q4.ERR_NULL
    assert call(t=None) == q4.ERR_NULL
    assert call(o=None) == q4.ERR_NULL
    assert call(ctx=0) == q4.ERR_SHAPE
    assert call(pages=0) == q4.ERR_SHAPE
    assert call(nq=30, nkv=4) == q4.ERR_SHAPE        # nq % nkv
    assert call(d=80) == q4.ERR_SHAPE                # not a multiple of 32
    assert call(d=288) == q4.ERR_SHAPE
    assert call(scale=float("inf")) == q4.ERR_SHAPE
    assert call(q=Q + 8) == q4.ERR_ALIGN
    assert call(c=C + 8) == q4.ERR_ALIGN
    assert call(o=O + 2) == q4.ERR_ALIGN
    assert call(ws=None) == q4.ERR_WORKSPACE
    assert call(wsb=need - 4) == q4.ERR_WORKSPACE
    assert call(o=Q + 64) == q4.ERR_ALIAS            # out over q
    assert call(o=C + 4096) == q4.ERR_ALIAS          # out inside the cache
    assert call(ws=O) == q4.ERR_ALIAS                # workspace over out


def test_kv_int8_errors(q4, orc):
    lib = q4.lib
    assert lib.q4_kv_int8_page_bytes(32, 96) == orc.kv8_page_bytes(32, 96) == 102400
    for nkv, d in ((0, 96), (32, 100), (32, 288), (32, 16)):
        assert lib.q4_kv_int8_page_bytes(nkv, d) == 0
    QKV, C, T = A + 0x200000, A + 0x1000000, A + 0x300000
    f = lib.q4_kv_append_int8
    assert f(None, 32, 32, 96, 0, C, T, 4, None) == q4.ERR_NULL
    assert f(QKV, 32, 32, 96, 0, None, T, 4, None) == q4.ERR_NULL
    assert f(QKV, 32, 32, 96, 0, C, None, 4, None) == q4.ERR_NULL
    assert f(QKV, 32, 32, 100, 0, C, T, 4, None) == q4.ERR_SHAPE
    assert f(QKV, 0, 32, 96, 0, C, T, 4, None) == q4.ERR_SHAPE
    assert f(QKV, 32, 32, 96, -1, C, T, 4, None) == q4.ERR_SHAPE
    assert f(QKV, 32, 32, 96, 0, C, T, 0, None) == q4.ERR_SHAPE
    assert f(QKV + 1, 32, 32, 96, 0, C, T, 4, None) == q4.ERR_ALIGN
    assert f(QKV, 32, 32, 96, 0, C + 8, T, 4, None) == q4.ERR_ALIGN
    assert f(QKV, 32, 32, 96, 0, C, T + 2, 4, None) == q4.ERR_ALIGN
    assert f(QKV, 32, 32, 96, 0, QKV, T, 4, None) == q4.ERR_ALIAS        # cache over qkv
    assert f(QKV, 32, 32, 96, 0, C, C + 64, 4, None) == q4.ERR_ALIAS     # table inside cache
    g = lib.q4_attention_decode_int8
    Q, O, Wk = A + 0x200000, A + 0x400000, A + 0x500000
    need = lib.q4_workspace_bytes(q4.OP_ATTENTION, 4096, 32, 96)
    ok = (Q, C, T, 300, 4096, 32, 32, 96, 0.1, O, Wk, need, None)
    def call(**kw):
        names = ("q", "c", "t", "pages", "ctx", "nq", "nkv", "d", "scale", "o", "ws", "wsb", "s")
        args = dict(zip(names, ok))
        args.update(kw)
        return g(*[args[n] for n in names])
    assert call(c=None) == q4.ERR_NULL
    assert call(o=None) == q4.ERR_NULL
    assert call(ctx=0) == q4.ERR_SHAPE
    assert call(d=80) == q4.ERR_SHAPE
    assert call(nq=30, nkv=4) == q4.ERR_SHAPE
    assert call(scale=float("nan")) == q4.ERR_SHAPE
    assert call(c=C + 8) == q4.ERR_ALIGN
    assert call(q=Q + 8) == q4.ERR_ALIGN
    assert call(ws=None) == q4.ERR_WORKSPACE
    assert call(o=C + 4096) == q4.ERR_ALIAS          # out inside the cache
    assert call(ws=O) == q4.ERR_ALIAS


def test_lmhead_errors(q4):
    lib = q4.lib
    X, L, I, WS = A + 0x200000, A + 0x300000, A + 0x400000, A + 0x500000
    w = weight(q4, n=32064, k=3072)
    r = ctypes.byref(w)
    need = lib.q4_workspace_bytes(q4.OP_LMHEAD, 1, 32064, 3072)
    assert need >= 8
    assert lib.q4_workspace_bytes(q4.OP_GEMV, 1, 32064, 3072) == 0
    assert lib.q4_lmhead_f32(r, X, None, I, WS, need, None) == q4.ERR_NULL
    assert lib.q4_lmhead_f32(r, X, L, I, None, 0, None) == q4.ERR_WORKSPACE
    assert lib.q4_lmhead_f32(r, X, L, I, WS, need - 1, None) == q4.ERR_WORKSPACE
    assert lib.q4_lmhead_f32(r, X, L, I, WS + 8, need, None) == q4.ERR_ALIGN
    assert lib.q4_lmhead_f32(r, X, L + 4, I, WS, need, None) == q4.ERR_ALIGN
    assert lib.q4_lmhead_f32(r, X, L, I + 2, WS, need, None) == q4.ERR_ALIGN
    assert lib.q4_lmhead_f32(r, X, L, WS + 8, WS, need, None) == q4.ERR_ALIAS
    assert lib.q4_lmhead_f32(r, X, L, L + 64, WS, need, None) == q4.ERR_ALIAS
    assert lib.q4_lmhead_f32(r, X, X, None, None, 0, None) == q4.ERR_ALIAS


def test_strerror_and_last_error(q4):
    lib = q4.lib
    texts = {c: lib.q4_strerror(c).decode() for c in range(-8, 1)}
    assert len(set(texts.values())) == 9 and all(texts.values())
    assert "unknown" in lib.q4_strerror(-99).decode()
    assert lib.q4_last_hip_error() == 0


def test_read_probe_errors(q4):
    lib = q4.lib
    S, K = A + 0x100000, A + 0x900000
    nb = 5320704
    assert lib.q4_read_probe(None, nb, K, 8192, None) == q4.ERR_NULL
    assert lib.q4_read_probe(S, nb, None, 8192, None) == q4.ERR_NULL
    assert lib.q4_read_probe(S, 0, K, 8192, None) == q4.ERR_SHAPE
    assert lib.q4_read_probe(S, nb + 8, K, 8192, None) == q4.ERR_SHAPE
    assert lib.q4_read_probe(S + 8, nb, K, 8192, None) == q4.ERR_ALIGN
    assert lib.q4_read_probe(S, nb, K + 2, 8192, None) == q4.ERR_ALIGN
    assert lib.q4_read_probe(S, nb, K, 4, None) == q4.ERR_SIZE       # one word, many blocks
    assert lib.q4_read_probe(S, nb, S + 4096, 8192, None) == q4.ERR_ALIAS


def test_chain_errors(q4):
    lib = q4.lib
    X, Y, Y2, WS = A + 0x4000000, A + 0x4100000, A + 0x4200000, A + 0x5000000
    w = weight(q4, n=3072, k=3072)
    w2 = weight(q4, n=512, k=3072, data=A + 0x2000000)
    small = weight(q4, n=64, k=1024, data=A + 0x3000000)

    def stages(*specs):
        arr = (q4.q4_chain_stage * len(specs))()
        for d, (wt, x, src, after, y) in zip(arr, specs):
            d.w = ctypes.pointer(wt)
            d.x, d.src, d.after, d.y = x, src, after, y
        return arr

    ok = stages((w, X, -1, -1, Y), (w2, None, 0, -1, Y2))
    need = lib.q4_chain_workspace_bytes(ok, 2)
    assert need > 0
    assert lib.q4_chain(ok, 2, WS, need, None) != q4.ERR_NULL   # valid up to the launch
    assert lib.q4_chain(None, 2, WS, need, None) == q4.ERR_NULL
    assert lib.q4_chain(ok, 0, WS, need, None) == q4.ERR_SHAPE
    assert lib.q4_chain(ok, 7, WS, need, None) == q4.ERR_SHAPE
    assert lib.q4_chain(ok, 2, None, 0, None) == q4.ERR_WORKSPACE
    assert lib.q4_chain(ok, 2, WS, need - 1, None) == q4.ERR_WORKSPACE
    assert lib.q4_chain(ok, 2, WS + 128, need, None) == q4.ERR_ALIGN
    assert lib.q4_chain(ok, 2, X, need, None) == q4.ERR_ALIAS
    assert lib.q4_chain(stages((w, None, -1, -1, Y),), 1, WS, need, None) == q4.ERR_NULL
    assert lib.q4_chain(stages((w, X, 0, -1, Y),), 1, WS, need, None) == q4.ERR_SHAPE    # src not earlier
    assert lib.q4_chain(stages((w, X, -1, 0, Y),), 1, WS, need, None) == q4.ERR_SHAPE    # after not earlier
    assert lib.q4_chain(stages((w2, X, -1, -1, Y), (w, None, 0, -1, Y2)), 2, WS, need, None) == q4.ERR_SHAPE  # n != k
    assert lib.q4_chain(stages((small, X, -1, -1, Y),), 1, WS, need, None) == q4.ERR_SHAPE   # k = 1024
    assert lib.q4_chain(stages((w, X + 8, -1, -1, Y),), 1, WS, need, None) == q4.ERR_ALIGN
    assert lib.q4_chain(stages((w, X, -1, -1, Y + 2),), 1, WS, need, None) == q4.ERR_ALIGN
    assert lib.q4_chain(stages((w, X, -1, -1, X),), 1, WS, need, None) == q4.ERR_ALIAS
    assert lib.q4_chain(stages((w, X, -1, -1, Y), (w2, None, 0, -1, Y)), 2, WS, need, None) == q4.ERR_ALIAS
    gu = weight(q4, n=3072, k=3072, layout=q4.LAYOUT_ROPE)
    assert lib.q4_chain(stages((gu, X, -1, -1, Y),), 1, WS, need, None) == q4.ERR_LAYOUT

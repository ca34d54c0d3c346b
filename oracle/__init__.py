"""CPU oracle for the int4 dequantizing matmul -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The library never does, and shares no code with it.

The arithmetic lives in ``q4_oracle.c`` (plain C, f64, one term at a time);
this module compiles it with gcc into ``liboracle.so`` beside the source and
wraps each entry point for numpy arrays.  See the C file's header for the
format definition and the page citations.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (exact rational brute force, closed forms, one-hot
inputs, identities, the numpy f16 codec, and the byte-level layout spec); the
mutation test in ``tests/test_oracle_mutants.py`` shows that plausible slips
in the C source fail those pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "q4_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(out: str = LIBRARY, source: str = SOURCE) -> str:
    """Compile the oracle with gcc; returns the library path."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


class Oracle:
    """numpy-facing wrapper around one loaded oracle library."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.q4o_half_to_double.argtypes = [ctypes.c_uint16]
        lib.q4o_half_to_double.restype = ctypes.c_double
        lib.q4o_double_to_half.argtypes = [ctypes.c_double]
        lib.q4o_double_to_half.restype = ctypes.c_uint16
        lib.q4o_gemv.argtypes = [_P, _P, _P, _I64, _I64, _P, _P]
        lib.q4o_gemv.restype = ctypes.c_int
        lib.q4o_kv_quant_row.argtypes = [_P, _I64, _P, _P]
        lib.q4o_kv_quant_row.restype = None
        lib.q4o_kv8_page_bytes.argtypes = [_I64, _I64]
        lib.q4o_kv8_page_bytes.restype = ctypes.c_int64
        lib.q4o_kv_append_int8.argtypes = [_P, _I64, _I64, _I64, _I64, _P, _P, _I64]
        lib.q4o_kv_append_int8.restype = ctypes.c_int
        lib.q4o_attention_decode_int8.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                                  ctypes.c_double, _P, _P]
        lib.q4o_attention_decode_int8.restype = ctypes.c_int
        lib.q4o_gemv3.argtypes = [_P, _P, _P, _I64, _I64, _P, _P]
        lib.q4o_gemv3.restype = ctypes.c_int
        lib.q4o_encode3.argtypes = [_P, _P, _I64, _I64, _P]
        lib.q4o_gemm3.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _P]
        lib.q4o_gemm3.restype = ctypes.c_int
        lib.q4o_encode3_gate_up.argtypes = [_P, _P, _P, _P, _I64, _I64, _P]
        lib.q4o_encode3_gate_up.restype = ctypes.c_int
        lib.q4o_ffn_gate_up_silu3.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _P]
        lib.q4o_ffn_gate_up_silu3.restype = ctypes.c_int
        lib.q4o_encode3.restype = ctypes.c_int
        lib.q4o_layout3_bytes.argtypes = [_I64, _I64]
        lib.q4o_layout3_bytes.restype = ctypes.c_int64
        lib.q4o_gemm.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P, _P]
        lib.q4o_gemm.restype = ctypes.c_int
        lib.q4o_silu.argtypes = [ctypes.c_double]
        lib.q4o_silu.restype = ctypes.c_double
        lib.q4o_ffn_gate_up_silu.argtypes = [_P, _P, _P, _P, _P, _I64, _I64,
                                             _P, _P, _P, _P, _P]
        lib.q4o_ffn_gate_up_silu.restype = ctypes.c_int
        lib.q4o_add_rmsnorm.argtypes = [_P, _P, _P, _I64, ctypes.c_double, _P, _P]
        lib.q4o_add_rmsnorm.restype = ctypes.c_int
        lib.q4o_rope_pair.argtypes = [ctypes.c_double, ctypes.c_double, _I64, _I64, _I64,
                                      ctypes.c_double, _P, _P]
        lib.q4o_rope_pair.restype = None
        lib.q4o_qkv_rope.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, ctypes.c_double,
                                     _P, _P]
        lib.q4o_qkv_rope.restype = ctypes.c_int
        lib.q4o_encode_rope.argtypes = [_P, _P, _I64, _I64, _I64, _P]
        lib.q4o_encode_rope.restype = ctypes.c_int
        lib.q4o_attention_decode.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                             ctypes.c_double, _P, _P]
        lib.q4o_attention_decode.restype = ctypes.c_int
        lib.q4o_argmax.argtypes = [_P, _I64]
        lib.q4o_argmax.restype = ctypes.c_int64
        lib.q4o_lmhead.argtypes = [_P, _P, _P, _I64, _I64, _P, _P]
        lib.q4o_lmhead.restype = ctypes.c_int64
        lib.q4o_layout_geometry.argtypes = [_I64, _I64, _P]
        lib.q4o_layout_geometry.restype = ctypes.c_int
        lib.q4o_layout_bytes.argtypes = [_I64, _I64]
        lib.q4o_layout_bytes.restype = ctypes.c_int64
        lib.q4o_encode_rows.argtypes = [_P, _P, _I64, _I64, _P]
        lib.q4o_encode_rows.restype = ctypes.c_int
        lib.q4o_encode_gate_up.argtypes = [_P, _P, _P, _P, _I64, _I64, _P]
        lib.q4o_encode_gate_up.restype = ctypes.c_int
        self.lib = lib

    # -- f16 codec -------------------------------------------------------
    def half_to_double(self, bits: int) -> float:
        return self.lib.q4o_half_to_double(int(bits))

    def double_to_half(self, v: float) -> int:
        return int(self.lib.q4o_double_to_half(float(v)))

    def halves_to_doubles(self, bits: np.ndarray) -> np.ndarray:
        flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
        out = np.fromiter((self.lib.q4o_half_to_double(int(b)) for b in flat),
                          dtype=np.float64, count=flat.size)
        return out.reshape(np.shape(bits))

    def doubles_to_halves(self, v: np.ndarray) -> np.ndarray:
        flat = np.ascontiguousarray(v, dtype=np.float64).ravel()
        out = np.fromiter((self.lib.q4o_double_to_half(float(x)) for x in flat),
                          dtype=np.uint16, count=flat.size)
        return out.reshape(np.shape(v))

    # -- the matmul and its variants -------------------------------------
    @staticmethod
    def _check_w(words, scales, n, k):
        assert words.dtype == np.uint32 and words.shape == (n, k // 8)
        assert scales.dtype == np.uint16 and scales.shape == (n, k // 32)

    def gemv(self, words, scales, x):
        """(y, a) in f64: y = x.dequant(W)^T, a = sum |x_k w_k|."""
        n = words.shape[0]
        k = x.shape[0]
        self._check_w(words, scales, n, k)
        words, scales = np.ascontiguousarray(words), np.ascontiguousarray(scales)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        y = np.empty(n, np.float64)
        a = np.empty(n, np.float64)
        rc = self.lib.q4o_gemv(_ptr(words), _ptr(scales), _ptr(x), n, k,
                               _ptr(y), _ptr(a))
        assert rc == 0
        return y, a

    def _check_w3(self, words3, scales, n, k):
        assert words3.dtype == np.uint32 and words3.shape == (n, 3 * k // 32), words3.shape
        assert scales.dtype == np.uint16 and scales.shape == (n, k // 32), scales.shape

    def gemv3(self, words3, scales, x):
        """(y, a) in f64 for an int3 weight: words3 uint32 [n][3k/32] (each
        row one LSB-first stream of 3-bit codes), w = (q - 4) * scale."""
        n, k = words3.shape[0], x.shape[0]
        self._check_w3(words3, scales, n, k)
        words3, scales = np.ascontiguousarray(words3), np.ascontiguousarray(scales)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        y = np.empty(n, np.float64)
        a = np.empty(n, np.float64)
        rc = self.lib.q4o_gemv3(_ptr(words3), _ptr(scales), _ptr(x), n, k, _ptr(y), _ptr(a))
        assert rc == 0
        return y, a

    def kv_quant_row(self, x):
        """(codes int8 [d], scale f32) of one f16 row (symmetric, per row)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        q = np.empty(x.size, np.int8)
        sc = np.zeros(1, np.float32)
        self.lib.q4o_kv_quant_row(_ptr(x), x.size, _ptr(q), _ptr(sc))
        return q, sc[0]

    def kv8_page_bytes(self, nkv: int, d: int) -> int:
        return int(self.lib.q4o_kv8_page_bytes(nkv, d))

    def kv_append_int8(self, qkv, nq: int, nkv: int, d: int, pos: int, cache8, page_table):
        """Quantise and append the k, v heads of qkv f16 [(nq + 2 nkv) d] into
        cache8 (uint8 [pages][page bytes], modified in place)."""
        qkv = np.ascontiguousarray(qkv, dtype=np.uint16)
        assert qkv.size == (nq + 2 * nkv) * d
        assert cache8.dtype == np.uint8 and cache8.flags["C_CONTIGUOUS"]
        assert cache8.shape[1] == self.kv8_page_bytes(nkv, d)
        pt = np.ascontiguousarray(page_table, dtype=np.int32)
        rc = self.lib.q4o_kv_append_int8(_ptr(qkv), nq, nkv, d, pos, _ptr(cache8), _ptr(pt),
                                         cache8.shape[0])
        assert rc == 0

    def attention_decode_int8(self, q, cache8, page_table, ctx: int, nq: int, nkv: int, d: int,
                              scale: float):
        """(out, a) f64 [nq][d] over the int8 cache (uint8 [pages][page bytes])."""
        q = np.ascontiguousarray(q, dtype=np.uint16).reshape(nq * d)
        assert cache8.dtype == np.uint8 and cache8.shape[1] == self.kv8_page_bytes(nkv, d)
        cache8 = np.ascontiguousarray(cache8)
        pt = np.ascontiguousarray(page_table, dtype=np.int32)
        out = np.empty((nq, d), np.float64)
        a = np.empty((nq, d), np.float64)
        rc = self.lib.q4o_attention_decode_int8(_ptr(q), _ptr(cache8), _ptr(pt), cache8.shape[0],
                                                ctx, nq, nkv, d, float(scale), _ptr(out), _ptr(a))
        assert rc == 0
        return out, a

    def gemm3(self, words3, scales, X):
        """(Y, A) f64 [m][n] for an int3 weight and activation rows X [m][k]."""
        m, k = X.shape
        n = words3.shape[0]
        self._check_w3(words3, scales, n, k)
        words3, scales = np.ascontiguousarray(words3), np.ascontiguousarray(scales)
        X = np.ascontiguousarray(X, dtype=np.uint16)
        Y = np.empty((m, n), np.float64)
        A = np.empty((m, n), np.float64)
        rc = self.lib.q4o_gemm3(_ptr(words3), _ptr(scales), _ptr(X), m, n, k, _ptr(Y), _ptr(A))
        assert rc == 0
        return Y, A

    def ffn_gate_up_silu3(self, gw3, gs, uw3, us, x):
        """int3 FFN: dict with h, g, u, ag, au (all f64 [n])."""
        n, k = gw3.shape[0], x.shape[0]
        self._check_w3(gw3, gs, n, k)
        self._check_w3(uw3, us, n, k)
        arrs = [np.ascontiguousarray(a) for a in (gw3, gs, uw3, us)]
        x = np.ascontiguousarray(x, dtype=np.uint16)
        out = {name: np.empty(n, np.float64) for name in ("h", "g", "u", "ag", "au")}
        rc = self.lib.q4o_ffn_gate_up_silu3(
            *[_ptr(a) for a in arrs], _ptr(x), n, k,
            *[_ptr(out[name]) for name in ("h", "g", "u", "ag", "au")])
        assert rc == 0
        return out

    def encode3_gate_up(self, gw3, gs, uw3, us) -> np.ndarray:
        """The int3 gate/up device layout (2n interleaved logical rows)."""
        n, k = gw3.shape[0], gw3.shape[1] * 32 // 3
        self._check_w3(gw3, gs, n, k)
        self._check_w3(uw3, us, n, k)
        arrs = [np.ascontiguousarray(a) for a in (gw3, gs, uw3, us)]
        dst = np.full(int(self.lib.q4o_layout3_bytes(2 * n, k)), 0xA5, np.uint8)
        rc = self.lib.q4o_encode3_gate_up(*[_ptr(a) for a in arrs], n, k, _ptr(dst))
        assert rc == 0
        return dst

    def encode3(self, words3, scales) -> np.ndarray:
        """The int3 device layout (bytes) of words3 [n][3k/32], scales [n][k/32]."""
        n, k = words3.shape[0], words3.shape[1] * 32 // 3
        self._check_w3(words3, scales, n, k)
        words3, scales = np.ascontiguousarray(words3), np.ascontiguousarray(scales)
        dst = np.full(int(self.lib.q4o_layout3_bytes(n, k)), 0xA5, np.uint8)
        rc = self.lib.q4o_encode3(_ptr(words3), _ptr(scales), n, k, _ptr(dst))
        assert rc == 0
        return dst

    def gemm(self, words, scales, X):
        m, k = X.shape
        n = words.shape[0]
        self._check_w(words, scales, n, k)
        words, scales = np.ascontiguousarray(words), np.ascontiguousarray(scales)
        X = np.ascontiguousarray(X, dtype=np.uint16)
        Y = np.empty((m, n), np.float64)
        A = np.empty((m, n), np.float64)
        rc = self.lib.q4o_gemm(_ptr(words), _ptr(scales), _ptr(X), m, n, k,
                               _ptr(Y), _ptr(A))
        assert rc == 0
        return Y, A

    def silu(self, g: float) -> float:
        return self.lib.q4o_silu(float(g))

    def ffn_gate_up_silu(self, gw, gs, uw, us, x):
        """dict with h, g, u, ag, au (all f64 [n])."""
        n = gw.shape[0]
        k = x.shape[0]
        self._check_w(gw, gs, n, k)
        self._check_w(uw, us, n, k)
        arrs = [np.ascontiguousarray(a) for a in (gw, gs, uw, us)]
        x = np.ascontiguousarray(x, dtype=np.uint16)
        out = {name: np.empty(n, np.float64) for name in ("h", "g", "u", "ag", "au")}
        rc = self.lib.q4o_ffn_gate_up_silu(
            *[_ptr(a) for a in arrs], _ptr(x), n, k,
            *[_ptr(out[name]) for name in ("h", "g", "u", "ag", "au")])
        assert rc == 0
        return out

    def add_rmsnorm(self, x, r, gamma, eps: float):
        """(h, xn) f16 bits [k]: the new residual f16(x + r) (x when r is None)
        and the normalised activation f16(h * gamma / sqrt(mean(h^2) + eps))."""
        k = x.shape[0]
        x = np.ascontiguousarray(x, dtype=np.uint16)
        gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
        assert gamma.shape == (k,)
        rp = None
        if r is not None:
            r = np.ascontiguousarray(r, dtype=np.uint16)
            assert r.shape == (k,)
            rp = _ptr(r)
        h = np.empty(k, np.uint16)
        xn = np.empty(k, np.uint16)
        rc = self.lib.q4o_add_rmsnorm(_ptr(x), rp, _ptr(gamma), k, float(eps), _ptr(h), _ptr(xn))
        assert rc == 0
        return h, xn

    def rope_pair(self, yi: float, yj: float, i: int, d: int, pos: int, base: float):
        oi, oj = ctypes.c_double(), ctypes.c_double()
        self.lib.q4o_rope_pair(float(yi), float(yj), i, d, pos, float(base),
                               ctypes.addressof(oi), ctypes.addressof(oj))
        return oi.value, oj.value

    def qkv_rope(self, words, scales, x, d: int, nq: int, pos: int, base: float):
        """(y f64 [n] with RoPE on the q and k heads, a f64 [n])."""
        n = words.shape[0]
        k = x.shape[0]
        self._check_w(words, scales, n, k)
        words, scales = np.ascontiguousarray(words), np.ascontiguousarray(scales)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        y = np.empty(n, np.float64)
        a = np.empty(n, np.float64)
        rc = self.lib.q4o_qkv_rope(_ptr(words), _ptr(scales), _ptr(x), n, k, d, nq, pos,
                                   float(base), _ptr(y), _ptr(a))
        assert rc == 0
        return y, a

    def attention_decode(self, q, cache, page_table, ctx: int, nq: int, nkv: int, d: int,
                         scale: float):
        """(out f64 [nq][d], a f64 [nq][d]) of one decode token over positions
        0 .. ctx-1 of the paged cache f16 bits [pages][2][nkv][16][d]."""
        q = np.ascontiguousarray(q, dtype=np.uint16).reshape(nq * d)
        cache = np.ascontiguousarray(cache, dtype=np.uint16)
        assert cache.ndim == 5 and cache.shape[1:] == (2, nkv, 16, d)
        pt = np.ascontiguousarray(page_table, dtype=np.int32)
        assert pt.size >= (ctx + 15) // 16
        out = np.empty((nq, d), np.float64)
        a = np.empty((nq, d), np.float64)
        rc = self.lib.q4o_attention_decode(_ptr(q), _ptr(cache), _ptr(pt), cache.shape[0], ctx,
                                           nq, nkv, d, float(scale), _ptr(out), _ptr(a))
        assert rc == 0
        return out, a

    def argmax(self, v) -> int:
        v = np.ascontiguousarray(v, dtype=np.float64)
        return int(self.lib.q4o_argmax(_ptr(v), v.size))

    def lmhead(self, words, scales, x):
        """(logits f64, a f64, argmax index)."""
        n = words.shape[0]
        k = x.shape[0]
        self._check_w(words, scales, n, k)
        words, scales = np.ascontiguousarray(words), np.ascontiguousarray(scales)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        y = np.empty(n, np.float64)
        a = np.empty(n, np.float64)
        idx = self.lib.q4o_lmhead(_ptr(words), _ptr(scales), _ptr(x), n, k,
                                  _ptr(y), _ptr(a))
        return y, a, int(idx)

    # -- device layout encoder (for the byte-exact pack test) ------------
    def layout_geometry(self, rows: int, k: int) -> dict:
        out = np.zeros(6, np.int64)
        rc = self.lib.q4o_layout_geometry(rows, k, _ptr(out))
        assert rc == 0
        return dict(zip(("L", "CG", "P", "TR", "tiles", "tile_bytes"),
                        (int(v) for v in out)))

    def layout_bytes(self, rows: int, k: int) -> int:
        return int(self.lib.q4o_layout_bytes(rows, k))

    def encode_rows(self, words, scales) -> np.ndarray:
        n, k = words.shape[0], words.shape[1] * 8
        self._check_w(words, scales, n, k)
        words, scales = np.ascontiguousarray(words), np.ascontiguousarray(scales)
        dst = np.full(self.layout_bytes(n, k), 0xA5, np.uint8)
        rc = self.lib.q4o_encode_rows(_ptr(words), _ptr(scales), n, k, _ptr(dst))
        assert rc == 0
        return dst

    def encode_rope(self, words, scales, d: int) -> np.ndarray:
        n, k = words.shape[0], words.shape[1] * 8
        self._check_w(words, scales, n, k)
        words, scales = np.ascontiguousarray(words), np.ascontiguousarray(scales)
        dst = np.full(self.layout_bytes(n, k), 0xA5, np.uint8)
        rc = self.lib.q4o_encode_rope(_ptr(words), _ptr(scales), n, k, d, _ptr(dst))
        assert rc == 0
        return dst

    def encode_gate_up(self, gw, gs, uw, us) -> np.ndarray:
        n, k = gw.shape[0], gw.shape[1] * 8
        self._check_w(gw, gs, n, k)
        self._check_w(uw, us, n, k)
        arrs = [np.ascontiguousarray(a) for a in (gw, gs, uw, us)]
        dst = np.full(self.layout_bytes(2 * n, k), 0xA5, np.uint8)
        rc = self.lib.q4o_encode_gate_up(*[_ptr(a) for a in arrs], n, k, _ptr(dst))
        assert rc == 0
        return dst


_DEFAULT: Optional[Oracle] = None


def load(path: Optional[str] = None) -> Oracle:
    """Load the oracle (building it first if the library is missing or older
    than its source)."""
    global _DEFAULT
    if path is not None:
        return Oracle(path)
    if _DEFAULT is None:
        if (not os.path.exists(LIBRARY) or
                os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT

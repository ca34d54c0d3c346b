"""int4_quantized_decode_q4_amd -- Python binding of libq4.

libq4 is the int4-dequantizing matrix multiply of LLM decode for AMD
Instinct MI355X (gfx950): ``y = x . dequant(W)^T`` with W as 4-bit codes and
one f16 scale per 32 weights along k (the "q4f16_1" weights of the Zero-TVM
article "Zero-TVM：手写 WGSL 着色器在浏览器中运行 Phi-3-mini，挑战编译器霸权",
section 完整的推理流水线; the fused FFN of its section 内核融合).

This module only marshals arguments: torch tensors provide device memory and
the current stream, and every step runs in the HIP kernels of ``libq4.so``.
There is no fallback: importing fails if the library is not built
(``python int4_quantized_decode_q4_amd/build.py``), and every call raises
``Q4Error`` with the library's return code on failure.

Tensor conventions: f16 data as ``torch.float16`` (or 16-bit integer views);
canonical words as 32-bit integers [n][k/8]; scales as 16-bit [n][k/32]; all on
one CUDA (HIP) device, contiguous.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq4.so")
if not os.path.exists(LIBRARY):
    raise ImportError(
        f"{LIBRARY} is not built; run `python int4_quantized_decode_q4_amd/build.py`")

_lib = ctypes.CDLL(LIBRARY)

OK = 0
ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_LAYOUT = -1, -2, -3, -4
ERR_WORKSPACE, ERR_ALIAS, ERR_HIP, ERR_SIZE = -5, -6, -7, -8
LAYOUT_ROWS, LAYOUT_GATE_UP, LAYOUT_ROPE, LAYOUT_INT3, LAYOUT_VERSION = 1, 2, 3, 4, 1
LAYOUT_INT3_GATE_UP = 5
GEMM_AUTO, GEMM_VALU, GEMM_MFMA = 0, 1, 2
OP_GEMV, OP_GEMM, OP_FFN, OP_LMHEAD, OP_ATTENTION = 1, 2, 3, 4, 5


class q4_weight(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("version", ctypes.c_int32),
                ("data", ctypes.c_void_p), ("bytes", ctypes.c_int64),
                ("head_dim", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class q4_chain_stage(ctypes.Structure):
    _fields_ = [("w", ctypes.POINTER(q4_weight)), ("x", ctypes.c_void_p),
                ("src", ctypes.c_int32), ("after", ctypes.c_int32),
                ("residual", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("residual_out", ctypes.c_void_p), ("y", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64
_W = ctypes.POINTER(q4_weight)
_CS = ctypes.POINTER(q4_chain_stage)

_SIGNATURES = {
    "q4_packed_bytes": (_I64, [_I32, _I32, _I32]),
    "q4_workspace_bytes": (_I64, [_I32, _I32, _I32, _I32]),
    "q4_pack": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _I64, _W, _P]),
    "q4_pack_gate_up": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _P, _I64, _W, _P]),
    "q4_pack_rope": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _I64, _W, _P]),
    "q4_unpack": (ctypes.c_int, [_W, _P, _P, _P]),
    "q4_pack_int3": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _I64, _W, _P]),
    "q4_pack_int3_gate_up": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _P, _I64, _W, _P]),
    "q4_kv_int8_page_bytes": (ctypes.c_int64, [_I32, _I32]),
    "q4_kv_append_int8": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _I32, _P]),
    "q4_attention_decode_int8": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                                ctypes.c_float, _P, _P, _I64, _P]),
    "q4_qkv_rope_append": (ctypes.c_int, [_W, _P, _I32, _I32, ctypes.c_double, _P, _P, _P, _I32,
                                          _P]),
    "q4_add_rmsnorm_qkv_rope_append": (ctypes.c_int, [_W, _P, _P, _P, ctypes.c_float, _P, _I32,
                                                      _I32, ctypes.c_double, _P, _P, _P, _I32,
                                                      _P]),
    "q4_gemv": (ctypes.c_int, [_W, _P, _P, _P]),
    "q4_gemm": (ctypes.c_int, [_W, _P, _I32, _P, _P, _I64, _P]),
    "q4_gemm_path": (ctypes.c_int, [_W, _P, _I32, _P, _I32, _P]),
    "q4_ffn_gate_up_silu": (ctypes.c_int, [_W, _P, _P, _P]),
    "q4_add_rmsnorm_gemv": (ctypes.c_int, [_W, _P, _P, _P, ctypes.c_float, _P, _P, _P]),
    "q4_add_rmsnorm_ffn_gate_up_silu": (ctypes.c_int, [_W, _P, _P, _P, ctypes.c_float, _P, _P, _P]),
    "q4_lmhead_f32": (ctypes.c_int, [_W, _P, _P, _P, _P, _I64, _P]),
    "q4_lmhead_f32_noalloc": (ctypes.c_int, [_W, _P, _P, _P, _P]),
    "q4_attention_decode": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                           ctypes.c_float, _P, _P, _I64, _P]),
    "q4_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "q4_last_hip_error": (ctypes.c_int, []),
    "q4_source_hash": (ctypes.c_char_p, []),
    "q4_layout_geometry": (ctypes.c_int, [_I32, _I32, _P]),
    "q4_read_probe": (ctypes.c_int, [_P, _I64, _P, _I64, _P]),
    "q4_chain_workspace_bytes": (_I64, [_CS, _I32]),
    "q4_chain": (ctypes.c_int, [_CS, _I32, _P, _I64, _P]),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

lib = _lib   # the raw ctypes handle, for callers that want the C ABI itself


class Q4Error(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.q4_strerror(code).decode()
        if code == ERR_HIP:
            msg += f" (hipError {_lib.q4_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{code}]")


def source_hash() -> str:
    """Digest of the sources the loaded libq4.so was built from
    (q4_source_hash); compare with build.py's sources_digest()."""
    return _lib.q4_source_hash().decode()


def _check(code: int, where: str) -> None:
    if code != OK:
        raise Q4Error(code, where)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, itemsize: int, shape=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.element_size() != itemsize:
        raise TypeError(f"{name} must have {itemsize}-byte elements, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


class PackedWeight:
    """A weight in the device layout: the owning byte tensor plus the C
    descriptor that every op takes."""

    def __init__(self, buf: torch.Tensor, desc: q4_weight):
        self.buf = buf
        self.desc = desc

    @property
    def n(self) -> int:
        return self.desc.n

    @property
    def k(self) -> int:
        return self.desc.k

    @property
    def layout(self) -> int:
        return self.desc.layout

    @property
    def nbytes(self) -> int:
        return self.desc.bytes

    @property
    def device(self) -> torch.device:
        return self.buf.device

    def clone(self) -> "PackedWeight":
        """A copy in new device memory (same bytes, every descriptor field)."""
        buf = self.buf.clone()
        if buf.data_ptr() % 256:
            raise RuntimeError("allocator returned a buffer that is not 256-byte aligned")
        desc = q4_weight()
        ctypes.memmove(ctypes.byref(desc), ctypes.byref(self.desc), ctypes.sizeof(q4_weight))
        desc.data = buf.data_ptr()
        return PackedWeight(buf, desc)


def packed_bytes(n: int, k: int, layout: int = LAYOUT_ROWS) -> int:
    return int(_lib.q4_packed_bytes(n, k, layout))


def layout_geometry(rows: int, k: int) -> dict:
    out = (ctypes.c_int64 * 6)()
    _check(_lib.q4_layout_geometry(rows, k, ctypes.cast(out, _P)), "q4_layout_geometry")
    return dict(zip(("L", "CG", "P", "TR", "tiles", "tile_bytes"), (int(v) for v in out)))


def _alloc_packed(n: int, k: int, layout: int, device) -> torch.Tensor:
    nb = packed_bytes(n, k, layout)
    if nb <= 0:
        raise Q4Error(ERR_SHAPE, "packed_bytes")
    buf = torch.empty(nb, dtype=torch.uint8, device=device)
    if buf.data_ptr() % 256:
        raise RuntimeError("allocator returned a buffer that is not 256-byte aligned")
    return buf


def pack(words: torch.Tensor, scales: torch.Tensor) -> PackedWeight:
    """Canonical words [n][k/8] (32-bit) and scales [n][k/32] (16-bit) ->
    device layout (q4_pack)."""
    n, kw = words.shape
    k = kw * 8
    pw = _dev(words, "words", 4, (n, kw))
    ps = _dev(scales, "scales", 2, (n, k // 32))
    buf = _alloc_packed(n, k, LAYOUT_ROWS, words.device)
    desc = q4_weight()
    _check(_lib.q4_pack(pw, ps, n, k, buf.data_ptr(), buf.numel(), ctypes.byref(desc),
                        _stream(words)), "q4_pack")
    return PackedWeight(buf, desc)


def pack_gate_up(gw, gs, uw, us) -> PackedWeight:
    """Gate and up halves, each canonical [n][k/8] / [n][k/32] -> one
    interleaved layout for ffn_gate_up_silu (q4_pack_gate_up)."""
    n, kw = gw.shape
    k = kw * 8
    ptrs = [_dev(gw, "gate words", 4, (n, kw)), _dev(gs, "gate scales", 2, (n, k // 32)),
            _dev(uw, "up words", 4, (n, kw)), _dev(us, "up scales", 2, (n, k // 32))]
    buf = _alloc_packed(n, k, LAYOUT_GATE_UP, gw.device)
    desc = q4_weight()
    _check(_lib.q4_pack_gate_up(*ptrs, n, k, buf.data_ptr(), buf.numel(), ctypes.byref(desc),
                                _stream(gw)), "q4_pack_gate_up")
    return PackedWeight(buf, desc)


def pack_rope(words: torch.Tensor, scales: torch.Tensor, head_dim: int) -> PackedWeight:
    """Canonical [n][k/8] / [n][k/32] of the concatenated q, k, v head rows
    -> the rotary-paired layout for qkv_rope_append (q4_pack_rope)."""
    n, kw = words.shape
    k = kw * 8
    pw = _dev(words, "words", 4, (n, kw))
    ps = _dev(scales, "scales", 2, (n, k // 32))
    buf = _alloc_packed(n, k, LAYOUT_ROPE, words.device)
    desc = q4_weight()
    _check(_lib.q4_pack_rope(pw, ps, n, k, head_dim, buf.data_ptr(), buf.numel(),
                             ctypes.byref(desc), _stream(words)), "q4_pack_rope")
    return PackedWeight(buf, desc)


def pack_int3(words3: torch.Tensor, scales: torch.Tensor) -> PackedWeight:
    """int3 weight: canonical words3 [n][3k/32] (32-bit; each row one LSB-first
    stream of 3-bit codes, w = (q - 4) * scale) and scales [n][k/32] (16-bit)
    -> the int3 device layout, for gemv (q4_pack_int3)."""
    n, kw = words3.shape
    if kw % 3:
        raise ValueError("words3 must have 3 words per group of 32 codes")
    k = kw * 32 // 3
    pw = _dev(words3, "words3", 4, (n, kw))
    ps = _dev(scales, "scales", 2, (n, k // 32))
    buf = _alloc_packed(n, k, LAYOUT_INT3, words3.device)
    desc = q4_weight()
    _check(_lib.q4_pack_int3(pw, ps, n, k, buf.data_ptr(), buf.numel(), ctypes.byref(desc),
                             _stream(words3)), "q4_pack_int3")
    return PackedWeight(buf, desc)


def pack_int3_gate_up(gw3, gs, uw3, us) -> PackedWeight:
    """Gate and up halves as int3 weights, each canonical words3 [n][3k/32] /
    scales [n][k/32] -> one interleaved layout for ffn_gate_up_silu
    (q4_pack_int3_gate_up)."""
    n, kw = gw3.shape
    if kw % 3:
        raise ValueError("words3 must have 3 words per group of 32 codes")
    k = kw * 32 // 3
    ptrs = [_dev(gw3, "gate words3", 4, (n, kw)), _dev(gs, "gate scales", 2, (n, k // 32)),
            _dev(uw3, "up words3", 4, (n, kw)), _dev(us, "up scales", 2, (n, k // 32))]
    buf = _alloc_packed(n, k, LAYOUT_INT3_GATE_UP, gw3.device)
    desc = q4_weight()
    _check(_lib.q4_pack_int3_gate_up(*ptrs, n, k, buf.data_ptr(), buf.numel(), ctypes.byref(desc),
                                     _stream(gw3)), "q4_pack_int3_gate_up")
    return PackedWeight(buf, desc)


def unpack(w: PackedWeight) -> Tuple[torch.Tensor, torch.Tensor]:
    """Device layout -> canonical (words int32 [rows][k/8] -- int3: [rows][3k/32]
    --, scales int16 [rows][k/32]); rows = 2n for a gate/up weight (gate 0,
    up 0, gate 1, ...)."""
    rows = w.n * (2 if w.layout in (LAYOUT_GATE_UP, LAYOUT_INT3_GATE_UP) else 1)
    wcols = 3 * w.k // 32 if w.layout in (LAYOUT_INT3, LAYOUT_INT3_GATE_UP) else w.k // 8
    words = torch.empty((rows, wcols), dtype=torch.int32, device=w.device)
    scales = torch.empty((rows, w.k // 32), dtype=torch.int16, device=w.device)
    _check(_lib.q4_unpack(ctypes.byref(w.desc), words.data_ptr(), scales.data_ptr(),
                          _stream(words)), "q4_unpack")
    return words, scales


def gemv(w: PackedWeight, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y f16 [n] = x f16 [k] . dequant(W)^T (q4_gemv); W int4 rows or int3."""
    px = _dev(x, "x", 2, (w.k,))
    if out is None:
        out = torch.empty(w.n, dtype=torch.float16, device=x.device)
    py = _dev(out, "out", 2, (w.n,))
    _check(_lib.q4_gemv(ctypes.byref(w.desc), px, py, _stream(x)), "q4_gemv")
    return out


def gemm(w: PackedWeight, X: torch.Tensor, out: Optional[torch.Tensor] = None,
         path: int = GEMM_AUTO) -> torch.Tensor:
    """Y f16 [m][n] = X f16 [m][k] . dequant(W)^T (q4_gemm; q4_gemm_path when a
    kernel is forced: GEMM_VALU or GEMM_MFMA)."""
    m = X.shape[0]
    px = _dev(X, "X", 2, (m, w.k))
    if out is None:
        out = torch.empty((m, w.n), dtype=torch.float16, device=X.device)
    py = _dev(out, "out", 2, (m, w.n))
    if path == GEMM_AUTO:
        _check(_lib.q4_gemm(ctypes.byref(w.desc), px, m, py, None, 0, _stream(X)), "q4_gemm")
    else:
        _check(_lib.q4_gemm_path(ctypes.byref(w.desc), px, m, py, path, _stream(X)),
               "q4_gemm_path")
    return out


def ffn_gate_up_silu(w: PackedWeight, x: torch.Tensor,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h f16 [n] = SiLU(x.Wg^T) * (x.Wu^T) in one kernel (q4_ffn_gate_up_silu)."""
    px = _dev(x, "x", 2, (w.k,))
    if out is None:
        out = torch.empty(w.n, dtype=torch.float16, device=x.device)
    ph = _dev(out, "out", 2, (w.n,))
    _check(_lib.q4_ffn_gate_up_silu(ctypes.byref(w.desc), px, ph, _stream(x)),
           "q4_ffn_gate_up_silu")
    return out


def _norm_args(w: PackedWeight, x, residual, gamma, residual_out):
    px = _dev(x, "x", 2, (w.k,))
    pr = None if residual is None else _dev(residual, "residual", 2, (w.k,))
    pg = _dev(gamma, "gamma", 2, (w.k,))
    pro = None if residual_out is None else _dev(residual_out, "residual_out", 2, (w.k,))
    return px, pr, pg, pro


def add_rmsnorm_gemv(w: PackedWeight, x: torch.Tensor, residual: Optional[torch.Tensor],
                     gamma: torch.Tensor, eps: float, residual_out: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y f16 [n] = f16(h * gamma / sqrt(mean(h^2) + eps)) . dequant(W)^T with
    h = f16(x + residual) (x when residual is None) written to residual_out
    when given (q4_add_rmsnorm_gemv)."""
    px, pr, pg, pro = _norm_args(w, x, residual, gamma, residual_out)
    if out is None:
        out = torch.empty(w.n, dtype=torch.float16, device=x.device)
    py = _dev(out, "out", 2, (w.n,))
    _check(_lib.q4_add_rmsnorm_gemv(ctypes.byref(w.desc), px, pr, pg, float(eps), pro, py,
                                    _stream(x)), "q4_add_rmsnorm_gemv")
    return out


def add_rmsnorm_ffn_gate_up_silu(w: PackedWeight, x: torch.Tensor,
                                 residual: Optional[torch.Tensor], gamma: torch.Tensor,
                                 eps: float, residual_out: Optional[torch.Tensor] = None,
                                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The same add + RMSNorm prologue in front of the fused gate/up SiLU
    (q4_add_rmsnorm_ffn_gate_up_silu)."""
    px, pr, pg, pro = _norm_args(w, x, residual, gamma, residual_out)
    if out is None:
        out = torch.empty(w.n, dtype=torch.float16, device=x.device)
    ph = _dev(out, "out", 2, (w.n,))
    _check(_lib.q4_add_rmsnorm_ffn_gate_up_silu(ctypes.byref(w.desc), px, pr, pg, float(eps),
                                                pro, ph, _stream(x)),
           "q4_add_rmsnorm_ffn_gate_up_silu")
    return out


def qkv_rope_append(w: PackedWeight, x: torch.Tensor, n_q_heads: int, pos: int,
                    rope_base: float, kv_cache: Optional[torch.Tensor] = None,
                    page_table: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, norm=None) -> torch.Tensor:
    """qkv f16 [n]: the fused QKV projection with RoPE on the q and k heads,
    the k and v heads appended to kv_cache f16 [pages][2][n_kv][16][d] at
    slot pos % 16 of page page_table[pos // 16] (q4_qkv_rope_append).
    norm = (residual or None, gamma, eps, residual_out or None) runs the add
    + RMSNorm prologue first (q4_add_rmsnorm_qkv_rope_append)."""
    px = _dev(x, "x", 2, (w.k,))
    if out is None:
        out = torch.empty(w.n, dtype=torch.float16, device=x.device)
    py = _dev(out, "out", 2, (w.n,))
    pc, pt, npages = None, None, 0
    if kv_cache is not None:
        if w.layout != LAYOUT_ROPE or w.desc.head_dim < 2:
            raise ValueError("qkv_rope_append takes a weight packed by pack_rope")
        d = w.desc.head_dim
        nkv2 = w.n // d - n_q_heads
        if n_q_heads < 0 or nkv2 < 0 or nkv2 % 2:
            raise ValueError(f"{w.n // d} heads of {d} rows do not split into {n_q_heads} q heads "
                             "and equal k and v heads")
        if kv_cache.dim() != 5:
            raise ValueError("kv_cache must be [pages][2][n_kv][16][d]")
        npages = kv_cache.shape[0]
        pc = _dev(kv_cache, "kv_cache", 2, (npages, 2, nkv2 // 2, 16, d))
        if page_table is None:
            raise ValueError("a page table is needed with a cache")
        pt = _dev(page_table, "page_table", 4)
        if pos < 0 or page_table.numel() < pos // 16 + 1:
            raise ValueError(f"page_table has {page_table.numel()} entries; position {pos} needs "
                             f"{pos // 16 + 1}")
    if norm is None:
        _check(_lib.q4_qkv_rope_append(ctypes.byref(w.desc), px, n_q_heads, pos, float(rope_base),
                                       py, pc, pt, npages, _stream(x)), "q4_qkv_rope_append")
    else:
        residual, gamma, eps, residual_out = norm
        _, pr, pg, pro = _norm_args(w, x, residual, gamma, residual_out)
        _check(_lib.q4_add_rmsnorm_qkv_rope_append(ctypes.byref(w.desc), px, pr, pg, float(eps),
                                                   pro, n_q_heads, pos, float(rope_base), py, pc,
                                                   pt, npages, _stream(x)),
               "q4_add_rmsnorm_qkv_rope_append")
    return out


def attention_decode(q: torch.Tensor, kv_cache: torch.Tensor, page_table: torch.Tensor, ctx: int,
                     n_q_heads: int, scale: float, out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out f16 [nq][d]: one decode token's attention over positions 0..ctx-1
    of the paged cache f16 [pages][2][n_kv][16][d] (q4_attention_decode)."""
    if kv_cache.dim() != 5:
        raise ValueError("kv_cache must be a contiguous 16-bit [pages][2][n_kv][16][d] tensor")
    pages, _, nkv, _, d = kv_cache.shape
    pc = _dev(kv_cache, "kv_cache", 2, (pages, 2, nkv, 16, d))
    pq = _dev(q, "q", 2)
    if q.numel() != n_q_heads * d:
        raise ValueError(f"q has {q.numel()} elements, expected {n_q_heads * d}")
    pt = _dev(page_table, "page_table", 4)
    _check_table(page_table, ctx)
    if out is None:
        out = torch.empty((n_q_heads, d), dtype=torch.float16, device=q.device)
    po = _dev(out, "out", 2)
    need = int(_lib.q4_workspace_bytes(OP_ATTENTION, ctx, n_q_heads, d))
    pws = None
    if need > 0:
        if ws is None:
            ws = workspace(q.device, need)
        pws = ws.data_ptr()
    _check(_lib.q4_attention_decode(pq, pc, pt, pages, ctx, n_q_heads, nkv, d,
                                    float(scale), po, pws, need if need > 0 else 0, _stream(q)),
           "q4_attention_decode")
    return out


def kv_int8_page_bytes(n_kv_heads: int, head_dim: int) -> int:
    return int(_lib.q4_kv_int8_page_bytes(n_kv_heads, head_dim))


def kv_append_int8(qkv: torch.Tensor, n_q_heads: int, n_kv_heads: int, head_dim: int, pos: int,
                   cache8: torch.Tensor, page_table: torch.Tensor) -> None:
    """Quantise the k and v heads of a fused QKV output into the int8 cache
    (uint8 [pages][q4_kv_int8_page_bytes]) at position pos (q4_kv_append_int8)."""
    pq = _dev(qkv, "qkv", 2)
    if qkv.numel() != (n_q_heads + 2 * n_kv_heads) * head_dim:
        raise ValueError("qkv does not hold n_q_heads + 2 n_kv_heads heads of head_dim")
    pb = kv_int8_page_bytes(n_kv_heads, head_dim)
    if cache8.dim() != 2 or cache8.shape[1] != pb:
        raise ValueError(f"cache8 must be [pages][{pb}] bytes")
    pc = _dev(cache8, "cache8", 1)
    pt = _dev(page_table, "page_table", 4)
    if pos < 0 or page_table.numel() < pos // 16 + 1:
        raise ValueError(f"page_table has {page_table.numel()} entries; position {pos} needs "
                         f"{pos // 16 + 1}")
    _check(_lib.q4_kv_append_int8(pq, n_q_heads, n_kv_heads, head_dim, pos, pc, pt,
                                  cache8.shape[0], _stream(qkv)), "q4_kv_append_int8")


def attention_decode_int8(q: torch.Tensor, cache8: torch.Tensor, page_table: torch.Tensor,
                          ctx: int, n_q_heads: int, n_kv_heads: int, head_dim: int, scale: float,
                          out: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out f16 [nq][d]: attention of one decode token over the int8 cache
    (q4_attention_decode_int8)."""
    pb = kv_int8_page_bytes(n_kv_heads, head_dim)
    if cache8.dim() != 2 or cache8.shape[1] != pb:
        raise ValueError(f"cache8 must be [pages][{pb}] bytes")
    pq = _dev(q, "q", 2)
    if q.numel() != n_q_heads * head_dim:
        raise ValueError(f"q has {q.numel()} elements, expected {n_q_heads * head_dim}")
    pt = _dev(page_table, "page_table", 4)
    _check_table(page_table, ctx)
    if out is None:
        out = torch.empty((n_q_heads, head_dim), dtype=torch.float16, device=q.device)
    po = _dev(out, "out", 2)
    need = int(_lib.q4_workspace_bytes(OP_ATTENTION, ctx, n_q_heads, head_dim))
    pws = None
    if need > 0:
        if ws is None:
            ws = workspace(q.device, need)
        pws = ws.data_ptr()
    _check(_lib.q4_attention_decode_int8(pq, _dev(cache8, "cache8", 1), pt, cache8.shape[0], ctx,
                                         n_q_heads, n_kv_heads, head_dim, float(scale), po, pws,
                                         need if need > 0 else 0, _stream(q)),
           "q4_attention_decode_int8")
    return out


def _check_table(page_table: torch.Tensor, ctx: int) -> None:
    """The page table must cover positions 0 .. ctx - 1 (16 per page)."""
    if ctx < 1 or page_table.numel() < (ctx + 15) // 16:
        raise ValueError(f"page_table has {page_table.numel()} entries; a context of {ctx} "
                         f"needs {(ctx + 15) // 16}")


_workspaces: dict = {}
_retired: list = []


def workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """A workspace of at least nbytes on `device`, kept per device.  A buffer
    that is outgrown is replaced but never freed: a HIP graph captured
    earlier may still hold its address."""
    key = (device.type, device.index)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _retired.append(ws)
        ws = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


_lm_ws: dict = {}


def lmhead_workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """The LM head's own workspace on `device`: zero-filled when made, then
    only used by lmhead_f32 (its counters return to zero after every call);
    an outgrown one is kept alive, never freed (a graph may hold it)."""
    key = (device.type, device.index)
    ws = _lm_ws.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _retired.append(ws)
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _lm_ws[key] = ws
    return ws


def lmhead_f32_noalloc(w: PackedWeight, x: torch.Tensor, logits: torch.Tensor,
                       argmax: Optional[torch.Tensor] = None) -> None:
    """q4_lmhead_f32 with the argmax candidates in the library's static
    scratch (q4_lmhead_f32_noalloc): nothing is allocated, so the caller
    passes the outputs."""
    px = _dev(x, "x", 2, (w.k,))
    pl = _dev(logits, "logits", 4, (w.n,))
    pa = None if argmax is None else _dev(argmax, "argmax", 4, (1,))
    _check(_lib.q4_lmhead_f32_noalloc(ctypes.byref(w.desc), px, pl, pa, _stream(x)),
           "q4_lmhead_f32_noalloc")


def lmhead_f32(w: PackedWeight, x: torch.Tensor, logits: Optional[torch.Tensor] = None,
               argmax: Optional[torch.Tensor] = None, with_argmax: bool = True,
               ws: Optional[torch.Tensor] = None):
    """(logits f32 [n], argmax int32 [1] or None) (q4_lmhead_f32)."""
    px = _dev(x, "x", 2, (w.k,))
    if logits is None:
        logits = torch.empty(w.n, dtype=torch.float32, device=x.device)
    pl = _dev(logits, "logits", 4, (w.n,))
    pa, pws, nws = None, None, 0
    if with_argmax or argmax is not None:
        if argmax is None:
            argmax = torch.empty(1, dtype=torch.int32, device=x.device)
        pa = _dev(argmax, "argmax", 4, (1,))
        need = int(_lib.q4_workspace_bytes(OP_LMHEAD, 1, w.n, w.k))
        if ws is None:
            ws = lmhead_workspace(x.device, need)
        pws, nws = _dev(ws, "ws", 1), ws.numel()
    _check(_lib.q4_lmhead_f32(ctypes.byref(w.desc), px, pl, pa, pws, nws, _stream(x)),
           "q4_lmhead_f32")
    return logits, argmax


def read_probe(src: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A plain streaming read of every byte of src (q4_read_probe), the
    measurement ceiling of the matmuls; returns the sink (one word per block)."""
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise TypeError("src must be a contiguous CUDA (HIP) tensor")
    if sink is None:
        sink = torch.empty(2048, dtype=torch.int32, device=src.device)
    ps = _dev(sink, "sink", 4)
    nbytes = src.numel() * src.element_size()
    _check(_lib.q4_read_probe(src.data_ptr(), nbytes, ps, sink.numel() * 4, _stream(src)),
           "q4_read_probe")
    return sink


class Stage:
    """One stage of `chain`: y = x . dequant(W)^T (a Q4_LAYOUT_ROWS weight)
    or h = SiLU(x . Wg^T) * (x . Wu^T) (a gate/up weight), where x is given
    or is the output of stage `src`; with `gamma` the add + RMSNorm prologue
    runs first (h = x + residual -> residual_out); the stage does not start
    computing before stage `after` has finished."""

    def __init__(self, w: PackedWeight, x: Optional[torch.Tensor] = None, src: int = -1,
                 after: int = -1, residual: Optional[torch.Tensor] = None,
                 gamma: Optional[torch.Tensor] = None, eps: float = 0.0,
                 residual_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
        self.w, self.x, self.src, self.after = w, x, src, after
        self.residual, self.gamma, self.eps, self.residual_out = residual, gamma, eps, residual_out
        self.out = out


def _chain_descs(stages):
    arr = (q4_chain_stage * len(stages))()
    for i, st in enumerate(stages):
        d = arr[i]
        d.w = ctypes.pointer(st.w.desc)
        k, n = st.w.k, st.w.n
        d.x = None if st.x is None else _dev(st.x, f"stage {i} x", 2, (k,))
        d.src, d.after = int(st.src), int(st.after)
        d.residual = None if st.residual is None else _dev(st.residual, f"stage {i} residual", 2, (k,))
        d.gamma = None if st.gamma is None else _dev(st.gamma, f"stage {i} gamma", 2, (k,))
        d.eps = float(st.eps)
        d.reserved = 0
        d.residual_out = (None if st.residual_out is None else
                          _dev(st.residual_out, f"stage {i} residual_out", 2, (k,)))
        if st.out is None:
            st.out = torch.empty(n, dtype=torch.float16, device=st.w.device)
        d.y = _dev(st.out, f"stage {i} out", 2, (n,))
    return arr


_chain_ws: dict = {}


def chain_workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """The chain workspace of `device` (zero-filled when made, then owned by
    the library: it carries per-block launch counters from call to call, so
    all chain calls that share it must run on one stream).  An outgrown one
    is replaced by a new zero-filled buffer and kept alive, never freed (a
    captured HIP graph may still use it)."""
    key = (device.type, device.index)
    ws = _chain_ws.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _retired.append(ws)
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _chain_ws[key] = ws
    return ws


def chain(stages, ws: Optional[torch.Tensor] = None):
    """Run the stages in one launch (q4_chain); returns their outputs."""
    arr = _chain_descs(stages)
    need = int(_lib.q4_chain_workspace_bytes(arr, len(stages)))
    if need <= 0:
        # the same validation the call does, for its error code
        _check(_lib.q4_chain(arr, len(stages), None, 0, None), "q4_chain")
    dev = stages[0].w.device
    if ws is None:
        ws = chain_workspace(dev, need)
    pws = _dev(ws, "ws", 1)
    _check(_lib.q4_chain(arr, len(stages), pws, ws.numel(), _stream(ws)), "q4_chain")
    return [st.out for st in stages]


def chain_error(ws: Optional[torch.Tensor] = None, device=None) -> int:
    """Word 0 of a chain workspace (non-zero: a wait of some call ran out of
    time); synchronises with the device."""
    if ws is None:
        ws = _chain_ws.get(("cuda", torch.device(device or "cuda").index or 0))
        if ws is None:
            return 0
    return int(ws[:4].view(torch.int32).item())

"""ctypes binding of libsckv.so: the C ABI's calls under the same names.

Argument marshalling only (torch tensor -> device pointer, current HIP stream,
status -> exception).  Every step of the computation runs in the library's
HIP kernels; there is no CPU path.  If the library is missing the import
fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsckv.so")

SCKV_OK = 0
SCKV_EINVAL = -1
SCKV_EUNSUPPORTED = -2
SCKV_EHIP = -3
SCKV_EWORKSPACE = -4

SCKV_FP4_E4M3_B16 = 0
SCKV_FP4_E8M0_B32 = 1

SCKV_OP_INDEX_SCORES_TOPK = 0
SCKV_OP_SPARSE_ATTN_SINK = 1
SCKV_OP_INDEX_SCORES_TOPK_FP4 = 2


class SckvError(RuntimeError):
    def __init__(self, call: str, code: int, msg: str):
        super().__init__(f"{call} failed ({code}): {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.sckv_quant.argtypes = [vp, vp, i64, i32, vp]
    L.sckv_quant_rows.argtypes = [vp, i64, vp, i64, i64, i64, i32, vp]
    L.sckv_quant_pack.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, i32, vp]
    L.sckv_ring_write.argtypes = [vp, i64, vp, i64, i32, i64, i64, i32, i32, vp]
    L.sckv_decode_prepare.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, i32, vp, i64, vp, i64, i32, i32,
                                      i32, i64, vp, i64, vp, i64, i32, i64, vp, i64, vp, i64, vp]
    L.sckv_prefill_prepare.argtypes = [i32, i64, i64, i32, i32, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, i32,
                                       i64, i64, vp, i64, i32, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                                       i32, i64, i32, ctypes.c_int32, vp]
    L.sckv_rope_quant_pack.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, vp, i64, i32, i64, i64, vp]
    L.sckv_yarn_freqs_cis.argtypes = [vp, i32, i64, i64, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                      ctypes.c_float]
    L.sckv_rope_quant_rows.argtypes = [vp, i64, vp, i64, i64, i64, vp, i64, i32, i64, i64, vp]
    L.sckv_rows_a_len.argtypes = [i32, i64, i64]
    L.sckv_rows_a_len.restype = i64
    L.sckv_window_idx.argtypes = [i32, i64, i64, i32, vp, i64, vp]
    L.sckv_visible_idx.argtypes = [i32, i64, i64, i32, i64, i32, ctypes.c_int32, vp, i64, i64, vp]
    L.sckv_index_scores_topk.argtypes = [vp, vp, vp, i32, i64, i32, i32, i64, i32, i64, i32, ctypes.c_int32, vp,
                                         i64, i64, vp, vp, sz, vp]
    L.sckv_index_scores_topk_fp4.argtypes = [vp, vp, vp, vp, i32, i64, i32, i32, i64, i32, i64, i32, ctypes.c_int32,
                                             vp, i64, i64, vp, vp, sz, vp]
    L.sckv_sparse_attn_sink.argtypes = [vp, vp, i64, vp, i64, vp, i32, vp, ctypes.c_float, i32, i64, i32, i32, vp,
                                        vp, sz, vp]
    L.sckv_decode_step.argtypes = [vp, vp, vp, vp, i64, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp,
                                   ctypes.c_float, i32, i32, i64, i32, i32, i64, vp, vp, vp, sz, vp]
    L.sckv_decode_step_workspace_bytes.argtypes = [i32, i32, i32, i64, i32]
    L.sckv_decode_step_workspace_bytes.restype = sz
    L.sckv_sparse_attn_sink_fp4.argtypes = [vp, vp, i64, vp, vp, i64, vp, i32, vp, ctypes.c_float, i32, i64, i32, i32,
                                            vp, vp, sz, vp]
    L.sckv_sparse_attn_sink_noalloc.argtypes = [vp, vp, i64, vp, i64, vp, i32, vp, ctypes.c_float, i32, i64, i32,
                                                i32, vp, vp]
    L.sckv_sparse_attn_sink_noalloc_max_bytes.argtypes = []
    L.sckv_sparse_attn_sink_noalloc_max_bytes.restype = sz
    L.sckv_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i64]
    L.sckv_workspace_bytes.restype = sz
    L.sckv_last_error.argtypes = []
    L.sckv_last_error.restype = ctypes.c_char_p
    L.sckv_abi_version.argtypes = []
    for name in ("sckv_quant", "sckv_quant_rows", "sckv_quant_pack", "sckv_ring_write", "sckv_decode_prepare",
                 "sckv_prefill_prepare",
                 "sckv_window_idx",
                 "sckv_visible_idx", "sckv_index_scores_topk", "sckv_index_scores_topk_fp4", "sckv_sparse_attn_sink",
                 "sckv_abi_version"):
        getattr(L, name).restype = ctypes.c_int
    return L


lib = _load()


def _check(call: str, rc: int):
    if rc != SCKV_OK:
        raise SckvError(call, rc, sckv_last_error())


def _ptr(t: torch.Tensor | None, dtype=None, name: str = "") -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def sckv_last_error() -> str:
    return lib.sckv_last_error().decode()


def sckv_abi_version() -> int:
    return lib.sckv_abi_version()


def sckv_workspace_bytes(op: int, B: int, m: int, H: int, D: int, n: int) -> int:
    return lib.sckv_workspace_bytes(op, B, m, H, D, n)


def workspace(op: int, B: int, m: int, H: int, D: int, n: int, device="cuda") -> torch.Tensor:
    """A device byte buffer of the size the library asks for (plumbing only)."""
    nbytes = sckv_workspace_bytes(op, B, m, H, D, n)
    if nbytes == ctypes.c_size_t(-1).value:
        raise SckvError("sckv_workspace_bytes", SCKV_EINVAL, "invalid arguments")
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def sckv_quant(x: torch.Tensor, y: torch.Tensor, mode: int, stream=None):
    if x.numel() != y.numel():
        raise ValueError("sckv_quant: x and y sizes differ")
    _check("sckv_quant", lib.sckv_quant(_ptr(x, torch.bfloat16, "x"), _ptr(y, torch.bfloat16, "y"), x.numel(), mode,
                                        _stream(stream)))


def sckv_quant_rows(x: torch.Tensor, ldx: int, y: torch.Tensor, ldy: int, rows: int, cols: int, mode: int,
                    stream=None):
    """x / y: any bf16 device tensors whose data pointers start the first row."""
    for t, n in ((x, "x"), (y, "y")):
        if not t.is_cuda or t.dtype != torch.bfloat16:
            raise ValueError(f"{n}: expected a bf16 device tensor")
    _check("sckv_quant_rows", lib.sckv_quant_rows(x.data_ptr(), ldx, y.data_ptr(), ldy, rows, cols, mode,
                                                  _stream(stream)))


def sckv_quant_pack(x: torch.Tensor, ldx: int, codes: torch.Tensor, ldc: int, scales: torch.Tensor, lds: int,
                    rows: int, cols: int, mode: int, stream=None):
    """x: bf16 device tensor; codes / scales: uint8 device tensors (row strides
    ldx in elements, ldc / lds in bytes)."""
    if not x.is_cuda or x.dtype != torch.bfloat16:
        raise ValueError("x: expected a bf16 device tensor")
    for t, n in ((codes, "codes"), (scales, "scales")):
        if not t.is_cuda or t.dtype != torch.uint8:
            raise ValueError(f"{n}: expected a uint8 device tensor")
    _check("sckv_quant_pack", lib.sckv_quant_pack(x.data_ptr(), ldx, codes.data_ptr(), ldc, scales.data_ptr(), lds,
                                                  rows, cols, mode, _stream(stream)))


def sckv_ring_write(rows: torch.Tensor, rows_bstride: int, ring: torch.Tensor, ring_bstride: int, B: int, m: int,
                    start_pos: int, win: int, D: int, stream=None):
    for t, n in ((rows, "rows"), (ring, "ring")):
        if not t.is_cuda or t.dtype != torch.bfloat16:
            raise ValueError(f"{n}: expected a bf16 device tensor")
    _check("sckv_ring_write", lib.sckv_ring_write(rows.data_ptr(), rows_bstride, ring.data_ptr(), ring_bstride, B, m,
                                                  start_pos, win, D, _stream(stream)))


def sckv_decode_prepare(lat_new, ld_lat_new: int, lat_dst, ld_lat_dst: int, k_new, ld_k_new: int, k_codes,
                        ld_codes: int, k_scales, ld_scales: int, Di: int, kv_new: torch.Tensor, ld_kv_new: int,
                        ring: torch.Tensor, ld_ring: int, B: int, D: int, win: int, start_pos: int,
                        idx: torch.Tensor, ld_idx: int, rope_table: torch.Tensor | None = None, rope_dim: int = 0,
                        lat_pos: int = 0, lat_codes=None, ld_lat_codes: int = 0, lat_scales=None,
                        ld_lat_scales: int = 0, stream=None):
    """Row arguments: device tensors whose data pointers start the first row
    (lat_new / lat_dst / k_new / k_codes / k_scales / rope_table may be None;
    rope_table is the [n_pos, rope_dim/2, 2] f32 device table)."""
    def p(t, dtype, name):
        if t is None:
            return None
        if not t.is_cuda or t.dtype != dtype:
            raise ValueError(f"{name}: expected a {dtype} device tensor")
        return t.data_ptr()
    _check("sckv_decode_prepare", lib.sckv_decode_prepare(
        p(lat_new, torch.bfloat16, "lat_new"), ld_lat_new, p(lat_dst, torch.bfloat16, "lat_dst"), ld_lat_dst,
        p(k_new, torch.bfloat16, "k_new"), ld_k_new, p(k_codes, torch.uint8, "k_codes"), ld_codes,
        p(k_scales, torch.uint8, "k_scales"), ld_scales, Di, p(kv_new, torch.bfloat16, "kv_new"), ld_kv_new,
        p(ring, torch.bfloat16, "ring"), ld_ring, B, D, win, start_pos, p(idx, torch.int32, "idx"), ld_idx,
        p(rope_table, torch.float32, "rope_table"), 0 if rope_table is None else rope_table.shape[0], rope_dim,
        lat_pos, p(lat_codes, torch.uint8, "lat_codes"), ld_lat_codes, p(lat_scales, torch.uint8, "lat_scales"),
        ld_lat_scales, _stream(stream)))


def sckv_prefill_prepare(B: int, m: int, start_pos: int, win: int, D: int, n_new: int, lat_new, bs_lat_new: int,
                         lat_dst, bs_lat_dst: int, lat_codes, bs_lat_codes: int, lat_scales, bs_lat_scales: int,
                         rope_table, rope_dim: int, pos0: int, pos_step: int, k_new, bs_k_new: int, Di: int, k_dst,
                         bs_k_dst: int, k_codes, bs_k_codes: int, k_scales, bs_k_scales: int, ring_src,
                         bs_ring_src: int, ring, bs_ring: int, idx: torch.Tensor, ld_idx: int, ratio: int = 1,
                         n_c: int = 0, K: int = 0, offset: int = 0, stream=None):
    """Row arguments: device tensors whose data pointers start sequence 0's
    first row (any of the optional parts may be None); rope_table is the
    [n_pos, rope_dim/2, 2] f32 device table or None."""
    def p(t, dtype, name):
        if t is None:
            return None
        if not t.is_cuda or t.dtype != dtype:
            raise ValueError(f"{name}: expected a {dtype} device tensor")
        return t.data_ptr()
    bf, u8 = torch.bfloat16, torch.uint8
    _check("sckv_prefill_prepare", lib.sckv_prefill_prepare(
        B, m, start_pos, win, D, n_new, p(lat_new, bf, "lat_new"), bs_lat_new, p(lat_dst, bf, "lat_dst"), bs_lat_dst,
        p(lat_codes, u8, "lat_codes"), bs_lat_codes, p(lat_scales, u8, "lat_scales"), bs_lat_scales,
        p(rope_table, torch.float32, "rope_table"), 0 if rope_table is None else rope_table.shape[0], rope_dim, pos0,
        pos_step, p(k_new, bf, "k_new"), bs_k_new, Di, p(k_dst, bf, "k_dst"), bs_k_dst, p(k_codes, u8, "k_codes"),
        bs_k_codes, p(k_scales, u8, "k_scales"), bs_k_scales, p(ring_src, bf, "ring_src"), bs_ring_src,
        p(ring, bf, "ring"), bs_ring, p(idx, torch.int32, "idx"), ld_idx, ratio, n_c, K, offset, _stream(stream)))


def sckv_yarn_freqs_cis(dim: int, seqlen: int, original_seq_len: int, base: float, factor: float, beta_fast: float,
                        beta_slow: float) -> torch.Tensor:
    """The rotation table, built on the host by the library: a CPU f32 tensor
    [seqlen, dim/2, 2] (copy it to the device for the rotating calls)."""
    t = torch.empty((seqlen, dim // 2, 2), dtype=torch.float32)
    _check("sckv_yarn_freqs_cis", lib.sckv_yarn_freqs_cis(t.data_ptr(), dim, seqlen, original_seq_len, base, factor,
                                                          beta_fast, beta_slow))
    return t


def sckv_rope_quant_rows(x: torch.Tensor, ldx: int, y: torch.Tensor, ldy: int, rows: int, cols: int,
                         table: torch.Tensor, rope_dim: int, pos0: int, pos_step: int, stream=None):
    """x / y: bf16 device tensors whose data pointers start the first row;
    table: the [n_pos, rope_dim/2, 2] f32 device table."""
    for t, n in ((x, "x"), (y, "y")):
        if not t.is_cuda or t.dtype != torch.bfloat16:
            raise ValueError(f"{n}: expected a bf16 device tensor")
    _check("sckv_rope_quant_rows", lib.sckv_rope_quant_rows(
        x.data_ptr(), ldx, y.data_ptr(), ldy, rows, cols, _ptr(table, torch.float32, "table"), table.shape[0],
        rope_dim, pos0, pos_step, _stream(stream)))


def sckv_rope_quant_pack(x: torch.Tensor, ldx: int, codes: torch.Tensor, ldc: int, scales: torch.Tensor, lds: int,
                         rows: int, cols: int, table: torch.Tensor, rope_dim: int, pos0: int, pos_step: int,
                         stream=None):
    """x: bf16 device tensor; codes / scales: uint8 device tensors, each
    tensor's data pointer at its first row; table: [n_pos, rope_dim/2, 2] f32."""
    if not x.is_cuda or x.dtype != torch.bfloat16:
        raise ValueError("x: expected a bf16 device tensor")
    for t, n in ((codes, "codes"), (scales, "scales")):
        if not t.is_cuda or t.dtype != torch.uint8:
            raise ValueError(f"{n}: expected a uint8 device tensor")
    _check("sckv_rope_quant_pack", lib.sckv_rope_quant_pack(
        x.data_ptr(), ldx, codes.data_ptr(), ldc, scales.data_ptr(), lds, rows, cols,
        _ptr(table, torch.float32, "table"), table.shape[0], rope_dim, pos0, pos_step, _stream(stream)))


def sckv_rows_a_len(win: int, m: int, start_pos: int) -> int:
    return lib.sckv_rows_a_len(win, m, start_pos)


def sckv_window_idx(B: int, m: int, start_pos: int, win: int, idx: torch.Tensor, ld: int, stream=None):
    _check("sckv_window_idx", lib.sckv_window_idx(B, m, start_pos, win, _ptr(idx, torch.int32, "idx"), ld,
                                                  _stream(stream)))


def sckv_visible_idx(B: int, m: int, start_pos: int, ratio: int, n_c: int, K: int, offset: int, idx: torch.Tensor,
                     ld: int, col0: int, stream=None):
    _check("sckv_visible_idx", lib.sckv_visible_idx(B, m, start_pos, ratio, n_c, K, offset,
                                                    _ptr(idx, torch.int32, "idx"), ld, col0, _stream(stream)))


def sckv_index_scores_topk(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, B: int, m: int, Hi: int, Di: int,
                           n_c: int, ratio: int, start_pos: int, K: int, offset: int, idx: torch.Tensor, ld: int,
                           col0: int, scores: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                           stream=None):
    if ws is None:
        ws = workspace(SCKV_OP_INDEX_SCORES_TOPK, B, m, Hi, Di, n_c, device=idx.device)
    _check("sckv_index_scores_topk", lib.sckv_index_scores_topk(
        _ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"), _ptr(w, torch.float32, "w"), B, m, Hi, Di, n_c,
        ratio, start_pos, K, offset, _ptr(idx, torch.int32, "idx"), ld, col0, _ptr(scores, torch.bfloat16, "scores"),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def sckv_index_scores_topk_fp4(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, w: torch.Tensor, B: int,
                               m: int, Hi: int, Di: int, n_c: int, ratio: int, start_pos: int, K: int, offset: int,
                               idx: torch.Tensor, ld: int, col0: int, scores: torch.Tensor | None = None,
                               ws: torch.Tensor | None = None, stream=None):
    if ws is None:
        ws = workspace(SCKV_OP_INDEX_SCORES_TOPK_FP4, B, m, Hi, Di, n_c, device=idx.device)
    _check("sckv_index_scores_topk_fp4", lib.sckv_index_scores_topk_fp4(
        _ptr(q, torch.bfloat16, "q"), _ptr(k_codes, torch.uint8, "k_codes"), _ptr(k_scales, torch.uint8, "k_scales"),
        _ptr(w, torch.float32, "w"), B, m, Hi, Di, n_c, ratio, start_pos, K, offset, _ptr(idx, torch.int32, "idx"),
        ld, col0, _ptr(scores, torch.bfloat16, "scores"), _ptr(ws, None, "ws"), ws.numel() * ws.element_size(),
        _stream(stream)))


def sckv_sparse_attn_sink(q: torch.Tensor, rows_a: torch.Tensor, ra: int, rows_b: torch.Tensor | None, rb: int,
                          idx: torch.Tensor, T: int, sink: torch.Tensor, scale: float, B: int, m: int, H: int, D: int,
                          out: torch.Tensor, ws: torch.Tensor | None = None, stream=None):
    if ws is None:
        ws = workspace(SCKV_OP_SPARSE_ATTN_SINK, B, m, H, D, T, device=out.device)
    _check("sckv_sparse_attn_sink", lib.sckv_sparse_attn_sink(
        _ptr(q, torch.bfloat16, "q"), _ptr(rows_a, torch.bfloat16, "rows_a"), ra,
        _ptr(rows_b, torch.bfloat16, "rows_b"), rb, _ptr(idx, torch.int32, "idx"), T,
        _ptr(sink, torch.float32, "sink"), float(scale), B, m, H, D, _ptr(out, torch.bfloat16, "out"),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def sckv_sparse_attn_sink_noalloc(q: torch.Tensor, rows_a: torch.Tensor, ra: int, rows_b: torch.Tensor | None,
                                  rb: int, idx: torch.Tensor, T: int, sink: torch.Tensor, scale: float, B: int, m: int,
                                  H: int, D: int, out: torch.Tensor, stream=None):
    _check("sckv_sparse_attn_sink_noalloc", lib.sckv_sparse_attn_sink_noalloc(
        _ptr(q, torch.bfloat16, "q"), _ptr(rows_a, torch.bfloat16, "rows_a"), ra,
        _ptr(rows_b, torch.bfloat16, "rows_b"), rb, _ptr(idx, torch.int32, "idx"), T,
        _ptr(sink, torch.float32, "sink"), float(scale), B, m, H, D, _ptr(out, torch.bfloat16, "out"),
        _stream(stream)))


def sckv_sparse_attn_sink_noalloc_max_bytes() -> int:
    return int(lib.sckv_sparse_attn_sink_noalloc_max_bytes())


def sckv_sparse_attn_sink_fp4(q: torch.Tensor, rows_a: torch.Tensor, ra: int, rows_b_codes: torch.Tensor | None,
                              rows_b_scales: torch.Tensor | None, rb: int, idx: torch.Tensor, T: int,
                              sink: torch.Tensor, scale: float, B: int, m: int, H: int, D: int, out: torch.Tensor,
                              ws: torch.Tensor | None = None, stream=None):
    if ws is None:
        ws = workspace(SCKV_OP_SPARSE_ATTN_SINK, B, m, H, D, T, device=out.device)
    _check("sckv_sparse_attn_sink_fp4", lib.sckv_sparse_attn_sink_fp4(
        _ptr(q, torch.bfloat16, "q"), _ptr(rows_a, torch.bfloat16, "rows_a"), ra,
        _ptr(rows_b_codes, torch.uint8, "rows_b_codes"), _ptr(rows_b_scales, torch.uint8, "rows_b_scales"), rb,
        _ptr(idx, torch.int32, "idx"), T, _ptr(sink, torch.float32, "sink"), float(scale), B, m, H, D,
        _ptr(out, torch.bfloat16, "out"), _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def sckv_decode_step_workspace_bytes(B: int, H: int, D: int, n_c: int, T: int) -> int:
    return int(lib.sckv_decode_step_workspace_bytes(B, H, D, n_c, T))


def sckv_decode_step(lat_new, k_new, kv_new: torch.Tensor, rope_table: torch.Tensor | None, rope_dim: int,
                     latent: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, ring: torch.Tensor,
                     iq: torch.Tensor, w: torch.Tensor, Hi: int, Di: int, ratio: int, K: int, q: torch.Tensor,
                     sink: torch.Tensor, scale: float, H: int, B: int, n_c: int, D: int, win: int, start_pos: int,
                     idx: torch.Tensor, out: torch.Tensor, ws: torch.Tensor | None = None, stream=None):
    """All tensors contiguous device tensors (lat_new / k_new / rope_table may be None)."""
    if ws is None:
        nb = sckv_decode_step_workspace_bytes(B, H, D, n_c, win + K)
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=out.device)  # barrier words start at zero
    _check("sckv_decode_step", lib.sckv_decode_step(
        _ptr(lat_new, torch.bfloat16, "lat_new"), _ptr(k_new, torch.bfloat16, "k_new"),
        _ptr(kv_new, torch.bfloat16, "kv_new"), _ptr(rope_table, torch.float32, "rope_table"),
        0 if rope_table is None else rope_table.shape[0], rope_dim, _ptr(latent, torch.bfloat16, "latent"),
        _ptr(k_codes, torch.uint8, "k_codes"), _ptr(k_scales, torch.uint8, "k_scales"),
        _ptr(ring, torch.bfloat16, "ring"), _ptr(iq, torch.bfloat16, "iq"), _ptr(w, torch.float32, "w"), Hi, Di,
        ratio, K, _ptr(q, torch.bfloat16, "q"), _ptr(sink, torch.float32, "sink"), float(scale), H, B, n_c, D, win,
        start_pos, _ptr(idx, torch.int32, "idx"), _ptr(out, torch.bfloat16, "out"), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)))

"""Python face of the plain C oracle (oracle/sckv_oracle.c).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the bench's
CPU-baseline leg import this module; the product path never does.  It imports
nothing from the HIP package and shares no code with it.

Arrays are numpy: bf16 values as uint16 bit patterns, indices as int32,
sinks / indexer weights as float32, attention outputs as float64.
Citations are to the pages "metrale_model_arch/deepseek_v41_ref/compress.rs"
(compress.rs) and "metrale_model_arch/attn_v41/forward.rs" (forward.rs).
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsckv_oracle.so")

_lib = None

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_int = ctypes.c_int


def lib():
    """Load (building first if needed) the oracle's shared library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from oracle.build import build  # noqa: PLC0415

        build()
    L = ctypes.CDLL(LIB_PATH)
    L.sckvo_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.sckvo_bf16_to_f32.restype = ctypes.c_float
    L.sckvo_f32_to_bf16.argtypes = [ctypes.c_float]
    L.sckvo_f32_to_bf16.restype = ctypes.c_uint16
    L.sckvo_e2m1_rne.argtypes = [ctypes.c_float]
    L.sckvo_e2m1_rne.restype = ctypes.c_float
    L.sckvo_pow2_ceil.argtypes = [ctypes.c_float]
    L.sckvo_pow2_ceil.restype = ctypes.c_float
    L.sckvo_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    L.sckvo_e4m3_to_f32.restype = ctypes.c_float
    L.sckvo_f32_to_e4m3.argtypes = [ctypes.c_float]
    L.sckvo_f32_to_e4m3.restype = ctypes.c_uint8
    L.sckvo_quant_e8m0.argtypes = [_u16p, _u16p, _i64, _i64]
    L.sckvo_quant_e8m0.restype = None
    L.sckvo_quant_e4m3.argtypes = [_u16p, _u16p, _i64, _i64]
    L.sckvo_quant_e4m3.restype = None
    L.sckvo_pack_fp4.argtypes = [_u16p, _i64, _i64, _int, _u8p, _u8p]
    L.sckvo_pack_fp4.restype = None
    L.sckvo_unpack_fp4.argtypes = [_u8p, _u8p, _i64, _i64, _int, _u16p]
    L.sckvo_unpack_fp4.restype = None
    L.sckvo_ring_write.argtypes = [_u16p, _int, _int, _u16p, _i64, _i64]
    L.sckvo_ring_write.restype = None
    L.sckvo_rows_a_len.argtypes = [_int, _i64, _i64]
    L.sckvo_rows_a_len.restype = _i64
    L.sckvo_window_idx.argtypes = [_int, _i64, _i64, _i32p, _i64]
    L.sckvo_window_idx.restype = _i64
    L.sckvo_visible.argtypes = [_i64, _int, _i64]
    L.sckvo_visible.restype = _i64
    L.sckvo_visible_idx.argtypes = [_i64, _i64, _int, _i64, _int, ctypes.c_int32, _i32p, _i64, _i64]
    L.sckvo_visible_idx.restype = None
    L.sckvo_index_scores.argtypes = [_u16p, _u16p, _f32p, _i64, _int, _int, _i64, _int, _i64, _i64p, _i64, _u16p]
    L.sckvo_index_scores.restype = _i64
    L.sckvo_topk.argtypes = [_u16p, _i64, _int, ctypes.c_int32, _i32p]
    L.sckvo_topk.restype = None
    L.sckvo_sparse_attn.argtypes = [_u16p, _u16p, _i64, _u16p, _i64, _i32p, _int, _f32p, ctypes.c_float, _int, _int,
                                    _i64p, _i64, _f64p]
    L.sckvo_sparse_attn.restype = _int
    L.sckvo_yarn_freqs_cis.argtypes = [_int, _i64, _i64, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_float, _f32p]
    L.sckvo_yarn_freqs_cis.restype = None
    L.sckvo_latent_position.argtypes = [_i64, _int]
    L.sckvo_latent_position.restype = _i64
    L.sckvo_rope_rows.argtypes = [_u16p, _i64, _int, _int, _f32p, _i64, _i64p, _int, _u16p]
    L.sckvo_rope_rows.restype = _int
    _lib = L
    return L


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


# --- scalar helpers -------------------------------------------------------

def bf16_to_f32(bits: int) -> float:
    return lib().sckvo_bf16_to_f32(int(bits))


def f32_to_bf16(x: float) -> int:
    """bf16 round-to-nearest-even of a binary32 value (compress.rs: to_bf16_rne)."""
    return lib().sckvo_f32_to_bf16(float(np.float32(x)))


def e2m1_rne(y: float) -> float:
    """compress.rs: to_e2m1_rne -- nearest e2m1 magnitude, ties to the even code, sign kept."""
    return lib().sckvo_e2m1_rne(float(np.float32(y)))


def pow2_ceil(x: float) -> float:
    return lib().sckvo_pow2_ceil(float(np.float32(x)))


def f32_to_e4m3(x: float) -> int:
    return lib().sckvo_f32_to_e4m3(float(np.float32(x)))


def e4m3_to_f32(code: int) -> float:
    return lib().sckvo_e4m3_to_f32(int(code))


# --- the two fp4 round trips (compress.rs: fp4_quant_e8m0_inplace / _e4m3_) --

E8M0_B32 = "e8m0_b32"
E4M3_B16 = "e4m3_b16"


def quant(x_bits, mode: str, block: int | None = None):
    """fp4 (e2m1) round trip of a flat bf16 array; returns new uint16 bits.

    mode E8M0_B32: power-of-two scales, block 32 (indexer q and k);
    mode E4M3_B16: e4m3 scales, block 16 (compressed KV latent)."""
    x = _u16(x_bits).reshape(-1)
    y = np.empty_like(x)
    if mode == E8M0_B32:
        lib().sckvo_quant_e8m0(x, y, x.size, block or 32)
    elif mode == E4M3_B16:
        lib().sckvo_quant_e4m3(x, y, x.size, block or 16)
    else:
        raise ValueError(mode)
    return y.reshape(np.shape(x_bits))


def pack(x_bits, mode: str):
    """Packed storage of the round trip of a flat bf16 array: (codes uint8
    [n/2], two 4-bit e2m1 codes a byte, the even element in the low nibble;
    scales uint8 [n/block], E8M0 exponents or E4M3 codes)."""
    x = _u16(x_bits).reshape(-1)
    block, m = (32, 1) if mode == E8M0_B32 else (16, 0)
    if x.size % block:
        raise ValueError("size is not a multiple of the block")
    codes = np.zeros(x.size // 2, dtype=np.uint8)
    scales = np.zeros(x.size // block, dtype=np.uint8)
    lib().sckvo_pack_fp4(x, x.size, block, m, codes, scales)
    return codes, scales


def unpack(codes, scales, n: int, mode: str):
    """bf16 bits of the values packed codes and scales stand for."""
    block, m = (32, 1) if mode == E8M0_B32 else (16, 0)
    y = np.empty(n, dtype=np.uint16)
    lib().sckvo_unpack_fp4(np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1),
                           np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1), n, block, m, y)
    return y


# --- window ring, window rows, visibility (forward.rs ring copies) ---------

def ring_write(ring_bits, rows_bits, start_pos: int):
    """Write m new kv rows into the ring (slot = position mod win); returns the new ring."""
    ring = _u16(ring_bits).copy()
    win, D = ring.shape
    rows = _u16(rows_bits).reshape(-1, D)
    lib().sckvo_ring_write(ring, win, D, rows, rows.shape[0], start_pos)
    return ring


def rows_a_len(win: int, m: int, start_pos: int) -> int:
    return lib().sckvo_rows_a_len(win, m, start_pos)


def window_idx(win: int, m: int, start_pos: int):
    """[m, win] int32 window rows per query and rows_a's length."""
    idx = np.zeros((m, win), dtype=np.int32)
    ra = lib().sckvo_window_idx(win, m, start_pos, idx, win)
    return idx, ra


def visible(p: int, ratio: int, n_c: int) -> int:
    return lib().sckvo_visible(p, ratio, n_c)


def visible_idx(m: int, start_pos: int, ratio: int, n_c: int, K: int, offset: int):
    idx = np.zeros((m, K), dtype=np.int32)
    lib().sckvo_visible_idx(m, start_pos, ratio, n_c, K, offset, idx, K, 0)
    return idx


# --- indexer scores and top-k ----------------------------------------------

def index_scores(q_raw_bits, k_hat_bits, w, start_pos: int, ratio: int, qsel=None):
    """Indexer scores (bf16 bits) [len(qsel), n_c]; invisible rows hold 0xffff.

    q_raw_bits [m, Hi, Di] raw (the round trip is applied here), k_hat_bits
    [n_c, Di] already round-tripped, w float32 [m, Hi].  Returns (scores,
    number of inexact dots)."""
    q = _u16(q_raw_bits)
    m, Hi, Di = q.shape
    k = _u16(k_hat_bits)
    n_c = k.shape[0]
    w = np.ascontiguousarray(w, dtype=np.float32)
    qsel = np.arange(m, dtype=np.int64) if qsel is None else np.ascontiguousarray(qsel, dtype=np.int64)
    out = np.zeros((qsel.size, n_c), dtype=np.uint16)
    bad = lib().sckvo_index_scores(q, k, w, m, Hi, Di, n_c, ratio, start_pos, qsel, qsel.size, out)
    return out, bad


def topk(score_bits, visible_rows: int, K: int, offset: int):
    """Top-k of one query's scores over rows 0..visible_rows-1, ties to the lower row."""
    s = _u16(score_bits).reshape(-1)
    out = np.zeros(K, dtype=np.int32)
    lib().sckvo_topk(s, visible_rows, K, offset, out)
    return out


# --- sparse MQA attention with a sink --------------------------------------

def sparse_attn(q_bits, rows_a_bits, rows_b_bits, idx, sink, scale: float, qsel=None):
    """binary64 [len(qsel), H, D] outputs of sparse attention with a per-head sink."""
    q = _u16(q_bits)
    m, H, D = q.shape
    ra_rows = _u16(rows_a_bits).reshape(-1, D)
    rb_rows = _u16(rows_b_bits).reshape(-1, D) if rows_b_bits is not None else np.zeros((0, D), np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T = idx.shape[1]
    sink = np.ascontiguousarray(sink, dtype=np.float32)
    qsel = np.arange(m, dtype=np.int64) if qsel is None else np.ascontiguousarray(qsel, dtype=np.int64)
    out = np.zeros((qsel.size, H, D), dtype=np.float64)
    rb_arg = rb_rows if rb_rows.size else np.zeros((1, D), np.uint16)
    rc = lib().sckvo_sparse_attn(q, ra_rows, ra_rows.shape[0], rb_arg, rb_rows.shape[0], idx, T, sink,
                                 float(np.float32(scale)), H, D, qsel, qsel.size, out)
    if rc != 0:
        raise ValueError("oracle: index out of range")
    return out


# --- one step of the whole path --------------------------------------------

def compressed_idx(q_raw_bits, k_hat_bits, w, start_pos: int, ratio: int, K: int, offset: int, qsel=None):
    """The compressed half of each selected query's index list: top-K of the
    indexer scores, offset added, -1 padded.  Returns (idx [nsel, K], inexact)."""
    q = _u16(q_raw_bits)
    m = q.shape[0]
    n_c = _u16(k_hat_bits).shape[0]
    qsel = np.arange(m, dtype=np.int64) if qsel is None else np.asarray(qsel, dtype=np.int64)
    scores, bad = index_scores(q, k_hat_bits, w, start_pos, ratio, qsel)
    out = np.zeros((qsel.size, K), dtype=np.int32)
    for i, t in enumerate(qsel):
        v = visible(start_pos + int(t), ratio, n_c)
        out[i] = topk(scores[i], v, K, offset)
    return out, bad


# --- YaRN RoPE of the compressed latent (compress.rs yarn_freqs_cis; the rope
# of a new latent group before its fp4 round trip and cache copy) -----------

def yarn_freqs_cis(dim: int, seqlen: int, original_seq_len: int, base: float, factor: float, beta_fast: float,
                   beta_slow: float):
    """float32 [seqlen, dim/2, 2] table of (cos, sin) per position and pair."""
    out = np.zeros((seqlen, dim // 2, 2), dtype=np.float32)
    lib().sckvo_yarn_freqs_cis(dim, seqlen, original_seq_len, base, factor, beta_fast, beta_slow, out)
    return out


def latent_position(j: int, ratio: int) -> int:
    """Position of compressed row j: the first position of its group."""
    return lib().sckvo_latent_position(j, ratio)


def rope_rows(x_bits, rope_dim: int, table, pos, inverse: bool = False):
    """bf16 bits of the rows x [rows, cols] with their last rope_dim values
    rotated at the positions pos [rows] (interleaved pairs)."""
    x = _u16(x_bits)
    rows, cols = x.shape
    t = np.ascontiguousarray(table, dtype=np.float32)
    pos = np.ascontiguousarray(pos, dtype=np.int64).reshape(-1)
    y = np.empty_like(x)
    if lib().sckvo_rope_rows(x, rows, cols, rope_dim, t.reshape(-1), t.shape[0], pos, int(inverse), y) != 0:
        raise ValueError("oracle: position outside the rotation table")
    return y


def latent_rope_quant(x_bits, rope_dim: int, table, pos):
    """The latent path of a new compressed row: rotate (bf16 result), then the
    e4m3-scale fp4 round trip."""
    r = rope_rows(x_bits, rope_dim, table, pos)
    return quant(r.reshape(-1), E4M3_B16).reshape(r.shape)

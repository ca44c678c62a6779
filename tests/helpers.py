"""Shared helpers of the tests: bit views and the oracle's reference step.

The reference step calls only oracle/ (plain C, CPU) on the raw seeded inputs;
it never sees a value produced by the HIP path.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import oracle


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (moved to the CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, device="cpu") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def vals(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def oracle_rows_a(w, x, b: int) -> np.ndarray:
    """rows_a of instance b as the step sees it (fresh rows, ring after the
    new row's write, or ring then chunk)."""
    kv = bits(x["kv_new"][b])
    if w.start_pos == 0:
        return kv
    ring = bits(x["ring"][b])
    if w.m == 1:
        return oracle.ring_write(ring, kv, w.start_pos)
    return np.concatenate([ring, kv], axis=0)


def oracle_rope_table(w):
    return oracle.yarn_freqs_cis(w.rope_dim, w.rope_positions, w.rope_orig_len, w.rope_base, w.rope_factor,
                                 w.rope_beta_fast, w.rope_beta_slow)


def oracle_latent(w, x, b: int) -> np.ndarray:
    """The latent cache after the step: every compressed row j turned at its
    position j * ratio, then round-tripped (the rows before this step as
    earlier steps left them, the new ones as this step writes them)."""
    pos = np.array([oracle.latent_position(j, w.ratio) for j in range(w.n_c)], dtype=np.int64)
    return oracle.latent_rope_quant(bits(x["latent_raw"][b]).reshape(w.n_c, w.D), w.rope_dim, oracle_rope_table(w),
                                    pos)


def oracle_threads() -> int:
    """Worker threads for oracle calls over many queries (the oracle releases
    the GIL inside its C calls; each query's result is independent of the
    others, so splitting the queries changes nothing)."""
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(fn, qsel, threads):
    """fn(sub-array of qsel) over contiguous chunks, results concatenated."""
    if threads <= 1 or qsel.size < 2 * threads:
        return fn(qsel)
    parts = np.array_split(qsel, threads * 4)
    with ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(fn, [p for p in parts if p.size]))
    return np.concatenate(res, axis=0)


def oracle_step(w, x, b: int = 0, qsel=None, attn_qsel=None, threads: int = 1):
    """The oracle's index lists [len(qsel), T] and float64 attention outputs
    [len(attn_qsel), H, D] (attn_qsel defaults to qsel) for instance b of a
    step of workload w; threads > 1 splits the queries over worker threads."""
    qsel = np.arange(w.m, dtype=np.int64) if qsel is None else np.asarray(qsel, dtype=np.int64)
    attn_qsel = qsel if attn_qsel is None else np.asarray(attn_qsel, dtype=np.int64)
    latent = oracle_latent(w, x, b)
    rows_a = oracle_rows_a(w, x, b)
    widx, ra = oracle.window_idx(w.win, w.m, w.start_pos)
    assert ra == rows_a.shape[0]
    need = np.union1d(qsel, attn_qsel)
    if w.Hi:
        k = oracle.quant(bits(x["ik_raw"][b]).reshape(-1), oracle.E8M0_B32).reshape(w.n_c, w.Di)
        iq, iw = bits(x["iq"][b]), x["iw"][b].numpy()

        def comp(sel):
            c, inexact = oracle.compressed_idx(iq, k, iw, w.start_pos, w.ratio, w.K, ra, sel)
            assert inexact == 0, "indexer dot outside the exactness condition"
            return c

        cidx = _chunked(comp, need, threads)
    else:
        cidx = oracle.visible_idx(w.m, w.start_pos, w.ratio, w.n_c, w.K, ra)[need]
    idx_need = np.concatenate([widx[need], cidx], axis=1).astype(np.int32)
    idx_full = np.full((w.m, w.T), -1, dtype=np.int32)
    idx_full[need] = idx_need
    q, sink = bits(x["q"][b]), x["sink"].numpy()
    out = _chunked(lambda sel: oracle.sparse_attn(q, rows_a, latent, idx_full, sink, w.scale, sel), attn_qsel,
                   threads)
    return idx_full[qsel], out


def attn_tolerance_ok(gpu: np.ndarray, ref: np.ndarray):
    """|gpu - oracle| <= 1e-2 * max|oracle| + 1e-3 elementwise, max over the
    compared outputs.  Returns (ok, worst excess ratio)."""
    bound = 1e-2 * np.abs(ref).max() + 1e-3
    err = np.abs(gpu.astype(np.float64) - ref)
    return bool(np.all(err <= bound)), float(err.max() / bound)


def spread_queries(w, n: int = 256):
    """About n queries spread evenly over the step (first and last included),
    plus the edge cases of sample_queries."""
    grid = np.unique(np.linspace(0, w.m - 1, min(n, w.m)).round().astype(np.int64))
    return np.union1d(grid, sample_queries(w))


def sample_queries(w, extra: int = 4, seed: int = 0):
    """Queries the oracle can afford at full size: edges of the window and of
    the visibility ramp, plus a few seeded random ones."""
    m = w.m
    fixed = [0, 1, 2, 3, 4, w.win - 1, w.win, w.win + 1, m // 2, m - 2, m - 1]
    if w.Hi:
        r = w.ratio
        fixed += [w.K * r - 1 - w.start_pos, w.K * r - w.start_pos]  # around V = K
    rng = np.random.default_rng(seed)
    fixed += list(rng.integers(0, m, size=extra))
    return np.array(sorted({int(t) for t in fixed if 0 <= t < m}), dtype=np.int64)

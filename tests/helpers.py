"""Shared helpers of the tests: bit views and the oracle's reference step.

The reference step calls only oracle/ (plain C, CPU) on the raw seeded inputs;
it never sees a value produced by the HIP path.
"""
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


def oracle_step(w, x, b: int = 0, qsel=None):
    """The oracle's index lists [len(qsel), T] and float64 outputs
    [len(qsel), H, D] for instance b of a step of workload w."""
    qsel = np.arange(w.m, dtype=np.int64) if qsel is None else np.asarray(qsel, dtype=np.int64)
    latent = oracle.quant(bits(x["latent_raw"][b]).reshape(-1), oracle.E4M3_B16).reshape(w.n_c, w.D)
    rows_a = oracle_rows_a(w, x, b)
    widx, ra = oracle.window_idx(w.win, w.m, w.start_pos)
    assert ra == rows_a.shape[0]
    if w.Hi:
        k = oracle.quant(bits(x["ik_raw"][b]).reshape(-1), oracle.E8M0_B32).reshape(w.n_c, w.Di)
        cidx, inexact = oracle.compressed_idx(bits(x["iq"][b]), k, x["iw"][b].numpy(), w.start_pos, w.ratio, w.K, ra,
                                              qsel)
        assert inexact == 0, "indexer dot outside the exactness condition"
    else:
        cidx = oracle.visible_idx(w.m, w.start_pos, w.ratio, w.n_c, w.K, ra)[qsel]
    idx_sel = np.concatenate([widx[qsel], cidx], axis=1).astype(np.int32)
    idx_full = np.full((w.m, w.T), -1, dtype=np.int32)
    idx_full[qsel] = idx_sel
    out = oracle.sparse_attn(bits(x["q"][b]), rows_a, latent, idx_full, x["sink"].numpy(), w.scale, qsel)
    return idx_sel, out


def attn_tolerance_ok(gpu: np.ndarray, ref: np.ndarray):
    """|gpu - oracle| <= 1e-2 * max|oracle| + 1e-3 elementwise, max over the
    compared outputs.  Returns (ok, worst excess ratio)."""
    bound = 1e-2 * np.abs(ref).max() + 1e-3
    err = np.abs(gpu.astype(np.float64) - ref)
    return bool(np.all(err <= bound)), float(err.max() / bound)


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

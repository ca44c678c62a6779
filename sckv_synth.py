"""Seeded synthetic inputs and the workload table.

This module is shared by the tests, the bench and the smoke check.  It holds
workload shapes and a seeded normal generator only -- none of the method's
arithmetic (no quantisation, no scoring, no attention).  Every tensor is
drawn from its own torch CPU generator whose seed is derived from
(seed, workload name, tensor name), so the same bytes feed the HIP path and
the oracle.

Value recipe (the pages give dtypes and shapes but print no data):
  q, kv / ring / chunk rows, raw latent rows, raw indexer q and k: N(0, 1)
      drawn in float32 and rounded to bf16 (torch's round-to-nearest-even);
  indexer head weights w: N(0, 1) * (Hi * Di) ** -0.5 in float32;
  sink logits: N(0, 1) in float32.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    m: int            # tokens this step
    start_pos: int    # position of the first token
    H: int            # query heads (MQA: one shared kv row per position)
    D: int            # head dim = latent row width
    win: int          # window ring rows
    ratio: int        # positions per compressed row
    n_c: int          # compressed rows after this step = (start_pos + m) // ratio
    Hi: int           # indexer heads (0: no indexer, every visible row attended)
    Di: int           # indexer head dim
    K: int            # compressed columns of the index list (top-k, or all visible)
    seed: int = 0
    # rotary embedding of the latent rows (the last rope_dim values of a row;
    # YaRN table parameters -- the pages print none, these are the model
    # family's published settings)
    rope_dim: int = 64
    rope_base: float = 10000.0
    rope_factor: float = 40.0
    rope_orig_len: int = 4096
    rope_beta_fast: float = 32.0
    rope_beta_slow: float = 1.0

    @property
    def T(self) -> int:
        """Columns of the merged index list: window then compressed."""
        return self.win + self.K

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(D), as binary32."""
        return float(torch.tensor(float(self.D), dtype=torch.float32).pow(-0.5).item())

    @property
    def rope_positions(self) -> int:
        """Rows of the rotation table a step needs: compressed row j sits at
        position j * ratio."""
        return max(1, (self.n_c - 1) * self.ratio + 1)

    @property
    def first_new_row(self) -> int:
        """First compressed row completed by this step (cache row start_pos // ratio)."""
        return self.start_pos // self.ratio

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the hot path (shapes, derived values checked in tests).
WORKLOADS = {
    "tiny_decode": Workload("tiny_decode", m=1, start_pos=255, H=8, D=64, win=16, ratio=4, n_c=64,
                            Hi=4, Di=32, K=16, rope_dim=8),
    "decode": Workload("decode", m=1, start_pos=32767, H=64, D=512, win=128, ratio=4, n_c=8192,
                       Hi=64, Di=128, K=512),
    "long_decode": Workload("long_decode", m=1, start_pos=131071, H=64, D=512, win=128, ratio=4, n_c=32768,
                            Hi=64, Di=128, K=2048),
    "causal_prefill": Workload("causal_prefill", m=4096, start_pos=0, H=64, D=512, win=128, ratio=4, n_c=1024,
                               Hi=64, Di=128, K=512),
    "chunked_prefill": Workload("chunked_prefill", m=2048, start_pos=63488, H=64, D=512, win=128, ratio=128,
                                n_c=512, Hi=0, Di=0, K=512),
}


def _gen(seed: int, workload: str, tensor: str, device: str = "cpu") -> torch.Generator:
    key = zlib.crc32(f"{seed}/{workload}/{tensor}".encode())
    g = torch.Generator(device=device)
    g.manual_seed(key)
    return g


def normal_f32(shape, seed: int, workload: str, tensor: str, device: str = "cpu") -> torch.Tensor:
    return torch.randn(tuple(shape), generator=_gen(seed, workload, tensor, device), dtype=torch.float32,
                       device=device)


def normal_bf16(shape, seed: int, workload: str, tensor: str, device: str = "cpu") -> torch.Tensor:
    return normal_f32(shape, seed, workload, tensor, device).to(torch.bfloat16)


def make_inputs(w: Workload, B: int = 1, device: str = "cpu") -> dict:
    """Raw inputs of one step for B independent sequences of workload w (CPU tensors).

    Keys: q [B,m,H,D] bf16; sink [H] f32; kv_new [B,m,D] bf16 (this step's kv
    rows); ring [B,win,D] bf16 (the ring before the step; unused at
    start_pos 0); latent_raw [B,n_c,D] bf16 (compressed rows before the fp4
    round trip); and, when the workload has an indexer, iq [B,m,Hi,Di] bf16,
    ik_raw [B,n_c,Di] bf16, iw [B,m,Hi] f32.

    device="cpu" (the tests, the oracle) draws from torch's CPU generator;
    device="cuda" draws the same distributions from the device generator
    (different numbers; used for large bench batches)."""
    s, n, d = w.seed, w.name, device
    out = {
        "q": normal_bf16((B, w.m, w.H, w.D), s, n, "q", d),
        "sink": normal_f32((w.H,), s, n, "sink", d),
        "kv_new": normal_bf16((B, w.m, w.D), s, n, "kv_new", d),
        "ring": normal_bf16((B, w.win, w.D), s, n, "ring", d),
        "latent_raw": normal_bf16((B, w.n_c, w.D), s, n, "latent_raw", d),
    }
    if w.Hi:
        out["iq"] = normal_bf16((B, w.m, w.Hi, w.Di), s, n, "iq", d)
        out["ik_raw"] = normal_bf16((B, w.n_c, w.Di), s, n, "ik_raw", d)
        out["iw"] = normal_f32((B, w.m, w.Hi), s, n, "iw", d) * float((w.Hi * w.Di) ** -0.5)
    return out


def bits(t: torch.Tensor):
    """uint16 numpy view of a bf16 CPU tensor's bit patterns."""
    import numpy as np

    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a) -> torch.Tensor:
    """bf16 CPU tensor from uint16 bit patterns."""
    import numpy as np

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)

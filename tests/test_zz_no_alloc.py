"""The no-allocation attention entry point (sckv_sparse_attn_sink_noalloc,
for callers that cannot allocate device memory) against the entry point with
a caller workspace, through the C ABI: two calls in a row, the second with a
smaller input, both splitting their lists over workgroups so the static
scratch really holds partials; the outputs must agree bit for bit (the same
kernels and split) and sit within the attention tolerance of the oracle."""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from tests.helpers import attn_tolerance_ok, bits, from_bits, vals

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _case(B, m, H, D, ra, rb, T, seed):
    rng = np.random.default_rng(seed)
    bf = lambda a: bits(torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16))  # noqa: E731
    q = bf(rng.standard_normal((B, m, H, D)))
    A = bf(rng.standard_normal((B, ra, D)))
    Rb = bf(rng.standard_normal((B, rb, D)))
    idx = rng.integers(0, ra + rb, size=(B, m, T)).astype(np.int32)
    idx[rng.random((B, m, T)) < 0.1] = -1
    sink = rng.standard_normal(H).astype(np.float32)
    return q, A, Rb, idx, sink


def test_noalloc_matches_workspace_entry():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    import sparse_compressed_kv_e2m1_amd as sk

    cap = sk.sckv_sparse_attn_sink_noalloc_max_bytes()
    assert cap == 32 << 20
    # (B, m, H, D, ra, rb, T): decode-like lists long enough to split, then a smaller one
    cases = [(2, 1, 64, 512, 128, 2048, 2176, 11), (1, 1, 64, 512, 128, 600, 640, 12)]
    for B, m, H, D, ra, rb, T, seed in cases:
        need = sk.sckv_workspace_bytes(sk.SCKV_OP_SPARSE_ATTN_SINK, B, m, H, D, T)
        assert 0 < need <= cap, need  # the split path, inside the static scratch
        q, A, Rb, idx, sink = _case(B, m, H, D, ra, rb, T, seed)
        args = (from_bits(q, "cuda"), from_bits(A, "cuda"), ra, from_bits(Rb, "cuda"), rb,
                torch.from_numpy(idx).cuda(), T, torch.from_numpy(sink).cuda(), float(np.float32(D ** -0.5)), B, m, H,
                D)
        out_ws = torch.empty((B, m, H, D), dtype=torch.bfloat16, device="cuda")
        out_na = torch.full((B, m, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        say(f"noalloc attention B={B} m={m} T={T}: {need} bytes of partials")
        sk.sckv_sparse_attn_sink(*args, out_ws)
        sk.sckv_sparse_attn_sink_noalloc(*args, out_na)
        torch.cuda.synchronize()
        assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16)), (B, T)
        got = vals(bits(out_na))
        for b in range(B):
            ref = oracle.sparse_attn(q[b], A[b], Rb[b], idx[b], sink, float(np.float32(D ** -0.5)))
            ok, worst = attn_tolerance_ok(got[b], ref)
            assert ok, (b, worst)


def test_noalloc_rejects_beyond_scratch():
    import sparse_compressed_kv_e2m1_amd as sk

    B, m, H, D, T = 255, 1, 64, 512, 640  # 510 partials of 128 KiB: beyond 32 MiB
    assert sk.sckv_workspace_bytes(sk.SCKV_OP_SPARSE_ATTN_SINK, B, m, H, D, T) > sk.sckv_sparse_attn_sink_noalloc_max_bytes()
    q = torch.zeros((B, m, H, D), dtype=torch.bfloat16, device="cuda")
    rows = torch.zeros((B, 8, D), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((B, m, T), dtype=torch.int32, device="cuda")
    sink = torch.zeros(H, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(sk.SckvError) as e:
        sk.sckv_sparse_attn_sink_noalloc(q, rows, 8, None, 0, idx, T, sink, 0.05, B, m, H, D, out)
    assert e.value.code == sk.SCKV_EUNSUPPORTED and "static scratch" in str(e.value)

"""Pins of the oracle's ring, window rows, visibility, indexer score, top-k
and attention (no GPU).

Pages: "metrale_model_arch/attn_v41/forward.rs" (AttnV41::forward: ring
copies, offset = rows_a length, compress_len, merge) and
"metrale_model_arch/deepseek_v41_ref/compress.rs" (attention_any, module doc).
"""
import collections
import math

import numpy as np
import pytest
import torch

import sckv_synth as synth
from oracle import oracle


def bf16_of(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def vals(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Ring (forward.rs: the window ring's stream-ordered copies)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("m", [1, 5, 16, 17, 40, 48, 131])
def test_ring_prefill_slots_closed_form(m):
    """start_pos 0: the ring holds the last min(m, win) rows, the row of
    position p in slot p mod win; slots no position reached keep their old rows."""
    win, D = 16, 4
    rng = np.random.default_rng(m)
    kv = rng.integers(0, 60000, size=(m, D)).astype(np.uint16)
    ring0 = rng.integers(0, 60000, size=(win, D)).astype(np.uint16)
    got = oracle.ring_write(ring0, kv, 0)
    written = set()
    for p in range(max(0, m - win), m):
        assert np.array_equal(got[p % win], kv[p]), p
        written.add(p % win)
    for j in set(range(win)) - written:
        assert np.array_equal(got[j], ring0[j]), j


def test_ring_against_deque():
    """Brute force: a deque of the last win (position, row) pairs over a random
    sequence of steps; afterwards ring[p mod win] is the row of p."""
    win, D = 8, 3
    rng = np.random.default_rng(7)
    ring = np.zeros((win, D), np.uint16)
    dq = collections.deque(maxlen=win)
    pos = 0
    for _ in range(60):
        m = int(rng.choice([1, 1, 1, 2, 3, 7, 8, 9, 20]))
        rows = rng.integers(0, 60000, size=(m, D)).astype(np.uint16)
        ring = oracle.ring_write(ring, rows, pos)
        for t in range(m):
            dq.append((pos + t, rows[t]))
        pos += m
        for p, r in dq:
            assert np.array_equal(ring[p % win], r)


def test_ring_after_chunked_prefill():
    """After a 2048-token chunk at start_pos 63488 with win 128, slot j holds
    chunk row 1920 + j (63488 is a multiple of 128)."""
    win, D, m = 128, 2, 2048
    rows = np.stack([np.arange(m), np.arange(m)], 1).astype(np.uint16)
    ring = oracle.ring_write(np.zeros((win, D), np.uint16), rows, 63488)
    assert np.array_equal(ring[:, 0], np.arange(1920, 2048))


# --------------------------------------------------------------------------
# Window rows and visibility (forward.rs: window_topk_idxs, offset, compress_len)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("win,m,start_pos", [(16, 1, 255), (16, 1, 3), (16, 1, 0), (8, 20, 0), (8, 5, 0),
                                             (8, 12, 40), (8, 3, 5), (128, 1, 32767)])
def test_window_rows_brute_force(win, m, start_pos):
    """Write distinct row ids through the ring and rows_a as the step sees them,
    then check each query's window lists exactly the positions
    max(0, p - win + 1) .. p, oldest first, then -1."""
    D = 1
    rng = np.random.default_rng(win * 1000 + m)
    hist_len = start_pos
    hist = np.arange(1, hist_len + m + 1, dtype=np.uint16).reshape(-1, 1)  # row id of position p = p + 1
    ring = np.zeros((win, D), np.uint16)
    if hist_len:
        ring = oracle.ring_write(ring, hist[:hist_len], 0)
    new = hist[hist_len:]
    if start_pos == 0:
        rows_a = new
    elif m == 1:
        rows_a = oracle.ring_write(ring, new, start_pos)
    else:
        rows_a = np.concatenate([ring, new])
    idx, ra = oracle.window_idx(win, m, start_pos)
    assert ra == rows_a.shape[0] == oracle.rows_a_len(win, m, start_pos)
    for t in range(m):
        p = start_pos + t
        want = [q + 1 for q in range(max(0, p - win + 1), p + 1)]
        got = [int(rows_a[i, 0]) for i in idx[t] if i != -1]
        assert got == want, (t, got, want)
        nvalid = len(want)
        assert np.all(idx[t, nvalid:] == -1) and np.all(idx[t, :nvalid] >= 0)
    del rng


def test_visibility_closed_form_and_counts():
    """Row j is visible to p iff (j + 1) * ratio <= p + 1, so V_p =
    min(n_c, floor((p + 1) / ratio)); pair counts of the two prefill workloads
    (sums of that closed form)."""
    for ratio, n_c in [(4, 1024), (128, 512), (4, 64)]:
        for p in list(range(0, 600)) + [4095, 65535]:
            assert oracle.visible(p, ratio, n_c) == min(n_c, (p + 1) // ratio)
    w = synth.WORKLOADS["causal_prefill"]
    V = np.array([min(w.n_c, (p + 1) // w.ratio) for p in range(w.m)])
    assert sum(min(w.win, t + 1) for t in range(w.m)) == 516160
    assert V.sum() == 2096128
    assert np.minimum(V, w.K).sum() == 1572352
    assert (V < w.K).sum() == 2047 and (V == 0).sum() == 3
    w5 = synth.WORKLOADS["chunked_prefill"]
    V5 = np.array([min(w5.n_c, (w5.start_pos + t + 1) // w5.ratio) for t in range(w5.m)])
    assert V5.min() == 496 and V5.max() == 512 and V5.sum() == 1031184


def test_workload_table_derived_values():
    """compress_len = (start_pos + m) // ratio, and the first new cache row is
    start_pos // ratio (forward.rs)."""
    for w in synth.WORKLOADS.values():
        assert w.n_c == (w.start_pos + w.m) // w.ratio
    assert [w.T for w in synth.WORKLOADS.values()] == [32, 640, 2176, 640, 640]
    assert synth.WORKLOADS["tiny_decode"].scale == 0.125


def test_visible_idx():
    idx = oracle.visible_idx(5, 60, 8, 8, 10, 100)
    for t in range(5):
        v = min(8, (60 + t + 1) // 8)
        assert list(idx[t]) == [100 + j for j in range(v)] + [-1] * (10 - v)


# --------------------------------------------------------------------------
# Indexer score (compress.rs module doc: fp4 q/k with power-of-two scales in
# blocks of 32; bf16 scores).  The head-combination formula is a reading.
# --------------------------------------------------------------------------

def _indexer_inputs(m, Hi, Di, n_c, seed, w_kind="normal"):
    rng = np.random.default_rng(seed)
    q = bf16_of(rng.standard_normal((m, Hi, Di)))
    k_raw = bf16_of(rng.standard_normal((n_c, Di)))
    k = oracle.quant(k_raw.reshape(-1), oracle.E8M0_B32).reshape(n_c, Di)
    if w_kind == "ones":
        w = np.ones((m, Hi), np.float32)
    elif w_kind == "pow2":
        w = (rng.choice([-1, 1], size=(m, Hi)) * 2.0 ** rng.integers(-3, 2, size=(m, Hi))).astype(np.float32)
    else:
        w = (rng.standard_normal((m, Hi)) * (Hi * Di) ** -0.5).astype(np.float32)
    return q, k, w


def _exact_reference(q, k, w, start_pos, ratio):
    """numpy float64 reference: q_hat via the oracle's round trip (pinned
    separately), exact per-head dots (float64 matmul of small-integer-scaled
    values is exact here), relu, weight, and the head sum in float64."""
    m, Hi, Di = q.shape
    qh = vals(oracle.quant(q.reshape(-1), oracle.E8M0_B32)).reshape(m, Hi, Di).astype(np.float64)
    kh = vals(k).astype(np.float64)
    d = np.einsum("thd,sd->ths", qh, kh)
    r = np.maximum(d, 0.0) * w.astype(np.float64)[:, :, None]
    return r.sum(axis=1)  # [m, n_c]


@pytest.mark.parametrize("w_kind", ["ones", "pow2"])
def test_score_order_free_cases(w_kind):
    """With w = 1 (or w = +-2^k) every product and partial sum is exact in
    binary32, so the butterfly result must equal the exact sum rounded once to
    bf16, whatever the order."""
    m, Hi, Di, n_c, ratio = 3, 16, 64, 40, 1
    q, k, w = _indexer_inputs(m, Hi, Di, n_c, 11, w_kind)
    sc, bad = oracle.index_scores(q, k, w, start_pos=n_c - 1, ratio=ratio)
    assert bad == 0
    exact = _exact_reference(q, k, w, n_c - 1, ratio)
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.all(exact.astype(np.float32).astype(np.float64) == exact)
    got = sc.copy()
    # -0 and +0 are the same score
    got[got == 0x8000] = 0
    want[want == 0x8000] = 0
    assert np.array_equal(got, want)


def test_score_close_to_exact_general_weights():
    """General binary32 weights: the score is within a few bf16 ulps of the
    exact real value (rounding of 2*Hi binary32 operations then one bf16 rounding)."""
    m, Hi, Di, n_c = 4, 64, 128, 96
    q, k, w = _indexer_inputs(m, Hi, Di, n_c, 12)
    sc, bad = oracle.index_scores(q, k, w, start_pos=4 * n_c - 1, ratio=4)
    assert bad == 0
    exact = _exact_reference(q, k, w, 0, 4)
    got = vals(sc).astype(np.float64)
    tol = np.abs(exact) * 2.0**-7 + 1e-30 + np.abs(exact).max() * 2.0**-20
    assert np.all(np.abs(got - exact) <= tol)


def test_score_butterfly_head_order():
    """A case where the pairwise order matters: r = [1, 2^-25, -1, 2^-25]
    summed pairwise (stride 2 then 1) gives ((1 + -1) + (2^-25 + 2^-25)) =
    2^-24, while left to right gives 0.  Built through w with relu(d) = 1."""
    Hi, Di = 4, 32
    q = np.zeros((1, Hi, Di), np.float32)
    q[0, :, 0] = 1.0  # q_hat[h] = e_0
    k = np.zeros((1, Di), np.float32)
    k[0, 0] = 1.0
    qb, kb = bf16_of(q), bf16_of(k)
    w = np.array([[1.0, 2.0**-25, -1.0, 2.0**-25]], np.float32)
    sc, bad = oracle.index_scores(qb, kb, w, start_pos=0, ratio=1)
    assert bad == 0 and vals(sc)[0, 0] == np.float32(2.0**-24)


def test_score_visibility_and_exactness_flag():
    q, k, w = _indexer_inputs(6, 4, 32, 8, 13)
    sc, _ = oracle.index_scores(q, k, w, start_pos=10, ratio=4)
    for t in range(6):
        v = min(8, (10 + t + 1) // 4)
        assert np.all(sc[t, v:] == 0xFFFF) and np.all(sc[t, :v] != 0xFFFF)
    # a dot whose exact value needs more than 24 significant bits is flagged
    qi = np.zeros((1, 1, 32), np.float32)
    qi[0, 0, 0], qi[0, 0, 1] = 6.0, 6.0 * 2.0**-30
    ki = np.zeros((1, 32), np.float32)
    ki[0, 0], ki[0, 1] = 1.0, 1.0
    _, bad = oracle.index_scores(bf16_of(qi), bf16_of(ki), np.ones((1, 1), np.float32), start_pos=0, ratio=1)
    # q's round trip flushes the tiny element to 0 in a block of 32 with scale 1, so it is exact
    assert bad == 0
    qi = np.zeros((1, 1, 64), np.float32)
    qi[0, 0, 0], qi[0, 0, 32] = 6.0, 6.0 * 2.0**-30
    ki = np.zeros((1, 64), np.float32)
    ki[0, 0], ki[0, 32] = 1.0, 1.0
    _, bad = oracle.index_scores(bf16_of(qi), bf16_of(ki), np.ones((1, 1), np.float32), start_pos=0, ratio=1)
    assert bad == 1


def test_score_exactness_flag_counts_partial_sums():
    """Exactness is a property of every partial sum, not only of the final
    value: q blocks of 2^24, 1 and -2^24 against a row of ones give the exact
    dot 1 (a binary32 value), but the partial sum 2^24 + 1 is not one, so a
    binary32 accumulation in that order returns 0.  The dot must be flagged."""
    qi = np.zeros((1, 1, 128), np.float32)
    qi[0, 0, 0], qi[0, 0, 32], qi[0, 0, 64] = 2.0**24, 1.0, -(2.0**24)
    ki = np.ones((1, 128), np.float32)
    qb, kb = bf16_of(qi), bf16_of(ki)
    assert np.array_equal(oracle.quant(qb.reshape(-1), oracle.E8M0_B32), qb.reshape(-1))  # on the fp4 grid
    assert np.array_equal(oracle.quant(kb.reshape(-1), oracle.E8M0_B32), kb.reshape(-1))
    acc = np.float32(0)
    for v in (2.0**24, 1.0, -(2.0**24)):
        acc = np.float32(acc + np.float32(v))
    assert acc == 0.0  # the in-order binary32 sum loses the 1
    _, bad = oracle.index_scores(qb, kb, np.ones((1, 1), np.float32), start_pos=0, ratio=1)
    assert bad == 1
    # the same magnitudes without cancellation (2^23 + 1 + 2^23 < 2^24 units) are exact in every order
    qi[0, 0, 0], qi[0, 0, 64] = 2.0**22, 2.0**22
    _, bad = oracle.index_scores(bf16_of(qi), kb, np.ones((1, 1), np.float32), start_pos=0, ratio=1)
    assert bad == 0


def test_score_dots_exact_on_workload_shapes():
    """The exactness condition of the score holds for seeded N(0,1) inputs of
    the decode shape (a sample of rows)."""
    w = synth.WORKLOADS["decode"]
    x = synth.make_inputs(w.with_(n_c=512, start_pos=2047))
    k = oracle.quant(synth.bits(x["ik_raw"][0]).reshape(-1), oracle.E8M0_B32).reshape(512, w.Di)
    _, bad = oracle.index_scores(synth.bits(x["iq"][0]), k, x["iw"][0].numpy(), start_pos=2047, ratio=4)
    assert bad == 0


# --------------------------------------------------------------------------
# Top-k (tie toward the lower index; ascending emit; -1 padding)
# --------------------------------------------------------------------------

def test_topk_distinct_matches_torch():
    rng = np.random.default_rng(5)
    for n, K in [(100, 10), (1000, 512), (37, 37), (37, 50)]:
        # n distinct positive bf16 values (bit patterns of finite positives, sorted = value order)
        sb = rng.choice(np.arange(1, 0x7F80), n, replace=False).astype(np.uint16)
        s = vals(sb)
        got = oracle.topk(sb, n, K, 1000)
        kk = min(K, n)
        want = sorted(torch.topk(torch.from_numpy(s), kk).indices.tolist())
        assert list(got[:kk]) == [1000 + i for i in want] and np.all(got[kk:] == -1)


def test_topk_ties_go_to_lower_index():
    """Brute force: rows sorted by (score descending, row ascending), first K."""
    rng = np.random.default_rng(6)
    for trial in range(50):
        n = int(rng.integers(1, 300))
        K = int(rng.integers(1, 64))
        vis = int(rng.integers(0, n + 1))
        s = rng.integers(-3, 4, size=n).astype(np.float32)
        s[rng.random(n) < 0.2] = -0.0
        sb = bf16_of(s)
        got = oracle.topk(sb, vis, K, 7)
        order = sorted(range(vis), key=lambda i: (-float(s[i]), i))[:K]
        want = sorted(order)
        kt = min(K, vis)
        assert list(got[:kt]) == [7 + i for i in want] and np.all(got[kt:] == -1), trial


def test_topk_all_equal():
    got = oracle.topk(bf16_of(np.zeros(50)), 50, 8, 0)
    assert list(got) == list(range(8))


# --------------------------------------------------------------------------
# Attention with a sink (compress.rs: sparse_attn call, scale = hd^-1/2)
# --------------------------------------------------------------------------

def _numpy_attention(q, rows, idx, sink, scale):
    """Independent formulation in numpy float64 (vectorised over heads)."""
    m, H, D = q.shape
    out = np.zeros((m, H, D))
    for t in range(m):
        sel = [i for i in idx[t] if i != -1]
        if not sel:
            continue
        R = rows[sel]                      # [n, D]
        l = scale * (q[t] @ R.T)           # [H, n]
        M = np.maximum(l.max(axis=1), sink)
        e = np.exp(l - M[:, None])
        Z = e.sum(axis=1) + np.exp(sink - M)
        out[t] = (e @ R) / Z[:, None]
    return out


def test_attention_brute_force_tiny_decode():
    w = synth.WORKLOADS["tiny_decode"]
    x = synth.make_inputs(w)
    rng = np.random.default_rng(8)
    ra = w.win
    rows_a = synth.bits(x["ring"][0])
    rows_b = oracle.quant(synth.bits(x["latent_raw"][0]).reshape(-1), oracle.E4M3_B16).reshape(w.n_c, w.D)
    idx = np.concatenate([oracle.window_idx(w.win, 1, w.start_pos)[0],
                          np.sort(rng.choice(w.n_c, w.K, replace=False))[None, :].astype(np.int32) + ra], 1)
    q = synth.bits(x["q"][0])
    got = oracle.sparse_attn(q, rows_a, rows_b, idx, x["sink"].numpy(), w.scale)
    rows = vals(np.concatenate([rows_a, rows_b])).astype(np.float64)
    want = _numpy_attention(vals(q).astype(np.float64), rows, idx, x["sink"].numpy().astype(np.float64), w.scale)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def test_attention_no_sink_is_textbook_softmax():
    """sink -> -inf: torch's scaled_dot_product_attention (float64) on the gathered rows."""
    rng = np.random.default_rng(9)
    H, D, n, nr = 4, 32, 20, 30
    q = bf16_of(rng.standard_normal((1, H, D)))
    rows = bf16_of(rng.standard_normal((nr, D)))
    sel = rng.choice(nr, n, replace=False).astype(np.int32)
    idx = np.concatenate([sel, [-1, -1]])[None, :].astype(np.int32)
    sink = np.full(H, -1e30, np.float32)
    scale = 0.125
    got = oracle.sparse_attn(q, rows, None, idx, sink, scale)
    Q = torch.from_numpy(vals(q).astype(np.float64)).reshape(1, H, 1, D)
    R = torch.from_numpy(vals(rows)[sel].astype(np.float64)).reshape(1, 1, n, D).expand(1, H, n, D)
    want = torch.nn.functional.scaled_dot_product_attention(Q, R, R, scale=scale).reshape(1, H, D).numpy()
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def test_attention_closed_forms():
    """Identical rows v with logit l: o = v * n e^l / (n e^l + e^sink);
    one row: o = v * sigmoid(l - sink); no valid entry: o = 0; -1 entries
    ignored; duplicates counted twice; order does not matter."""
    D, H = 16, 2
    v = bf16_of(np.linspace(-1, 1, D))
    q = bf16_of(np.stack([np.linspace(0.5, -0.5, D), np.ones(D)])[None])  # [1, H, D]
    rows = np.stack([v] * 5)
    sink = np.array([0.3, -1.2], np.float32)
    scale = 0.25
    vf = vals(v).astype(np.float64)
    qf = vals(q).astype(np.float64)[0]
    for n in [1, 3, 5]:
        idx = np.array([list(range(n)) + [-1] * (6 - n)], np.int32)
        got = oracle.sparse_attn(q, rows, None, idx, sink, scale)[0]
        for h in range(H):
            l = float(np.float32(scale)) * (qf[h] @ vf)
            want = vf * n * math.exp(l) / (n * math.exp(l) + math.exp(float(sink[h])))
            assert np.allclose(got[h], want, rtol=1e-12, atol=1e-15)
            if n == 1:
                assert np.allclose(got[h], vf / (1 + math.exp(float(sink[h]) - l)), rtol=1e-12)
    empty = oracle.sparse_attn(q, rows, None, np.full((1, 4), -1, np.int32), sink, scale)
    assert np.all(empty == 0)
    rng = np.random.default_rng(10)
    rr = bf16_of(rng.standard_normal((9, D)))
    a = oracle.sparse_attn(q, rr, None, np.array([[0, 3, 5, -1, 8]], np.int32), sink, scale)
    b = oracle.sparse_attn(q, rr, None, np.array([[8, -1, 5, 0, 3]], np.int32), sink, scale)
    assert np.allclose(a, b, rtol=1e-13)
    c = oracle.sparse_attn(q, rr, None, np.array([[0, 0, 5]], np.int32), sink, scale)
    d = oracle.sparse_attn(q, rr, None, np.array([[0, 5]], np.int32), sink, scale)
    assert not np.allclose(c, d)


def test_attention_rows_a_rows_b_addressing():
    """idx < ra names rows_a, larger idx names rows_b[idx - ra] (forward.rs offset)."""
    rng = np.random.default_rng(11)
    D, H = 8, 1
    a = bf16_of(rng.standard_normal((3, D)))
    b = bf16_of(rng.standard_normal((4, D)))
    q = bf16_of(rng.standard_normal((1, H, D)))
    sink = np.zeros(H, np.float32)
    got = oracle.sparse_attn(q, a, b, np.array([[1, 4, 6]], np.int32), sink, 1.0)
    want = oracle.sparse_attn(q, np.concatenate([a, b]), None, np.array([[1, 4, 6]], np.int32), sink, 1.0)
    assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        oracle.sparse_attn(q, a, b, np.array([[7]], np.int32), sink, 1.0)

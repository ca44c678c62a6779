"""One step of the compressed sparse attention hot path for B independent
sequences, as a sequence of C-ABI calls on one HIP stream (no host round
trip, no CPU compute).

Order of a step (page "metrale_model_arch/attn_v41/forward.rs",
AttnV41::forward; page "metrale_model_arch/deepseek_v41_ref/compress.rs",
attention_any):
  1. rotary turn (YaRN table, position j * ratio for compressed row j) and fp4
     round trip of the step's new compressed latent rows into the latent
     cache (e4m3 scales, block 16); fp4 round trip of the new indexer k rows
     into the k cache (power-of-two scales, block 32);
  2. decode (m == 1, start_pos > 0): the new kv row goes into its ring slot
     before attention;
  3. window columns of every query's index list;
  4. compressed columns: indexer scores + top-K, or every visible row on a
     layer without an indexer;
  5. sparse attention with the sink over [rows_a | latent cache];
  6. start_pos == 0 or a chunk: the step's last rows go into the ring after
     attention (a chunk reads the ring as it was before the chunk).

Device memory layout (per sequence b; all bf16 unless noted):
  q [B, m, H, D]; rows_a: the fresh kv [B, m, D] (start_pos 0), the ring
  [B, win, D] (decode), or [B, win + m, D] = ring then chunk (chunked
  prefill); latent cache [B, n_c, D]; indexer k cache [B, n_c, Di];
  indexer q [B, m, Hi, Di]; w f32 [B, m, Hi]; sink f32 [H];
  idx int32 [B, m, win + K]; out [B, m, H, D].
"""
from __future__ import annotations

import torch

from . import _binding as sk


def uses_decode_prepare(w, kcache: str) -> bool:
    """A decode step (m == 1 at start_pos > 0) with an indexer over the packed
    k cache sets up with the one-launch sckv_decode_prepare."""
    return w.start_pos > 0 and w.m == 1 and bool(w.Hi) and kcache == "fp4" and w.n_c - w.first_new_row <= 1


def uses_decode_step(w, kcache: str, latent: str = "bf16", B: int = 1) -> bool:
    """A decode step of at most 64 sequences in the shapes sckv_decode_step is
    built for (it runs as that one launch when asked for)."""
    return (uses_decode_prepare(w, kcache) and latent == "bf16" and w.Hi == 64 and w.Di == 128 and w.D == 512
            and 33 <= w.H <= 64 and B <= 64 and w.n_c <= 32768 and w.T <= 4096)


def uses_prefill_prepare(w, prepare: str = "one") -> bool:
    """A step that is not a decode step sets up with the one-launch
    sckv_prefill_prepare (unless asked for the separate calls)."""
    return prepare == "one" and not (w.start_pos > 0 and w.m == 1)


def step_call_names(w, kcache: str, latent: str = "bf16", B: int = 1, decode_launch: str = "separate",
                    prepare: str = "one") -> list:
    """Names of a step's library calls, in order (the names PathState.calls
    gives them)."""
    if decode_launch == "one" and uses_decode_step(w, kcache, latent, B):
        return ["decode_step"]
    one = uses_prefill_prepare(w, prepare)
    if uses_decode_prepare(w, kcache):
        names = ["decode_prepare"]
    elif one:
        names = ["prefill_prepare"]
    else:
        names = ["quant_latent"] + (["quant_index_k"] if w.Hi else [])
        names += (["ring_write"] if (w.start_pos > 0 and w.m == 1) else []) + ["window_idx"]
    if w.Hi:
        names += ["index_scores_topk"]
    elif not one:
        names += ["visible_idx"]
    names += ["sparse_attn_sink"]
    if w.start_pos > 0 and w.m > 1 or (w.start_pos == 0 and not one):
        names += ["ring_write"]
    return names


class PathState:
    """Device buffers of one step for B sequences of a workload, built from
    raw CPU inputs (see sckv_synth.make_inputs).  setup() round-trips the cache
    rows that existed before this step; step() runs the hot path."""

    def __init__(self, w, inputs: dict, B: int = 1, device="cuda", kcache: str = "bf16", latent: str = "bf16",
                 decode_launch: str = "separate", prepare: str = "one"):
        """kcache: "bf16" keeps the indexer k cache as round-tripped bf16 rows
        (the pages' layout); "fp4" keeps it packed (4-bit codes + one E8M0 byte
        per 32 values) and scores it on the scaled fp4 matrix cores.
        latent: "bf16" keeps the latent cache as round-tripped bf16 rows (the
        pages' layout); "fp4" keeps it packed (4-bit codes + one e4m3 byte per
        16 values, 288 bytes a 512-wide row) and the attention expands the
        rows it gathers on chip (D = 512).
        decode_launch: "separate" (default) runs a decode step as its separate
        calls; "one" runs a small-batch decode step as the one cooperative
        launch sckv_decode_step when its shapes allow (the same results; on
        MI355X its grid barriers cost more than the launch gaps they remove).
        prepare: "one" (default) sets up a step that is not a decode step
        (the new rows' round trips, the index columns that need no scores and
        a fresh step's ring write) with the one launch sckv_prefill_prepare;
        "separate" runs those as their separate calls (the same results)."""
        if kcache not in ("bf16", "fp4"):
            raise ValueError(kcache)
        if latent not in ("bf16", "fp4") or (latent == "fp4" and w.D != 512):
            raise ValueError(f"latent={latent} (packed latent rows need D = 512)")
        if decode_launch not in ("one", "separate"):
            raise ValueError(decode_launch)
        if prepare not in ("one", "separate"):
            raise ValueError(prepare)
        self.prepare = prepare
        self.w, self.B, self.device, self.kcache, self.latent_fmt = w, B, device, kcache, latent
        self.decode_launch = decode_launch
        dev = lambda t: t.to(device).contiguous()  # noqa: E731
        self.q = dev(inputs["q"])
        self.sink = dev(inputs["sink"])
        m, win, D = w.m, w.win, w.D
        if w.start_pos == 0:
            self.mode = "fresh"
            self.rows_a = dev(inputs["kv_new"])
            self.ring = torch.zeros((B, win, D), dtype=torch.bfloat16, device=device)
        elif m == 1:
            self.mode = "ring"
            self.rows_a = dev(inputs["ring"])  # the ring itself; the new row is written in step()
            self.ring = self.rows_a
            self.kv_new = dev(inputs["kv_new"])
        else:
            self.mode = "chunk"
            buf = torch.empty((B, win + m, D), dtype=torch.bfloat16, device=device)
            buf[:, :win] = inputs["ring"].to(device)
            buf[:, win:] = inputs["kv_new"].to(device)
            self.rows_a = buf
        self.ra = sk.sckv_rows_a_len(win, m, w.start_pos)
        assert self.ra == self.rows_a.shape[1]
        self.first_new = w.first_new_row
        self.n_new = w.n_c - self.first_new
        lat = inputs["latent_raw"]
        self.latent = dev(lat)
        # the latent rows' rotation table, built once (on the host, by the library)
        self.rope_table = sk.sckv_yarn_freqs_cis(w.rope_dim, w.rope_positions, w.rope_orig_len, w.rope_base,
                                                 w.rope_factor, w.rope_beta_fast, w.rope_beta_slow).to(device)
        self.latent_new = lat[:, self.first_new:].to(device).clone()  # a buffer of its own, never a view
        if latent == "fp4":
            self.lat_codes = torch.zeros((B, w.n_c, D // 2), dtype=torch.uint8, device=device)
            self.lat_scales = torch.zeros((B, w.n_c, D // 16), dtype=torch.uint8, device=device)
        if w.Hi:
            self.iq = dev(inputs["iq"])
            self.iw = dev(inputs["iw"])
            self.ik = dev(inputs["ik_raw"])
            self.ik_new = inputs["ik_raw"][:, self.first_new:].to(device).clone()
            if kcache == "fp4":
                self.ik_codes = torch.zeros((B, w.n_c, w.Di // 2), dtype=torch.uint8, device=device)
                self.ik_scales = torch.zeros((B, w.n_c, w.Di // 32), dtype=torch.uint8, device=device)
                self.ws_index = sk.workspace(sk.SCKV_OP_INDEX_SCORES_TOPK_FP4, B, m, w.Hi, w.Di, w.n_c, device=device)
            else:
                self.ws_index = sk.workspace(sk.SCKV_OP_INDEX_SCORES_TOPK, B, m, w.Hi, w.Di, w.n_c, device=device)
        self.T = w.T
        self.idx = torch.empty((B, m, self.T), dtype=torch.int32, device=device)
        self.out = torch.empty((B, m, w.H, D), dtype=torch.bfloat16, device=device)
        self.ws_attn = sk.workspace(sk.SCKV_OP_SPARSE_ATTN_SINK, B, m, w.H, D, self.T, device=device)

    def setup(self):
        """Round-trip the compressed rows that precede this step (the caches
        as earlier steps left them)."""
        w, B = self.w, self.B
        if self.first_new > 0:
            for b in range(B):  # row j of each sequence turned at j * ratio, then round-tripped
                if self.latent_fmt == "fp4":
                    sk.sckv_rope_quant_pack(self.latent[b], w.D, self.lat_codes[b], w.D // 2, self.lat_scales[b],
                                            w.D // 16, self.first_new, w.D, self.rope_table, w.rope_dim, 0, w.ratio)
                else:
                    sk.sckv_rope_quant_rows(self.latent[b], w.D, self.latent[b], w.D, self.first_new, w.D,
                                            self.rope_table, w.rope_dim, 0, w.ratio)
            if w.Hi and self.kcache == "fp4":
                # every row packed (the step's own new rows are packed again by its first calls)
                sk.sckv_quant_pack(self.ik, w.Di, self.ik_codes, w.Di // 2, self.ik_scales, w.Di // 32, B * w.n_c,
                                   w.Di, sk.SCKV_FP4_E8M0_B32)
            elif w.Hi:
                sk.sckv_quant_rows(self.ik, w.n_c * w.Di, self.ik, w.n_c * w.Di, B, self.first_new * w.Di,
                                   sk.SCKV_FP4_E8M0_B32)

    def _quant_new(self, src, dst, width, mode):
        w, B = self.w, self.B
        if self.n_new == 0:
            return
        if mode == sk.SCKV_FP4_E4M3_B16 and self.latent_fmt == "fp4":
            # the latent, packed: rotary turn at j * ratio, round trip, codes + scale bytes
            pos0, f, D = self.first_new * w.ratio, self.first_new, w.D
            if self.n_new == 1:
                sk.sckv_rope_quant_pack(src, width, self.lat_codes[:, f], w.n_c * D // 2, self.lat_scales[:, f],
                                        w.n_c * D // 16, B, width, self.rope_table, w.rope_dim, pos0, 0)
            else:
                for b in range(B):
                    sk.sckv_rope_quant_pack(src[b], width, self.lat_codes[b, f], D // 2, self.lat_scales[b, f],
                                            D // 16, self.n_new, width, self.rope_table, w.rope_dim, pos0, w.ratio)
            return
        if mode == sk.SCKV_FP4_E4M3_B16:
            # the latent: rotary turn at j * ratio, then the round trip
            pos0 = self.first_new * w.ratio
            if self.n_new == 1:  # one row per sequence, all at one position
                sk.sckv_rope_quant_rows(src, width, dst[:, self.first_new:], w.n_c * width, B, width, self.rope_table,
                                        w.rope_dim, pos0, 0)
            else:
                for b in range(B):
                    sk.sckv_rope_quant_rows(src[b], width, dst[b, self.first_new:], width, self.n_new, width,
                                            self.rope_table, w.rope_dim, pos0, w.ratio)
            return
        if self.n_new == 1 or B == 1:
            # B x n_new rows: either one row per sequence, or one sequence
            rows, ldx, ldy, cols = (B, width, w.n_c * width, width) if self.n_new == 1 else (self.n_new, width, width,
                                                                                               width)
            sk.sckv_quant_rows(src, ldx, dst[:, self.first_new:], ldy, rows, cols, mode)
        else:
            for b in range(B):
                sk.sckv_quant_rows(src[b], width, dst[b, self.first_new:], width, self.n_new, width, mode)

    def _pack_new_k(self):
        """The step's new indexer k rows into the packed cache."""
        w, B, Di = self.w, self.B, self.w.Di
        if self.n_new == 0:
            return
        f = self.first_new
        if self.n_new == 1 or B == 1:
            rows, ldc, lds = (B, w.n_c * Di // 2, w.n_c * Di // 32) if self.n_new == 1 else (self.n_new, Di // 2,
                                                                                              Di // 32)
            sk.sckv_quant_pack(self.ik_new, Di, self.ik_codes[:, f], ldc, self.ik_scales[:, f], lds, rows, Di,
                               sk.SCKV_FP4_E8M0_B32)
        else:
            for b in range(B):
                sk.sckv_quant_pack(self.ik_new[b], Di, self.ik_codes[b, f], Di // 2, self.ik_scales[b, f], Di // 32,
                                   self.n_new, Di, sk.SCKV_FP4_E8M0_B32)

    def _prefill_prepare(self):
        """Step 1, step 3, step 4 without an indexer and, from position 0,
        step 6 of the module doc in one launch."""
        w, B = self.w, self.B
        m, win, D, Di = w.m, w.win, w.D, w.Di
        f, nn = self.first_new, self.n_new
        pk = self.latent_fmt == "fp4"
        kp = bool(w.Hi) and self.kcache == "fp4"
        kb = bool(w.Hi) and self.kcache != "fp4"
        fresh = self.mode == "fresh"
        sk.sckv_prefill_prepare(
            B, m, w.start_pos, win, D, nn, self.latent_new if nn else None, nn * D,
            self.latent[:, f] if (nn and not pk) else None, w.n_c * D,
            self.lat_codes[:, f] if (nn and pk) else None, w.n_c * D // 2,
            self.lat_scales[:, f] if (nn and pk) else None, w.n_c * D // 16,
            self.rope_table, w.rope_dim, f * w.ratio, w.ratio,
            self.ik_new if (nn and w.Hi) else None, nn * Di, Di,
            self.ik[:, f] if (nn and kb) else None, w.n_c * Di,
            self.ik_codes[:, f] if (nn and kp) else None, w.n_c * Di // 2,
            self.ik_scales[:, f] if (nn and kp) else None, w.n_c * Di // 32,
            self.rows_a if fresh else None, m * D, self.ring if fresh else None, win * D,
            self.idx, self.T, w.ratio, w.n_c, 0 if w.Hi else w.K, self.ra)

    def calls(self):
        """The step's library calls in order, as (name, thunk) pairs."""
        w, B = self.w, self.B
        m, win, D = w.m, w.win, w.D
        if self.decode_launch == "one" and uses_decode_step(w, self.kcache, self.latent_fmt, B):
            # the whole decode step in one launch (the same results as the calls below)
            new = self.n_new == 1
            if not hasattr(self, "ws_step"):
                nb = sk.sckv_decode_step_workspace_bytes(B, w.H, D, w.n_c, self.T)
                # zeroed: its first 256 bytes are the launch's barrier words
                self.ws_step = torch.zeros(max(nb, 256), dtype=torch.uint8, device=self.device)
            return [("decode_step", lambda: sk.sckv_decode_step(
                self.latent_new if new else None, self.ik_new if new else None, self.kv_new, self.rope_table,
                w.rope_dim, self.latent, self.ik_codes, self.ik_scales, self.ring, self.iq, self.iw, w.Hi, w.Di,
                w.ratio, w.K, self.q, self.sink, w.scale, w.H, B, w.n_c, D, win, w.start_pos, self.idx, self.out,
                ws=self.ws_step))]
        if uses_decode_prepare(w, self.kcache):
            # decode: the latent and k rows, the ring slot and the window
            # columns in one launch (the same results as the four calls below)
            f = self.first_new
            new = self.n_new == 1
            pk = self.latent_fmt == "fp4"
            out = [("decode_prepare", lambda: sk.sckv_decode_prepare(
                self.latent_new if new else None, D, self.latent[:, f] if (new and not pk) else None, w.n_c * D,
                self.ik_new if new else None, w.Di, self.ik_codes[:, f] if new else None, w.n_c * w.Di // 2,
                self.ik_scales[:, f] if new else None, w.n_c * w.Di // 32, w.Di, self.kv_new, D, self.ring, win * D,
                B, D, win, w.start_pos, self.idx, self.T, self.rope_table, w.rope_dim, f * w.ratio,
                self.lat_codes[:, f] if (new and pk) else None, w.n_c * D // 2,
                self.lat_scales[:, f] if (new and pk) else None, w.n_c * D // 16))]
            return out + self._score_and_attend_calls()
        if uses_prefill_prepare(w, self.prepare):
            return [("prefill_prepare", self._prefill_prepare)] + self._score_and_attend_calls()
        out = [("quant_latent", lambda: self._quant_new(self.latent_new, self.latent, D, sk.SCKV_FP4_E4M3_B16))]
        if w.Hi and self.kcache == "fp4":
            out.append(("quant_index_k", self._pack_new_k))
        elif w.Hi:
            out.append(("quant_index_k", lambda: self._quant_new(self.ik_new, self.ik, w.Di, sk.SCKV_FP4_E8M0_B32)))
        if self.mode == "ring":
            out.append(("ring_write", lambda: sk.sckv_ring_write(self.kv_new, D, self.ring, win * D, B, 1,
                                                                 w.start_pos, win, D)))
        out.append(("window_idx", lambda: sk.sckv_window_idx(B, m, w.start_pos, win, self.idx, self.T)))
        return out + self._score_and_attend_calls()

    def _score_and_attend_calls(self):
        """Steps 4-6 of the module doc as (name, thunk) pairs."""
        w, B = self.w, self.B
        m, win, D = w.m, w.win, w.D
        out = []
        if w.Hi and self.kcache == "fp4":
            out.append(("index_scores_topk", lambda: sk.sckv_index_scores_topk_fp4(
                self.iq, self.ik_codes, self.ik_scales, self.iw, B, m, w.Hi, w.Di, w.n_c, w.ratio, w.start_pos, w.K,
                self.ra, self.idx, self.T, win, ws=self.ws_index)))
        elif w.Hi:
            out.append(("index_scores_topk", lambda: sk.sckv_index_scores_topk(
                self.iq, self.ik, self.iw, B, m, w.Hi, w.Di, w.n_c, w.ratio, w.start_pos, w.K, self.ra, self.idx,
                self.T, win, ws=self.ws_index)))
        elif not uses_prefill_prepare(w, self.prepare):
            out.append(("visible_idx", lambda: sk.sckv_visible_idx(B, m, w.start_pos, w.ratio, w.n_c, w.K, self.ra,
                                                                   self.idx, self.T, win)))
        if self.latent_fmt == "fp4":
            out.append(("sparse_attn_sink", lambda: sk.sckv_sparse_attn_sink_fp4(
                self.q, self.rows_a, self.ra, self.lat_codes, self.lat_scales, w.n_c, self.idx, self.T, self.sink,
                w.scale, B, m, w.H, D, self.out, ws=self.ws_attn)))
        else:
            out.append(("sparse_attn_sink", lambda: sk.sckv_sparse_attn_sink(
                self.q, self.rows_a, self.ra, self.latent, w.n_c, self.idx, self.T, self.sink, w.scale, B, m, w.H, D,
                self.out, ws=self.ws_attn)))
        if self.mode == "fresh" and not uses_prefill_prepare(w, self.prepare):
            out.append(("ring_write", lambda: sk.sckv_ring_write(self.rows_a, m * D, self.ring, win * D, B, m,
                                                                 w.start_pos, win, D)))
        elif self.mode == "chunk":
            out.append(("ring_write", lambda: sk.sckv_ring_write(self.rows_a[:, win:], (win + m) * D, self.rows_a,
                                                                 (win + m) * D, B, m, w.start_pos, win, D)))
        return out

    def capture_graph(self):
        """One step (the same library calls on torch's current stream) captured
        into a HIP graph; replaying it runs the step without per-launch host
        work.  The library records no memset, allocation or synchronization,
        and every buffer the step uses is allocated here beforehand."""
        side = torch.cuda.Stream(device=self.device)  # default priority
        side.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream(self.device).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step()
        return graph

    def step(self):
        """One pass of the hot path (steps 1-6 of the module doc)."""
        if not hasattr(self, "_calls"):
            self._calls = self.calls()
            assert [n for n, _ in self._calls] == step_call_names(self.w, self.kcache, self.latent_fmt, self.B,
                                                                 self.decode_launch, self.prepare)
        for _, f in self._calls:
            f()
        return self.out

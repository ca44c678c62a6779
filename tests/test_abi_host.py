"""Host-side checks of the C ABI (no GPU): the library loads, exports every
call include/sckv.h declares, and rejects invalid arguments before enqueuing
anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_calls(header="sckv.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sckv_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_calls():
    names = declared_calls()
    for n in ["sckv_quant", "sckv_quant_rows", "sckv_ring_write", "sckv_rows_a_len", "sckv_window_idx",
              "sckv_visible_idx", "sckv_index_scores_topk", "sckv_sparse_attn_sink", "sckv_workspace_bytes",
              "sckv_last_error", "sckv_abi_version", "sckv_quant_pack", "sckv_index_scores_topk_fp4",
              "sckv_decode_prepare", "sckv_yarn_freqs_cis", "sckv_rope_quant_rows", "sckv_rope_quant_pack",
              "sckv_decode_step", "sckv_sparse_attn_sink_fp4", "sckv_prefill_prepare"]:
        assert n in names


def test_library_exports_every_declared_call():
    import sparse_compressed_kv_e2m1_amd as sk

    lib = ctypes.CDLL(sk.LIB_PATH)
    for n in declared_calls():
        assert hasattr(lib, n), n
    assert sk.sckv_abi_version() == 2
    assert "sckv_sparse_attn_sink_noalloc" in declared_calls()
    assert sk.sckv_sparse_attn_sink_noalloc_max_bytes() == 32 << 20


def test_peak_library_exports_every_declared_call():
    """The measurement kernels (roofline denominators) live in a library of
    their own, declared in include/sckv_peak.h."""
    peak = ctypes.CDLL(os.path.join(ROOT, "sparse_compressed_kv_e2m1_amd", "libsckv_peak.so"))
    names = declared_calls("sckv_peak.h")
    assert {"sckv_peak_copy", "sckv_peak_read", "sckv_peak_gather", "sckv_peak_mfma",
            "sckv_peak_mfma_flops"} <= set(names)
    for n in names:
        assert hasattr(peak, n), n
    peak.sckv_peak_mfma_flops.restype = ctypes.c_double
    peak.sckv_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    assert peak.sckv_peak_mfma_flops(0, 10, 3) == 32 * 32 * 16 * 2 * 8 * 10 * 3 * 4
    assert peak.sckv_peak_mfma_flops(1, 10, 3) == 32 * 32 * 64 * 2 * 8 * 10 * 3 * 4
    peak.sckv_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    assert peak.sckv_peak_copy(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 63, 1, 4, None) == -1  # size
    assert peak.sckv_peak_copy(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 64, 1, 5, None) == -1  # depth
    peak.sckv_peak_gather.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    a, i, o = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    assert peak.sckv_peak_gather(a, 0, i, 8, o, 1, 4, None) == -1  # no rows
    assert peak.sckv_peak_gather(a, 16, i, 8, o, 1, 3, None) == -1  # depth
    assert peak.sckv_peak_gather(ctypes.c_void_p(0x1008), 16, i, 8, o, 1, 4, None) == -1  # misaligned rows


def test_header_compiles_as_c():
    """The header is plain C (no HIP or torch types)."""
    import subprocess
    import tempfile

    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write('#include "sckv.h"\n#include "sckv_peak.h"\n'
                           'int main(void){return sckv_abi_version() == 1 ? 0 : 1;}\n')
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                        c], check=True)


@pytest.fixture(scope="module")
def L():
    import sparse_compressed_kv_e2m1_amd as sk

    return sk.lib


def test_error_paths(L):
    import sparse_compressed_kv_e2m1_amd as sk

    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks
    # quant: n not a multiple of the block, bad mode, null pointers
    assert L.sckv_quant(fake, fake, 17, sk.SCKV_FP4_E4M3_B16, None) == sk.SCKV_EINVAL
    assert "multiple" in sk.sckv_last_error()
    assert L.sckv_quant(fake, fake, 32, 7, None) == sk.SCKV_EINVAL
    assert L.sckv_quant(None, fake, 32, sk.SCKV_FP4_E8M0_B32, None) == sk.SCKV_EINVAL
    assert L.sckv_quant(fake, fake, 0, sk.SCKV_FP4_E8M0_B32, None) == sk.SCKV_OK  # empty is a no-op
    assert L.sckv_quant_rows(fake, 8, fake, 8, 2, 16, sk.SCKV_FP4_E4M3_B16, None) == sk.SCKV_EINVAL  # ld < cols
    assert L.sckv_quant_rows(fake, 16, ctypes.c_void_p(0x1010), 16, 2, 16, sk.SCKV_FP4_E4M3_B16,
                             None) == sk.SCKV_EINVAL  # overlap
    # packed round trip: block multiple, strides, overlap, mode
    big = ctypes.c_void_p(0x100000)
    assert L.sckv_quant_pack(fake, 40, big, 20, ctypes.c_void_p(0x200000), 2, 1, 40, sk.SCKV_FP4_E8M0_B32,
                             None) == sk.SCKV_EINVAL  # 40 values: not a multiple of 32
    assert L.sckv_quant_pack(fake, 64, big, 16, ctypes.c_void_p(0x200000), 2, 2, 64, sk.SCKV_FP4_E8M0_B32,
                             None) == sk.SCKV_EINVAL  # ldc 16 < 32 code bytes
    assert L.sckv_quant_pack(fake, 64, ctypes.c_void_p(0x1020), 32, ctypes.c_void_p(0x200000), 2, 2, 64,
                             sk.SCKV_FP4_E8M0_B32, None) == sk.SCKV_EINVAL  # codes overlap x
    assert L.sckv_quant_pack(fake, 64, big, 32, ctypes.c_void_p(0x200000), 2, 2, 64, 5, None) == sk.SCKV_EINVAL
    assert L.sckv_quant_pack(fake, 64, big, 32, None, 2, 2, 64, sk.SCKV_FP4_E8M0_B32, None) == sk.SCKV_EINVAL
    # ring
    assert L.sckv_ring_write(fake, 64, fake, 64, 1, 1, 5, 0, 64, None) == sk.SCKV_EINVAL
    assert L.sckv_ring_write(fake, 64, fake, 64 * 16, 1, 1, 5, 16, 64, None) == sk.SCKV_EINVAL  # overlap
    # window / visible
    assert L.sckv_window_idx(1, 4, 0, 16, None, 16, None) == sk.SCKV_EINVAL
    assert L.sckv_window_idx(1, 4, 0, 16, fake, 8, None) == sk.SCKV_EINVAL
    assert L.sckv_visible_idx(1, 1, 1000, 4, 1000, 16, 0, fake, 32, 16, None) == sk.SCKV_EINVAL  # V > K
    # indexer
    args = dict(B=1, m=1, Hi=64, Di=128, n_c=8192, ratio=4, start_pos=32767, K=512, offset=128, ld=640, col0=128)

    def ix(**kw):
        a = {**args, **kw}
        return L.sckv_index_scores_topk(fake, fake, fake, a["B"], a["m"], a["Hi"], a["Di"], a["n_c"], a["ratio"],
                                        a["start_pos"], a["K"], a["offset"], kw.get("idx", fake), a["ld"], a["col0"],
                                        None, kw.get("ws", fake), kw.get("ws_bytes", 1 << 30), None)

    assert ix(Hi=48) == sk.SCKV_EINVAL
    assert ix(Hi=128) == sk.SCKV_EUNSUPPORTED
    assert ix(Di=96) == sk.SCKV_EUNSUPPORTED
    assert ix(ld=600) == sk.SCKV_EINVAL
    assert ix(idx=None) == sk.SCKV_EINVAL
    assert ix(ws=None) == sk.SCKV_EWORKSPACE
    assert ix(ws_bytes=100) == sk.SCKV_EWORKSPACE
    assert ix(ratio=0) == sk.SCKV_EINVAL

    # attention
    def at(**kw):
        a = dict(ra=128, rb=8192, T=640, B=1, m=1, H=64, D=512, scale=0.044, ws_bytes=1 << 30)
        a.update(kw)
        return L.sckv_sparse_attn_sink(fake, fake, a["ra"], fake, a["rb"], fake, a["T"], fake,
                                       ctypes.c_float(a["scale"]), a["B"], a["m"], a["H"], a["D"],
                                       kw.get("out", fake), kw.get("ws", fake), a["ws_bytes"], None)

    assert at(H=65) == sk.SCKV_EUNSUPPORTED
    assert at(D=96) == sk.SCKV_EUNSUPPORTED
    assert at(T=0) == sk.SCKV_EINVAL
    assert at(T=70000) == sk.SCKV_EUNSUPPORTED
    assert at(out=None) == sk.SCKV_EINVAL
    assert at(scale=0.0) == sk.SCKV_EINVAL
    assert at(ws=None) == sk.SCKV_EWORKSPACE  # decode at B = 1 splits rows over workgroups
    assert at(B=0) == sk.SCKV_OK
    assert at(out=ctypes.c_void_p(0x1008)) == sk.SCKV_EINVAL  # rows leave as 16-byte pieces

    # decode set-up: sizes, strides, alignment, missing destinations
    def dp(**kw):
        a = dict(ld_lat_new=512, ld_lat_dst=512, ld_k_new=128, ld_codes=64, ld_scales=4, Di=128, ld_kv_new=512,
                 ld_ring=128 * 512, B=2, D=512, win=128, start_pos=1000, ld_idx=640, n_pos=4000, rope_dim=64,
                 lat_pos=996, ld_lat_codes=256, ld_lat_scales=32)
        a.update({k: v for k, v in kw.items() if k in a})
        return L.sckv_decode_prepare(kw.get("lat_new", fake), a["ld_lat_new"], kw.get("lat_dst", fake),
                                     a["ld_lat_dst"], kw.get("k_new", fake), a["ld_k_new"], kw.get("k_codes", fake),
                                     a["ld_codes"], kw.get("k_scales", fake), a["ld_scales"], a["Di"],
                                     kw.get("kv_new", fake), a["ld_kv_new"], kw.get("ring", fake), a["ld_ring"],
                                     a["B"], a["D"], a["win"], a["start_pos"], kw.get("idx", fake), a["ld_idx"],
                                     kw.get("rope_table", None), a["n_pos"], a["rope_dim"], a["lat_pos"],
                                     kw.get("lat_codes", None), a["ld_lat_codes"], kw.get("lat_scales", None),
                                     a["ld_lat_scales"], None)

    assert dp(D=520) == sk.SCKV_EINVAL                 # not a multiple of 16
    assert dp(Di=100) == sk.SCKV_EINVAL                # not a multiple of 32
    assert dp(lat_dst=None) == sk.SCKV_EINVAL
    assert dp(k_codes=None) == sk.SCKV_EINVAL
    assert dp(kv_new=None) == sk.SCKV_EINVAL
    assert dp(idx=None) == sk.SCKV_EINVAL
    assert dp(ld_ring=1000) == sk.SCKV_EINVAL          # shorter than win * D
    assert dp(rope_table=fake, rope_dim=63) == sk.SCKV_EINVAL   # odd rotation width
    assert dp(rope_table=fake, rope_dim=520) == sk.SCKV_EINVAL  # wider than the row
    assert dp(rope_table=fake, lat_pos=4000) == sk.SCKV_EINVAL  # position outside the table
    assert dp(rope_table=ctypes.c_void_p(0x1004)) == sk.SCKV_EINVAL  # table not 8-byte aligned
    assert dp(lat_codes=fake, lat_scales=fake) == sk.SCKV_EINVAL      # packed and bf16 destinations at once
    assert dp(lat_dst=None, lat_codes=fake) == sk.SCKV_EINVAL         # packed codes without scale bytes
    assert dp(lat_dst=None, lat_codes=fake, lat_scales=fake, ld_lat_codes=200) == sk.SCKV_EINVAL  # short stride

    # set-up of a step that is not a decode step: sizes, strides, alignment,
    # destinations, overlap, the visible-count and rotation checks
    def pp(**kw):
        P = lambda v: ctypes.c_void_p(v)  # noqa: E731
        a = dict(B=1, m=4096, start_pos=0, win=128, D=512, n_new=1024, bs_lat_new=1024 * 512,
                 bs_lat_dst=1024 * 512, bs_lat_codes=1024 * 256, bs_lat_scales=1024 * 32, n_pos=4096, rope_dim=64,
                 pos0=0, pos_step=4, bs_k_new=1024 * 128, Di=128, bs_k_dst=0, bs_k_codes=1024 * 64,
                 bs_k_scales=1024 * 4, bs_ring_src=4096 * 512, bs_ring=128 * 512, ld_idx=640, ratio=4, n_c=1024,
                 K=0, offset=4096)
        a.update({k: v for k, v in kw.items() if k in a})
        ptr = dict(lat_new=P(0x10000000), lat_dst=P(0x20000000), lat_codes=None, lat_scales=None,
                   rope_table=P(0x30000000), k_new=P(0x40000000), k_dst=None, k_codes=P(0x50000000),
                   k_scales=P(0x60000000), ring_src=P(0x70000000), ring=P(0x80000000), idx=P(0x90000000))
        ptr.update({k: v for k, v in kw.items() if k in ptr})
        return L.sckv_prefill_prepare(
            a["B"], a["m"], a["start_pos"], a["win"], a["D"], a["n_new"], ptr["lat_new"], a["bs_lat_new"],
            ptr["lat_dst"], a["bs_lat_dst"], ptr["lat_codes"], a["bs_lat_codes"], ptr["lat_scales"],
            a["bs_lat_scales"], ptr["rope_table"], a["n_pos"], a["rope_dim"], a["pos0"], a["pos_step"], ptr["k_new"],
            a["bs_k_new"], a["Di"], ptr["k_dst"], a["bs_k_dst"], ptr["k_codes"], a["bs_k_codes"], ptr["k_scales"],
            a["bs_k_scales"], ptr["ring_src"], a["bs_ring_src"], ptr["ring"], a["bs_ring"], ptr["idx"], a["ld_idx"],
            a["ratio"], a["n_c"], a["K"], a["offset"], None)

    assert pp(B=0) == sk.SCKV_OK                                  # nothing to do (valid arguments)
    assert pp(D=520) == sk.SCKV_EINVAL                            # not a multiple of 16
    assert pp(Di=100) == sk.SCKV_EINVAL                           # not a multiple of 32
    assert pp(idx=None) == sk.SCKV_EINVAL
    assert pp(ld_idx=100) == sk.SCKV_EINVAL                       # shorter than win + K
    assert pp(lat_dst=None) == sk.SCKV_EINVAL                     # no latent destination
    assert pp(lat_codes=ctypes.c_void_p(0xA0000000), lat_scales=ctypes.c_void_p(0xB0000000)) == sk.SCKV_EINVAL
    assert pp(k_codes=None) == sk.SCKV_EINVAL                     # scale bytes without codes
    assert pp(bs_lat_dst=1000) == sk.SCKV_EINVAL                  # batch stride shorter than the rows
    assert pp(lat_new=ctypes.c_void_p(0x10000008)) == sk.SCKV_EINVAL  # not 16-byte aligned
    assert pp(lat_dst=ctypes.c_void_p(0x10000100)) == sk.SCKV_EINVAL  # overlaps its source
    assert pp(k_codes=ctypes.c_void_p(0x40000100)) == sk.SCKV_EINVAL  # overlaps its source
    assert pp(rope_dim=63) == sk.SCKV_EINVAL                      # odd rotation width
    assert pp(pos0=4, n_pos=4096) == sk.SCKV_EINVAL               # last row at 4 + 1023 * 4 = 4096: outside
    assert pp(rope_table=ctypes.c_void_p(0x30000004)) == sk.SCKV_EINVAL  # table not 8-byte aligned
    assert pp(K=400, ld_idx=528) == sk.SCKV_EINVAL                # fewer columns than visible rows (1024)
    assert pp(ring=None) == sk.SCKV_EINVAL                        # a ring source without a ring
    assert pp(bs_ring=1000) == sk.SCKV_EINVAL                     # shorter than win * D
    assert pp(ring=ctypes.c_void_p(0x70000100)) == sk.SCKV_EINVAL  # rows and ring overlap
    assert pp(B=70000) == sk.SCKV_EUNSUPPORTED
    assert pp(start_pos=-1) == sk.SCKV_EINVAL

    def rq(**kw):
        a = dict(ldx=512, ldy=512, rows=4, cols=512, n_pos=100, rope_dim=64, pos0=0, pos_step=4)
        a.update({k: v for k, v in kw.items() if k in a})
        return L.sckv_rope_quant_rows(kw.get("x", fake), a["ldx"], kw.get("y", ctypes.c_void_p(0x100000)), a["ldy"],
                                      a["rows"], a["cols"], kw.get("table", fake), a["n_pos"], a["rope_dim"],
                                      a["pos0"], a["pos_step"], None)

    assert rq(cols=520) == sk.SCKV_EINVAL               # not a multiple of 16
    assert rq(rope_dim=0) == sk.SCKV_EINVAL
    assert rq(rope_dim=7) == sk.SCKV_EINVAL
    assert rq(pos0=97, pos_step=1) == sk.SCKV_EINVAL    # last row at position 100: outside
    assert rq(pos_step=-1) == sk.SCKV_EINVAL
    assert rq(table=None) == sk.SCKV_EINVAL
    assert rq(rows=0) == sk.SCKV_OK
    assert dp(ld_idx=100) == sk.SCKV_EINVAL            # shorter than win
    assert dp(ring=ctypes.c_void_p(0x1004)) == sk.SCKV_EINVAL  # not 16-byte aligned
    assert dp(ld_codes=72) == sk.SCKV_EINVAL           # code rows not 16-byte strided
    assert dp(start_pos=-1) == sk.SCKV_EINVAL
    assert dp(B=0) == sk.SCKV_OK


def test_workspace_sizes(L):
    import sparse_compressed_kv_e2m1_amd as sk

    assert sk.sckv_workspace_bytes(sk.SCKV_OP_INDEX_SCORES_TOPK, 1, 4096, 64, 128, 1024) == 4096 * 1024 * 2
    assert sk.sckv_workspace_bytes(sk.SCKV_OP_SPARSE_ATTN_SINK, 1, 4096, 64, 512, 640) == 0  # no split at m = 4096
    assert sk.sckv_workspace_bytes(sk.SCKV_OP_SPARSE_ATTN_SINK, 1, 1, 64, 512, 640) > 0
    assert sk.sckv_workspace_bytes(9, 1, 1, 1, 1, 1) == ctypes.c_size_t(-1).value
    assert sk.sckv_rows_a_len(128, 4096, 0) == 4096
    assert sk.sckv_rows_a_len(128, 1, 32767) == 128
    assert sk.sckv_rows_a_len(128, 2048, 63488) == 2176
    assert sk.sckv_rows_a_len(0, 1, 1) == -1


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The package never imports the oracle and has no CPU compute path."""
    pkg = os.path.join(ROOT, "sparse_compressed_kv_e2m1_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                for bad in ("import oracle", "from oracle", "libsckv_oracle", "sckvo_", "oracle.py"):
                    assert bad not in text, (f, bad)


def test_rotation_table_matches_oracle():
    """The library's host-built rotation table (sckv_yarn_freqs_cis) is the
    oracle's, bit for bit, at the workloads' parameters and at plain RoPE; bad
    parameters are refused."""
    import numpy as np

    import sckv_synth as synth
    import sparse_compressed_kv_e2m1_amd as sk
    from oracle import oracle

    for w in synth.WORKLOADS.values():
        args = (w.rope_dim, w.rope_positions, w.rope_orig_len, w.rope_base, w.rope_factor, w.rope_beta_fast,
                w.rope_beta_slow)
        got = sk.sckv_yarn_freqs_cis(*args).numpy()
        want = oracle.yarn_freqs_cis(*args)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), w.name
    got = sk.sckv_yarn_freqs_cis(128, 300, 8192, 500000.0, 1.0, 32.0, 1.0).numpy()
    assert np.array_equal(got.view(np.uint32), oracle.yarn_freqs_cis(128, 300, 8192, 500000.0, 1.0, 32.0, 1.0)
                          .view(np.uint32))
    for bad in ((63, 4, 4096, 1e4, 40.0, 32.0, 1.0), (64, 4, 4096, 1.0, 40.0, 32.0, 1.0),
                (64, 4, 4096, 1e4, 0.0, 32.0, 1.0)):
        with pytest.raises(sk.SckvError):
            sk.sckv_yarn_freqs_cis(*bad)


def test_decode_step_host_checks(L):
    """sckv_decode_step refuses what it is not built for before enqueuing
    anything (fake pointers are never dereferenced)."""
    import sparse_compressed_kv_e2m1_amd as sk

    f = ctypes.c_void_p(0x10000)

    def ds(**kw):
        a = dict(lat_new=f, k_new=f, n_pos=40000, rope_dim=64, Hi=64, Di=128, ratio=4, K=512, H=64, B=2, n_c=8192,
                 D=512, win=128, start_pos=32767, ws_bytes=1 << 40)
        a.update(kw)
        return L.sckv_decode_step(a["lat_new"], a["k_new"], f, f, a["n_pos"], a["rope_dim"], f, f, f, f, f, f,
                                  a["Hi"], a["Di"], a["ratio"], a["K"], f, f, ctypes.c_float(0.05), a["H"], a["B"],
                                  a["n_c"], a["D"], a["win"], a["start_pos"], f, f, f, ctypes.c_size_t(a["ws_bytes"]),
                                  None)

    assert ds(B=65) == sk.SCKV_EUNSUPPORTED        # more than 64 sequences
    assert ds(H=16) == sk.SCKV_EUNSUPPORTED        # head groups the step is not built for
    assert ds(Hi=32) == sk.SCKV_EUNSUPPORTED
    assert ds(n_c=40000, start_pos=159999) == sk.SCKV_EUNSUPPORTED
    assert ds(K=5000) == sk.SCKV_EUNSUPPORTED      # win + K above 4096
    assert ds(k_new=None) == sk.SCKV_EINVAL        # one new row without the other
    assert ds(start_pos=32768, n_c=8192) == sk.SCKV_EINVAL  # no row completes at this step
    assert ds(n_c=8193) == sk.SCKV_EINVAL          # rows not yet visible
    assert ds(ws_bytes=100) == sk.SCKV_EWORKSPACE
    assert ds(B=0) == sk.SCKV_OK
    assert sk.sckv_decode_step_workspace_bytes(1, 64, 512, 8192, 640) >= 8192 * 2


def test_step_call_composition():
    """The calls a step is made of (host logic only): decode steps set up with
    sckv_decode_prepare (packed k cache) or the separate calls; every other
    step with sckv_prefill_prepare, or its separate calls when asked; a
    chunk's ring write follows its attention.  The one-launch set-up's
    algorithmic bytes are those of the calls it replaces."""
    import importlib.util

    import sckv_synth as synth
    from sparse_compressed_kv_e2m1_amd.step import step_call_names

    W = synth.WORKLOADS
    assert step_call_names(W["decode"], "fp4") == ["decode_prepare", "index_scores_topk", "sparse_attn_sink"]
    assert step_call_names(W["decode"], "bf16") == ["quant_latent", "quant_index_k", "ring_write", "window_idx",
                                                    "index_scores_topk", "sparse_attn_sink"]
    assert step_call_names(W["causal_prefill"], "fp4") == ["prefill_prepare", "index_scores_topk",
                                                           "sparse_attn_sink"]
    assert step_call_names(W["causal_prefill"], "fp4", prepare="separate") == [
        "quant_latent", "quant_index_k", "window_idx", "index_scores_topk", "sparse_attn_sink", "ring_write"]
    assert step_call_names(W["chunked_prefill"], "bf16") == ["prefill_prepare", "sparse_attn_sink", "ring_write"]
    assert step_call_names(W["chunked_prefill"], "bf16", prepare="separate") == [
        "quant_latent", "window_idx", "visible_idx", "sparse_attn_sink", "ring_write"]

    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for name, kc in (("causal_prefill", "fp4"), ("chunked_prefill", "bf16")):
        w = W[name]
        parts = [c for c in step_call_names(w, kc, prepare="separate") if c not in ("index_scores_topk",
                                                                                    "sparse_attn_sink")]
        if w.start_pos > 0:
            parts.remove("ring_write")  # a chunk's ring write stays a call of its own
        assert bench.counts(w, 1, "prefill_prepare", kc)["bytes"] == sum(bench.counts(w, 1, c, kc)["bytes"]
                                                                       for c in parts)

/*
 * sckv.h -- C ABI of the MI355X (gfx950) compressed sparse attention hot path.
 *
 * The operations come from three web pages of a DeepSeek-V4.1-style model:
 *   "metrale_model_arch/deepseek_v41_ref/compress.rs"  (compress.rs)
 *   "metrale_model_arch/attn_v41/forward.rs"            (forward.rs)
 *   "metrale_model_arch/deepseek_v41_layer.rs"          (layer.rs; context only)
 *
 * Conventions shared by every call:
 *   - Tensors are caller-owned, contiguous, row-major DEVICE memory unless a
 *     stride argument says otherwise.  bf16 tensors are passed as void* and
 *     hold bf16 bit patterns; indices are int32; f32 is float.
 *   - B is a leading batch of independent sequences with identical shapes
 *     (B = 1 is one sequence, as on the pages).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream; none allocates device memory,
 *     synchronises or keeps state between calls.  Faults inside a kernel show
 *     up at the caller's next synchronisation.
 *   - Arguments are checked on the host before anything is enqueued; on a
 *     failed check nothing is enqueued, the call returns a negative status and
 *     sckv_last_error() describes it (the pages' ensure!/context checks).
 *   - Return values: SCKV_OK (0) or one of the negative codes below.
 */
#ifndef SCKV_H_
#define SCKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sckv_status {
    SCKV_OK = 0,
    SCKV_EINVAL = -1,       /* bad shape, null pointer, bad mode, misaligned pointer */
    SCKV_EUNSUPPORTED = -2, /* a valid shape the library has no kernel for (see each call) */
    SCKV_EHIP = -3,         /* the HIP runtime refused a launch */
    SCKV_EWORKSPACE = -4    /* workspace pointer NULL or smaller than sckv_workspace_bytes() */
};

/* fp4 round-trip modes (compress.rs: fp4_quant_e4m3_inplace / fp4_quant_e8m0_inplace). */
enum sckv_quant_mode {
    SCKV_FP4_E4M3_B16 = 0, /* compressed KV latent: e4m3 block scales, 16 values a block */
    SCKV_FP4_E8M0_B32 = 1  /* indexer q and k: power-of-two block scales, 32 values a block */
};

/* Operations whose workspace size sckv_workspace_bytes() reports. */
enum sckv_op {
    SCKV_OP_INDEX_SCORES_TOPK = 0,
    SCKV_OP_SPARSE_ATTN_SINK = 1,
    SCKV_OP_INDEX_SCORES_TOPK_FP4 = 2
};

/*
 * sckv_quant -- the fp4 (e2m1) round trip of a flat bf16 array, in blocks of
 * 16 (E4M3_B16) or 32 (E8M0_B32) consecutive values (compress.rs:
 * fp4_quant_e4m3_inplace, fp4_quant_e8m0_inplace; forward.rs: the fp4_quant
 * call on the new latent groups before the cache copy).
 * For each block: amax = max |v|, floored at 6*2^-9 (E4M3) or 6*2^-126 (E8M0);
 * s = e4m3_rne(amax/6) (saturating at 448) or the power-of-two ceiling of
 * amax/6; every v becomes bf16(e2m1_rne(clamp(v/s, -6, 6)) * s), where v/s is
 * the correctly rounded binary32 quotient and e2m1_rne rounds to the nearest
 * of {0,.5,1,1.5,2,3,4,6} with ties to the even code and keeps the sign.
 *   x, y   [n] bf16 device arrays; x == y (in place) is allowed, any other
 *          overlap is not.
 *   n      number of values; must be a multiple of the block (16 or 32), else
 *          SCKV_EINVAL.  n == 0 is a no-op.
 *   mode   enum sckv_quant_mode.
 */
int sckv_quant(const void* x, void* y, int64_t n, int mode, void* stream);

/*
 * sckv_quant_rows -- the same round trip over `rows` rows of `cols` values
 * with row strides ldx / ldy (in elements), e.g. one new cache row in each of
 * B sequences.  cols must be a multiple of the block; blocks never cross rows.
 * In place (x == y, ldx == ldy) is allowed.
 */
int sckv_quant_rows(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols, int mode,
                    void* stream);

/*
 * sckv_quant_pack -- the same round trip as sckv_quant_rows, stored packed:
 * each value as its 4-bit e2m1 code (bits 0-2 the index into
 * {0, .5, 1, 1.5, 2, 3, 4, 6}, bit 3 the sign, so small negative values give
 * code 8, i.e. -0) and each block's scale as one byte: the E8M0 exponent e of
 * s = 2^(e - 127) (SCKV_FP4_E8M0_B32) or the E4M3FN code of s
 * (SCKV_FP4_E4M3_B16).  Codes of elements 2j and 2j+1 of a row share byte j,
 * 2j in the low nibble.  code value * scale is exactly the bf16 value
 * sckv_quant_rows would produce.  The packing is this library's storage of the
 * pages' round trip (the pages keep the values in bf16): 68 bytes instead of
 * 256 for a 128-wide indexer k row, 288 instead of 1024 for a 512-wide
 * latent row.
 *   x       [rows, cols] bf16, row stride ldx (elements)
 *   codes   [rows, cols/2] bytes, row stride ldc (bytes)
 *   scales  [rows, cols/block] bytes, row stride lds (bytes)
 * cols must be a multiple of the block; the three regions must not overlap.
 */
int sckv_quant_pack(const void* x, int64_t ldx, void* codes, int64_t ldc, void* scales, int64_t lds, int64_t rows,
                    int64_t cols, int mode, void* stream);

/*
 * sckv_yarn_freqs_cis -- HOST function: the rotation table of the compressed
 * layers' latent rotary embedding (compress.rs yarn_freqs_cis), computed once
 * per model on the host in binary32, in the page's order:
 *   f_i   = 1 / base^(2i/dim) for pair i < dim/2;
 *   low   = max(floor(d(beta_fast)), 0), high = min(ceil(d(beta_slow)), dim-1)
 *           with d(r) = dim ln(original_seq_len / (2 pi r)) / (2 ln base)
 *           (binary64, then binary32);
 *   ramp  = clamp((i - low) / max(high - low, 0.001), 0, 1), smooth = 1 - ramp,
 *   f_i   = f_i / factor * (1 - smooth) + f_i * smooth;
 *   table[p][i] = (cos(p f_i), sin(p f_i)) with the binary32 angle p * f_i.
 *   table  [seqlen, dim/2, 2] f32, HOST memory the caller owns (copy it to
 *          the device for sckv_rope_quant_rows / sckv_decode_prepare).
 * dim even and positive, base > 1, factor, beta_fast, beta_slow > 0, else
 * SCKV_EINVAL.  No device work.
 */
int sckv_yarn_freqs_cis(float* table, int dim, int64_t seqlen, int64_t original_seq_len, float base, float factor,
                        float beta_fast, float beta_slow);

/*
 * sckv_rope_quant_rows -- the latent path of new compressed rows (compress.rs
 * attention_any, forward.rs AttnV41::forward: the new latent groups are
 * rotated at their positions, then fp4 round-tripped with e4m3 scales in
 * blocks of 16, then written to the cache): row r of x is turned at position
 * pos0 + r * pos_step, then goes through sckv_quant_rows(SCKV_FP4_E4M3_B16).
 * The rotation (apply_rotary, not printed; the reading implemented): the last
 * rope_dim values of a row are rope_dim/2 pairs (2i, 2i+1) of that slice,
 * pair i of the row at position p becomes
 *   (x0 c - x1 s, x0 s + x1 c),  (c, s) = table[p][i],
 * with binary32 products and sums (no fused multiply-add), each result
 * rounded to bf16 (the latent buffer holds bf16) before the round trip; the
 * other values pass unchanged.  Compressed row j's position is j * ratio
 * (the page's g * ratio from position 0, start_pos + 1 - ratio in decode).
 *   x, y   [rows, cols] bf16, row strides ldx / ldy; in place allowed (x == y,
 *          ldx == ldy), other overlap not
 *   table  [n_pos, rope_dim/2, 2] f32 device array (sckv_yarn_freqs_cis),
 *          8-byte aligned
 * cols % 16 == 0, rope_dim even with 0 < rope_dim <= cols, pos0 >= 0,
 * pos_step >= 0 and every row's position below n_pos, else SCKV_EINVAL.
 */
int sckv_rope_quant_rows(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols,
                         const float* table, int64_t n_pos, int rope_dim, int64_t pos0, int64_t pos_step,
                         void* stream);

/*
 * sckv_rope_quant_pack -- sckv_rope_quant_rows stored packed: the rotated,
 * round-tripped latent rows as sckv_quant_pack(SCKV_FP4_E4M3_B16) stores them
 * (4-bit e2m1 codes, two a byte, the even element low; one E4M3FN scale byte
 * per 16 values).  288 bytes instead of 1024 for a 512-wide latent row; code
 * value * scale is exactly the bf16 value sckv_rope_quant_rows produces.
 *   x       [rows, cols] bf16, row stride ldx (elements)
 *   codes   [rows, cols/2] bytes, row stride ldc (bytes)
 *   scales  [rows, cols/16] bytes, row stride lds (bytes)
 *   table, n_pos, rope_dim, pos0, pos_step as in sckv_rope_quant_rows
 * x, codes and scales must not overlap.
 */
int sckv_rope_quant_pack(const void* x, int64_t ldx, void* codes, int64_t ldc, void* scales, int64_t lds, int64_t rows,
                         int64_t cols, const float* table, int64_t n_pos, int rope_dim, int64_t pos0, int64_t pos_step,
                         void* stream);

/*
 * sckv_ring_write -- write this step's m kv rows into the window ring: the row
 * of position p goes to slot p mod win; only the last min(m, win) positions
 * are written (forward.rs: the ring's one or two stream-ordered copies at
 * start_pos 0, the single-row copy at slot start_pos mod win otherwise).
 *   rows  [B, m, D] bf16 with batch stride rows_bstride (elements)
 *   ring  [B, win, D] bf16 with batch stride ring_bstride (elements)
 * The two regions must not overlap (the chunked layout [ring | chunk] in one
 * buffer, rows = buffer + win*D, satisfies this).
 */
int sckv_ring_write(const void* rows, int64_t rows_bstride, void* ring, int64_t ring_bstride, int B, int64_t m,
                    int64_t start_pos, int win, int D, void* stream);

/*
 * sckv_rows_a_len -- length of rows_a, the first row base of a step (the
 * compressed rows' index offset, forward.rs `offset = rows_a_len`):
 *   start_pos == 0        m        (rows_a = this step's fresh kv rows)
 *   m == 1, start_pos > 0 win      (rows_a = the ring, after the new row's write)
 *   m > 1,  start_pos > 0 win + m  (rows_a = the ring before the chunk, then
 *                                   the m chunk rows; an extension: the pages
 *                                   copy a single row at start_pos > 0)
 * Host-only, no device work.  Returns -1 for invalid arguments.
 */
int64_t sckv_rows_a_len(int win, int64_t m, int64_t start_pos);

/*
 * sckv_window_idx -- the window part of every query's index list (forward.rs:
 * window_topk_idxs, whose body is not printed; the reading used here): for the
 * query at position p the rows_a indices of positions max(0, p-win+1) .. p,
 * oldest first, then -1 up to win entries.  rows_a is laid out as
 * sckv_rows_a_len() describes.
 *   idx  [B, m, ld] int32; columns 0 .. win-1 are written (same for every b).
 *   ld >= win.
 */
int sckv_window_idx(int B, int64_t m, int64_t start_pos, int win, int32_t* idx, int64_t ld, void* stream);

/*
 * sckv_decode_prepare -- the set-up calls of a decode step (m = 1, start_pos
 * > 0) for B sequences in one launch (forward.rs AttnV41::forward: the fp4
 * round trip of a completed latent group before its cache copy, the ring copy
 * at slot start_pos mod win before attention, window_topk_idxs; compress.rs
 * fp4_quant_e4m3_inplace, fp4_quant_e8m0_inplace).  The result is exactly
 * that of, in any order (the four write disjoint memory):
 *   sckv_quant_rows(lat_new, ld_lat_new, lat_dst, ld_lat_dst, B, D, SCKV_FP4_E4M3_B16)
 *     (sckv_rope_quant_rows with the same rows when rope_table is given)
 *   sckv_quant_pack(k_new, ld_k_new, k_codes, ld_codes, k_scales, ld_scales, B, Di, SCKV_FP4_E8M0_B32)
 *   sckv_ring_write(kv_new, ld_kv_new, ring, ld_ring, B, 1, start_pos, win, D)
 *   sckv_window_idx(B, 1, start_pos, win, idx, ld_idx)
 *   lat_new    [B] raw latent rows of D bf16, stride ld_lat_new (elements), or
 *              NULL when no compressed row completes at this step (then
 *              lat_dst is not touched)
 *   lat_dst    the B destination rows in the latent cache, stride ld_lat_dst
 *   k_new      [B] raw indexer k rows of Di bf16, stride ld_k_new, or NULL
 *   k_codes    destination code rows (Di/2 bytes), stride ld_codes (bytes)
 *   k_scales   destination scale bytes (Di/32), stride ld_scales (bytes)
 *   kv_new     [B] new kv rows of D bf16, stride ld_kv_new
 *   ring       [B, win, D] bf16, stride ld_ring per sequence (>= win*D)
 *   idx        [B, 1, ld_idx] int32; columns 0 .. win-1 written
 *   rope_table the rotation table ([n_pos, rope_dim/2, 2] f32 on the device,
 *              sckv_yarn_freqs_cis), or NULL: with a table the latent rows
 *              are turned at position lat_pos before their round trip, exactly
 *              as sckv_rope_quant_rows(lat_new, ld_lat_new, lat_dst,
 *              ld_lat_dst, B, D, rope_table, n_pos, rope_dim, lat_pos, 0)
 *   lat_codes  with lat_dst NULL: the latent rows are stored packed instead,
 *              as sckv_rope_quant_pack (or sckv_quant_pack in SCKV_FP4_E4M3_B16
 *              without a table) would: codes rows of D/2 bytes, stride
 *              ld_lat_codes, and lat_scales rows of D/16 e4m3 scale bytes,
 *              stride ld_lat_scales (bytes)
 * D % 16 == 0, Di % 32 == 0; every row pointer 16-byte aligned and every
 * stride a multiple of 16 bytes (ld_scales excepted), else SCKV_EINVAL.
 */
int sckv_decode_prepare(const void* lat_new, int64_t ld_lat_new, void* lat_dst, int64_t ld_lat_dst,
                        const void* k_new, int64_t ld_k_new, void* k_codes, int64_t ld_codes, void* k_scales,
                        int64_t ld_scales, int Di, const void* kv_new, int64_t ld_kv_new, void* ring,
                        int64_t ld_ring, int B, int D, int win, int64_t start_pos, int32_t* idx, int64_t ld_idx,
                        const float* rope_table, int64_t n_pos, int rope_dim, int64_t lat_pos, void* lat_codes,
                        int64_t ld_lat_codes, void* lat_scales, int64_t ld_lat_scales, void* stream);

/*
 * sckv_prefill_prepare -- the set-up calls of a step of m >= 1 queries for B
 * sequences in one launch (forward.rs AttnV41::forward: the fp4 round trip of
 * the completed latent groups before their cache copy, window_topk_idxs,
 * compress_len = (start_pos + m) / ratio, the ring's stream-ordered copies;
 * compress.rs fp4_quant_e4m3_inplace, fp4_quant_e8m0_inplace and the rotation
 * of a new latent group before its round trip).  The result is exactly that
 * of, in any order (the parts read only these inputs and write disjoint
 * memory), for every sequence b (X_b = X + b * bs_X):
 *   sckv_rope_quant_rows(lat_new_b, D, lat_dst_b, D, n_new, D, rope_table,
 *       n_pos, rope_dim, pos0, pos_step)           (latent rows, bf16 out)
 *     or sckv_rope_quant_pack(lat_new_b, D, lat_codes_b, D/2, lat_scales_b,
 *       D/16, n_new, D, ...)                        (latent rows, packed)
 *     (sckv_quant_rows / sckv_quant_pack in SCKV_FP4_E4M3_B16 when
 *     rope_table is NULL)
 *   sckv_quant_rows(k_new_b, Di, k_dst_b, Di, n_new, Di, SCKV_FP4_E8M0_B32)
 *     or sckv_quant_pack(k_new_b, Di, k_codes_b, Di/2, k_scales_b, Di/32,
 *       n_new, Di, SCKV_FP4_E8M0_B32)
 *   sckv_window_idx(B, m, start_pos, win, idx, ld_idx)
 *   sckv_visible_idx(B, m, start_pos, ratio, n_c, K, offset, idx, ld_idx, win)
 *     (only when K > 0)
 *   sckv_ring_write(ring_src, bs_ring_src, ring, bs_ring, B, m, start_pos,
 *       win, D)                                      (only when ring_src is given)
 * Every row set is contiguous within a sequence (row stride = row length);
 * the batch strides bs_* count elements for bf16 rows and bytes for codes
 * and scales.
 *   lat_new    [B, n_new, D] raw latent rows, or NULL (or n_new = 0): no
 *              latent part; give lat_dst ([B] x n_new bf16 rows, e.g. the
 *              cache's first new row) or lat_codes + lat_scales, not both
 *   k_new      [B, n_new, Di] raw indexer k rows, or NULL: no k part; give
 *              k_dst or k_codes + k_scales, not both
 *   ring_src   [B, m, D] the step's kv rows, or NULL: no ring write.  The
 *              ring is written in this launch, so give it only when nothing
 *              later in the step reads the ring's earlier rows (a step from
 *              position 0); a chunk's ring write follows its attention
 *   idx        [B, m, ld_idx] int32, ld_idx >= win + K
 * Sources and destinations must not overlap (no in-place round trip).
 * D % 16 == 0, Di % 32 == 0; bf16 rows and k codes 16-byte aligned, latent
 * codes 8-byte aligned, batch strides multiples of 16 bytes (8 for latent
 * codes, scales any), else SCKV_EINVAL; the checks of the separate calls
 * (rotation table, K >= every visible count) apply.
 */
int sckv_prefill_prepare(int B, int64_t m, int64_t start_pos, int win, int D, int64_t n_new, const void* lat_new,
                         int64_t bs_lat_new, void* lat_dst, int64_t bs_lat_dst, void* lat_codes, int64_t bs_lat_codes,
                         void* lat_scales, int64_t bs_lat_scales, const float* rope_table, int64_t n_pos,
                         int rope_dim, int64_t pos0, int64_t pos_step, const void* k_new, int64_t bs_k_new, int Di,
                         void* k_dst, int64_t bs_k_dst, void* k_codes, int64_t bs_k_codes, void* k_scales,
                         int64_t bs_k_scales, const void* ring_src, int64_t bs_ring_src, void* ring, int64_t bs_ring,
                         int32_t* idx, int64_t ld_idx, int ratio, int64_t n_c, int K, int32_t offset, void* stream);

/*
 * sckv_decode_step -- a whole decode step (m = 1 at start_pos > 0) of B <= 64
 * sequences in ONE launch (forward.rs AttnV41::forward: ring copy, window
 * list, indexer, merge, attend_and_project; compress.rs: the round trips, the
 * rotation, attention_any).  It computes the same as
 *   sckv_decode_prepare(lat_new, D, latent row n_c-1, n_c*D, k_new, Di, k_codes
 *       row n_c-1, n_c*Di/2, k_scales row n_c-1, n_c*Di/32, Di, kv_new, D, ring,
 *       win*D, B, D, win, start_pos, idx, win+K, rope_table, n_pos, rope_dim,
 *       (n_c-1)*ratio, NULL, 0, NULL, 0)
 *   sckv_index_scores_topk_fp4(iq, k_codes, k_scales, w, B, 1, Hi, Di, n_c,
 *       ratio, start_pos, K, win, idx, win+K, win, NULL, ...)
 *   sckv_sparse_attn_sink(q, ring, win, latent, n_c, idx, win+K, sink, scale,
 *       B, 1, H, D, out, ...)
 * run as phases of one cooperative launch with grid-wide barriers between
 * them (the keys, index lists and split partials pass through ws): the ring,
 * caches and index lists bit for bit; the outputs to rounding, as its
 * attention phase splits each query's list into 64-head work items where
 * sckv_sparse_attn_sink at B <= 64 uses 16-head workgroups (the two sum the
 * split partials in different groupings; both within the attention
 * tolerance of the exact result).  For
 * callers that need a step as a single launch: on MI355X each grid barrier
 * (device-scope atomics across the eight XCDs' L2s) costs a few microseconds,
 * more than the launch gaps of the separate calls, so those are faster at
 * every batch size measured (B = 1 at n_c = 8192: 69 us launched, 74 us
 * replayed from a HIP graph, against 44 and 30 us for the separate calls).
 *   lat_new, k_new  [B] new raw latent rows (D bf16) and raw indexer k rows (Di
 *                   bf16), contiguous, or both NULL when no compressed row
 *                   completes at this step (else (start_pos+1) % ratio == 0 and
 *                   n_c == (start_pos+1)/ratio: they become row n_c - 1)
 *   kv_new          [B, D] the new kv rows (ring slot start_pos mod win)
 *   rope_table      [n_pos, rope_dim/2, 2] f32 rotation table or NULL
 *   latent          [B, n_c, D] bf16 latent cache; k_codes [B, n_c, Di/2],
 *                   k_scales [B, n_c, Di/32] the packed indexer k cache;
 *                   ring [B, win, D]
 *   iq [B, Hi, Di] raw indexer q; w [B, Hi] f32; q [B, H, D]; sink [H] f32
 *   idx [B, win+K] int32 (written); out [B, H, D] bf16 (written)
 *   ws   at least sckv_decode_step_workspace_bytes(B, H, D, n_c, win+K); its
 *        first 256 bytes hold the launch's barrier counters: they must be
 *        zero before the first call that uses the workspace (allocate it
 *        zeroed), and every completed call leaves them zero.  Calls that
 *        share a workspace must not overlap (one stream).
 * Supported: Hi = 64, Di = 128, D = 512, 33 <= H <= 64, B <= 64, n_c <= 32768
 * with every compressed row visible at start_pos, win + K <= 4096, a device
 * with cooperative launch (else SCKV_EUNSUPPORTED); 16-byte aligned rows.
 */
int sckv_decode_step(const void* lat_new, const void* k_new, const void* kv_new, const float* rope_table,
                     int64_t n_pos, int rope_dim, void* latent, void* k_codes, void* k_scales, void* ring,
                     const void* iq, const float* w, int Hi, int Di, int ratio, int K, const void* q,
                     const float* sink, float scale, int H, int B, int64_t n_c, int D, int win, int64_t start_pos,
                     int32_t* idx, void* out, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of sckv_decode_step ((size_t)-1 for invalid arguments). */
size_t sckv_decode_step_workspace_bytes(int B, int H, int D, int64_t n_c, int T);

/*
 * sckv_visible_idx -- the compressed part of every query's index list when
 * every causally visible compressed row is attended (a layer without an
 * indexer): offset + j for j < V_p, then -1 up to K, where compressed row j is
 * visible to position p iff (j+1)*ratio <= p+1 and j < n_c (forward.rs:
 * compress_len = (start_pos+m)/ratio).
 *   idx  [B, m, ld] int32; columns col0 .. col0+K-1 are written.
 *   K must be >= every V_p of the step (else SCKV_EINVAL).
 */
int sckv_visible_idx(int B, int64_t m, int64_t start_pos, int ratio, int64_t n_c, int K, int32_t offset,
                     int32_t* idx, int64_t ld, int64_t col0, void* stream);

/*
 * sckv_index_scores_topk -- indexer scores of every query against its visible
 * compressed rows, then a per-query top-K (forward.rs: the indexer call and
 * the [window | compressed] merge; compress.rs module doc: q and k go through
 * the fp4 round trip with power-of-two scales in blocks of 32, and scores are
 * bf16 values).  The scoring formula is not printed on the pages; the reading
 * implemented is the lightning-indexer form:
 *   q_hat[t,h]  = E8M0_B32 round trip of the raw q[t,h,:] (fused; bit-identical
 *                 to sckv_quant on q),
 *   d[t,h,s]    = q_hat[t,h,:] . k[s,:], accumulated in binary32 (exact for
 *                 round-tripped N(0,1)-scale data; see the exactness note),
 *   r[t,h,s]    = fl32(w[t,h] * (d > 0 ? d : +0)),
 *   score[t,s]  = bf16_rne of the pairwise head sum, strides Hi/2, .., 1.
 * Top-K: the K_t = min(K, V_t) visible rows with the largest scores (-0 equals
 * +0), ties to the lower row; written as offset + s in ascending s into
 * columns col0 .. col0+K_t-1 of idx, then -1 up to K.  V_t = 0 writes K x -1.
 *   q        [B, m, Hi, Di] bf16, raw (before the round trip)
 *   k        [B, n_c, Di] bf16, already round-tripped (E8M0_B32)
 *   w        [B, m, Hi] f32 per-head weights
 *   idx      [B, m, ld] int32
 *   scores   optional [B, m, n_c] bf16 output of the scores (NULL = none);
 *            entries of invisible rows are left unchanged.
 *   ws       device workspace of at least
 *            sckv_workspace_bytes(SCKV_OP_INDEX_SCORES_TOPK, B, m, Hi, Di, n_c).
 * Supported: Hi a power of two <= 64, Di in {32, 64, 128, 256}, n_c <= 65536.
 * Exactness note: the binary32 dot equals the exact dot whenever the exact
 * value is a binary32 value, which holds when the 2*Di products' block scales
 * lie within a few powers of two of each other (always the case for
 * round-tripped data of one magnitude); then every bit matches the oracle.
 */
int sckv_index_scores_topk(const void* q, const void* k, const float* w, int B, int64_t m, int Hi, int Di,
                           int64_t n_c, int ratio, int64_t start_pos, int K, int32_t offset, int32_t* idx,
                           int64_t ld, int64_t col0, void* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * sckv_index_scores_topk_fp4 -- sckv_index_scores_topk with the k cache
 * stored packed (sckv_quant_pack, SCKV_FP4_E8M0_B32): the same scores, bit for
 * bit, and the same top-K lists.  q is still the raw bf16 q; each workgroup
 * takes its query's round trip and packs it in on-chip memory, and both
 * operands go through the gfx950 scaled fp4 matrix cores (e2m1 x e2m1 with one E8M0 scale per 32 values, exact
 * products; the exactness note above applies unchanged).
 *   k_codes   [B, n_c, Di/2] bytes, contiguous, 16-byte aligned
 *   k_scales  [B, n_c, Di/32] bytes, contiguous, 4-byte aligned
 *   ws        at least sckv_workspace_bytes(SCKV_OP_INDEX_SCORES_TOPK_FP4,
 *             B, m, Hi, Di, n_c)
 * Supported: as sckv_index_scores_topk, with Di in {128, 256}.
 */
int sckv_index_scores_topk_fp4(const void* q, const void* k_codes, const void* k_scales, const float* w, int B,
                               int64_t m, int Hi, int Di, int64_t n_c, int ratio, int64_t start_pos, int K,
                               int32_t offset, int32_t* idx, int64_t ld, int64_t col0, void* scores, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * sckv_sparse_attn_sink -- sparse MQA attention over the rows named by each
 * query's index list, with a per-head sink logit (compress.rs attention_any:
 * the sparse_attn call with scale = head_dim^-1/2, the kv rows being the
 * window rows followed by the compressed rows; forward.rs attend_and_project:
 * two row bases rows_a / rows_b addressed through one index list).  For query
 * t and head h: entry i of idx[t] names rows_a[idx] when idx < ra, else
 * rows_b[idx - ra]; -1 (and any value outside [0, ra+rb)) is skipped.  Each
 * row is both key and value.  With l_i = scale * q[t,h,:] . row_i:
 *   out[t,h,:] = sum_i e^(l_i - M) row_i / (e^(sink_h - M) + sum_i e^(l_i - M)),
 * M = max(sink_h, max_i l_i); no valid entry gives 0.  f32 accumulation,
 * bf16 output.
 *   q      [B, m, H, D] bf16
 *   rows_a [B, ra, D] bf16     rows_b [B, rb, D] bf16 (NULL allowed when rb == 0)
 *   idx    [B, m, T] int32     sink [H] f32     out [B, m, H, D] bf16
 *   q, rows_a, rows_b and out 16-byte aligned, idx and sink 4-byte aligned
 *   (else SCKV_EINVAL)
 *   ws     device workspace of at least
 *          sckv_workspace_bytes(SCKV_OP_SPARSE_ATTN_SINK, B, m, H, D, T).
 * Supported: H <= 64, D in {64, 128, 256, 512}, 1 <= T <= 65536.
 */
int sckv_sparse_attn_sink(const void* q, const void* rows_a, int64_t ra, const void* rows_b, int64_t rb,
                          const int32_t* idx, int T, const float* sink, float scale, int B, int64_t m, int H, int D,
                          void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * sckv_sparse_attn_sink_fp4 -- sckv_sparse_attn_sink with the compressed rows
 * (rows_b, the latent cache) stored packed as sckv_rope_quant_pack /
 * sckv_quant_pack(SCKV_FP4_E4M3_B16) store them: the same results, bit for
 * bit, as sckv_sparse_attn_sink over the bf16 values they stand for (code
 * value * scale, which is exactly the latent round trip).  Each packed row is
 * read once (288 bytes instead of 1024 at D = 512) and expanded to bf16 on
 * chip.  rows_a stays bf16 (the window rows are not round-tripped).
 *   rows_b_codes   [B, rb, D/2] bytes, 16-byte aligned
 *   rows_b_scales  [B, rb, D/16] bytes (e4m3 codes), 16-byte aligned
 * Supported: D = 512 (else SCKV_EUNSUPPORTED); the rest as
 * sckv_sparse_attn_sink, with the same workspace size.
 */
int sckv_sparse_attn_sink_fp4(const void* q, const void* rows_a, int64_t ra, const void* rows_b_codes,
                              const void* rows_b_scales, int64_t rb, const int32_t* idx, int T, const float* sink,
                              float scale, int B, int64_t m, int H, int D, void* out, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * sckv_sparse_attn_sink_noalloc -- sckv_sparse_attn_sink for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without the
 * workspace, the same kernels and the same results bit for bit.  The split
 * partials that sckv_sparse_attn_sink keeps in the caller's workspace live in
 * a static device array of sckv_sparse_attn_sink_noalloc_max_bytes() bytes
 * (32 MiB) that the library holds on each GPU it runs on until the process
 * ends; the call allocates nothing.  Shapes whose partials need more than
 * that (sckv_workspace_bytes(SCKV_OP_SPARSE_ATTN_SINK, ...) above the
 * maximum, e.g. 64 heads x 512 at fewer than 256 queries with long lists)
 * return SCKV_EUNSUPPORTED with nothing enqueued.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other
 * host threads) race and must be ordered by the caller.
 */
int sckv_sparse_attn_sink_noalloc(const void* q, const void* rows_a, int64_t ra, const void* rows_b, int64_t rb,
                                  const int32_t* idx, int T, const float* sink, float scale, int B, int64_t m, int H,
                                  int D, void* out, void* stream);

/* Bytes of the static scratch of sckv_sparse_attn_sink_noalloc. */
size_t sckv_sparse_attn_sink_noalloc_max_bytes(void);

/*
 * sckv_workspace_bytes -- device workspace an operation needs for the given
 * shape: op = SCKV_OP_INDEX_SCORES_TOPK or SCKV_OP_INDEX_SCORES_TOPK_FP4 with
 * (H, D, n) = (Hi, Di, n_c), or SCKV_OP_SPARSE_ATTN_SINK with (H, D, n) =
 * (H, D, T).  0 means none needed.
 * Returns (size_t)-1 for invalid arguments.
 */
size_t sckv_workspace_bytes(int op, int B, int64_t m, int H, int D, int64_t n);

/* Thread-local description of the last failed call on this thread ("" if none). */
const char* sckv_last_error(void);

/* ABI version of this header: 2. */
int sckv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SCKV_H_ */

/*
 * sckv_oracle.c -- plain, slow CPU oracle of the compressed sparse attention
 * hot path (fp4 e2m1 round trips, indexer scores and top-k, sparse MQA
 * attention with a per-head sink).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code, header,
 * table or constant with the HIP library: every rule below is written out
 * again from the pages' text.
 *
 * Sources (web pages, cited by title and item):
 *   [compress.rs]  "metrale_model_arch/deepseek_v41_ref/compress.rs" --
 *                  module doc (precision statement), FP4_BLOCK, LATENT_BLOCK,
 *                  FP4_MAX, E2M1, to_e2m1_rne, fp4_quant_e8m0_inplace,
 *                  fp4_quant_e4m3_inplace, attention_any.
 *   [forward.rs]   "metrale_model_arch/attn_v41/forward.rs" -- AttnV41::forward
 *                  (window ring copies, offset, compress_len, merge, workspace
 *                  bound).
 * Steps the pages name but do not print (pow2_ceil, the e4m3 conversion,
 * window_topk_idxs, the indexer formula, sparse_attn) follow the readings
 * listed at each function.
 *
 * Floating point: compiled with -O2 -ffp-contract=off -fno-fast-math on
 * x86-64 (SSE2), so every float operation is one IEEE binary32 operation and
 * every double operation one binary64 operation; no flush of subnormals.
 *
 * bf16 values travel as uint16_t bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 <-> f32                                                             */
/* ------------------------------------------------------------------------ */

/* Widening is exact: the bf16 bits are the top half of the binary32 bits. */
float sckvo_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 value to the nearest bf16 value, ties to the even
 * significand (the pages' to_bf16_rne).  Written from the definition: the two
 * bf16 neighbours of x are the value with the low 16 bits cleared (towards
 * zero) and the next bf16 value away from zero; pick the nearer one, on a tie
 * the one whose last kept bit is 0.  The sign of zero is kept.  NaN input is
 * outside the contract (the pages' inputs are finite). */
uint16_t sckvo_f32_to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t lo_bits = (uint16_t)(u >> 16);          /* towards zero */
    uint16_t hi_bits = (uint16_t)(lo_bits + 1);      /* away from zero (may become inf) */
    double ax = fabs((double)x);
    double lo = fabs((double)sckvo_bf16_to_f32(lo_bits));
    double hi = fabs((double)sckvo_bf16_to_f32(hi_bits));
    if (isinf(hi)) hi = ldexp(1.0, 128); /* as if the exponent were unbounded: overflow rounds to inf */
    if (ax == lo) return lo_bits;
    double dlo = ax - lo, dhi = hi - ax;              /* exact in binary64 */
    if (dlo < dhi) return lo_bits;
    if (dhi < dlo) return hi_bits;
    return (lo_bits & 1u) ? hi_bits : lo_bits;
}

/* ------------------------------------------------------------------------ */
/* e2m1 rounding  [compress.rs: E2M1, to_e2m1_rne]                          */
/* ------------------------------------------------------------------------ */

/* The eight magnitudes of the e2m1 grid, as printed on the page (FP4_MAX is
 * the largest). */
static const float ORACLE_E2M1_GRID[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* Round y onto the e2m1 grid: the grid magnitude nearest to |y|; when |y|
 * is exactly half-way between two grid magnitudes the one with the even
 * code (index into the grid) wins.  The sign of y is carried over with
 * copysign, so a small negative y gives -0. */
float sckvo_e2m1_rne(float y) {
    float a = fabsf(y);
    /* Past the top of the grid the nearest point is the top (6); said
     * explicitly because a - 4 and a - 6 are no longer distinct doubles for
     * huge a.  Inside the quantisers |y| <= 6 always (FP4_MAX clamp). */
    if (a >= ORACLE_E2M1_GRID[7]) return copysignf(ORACLE_E2M1_GRID[7], y);
    int best = 0;
    double best_d = fabs((double)a - (double)ORACLE_E2M1_GRID[0]);
    for (int c = 1; c < 8; ++c) {
        double d = fabs((double)a - (double)ORACLE_E2M1_GRID[c]);
        if (d < best_d || (d == best_d && (c % 2) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return copysignf(ORACLE_E2M1_GRID[best], y);
}

/* ------------------------------------------------------------------------ */
/* Scale helpers                                                            */
/* ------------------------------------------------------------------------ */

/* pow2_ceil (named on the compress.rs page, body not printed).  Reading: the
 * smallest power of two that is >= x, for finite x > 0.  Plain search by
 * doubling and halving; every intermediate is an exact power of two. */
float sckvo_pow2_ceil(float x) {
    double p = 1.0;
    double xd = (double)x;
    if (!(xd > 0.0) || isinf(xd)) return NAN; /* outside the contract */
    while (p < xd) p *= 2.0;
    while (p / 2.0 >= xd) p /= 2.0;
    return (float)p;
}

/* The value of an OCP E4M3FN code (bias 7, three mantissa bits, subnormals
 * k * 2^-9, no infinities, 0x7f / 0xff = NaN). */
float sckvo_e4m3_to_f32(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 0xf;
    int mnt = code & 7;
    double v;
    if (e == 0xf && mnt == 7) return NAN;
    if (e == 0)
        v = ldexp((double)mnt, -9);
    else
        v = ldexp(1.0 + mnt / 8.0, e - 7);
    return (float)(sign ? -v : v);
}

/* f32 -> E4M3FN, round to nearest, ties to the even code (f32_to_e4m3_rne is
 * named on the compress.rs page, body not printed).  Brute force over the 127
 * non-negative finite codes.  Reading for magnitudes past the largest finite
 * value (448): saturate to 448.  Returns the code. */
uint8_t sckvo_f32_to_e4m3(float x) {
    double a = fabs((double)x);
    int best = 0;
    double best_d = a;
    for (int c = 1; c <= 0x7e; ++c) {
        double d = fabs(a - (double)sckvo_e4m3_to_f32((uint8_t)c));
        if (d < best_d || (d == best_d && (c % 2) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | (signbit(x) ? 0x80 : 0));
}

/* ------------------------------------------------------------------------ */
/* The two fp4 round trips  [compress.rs: fp4_quant_e8m0_inplace,            */
/* fp4_quant_e4m3_inplace, FP4_BLOCK = 32, LATENT_BLOCK = 16]                */
/* ------------------------------------------------------------------------ */

/* One value of a block: divide by the block scale (IEEE binary32 division),
 * clamp to [-6, 6], round onto e2m1, multiply back by the scale and round the
 * product to bf16. */
static uint16_t oracle_fp4_value(float v, float s) {
    float y = v / s;
    if (y > 6.0f) y = 6.0f;
    if (y < -6.0f) y = -6.0f;
    float e = sckvo_e2m1_rne(y);
    return sckvo_f32_to_bf16(e * s);
}

/* The largest magnitude in a block, as binary32. */
static float oracle_block_amax(const uint16_t* x, int64_t len) {
    float amax = 0.0f;
    for (int64_t i = 0; i < len; ++i) {
        float a = fabsf(sckvo_bf16_to_f32(x[i]));
        if (a > amax) amax = a;
    }
    return amax;
}

/* Power-of-two scales (indexer q and k; block 32 on the pages).  amax is
 * floored at 6 * 2^-126 and the scale is pow2_ceil(amax / 6).  Blocks are
 * consecutive runs of `block` values; a shorter last block is quantised on its
 * own, as slice chunks are. */
void sckvo_quant_e8m0(const uint16_t* x, uint16_t* y, int64_t n, int64_t block) {
    const float floor_amax = 6.0f * ldexpf(1.0f, -126);
    for (int64_t b0 = 0; b0 < n; b0 += block) {
        int64_t len = (n - b0 < block) ? n - b0 : block;
        float amax = oracle_block_amax(x + b0, len);
        if (amax < floor_amax) amax = floor_amax;
        float s = sckvo_pow2_ceil(amax / 6.0f);
        for (int64_t i = 0; i < len; ++i) y[b0 + i] = oracle_fp4_value(sckvo_bf16_to_f32(x[b0 + i]), s);
    }
}

/* e4m3 scales (the compressed KV latent; block 16 on the pages).  amax is
 * floored at 6 * 2^-9 and the scale is amax / 6 rounded through e4m3. */
void sckvo_quant_e4m3(const uint16_t* x, uint16_t* y, int64_t n, int64_t block) {
    const float floor_amax = 6.0f * ldexpf(1.0f, -9);
    for (int64_t b0 = 0; b0 < n; b0 += block) {
        int64_t len = (n - b0 < block) ? n - b0 : block;
        float amax = oracle_block_amax(x + b0, len);
        if (amax < floor_amax) amax = floor_amax;
        float s = sckvo_e4m3_to_f32(sckvo_f32_to_e4m3(amax / 6.0f));
        for (int64_t i = 0; i < len; ++i) y[b0 + i] = oracle_fp4_value(sckvo_bf16_to_f32(x[b0 + i]), s);
    }
}

/* ------------------------------------------------------------------------ */
/* Packed storage of the round trip (not on the pages: the e2m1 values and  */
/* their block scales in 4-bit codes and one scale byte per block)           */
/* ------------------------------------------------------------------------ */

/* Storage format (a reading; the pages keep the round-tripped values in
 * bf16): value i of a block is the 4-bit e2m1 code (bit 3 the sign, bits 0-2
 * the index into {0, .5, 1, 1.5, 2, 3, 4, 6}); codes 2j and 2j+1 of the flat
 * array share byte j, 2j in the low nibble.  One scale byte per block: the
 * E8M0 exponent e (scale 2^(e - 127)) for power-of-two scales, the E4M3FN
 * code of the scale otherwise.  A value and its code give the same number, so
 * unpacking returns exactly the round trip. */
static const float oracle_grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static int oracle_e2m1_code(float r) {
    float a = fabsf(r);
    int idx = -1;
    for (int i = 0; i < 8; ++i)
        if (oracle_grid[i] == a) idx = i;
    if (idx < 0) abort(); /* r is always a grid value here */
    return idx | (signbit(r) ? 8 : 0);
}

/* mode 1: power-of-two scales (E8M0), mode 0: e4m3 scales; n a multiple of block. */
void sckvo_pack_fp4(const uint16_t* x, int64_t n, int64_t block, int mode, uint8_t* codes, uint8_t* scales) {
    const float floor_amax = mode ? 6.0f * ldexpf(1.0f, -126) : 6.0f * ldexpf(1.0f, -9);
    memset(codes, 0, (size_t)(n / 2));
    for (int64_t b0 = 0; b0 < n; b0 += block) {
        float amax = oracle_block_amax(x + b0, block);
        if (amax < floor_amax) amax = floor_amax;
        float s;
        if (mode) {
            s = sckvo_pow2_ceil(amax / 6.0f);
            int e;
            frexpf(s, &e); /* s = 0.5 * 2^e exactly */
            scales[b0 / block] = (uint8_t)(e - 1 + 127);
        } else {
            uint8_t c = sckvo_f32_to_e4m3(amax / 6.0f);
            s = sckvo_e4m3_to_f32(c);
            scales[b0 / block] = c;
        }
        for (int64_t i = 0; i < block; ++i) {
            float y = sckvo_bf16_to_f32(x[b0 + i]) / s;
            if (y > 6.0f) y = 6.0f;
            if (y < -6.0f) y = -6.0f;
            int code = oracle_e2m1_code(sckvo_e2m1_rne(y));
            int64_t k = b0 + i;
            codes[k / 2] |= (uint8_t)(code << ((k & 1) ? 4 : 0));
        }
    }
}

/* The bf16 values that packed codes and scales stand for. */
void sckvo_unpack_fp4(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t block, int mode, uint16_t* y) {
    for (int64_t k = 0; k < n; ++k) {
        int code = (codes[k / 2] >> ((k & 1) ? 4 : 0)) & 15;
        uint8_t sb = scales[k / block];
        double s = mode ? ldexp(1.0, (int)sb - 127) : (double)sckvo_e4m3_to_f32(sb);
        double v = (double)oracle_grid[code & 7] * s;
        y[k] = sckvo_f32_to_bf16((float)((code & 8) ? -v : v));
    }
}

/* ------------------------------------------------------------------------ */
/* Window ring, window rows, visibility  [forward.rs: ring copies, offset,   */
/* compress_len; compress.rs: attention_any]                                 */
/* ------------------------------------------------------------------------ */

/* The ring holds the kv row of position p in slot p mod win.  Writing the m
 * new rows one position at a time, in order, leaves the same ring as the
 * pages' one or two bulk copies (later positions overwrite earlier ones). */
void sckvo_ring_write(uint16_t* ring, int win, int D, const uint16_t* rows, int64_t m, int64_t start_pos) {
    for (int64_t t = 0; t < m; ++t) {
        int64_t slot = (start_pos + t) % win;
        memcpy(ring + slot * (int64_t)D, rows + t * (int64_t)D, (size_t)D * sizeof(uint16_t));
    }
}

/* Where the kv row of position q lives in rows_a for a step of m tokens at
 * start_pos (reading of window_topk_idxs, whose body is not printed):
 *   start_pos == 0          rows_a = the m fresh rows        -> row q
 *   m == 1, start_pos > 0   rows_a = the ring after the write -> slot q mod win
 *   m > 1,  start_pos > 0   rows_a = the ring before the chunk, then the m
 *                           chunk rows -> q mod win for q < start_pos,
 *                           win + (q - start_pos) otherwise.
 * Returns rows_a's length (the compressed rows' offset). */
static int64_t oracle_window_row(int win, int64_t m, int64_t start_pos, int64_t q) {
    if (start_pos == 0) return q;
    if (m == 1) return q % win;
    if (q < start_pos) return q % win;
    return win + (q - start_pos);
}

int64_t sckvo_rows_a_len(int win, int64_t m, int64_t start_pos) {
    if (start_pos == 0) return m;
    if (m == 1) return win;
    return win + m;
}

/* The window part of every query's index list: width win; the rows of the
 * positions max(0, p - win + 1) .. p, oldest first, then -1 up to the width.
 * idx is [m, ld]; columns 0 .. win-1 are written. */
int64_t sckvo_window_idx(int win, int64_t m, int64_t start_pos, int32_t* idx, int64_t ld) {
    for (int64_t t = 0; t < m; ++t) {
        int64_t p = start_pos + t;
        int64_t first = p - win + 1;
        if (first < 0) first = 0;
        int64_t j = 0;
        for (int64_t q = first; q <= p; ++q) idx[t * ld + j++] = (int32_t)oracle_window_row(win, m, start_pos, q);
        for (; j < win; ++j) idx[t * ld + j] = -1;
    }
    return sckvo_rows_a_len(win, m, start_pos);
}

/* Number of compressed rows visible to position p: row j is visible iff
 * (j + 1) * ratio <= p + 1, and only the n_c rows that exist count. */
int64_t sckvo_visible(int64_t p, int ratio, int64_t n_c) {
    int64_t v = 0;
    for (int64_t j = 0; j < n_c; ++j)
        if ((j + 1) * (int64_t)ratio <= p + 1) v = j + 1;
    return v;
}

/* The compressed part when every visible row is attended (no indexer):
 * offset + j for the visible rows in ascending order, then -1 up to K. */
void sckvo_visible_idx(int64_t m, int64_t start_pos, int ratio, int64_t n_c, int K, int32_t offset,
                       int32_t* idx, int64_t ld, int64_t col0) {
    for (int64_t t = 0; t < m; ++t) {
        int64_t v = sckvo_visible(start_pos + t, ratio, n_c);
        for (int64_t j = 0; j < K; ++j) idx[t * ld + col0 + j] = (j < v) ? (int32_t)(offset + j) : -1;
    }
}

/* ------------------------------------------------------------------------ */
/* Indexer score  [compress.rs module doc: q and k through the e2m1 round    */
/* trip with power-of-two scales in blocks of 32; scores are bf16 values]    */
/* ------------------------------------------------------------------------ */

/* A bf16 value as an integer significand and a power of two: v = m * 2^e
 * with |m| < 2^8, because bf16 keeps 8 significant bits (v = fr * 2^x with
 * 0.5 <= |fr| < 1 from frexp, so m = fr * 2^8 is an integer and e = x - 8).
 * Zero gives m = 0. */
static void oracle_split_bf16(const uint16_t* a, int64_t n, int* m, int* e) {
    for (int64_t i = 0; i < n; ++i) {
        int x;
        double fr = frexp((double)sckvo_bf16_to_f32(a[i]), &x);
        m[i] = (int)ldexp(fr, 8);
        e[i] = x - 8;
    }
}

/* Exact dot product of two bf16 vectors given as oracle_split_bf16 pairs.
 * The products are summed as integers over their smallest exponent, so the
 * sum is exact.  *exact_f32 is set to 1 when every partial sum of the
 * products, taken in ANY order, is a binary32 value -- then any binary32
 * accumulation (matrix cores included) gives the exact value bit for bit.
 * That holds when all products are integer multiples of 2^g (g = the lowest
 * set bit over all of them), sum |product| < 2^(g+24) (24 significant bits),
 * g >= -149 (the binary32 subnormal quantum) and g + 24 <= 128 (no overflow).
 * Returns the exact sum rounded to binary64. */
static double oracle_exact_dot(const int* ma, const int* ea, const int* mb, const int* eb, int n, int* exact_f32) {
    int e_min = 1 << 30;
    for (int i = 0; i < n; ++i)
        if (ma[i] != 0 && mb[i] != 0 && ea[i] + eb[i] < e_min) e_min = ea[i] + eb[i];
    __int128 acc = 0, sum_abs = 0, bits_or = 0;
    for (int i = 0; i < n; ++i) {
        if (ma[i] == 0 || mb[i] == 0) continue;
        int sh = ea[i] + eb[i] - e_min;
        if (sh > 100) abort(); /* outside what this oracle can sum exactly */
        __int128 p = ((__int128)((int64_t)ma[i] * mb[i])) << sh;
        __int128 ap = p < 0 ? -p : p;
        acc += p;
        sum_abs += ap;
        bits_or |= ap;
    }
    if (bits_or == 0) {
        *exact_f32 = 1;
        return 0.0;
    }
    int g = 0; /* products are multiples of 2^(e_min + g) */
    while (((bits_or >> g) & 1) == 0) ++g;
    int e_low = e_min + g;
    *exact_f32 = ((sum_abs >> g) < ((__int128)1 << 24)) && e_low >= -149 && e_low + 24 <= 128;
    if (acc == 0) return 0.0;
    /* the exact sum acc * 2^e_min, rounded to binary64 (exact when at most 53
     * significant bits, which exactness above implies) */
    while ((acc & 1) == 0) {
        acc /= 2;
        ++e_min;
    }
    __int128 mag = acc < 0 ? -acc : acc;
    if (mag >= ((__int128)1 << 53)) abort(); /* beyond an exact binary64 */
    return ldexp((double)(int64_t)acc, e_min);
}

/* Indexer scores for the queries listed in qsel (reading of the indexer, whose
 * body is not printed; the lightning-indexer form):
 *   q_hat[t,h,:] = the power-of-two fp4 round trip of the raw q row (blocks of
 *                  32 along the head dimension),
 *   d_h          = the exact dot q_hat[t,h,:] . k_hat[s,:], as binary32,
 *   r_h          = fl32(w[t,h] * relu(d_h)), relu(d) = d if d > 0 else +0,
 *   head sum     = pairwise, stride Hi/2, Hi/4, ..., 1: r_h += r_{h+stride},
 *   score        = bf16(r_0).
 * Only the rows visible to the query are scored; scores[i, s] for s at or
 * past the visible count is left as 0xffff.  k_hat is already round-tripped.
 * Returns the number of dot products whose exact value is not a binary32
 * value (the contract assumes none). */
int64_t sckvo_index_scores(const uint16_t* q_raw, const uint16_t* k_hat, const float* w, int64_t m, int Hi, int Di,
                           int64_t n_c, int ratio, int64_t start_pos, const int64_t* qsel, int64_t nsel,
                           uint16_t* scores) {
    int64_t inexact = 0;
    uint16_t* qh = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)Hi * Di);
    int* qm = (int*)malloc(sizeof(int) * (size_t)Hi * Di);
    int* qe = (int*)malloc(sizeof(int) * (size_t)Hi * Di);
    int* km = (int*)malloc(sizeof(int) * (size_t)(n_c > 0 ? n_c : 1) * Di);
    int* ke = (int*)malloc(sizeof(int) * (size_t)(n_c > 0 ? n_c : 1) * Di);
    float* r = (float*)malloc(sizeof(float) * (size_t)Hi);
    oracle_split_bf16(k_hat, n_c * (int64_t)Di, km, ke);
    for (int64_t i = 0; i < nsel; ++i) {
        int64_t t = qsel[i];
        if (t < 0 || t >= m) abort();
        const uint16_t* qrow = q_raw + t * (int64_t)Hi * Di;
        sckvo_quant_e8m0(qrow, qh, (int64_t)Hi * Di, 32);
        oracle_split_bf16(qh, (int64_t)Hi * Di, qm, qe);
        int64_t vis = sckvo_visible(start_pos + t, ratio, n_c);
        for (int64_t s = 0; s < n_c; ++s) {
            if (s >= vis) {
                scores[i * n_c + s] = 0xffff;
                continue;
            }
            for (int h = 0; h < Hi; ++h) {
                int ex = 0;
                double d = oracle_exact_dot(qm + (int64_t)h * Di, qe + (int64_t)h * Di, km + s * (int64_t)Di,
                                            ke + s * (int64_t)Di, Di, &ex);
                if (!ex) ++inexact;
                float df = (float)d;
                float relu = (df > 0.0f) ? df : 0.0f;
                r[h] = w[t * Hi + h] * relu;
            }
            for (int stride = Hi / 2; stride >= 1; stride /= 2)
                for (int h = 0; h < stride; ++h) r[h] = r[h] + r[h + stride];
            scores[i * n_c + s] = sckvo_f32_to_bf16(r[0]);
        }
    }
    free(qm);
    free(qe);
    free(km);
    free(ke);
    free(qh);
    free(r);
    return inexact;
}

/* ------------------------------------------------------------------------ */
/* Top-k  [forward.rs: merge; the tie rule is "toward the lower index"]     */
/* ------------------------------------------------------------------------ */

typedef struct {
    float score;
    int64_t s;
} oracle_cand;

/* Larger score first; equal scores (-0 equals +0) keep the lower row first. */
static int oracle_cand_cmp(const void* pa, const void* pb) {
    const oracle_cand* a = (const oracle_cand*)pa;
    const oracle_cand* b = (const oracle_cand*)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->s < b->s) ? -1 : (a->s > b->s) ? 1 : 0;
}

static int oracle_row_cmp(const void* pa, const void* pb) {
    int64_t a = ((const oracle_cand*)pa)->s, b = ((const oracle_cand*)pb)->s;
    return (a < b) ? -1 : (a > b) ? 1 : 0;
}

/* Select the min(K, visible) rows with the largest scores among rows
 * 0 .. visible-1, ties toward the lower row; write offset + row for them in
 * ascending row order, then -1 up to K.  scores are bf16 bits. */
void sckvo_topk(const uint16_t* scores, int64_t visible, int K, int32_t offset, int32_t* out) {
    oracle_cand* c = (oracle_cand*)malloc(sizeof(oracle_cand) * (size_t)(visible > 0 ? visible : 1));
    for (int64_t s = 0; s < visible; ++s) {
        c[s].score = sckvo_bf16_to_f32(scores[s]);
        c[s].s = s;
    }
    qsort(c, (size_t)visible, sizeof(oracle_cand), oracle_cand_cmp);
    int64_t kt = visible < K ? visible : K;
    qsort(c, (size_t)kt, sizeof(oracle_cand), oracle_row_cmp);
    for (int64_t j = 0; j < K; ++j) out[j] = (j < kt) ? (int32_t)(offset + c[j].s) : -1;
    free(c);
}

/* ------------------------------------------------------------------------ */
/* Sparse MQA attention with a per-head sink  [compress.rs: attention_any,   */
/* sparse_attn call; forward.rs: attend_and_project over rows_a / rows_b]    */
/* ------------------------------------------------------------------------ */

/* For every selected query t and head h (reading of sparse_attn, whose body
 * is not printed): the valid entries are idx[t, i] != -1; entry i names row
 * rows_a[idx] when idx < ra, else rows_b[idx - ra]; the row is both key and
 * value.  l_i = scale * (q[t,h,:] . row_i) in binary64; the softmax runs over
 * {l_i} and the sink logit sink[h], which has no value row:
 *   M = max(sink_h, max_i l_i),  Z = e^(sink_h - M) + sum_i e^(l_i - M),
 *   o = sum_i e^(l_i - M) * row_i / Z.
 * No valid entry gives o = 0.  out is binary64 [nsel, H, D].  Returns -1 when
 * an index is out of range, else 0. */
int sckvo_sparse_attn(const uint16_t* q, const uint16_t* rows_a, int64_t ra, const uint16_t* rows_b, int64_t rb,
                      const int32_t* idx, int T, const float* sink, float scale, int H, int D, const int64_t* qsel,
                      int64_t nsel, double* out) {
    double* l = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    const uint16_t** rp = (const uint16_t**)malloc(sizeof(uint16_t*) * (size_t)(T > 0 ? T : 1));
    int rc = 0;
    for (int64_t i = 0; i < nsel && rc == 0; ++i) {
        int64_t t = qsel[i];
        const int32_t* it = idx + t * (int64_t)T;
        int nv = 0;
        for (int j = 0; j < T; ++j) {
            int32_t x = it[j];
            if (x == -1) continue;
            if (x < 0 || x >= ra + rb) {
                rc = -1;
                break;
            }
            rp[nv++] = (x < ra) ? rows_a + (int64_t)x * D : rows_b + (int64_t)(x - ra) * D;
        }
        if (rc) break;
        for (int h = 0; h < H; ++h) {
            const uint16_t* qv = q + (t * (int64_t)H + h) * D;
            double* o = out + (i * (int64_t)H + h) * D;
            double M = (double)sink[h];
            for (int j = 0; j < nv; ++j) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += (double)sckvo_bf16_to_f32(qv[d]) * (double)sckvo_bf16_to_f32(rp[j][d]);
                l[j] = (double)scale * dot;
                if (l[j] > M) M = l[j];
            }
            double Z = exp((double)sink[h] - M);
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            for (int j = 0; j < nv; ++j) {
                double p = exp(l[j] - M);
                Z += p;
                for (int d = 0; d < D; ++d) o[d] += p * (double)sckvo_bf16_to_f32(rp[j][d]);
            }
            for (int d = 0; d < D; ++d) o[d] /= Z;
        }
    }
    free(l);
    free(rp);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* YaRN RoPE of the compressed latent  [compress.rs: yarn_freqs_cis, and     */
/* attention_any: a new latent group is rotated at its position, then fp4    */
/* round-tripped with e4m3 scales, then copied into the cache; forward.rs:   */
/* the rope call on the latent before fp4_quant and the cache copy]          */
/* ------------------------------------------------------------------------ */

/* The rotation table of the compressed layers for positions 0 .. seqlen-1
 * (compress.rs yarn_freqs_cis), steps in the page's order:
 *   1. pair i (0 <= i < dim/2) has the base frequency 1 / base^(2i/dim), in
 *      binary32 (the exponent 2i/dim is itself a binary32 quotient);
 *   2. in binary64, the correction dimension of a rotation count r is
 *      dim * ln(L / (r * 2 * pi)) / (2 ln base) with L = original_seq_len;
 *      low = max(floor(that of beta_fast), 0), high = min(ceil(that of
 *      beta_slow), dim - 1), both then binary32;
 *   3. ramp_i = clamp((i - low) / max(high - low, 0.001), 0, 1) and the
 *      frequency becomes f/factor * ramp_i + f * (1 - ramp_i), in binary32 in
 *      the page's operation order (f / factor * (1 - smooth) + f * smooth with
 *      smooth = 1 - ramp);
 *   4. entry (p, i) is (cos a, sin a) of the binary32 angle a = p * f_i.
 * out is [seqlen][dim/2][2] binary32.  dim must be even and positive. */
void sckvo_yarn_freqs_cis(int dim, int64_t seqlen, int64_t original_seq_len, float base, float factor,
                          float beta_fast, float beta_slow, float* out) {
    const int half = dim / 2;
    float* f = (float*)malloc(sizeof(float) * (size_t)(half > 0 ? half : 1));
    for (int i = 0; i < half; ++i) f[i] = 1.0f / powf(base, (float)(2 * i) / (float)dim);
    const double two_ln_base = 2.0 * log((double)base);
    const double c_fast = (double)dim * log((double)original_seq_len / ((double)beta_fast * 2.0 * M_PI)) / two_ln_base;
    const double c_slow = (double)dim * log((double)original_seq_len / ((double)beta_slow * 2.0 * M_PI)) / two_ln_base;
    double lo = floor(c_fast);
    if (lo < 0.0) lo = 0.0;
    double hi = ceil(c_slow);
    if (hi > (double)(dim - 1)) hi = (double)(dim - 1);
    const float low = (float)lo, high = (float)hi;
    float span = high - low;
    if (span < 1e-3f) span = 1e-3f;
    for (int i = 0; i < half; ++i) {
        float ramp = ((float)i - low) / span;
        if (ramp < 0.0f) ramp = 0.0f;
        if (ramp > 1.0f) ramp = 1.0f;
        const float smooth = 1.0f - ramp;
        f[i] = f[i] / factor * (1.0f - smooth) + f[i] * smooth;
    }
    for (int64_t p = 0; p < seqlen; ++p)
        for (int i = 0; i < half; ++i) {
            const float a = (float)p * f[i];
            out[(p * half + i) * 2 + 0] = cosf(a);
            out[(p * half + i) * 2 + 1] = sinf(a);
        }
    free(f);
}

/* Position of compressed row j of a layer with `ratio` positions a row: the
 * first position of its group, j * ratio.  This is the page's g * ratio for
 * the groups of a prefill from position 0 and its start_pos + 1 - ratio for
 * the one group a decode step completes (j = (start_pos + 1) / ratio - 1);
 * for a chunk at start_pos > 0 (an extension) the same rule names each new
 * row's group. */
int64_t sckvo_latent_position(int64_t j, int ratio) { return j * (int64_t)ratio; }

/* Rotary embedding of bf16 rows (compress.rs and forward.rs name apply_rotary
 * / rope without printing them; the reading used here): the last rope_dim
 * values of each row of `cols` are rope_dim/2 pairs (2i, 2i+1) of the rope
 * slice, pair i a complex number x0 + i x1 turned by the table angle (p, i)
 * of the row's position p:
 *   forward  y0 = x0 c - x1 s,  y1 = x0 s + x1 c
 *   inverse  y0 = x0 c + x1 s,  y1 = x1 c - x0 s
 * every product and sum one binary32 operation (no fused multiply-add), the
 * result rounded to bf16 (the latent buffer the rotation writes holds bf16);
 * the other values are copied.  table is [n_pos][rope_dim/2][2] (cos, sin);
 * pos[r] is row r's position.  Returns -1 when a position is outside the
 * table, else 0. */
int sckvo_rope_rows(const uint16_t* x, int64_t rows, int cols, int rope_dim, const float* table, int64_t n_pos,
                    const int64_t* pos, int inverse, uint16_t* y) {
    const int half = rope_dim / 2;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t p = pos[r];
        if (p < 0 || p >= n_pos) return -1;
        const uint16_t* xr = x + r * cols;
        uint16_t* yr = y + r * cols;
        for (int c = 0; c < cols; ++c) yr[c] = xr[c];
        for (int i = 0; i < half; ++i) {
            const int j = cols - rope_dim + 2 * i;
            const float x0 = sckvo_bf16_to_f32(xr[j]), x1 = sckvo_bf16_to_f32(xr[j + 1]);
            const float c = table[(p * half + i) * 2 + 0], s = table[(p * half + i) * 2 + 1];
            float y0, y1;
            if (!inverse) {
                y0 = x0 * c - x1 * s;
                y1 = x0 * s + x1 * c;
            } else {
                y0 = x0 * c + x1 * s;
                y1 = x1 * c - x0 * s;
            }
            yr[j] = sckvo_f32_to_bf16(y0);
            yr[j + 1] = sckvo_f32_to_bf16(y1);
        }
    }
    return 0;
}

// indexer.hip -- indexer scores of every query against its visible compressed
// rows (MFMA contraction, fused q round trip, fixed pairwise head sum) and the
// per-query top-K (bitwise threshold search over keys held in registers, then
// an ordered compaction).
//
// Pages: "metrale_model_arch/deepseek_v41_ref/compress.rs" (module doc: q and
// k through the e2m1 round trip with power-of-two scales in blocks of 32,
// scores are bf16 values) and "metrale_model_arch/attn_v41/forward.rs" (the
// indexer call with offset = rows_a's length, compress_len, the merge of the
// window and compressed lists).  The head combination is the lightning-indexer
// reading: score = bf16(pairwise sum over h of fl32(w[t,h] * relu(q_hat.k))).
//
// Score kernel.  One workgroup (4 waves) = one query x a range of compressed
// rows; each wave takes a contiguous run of that range in 32-row tiles.  The
// workgroup first round-trips the raw q into LDS (one 32-value block per
// thread), then every wave holds q_hat in registers in MFMA A layout: heads are
// the M dimension (32 or 64), rows the N dimension, the indexer head dim the
// K dimension.  k tiles stream HBM -> LDS through a wave-private ring of
// asynchronous copies (global_load_lds_dwordx4, 1 KiB per instruction,
// 16-byte chunks swizzled by row so the B-operand reads hit every bank).  All
// products are exact and, for round-tripped data, every partial sum is a
// binary32 value, so the MFMA accumulation order does not matter.  The head
// sum follows the fixed pairwise order (stride Hi/2 first): in the D tile
// layout strides 32, 16, 8, 2 and 1 stay inside a lane and stride 4 is the
// lane^32 exchange.  Ordered 16-bit keys collect in LDS and leave with
// coalesced stores.
#include "mfma.h"
#include "sckv_device.h"

namespace sckv {
namespace {

constexpr int SCORE_WAVES = 4;
constexpr int TOPK_THREADS = 512;

// Ordered 16-bit key of a bf16 score: -0 counts as +0; a larger key is a
// larger score.
__device__ __forceinline__ uint32_t score_key(uint32_t b) {
    if (b == 0x8000u) b = 0u;
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}

// Shape of one score workgroup for MT head tiles and head dim DI.
template <int MT, int DI>
struct ScoreShape {
    static constexpr int HP = MT * 32;                 // padded heads
    static constexpr int KS = DI / 16;                 // k-steps
    static constexpr int ROWB = DI * 2;                // bytes per k row
    static constexpr int TILE = 32 * ROWB;             // bytes per 32-row tile
    static constexpr int NINST = TILE / 1024;          // 16-byte-per-lane copies per tile
    static constexpr int NST = (TILE >= 16384) ? 1 : 4;  // tiles per wave in the ring
    static constexpr int PD = NST - 1;                   // tiles requested ahead of the one used
    static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
    static constexpr int SWZ = (CPR < 8 ? CPR : 8) - 1;  // chunk swizzle mask
    static constexpr int QS = DI * 2 + 16;             // bytes per q_hat row in LDS (padded)
    static constexpr int OFF_Q = SCORE_WAVES * NST * TILE;
    static constexpr int OFF_KEYS = OFF_Q + HP * QS;
    static constexpr size_t lds_bytes(int rows_per_wg, bool with_scores) {
        return (size_t)OFF_KEYS + (size_t)rows_per_wg * 2 * (with_scores ? 2 : 1);
    }
    static_assert(NINST >= 1 && NINST * PD < 64 && PD <= 3, "copy counts");
};

template <int NINST, int NAHEAD>
__device__ __forceinline__ void wait_tiles(int ahead) {
    // at most `ahead` later tiles (NINST copies each) may still be in flight
    if (ahead <= 0)
        wait_vmcnt<0>();
    else if (ahead == 1 || NAHEAD < 2)
        wait_vmcnt<NINST>();
    else
        wait_vmcnt<(2 * NINST < 64 ? 2 * NINST : 63)>();
}

template <int MT, int DI>
__global__ __launch_bounds__(SCORE_WAVES * 64) void index_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w, int64_t m, int Hi,
    int64_t n_c, int ratio, int64_t start_pos, int rows_per_wg, int nsplit, uint16_t* __restrict__ keys,
    uint16_t* __restrict__ scores) {
    using S = ScoreShape<MT, DI>;
    constexpr int KS = S::KS;
    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* qh_l = lds + S::OFF_Q;
    uint16_t* keys_l = reinterpret_cast<uint16_t*>(lds + S::OFF_KEYS);
    uint16_t* sc_l = keys_l + rows_per_wg;
    const uint32_t lds0 = lds_offset(lds);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t qi = blockIdx.x / nsplit;
    const int split = (int)(blockIdx.x - qi * nsplit);
    const int64_t b = qi / m;
    const int64_t t = qi - b * m;

    int64_t vis = (start_pos + t + 1) / ratio;
    vis = vis < n_c ? vis : n_c;
    const int64_t row0 = (int64_t)split * rows_per_wg;
    if (row0 >= vis) return;
    int64_t row_end = row0 + rows_per_wg;
    row_end = row_end < vis ? row_end : vis;

    // ---- q_hat = E8M0_B32 round trip of the raw q, one 32-value block per thread and step, into LDS
    const uint16_t* qrow = q + qi * (int64_t)Hi * DI;
    for (int blk = threadIdx.x; blk < S::HP * (DI / 32); blk += SCORE_WAVES * 64) {
        const int h = blk / (DI / 32);
        const int c = blk - h * (DI / 32);
        u32x4 raw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = (h < Hi) ? load16(qrow + (int64_t)h * DI + c * 32 + i * 8) : u32x4{0, 0, 0, 0};
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[i][e] & 0xffffu)));
                amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[i][e] >> 16)));
            }
        const float s = block_scale<SCKV_FP4_E8M0_B32>(amax);
        const float inv_s = pow2_reciprocal(s);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t v = raw[i][e];
                raw[i][e] = fp4_value_bits_pow2(bf16_bits_to_f32(v & 0xffffu), s, inv_s) |
                            (fp4_value_bits_pow2(bf16_bits_to_f32(v >> 16), s, inv_s) << 16);
            }
            *reinterpret_cast<u32x4*>(qh_l + h * S::QS + (c * 32 + i * 8) * 2) = raw[i];
        }
    }
    // ---- head weights in D layout: head mt*32 + d_row(i, lane)
    float wd[MT][16];
    const float* wrow = w + qi * (int64_t)Hi;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = mt * 32 + d_row(i, lane);
            wd[mt][i] = (h < Hi) ? wrow[h] : 0.0f;
        }
    // every ordinary load is done before the first tile copy is issued
    wait_vmcnt<0>();
    __syncthreads();
    bf16x8 qa[MT][KS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qa[mt][ks] = *reinterpret_cast<const bf16x8*>(qh_l + (mt * 32 + (lane & 31)) * S::QS +
                                                          (ks * 16 + (lane >> 5) * 8) * 2);

    // ---- this wave's rows: a contiguous run, streamed in 32-row tiles through
    // a wave-private ring; lane i of copy j brings 16 bytes of tile byte j*1024 +
    // 16 i, taken from chunk (chunk ^ (row & SWZ)) of its row so that the B-operand
    // reads below (32 rows at one chunk) spread over all banks.
    const int64_t nrows = row_end - row0;
    const int64_t per_wave = (((nrows + SCORE_WAVES - 1) / SCORE_WAVES) + 31) / 32 * 32;
    const int64_t w0 = row0 + (int64_t)wave * per_wave;
    int64_t w1 = w0 + per_wave;
    w1 = w1 < row_end ? w1 : row_end;
    const int ntiles = (w0 < w1) ? (int)((w1 - w0 + 31) / 32) : 0;
    const uint16_t* kb = k + b * n_c * DI;
    const uint32_t ring = lds0 + (uint32_t)(wave * S::NST * S::TILE);
    auto issue = [&](int tile) {
        const int64_t s0 = w0 + (int64_t)tile * 32;
        const uint32_t st = ring + (uint32_t)((tile % S::NST) * S::TILE);
#pragma unroll
        for (int j = 0; j < S::NINST; ++j) {
            const int byte = j * 1024 + lane * 16;
            const int r = byte / S::ROWB;
            const int ch = (byte % S::ROWB) / 16;
            int64_t row = s0 + r;
            row = row < n_c ? row : n_c - 1;  // tail rows re-read a real row; their results are dropped
            const uint32_t off = (uint32_t)(row * S::ROWB + ((ch ^ (r & S::SWZ)) * 16));
            dma16_s(kb, off, st + (uint32_t)(j * 1024));
        }
    };
#pragma unroll
    for (int i = 0; i < S::PD; ++i)
        if (i < ntiles) issue(i);

    for (int tile = 0; tile < ntiles; ++tile) {
        if (S::PD == 0) issue(tile);
        // tiles tile+1 .. tile+PD-1 may still be in flight; tile itself must be done
        const int ahead = (ntiles - 1 - tile) < (S::PD - 1) ? (ntiles - 1 - tile) : (S::PD - 1);
        wait_tiles<S::NINST, S::PD - 1>(ahead);
        if (S::PD > 0 && tile + S::PD < ntiles) issue(tile + S::PD);  // into the stage tile-1 used
        const unsigned char* stp = lds + (wave * S::NST + tile % S::NST) * S::TILE;
        const int r = lane & 31;
        f32x16 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = zero16();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int ch = ks * 2 + (lane >> 5);
            const bf16x8 kr = *reinterpret_cast<const bf16x8*>(stp + r * S::ROWB + ((ch ^ (r & S::SWZ)) * 16));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma32x32x16(qa[mt][ks], kr, acc[mt]);
        }
        // r_h = fl32(w_h * relu(d_h)); relu maps every d <= 0 (and -0) to +0
        float v[MT * 16];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float d = acc[mt][i];
                v[mt * 16 + i] = wd[mt][i] * ((d > 0.0f) ? d : 0.0f);
            }
        // pairwise head sum, stride Hi/2 first (h and h + stride)
        if (MT == 2 && Hi > 32) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = v[i] + v[16 + i];
        }
        if (Hi > 16) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = v[i] + v[i + 8];
        }
        if (Hi > 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = v[i] + v[i + 4];
        }
        if (Hi > 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = v[i] + shfl_xor32(v[i]);
        }
        if (Hi > 2) {
            v[0] = v[0] + v[2];
            v[1] = v[1] + v[3];
        }
        if (Hi > 1) v[0] = v[0] + v[1];
        const int64_t s = w0 + (int64_t)tile * 32 + r;
        if (lane < 32 && s < w1) {
            const uint32_t bits = f32_to_bf16_bits(v[0]);
            keys_l[s - row0] = (uint16_t)score_key(bits);
            if (scores) sc_l[s - row0] = (uint16_t)bits;
        }
    }
    // ---- flush this workgroup's keys (and scores) with coalesced stores
    __syncthreads();
    uint16_t* kout = keys + qi * n_c + row0;
    for (int64_t i = threadIdx.x; i < nrows; i += SCORE_WAVES * 64) kout[i] = keys_l[i];
    if (scores) {
        uint16_t* sout = scores + qi * n_c + row0;
        for (int64_t i = threadIdx.x; i < nrows; i += SCORE_WAVES * 64) sout[i] = sc_l[i];
    }
}

// ---- top-k: one block per query, keys held in registers
//
// Thread t owns the KPT consecutive rows [t*KPT, t*KPT + KPT).  The K-th
// largest key tau is built bit by bit (16 rounds: keep bit b when at least K
// keys are >= the candidate), counting in registers and summing over the
// block; then the rows with key > tau and the first (K - #greater) rows with
// key == tau (lowest rows first) are written in ascending row order with two
// block prefix sums.  No atomics; missing rows hold key 0, below every real
// key (finite scores have keys >= 0x007f).

constexpr int TOPK_WAVES = TOPK_THREADS / 64;

// DPP helpers (no LDS round trip).  update_dpp(old, src, ctrl, row_mask,
// bank_mask, bound_ctrl): lanes outside row_mask keep `old`.
#define SCKV_DPP(v, ctrl, rmask, bc) \
    ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v), (ctrl), (rmask), 0xf, (bc)))

// Sum of x over the wave (uniform result): butterfly inside each 16-lane row,
// then the four row sums through readlane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
    x += SCKV_DPP(x, 0xb1, 0xf, false);   // quad_perm [1,0,3,2]
    x += SCKV_DPP(x, 0x4e, 0xf, false);   // quad_perm [2,3,0,1]
    x += SCKV_DPP(x, 0x141, 0xf, false);  // row_half_mirror
    x += SCKV_DPP(x, 0x140, 0xf, false);  // row_mirror
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 0) + (uint32_t)__builtin_amdgcn_readlane((int)x, 16) +
           (uint32_t)__builtin_amdgcn_readlane((int)x, 32) + (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
}

// Inclusive prefix sum over the wave's lanes: shifts inside 16-lane rows, then
// row 15 / lane 31 broadcasts into the later rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += SCKV_DPP(x, 0x111, 0xf, true);  // row_shr:1
    x += SCKV_DPP(x, 0x112, 0xf, true);  // row_shr:2
    x += SCKV_DPP(x, 0x114, 0xf, true);  // row_shr:4
    x += SCKV_DPP(x, 0x118, 0xf, true);  // row_shr:8
    x += SCKV_DPP(x, 0x142, 0xa, false);  // row_bcast15 into rows 1 and 3
    x += SCKV_DPP(x, 0x143, 0xc, false);  // row_bcast31 into rows 2 and 3
    return x;
}

// Sum over the block; buf holds TOPK_WAVES words and must not be reused by the
// very next call (callers alternate two buffers).
__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t* buf) {
    const uint32_t w = wave_sum(x);
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = w;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < TOPK_WAVES; ++i) t += buf[i];
    return t;
}

// Exclusive prefix sum over the block's threads.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* tot) {
    const uint32_t incl = wave_incl_scan(x);
    if ((threadIdx.x & 63) == 63) tot[threadIdx.x >> 6] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < (int)(threadIdx.x >> 6); ++i) before += tot[i];
    __syncthreads();
    return before + incl - x;
}

template <int KPT>
__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(const uint16_t* __restrict__ keys, int64_t n_c,
                                                            int64_t m, int ratio, int64_t start_pos, int K,
                                                            int32_t offset, int32_t* __restrict__ idx, int64_t ld,
                                                            int64_t col0) {
    __shared__ uint32_t red[2][TOPK_WAVES];
    __shared__ uint32_t tot[TOPK_WAVES];
    const int tid = threadIdx.x;
    const int64_t qi = blockIdx.x;
    const int64_t t = qi % m;
    int64_t vis = (start_pos + t + 1) / ratio;
    vis = vis < n_c ? vis : n_c;
    int32_t* out = idx + qi * ld + col0;
    if (vis <= K) {
        for (int j = tid; j < K; j += TOPK_THREADS) out[j] = (j < vis) ? (int32_t)(offset + j) : -1;
        return;
    }
    const uint16_t* kp = keys + qi * n_c;
    const int64_t s0 = (int64_t)tid * KPT;
    uint32_t key[KPT];
    if (KPT % 8 == 0 && (n_c % 8) == 0) {
        // whole 16-byte groups of 8 keys; groups past n_c are not read
#pragma unroll
        for (int j8 = 0; j8 < KPT / 8; ++j8) {
            const int64_t g0 = s0 + 8 * j8;
            const u32x4 v = (g0 + 8 <= n_c) ? load16(kp + g0) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                key[8 * j8 + 2 * e] = v[e] & 0xffffu;
                key[8 * j8 + 2 * e + 1] = v[e] >> 16;
            }
        }
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = (s0 + j < vis) ? key[j] : 0u;
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = (s0 + j < vis) ? (uint32_t)kp[s0 + j] : 0u;
    }

    uint32_t tau = 0;
    int rb = 0;
#pragma unroll 1
    for (int bit = 15; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += key[j] >= cand;
        const uint32_t total = block_sum(c, red[rb]);
        rb ^= 1;
        if (total >= (uint32_t)K) tau = cand;
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        gt += key[j] > tau;
        eq += key[j] == tau;
    }
    const uint32_t gt_total = block_sum(gt, red[rb]);
    const uint32_t need_eq = (uint32_t)K - gt_total;  // >= 1 by the choice of tau
    const uint32_t eq_before = block_excl_scan(eq, tot);
    uint32_t take_eq = (need_eq > eq_before) ? (need_eq - eq_before) : 0u;
    take_eq = take_eq < eq ? take_eq : eq;
    uint32_t pos = block_excl_scan(gt + take_eq, tot);
    uint32_t eq_seen = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const uint32_t k = key[j];
        bool take = k > tau;
        if (k == tau) {
            take = eq_seen < take_eq;
            ++eq_seen;
        }
        if (take && pos < (uint32_t)K) out[pos++] = (int32_t)(offset + s0 + j);
    }
}

void launch_topk(const uint16_t* keys, int64_t nq, int64_t n_c, int64_t m, int ratio, int64_t start_pos, int K,
                 int32_t offset, int32_t* idx, int64_t ld, int64_t col0, hipStream_t s) {
    const int64_t kpt = (n_c + TOPK_THREADS - 1) / TOPK_THREADS;
#define SCKV_TOPK(KPT)                                                                                        \
    topk_kernel<KPT><<<dim3((unsigned)nq), dim3(TOPK_THREADS), 0, s>>>(keys, n_c, m, ratio, start_pos, K, offset, \
                                                                        idx, ld, col0)
    if (kpt <= 2)
        SCKV_TOPK(2);
    else if (kpt <= 8)
        SCKV_TOPK(8);
    else if (kpt <= 32)
        SCKV_TOPK(32);
    else if (kpt <= 64)
        SCKV_TOPK(64);
    else
        SCKV_TOPK(128);
#undef SCKV_TOPK
}

template <int MT, int DI>
int launch_scores(const uint16_t* q, const uint16_t* k, const float* w, int64_t nq, int64_t m, int Hi, int64_t n_c,
                  int ratio, int64_t start_pos, int rows_per_wg, int nsplit, uint16_t* keys, uint16_t* scores,
                  hipStream_t stream) {
    using Sh = ScoreShape<MT, DI>;
    const size_t lds = Sh::lds_bytes(rows_per_wg, scores != nullptr);
    if (lds > 160 * 1024) return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: score tile does not fit in LDS");
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)index_score_kernel<MT, DI>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return fail(SCKV_EHIP, std::string("sckv_index_scores_topk: ") + hipGetErrorString(e));
    }
    index_score_kernel<MT, DI><<<dim3((unsigned)(nq * nsplit)), dim3(SCORE_WAVES * 64), lds, stream>>>(
        q, k, w, m, Hi, n_c, ratio, start_pos, rows_per_wg, nsplit, keys, scores);
    return SCKV_OK;
}

// Rows per workgroup: a multiple of 128 (4 waves x 32 rows), at most 2048
// (the keys are buffered in LDS), and small enough that the launch has about
// 512 workgroups when the queries alone do not.
int score_rows_per_wg(int64_t nq, int64_t n_c) {
    int64_t tiles = (n_c + 127) / 128;  // 128-row tiles of one query
    int64_t want_splits = (512 + nq - 1) / nq;
    if (want_splits > tiles) want_splits = tiles;
    if (want_splits < 1) want_splits = 1;
    int64_t tiles_per = (tiles + want_splits - 1) / want_splits;
    if (tiles_per > 16) tiles_per = 16;
    return (int)(tiles_per * 128);
}

}  // namespace

size_t index_workspace_bytes(int B, int64_t m, int64_t n_c) {
    // one 16-bit key per (query, compressed row), 256-byte aligned
    const size_t bytes = (size_t)B * (size_t)m * (size_t)n_c * 2u;
    return (bytes + 255u) & ~(size_t)255u;
}

}  // namespace sckv

extern "C" int sckv_index_scores_topk(const void* q, const void* k, const float* w, int B, int64_t m, int Hi, int Di,
                                      int64_t n_c, int ratio, int64_t start_pos, int K, int32_t offset,
                                      int32_t* idx, int64_t ld, int64_t col0, void* scores, void* ws,
                                      size_t ws_bytes, void* stream) {
    using namespace sckv;
    if (B < 0 || m < 0 || n_c < 0 || ratio <= 0 || start_pos < 0 || K < 0 || col0 < 0 || offset < 0)
        return fail(SCKV_EINVAL, "sckv_index_scores_topk: bad sizes");
    if (Hi <= 0 || (Hi & (Hi - 1)) != 0) return fail(SCKV_EINVAL, "sckv_index_scores_topk: Hi must be a power of two");
    if (Hi > 64) return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: Hi > 64");
    if (Di != 32 && Di != 64 && Di != 128 && Di != 256)
        return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: Di not in {32, 64, 128, 256}");
    if (B == 0 || m == 0 || K == 0) return SCKV_OK;
    if (!idx) return fail(SCKV_EINVAL, "sckv_index_scores_topk: null idx");
    if (ld < col0 + K) return fail(SCKV_EINVAL, "sckv_index_scores_topk: ld < col0 + K");
    if (n_c > 65536 || (int64_t)offset + n_c > 0x7fffffffLL)
        return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: n_c > 65536 or offset + n_c >= 2^31");
    const int64_t nq = (int64_t)B * m;
    hipStream_t s = (hipStream_t)stream;
    // no compressed row is visible to any query: every list is K x -1 (the pages' empty selection)
    int64_t vmax = (start_pos + m) / ratio;
    vmax = vmax < n_c ? vmax : n_c;
    if (vmax == 0) {
        launch_topk(nullptr, nq, 0, m, ratio, start_pos, K, offset, idx, ld, col0, s);
        return check_launch("sckv_index_scores_topk");
    }
    if (!q || !k || !w) return fail(SCKV_EINVAL, "sckv_index_scores_topk: null input");
    if ((uintptr_t)q % 16 || (uintptr_t)k % 16)
        return fail(SCKV_EINVAL, "sckv_index_scores_topk: q and k must be 16-byte aligned");
    if ((uintptr_t)w % 4 || (uintptr_t)idx % 4) return fail(SCKV_EINVAL, "sckv_index_scores_topk: misaligned w/idx");
    if (scores && (uintptr_t)scores % 2) return fail(SCKV_EINVAL, "sckv_index_scores_topk: misaligned scores");
    const size_t need = index_workspace_bytes(B, m, n_c);
    if (!ws || ws_bytes < need) return fail(SCKV_EWORKSPACE, "sckv_index_scores_topk: workspace too small");
    if (nq > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: too many queries");
    const int rpw = score_rows_per_wg(nq, n_c);
    const int nsplit = (int)((n_c + rpw - 1) / rpw);
    if (nq * nsplit > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: grid too large");
    uint16_t* keys = (uint16_t*)ws;
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    uint16_t* sc = (uint16_t*)scores;
    const bool two = Hi > 32;
#define SCKV_SCORES(MT, DI) launch_scores<MT, DI>(qq, kk, w, nq, m, Hi, n_c, ratio, start_pos, rpw, nsplit, keys, sc, s)
    int rc;
    switch (Di) {
        case 32: rc = two ? SCKV_SCORES(2, 32) : SCKV_SCORES(1, 32); break;
        case 64: rc = two ? SCKV_SCORES(2, 64) : SCKV_SCORES(1, 64); break;
        case 128: rc = two ? SCKV_SCORES(2, 128) : SCKV_SCORES(1, 128); break;
        default: rc = two ? SCKV_SCORES(2, 256) : SCKV_SCORES(1, 256); break;
    }
#undef SCKV_SCORES
    if (rc) return rc;
    rc = check_launch("sckv_index_scores_topk (scores)");
    if (rc) return rc;
    launch_topk(keys, nq, n_c, m, ratio, start_pos, K, offset, idx, ld, col0, s);
    return check_launch("sckv_index_scores_topk (top-k)");
}

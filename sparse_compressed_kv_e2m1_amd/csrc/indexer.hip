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
// raw q rows and head weights arrive in LDS by asynchronous copies with the
// first k tiles requested right behind them; the workgroup round-trips q in
// place (one 32-value block per thread) while those tiles are in flight, then
// every wave holds q_hat in registers in MFMA A layout: heads are
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
constexpr int FUSED_MIN_QUERIES = 192;  // fused scores + top-K from this many queries on

// Ordered 16-bit key of a bf16 score: -0 counts as +0; a larger key is a
// larger score.
__device__ __forceinline__ uint32_t score_key(uint32_t b) {
    if (b == 0x8000u) b = 0u;
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
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

// Sum over the block of NWAVES waves; buf holds NWAVES words and must not be
// reused by the very next call (callers alternate two buffers).
template <int NWAVES>
__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t* buf) {
    const uint32_t w = wave_sum(x);
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = w;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) t += buf[i];
    return t;
}

// Exclusive prefix sum over the block's threads (tot: NWAVES words).
template <int NWAVES>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* tot) {
    const uint32_t incl = wave_incl_scan(x);
    if ((threadIdx.x & 63) == 63) tot[threadIdx.x >> 6] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < (int)(threadIdx.x >> 6); ++i) before += tot[i];
    __syncthreads();
    return before + incl - x;
}

// Top-K of the keys held by the block: thread t owns key[0..KPT) of rows
// s0 .. s0+KPT-1 (rows at or past the visible count hold key 0).  Writes
// offset + s of the K selected rows in ascending s to out[0..K).  Needs
// V > K visible rows (so tau ends up >= 1 and every missing key is below it).
template <int KPT, int NWAVES>
__device__ __forceinline__ void topk_select(const uint32_t (&key)[KPT], int64_t s0, int K, int32_t offset,
                                            int32_t* __restrict__ out, uint32_t (*red)[NWAVES], uint32_t* tot) {
    uint32_t tau = 0;
    int rb = 0;
#pragma unroll 1
    for (int bit = 15; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += key[j] >= cand;
        const uint32_t total = block_sum<NWAVES>(c, red[rb]);
        rb ^= 1;
        if (total >= (uint32_t)K) tau = cand;
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        gt += key[j] > tau;
        eq += key[j] == tau;
    }
    const uint32_t gt_total = block_sum<NWAVES>(gt, red[rb]);
    const uint32_t need_eq = (uint32_t)K - gt_total;  // >= 1 by the choice of tau
    const uint32_t eq_before = block_excl_scan<NWAVES>(eq, tot);
    uint32_t take_eq = (need_eq > eq_before) ? (need_eq - eq_before) : 0u;
    take_eq = take_eq < eq ? take_eq : eq;
    uint32_t pos = block_excl_scan<NWAVES>(gt + take_eq, tot);
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

// Shape of one score workgroup for MT head tiles and head dim DI; NST_ > 0
// sets the ring depth (tiles per wave) instead of the default.
template <int MT, int DI, int NST_ = 0>
struct ScoreShape {
    static constexpr int HP = MT * 32;                 // padded heads
    static constexpr int KS = DI / 16;                 // k-steps
    static constexpr int ROWB = DI * 2;                // bytes per k row
    static constexpr int TILE = 32 * ROWB;             // bytes per 32-row tile
    static constexpr int NINST = TILE / 1024;          // 16-byte-per-lane copies per tile
    static constexpr int NST = NST_ > 0 ? NST_ : ((TILE >= 16384) ? 1 : 4);  // tiles per wave in the ring
    static constexpr int PD = NST - 1;                   // tiles requested ahead of the one used
    static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
    static constexpr int SWZ = (CPR < 8 ? CPR : 8) - 1;  // chunk swizzle mask
    static constexpr int QS = DI * 2;                  // bytes per q row in LDS (raw, then q_hat in place)
    static constexpr int OFF_Q = SCORE_WAVES * NST * TILE;
    static constexpr int OFF_W = OFF_Q + HP * QS;      // 64 f32 head weights
    // keys (then scores) reuse the q / w space once q_hat and the weights sit
    // in registers
    static constexpr int OFF_KEYS = OFF_Q;
    static constexpr size_t lds_bytes(int rows_per_wg, bool with_scores) {
        const size_t qw = (size_t)HP * QS + 64 * 4;
        const size_t ks = (size_t)rows_per_wg * 2 * (with_scores ? 2 : 1);
        return (size_t)OFF_Q + (qw > ks ? qw : ks);
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

// Ring depth of the fused kernel: the keys of a whole query share the LDS
// with the ring (KPT keys per thread, 256 threads).
constexpr int fused_ring_depth(int DI, int KPT) {
    return (64 * DI >= 16384) ? 1 : (KPT >= 128 ? 2 : 4);
}

// KPT == 0: scores of a row range, ordered keys flushed to `keys` for the
// top-k kernel.  KPT > 0 (fused, one workgroup per query, no split): the
// whole query's keys stay in LDS and the workgroup selects its top-K itself.
template <int MT, int DI, int KPT>
__global__ __launch_bounds__(SCORE_WAVES * 64) void index_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ w, int64_t m, int Hi,
    int64_t n_c, int ratio, int64_t start_pos, int rows_per_wg, int nsplit, uint16_t* __restrict__ keys,
    uint16_t* __restrict__ scores, int K, int32_t offset, int32_t* __restrict__ idx, int64_t ld, int64_t col0) {
    using S = ScoreShape<MT, DI, KPT == 0 ? 0 : fused_ring_depth(DI, KPT)>;
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
    if (KPT > 0 && vis <= K) {
        // every visible row is selected: no scores needed
        int32_t* out = idx + qi * ld + col0;
        for (int j = threadIdx.x; j < K; j += SCORE_WAVES * 64) out[j] = (j < vis) ? (int32_t)(offset + j) : -1;
        return;
    }
    // (the split path leaves such queries to the top-k kernel; it still writes
    // their scores when asked for)
    if (KPT == 0 && !scores && vis <= K) return;
    const int64_t row0 = (int64_t)split * rows_per_wg;
    if (row0 >= vis) return;
    int64_t row_end = row0 + rows_per_wg;
    row_end = row_end < vis ? row_end : vis;

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
    // ---- prologue.  The raw q rows and the head weights come in by asynchronous
    // copies, this wave's first k tiles are requested right behind them, and the
    // q round trip runs while those tiles are in flight.  No ordinary global
    // load is issued in this kernel, so every vmcnt wait below is explicit.
    const int qbytes = Hi * DI * 2;
    const uint16_t* qrow = q + qi * (int64_t)Hi * DI;
    for (int j = wave; j * 1024 < qbytes; j += SCORE_WAVES)
        if (j * 1024 + lane * 16 < qbytes) dma16_s(qrow, (uint32_t)(j * 1024 + lane * 16), lds0 + S::OFF_Q + j * 1024);
    if (wave == 0 && lane < Hi) dma4_s(w + qi * (int64_t)Hi, (uint32_t)lane * 4u, lds0 + S::OFF_W);
#pragma unroll
    for (int i = 0; i < S::PD; ++i)
        if (i < ntiles) issue(i);
    // q and w landed (only the tile copies may still be in flight), in every wave
    if (ntiles >= S::PD)
        wait_vmcnt<S::PD * S::NINST>();
    else
        wait_vmcnt<0>();
    __syncthreads();
    // q_hat = E8M0_B32 round trip of q, one 32-value block per thread and step,
    // in place; padded heads (h >= Hi) become zero rows
    for (int blk = threadIdx.x; blk < S::HP * (DI / 32); blk += SCORE_WAVES * 64) {
        const int h = blk / (DI / 32);
        const int c = blk - h * (DI / 32);
        u32x4* qb = reinterpret_cast<u32x4*>(qh_l + h * S::QS + c * 64);
        u32x4 raw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = (h < Hi) ? qb[i] : u32x4{0, 0, 0, 0};
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[i][e] & 0xffffu)));
                amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[i][e] >> 16)));
            }
        const float sc = block_scale<SCKV_FP4_E8M0_B32>(amax);
        const float inv_s = pow2_reciprocal(sc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t v = raw[i][e];
                raw[i][e] = fp4_value_bits_pow2(bf16_bits_to_f32(v & 0xffffu), sc, inv_s) |
                            (fp4_value_bits_pow2(bf16_bits_to_f32(v >> 16), sc, inv_s) << 16);
            }
            qb[i] = raw[i];
        }
    }
    __syncthreads();
    bf16x8 qa[MT][KS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qa[mt][ks] = *reinterpret_cast<const bf16x8*>(qh_l + (mt * 32 + (lane & 31)) * S::QS +
                                                          (ks * 16 + (lane >> 5) * 8) * 2);
    // head weights in D layout: head mt*32 + d_row(i, lane)
    const float* w_l = reinterpret_cast<const float*>(lds + S::OFF_W);
    float wd[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = mt * 32 + d_row(i, lane);
            wd[mt][i] = (h < Hi) ? w_l[h] : 0.0f;
        }
    __syncthreads();  // every wave holds q_hat and w before keys overwrite them


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
    __syncthreads();
    if (KPT == 0) {
        // ---- flush this workgroup's keys (and scores) with coalesced stores
        uint16_t* kout = keys + qi * n_c + row0;
        for (int64_t i = threadIdx.x; i < nrows; i += SCORE_WAVES * 64) kout[i] = keys_l[i];
        if (scores) {
            uint16_t* sout = scores + qi * n_c + row0;
            for (int64_t i = threadIdx.x; i < nrows; i += SCORE_WAVES * 64) sout[i] = sc_l[i];
        }
    } else {
        // ---- fused top-K over the query's keys in LDS (row0 == 0, nrows == vis > K)
        constexpr int KP = KPT > 0 ? KPT : 8;
        __shared__ uint32_t red[2][SCORE_WAVES];
        __shared__ uint32_t tot[SCORE_WAVES];
        const int64_t s0 = (int64_t)threadIdx.x * KP;
        uint32_t key[KP];
#pragma unroll
        for (int j8 = 0; j8 < KP / 8; ++j8) {
            const u32x4 v = (s0 + 8 * j8 + 8 <= rows_per_wg) ? *reinterpret_cast<const u32x4*>(keys_l + s0 + 8 * j8)
                                                              : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                key[8 * j8 + 2 * e] = v[e] & 0xffffu;
                key[8 * j8 + 2 * e + 1] = v[e] >> 16;
            }
        }
#pragma unroll
        for (int j = 0; j < KP; ++j) key[j] = (s0 + j < nrows) ? key[j] : 0u;
        topk_select<KP, SCORE_WAVES>(key, s0, K, offset, idx + qi * ld + col0, red, tot);
    }
}

template <int KPT>
__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(const uint16_t* __restrict__ keys, int64_t n_c,
                                                            int64_t m, int ratio, int64_t start_pos, int K,
                                                            int32_t offset, int32_t* __restrict__ idx, int64_t ld,
                                                            int64_t col0) {
    __shared__ uint32_t red[2][TOPK_THREADS / 64];
    __shared__ uint32_t tot[TOPK_THREADS / 64];
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

    topk_select<KPT, TOPK_THREADS / 64>(key, s0, K, offset, out, red, tot);
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

// LDS bytes of a score launch (KPT as in index_score_kernel).
template <int MT, int DI, int KPT>
size_t score_lds_bytes(int rows_per_wg, bool with_scores) {
    using Sh = ScoreShape<MT, DI, KPT == 0 ? 0 : fused_ring_depth(DI, KPT)>;
    return Sh::lds_bytes(rows_per_wg, with_scores);
}

template <int MT, int DI, int KPT>
int launch_scores(const uint16_t* q, const uint16_t* k, const float* w, int64_t nq, int64_t m, int Hi, int64_t n_c,
                  int ratio, int64_t start_pos, int rows_per_wg, int nsplit, uint16_t* keys, uint16_t* scores, int K,
                  int32_t offset, int32_t* idx, int64_t ld, int64_t col0, hipStream_t stream) {
    const size_t lds = score_lds_bytes<MT, DI, KPT>(rows_per_wg, scores != nullptr);
    if (lds > 160 * 1024) return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: score tile does not fit in LDS");
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)index_score_kernel<MT, DI, KPT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return fail(SCKV_EHIP, std::string("sckv_index_scores_topk: ") + hipGetErrorString(e));
    }
    index_score_kernel<MT, DI, KPT><<<dim3((unsigned)(nq * nsplit)), dim3(SCORE_WAVES * 64), lds, stream>>>(
        q, k, w, m, Hi, n_c, ratio, start_pos, rows_per_wg, nsplit, keys, scores, K, offset, idx, ld, col0);
    return SCKV_OK;
}

// Fused scores + top-K for one (MT, DI) with KPT keys per thread for the whole
// query; SCKV_EUNSUPPORTED (nothing launched) when it does not fit in LDS.
template <int MT, int DI>
int launch_fused(const uint16_t* q, const uint16_t* k, const float* w, int64_t nq, int64_t m, int Hi, int64_t n_c,
                 int ratio, int64_t start_pos, int K, int32_t offset, int32_t* idx, int64_t ld, int64_t col0,
                 hipStream_t s) {
    const int rows = (int)((n_c + 127) / 128 * 128);
    const int need = (rows + SCORE_WAVES * 64 - 1) / (SCORE_WAVES * 64);
#define SCKV_FUSED(KPT)                                                                                          \
    (score_lds_bytes<MT, DI, KPT>(rows, false) > 160 * 1024                                                       \
         ? SCKV_EUNSUPPORTED                                                                                      \
         : launch_scores<MT, DI, KPT>(q, k, w, nq, m, Hi, n_c, ratio, start_pos, rows, 1, nullptr, nullptr, K, \
                                      offset, idx, ld, col0, s))
    if (need <= 8) return SCKV_FUSED(8);
    if (need <= 32) return SCKV_FUSED(32);
    if (need <= 128) return SCKV_FUSED(128);
#undef SCKV_FUSED
    return SCKV_EUNSUPPORTED;
}

// Rows per workgroup: a multiple of 128 (4 waves x 32 rows), small enough that
// the launch has about 256 workgroups when the queries alone do not, and at
// most 4096 (2048 when scores are also written: keys and scores are buffered
// in LDS).
int score_rows_per_wg(int64_t nq, int64_t n_c, bool with_scores) {
    int64_t tiles = (n_c + 127) / 128;  // 128-row tiles of one query
    int64_t want_splits = (256 + nq - 1) / nq;
    if (want_splits > tiles) want_splits = tiles;
    if (want_splits < 1) want_splits = 1;
    int64_t tiles_per = (tiles + want_splits - 1) / want_splits;
    const int64_t cap = with_scores ? 16 : 32;
    if (tiles_per > cap) tiles_per = cap;
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
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    uint16_t* sc = (uint16_t*)scores;
    const bool two = Hi > 32;
    int rc;
    if (!scores && nq >= FUSED_MIN_QUERIES && n_c <= 32768) {
        // enough queries to fill the chip with one workgroup each: scores and
        // top-K in one launch, the keys never leaving LDS
#define SCKV_FUSED(MT, DI) launch_fused<MT, DI>(qq, kk, w, nq, m, Hi, n_c, ratio, start_pos, K, offset, idx, ld, col0, s)
        switch (Di) {
            case 32: rc = two ? SCKV_FUSED(2, 32) : SCKV_FUSED(1, 32); break;
            case 64: rc = two ? SCKV_FUSED(2, 64) : SCKV_FUSED(1, 64); break;
            case 128: rc = two ? SCKV_FUSED(2, 128) : SCKV_FUSED(1, 128); break;
            default: rc = two ? SCKV_FUSED(2, 256) : SCKV_FUSED(1, 256); break;
        }
#undef SCKV_FUSED
        if (rc != SCKV_EUNSUPPORTED) return rc ? rc : check_launch("sckv_index_scores_topk (fused)");
    }
    const int rpw = score_rows_per_wg(nq, n_c, scores != nullptr);
    const int nsplit = (int)((n_c + rpw - 1) / rpw);
    if (nq * nsplit > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: grid too large");
    uint16_t* keys = (uint16_t*)ws;
#define SCKV_SCORES(MT, DI)                                                                                   \
    launch_scores<MT, DI, 0>(qq, kk, w, nq, m, Hi, n_c, ratio, start_pos, rpw, nsplit, keys, sc, K, offset, idx, \
                             ld, col0, s)
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

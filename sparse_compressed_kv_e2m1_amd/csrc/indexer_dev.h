// indexer_dev.h -- device code of the indexer (scores of a row range or of a
// whole query, and the per-query top-K), as bodies that take their workgroup
// number: the kernels of indexer.hip run them with blockIdx.x, the one-launch
// decode step (decode_step.hip) with its own numbering of the same work.
#pragma once

#include "mfma.h"
#include "sckv_device.h"

namespace sckv {
namespace {

// waves of a score workgroup: 4 with bf16 k tiles (the LDS holds four
// 4-deep rings of 8 KiB tiles), 8 with packed fp4 tiles (small tiles; two
// waves a SIMD hide the w.relu / head-sum vector work behind each other)
constexpr int score_waves(bool fp4) { return fp4 ? 8 : 4; }
constexpr int TOPK_THREADS = 512;
constexpr int FUSED_MIN_QUERIES = 192;  // fused scores + top-K from this many queries on
constexpr size_t SCORE_STATIC_LDS = 2112;  // the score kernel's static LDS (histogram, scan words), rounded up

// Ordered 16-bit key of a bf16 score: -0 counts as +0; a larger key is a
// larger score.
__device__ __forceinline__ uint32_t score_key(uint32_t b) {
    if (b == 0x8000u) b = 0u;
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}

// ---- top-k: one block per query, keys held in registers
//
// Thread t owns the KPT consecutive rows [t*KPT, t*KPT + KPT).  The K-th
// largest key tau is found with counts in registers summed over the block
// (its high byte) and an LDS histogram (its low byte; topk_select), or bit by
// bit in 16 rounds of counts (keys two to a register, topk_select_packed);
// then the rows with key > tau and the first (K - #greater) rows with key ==
// tau (lowest rows first) are written in ascending row order after block
// prefix sums of the two counts (compact_selected; the bit-by-bit form keeps
// its own compaction).  Missing rows hold key 0, below every real key (finite
// scores have keys >= 0x007f).

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

// The bin b of a 256-bin histogram with (keys in bins above b) < k <= (keys
// in bins b and above), and the count of keys in bins above b; every wave
// computes the same (uniform) answer from LDS.  Needs 1 <= k <= total.
__device__ __forceinline__ void find_bin(const uint32_t* h, uint32_t k, uint32_t& bin, uint32_t& above) {
    const int lane = threadIdx.x & 63;
    const u32x4 c = *reinterpret_cast<const u32x4*>(h + 4 * lane);  // bins 4 lane .. 4 lane + 3
    const uint32_t s = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_incl_scan(s);                       // keys in bins < 4 (lane + 1)
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t ge = total - incl + s;                           // keys in bins >= 4 lane
    const uint32_t gt = ge - s;                                     // keys in bins >= 4 (lane + 1)
    const bool mine = gt < k && ge >= k;                            // exactly one lane
    const int L = __builtin_ctzll(__ballot(mine));
    uint32_t b = 4 * lane, run = gt;
    if (mine) {
#pragma unroll
        for (int i = 3; i >= 1; --i) {
            if (run + c[i] >= k) {
                b = 4 * lane + i;
                break;
            }
            run += c[i];
        }
    }
    bin = (uint32_t)__builtin_amdgcn_readlane((int)b, L);
    above = (uint32_t)__builtin_amdgcn_readlane((int)run, L);
}

// Max of x over the wave (uniform result), the same butterfly as wave_sum.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    x = max(x, SCKV_DPP(x, 0xb1, 0xf, false));
    x = max(x, SCKV_DPP(x, 0x4e, 0xf, false));
    x = max(x, SCKV_DPP(x, 0x141, 0xf, false));
    x = max(x, SCKV_DPP(x, 0x140, 0xf, false));
    return max(max((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48)));
}

// Max over the block of NWAVES waves (buf as in block_sum).
template <int NWAVES>
__device__ __forceinline__ uint32_t block_max(uint32_t x, uint32_t* buf) {
    const uint32_t w = wave_max(x);
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = w;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) t = max(t, buf[i]);
    return t;
}

// The ordered compaction that ends a selection: of thread t's rows s0 ..
// s0 + KPT - 1, those with key > tau and, over the block, the first need_eq
// rows (lowest first) with key == tau, written in ascending row order to
// dst[0 .. K).  The thread's matches are kept as bit masks; one block scan of
// its two counts packed in one word (greater in the high half, equal in the
// low half: with at most 2^15 keys a block the halves cannot carry) gives
// both prefix counts, and the thread then walks only its selected bits.
template <int KPT, int NWAVES>
__device__ __forceinline__ void compact_selected(const uint32_t (&key)[KPT], uint32_t tau, uint32_t need_eq,
                                                 int64_t s0, int K, int32_t offset, int32_t* __restrict__ dst,
                                                 uint32_t* tot) {
    constexpr int NM = (KPT + 31) / 32;
    uint32_t gtm[NM], eqm[NM];
#pragma unroll
    for (int i = 0; i < NM; ++i) gtm[i] = eqm[i] = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        gtm[j / 32] |= (key[j] > tau ? 1u : 0u) << (j % 32);
        eqm[j / 32] |= (key[j] == tau ? 1u : 0u) << (j % 32);
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        gt += (uint32_t)__builtin_popcount(gtm[i]);
        eq += (uint32_t)__builtin_popcount(eqm[i]);
    }
    uint32_t eq_before, pos;
    if constexpr (KPT * NWAVES * 64 <= 32768) {
        const uint32_t before = block_excl_scan<NWAVES>((gt << 16) | eq, tot);
        eq_before = before & 0xffffu;
        pos = (before >> 16) + (need_eq < eq_before ? need_eq : eq_before);
    } else {  // (more keys than the packed halves hold: two scans)
        eq_before = block_excl_scan<NWAVES>(eq, tot);
        const uint32_t t = (need_eq > eq_before) ? (need_eq - eq_before) : 0u;
        pos = block_excl_scan<NWAVES>(gt + (t < eq ? t : eq), tot);
    }
    uint32_t take_eq = (need_eq > eq_before) ? (need_eq - eq_before) : 0u;  // this thread's equal keys to take
    take_eq = take_eq < eq ? take_eq : eq;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        uint32_t e = eqm[i];
        while (take_eq > 0u && e != 0u) {  // the lowest equal rows first
            const uint32_t low = e & (0u - e);
            gtm[i] |= low;
            e ^= low;
            --take_eq;
        }
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        uint32_t sel = gtm[i];
        while (sel != 0u) {
            const int j = __builtin_ctz(sel);
            sel &= sel - 1u;
            if (pos < (uint32_t)K) dst[pos] = (int32_t)(offset + s0 + 32 * i + j);
            ++pos;
        }
    }
}

// Top-K of the keys held by the block: thread t owns key[0..KPT) of rows
// s0 .. s0+KPT-1 (rows at or past the visible count hold key 0).  Writes
// offset + s of the K selected rows in ascending s to out[0..K).  Needs
// V > K visible rows (so tau ends up >= 1 and every missing key is below it).
// The K-th largest key tau: its high byte h is the largest with at least K
// keys whose high byte is >= h, searched downwards from the high byte of the
// largest key (the top keys of a score list share one or two high bytes:
// typically one or two block counts) and, after four steps, by bisection;
// its low byte comes from a histogram (hist: 256 words of LDS) of the low
// bytes of the keys in that high byte.  About 5 block-wide barriers instead
// of 16 for a bit-by-bit search (measured: the 16 rounds of block sums set
// the time of one query's top-K, 6-7 us at 8192 keys).
template <int KPT, int NWAVES>
__device__ __forceinline__ void topk_select(const uint32_t (&key)[KPT], int64_t s0, int K, int32_t offset,
                                            int32_t* __restrict__ out, uint32_t (*red)[NWAVES], uint32_t* tot,
                                            uint32_t* hist) {
    for (int i = threadIdx.x; i < 256; i += NWAVES * 64) hist[i] = 0u;  // ordered by the next barrier
    int rb = 0;
    uint32_t kmax = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) kmax = max(kmax, key[j]);
    kmax = block_max<NWAVES>(kmax, red[rb]);
    rb ^= 1;
    // count of keys whose high byte is >= g (uniform)
    auto count_ge = [&](uint32_t g) {
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) c += (key[j] >> 8) >= g;
        const uint32_t t = block_sum<NWAVES>(c, red[rb]);
        rb ^= 1;
        return t;
    };
    uint32_t h = kmax >> 8;
    uint32_t above = 0;  // keys whose high byte is > h
    bool found = false;
#pragma unroll 1
    for (int step = 0; step < 4; ++step) {
        const uint32_t c = count_ge(h);
        if (c >= (uint32_t)K) {
            found = true;
            break;
        }
        above = c;
        --h;  // h >= 1 here: count_ge(0) counts every key, which is >= K
    }
    if (!found) {
        // the largest g in [0, h] with count_ge(g) >= K; `above` stays the
        // count for hi + 1
        uint32_t lo = 0, hi = h;
#pragma unroll 1
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            const uint32_t c = count_ge(mid);
            if (c >= (uint32_t)K) {
                lo = mid;
            } else {
                hi = mid - 1;
                above = c;
            }
        }
        h = lo;
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if ((key[j] >> 8) == h) atomicAdd(&hist[key[j] & 0xffu], 1u);
    __syncthreads();
    uint32_t lo_bin, above_lo;
    find_bin(hist, (uint32_t)K - above, lo_bin, above_lo);
    const uint32_t tau = (h << 8) | lo_bin;
    const uint32_t need_eq = (uint32_t)K - (above + above_lo);  // keys == tau to take, >= 1
    compact_selected<KPT, NWAVES>(key, tau, need_eq, s0, K, offset, out, tot);
}

// topk_select with the keys packed two to a register (key 2i in the low half
// of kp[i], key 2i + 1 in the high half): the same selection and compaction
// in half the key registers, for 128 keys a thread.
template <int KP2, int NWAVES>
__device__ __forceinline__ void topk_select_packed(const uint32_t (&kp_in)[KP2], int64_t s0, int K, int32_t offset,
                                                   int32_t* __restrict__ out, uint32_t (*red)[NWAVES], uint32_t* tot) {
    uint32_t kp[KP2];
#pragma unroll
    for (int i = 0; i < KP2; ++i) kp[i] = kp_in[i];
    uint32_t tau = 0;
    int rb = 0;
#pragma unroll 1
    for (int bit = 15; bit >= 0; --bit) {
        // (the words pass an empty asm each round, so that their halves are
        // taken apart inside the round instead of being hoisted out of the
        // loop into 2 KP2 registers)
#pragma unroll
        for (int i = 0; i < KP2; ++i) asm volatile("" : "+v"(kp[i]));
        const uint32_t cand = tau | (1u << bit);
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < KP2; ++i) c += ((kp[i] & 0xffffu) >= cand) + ((kp[i] >> 16) >= cand);
        const uint32_t total = block_sum<NWAVES>(c, red[rb]);
        rb ^= 1;
        if (total >= (uint32_t)K) tau = cand;
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < KP2; ++i) asm volatile("" : "+v"(kp[i]));
#pragma unroll
    for (int i = 0; i < KP2; ++i) {
        const uint32_t k0 = kp[i] & 0xffffu, k1 = kp[i] >> 16;
        gt += (k0 > tau) + (k1 > tau);
        eq += (k0 == tau) + (k1 == tau);
    }
    const uint32_t gt_total = block_sum<NWAVES>(gt, red[rb]);
    const uint32_t need_eq = (uint32_t)K - gt_total;  // >= 1 by the choice of tau
    const uint32_t eq_before = block_excl_scan<NWAVES>(eq, tot);
    uint32_t take_eq = (need_eq > eq_before) ? (need_eq - eq_before) : 0u;
    take_eq = take_eq < eq ? take_eq : eq;
    uint32_t pos = block_excl_scan<NWAVES>(gt + take_eq, tot);
    uint32_t eq_seen = 0;
#pragma unroll
    for (int i = 0; i < KP2; ++i) asm volatile("" : "+v"(kp[i]));
#pragma unroll
    for (int j = 0; j < 2 * KP2; ++j) {
        const uint32_t k = (j & 1) ? (kp[j >> 1] >> 16) : (kp[j >> 1] & 0xffffu);
        bool take = k > tau;
        if (k == tau) {
            take = eq_seen < take_eq;
            ++eq_seen;
        }
        if (take && pos < (uint32_t)K) out[pos++] = (int32_t)(offset + s0 + j);
    }
}


// topk_select for a block that already holds the histogram of its keys' high
// bytes (hist[0..256), built while the keys were produced): the K-th largest
// key tau is the high-byte bin found there plus the low-byte bin found in a
// second histogram (hist[256..512), zero on entry) over the keys of that bin
// only; then the same ordered compaction.  With `stage` (K free words of LDS)
// the selected rows gather there first and leave with coalesced stores
// instead of one scattered store per selected key.
template <int KPT, int NWAVES>
__device__ __forceinline__ void topk_select_hist(const uint32_t (&key)[KPT], int64_t s0, int K, int32_t offset,
                                                 int32_t* __restrict__ out, uint32_t* hist, uint32_t* tot,
                                                 int32_t* stage = nullptr) {
    uint32_t hi_bin, above_hi;
    find_bin(hist, (uint32_t)K, hi_bin, above_hi);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if ((key[j] >> 8) == hi_bin) atomicAdd(&hist[256 + (key[j] & 0xffu)], 1u);
    __syncthreads();
    uint32_t lo_bin, above_lo;
    find_bin(hist + 256, (uint32_t)K - above_hi, lo_bin, above_lo);
    const uint32_t tau = (hi_bin << 8) | lo_bin;
    const uint32_t need_eq = (uint32_t)K - (above_hi + above_lo);  // keys == tau to take, >= 1
    compact_selected<KPT, NWAVES>(key, tau, need_eq, s0, K, offset, stage ? stage : out, tot);
    if (stage) {
        __syncthreads();
        for (int i = threadIdx.x; i < K; i += NWAVES * 64) out[i] = stage[i];
    }
}

// Shape of one score workgroup for MT head tiles and head dim DI; NST_ > 0
// sets the ring depth (tiles per wave) instead of the default.  FP4: the k
// rows come packed (4-bit e2m1 codes, one E8M0 byte per 32 values) and the
// contraction runs on the scaled fp4 matrix cores.
template <int MT, int DI, int NST_ = 0, bool FP4 = false, int NW_ = 0>
struct ScoreShape {
    static constexpr int HP = MT * 32;                 // padded heads
    static constexpr int KS = FP4 ? DI / 64 : DI / 16; // k-steps (64 fp4 or 16 bf16 values each)
    static constexpr int ROWB = FP4 ? DI / 2 : DI * 2; // bytes per k row (codes only for FP4)
    static constexpr int SB = FP4 ? DI / 32 : 0;       // scale bytes per k row
    static constexpr int CT = 32 * ROWB;               // bytes of a 32-row tile's rows
    static constexpr int TILE = CT + 32 * SB;          // ... plus its scale bytes
    static constexpr int NINST = CT / 1024 + (FP4 ? 1 : 0);  // copies per tile (the last one: scales)
    static constexpr int NST = NST_ > 0 ? NST_ : (FP4 ? (TILE >= 4096 ? 3 : 8) : ((TILE >= 16384) ? 1 : 4));  // tiles per wave in the ring
    static constexpr int PD = NST - 1;                 // tiles requested ahead of the one used
    static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
    static constexpr int SWZ = (CPR < 8 ? CPR : 8) - 1;  // bf16 chunk swizzle mask
    static constexpr int RPS = 16 / (CPR < 16 ? CPR : 16);  // fp4: rows sharing one swizzle value
    static constexpr int QS = FP4 ? DI / 2 : DI * 2;   // bytes per q row in LDS (fp4: codes)
    static constexpr int NW = NW_ > 0 ? NW_ : score_waves(FP4);  // waves
    static constexpr int OFF_Q = NW * NST * TILE;
    static constexpr int OFF_QS = OFF_Q + HP * QS;     // fp4: q scale bytes [HP][SB]
    static constexpr int OFF_W = OFF_QS + HP * SB;     // 64 f32 head weights
    static constexpr int OFF_QR = OFF_W + 64 * 4;      // fp4: the raw bf16 q rows [HP][DI]
    // keys (then scores) reuse the q / w space once q_hat and the weights sit
    // in registers
    static constexpr int OFF_KEYS = OFF_Q;
    static constexpr size_t lds_bytes(int rows_per_wg, bool with_scores) {
        const size_t qw = (size_t)HP * QS + (size_t)HP * SB + 64 * 4 + (FP4 ? (size_t)HP * DI * 2 : 0);
        const size_t ks = (size_t)rows_per_wg * 2 * (with_scores ? 2 : 1);
        return (size_t)OFF_Q + (qw > ks ? qw : ks);
    }
    static_assert(NINST >= 1 && NINST * PD < 64 && PD <= 7 && (TILE % 16) == 0, "copy counts");
};

// Wait until at most `ahead` later tiles (NINST copies each) of this wave
// may still be in flight (0 <= ahead <= PDMAX - 1).
template <int NINST, int PDMAX>
__device__ __forceinline__ void wait_tiles(int ahead) {
    switch (ahead < PDMAX - 1 ? ahead : PDMAX - 1) {
        case 6: wait_vmcnt<(6 * NINST < 64 ? 6 * NINST : 63)>(); break;
        case 5: wait_vmcnt<(5 * NINST < 64 ? 5 * NINST : 63)>(); break;
        case 4: wait_vmcnt<(4 * NINST < 64 ? 4 * NINST : 63)>(); break;
        case 3: wait_vmcnt<(3 * NINST < 64 ? 3 * NINST : 63)>(); break;
        case 2: wait_vmcnt<(2 * NINST < 64 ? 2 * NINST : 63)>(); break;
        case 1: wait_vmcnt<NINST>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

// Ring depth of the fused kernel: the keys of a whole query share the LDS
// with the ring (KPT keys per thread, 256 threads).
// (NWV = 4: 2 deep, so that four 4-wave workgroups share a compute unit)
constexpr int fused_ring_depth(int DI, int KPT, bool FP4, int NWV = 0) {
    if (NWV == 4) return 2;
    // fp4, up to 16 keys a thread (at most 8192 rows, 16 tiles a wave): a
    // shallow ring, so that two workgroups share a compute unit and one's
    // prologue and top-K overlap the other's stream
    return FP4 ? (17 * DI >= 4096 ? (KPT >= 64 || KPT <= 8 ? 2 : 3) : (KPT >= 64 ? 4 : (KPT <= 16 ? 3 : 8)))
               : ((64 * DI >= 16384) ? 1 : (KPT >= 128 ? 2 : 4));
}

// The head that row r of a 32-head tile holds in the score products: the D
// layout gives lane l, value i the row 8 (i / 4) + 4 (l / 32) + i % 4, so row r
// holding head 2 (4 (r / 8) + r % 4) + (r / 4) % 2 puts head 2 i + l / 32 at
// value i of lane l.  Every pair the fixed head-sum tree adds (h, h + stride)
// for strides 32 (the other tile), 16, 8, 4, 2 then sits in one lane; only
// stride 1 crosses to lane l ^ 32.
__device__ __forceinline__ int head_of_row(int r) { return 2 * ((r >> 3) * 4 + (r & 3)) + ((r >> 2) & 1); }

// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands e2m1 (format 4): lane l
// holds, for row l%32, the 32 codes of k-block l/32 (16 bytes, in the low four
// registers) and that block's E8M0 scale in the low byte of its scale word.
// Within a block any order of the codes works as long as A and B agree.
__device__ __forceinline__ f32x16 mfma_fp4(u32x4 a, uint32_t sa, u32x4 b, uint32_t sb, f32x16 c) {
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    const i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    const i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// KPT == 0: scores of a row range, ordered keys flushed to `keys` for the
// top-k kernel.  KPT > 0 (fused, one workgroup per query, no split): the
// whole query's keys stay in LDS and the workgroup selects its top-K itself.
// q is the raw bf16 q [Hi][DI] of each query in both forms; the workgroup
// takes its round trip in LDS.  FP4: k arrives as codes [n_c][DI/2] and
// scale bytes [n_c][DI/32], and q_hat is packed the same way in LDS;
// otherwise k is bf16 [n_c][DI].
template <int MT, int DI, int KPT, bool FP4, int NWV = 0>
__device__ __forceinline__ void index_score_body(
    const void* __restrict__ q, const void* __restrict__ k,
    const uint8_t* __restrict__ k_scales, const float* __restrict__ w, int64_t m, int Hi_arg, int64_t n_c, int ratio,
    int64_t start_pos, int rows_per_wg, int nsplit, uint16_t* __restrict__ keys, uint16_t* __restrict__ scores, int K,
    int32_t offset, int32_t* __restrict__ idx, int64_t ld, int64_t col0, const uint32_t vb) {
    using S = ScoreShape<MT, DI, KPT == 0 ? 0 : fused_ring_depth(DI, KPT, FP4, NWV), FP4, NWV>;
    constexpr int KS = S::KS;
    // two head tiles hold Hi in 33..64, and Hi is a power of two: Hi = 64,
    // known at compile time (the head-sum steps below then need no selects)
    const int Hi = MT == 2 ? 64 : Hi_arg;
    extern __shared__ __align__(16) unsigned char lds[];
    unsigned char* qh_l = lds + S::OFF_Q;
    uint16_t* keys_l = reinterpret_cast<uint16_t*>(lds + S::OFF_KEYS);
    uint16_t* sc_l = keys_l + rows_per_wg;
    const uint32_t lds0 = lds_offset(lds);

    // (the thread number through an opaque copy: the per-thread arithmetic
    // derived from it then stays inside a caller's loop over work items
    // instead of being hoisted and kept live across it)
    int tidx;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tidx) : "v"((int)threadIdx.x));
    const int lane = tidx & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tidx >> 6);
    const int64_t qi = vb / nsplit;
    const int split = (int)(vb - qi * nsplit);
    const int64_t b = qi / m;
    const int64_t t = qi - b * m;

    int64_t vis = (start_pos + t + 1) / ratio;
    vis = vis < n_c ? vis : n_c;
    if (KPT > 0 && vis <= K) {
        // every visible row is selected: no scores needed
        int32_t* out = idx + qi * ld + col0;
        for (int j = tidx; j < K; j += S::NW * 64) out[j] = (j < vis) ? (int32_t)(offset + j) : -1;
        return;
    }
    // (the split path leaves such queries to the top-k kernel; it still writes
    // their scores when asked for)
    if (KPT == 0 && !scores && vis <= K) return;
    const int64_t row0 = (int64_t)split * rows_per_wg;
    if (row0 >= vis) return;
    int64_t row_end = row0 + rows_per_wg;
    row_end = row_end < vis ? row_end : vis;

    // ---- the workgroup's rows [row0, row_end) in 32-row tiles, each streamed
    // through the ring of the wave that takes it.  The waves take tiles in the
    // order they ask for them: wave w's first QD are w, w + NW, ...; after
    // that each request claims the next unclaimed tile from an LDS counter, so
    // that all waves run out of tiles together, however unevenly the memory
    // system serves them.  Lane i of copy j brings 16 bytes to tile byte
    // j*1024 + 16 i; which 16-byte chunk of which row lands there is swizzled
    // so that the B-operand reads below (32 rows at one chunk) spread over all
    // banks.  FP4: the tile's scale bytes follow its codes.
    const int64_t nrows = row_end - row0;
    const int ntiles_all = (int)((nrows + 31) / 32);
    constexpr int QD = S::PD > 0 ? S::PD : 1;  // tiles a wave has asked for and not yet used
    __shared__ uint32_t tile_ctr;
    const unsigned char* kb = reinterpret_cast<const unsigned char*>(k) + b * n_c * S::ROWB;
    const uint8_t* ksb = FP4 ? k_scales + b * n_c * S::SB : nullptr;
    const uint32_t ring = lds0 + (uint32_t)(wave * S::NST * S::TILE);
    // the wave's seq-th tile (ring stage seq % NST) is tile t
    // (a sequence's k rows span under 2^31 bytes: n_c <= 65536 rows of at most
    // 512 bytes, so the copy offsets are 32-bit)
    auto issue = [&](int seq, int t) {
        const int64_t s0 = row0 + (int64_t)t * 32;
        const uint32_t st = ring + (uint32_t)((seq % S::NST) * S::TILE);
        // a tile wholly inside the array (every one but possibly the last):
        // the tile's offset plus the lane's, no clamp
        const bool whole = s0 + 32 <= n_c;
#pragma unroll
        for (int j = 0; j < S::CT / 1024; ++j) {
            const int slot = j * 64 + lane;  // 16-byte slot of the tile
            const int r = slot / S::CPR;
            const int cp = slot % S::CPR;
            const int ch = FP4 ? (cp ^ ((r / S::RPS) % S::CPR)) : (cp ^ (r & S::SWZ));
            uint32_t off;
            if (whole) {
                off = (uint32_t)s0 * (uint32_t)S::ROWB + (uint32_t)(r * S::ROWB + ch * 16);
            } else {
                int64_t row = s0 + r;
                row = row < n_c ? row : n_c - 1;  // tail rows re-read a real row; their results are dropped
                off = (uint32_t)(row * S::ROWB + ch * 16);
            }
            dma16_s(kb, off, st + (uint32_t)(j * 1024));
        }
        if (FP4) {
            // scale bytes of the tile's 32 rows, 4 bytes a lane (SB = 2: 2 rows a lane)
            const int per = S::SB >= 4 ? S::SB / 4 : 1;      // lanes per row
            const int rpl = S::SB >= 4 ? 1 : 4 / S::SB;      // rows per lane
            const int nl = 32 * per / rpl;
            if (lane < nl) {
                uint32_t off;
                if (whole) {
                    off = (uint32_t)s0 * (uint32_t)S::SB + (uint32_t)(((lane / per) * rpl) * S::SB + (lane % per) * 4);
                } else {
                    int64_t row = s0 + (lane / per) * rpl;
                    const int64_t last = n_c - rpl;  // keep the 4-byte read inside the array
                    row = row < last ? row : (last > 0 ? last : 0);
                    off = (uint32_t)(row * S::SB + (lane % per) * 4);
                }
                dma4_s(ksb, off, st + (uint32_t)(S::CT));
            }
        }
    };
    // ---- prologue.  q and the head weights come in by asynchronous copies, this
    // wave's first k tiles are requested right behind them.  No ordinary
    // global load is issued in this kernel, so every vmcnt wait is explicit.
    // the raw bf16 q rows (fp4: into their own region, to be packed there)
    const int qbytes = Hi * DI * 2;
    const uint32_t qdst = lds0 + (FP4 ? S::OFF_QR : S::OFF_Q);
    const unsigned char* qrow = reinterpret_cast<const unsigned char*>(q) + qi * (int64_t)qbytes;
    for (int j = wave; j * 1024 < qbytes; j += S::NW)
        if (j * 1024 + lane * 16 < qbytes) dma16_s(qrow, (uint32_t)(j * 1024 + lane * 16), qdst + j * 1024);
    if (wave == 0 && lane < Hi) dma4_s(w + qi * (int64_t)Hi, (uint32_t)lane * 4u, lds0 + S::OFF_W);
    int tq[QD];  // this wave's tiles in request order (>= ntiles_all: none left)
#pragma unroll
    for (int i = 0; i < QD; ++i) tq[i] = wave + i * S::NW;
    if (tidx == 0) tile_ctr = (uint32_t)(S::NW * QD);  // read only after the barrier below
#pragma unroll
    for (int i = 0; i < S::PD; ++i)
        if (tq[i] < ntiles_all) issue(i, tq[i]);
    // fused top-K: the high-byte histogram of the keys fills while they are
    // produced (hist[0..256)); hist[256..512) serves the second pass
    __shared__ uint32_t hist[KPT > 0 ? 512 : 1];
    if (KPT > 0)
        for (int i = tidx; i < 512; i += S::NW * 64) hist[i] = 0u;
    // q and w landed (only the tile copies may still be in flight), in every wave
    if (S::PD == 0 || tq[S::PD > 0 ? S::PD - 1 : 0] < ntiles_all)
        wait_vmcnt<S::PD * S::NINST>();
    else
        wait_vmcnt<0>();
    __syncthreads();

    // ---- q_hat in A layout: head mt*32 + lane%32
    bf16x8 qa[FP4 ? 1 : MT][FP4 ? 1 : KS];
    u32x4 qc[FP4 ? MT : 1][FP4 ? KS : 1];     // fp4 codes of k-block 2*ks + lane/32
    uint32_t qsc[FP4 ? MT : 1][FP4 ? KS : 1];  // and their E8M0 scale
    if constexpr (!FP4) {
        // q_hat = E8M0_B32 round trip of the raw q, one 32-value block per thread
        // and step, in place; padded heads (h >= Hi) become zero rows
        for (int blk = tidx; blk < S::HP * (DI / 32); blk += S::NW * 64) {
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
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qa[mt][ks] = *reinterpret_cast<const bf16x8*>(qh_l + (mt * 32 + head_of_row(lane & 31)) * S::QS +
                                                              (ks * 16 + (lane >> 5) * 8) * 2);
    } else {
        // q_hat = E8M0_B32 round trip of the raw q, packed: one 32-value block per
        // thread and step (codes of values 2j, 2j+1 in byte j, low nibble first;
        // the block's E8M0 byte); padded heads (h >= Hi) are never read
        const unsigned char* qr_l = lds + S::OFF_QR;
        uint8_t* qs_w = lds + S::OFF_QS;
        for (int blk = tidx; blk < Hi * (DI / 32); blk += S::NW * 64) {
            const int h = blk / (DI / 32);
            const int c = blk - h * (DI / 32);
            const u32x4* qb = reinterpret_cast<const u32x4*>(qr_l + h * DI * 2 + c * 64);
            u32x4 raw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) raw[i] = qb[i];
            // amax as bf16 magnitude bits (for finite values their integer
            // order is the order of |v|)
            uint32_t am = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t mw = raw[i][e] & 0x7fff7fffu;
                    const uint32_t lo = mw & 0xffffu, hi = mw >> 16;
                    am = am > lo ? am : lo;
                    am = am > hi ? am : hi;
                }
            const float sc = block_scale<SCKV_FP4_E8M0_B32>(__uint_as_float(am << 16));
            // the codes by the gfx950 down-conversion (v_cvt_scalef32_pk_fp4_bf16:
            // two values divided by the scale, rounded to e2m1 with ties to even,
            // saturated at 6, sign kept).  Checked on gfx950 against the rounding
            // rule above for every finite bf16 value at every scale 2^-126 ..
            // 2^126, the whole range of power-of-two block scales of finite bf16
            // data (amax <= 3.4e38, so amax / 6 < 2^126).
            u32x4 cw;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // the 8 codes of raw[i] (values 8i .. 8i+7): byte e from word e (the
                // instruction's byte select).  The words are copied out of the
                // vector first: a bit cast of a vector element itself is read as
                // element 0 by this compiler.
                const uint32_t x0 = raw[i][0], x1 = raw[i][1], x2 = raw[i][2], x3 = raw[i][3];
                uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2, x0), sc, 0);
                word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, x1), sc, 1);
                word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, x2), sc, 2);
                word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, x3), sc, 3);
                cw[i] = word;
            }
            *reinterpret_cast<u32x4*>(qh_l + h * S::QS + c * 16) = cw;
            qs_w[h * S::SB + c] = (uint8_t)scale_byte<SCKV_FP4_E8M0_B32>(sc);
        }
        __syncthreads();
        const uint8_t* qs_l = lds + S::OFF_QS;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int h = mt * 32 + head_of_row(lane & 31);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int blk = 2 * ks + (lane >> 5);
                qc[mt][ks] = (h < Hi) ? *reinterpret_cast<const u32x4*>(qh_l + h * S::QS + blk * 16) : u32x4{0, 0, 0, 0};
                qsc[mt][ks] = (h < Hi) ? (uint32_t)qs_l[h * S::SB + blk] : 127u;
            }
        }
    }
    // head weights in D layout: value i of lane l is head mt*32 + 2 i + l / 32
    const float* w_l = reinterpret_cast<const float*>(lds + S::OFF_W);
    float wd[MT][16];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = mt * 32 + 2 * i + (lane >> 5);
            wd[mt][i] = (h < Hi) ? w_l[h] : 0.0f;
        }
    __syncthreads();  // every wave holds q_hat and w before keys overwrite them

    for (int seq = 0; tq[0] < ntiles_all; ++seq) {
        const int tile = tq[0];
        if (S::PD == 0) issue(seq, tile);
        // the tiles asked for after this one may still be in flight; this one must be done
        int ahead = 0;
#pragma unroll
        for (int i = 1; i < QD; ++i) ahead += tq[i] < ntiles_all ? 1 : 0;
        wait_tiles<S::NINST, (S::PD > 1 ? S::PD : 1)>(ahead);
        // the next tile (none once a claim has run past the end)
        int tn = ntiles_all;
        if (tq[QD - 1] < ntiles_all) {
            uint32_t v = 0;
            if (lane == 0) v = atomicAdd(&tile_ctr, 1u);
            tn = __builtin_amdgcn_readfirstlane((int)v);
        }
        if (S::PD > 0 && tn < ntiles_all) issue(seq + S::PD, tn);  // into the stage the last tile used
#pragma unroll
        for (int i = 0; i < QD - 1; ++i) tq[i] = tq[i + 1];
        tq[QD - 1] = tn;
        const unsigned char* stp = lds + (wave * S::NST + seq % S::NST) * S::TILE;
        const int r = lane & 31;
        f32x16 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = zero16();
        if constexpr (!FP4) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = ks * 2 + (lane >> 5);
                const bf16x8 kr = *reinterpret_cast<const bf16x8*>(stp + r * S::ROWB + ((ch ^ (r & S::SWZ)) * 16));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma32x32x16(qa[mt][ks], kr, acc[mt]);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int blk = 2 * ks + (lane >> 5);
                const int cp = blk ^ ((r / S::RPS) % S::CPR);
                const u32x4 kc = *reinterpret_cast<const u32x4*>(stp + (r * S::CPR + cp) * 16);
                const uint32_t ksc = stp[S::CT + r * S::SB + blk];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_fp4(qc[mt][ks], qsc[mt][ks], kc, ksc, acc[mt]);
            }
        }
        // r_h = fl32(w_h * relu(d_h)); relu maps every d <= 0 (and -0) to +0:
        // as a signed integer a float with the sign bit set is negative, so the
        // integer max with 0 is that relu in one operation
        float v[MT * 16];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int db = __float_as_int(acc[mt][i]);
                v[mt * 16 + i] = wd[mt][i] * __int_as_float(db > 0 ? db : 0);
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
            v[0] = v[0] + v[2];
            v[1] = v[1] + v[3];
        }
        if (Hi > 2) v[0] = v[0] + v[1];
        if (Hi > 1) {
            // heads h and h + 1 sit in lanes l and l ^ 32: the lane swap hands
            // both lanes (v of the lower lane, v of the upper lane)
            const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
            v[0] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
        }
        const int64_t s = row0 + (int64_t)tile * 32 + r;
        if (lane < 32 && s < row_end) {
            const uint32_t bits = f32_to_bf16_bits(v[0]);
            const uint32_t key = score_key(bits);
            keys_l[s - row0] = (uint16_t)key;
            if (KPT > 0) atomicAdd(&hist[key >> 8], 1u);
            if (scores) sc_l[s - row0] = (uint16_t)bits;
        }
    }
    __syncthreads();
    if (KPT == 0) {
        // ---- flush this workgroup's keys (and scores) with coalesced stores
        uint16_t* kout = keys + qi * n_c + row0;
        for (int64_t i = tidx; i < nrows; i += S::NW * 64) kout[i] = keys_l[i];
        if (scores) {
            uint16_t* sout = scores + qi * n_c + row0;
            for (int64_t i = tidx; i < nrows; i += S::NW * 64) sout[i] = sc_l[i];
        }
    } else {
        // ---- fused top-K over the query's keys in LDS (row0 == 0, nrows == vis > K)
        constexpr int KP = KPT > 0 ? KPT : 8;
        __shared__ uint32_t tot[S::NW];
        const int64_t s0 = (int64_t)(uint32_t)(tidx * KP);  // (32-bit product: uniform operands stay scalar)
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
        // the rings are idle now: they stage the selected rows when K fits
        int32_t* stage = (size_t)K * 4 <= (size_t)S::NW * S::NST * S::TILE ? reinterpret_cast<int32_t*>(lds) : nullptr;
        topk_select_hist<KP, S::NW>(key, s0, K, offset, idx + qi * ld + col0, hist, tot, stage);
    }
}

template <int KPT>
__device__ __forceinline__ void topk_body(const uint16_t* __restrict__ keys, int64_t n_c,
                                                            int64_t m, int ratio, int64_t start_pos, int K,
                                                            int32_t offset, int32_t* __restrict__ idx, int64_t ld,
                                                            int64_t col0, const uint32_t vb) {
    __shared__ uint32_t red[2][TOPK_THREADS / 64];
    __shared__ uint32_t tot[TOPK_THREADS / 64];
    __shared__ uint32_t hist[256];
    const int tid = threadIdx.x;
    const int64_t qi = vb;
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
    if constexpr (KPT >= 128) {
        // keys two to a register (128 keys a thread)
        uint32_t kw[KPT / 2];
        // groups of 8 keys: 16-byte loads when every query's keys start on a
        // 16-byte boundary (n_c % 8 == 0), else 4-byte loads (n_c even) or
        // 2-byte loads; only the group that crosses n_c is read key by key
#pragma unroll
        for (int j8 = 0; j8 < KPT / 8; ++j8) {
            const int64_t g0 = s0 + 8 * j8;
            u32x4 v = u32x4{0, 0, 0, 0};
            if (g0 + 8 <= n_c) {
                if ((n_c % 8) == 0) {
                    v = load16(kp + g0);
                } else if ((n_c % 2) == 0) {
                    const uint32_t* p32 = reinterpret_cast<const uint32_t*>(kp + g0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = p32[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (uint32_t)kp[g0 + 2 * e] | ((uint32_t)kp[g0 + 2 * e + 1] << 16);
                }
            } else if (g0 < n_c) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (g0 + e < n_c) v[e >> 1] |= (uint32_t)kp[g0 + e] << (16 * (e & 1));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) kw[4 * j8 + e] = v[e];
        }
#pragma unroll
        for (int i = 0; i < KPT / 2; ++i) {
            const uint32_t lo = (s0 + 2 * i < vis) ? (kw[i] & 0xffffu) : 0u;
            const uint32_t hi = (s0 + 2 * i + 1 < vis) ? (kw[i] & 0xffff0000u) : 0u;
            kw[i] = lo | hi;
        }
        topk_select_packed<KPT / 2, TOPK_THREADS / 64>(kw, s0, K, offset, out, red, tot);
        return;
    }
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

    topk_select<KPT, TOPK_THREADS / 64>(key, s0, K, offset, out, red, tot, hist);
}

// (host)
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
}  // namespace sckv

// attn_dev.h -- device code of the sparse attention with the sink (the
// chunk-loop workgroup and the combine of split partials), as bodies that
// take their workgroup number: the kernels of attn.hip run them with
// blockIdx, the one-launch decode step (decode_step.hip) with its own
// numbering of the same work.
#pragma once

#include "mfma.h"
#include "sckv_device.h"

namespace sckv {
namespace {

constexpr int CHUNK = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float STALE_MAX = 8.0f;  // base-2 slack before the running max moves
constexpr int MAX_CPS = 128;       // chunks one workgroup handles at most (its index range sits in LDS)
constexpr int MIN_SPLIT_CHUNKS = 4;  // chunks a workgroup takes at least when a query's list is split

// Head dim D, NHW head waves per set (16 heads each), NS sets (2: the sets
// take alternate chunks of one query; 1: unsplit lists only, so that two
// workgroups share a compute unit); CPS chunks of the index list at most (64,
// 72 or MAX_CPS; the smaller variants stage less of the list and run the short
// lists ~7% faster, measured).
template <int D, int NHW, int CPS, int NS = 2, bool CS = false>
struct AttnShape {
    static constexpr int WAVES = NS * NHW;
    static constexpr int HP = 16 * NHW;     // padded heads
    static constexpr int KS = D / 32;       // k-steps of S^T = R . Q^T
    static constexpr int NT = D / 16;       // 16-wide output tiles
    static constexpr int RPW = CHUNK / NHW; // rows a wave copies in per chunk of its set
    static constexpr int NST = 2;           // stages per set
    // row stride in a stage, 32 bytes of padding: measured on gfx950, the S^T
    // operand reads (16 rows at one 16-byte column) then run at the full
    // 256 B/clk and the transposing reads at ~170 B/clk, against 128 B/clk for
    // both with 16 bytes of padding
    static constexpr int RS = 2 * D + 32;
    static constexpr int STAGE = CHUNK * RS;
    static constexpr int OFF_IDX = NS * NST * STAGE;
    static constexpr int IDXB = CPS * CHUNK * 4;  // bytes of the index slice
    static constexpr int NIB = 1;
    static constexpr int OFF_FLAG = OFF_IDX + NIB * IDXB;  // one byte per chunk: names a valid row
    // CS (column split of P . R, one set only): every wave's probabilities
    // [NHW][64 lanes] x 16 bytes, the running-max factors [HP] f32 and one
    // "moved" byte per head wave
    static constexpr int OFF_P = (OFF_FLAG + CPS + 15) / 16 * 16;
    static constexpr int OFF_ALPHA = OFF_P + NHW * 64 * 16;
    static constexpr int OFF_MOVED = OFF_ALPHA + HP * 4;
    static constexpr size_t LDS_BYTES = CS ? (size_t)OFF_MOVED + 16 : (size_t)OFF_FLAG + CPS;
    static constexpr int IPT = CPS * CHUNK / (WAVES * 64);  // index entries a thread stages
    // the exchanged halves of O ([D][HP] f32) reuse the stages and both sets'
    // (max, sum) the index slice; afterwards each wave stages its 16 x D/2
    // output block (bf16, or f32 partials) in the stages
    static_assert(NS == 1 || ((size_t)D * HP * 4 <= (size_t)OFF_IDX && 2 * HP * 8 <= CPS * CHUNK * 4), "merge space");
    static_assert(CPS % 8 == 0 && CPS >= 64 && CPS <= 128, "one or two flag words");
    static_assert((CPS * CHUNK) % (WAVES * 64) == 0, "index staging rounds");
    static_assert(NS == 1 || (size_t)WAVES * 16 * (D / 2) * 4 <= (size_t)OFF_IDX, "output staging");
    // one set: unsplit lists only; each wave stages its 16 full bf16 rows
    static_assert(NS == 2 || (size_t)WAVES * 16 * (2 * D + 32) <= (size_t)OFF_IDX, "output staging (one set)");
    static_assert(!CS || (NS == 1 && D == 512 && NHW == 4 && (size_t)WAVES * HP * (D / NHW) * 2 <= (size_t)OFF_IDX),
                  "column split: one set of 4 head waves at D = 512");
    static_assert(RPW % 4 == 0 && (RS % 16) == 0, "shape");
};

// max / sum over the four lanes l, l^16, l^32, l^48 (same head in the MFMA
// result layout), on the gfx950 lane swaps (v_permlane16_swap /
// v_permlane32_swap: with both operands v, the pair returned is (v of the
// lower lane, v of the upper lane) of {l, l^16} or {l, l^32}), so every lane
// of a group adds the same two values in the same order
// (v_max_f32 written out: the values are never NaN, and fmaxf would first
// canonicalize both operands, two more instructions)
__device__ __forceinline__ float max_nn(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float pair_max16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max4x16(float v) { return pair_max32(pair_max16(v)); }
__device__ __forceinline__ float sum4x16(float v) { return pair_sum32(pair_sum16(v)); }

// the value of lane l ^ 1 (DPP quad permute 1, 0, 3, 2)
__device__ __forceinline__ float lane_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
}

// e4m3 scale byte (E4M3FN code of a positive finite scale) as binary32.
__device__ __forceinline__ float e4m3_code_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, mt = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (mt << 20)) : (float)mt * 0x1p-9f;
}

// PK: rows_b is the packed latent cache (sckv_rope_quant_pack / sckv_quant_pack
// in SCKV_FP4_E4M3_B16: codes [rb][D/2] bytes at rows_b, e4m3 scale bytes
// [rb][D/16] at rb_scales); D = 512 only.  A packed row's 256 code bytes and
// 32 scale bytes are copied into the last 288 bytes of its 2 D + 32-byte stage
// slot, and the wave that copied it expands it in place to the bf16 row
// (codes x scale, exact) before the chunk's barrier.
template <int D, int NHW, int CPS, int NS, bool CS, bool PK>
__device__ __forceinline__ void sparse_attn_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rows_a, int64_t ra,
    const uint16_t* __restrict__ rows_b, int64_t rb, const int32_t* __restrict__ idx, int T,
    const float* __restrict__ sink_all, float scale_log2, int64_t m, int HS, int chunks_per_split, int nsplit,
    uint16_t* __restrict__ out_all, float* __restrict__ part_o, float* __restrict__ part_ml,
    const uint8_t* __restrict__ rb_scales, const uint32_t vb, const int h0 = 0) {
    using S = AttnShape<D, NHW, CPS, NS, CS>;
    // this workgroup's heads: h0 .. h0 + H - 1 of the query's HS (at most 16 NHW)
    const int H = (HS - h0) < 16 * NHW ? (HS - h0) : 16 * NHW;
    const float* __restrict__ sink = sink_all + h0;
    uint16_t* __restrict__ out = out_all + (int64_t)h0 * D;  // row (qi, h0 + r) at out + (qi HS + r) D
    static_assert(!PK || D == 512, "packed rows_b at D = 512 only");
    constexpr int PKB = D / 2 + D / 16;  // packed bytes of a row (codes, then scale bytes)
    constexpr int PKO = S::RS - PKB;     // where they land in the row's stage slot
    constexpr int NTH = S::WAVES * 64;
    extern __shared__ __align__(16) unsigned char lds[];
    int32_t* idx_l = reinterpret_cast<int32_t*>(lds + S::OFF_IDX);
    const uint32_t lds0 = lds_offset(lds);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int set = NS == 2 ? wave / NHW : 0;  // chunk parity this wave computes
    const int hw = wave % NHW;   // heads 16 hw .. 16 hw + 15
    const int l16 = lane & 15;
    const int g = lane >> 4;
    const int64_t qi = vb / (uint32_t)nsplit;
    const int split = (int)(vb - qi * nsplit);
    const int64_t b = (uint32_t)qi / (uint32_t)m;  // query counts are below 2^31 (checked at launch)
    const uint16_t* rows_a_b = rows_a + b * ra * D;
    const uint16_t* rows_b_b = (rows_b && !PK) ? rows_b + b * rb * D : nullptr;
    const uint8_t* codes_b = PK ? reinterpret_cast<const uint8_t*>(rows_b) + b * rb * (D / 2) : nullptr;
    const uint8_t* scl_b = PK ? rb_scales + b * rb * (D / 16) : nullptr;
    const int32_t* idx_q = idx + qi * (int64_t)T;
    const uint16_t* qrow = q + (qi * (int64_t)HS + h0) * D;

    const int nchunks = (T + CHUNK - 1) / CHUNK;
    const int c_begin = split * chunks_per_split;
    int c_end = c_begin + chunks_per_split;
    c_end = c_end < nchunks ? c_end : nchunks;
    const int nch = c_end - c_begin;
    const uint32_t rab = (uint32_t)(ra + rb);
    // this workgroup's slice of the index list: loaded first (the first row
    // copies need it), q right behind it, so that q's latency overlaps the
    // index staging and the first copies
    const int e0 = c_begin * CHUNK;
    const int ne = (c_end * CHUNK < T ? c_end * CHUNK : T) - e0;
    // (every load address is clamped into its array rather than branched
    // around, so the loads issue back to back and only their consumers wait)
    // (only the rounds of NTH entries that reach into this slice: a uniform bound)
    // (16-byte pieces when T is a multiple of 4: the slice then starts and
    // ends on a piece boundary; else one entry a load)
    const bool vec4 = (T & 3) == 0;
    constexpr int IPT4 = (S::IPT + 3) / 4;
    int32_t iv_reg[S::IPT];
    int4 iv4[IPT4];
    if (vec4) {
#pragma unroll
        for (int k = 0; k < IPT4; ++k) {
            const int i0 = ((int)threadIdx.x + k * NTH) * 4;
            if (k * NTH * 4 < nch * CHUNK) iv4[k] = *reinterpret_cast<const int4*>(idx_q + e0 + (i0 < ne ? i0 : ne - 4));
        }
    } else {
#pragma unroll
        for (int k = 0; k < S::IPT; ++k) {
            const int i = (int)threadIdx.x + k * NTH;
            if (k * NTH < nch * CHUNK) iv_reg[k] = idx_q[e0 + (i < ne ? i : ne - 1)];
        }
    }
    asm volatile("" ::: "memory");  // keep every index load ahead of the q loads

    // ---- Q^T in B layout: head 16 hw + l16, dims ks*32 + g*8 + 0..7.  Lanes
    // of padding heads (head >= H) follow head H - 1; nothing of theirs is
    // written out.
    const int head = 16 * hw + l16;  // the head this lane follows in the softmax
    const int hq = head < H ? head : H - 1;
    bf16x8 qb[S::KS];
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) qb[ks] = as_bf16x8(load16(qrow + (int64_t)hq * D + ks * 32 + g * 8));
    // the sink logits of the wave's 16 heads by uniform (scalar) loads, lane
    // l16 keeping head 16 hw + l16's
    float sk = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float si = sink[(16 * hw + i) < H ? (16 * hw + i) : H - 1];
        sk = (l16 == i) ? si : sk;
    }
    float m_run = sk * LOG2E;  // base-2 running max, starting at the sink
    // e^(sink - M) at M = sink, counted once: by the first set of an unsplit query
    float l_run = (nsplit == 1 && set == 0) ? 1.0f : 0.0f;

    // the index slice into LDS, with one flag per chunk that names a valid row
    // (a ballot covers 64 entries, two chunks)
    uint8_t* flag_l = lds + S::OFF_FLAG;
    if (vec4) {
        // a wave's 64 pieces are 8 chunks; a chunk's flag is the OR of its 8 pieces
#pragma unroll
        for (int k = 0; k < IPT4; ++k) {
            if (k * NTH * 4 >= nch * CHUNK) break;
            const int i0 = ((int)threadIdx.x + k * NTH) * 4;
            int4 v = iv4[k];
            if (i0 >= ne) v = int4{-1, -1, -1, -1};
            if (i0 < nch * CHUNK) *reinterpret_cast<int4*>(idx_l + i0) = v;
            const bool any = i0 < nch * CHUNK && ((uint32_t)v.x < rab || (uint32_t)v.y < rab ||
                                                   (uint32_t)v.z < rab || (uint32_t)v.w < rab);
            const uint64_t bal = __ballot(any);
            const int c0 = (k * NTH + wave * 64) / 8;
            if (lane < 8 && c0 + lane < CPS) flag_l[c0 + lane] = (uint8_t)(((bal >> (8 * lane)) & 0xffull) != 0);
        }
    }
#pragma unroll
    for (int k = 0; k < S::IPT; ++k) {
        if (vec4 || k * NTH >= nch * CHUNK) break;  // chunks past nch: their flags are never read
        const int i = (int)threadIdx.x + k * NTH;
        const int32_t v = (i < ne) ? iv_reg[k] : -1;
        if (i < nch * CHUNK) idx_l[i] = v;
        const uint64_t bal = __ballot(i < nch * CHUNK && (uint32_t)v < rab);
        const int c0 = (k * NTH + wave * 64) / CHUNK;
        if (lane == 0) {
            flag_l[c0] = (uint8_t)((bal & 0xffffffffull) != 0);
            flag_l[c0 + 1] = (uint8_t)((bal >> 32) != 0);
        }
    }
    __syncthreads();

    // Non-empty chunks as a bitmap (uniform): bit j set when chunk c_begin + j
    // names at least one valid row.  Empty chunks are neither copied nor
    // computed.  Non-empty chunk number k goes to set k % 2.
    // up to 128 bits as two words (chunks 0-63, 64-127)
    struct Bits {
        uint64_t lo, hi;
    };
    const Bits todo = {__ballot(lane < nch && flag_l[lane] != 0),
                       CPS > 64 ? __ballot(lane + 64 < nch && flag_l[lane + 64] != 0) : 0ull};
    const int n = __builtin_popcountll(todo.lo) + __builtin_popcountll(todo.hi);
    const int n_own = NS == 1 ? n : ((n > set) ? (n - set + 1) / 2 : 0);  // chunks of this wave's set
    const int n_it = NS == 1 ? n : (n + 1) / 2;                           // iterations (same in every wave)
    auto drop_lowest = [](Bits& bits) {
        if (bits.lo)
            bits.lo &= bits.lo - 1;
        else
            bits.hi &= bits.hi - 1;
    };
    // this set's chunks in order: take one bit, skip the other set's next one
    auto next_own = [&](Bits& bits) -> int {
        const int j = bits.lo ? __builtin_ctzll(bits.lo) : 64 + __builtin_ctzll(bits.hi);
        drop_lowest(bits);
        if (NS == 2 && (bits.lo | bits.hi)) drop_lowest(bits);
        return j;
    };
    Bits ib = todo, cb = todo;
    if (NS == 2 && set == 1 && (ib.lo | ib.hi)) {
        drop_lowest(ib);
        drop_lowest(cb);
    }

    // Copy this wave's RPW rows of chunk j into stage `slot` of its set.
    // Invalid entries of a partly valid chunk copy this query's first q row
    // instead (finite data; their weights are zero).
    const uint16_t* rows_b_sh = rows_b_b ? rows_b_b - ra * D : rows_a_b;  // + iv*D == rows_b[iv - ra]
    auto issue = [&](int slot, int j) {
        const int32_t* ic = idx_l + j * CHUNK + hw * S::RPW;
        const uint32_t st = lds0 + (uint32_t)((set * S::NST + slot) * S::STAGE);
        if constexpr (D == 512) {
            // the rows' source addresses as a lane vector (lane r < RPW holds
            // row r's), computed once; each copy then takes two lane reads, its
            // LDS address and the copy (5 wait states between a lane read
            // writing a scalar register and a memory instruction reading it)
            const uint32_t iv = (uint32_t)ic[lane & (S::RPW - 1)];
            const uint16_t* base = (iv < (uint32_t)ra) ? rows_a_b : rows_b_sh;
            // PK: a packed row's codes and scale bytes (rows_b rows only)
            const bool pk = PK && iv >= (uint32_t)ra && iv < rab;
            const uint64_t addr = pk ? (uint64_t)(codes_b + (size_t)(iv - (uint32_t)ra) * (D / 2))
                                     : (uint64_t)((iv < rab) ? base + (size_t)iv * D : qrow);
            const uint64_t saddr = pk ? (uint64_t)(scl_b + (size_t)(iv - (uint32_t)ra) * (D / 16)) : 0ull;
#pragma unroll
            for (int rr = 0; rr < S::RPW; ++rr) {
                const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)addr, rr);
                const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(addr >> 32), rr);
                const uint32_t lb = st + (uint32_t)((hw * S::RPW + rr) * S::RS);
                if (PK && __builtin_amdgcn_readlane((int)pk, rr)) {
                    // 16 lanes copy the 256 code bytes, 2 lanes the 32 scale
                    // bytes, into the slot's last 288 bytes
                    const uint32_t slo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)saddr, rr);
                    const uint32_t shi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(saddr >> 32), rr);
                    if (lane < D / 32)
                        asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                                     :
                                     : "v"((uint32_t)lane * 16u), "s"((const void*)(((uint64_t)hi << 32) | lo)),
                                       "s"(lb + (uint32_t)PKO)
                                     : "memory", "m0");
                    if (lane < D / 256)
                        asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                                     :
                                     : "v"((uint32_t)lane * 16u), "s"((const void*)(((uint64_t)shi << 32) | slo)),
                                       "s"(lb + (uint32_t)(PKO + D / 2))
                                     : "memory", "m0");
                    continue;
                }
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                             :
                             : "v"((uint32_t)lane * 16u), "s"((const void*)(((uint64_t)hi << 32) | lo)), "s"(lb)
                             : "memory", "m0");
            }
            return;
        }
        int32_t ivv[S::RPW];
#pragma unroll
        for (int v4 = 0; v4 < S::RPW / 4; ++v4) {
            const int4 t4 = *reinterpret_cast<const int4*>(ic + 4 * v4);
            ivv[4 * v4 + 0] = t4.x;
            ivv[4 * v4 + 1] = t4.y;
            ivv[4 * v4 + 2] = t4.z;
            ivv[4 * v4 + 3] = t4.w;
        }
#pragma unroll
        for (int rr = 0; rr < S::RPW; ++rr) {
            const uint32_t iv = (uint32_t)__builtin_amdgcn_readfirstlane(ivv[rr]);
            const uint16_t* base = (iv < (uint32_t)ra) ? rows_a_b : rows_b_sh;
            const uint16_t* src = (iv < rab) ? base + (size_t)iv * D : qrow;
            if (lane < D / 8) dma16_s(src, (uint32_t)lane * 16u, st + (uint32_t)((hw * S::RPW + rr) * S::RS));
        }
    };

    // PK: expand this wave's packed rows of chunk j (stage at stp) in place:
    // lane (row 4 rho + lane / 16, piece k = lane % 16) turns the 16 code
    // bytes of values 32 k .. 32 k + 31 (blocks 2k, 2k + 1) into 64 bf16
    // bytes at the start of the row; every lane reads before any lane writes
    // (the writes need the read values), so the overlap of the last pieces'
    // outputs with the packed bytes is harmless.
    auto expand = [&](const unsigned char* stp, int j) {
        if constexpr (PK) {
            unsigned char* stw = const_cast<unsigned char*>(stp);
#pragma unroll
            for (int rho = 0; rho < S::RPW / 4; ++rho) {
                const int rr = 4 * rho + (lane >> 4);
                const int k = lane & 15;
                const uint32_t iv = (uint32_t)idx_l[j * CHUNK + hw * S::RPW + rr];
                if (iv >= (uint32_t)ra && iv < rab) {
                    unsigned char* row = stw + (hw * S::RPW + rr) * S::RS;
                    const u32x4 c = *reinterpret_cast<const u32x4*>(row + PKO + 16 * k);
                    const uint32_t sb = *reinterpret_cast<const uint16_t*>(row + PKO + D / 2 + 2 * k);
                    asm volatile("" ::: "memory");
                    const float s0 = e4m3_code_to_f32(sb & 0xffu), s1 = e4m3_code_to_f32(sb >> 8);
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const float sc = d < 2 ? s0 : s1;
                        // byte by of code word d: values 32 k + 8 d + 2 by (low nibble) and + 1;
                        // the products have at most 6 significant bits, so they and the
                        // bf16 packing are exact
                        const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[d], 1.0f, 0);
                        const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[d], 1.0f, 1);
                        const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[d], 1.0f, 2);
                        const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c[d], 1.0f, 3);
                        u32x4 ov;
                        ov[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v0[0] * sc, v0[1] * sc}, bf16x2));
                        ov[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v1[0] * sc, v1[1] * sc}, bf16x2));
                        ov[2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v2[0] * sc, v2[1] * sc}, bf16x2));
                        ov[3] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v3[0] * sc, v3[1] * sc}, bf16x2));
                        *reinterpret_cast<u32x4*>(row + 64 * k + 16 * d) = ov;
                    }
                }
            }
        } else {
            (void)stp;
            (void)j;
        }
    };

    f32x4 o[S::NT];
#pragma unroll
    for (int nt = 0; nt < S::NT; ++nt) o[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 pa;          // this chunk's probabilities, A operand of P . R
    float alpha = 1.0f; // rescale factor of the last max move (head of this lane)

    if (n_own > 0) issue(0, next_own(ib));

    // ---- chunk loop.  The inner loop never applies vector ALU work to O (so O
    // stays in accumulation registers); it leaves when one of the wave's heads
    // moved its running max, and the outer loop rescales O before P . R.
    int it = 0;
    bool resume = false;
    for (;;) {
        bool rescale = false;
        for (; it < n_it; ++it) {
            const unsigned char* stp = lds + (set * S::NST + (it & 1)) * S::STAGE;
            if (!resume) {
                wait_vmcnt<0>();  // this wave's copies of its current chunk landed
                const int j = (it < n_own) ? next_own(cb) : 0;
                if (PK && it < n_own) expand(stp, j);
                __syncthreads();  // everyone's did; last iteration's stages are free
                if (it + 1 < n_own) issue((it + 1) & 1, next_own(ib));
                if (it < n_own) {
                    const uint32_t mask =
                        (uint32_t)(__ballot((uint32_t)idx_l[j * CHUNK + (lane & 31)] < rab) & 0xffffffffull);
                    // S^T for rows 0-15 and 16-31: lane holds head l16, rows mt*16 + g*4 + 0..3
                    f32x4 sp[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
                    for (int ks = 0; ks < S::KS; ++ks)
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt) {
                            const bf16x8 rk = *reinterpret_cast<const bf16x8*>(stp + (mt * 16 + l16) * S::RS +
                                                                               ks * 64 + g * 16);
                            sp[mt] = mfma16x16x32(rk, qb[ks], sp[mt]);
                        }
                    {
                        // schedule: SA operand reads ahead of the products, then
                        // one read per product
                        constexpr int SA = 2 * S::KS < 6 ? 2 * S::KS : 6;
                        __builtin_amdgcn_sched_group_barrier(0x100, SA, 0);
#pragma unroll
                        for (int k2 = 0; k2 < 2 * S::KS - SA; ++k2) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        }
                        __builtin_amdgcn_sched_group_barrier(0x008, SA, 0);
                    }
                    float x[8];
#pragma unroll
                    for (int k8 = 0; k8 < 8; ++k8) x[k8] = sp[k8 >> 2][k8 & 3];  // raw products
                    if (mask != 0xffffffffu) {
                        // rows that name no valid entry (chunks at the ends of a
                        // list only) drop out of the softmax
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (!((mask >> (mt * 16 + g * 4 + i)) & 1u)) x[mt * 4 + i] = -INFINITY;
                    }
                    float cmax = -INFINITY;
#pragma unroll
                    for (int k8 = 0; k8 < 8; ++k8) cmax = fmaxf(cmax, x[k8]);
                    // (the scale is positive and rounding is monotone, so this is
                    // exactly the largest scaled logit)
                    cmax = max4x16(cmax) * scale_log2;
                    const float m_new = (cmax > m_run + STALE_MAX) ? cmax : m_run;
                    alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                    float psum = 0.0f;
                    uint32_t pk[4];
                    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
                    for (int j2 = 0; j2 < 4; ++j2) {
                        // hardware exp2 (v_exp_f32) and round-to-nearest-even pack to
                        // bf16 (v_cvt_pk_bf16_f32); the sum uses the rounded weights,
                        // two at a time through the bf16 dot product with (1, 1)
                        // (the logit scale and the max in one multiply-add)
                        const f32x2 pf = {__builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * j2], scale_log2, -m_new)),
                                          __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * j2 + 1], scale_log2, -m_new))};
                        const bf16x2 pbv = __builtin_convertvector(pf, bf16x2);
                        psum = __builtin_amdgcn_fdot2_f32_bf16(pbv, ones, psum, false);
                        pk[j2] = __builtin_bit_cast(uint32_t, pbv);
                    }
                    l_run = l_run * alpha + sum4x16(psum);
                    const bool moved = __ballot(m_new != m_run) != 0;
                    m_run = m_new;
                    pa = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
                    if constexpr (CS) {
                        // publish this wave's probabilities and, when one of its
                        // heads moved its running max, the factors (lanes 0..15
                        // hold heads 16 hw + l16)
                        *reinterpret_cast<bf16x8*>(lds + S::OFF_P + (hw * 64 + lane) * 16) = pa;
                        if (lane == 0) lds[S::OFF_MOVED + hw] = moved ? 1 : 0;
                        if (moved && g == 0)
                            reinterpret_cast<float*>(lds + S::OFF_ALPHA)[16 * hw + l16] = alpha;
                    } else if (moved) {
                        rescale = true;
                        break;
                    }
                }
            }
            resume = false;
            if (CS && it < n_own) {
                // column split: after every wave has published its
                // probabilities, wave hw accumulates O for all 64 heads over
                // columns 128 hw .. 128 hw + 127, transposed (O^T = R^T . P^T,
                // the same operand registers in swapped roles): accumulator
                // 8 hg + ct holds head 16 hg + l16, columns 128 hw + 16 ct +
                // g*4 + i, four consecutive columns of one head a lane
                __syncthreads();
                const uint32_t mv = *reinterpret_cast<const uint32_t*>(lds + S::OFF_MOVED);
                if (mv) {  // rare: rescale the head groups whose running max moved
                    const float* al = reinterpret_cast<const float*>(lds + S::OFF_ALPHA);
#pragma unroll
                    for (int hg = 0; hg < NHW; ++hg) {
                        if (((mv >> (8 * hg)) & 0xffu) == 0) continue;
                        const float a1 = al[16 * hg + l16];
#pragma unroll
                        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                            for (int i = 0; i < 4; ++i) o[hg * 8 + ct][i] *= a1;
                    }
                }
                bf16x8 pall[NHW];
#pragma unroll
                for (int hg = 0; hg < NHW; ++hg)
                    pall[hg] = *reinterpret_cast<const bf16x8*>(lds + S::OFF_P + (hg * 64 + lane) * 16);
                const int jj = l16 >> 2;
                const int c4 = 4 * (l16 & 3);
#pragma unroll
                for (int ct = 0; ct < 8; ++ct) {
                    const unsigned char* pc = stp + (hw * 128 + ct * 16 + c4) * 2;
                    const i16x4 lo = lds_read_tr16(pc + (g * 4 + jj) * S::RS);
                    const i16x4 hi = lds_read_tr16(pc + (16 + g * 4 + jj) * S::RS);
                    const bf16x8 bv =
                        __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int hg = 0; hg < NHW; ++hg) o[hg * 8 + ct] = mfma16x16x32(bv, pall[hg], o[hg * 8 + ct]);
                }
            } else if (it < n_own) {
                // O[heads, :] += P . R: k = g*8 + 0..3 are rows g*4 + 0..3, k = g*8 + 4..7
                // rows 16 + g*4 + 0..3 (the order the probabilities sit in)
                // accumulator nt of set 1 holds the 16 columns of tile nt ^ NT/2
                // (so that both sets finish accumulators 0 .. NT/2 - 1 at the end)
                const int jj = l16 >> 2;
                const int c4 = 4 * (l16 & 3);
                const unsigned char* pv_lo = stp + set * (S::NT / 2) * 32;        // nt < NT/2
                const unsigned char* pv_hi = stp + (1 - set) * (S::NT / 2) * 32;  // nt >= NT/2
#pragma unroll
                for (int nt = 0; nt < S::NT; ++nt) {
                    const unsigned char* pc = (nt < S::NT / 2 ? pv_lo + nt * 32 : pv_hi + (nt - S::NT / 2) * 32) + c4 * 2;
                    const i16x4 lo = lds_read_tr16(pc + (g * 4 + jj) * S::RS);
                    const i16x4 hi = lds_read_tr16(pc + (16 + g * 4 + jj) * S::RS);
                    const bf16x8 bv =
                        __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[nt] = mfma16x16x32(pa, bv, o[nt]);
                }
            }
        }
        if (!rescale) break;
        // rare: a running max moved by more than the slack; O rows are heads
        // 16 hw + g*4 + i, whose factors sit in lanes g*4 + i
        float a4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, g * 4 + i, 64);
#pragma unroll
        for (int nt = 0; nt < S::NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[nt][i] *= a4[i];
        resume = true;
    }

    if constexpr (CS) {
        // ---- epilogue, column split: 1/sum of each head from its owner
        // wave, then each wave normalizes its 64 heads x 128 columns into
        // its own staging rows (bf16, 256 bytes a row, 16-byte pieces
        // swizzled by the row; a lane's four columns of one head as 8
        // bytes) and writes them out as 16-byte pieces
        __syncthreads();  // all stages idle
        float* il = reinterpret_cast<float*>(lds + S::OFF_ALPHA);
        if (g == 0) il[16 * hw + l16] = 1.0f / l_run;
        __syncthreads();
        constexpr int PR = (D / NHW) * 2;  // bytes of a staged row (128 columns)
        constexpr int NPC = PR / 16;       // 16-byte pieces a row
        unsigned char* stg = lds + (size_t)wave * (S::HP * PR);
#pragma unroll
        for (int hg = 0; hg < NHW; ++hg) {
            const int r = 16 * hg + l16;
            const float fin = il[r];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const f32x4 v = o[hg * 8 + ct];
                const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[0] * fin, v[1] * fin}, bf16x2));
                const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[2] * fin, v[3] * fin}, bf16x2));
                const int c = ct * 16 + g * 4;  // column within the wave's 128
                const int pc = (c >> 3) ^ (r % NPC);
                *reinterpret_cast<uint2*>(stg + r * PR + pc * 16 + (c & 7) * 2) = uint2{lo, hi};
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < S::HP * NPC / 64; ++k) {
            const int piece = k * 64 + lane;
            const int r = piece / NPC, c = piece % NPC;
            if (r < H) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * PR + ((c ^ (r % NPC)) << 4));
                store16(reinterpret_cast<unsigned char*>(out + (qi * HS + r) * (int64_t)D + hw * (D / NHW)) + c * 16, v);
            }
        }
        return;
    }
    if constexpr (NS == 1) {
        // ---- epilogue, one set (unsplit lists only): no merge; each wave
        // normalizes its 16 heads over the whole head dim and writes them
        // through its own staging rows (bf16, pitch 2 D + 32 bytes) as
        // 16-byte pieces.  Lanes l16 and l16 ^ 1 pair up adjacent columns.
        __syncthreads();  // all stages idle
        float fin[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fin[i] = 1.0f / __shfl(l_run, g * 4 + i, 64);
        constexpr int PF = 2 * D + 32;
        unsigned char* stg = lds + (size_t)wave * (16 * PF);
        const bool odd = (l16 & 1) != 0;
#pragma unroll
        for (int k = 0; k < S::NT; ++k)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float a = o[k][i] * fin[i], b2 = o[k][i + 1] * fin[i + 1];
                const float other = lane_xor1(odd ? a : b2);
                const f32x2 pr = odd ? f32x2{other, b2} : f32x2{a, other};
                const uint32_t pb = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
                const int r = g * 4 + i + (odd ? 1 : 0);
                const int c = k * 16 + (l16 & ~1);
                *reinterpret_cast<uint32_t*>(stg + r * PF + c * 2) = pb;
            }
        wave_lds_sync();
        constexpr int CPR = 2 * D / 16;  // 16-byte pieces of a row
        const int nrow1 = (H - 16 * hw) < 16 ? (H - 16 * hw) : 16;
#pragma unroll
        for (int k = 0; k < 16 * CPR / 64; ++k) {
            const int piece = k * 64 + lane;
            const int r = piece / CPR, c = piece % CPR;
            if (r < nrow1) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * PF + c * 16);
                store16(reinterpret_cast<unsigned char*>(out + (qi * HS + 16 * hw + r) * (int64_t)D) + c * 16, v);
            }
        }
        return;
    }

    // ---- epilogue: the two sets merge their (max, sum, O) through LDS, each
    // finishing half of the columns: set 0 tiles nt < NT/2, set 1 the rest.
    // Both hold the tiles they finish in accumulators 0 .. NT/2 - 1 and hand
    // over accumulators NT/2 .. NT - 1 (set 1 keeps tile nt ^ NT/2 in
    // accumulator nt), so no accumulator is chosen at run time.
    // The exchanged tiles sit column-major, [D][HP] floats, a lane's four
    // rows as one 16-byte piece whose place in the column is swizzled by the
    // column (the 16 lanes of a group then cover every bank once).
    constexpr int NH = S::NT / 2;
    constexpr int HQ = S::HP / 4;  // 16-byte pieces of a column
    __syncthreads();  // all stages idle
    unsigned char* xo = lds;                                     // [D][HP] f32
    float* ml = reinterpret_cast<float*>(lds + S::OFF_IDX);     // [2][HP][2] (the index slice is done)
    auto xo_at = [&](int col) -> unsigned char* {
        return xo + (size_t)col * S::HP * 4 + (size_t)(((4 * hw + g) ^ (col % HQ)) * 16);
    };
#pragma unroll
    for (int k = 0; k < NH; ++k) {
        const int tile = (set == 0) ? NH + k : k;  // the other set's tiles
        *reinterpret_cast<f32x4*>(xo_at(tile * 16 + l16)) = o[NH + k];
    }
    if (g == 0) {
        ml[(set * S::HP + head) * 2 + 0] = m_run;
        ml[(set * S::HP + head) * 2 + 1] = l_run;
    }
    __syncthreads();
    const float m1 = ml[((1 - set) * S::HP + head) * 2 + 0], l1 = ml[((1 - set) * S::HP + head) * 2 + 1];
    const float M = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - M), a1 = __builtin_amdgcn_exp2f(m1 - M);
    const float L = l_run * a0 + l1 * a1;
    // per O row (head 16 hw + g*4 + i): the factors from lane g*4 + i
    float f0[4], f1[4], fin[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f0[i] = __shfl(a0, g * 4 + i, 64);
        f1[i] = __shfl(a1, g * 4 + i, 64);
        fin[i] = (nsplit == 1) ? 1.0f / __shfl(L, g * 4 + i, 64) : 1.0f;
    }
    float fo[NH][4];  // this wave's finished tiles
#pragma unroll
    for (int k = 0; k < NH; ++k) {
        const int tile = (set == 0) ? k : NH + k;
        const f32x4 ot = *reinterpret_cast<const f32x4*>(xo_at(tile * 16 + l16));
#pragma unroll
        for (int i = 0; i < 4; ++i) fo[k][i] = (o[k][i] * f0[i] + ot[i] * f1[i]) * fin[i];
    }
    __syncthreads();  // every read of the exchanged tiles is done
    // stage the 16 x D/2 block in LDS (wave-private space), then write it out
    // 16 bytes a lane
    const int nrow = (H - 16 * hw) < 16 ? (H - 16 * hw) : 16;  // rows that are real heads
    const int col0 = set * (D / 2);
    if (nsplit == 1) {
        // bf16 rows of D bytes at a pitch of D + 32 (the 8 rows one write
        // touches fall on distinct banks); lanes l16 and l16 ^ 1 pair up
        // adjacent columns, so that each writes two values (4 bytes)
        constexpr int P = D + 32;
        unsigned char* stg = lds + (size_t)wave * (16 * P);
        const bool odd = (l16 & 1) != 0;
#pragma unroll
        for (int k = 0; k < NH; ++k)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float other = lane_xor1(odd ? fo[k][i] : fo[k][i + 1]);
                const f32x2 pr = odd ? f32x2{other, fo[k][i + 1]} : f32x2{fo[k][i], other};
                const uint32_t pb = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
                const int r = g * 4 + i + (odd ? 1 : 0);
                const int c = k * 16 + (l16 & ~1);
                *reinterpret_cast<uint32_t*>(stg + r * P + c * 2) = pb;
            }
        wave_lds_sync();
        constexpr int CPRW = D / 16;  // 16-byte pieces of a half row
#pragma unroll
        for (int k = 0; k < 16 * CPRW / 64; ++k) {
            const int piece = k * 64 + lane;
            const int r = piece / CPRW, c = piece % CPRW;
            if (r < nrow) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * P + c * 16);
                store16(reinterpret_cast<unsigned char*>(out + (qi * HS + 16 * hw + r) * (int64_t)D + col0) + c * 16, v);
            }
        }
    } else {
        // f32 partial half rows (2 D bytes each, 16-byte pieces swizzled by
        // the row), then (max, sum) per head
        constexpr int CPRW = 2 * D / 16;  // 16-byte pieces of a half row
        constexpr int SWR = CPRW < 16 ? CPRW : 16;
        unsigned char* stg = lds + (size_t)wave * (16 * 2 * D);
#pragma unroll
        for (int k = 0; k < NH; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = g * 4 + i, c = k * 16 + l16;
                *reinterpret_cast<float*>(stg + r * (2 * D) + (((c >> 2) ^ (r % SWR)) << 4) + (c & 3) * 4) = fo[k][i];
            }
        wave_lds_sync();
        const int64_t pbase = (qi * nsplit + split) * (int64_t)HS + h0 + 16 * hw;
#pragma unroll
        for (int k = 0; k < 16 * CPRW / 64; ++k) {
            const int piece = k * 64 + lane;
            const int r = piece / CPRW, c = piece % CPRW;
            if (r < nrow) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * (2 * D) + ((c ^ (r % SWR)) << 4));
                store16(reinterpret_cast<unsigned char*>(part_o + (pbase + r) * D + col0) + c * 16, v);
            }
        }
        if (set == 0 && g == 0 && l16 < nrow) {
            part_ml[(pbase + l16) * 2 + 0] = M;
            part_ml[(pbase + l16) * 2 + 1] = L;
        }
    }
}

// Merge the nsplit partials of each (query, head): M = max(sink, m_j),
// Z = e^(sink - M) + sum_j l_j e^(m_j - M), o = sum_j O_j e^(m_j - M) / Z (base 2).
constexpr int COMBINE_THREADS = 256;
// LDS bytes the combine of one (query, head) needs with NTH threads: the
// split weights, the reduction words and the column sums of the split groups.
// (1024 / D split groups of D columns; 16 bytes of alignment)
constexpr size_t combine_lds_bytes(int NTH, int nsplit) { return (size_t)(nsplit + 2 * (NTH / 64) + 1024 + 4) * 4u; }

// Merge the nsplit partials of one (query, head) (log-sum-exp, the sink
// logit once):  M = max(sink, m_j),  Z = e^(sink - M) + sum_j l_j e^(m_j - M),
// out = sum_j O_j e^(m_j - M) / Z, in base 2.  The weights e^(m_j - M) are
// computed once into LDS; then G = 1024 / D groups of D/4 threads each sum 4
// columns (16-byte loads) over every G-th split, and the groups' sums meet in
// LDS.  G does not depend on NTH (threads past 256 idle in that part), so
// every workgroup size rounds the same way.  NTH >= 256 threads, D in 64..512,
// dynamic LDS of combine_lds_bytes(NTH, nsplit).
template <int NTH>
__device__ __forceinline__ void combine_body(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                             const float* __restrict__ sink, int nsplit, int H, int D,
                                             uint16_t* __restrict__ out, const int64_t qi, const int h) {
    extern __shared__ __align__(16) unsigned char lds[];
    float* wj = reinterpret_cast<float*>(lds);  // [nsplit]
    float* red = wj + nsplit;                   // [2][NTH / 64]
    float* colsum = red + 2 * (NTH / 64);       // [groups][D]
    colsum = reinterpret_cast<float*>((reinterpret_cast<uintptr_t>(colsum) + 15) & ~(uintptr_t)15);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    static_assert(NTH >= 256 && NTH % 64 == 0, "combine workgroup");
    const int per = D / 4;            // threads of a split group (4 columns each)
    const int groups = 1024 / D;      // split groups
    const int grp = tid / per, c4 = tid - grp * per;
    // this thread's splits are grp, grp + groups, ...: the first PRE of them
    // are requested before the weights are known (one memory round trip
    // instead of two), the rest where they are summed
    constexpr int PRE = 8;
    const int n_own = grp < groups && grp < nsplit ? (nsplit - grp + groups - 1) / groups : 0;
    const f32x4* po = reinterpret_cast<const f32x4*>(part_o + (qi * nsplit * H + h) * (int64_t)D) + c4;
    const int64_t stride4 = (int64_t)H * D / 4;  // one split further
    f32x4 pv[PRE];
#pragma unroll
    for (int kk = 0; kk < PRE; ++kk)
        pv[kk] = kk < n_own ? po[(grp + kk * groups) * stride4] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float s2 = sink[h] * LOG2E;
    const float* ml = part_ml + (qi * nsplit * H + h) * 2;  // split j at ml[j * H * 2]
    float mx = s2;
    for (int j = tid; j < nsplit; j += NTH) mx = fmaxf(mx, ml[(int64_t)j * H * 2]);
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float M = red[0];
    for (int i = 1; i < NTH / 64; ++i) M = fmaxf(M, red[i]);
    float z = 0.0f;
    for (int j = tid; j < nsplit; j += NTH) {
        const float e = exp2f(ml[(int64_t)j * H * 2] - M);
        wj[j] = e;
        z += ml[(int64_t)j * H * 2 + 1] * e;
    }
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o, 64);
    if (lane == 0) red[NTH / 64 + wave] = z;
    __syncthreads();
    float Z = exp2f(s2 - M);
    for (int i = 0; i < NTH / 64; ++i) Z += red[NTH / 64 + i];
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (grp < groups) {
        // the sums in a fixed order: fours of splits while four remain, then
        // one at a time (the preloaded ones first, in the same order)
        int k = 0;
#pragma unroll
        for (int qd = 0; qd < PRE / 4; ++qd) {
            if (k == 4 * qd && 4 * qd + 3 < n_own) {
                const int j = grp + 4 * qd * groups;
                acc += pv[4 * qd] * wj[j] + pv[4 * qd + 1] * wj[j + groups] + pv[4 * qd + 2] * wj[j + 2 * groups] +
                       pv[4 * qd + 3] * wj[j + 3 * groups];
                k += 4;
            }
        }
        if (k < PRE) {  // the fours ended inside the preloaded splits: so do all of them
#pragma unroll
            for (int kk = 0; kk < PRE; ++kk)
                if (kk >= k && kk < n_own) acc += pv[kk] * wj[grp + kk * groups];
            k = n_own;
        }
        int j = grp + k * groups;
        for (; j + 3 * groups < nsplit; j += 4 * groups) {  // four loads in flight
            const f32x4 v0 = po[j * stride4], v1 = po[(j + groups) * stride4];
            const f32x4 v2 = po[(j + 2 * groups) * stride4], v3 = po[(j + 3 * groups) * stride4];
            acc += v0 * wj[j] + v1 * wj[j + groups] + v2 * wj[j + 2 * groups] + v3 * wj[j + 3 * groups];
        }
        for (; j < nsplit; j += groups) acc += po[j * stride4] * wj[j];
        *reinterpret_cast<f32x4*>(colsum + grp * D + 4 * c4) = acc;
    }
    __syncthreads();
    const float invZ = 1.0f / Z;
    for (int d = tid; d < D; d += NTH) {
        float sum = 0.0f;
        for (int g = 0; g < groups; ++g) sum += colsum[g * D + d];
        out[(qi * H + h) * (int64_t)D + d] = (uint16_t)f32_to_bf16_bits(sum * invZ);
    }
}

// (host)
// Chunks per workgroup: split a query's chunks only when the queries alone do
// not give about one workgroup per compute unit.
void attn_split(int64_t nq, int T, int* chunks_per_split, int* nsplit) {
    const int nchunks = (T + CHUNK - 1) / CHUNK;
    int64_t want = (256 + nq - 1) / nq;
    if (want > nchunks) want = nchunks;
    if (want < 1) want = 1;
    int cps = (int)((nchunks + want - 1) / want);
    // at least MIN_SPLIT_CHUNKS chunks a workgroup: every split writes H x D
    // f32 partials that the combine reads back, which at one chunk a
    // workgroup cost more than the chunk itself (measured, decode at B = 1)
    if (cps < MIN_SPLIT_CHUNKS) cps = nchunks < MIN_SPLIT_CHUNKS ? nchunks : MIN_SPLIT_CHUNKS;
    if (cps > MAX_CPS) cps = MAX_CPS;
    *chunks_per_split = cps;
    *nsplit = (nchunks + cps - 1) / cps;
}

// Bytes of the split partials: [nq][nsplit][H][D] f32 O, then [nq][nsplit][H]
// (max, sum) pairs, each part 256-byte aligned; 0 without a split.
size_t attn_partials_bytes(int64_t nq, int nsplit, int H, int D) {
    if (nsplit <= 1) return 0;
    size_t bytes = (size_t)nq * (size_t)nsplit * (size_t)H * (size_t)D * 4u;
    bytes = (bytes + 255u) & ~(size_t)255u;
    bytes += (size_t)nq * (size_t)nsplit * (size_t)H * 2u * 4u;
    return (bytes + 255u) & ~(size_t)255u;
}

// Split of the attention call when the queries alone do not give a quarter of
// a workgroup per compute unit: the heads go to ceil(H / 16) workgroups of 16
// heads each (two waves, one chunk a set at a time), and the chunks to ranges
// of at least 2 (one per set), so that a query's work spreads over about 256
// workgroups with short chains of dependent copies.  hgroups = 1 when no split
// is needed.
inline void attn_split_groups(int64_t nq, int T, int H, int* chunks_per_split, int* nsplit, int* hgroups) {
    const int nchunks = (T + CHUNK - 1) / CHUNK;
    const int64_t want = (256 + nq - 1) / nq;  // workgroups per query
    // (from two to three workgroups a query the 64-head split is faster:
    // 16-head workgroups take 135 KB of LDS for 2 waves, one per compute unit)
    if (want < 4 || H <= 16) {
        *hgroups = 1;
        attn_split(nq, T, chunks_per_split, nsplit);
        return;
    }
    const int G = (H + 15) / 16;
    int64_t splits = (want + G - 1) / G;
    if (splits > nchunks) splits = nchunks;
    int cps = (int)((nchunks + splits - 1) / splits);
    if (cps < 2) cps = nchunks < 2 ? nchunks : 2;
    if (cps > MAX_CPS) cps = MAX_CPS;
    *hgroups = G;
    *chunks_per_split = cps;
    *nsplit = (nchunks + cps - 1) / cps;
}

}  // namespace
}  // namespace sckv

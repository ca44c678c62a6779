// attn.hip -- sparse MQA attention with a per-head sink over rows gathered
// through an index list from two row bases.
//
// Pages: "metrale_model_arch/deepseek_v41_ref/compress.rs" (attention_any:
// the sparse_attn call over [window rows | compressed rows] with scale =
// head_dim^-1/2 and the per-head sink) and "metrale_model_arch/attn_v41/
// forward.rs" (attend_and_project over rows_a / rows_b through one index
// list).  The sink is one extra logit per head in the softmax denominator with
// no value row; every row is both key and value (MQA, one shared row).
//
// Design (gfx950).  One workgroup = one query x a range of 32-row chunks of
// its index list.  All heads (padded to 32 or 64) form the MFMA M dimension,
// so every gathered row byte feeds every head.  NW waves split the head
// dimension D: wave w owns dims [w*DW, (w+1)*DW) of Q (in registers) and of O
// (in accumulators).  Per chunk:
//   1. rows arrive by asynchronous global->LDS copies (global_load_lds_dwordx4:
//      one instruction moves one whole 1 KiB row, fully coalesced), issued two
//      chunks ahead into a 3-stage ring; each wave brings in 32/NW rows;
//   2. S_w = Q[:, dims_w] . R[:, dims_w]^T on the matrix cores (B operand read
//      from the row-major stage);
//   3. the NW partial logit tiles meet in LDS; wave w sums the tiles of its own
//      HP/NW heads (fixed order) and runs the online softmax for them in base 2
//      (the running max starts at the sink logit and only moves when a logit
//      exceeds it by more than 2^8, so rescaling is rare); P goes back to LDS
//      in bf16;
//   4. every wave reads all of P (A layout) and O[:, dims_w] += P . R[:, dims_w],
//      the B operand coming from the same row-major stage through the
//      transposing LDS read (ds_read_b64_tr_b16), so no second copy of the rows.
// A query's chunks may be split over several workgroups; their partial
// (max, sum, O) are merged by a small combine kernel that adds the sink once.
#include "mfma.h"
#include "sckv_device.h"

namespace sckv {
namespace {

constexpr int CHUNK = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float STALE_MAX = 8.0f;  // base-2 slack before the running max moves
constexpr int MAX_CPS = 64;        // chunks one workgroup handles at most (its index range sits in LDS)

// MT head tiles of 32 per wave, NG head groups, NW waves per group splitting
// the head dim into slices of DW: NG * NW waves, NG * MT * 32 padded heads.
template <int MT, int NG, int DW, int NW>
struct AttnShape {
    static constexpr int WAVES = NG * NW;
    static constexpr int HG = MT * 32;             // padded heads of one group
    static constexpr int HP = NG * HG;             // padded heads
    static constexpr int D = DW * NW;
    static constexpr int KS = DW / 16;             // k-steps of Q.R^T per wave
    static constexpr int NT = DW / 32;             // 32-wide output tiles per wave
    static constexpr int RPW = CHUNK / WAVES;      // rows each wave copies in per chunk
    static constexpr int PD = (RPW <= 16) ? 2 : 1; // chunks in flight ahead of the one computed
    static constexpr int NST = PD + 1;             // stages in the ring
    static constexpr int RS = 2 * D + 32;          // bytes per row in a stage (32-byte pad: no bank conflicts)
    static constexpr int STAGE = CHUNK * RS;
    static constexpr int HW = HP / WAVES;          // heads whose softmax one wave owns
    static constexpr int LPH = 64 / HW;            // lanes per owned head
    static constexpr int VPL = CHUNK / LPH;        // logits per lane in the softmax
    static constexpr int SXS = CHUNK + 4;          // floats per head row of a partial-logit tile
    static constexpr int PS = CHUNK + 8;           // bf16 per head row of P
    static constexpr int OFF_SX = NST * STAGE;
    static constexpr int OFF_P = OFF_SX + NW * HP * SXS * 4;  // NW partial tiles per head
    static constexpr int OFF_ALPHA = OFF_P + HP * PS * 2;
    static constexpr int OFF_L = OFF_ALPHA + HP * 4;
    static constexpr int OFF_FLAG = OFF_L + HP * 4;
    static constexpr int OFF_IDX = OFF_FLAG + 4 * WAVES;
    static constexpr size_t LDS_BYTES = (size_t)OFF_IDX + (size_t)MAX_CPS * CHUNK * 4;
    static_assert(VPL % 4 == 0 && LPH >= 1 && LPH <= 16 && RPW % 4 == 0, "softmax split");
};

// Max / sum over aligned groups of G consecutive lanes (G = 1, 2, 4, 8, 16),
// every lane receiving the group's result, with DPP lane permutes (no LDS
// round trip): quad_perm swaps within 2 and 4 lanes, half-row and row mirrors
// pair the 4-lane and 8-lane halves.
template <int G>
__device__ __forceinline__ float group_max(float v) {
    if (G >= 2) v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false)));
    if (G >= 4) v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false)));
    if (G >= 8) v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false)));
    if (G >= 16) v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false)));
    return v;
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if (G >= 2) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false));
    if (G >= 4) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false));
    if (G >= 8) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false));
    if (G >= 16) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false));
    return v;
}

// Wait until at most n of this wave's row copies are in flight (n uniform, one of 0, RPW, 2*RPW).
template <int RPW>
__device__ __forceinline__ void wait_rows(int n) {
    if (n == 0)
        wait_vmcnt<0>();
    else if (n == RPW)
        wait_vmcnt<RPW>();
    else
        wait_vmcnt<(2 * RPW < 64 ? 2 * RPW : 63)>();
}

template <int MT, int NG, int DW, int NW>
__global__ __launch_bounds__(NG * NW * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rows_a, int64_t ra,
    const uint16_t* __restrict__ rows_b, int64_t rb, const int32_t* __restrict__ idx, int T,
    const float* __restrict__ sink, float scale_log2, int64_t m, int H, int chunks_per_split, int nsplit,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml) {
    using S = AttnShape<MT, NG, DW, NW>;
    constexpr int D = S::D;
    constexpr int NTH = S::WAVES * 64;
    extern __shared__ __align__(16) unsigned char lds[];
    float* sx = reinterpret_cast<float*>(lds + S::OFF_SX);
    uint16_t* pl = reinterpret_cast<uint16_t*>(lds + S::OFF_P);
    float* alpha_l = reinterpret_cast<float*>(lds + S::OFF_ALPHA);
    float* lsum_l = reinterpret_cast<float*>(lds + S::OFF_L);
    int* flags = reinterpret_cast<int*>(lds + S::OFF_FLAG);
    int32_t* idx_l = reinterpret_cast<int32_t*>(lds + S::OFF_IDX);
    const uint32_t lds0 = lds_offset(lds);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r_lane = lane & 31;  // row of this lane in B layout / head in A layout
    const int half = lane >> 5;
    const int64_t qi = blockIdx.x / nsplit;
    const int split = (int)(blockIdx.x - qi * nsplit);
    const int64_t b = qi / m;
    const int grp = wave / NW;          // head group: heads grp*HG .. grp*HG + HG-1
    const int dim0 = (wave % NW) * DW;  // head-dim slice
    const int hg0 = grp * S::HG;
    const uint16_t* rows_a_b = rows_a + b * ra * D;
    const uint16_t* rows_b_b = rows_b ? rows_b + b * rb * D : nullptr;
    const int32_t* idx_q = idx + qi * (int64_t)T;
    const uint16_t* qrow = q + qi * (int64_t)H * D;

    // ---- Q slice in A layout: head mt*32 + r_lane, dims dim0 + ks*16 + half*8 + 0..7
    bf16x8 qa[MT][S::KS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int h = hg0 + mt * 32 + r_lane;
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks)
            qa[mt][ks] = as_bf16x8((h < H) ? load16(qrow + (int64_t)h * D + dim0 + ks * 16 + half * 8)
                                           : u32x4{0, 0, 0, 0});
    }
    // softmax state of the head this lane helps own: hr, rows r0 .. r0+VPL-1
    const int hr = S::HW * wave + lane / S::LPH;
    const int r0 = (lane % S::LPH) * S::VPL;
    float m_run = (hr < H) ? sink[hr] * LOG2E : 0.0f;  // base-2 running max, starting at the sink
    float l_run = (nsplit == 1) ? 1.0f : 0.0f;          // e^(sink - M) at M = sink; splits add it when merged

    const int nchunks = (T + CHUNK - 1) / CHUNK;
    const int c_begin = split * chunks_per_split;
    int c_end = c_begin + chunks_per_split;
    c_end = c_end < nchunks ? c_end : nchunks;
    {
        // this workgroup's slice of the index list, staged once in LDS
        const int e0 = c_begin * CHUNK;
        const int ne = (c_end * CHUNK < T ? c_end * CHUNK : T) - e0;
        for (int i = threadIdx.x; i < (c_end - c_begin) * CHUNK; i += NTH) idx_l[i] = (i < ne) ? idx_q[e0 + i] : -1;
    }
    // Every ordinary global load above is complete before the first row copy is
    // issued, so no compiler-placed wait inside the loop can stall on the copies.
    wait_vmcnt<0>();
    __syncthreads();

    // Copy chunk c's rows (this wave's share) into its stage; returns the chunk's
    // valid-row mask (identical in every wave).  Invalid rows of a partly valid
    // chunk copy this query's first q row instead (finite data; masked later).
    auto issue = [&](int c) -> uint32_t {
        const int32_t* ic = idx_l + (c - c_begin) * CHUNK;
        const int32_t mine = ic[r_lane];
        const uint32_t mask =
            (uint32_t)(__ballot((mine >= 0) && ((int64_t)mine < ra + rb)) & 0xffffffffull);
        if (mask) {
            const uint32_t st = lds0 + (uint32_t)((c % S::NST) * S::STAGE);
            // this wave's RPW entries in one go (broadcast LDS reads), then scalar
            int32_t ivv[S::RPW];
#pragma unroll
            for (int v4 = 0; v4 < S::RPW / 4; ++v4) {
                const int4 t4 = *reinterpret_cast<const int4*>(ic + wave * S::RPW + 4 * v4);
                ivv[4 * v4 + 0] = t4.x;
                ivv[4 * v4 + 1] = t4.y;
                ivv[4 * v4 + 2] = t4.z;
                ivv[4 * v4 + 3] = t4.w;
            }
#pragma unroll
            for (int rr = 0; rr < S::RPW; ++rr) {
                const int r = wave * S::RPW + rr;
                const int32_t iv = __builtin_amdgcn_readfirstlane(ivv[rr]);
                const bool valid = (iv >= 0) && ((int64_t)iv < ra + rb);
                const uint16_t* src = !valid ? qrow
                                             : (((int64_t)iv < ra) ? rows_a_b + (int64_t)iv * D
                                                                   : rows_b_b + ((int64_t)iv - ra) * D);
                if (lane < D / 8) dma16_s(src, (uint32_t)lane * 16u, st + (uint32_t)(r * S::RS));
            }
        }
        return mask;
    };

    f32x16 o[MT][S::NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < S::NT; ++nt) o[mt][nt] = zero16();

    uint32_t mk[S::PD + 1];
#pragma unroll
    for (int j = 0; j < S::PD; ++j) mk[j] = (c_begin + j < c_end) ? issue(c_begin + j) : 0u;

    const int g = lane >> 4;
    const int quad = (lane & 15) >> 2;
    const int a4l = lane & 3;
    // O[:, dims_w] += P . R[:, dims_w] for the chunk in stage stp
    auto pv = [&](const unsigned char* stp) {
        bf16x8 pa[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int kr = 0; kr < 2; ++kr)
                pa[mt][kr] = *reinterpret_cast<const bf16x8*>(pl + (hg0 + mt * 32 + r_lane) * S::PS + kr * 16 + half * 8);
#pragma unroll
        for (int nt = 0; nt < S::NT; ++nt) {
            const int dcol = dim0 + nt * 32 + (g & 1) * 16 + 4 * a4l;
#pragma unroll
            for (int kr = 0; kr < 2; ++kr) {
                const int row = kr * 16 + (g >> 1) * 8 + quad;
                const i16x4 lo = lds_read_tr16(stp + row * S::RS + dcol * 2);
                const i16x4 hi = lds_read_tr16(stp + (row + 4) * S::RS + dcol * 2);
                const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) o[mt][nt] = mfma32x32x16(pa[mt][kr], bv, o[mt][nt]);
            }
        }
    };

    // Chunk loop.  The inner loop never touches O with vector ALU work (so O
    // stays in accumulation registers); it leaves only when a head's running
    // max must move, which the outer loop handles by rescaling O.
    int c = c_begin;
    for (;;) {
        bool moved = false;
        const unsigned char* stp = lds;
        for (; c < c_end; ++c) {
            // chunk c's copies done (later chunks' copies may still fly), then everyone's
            int after = 0;
#pragma unroll
            for (int j = 1; j < S::PD; ++j) after += mk[j] ? S::RPW : 0;
            if (mk[0]) wait_rows<S::RPW>(after);
            __syncthreads();
            mk[S::PD] = (c + S::PD < c_end) ? issue(c + S::PD) : 0u;  // into the stage chunk c-1 used
            const uint32_t mask = mk[0];
#pragma unroll
            for (int j = 0; j < S::PD; ++j) mk[j] = mk[j + 1];
            if (mask == 0) continue;
            stp = lds + (c % S::NST) * S::STAGE;

            // partial logits over this wave's dims, as S^T = R . Q^T: rows are the
            // MFMA M dimension, heads the N dimension, so each lane ends up with one
            // head and runs of 4 consecutive rows (the A/B register layouts of R and
            // Q are the same as for S = Q . R^T, only the operand order changes)
            f32x16 sp[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) sp[mt] = zero16();
#pragma unroll
            for (int ks = 0; ks < S::KS; ++ks) {
                const bf16x8 rk =
                    *reinterpret_cast<const bf16x8*>(stp + r_lane * S::RS + (dim0 + ks * 16 + half * 8) * 2);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) sp[mt] = mfma32x32x16(rk, qa[mt][ks], sp[mt]);
            }
            // sx[wave][head][row]: lane's head mt*32 + r_lane, rows d_row(4*i4, lane) .. +3
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4)
                    *reinterpret_cast<float4*>(sx + ((wave % NW) * S::HP + hg0 + mt * 32 + r_lane) * S::SXS + d_row(4 * i4, lane)) =
                        make_float4(sp[mt][4 * i4], sp[mt][4 * i4 + 1], sp[mt][4 * i4 + 2], sp[mt][4 * i4 + 3]);
            __syncthreads();

            // this wave's heads: sum the NW partial tiles (fixed order), online softmax
            float x[S::VPL];
#pragma unroll
            for (int j = 0; j < S::VPL; ++j) x[j] = 0.0f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const float* src = sx + (ww * S::HP + hr) * S::SXS + r0;
#pragma unroll
                for (int j4 = 0; j4 < S::VPL / 4; ++j4) {
                    const float4 a = *reinterpret_cast<const float4*>(src + 4 * j4);
                    x[4 * j4 + 0] += a.x;
                    x[4 * j4 + 1] += a.y;
                    x[4 * j4 + 2] += a.z;
                    x[4 * j4 + 3] += a.w;
                }
            }
            float cmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < S::VPL; ++j) {
                x[j] = ((mask >> (r0 + j)) & 1u) ? x[j] * scale_log2 : -INFINITY;
                cmax = fmaxf(cmax, x[j]);
            }
            cmax = group_max<S::LPH>(cmax);
            const float m_new = (cmax > m_run + STALE_MAX) ? cmax : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float psum = 0.0f;
            uint32_t pk[S::VPL / 2];
#pragma unroll
            for (int j = 0; j < S::VPL; j += 2) {
                // hardware exp2 (v_exp_f32) and round-to-nearest-even pack to bf16
                // (v_cvt_pk_bf16_f32); the sum uses the rounded weights
                const f32x2 pf = {__builtin_amdgcn_exp2f(x[j] - m_new), __builtin_amdgcn_exp2f(x[j + 1] - m_new)};
                const uint32_t pb = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, bf16x2));
                psum += __uint_as_float(pb << 16) + __uint_as_float(pb & 0xffff0000u);
                pk[j / 2] = pb;
            }
            psum = group_sum<S::LPH>(psum);
            l_run = l_run * alpha + psum;
            const bool my_move = m_new != m_run;
            m_run = m_new;
            {
                uint16_t* dst = pl + hr * S::PS + r0;
#pragma unroll
                for (int j4 = 0; j4 < S::VPL / 4; ++j4)
                    *reinterpret_cast<uint2*>(dst + 4 * j4) = make_uint2(pk[2 * j4], pk[2 * j4 + 1]);
            }
            if (lane % S::LPH == 0) alpha_l[hr] = alpha;
            const uint64_t any_moved = __ballot(my_move);
            if (lane == 0) flags[wave] = any_moved != 0;
            __syncthreads();
#pragma unroll
            for (int ww = 0; ww < S::WAVES; ++ww) moved |= flags[ww] != 0;
            if (moved) break;
            pv(stp);
        }
        if (!moved) break;
        // rare: some head's max moved by more than the slack; rescale O, then this chunk's P.R
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                const float4 a4 = *reinterpret_cast<const float4*>(alpha_l + hg0 + mt * 32 + ig * 8 + half * 4);
#pragma unroll
                for (int nt = 0; nt < S::NT; ++nt) {
                    o[mt][nt][ig * 4 + 0] *= a4.x;
                    o[mt][nt][ig * 4 + 1] *= a4.y;
                    o[mt][nt][ig * 4 + 2] *= a4.z;
                    o[mt][nt][ig * 4 + 3] *= a4.w;
                }
            }
        pv(stp);
        ++c;
    }

    // ---- epilogue
    if (nsplit == 1) {
        if (lane % S::LPH == 0) lsum_l[hr] = l_run;
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                const float4 l4 = *reinterpret_cast<const float4*>(lsum_l + hg0 + mt * 32 + ig * 8 + half * 4);
                const float inv[4] = {1.0f / l4.x, 1.0f / l4.y, 1.0f / l4.z, 1.0f / l4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int h = hg0 + mt * 32 + ig * 8 + half * 4 + e;
                    if (h < H) {
                        uint16_t* orow = out + (qi * H + h) * (int64_t)D + dim0;
#pragma unroll
                        for (int nt = 0; nt < S::NT; ++nt)
                            orow[nt * 32 + r_lane] = (uint16_t)f32_to_bf16_bits(o[mt][nt][ig * 4 + e] * inv[e]);
                    }
                }
            }
    } else {
        const int64_t pbase = (qi * nsplit + split) * (int64_t)H;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int h = hg0 + mt * 32 + d_row(i, lane);
                if (h < H) {
                    float* prow = part_o + (pbase + h) * D + dim0;
#pragma unroll
                    for (int nt = 0; nt < S::NT; ++nt) prow[nt * 32 + r_lane] = o[mt][nt][i];
                }
            }
        if (lane % S::LPH == 0 && hr < H) {
            part_ml[(pbase + hr) * 2 + 0] = m_run;
            part_ml[(pbase + hr) * 2 + 1] = l_run;
        }
    }
}

// Merge the nsplit partials of each (query, head): M = max(sink, m_j),
// Z = e^(sink - M) + sum_j l_j e^(m_j - M), o = sum_j O_j e^(m_j - M) / Z (base 2).
constexpr int COMBINE_THREADS = 256;
__global__ __launch_bounds__(COMBINE_THREADS) void combine_kernel(const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_ml,
                                                                  const float* __restrict__ sink, int nsplit, int H,
                                                                  int D, uint16_t* __restrict__ out) {
    const int64_t qi = blockIdx.x;
    const int h = blockIdx.y;
    const float s2 = sink[h] * LOG2E;
    float M = s2;
    for (int j = 0; j < nsplit; ++j) M = fmaxf(M, part_ml[((qi * nsplit + j) * H + h) * 2]);
    float Z = exp2f(s2 - M);
    for (int j = 0; j < nsplit; ++j) {
        const float* ml = part_ml + ((qi * nsplit + j) * H + h) * 2;
        Z += ml[1] * exp2f(ml[0] - M);
    }
    const float invZ = 1.0f / Z;
    for (int d = threadIdx.x; d < D; d += COMBINE_THREADS) {
        float acc = 0.0f;
        for (int j = 0; j < nsplit; ++j) {
            const float wj = exp2f(part_ml[((qi * nsplit + j) * H + h) * 2] - M);
            acc += part_o[((qi * nsplit + j) * H + h) * (int64_t)D + d] * wj;
        }
        out[(qi * H + h) * (int64_t)D + d] = (uint16_t)f32_to_bf16_bits(acc * invZ);
    }
}

// Chunks per workgroup: split a query's chunks only when the queries alone do
// not give about one workgroup per compute unit.
void attn_split(int64_t nq, int T, int* chunks_per_split, int* nsplit) {
    const int nchunks = (T + CHUNK - 1) / CHUNK;
    int64_t want = (256 + nq - 1) / nq;
    if (want > nchunks) want = nchunks;
    if (want < 1) want = 1;
    int cps = (int)((nchunks + want - 1) / want);
    if (cps > MAX_CPS) cps = MAX_CPS;
    *chunks_per_split = cps;
    *nsplit = (nchunks + cps - 1) / cps;
}

template <int MT, int NG, int DW, int NW>
int launch_attn(const uint16_t* q, const uint16_t* rows_a, int64_t ra, const uint16_t* rows_b, int64_t rb,
                const int32_t* idx, int T, const float* sink, float scale_log2, int64_t nq, int64_t m, int H,
                int cps, int nsplit, uint16_t* out, float* part_o, float* part_ml, hipStream_t s) {
    using Sh = AttnShape<MT, NG, DW, NW>;
    if (Sh::LDS_BYTES > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)sparse_attn_kernel<MT, NG, DW, NW>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)Sh::LDS_BYTES);
        if (e != hipSuccess) return fail(SCKV_EHIP, std::string("sckv_sparse_attn_sink: ") + hipGetErrorString(e));
    }
    sparse_attn_kernel<MT, NG, DW, NW><<<dim3((unsigned)(nq * nsplit)), dim3(Sh::WAVES * 64), Sh::LDS_BYTES, s>>>(
        q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, m, H, cps, nsplit, out, part_o, part_ml);
    return check_launch("sckv_sparse_attn_sink");
}

}  // namespace

size_t attn_workspace_bytes(int B, int64_t m, int H, int D, int64_t T) {
    int cps, nsplit;
    attn_split((int64_t)B * m, (int)T, &cps, &nsplit);
    if (nsplit == 1) return 0;
    const size_t nq = (size_t)B * (size_t)m;
    size_t bytes = nq * (size_t)nsplit * (size_t)H * (size_t)D * 4u;
    bytes = (bytes + 255u) & ~(size_t)255u;
    bytes += nq * (size_t)nsplit * (size_t)H * 2u * 4u;
    return (bytes + 255u) & ~(size_t)255u;
}

}  // namespace sckv

extern "C" int sckv_sparse_attn_sink(const void* q, const void* rows_a, int64_t ra, const void* rows_b, int64_t rb,
                                     const int32_t* idx, int T, const float* sink, float scale, int B, int64_t m,
                                     int H, int D, void* out, void* ws, size_t ws_bytes, void* stream) {
    using namespace sckv;
    if (B < 0 || m < 0 || ra < 0 || rb < 0 || H <= 0 || D <= 0 || T < 0)
        return fail(SCKV_EINVAL, "sckv_sparse_attn_sink: bad sizes");
    if (H > 64) return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink: H > 64");
    if (D != 64 && D != 128 && D != 256 && D != 512)
        return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink: D not in {64, 128, 256, 512}");
    if (T > 65536) return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink: T > 65536");
    if (B == 0 || m == 0) return SCKV_OK;
    if (T == 0) return fail(SCKV_EINVAL, "sckv_sparse_attn_sink: T == 0");
    if (!q || !idx || !sink || !out || (ra > 0 && !rows_a) || (rb > 0 && !rows_b))
        return fail(SCKV_EINVAL, "sckv_sparse_attn_sink: null pointer");
    if ((uintptr_t)q % 16 || (uintptr_t)rows_a % 16 || (uintptr_t)rows_b % 16 || (uintptr_t)out % 2 ||
        (uintptr_t)idx % 4 || (uintptr_t)sink % 4)
        return fail(SCKV_EINVAL, "sckv_sparse_attn_sink: q / rows must be 16-byte aligned");
    if (ra + rb > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink: ra + rb >= 2^31");
    if (!(scale > 0.0f) || !(scale < INFINITY)) return fail(SCKV_EINVAL, "sckv_sparse_attn_sink: bad scale");
    const int64_t nq = (int64_t)B * m;
    int cps, nsplit;
    attn_split(nq, T, &cps, &nsplit);
    if (nq * nsplit > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink: grid too large");
    const size_t need = attn_workspace_bytes(B, m, H, D, T);
    if (need && (!ws || ws_bytes < need)) return fail(SCKV_EWORKSPACE, "sckv_sparse_attn_sink: workspace too small");
    float* part_o = nullptr;
    float* part_ml = nullptr;
    if (nsplit > 1) {
        part_o = (float*)ws;
        size_t ob = (size_t)nq * nsplit * H * D * 4u;
        ob = (ob + 255u) & ~(size_t)255u;
        part_ml = (float*)((char*)ws + ob);
    }
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipStream_t s = (hipStream_t)stream;
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* aa = (const uint16_t*)rows_a;
    const uint16_t* bb = (const uint16_t*)rows_b;
    uint16_t* oo = (uint16_t*)out;
    int rc;
    const bool two = H > 32;
#define SCKV_ATTN(MT, DW, NW) \
    launch_attn<MT, 1, DW, NW>(qq, aa, ra, bb, rb, idx, T, sink, scale_log2, nq, m, H, cps, nsplit, oo, part_o, part_ml, s)
#define SCKV_ATTN2(MT, NG, DW, NW) \
    launch_attn<MT, NG, DW, NW>(qq, aa, ra, bb, rb, idx, T, sink, scale_log2, nq, m, H, cps, nsplit, oo, part_o, part_ml, s)
    switch (D) {
        case 64: rc = two ? SCKV_ATTN(2, 64, 1) : SCKV_ATTN(1, 64, 1); break;
        case 128: rc = two ? SCKV_ATTN(2, 128, 1) : SCKV_ATTN(1, 128, 1); break;
        case 256: rc = two ? SCKV_ATTN(2, 128, 2) : SCKV_ATTN(1, 128, 2); break;
        default: rc = two ? SCKV_ATTN2(1, 2, 128, 4) : SCKV_ATTN(1, 128, 4); break;
    }
#undef SCKV_ATTN
#undef SCKV_ATTN2
    if (rc || nsplit == 1) return rc;
    if (nq > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink: too many queries");
    combine_kernel<<<dim3((unsigned)nq, (unsigned)H), dim3(COMBINE_THREADS), 0, s>>>(part_o, part_ml, sink, nsplit, H,
                                                                                    D, oo);
    return check_launch("sckv_sparse_attn_sink (combine)");
}

// decode_dev.h -- device code of a decode step's set-up (the latent row's
// rotation and round trip, the packed indexer k row, the ring slot and the
// window columns), as a body that takes the sequence number: the kernel of
// decode.hip runs it with blockIdx.x, the one-launch decode step
// (decode_step.hip) as its first phase.
#pragma once

#include "sckv_device.h"

namespace sckv {
namespace {

constexpr int PREP_THREADS = 256;

struct PrepArgs {
    const uint16_t* lat_new;
    int64_t ld_lat_new;
    uint16_t* lat_dst;
    int64_t ld_lat_dst;
    const uint16_t* k_new;
    int64_t ld_k_new;
    uint8_t* k_codes;
    int64_t ld_codes;
    uint8_t* k_scales;
    int64_t ld_scales;
    int Di;
    const uint16_t* kv_new;
    int64_t ld_kv_new;
    uint16_t* ring;
    int64_t ld_ring;
    int D, win;
    int64_t start_pos;
    int32_t* idx;
    int64_t ld_idx;
    const float* rope_table;  // NULL: the latent row is not rotated
    int rope_dim;
    int64_t lat_pos;
    uint8_t* lat_codes;  // non-NULL: the latent row is stored packed (codes + e4m3 scale bytes)
    int64_t ld_lat_codes;
    uint8_t* lat_scales;
    int64_t ld_lat_scales;
};

// Max over aligned groups of 8 or 16 lanes by DPP (every lane of the group
// gets it): lane pairs, quads, then the half-row and row mirrors.
__device__ __forceinline__ float group_max(float v, int lanes) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, false)));  // quad_perm 1,0,3,2
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, false)));  // quad_perm 2,3,0,1
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, false)));  // row_half_mirror
    if (lanes == 16) v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, false)));  // row_mirror
    return v;
}

// Workgroup b = sequence b.  Every row pointer is 16-byte aligned and every
// stride a multiple of 16 bytes (checked on the host).  The rows are spread
// over the lanes two values a lane, so a block's 16 (latent) or 32 (k) values
// sit in 8 or 16 neighbouring lanes, which share the block amax by DPP; each
// value then goes through the same device code as in sckv_quant_rows /
// sckv_quant_pack.
__device__ __forceinline__ void decode_prepare_body(const PrepArgs& a, const int64_t b) {
    const int t = threadIdx.x;
    const uint32_t* lsrc = a.lat_new ? reinterpret_cast<const uint32_t*>(a.lat_new + b * a.ld_lat_new) : nullptr;
    const int rope_first = (a.D - a.rope_dim) / 2;  // first pair of the rope slice
    const float2* rt = (a.lat_new && a.rope_table)
                           ? reinterpret_cast<const float2*>(a.rope_table) + a.lat_pos * (a.rope_dim / 2)
                           : nullptr;
    const uint32_t* ksrc = a.k_new ? reinterpret_cast<const uint32_t*>(a.k_new + b * a.ld_k_new) : nullptr;
    const uint4* kvsrc = reinterpret_cast<const uint4*>(a.kv_new + b * a.ld_kv_new);
    // the loads of every part's first pass come first, at addresses clamped
    // into their rows (no per-lane branches), so that their latencies overlap
    // instead of following one another part by part
    uint32_t lat0 = 0u, k0 = 0u;
    float2 cs0 = make_float2(1.0f, 0.0f);
    {
        const int tl = t < a.D / 2 ? t : a.D / 2 - 1;
        int tr = t - rope_first;
        tr = tr < 0 ? 0 : (tr < a.rope_dim / 2 ? tr : a.rope_dim / 2 - 1);
        if (lsrc) lat0 = lsrc[tl];
        if (rt) cs0 = rt[tr];
        if (ksrc) k0 = ksrc[t < a.Di / 2 ? t : a.Di / 2 - 1];
    }
    const uint4 kv0 = kvsrc[t < a.D / 8 ? t : a.D / 8 - 1];

    // latent row: values 2p, 2p + 1 in lane p (E4M3_B16 round trip, bf16 out)
    if (lsrc) {
        uint32_t* dst = a.lat_dst ? reinterpret_cast<uint32_t*>(a.lat_dst + b * a.ld_lat_dst) : nullptr;
        auto pair = [&](int p, uint32_t w, float2 cs) {
            // the rotary turn of pair p before the round trip (sckv_rope_quant_rows)
            if (rt && p >= rope_first) w = rope_pair_bits(w, cs.x, cs.y);
            const float lo = bf16_bits_to_f32(w & 0xffffu), hi = bf16_bits_to_f32(w >> 16);
            const float amax = group_max(fmaxf(fabsf(lo), fabsf(hi)), 8);
            const float s = block_scale<SCKV_FP4_E4M3_B16>(amax);
            if (a.lat_codes) {
                // packed (sckv_rope_quant_pack): one code byte a lane, the
                // e4m3 scale byte from the block's first lane
                const uint32_t clo = e2m1_code(e2m1_round_mag(fminf(__fdiv_rn(fabsf(lo), s), 6.0f)), lo);
                const uint32_t chi = e2m1_code(e2m1_round_mag(fminf(__fdiv_rn(fabsf(hi), s), 6.0f)), hi);
                a.lat_codes[b * a.ld_lat_codes + p] = (uint8_t)(clo | (chi << 4));
                if ((p & 7) == 0) a.lat_scales[b * a.ld_lat_scales + p / 8] = (uint8_t)scale_byte<SCKV_FP4_E4M3_B16>(s);
            } else {
                dst[p] = fp4_value<SCKV_FP4_E4M3_B16>(lo, s, 0.0f) | (fp4_value<SCKV_FP4_E4M3_B16>(hi, s, 0.0f) << 16);
            }
        };
        // (a block's 8 lanes are all below D / 2 or all past it: D % 16 == 0)
        if (t < a.D / 2) pair(t, lat0, cs0);
        for (int p = t + PREP_THREADS; p < a.D / 2; p += PREP_THREADS)
            pair(p, lsrc[p], (rt && p >= rope_first) ? rt[p - rope_first] : make_float2(1.0f, 0.0f));
    }
    // indexer k row: values 2p, 2p + 1 in lane p (E8M0_B32, packed: one code
    // byte a lane, the scale byte from the block's first lane)
    if (ksrc) {
        uint8_t* codes = a.k_codes + b * a.ld_codes;
        uint8_t* scales = a.k_scales + b * a.ld_scales;
        auto pair = [&](int p, uint32_t w) {
            const float lo = bf16_bits_to_f32(w & 0xffffu), hi = bf16_bits_to_f32(w >> 16);
            const float amax = group_max(fmaxf(fabsf(lo), fabsf(hi)), 16);
            const float s = block_scale<SCKV_FP4_E8M0_B32>(amax);
            const float inv_s = pow2_reciprocal(s);
            const uint32_t clo = e2m1_code(e2m1_round_mag(fminf(fabsf(lo) * inv_s, 6.0f)), lo);
            const uint32_t chi = e2m1_code(e2m1_round_mag(fminf(fabsf(hi) * inv_s, 6.0f)), hi);
            codes[p] = (uint8_t)(clo | (chi << 4));
            if ((p & 15) == 0) scales[p / 16] = (uint8_t)scale_byte<SCKV_FP4_E8M0_B32>(s);
        };
        // (a block's 16 lanes are all below Di / 2 or all past it: Di % 32 == 0)
        if (t < a.Di / 2) pair(t, k0);
        for (int p = t + PREP_THREADS; p < a.Di / 2; p += PREP_THREADS) pair(p, ksrc[p]);
    }
    // the new kv row into ring slot start_pos mod win
    {
        uint4* dst = reinterpret_cast<uint4*>(a.ring + b * a.ld_ring + (a.start_pos % a.win) * a.D);
        if (t < a.D / 8) dst[t] = kv0;
        for (int i = t + PREP_THREADS; i < a.D / 8; i += PREP_THREADS) dst[i] = kvsrc[i];
    }
    // window columns of the query at p = start_pos: the n_w = min(win, p + 1)
    // newest positions, oldest first, then -1
    {
        int32_t* row = a.idx + b * a.ld_idx;
        for (int j = t; j < a.win; j += PREP_THREADS) row[j] = window_col(a.win, 1, a.start_pos, 0, j);
    }
}

}  // namespace
}  // namespace sckv

// decode.hip -- the set-up of a decode step (m = 1) in one launch: the fp4
// round trip of the completed latent row into the latent cache, the packed
// indexer k row, the new kv row into its ring slot and the window columns of
// the index list.
//
// Page "metrale_model_arch/attn_v41/forward.rs" (AttnV41::forward: the fp4
// round trip of a completed latent group before its cache copy, the ring copy
// at slot start_pos mod window before attention, window_topk_idxs) and page
// "metrale_model_arch/deepseek_v41_ref/compress.rs" (fp4_quant_e4m3_inplace,
// fp4_quant_e8m0_inplace, yarn_freqs_cis and the rotation of a new latent
// group before its round trip).  Each part computes exactly what the separate
// calls sckv_rope_quant_rows (or sckv_quant_rows without a rotation table),
// sckv_quant_pack, sckv_ring_write and sckv_window_idx compute
// (the same device code); they write disjoint memory, so one launch with a
// workgroup per sequence replaces four launches whose cost at decode size is
// almost all launch and drain time.
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
__global__ __launch_bounds__(PREP_THREADS) void decode_prepare_kernel(PrepArgs a) {
    const int64_t b = blockIdx.x;
    const int t = threadIdx.x;
    // latent row: values 2p, 2p + 1 in lane p (E4M3_B16 round trip, bf16 out)
    if (a.lat_new) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.lat_new + b * a.ld_lat_new);
        uint32_t* dst = a.lat_dst ? reinterpret_cast<uint32_t*>(a.lat_dst + b * a.ld_lat_dst) : nullptr;
        const int rope_first = (a.D - a.rope_dim) / 2;  // first pair of the rope slice
        const float2* rt = a.rope_table ? reinterpret_cast<const float2*>(a.rope_table) + a.lat_pos * (a.rope_dim / 2)
                                        : nullptr;
        for (int p = t; p < a.D / 2; p += PREP_THREADS) {
            uint32_t w = src[p];
            if (rt && p >= rope_first) {
                // the rotary turn of pair p before the round trip (sckv_rope_quant_rows)
                const float2 cs = rt[p - rope_first];
                w = rope_pair_bits(w, cs.x, cs.y);
            }
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
        }
    }
    // indexer k row: values 2p, 2p + 1 in lane p (E8M0_B32, packed: one code
    // byte a lane, the scale byte from the block's first lane)
    if (a.k_new) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.k_new + b * a.ld_k_new);
        uint8_t* codes = a.k_codes + b * a.ld_codes;
        uint8_t* scales = a.k_scales + b * a.ld_scales;
        for (int p = t; p < a.Di / 2; p += PREP_THREADS) {
            const uint32_t w = src[p];
            const float lo = bf16_bits_to_f32(w & 0xffffu), hi = bf16_bits_to_f32(w >> 16);
            const float amax = group_max(fmaxf(fabsf(lo), fabsf(hi)), 16);
            const float s = block_scale<SCKV_FP4_E8M0_B32>(amax);
            const float inv_s = pow2_reciprocal(s);
            const uint32_t clo = e2m1_code(e2m1_round_mag(fminf(fabsf(lo) * inv_s, 6.0f)), lo);
            const uint32_t chi = e2m1_code(e2m1_round_mag(fminf(fabsf(hi) * inv_s, 6.0f)), hi);
            codes[p] = (uint8_t)(clo | (chi << 4));
            if ((p & 15) == 0) scales[p / 16] = (uint8_t)scale_byte<SCKV_FP4_E8M0_B32>(s);
        }
    }
    // the new kv row into ring slot start_pos mod win
    {
        const uint4* src = reinterpret_cast<const uint4*>(a.kv_new + b * a.ld_kv_new);
        uint4* dst = reinterpret_cast<uint4*>(a.ring + b * a.ld_ring + (a.start_pos % a.win) * a.D);
        for (int i = t; i < a.D / 8; i += PREP_THREADS) dst[i] = src[i];
    }
    // window columns of the query at p = start_pos: the n_w = min(win, p + 1)
    // newest positions, oldest first, then -1
    {
        const int64_t p = a.start_pos;
        const int64_t n_w = (p + 1 < a.win) ? (p + 1) : a.win;
        int32_t* row = a.idx + b * a.ld_idx;
        for (int j = t; j < a.win; j += PREP_THREADS)
            row[j] = (j < n_w) ? (int32_t)window_row(a.win, 1, p, p - n_w + 1 + j) : -1;
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p % 16) == 0; }

}  // namespace
}  // namespace sckv

extern "C" int sckv_decode_prepare(const void* lat_new, int64_t ld_lat_new, void* lat_dst, int64_t ld_lat_dst,
                                   const void* k_new, int64_t ld_k_new, void* k_codes, int64_t ld_codes,
                                   void* k_scales, int64_t ld_scales, int Di, const void* kv_new, int64_t ld_kv_new,
                                   void* ring, int64_t ld_ring, int B, int D, int win, int64_t start_pos,
                                   int32_t* idx, int64_t ld_idx, const float* rope_table, int64_t n_pos,
                                   int rope_dim, int64_t lat_pos, void* lat_codes, int64_t ld_lat_codes,
                                   void* lat_scales, int64_t ld_lat_scales, void* stream) {
    using namespace sckv;
    const char* name = "sckv_decode_prepare";
    if (B < 0 || D <= 0 || win <= 0 || start_pos < 0) return fail(SCKV_EINVAL, std::string(name) + ": bad sizes");
    if (D % 16 != 0) return fail(SCKV_EINVAL, std::string(name) + ": D is not a multiple of 16");
    if (lat_new && !lat_codes && (!lat_dst || ld_lat_new < D || ld_lat_dst < D))
        return fail(SCKV_EINVAL, std::string(name) + ": latent rows: null destination or stride below D");
    if (lat_new && lat_codes &&
        (lat_dst || !lat_scales || ld_lat_new < D || ld_lat_codes < D / 2 || ld_lat_scales < D / 16))
        return fail(SCKV_EINVAL, std::string(name) + ": packed latent rows: give codes and scales (and no bf16 "
                                                     "destination) with strides of at least D/2 and D/16 bytes");
    if (k_new && (!k_codes || !k_scales || Di <= 0 || Di % 32 != 0 || ld_k_new < Di || ld_codes < Di / 2 ||
                  ld_scales < Di / 32))
        return fail(SCKV_EINVAL, std::string(name) + ": k rows: null destination, Di not a multiple of 32 or short stride");
    if (lat_new && rope_table &&
        (rope_dim <= 0 || rope_dim % 2 != 0 || rope_dim > D || lat_pos < 0 || lat_pos >= n_pos ||
         (uintptr_t)rope_table % 8))
        return fail(SCKV_EINVAL, std::string(name) + ": rotation: rope_dim must be even, positive and at most D, "
                                                     "lat_pos inside the table, the table 8-byte aligned");
    if (!kv_new || !ring || !idx) return fail(SCKV_EINVAL, std::string(name) + ": null pointer");
    if (ld_kv_new < D || ld_ring < (int64_t)win * D || ld_idx < win)
        return fail(SCKV_EINVAL, std::string(name) + ": a stride is shorter than its row");
    if (B == 0) return SCKV_OK;
    if (B > 0x7fffffff / 2) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": B too large");
    if (start_pos + win > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": positions past 2^31");
    // 16-byte vectors throughout
    const bool ok = aligned16(kv_new) && aligned16(ring) && (ld_kv_new % 8 == 0) && (ld_ring % 8 == 0) &&
                    (!lat_new || (aligned16(lat_new) && ld_lat_new % 8 == 0 &&
                                  (lat_codes || (aligned16(lat_dst) && ld_lat_dst % 8 == 0)))) &&
                    (!k_new || (aligned16(k_new) && aligned16(k_codes) && ld_k_new % 8 == 0 && ld_codes % 16 == 0));
    if (!ok) return fail(SCKV_EINVAL, std::string(name) + ": rows must be 16-byte aligned with 16-byte strides");
    PrepArgs a{(const uint16_t*)lat_new, ld_lat_new, (uint16_t*)lat_dst, ld_lat_dst, (const uint16_t*)k_new, ld_k_new,
               (uint8_t*)k_codes, ld_codes, (uint8_t*)k_scales, ld_scales, Di, (const uint16_t*)kv_new, ld_kv_new,
               (uint16_t*)ring, ld_ring, D, win, start_pos, idx, ld_idx, lat_new ? rope_table : nullptr,
               rope_dim, lat_pos, lat_new ? (uint8_t*)lat_codes : nullptr, ld_lat_codes, (uint8_t*)lat_scales,
               ld_lat_scales};
    decode_prepare_kernel<<<dim3((unsigned)B), dim3(PREP_THREADS), 0, (hipStream_t)stream>>>(a);
    return check_launch(name);
}

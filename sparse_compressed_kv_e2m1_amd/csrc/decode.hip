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
#include "decode_dev.h"

namespace sckv {
namespace {

__global__ __launch_bounds__(PREP_THREADS) void decode_prepare_kernel(PrepArgs a) { decode_prepare_body(a, blockIdx.x); }

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

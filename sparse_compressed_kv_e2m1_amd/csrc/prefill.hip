// prefill.hip -- the set-up of a step of m >= 1 queries in one launch: the
// rotation and fp4 round trip of the step's new compressed latent rows into
// the latent cache, the fp4 round trip (or packing) of its new indexer k rows,
// the window columns of every query's index list, the visible compressed
// columns on a layer without an indexer, and the ring write of a step that
// starts at position 0.
//
// Page "metrale_model_arch/attn_v41/forward.rs" (AttnV41::forward: the fp4
// round trip of completed latent groups before their cache copy,
// window_topk_idxs, compress_len = (start_pos + m) / ratio, the ring's
// stream-ordered copies) and page "metrale_model_arch/deepseek_v41_ref/
// compress.rs" (fp4_quant_e4m3_inplace, fp4_quant_e8m0_inplace, the rotation
// of a new latent group before its round trip).  Each part runs the device
// code of its separate call (sckv_rope_quant_rows / sckv_rope_quant_pack,
// sckv_quant_rows / sckv_quant_pack, sckv_window_idx, sckv_visible_idx,
// sckv_ring_write) on a range of the launch's workgroups; the parts read only
// the step's inputs and write disjoint memory, so the launch replaces up to
// five small launches whose time is mostly launch and drain.
#include "quant_dev.h"

namespace sckv {
namespace {

constexpr int PF_THREADS = QUANT_THREADS;

struct PrefillArgs {
    int64_t m, start_pos;
    int win, D, Di;
    int64_t n_new;
    // latent rows: n_new a sequence, contiguous, batch strides in elements / bytes
    const uint16_t* lat_new;
    int64_t bs_lat_new;
    uint16_t* lat_dst;  // bf16 destination, or NULL: stored packed
    int64_t bs_lat_dst;
    uint8_t* lat_codes;
    int64_t bs_lat_codes;
    uint8_t* lat_scales;
    int64_t bs_lat_scales;
    RopeArgs rope;  // rope.table NULL: no rotation
    // indexer k rows (k_new NULL: none)
    const uint16_t* k_new;
    int64_t bs_k_new;
    uint16_t* k_dst;  // bf16 destination, or NULL: stored packed
    int64_t bs_k_dst;
    uint8_t* k_codes;
    int64_t bs_k_codes;
    uint8_t* k_scales;
    int64_t bs_k_scales;
    // ring rows (ring_src NULL: none): positions ring_first_t .. m - 1
    const uint16_t* ring_src;
    int64_t bs_ring_src;
    uint16_t* ring;
    int64_t bs_ring;
    int64_t ring_first_t;
    // index list [B, m, ld_idx]: window columns 0 .. win - 1, visible
    // columns win .. win + K - 1 (K = 0: none)
    int32_t* idx;
    int64_t ld_idx;
    int ratio;
    int64_t n_c;
    int K;
    int32_t offset;
    int idx_vec;  // 4 columns a lane with 16-byte stores
    // workgroup ranges along x: [0, w_k) latent blocks, [w_k, w_win) k blocks,
    // [w_win, w_vis) window columns, [w_vis, w_ring) visible columns, [w_ring,
    // gridDim.x) ring rows
    uint32_t w_k, w_win, w_vis, w_ring;
};

// Columns [col0, col0 + ncol) of every query, one (vec: four) a lane, value f(t, j).
template <typename F>
__device__ __forceinline__ void idx_columns(int32_t* __restrict__ base, int64_t ld, int64_t m, int64_t col0, int ncol,
                                            int64_t lane, bool vec, F f) {
    if (vec) {
        const int per = ncol / 4;
        const int64_t t = lane / per;
        const int j = (int)(lane - t * per) * 4;
        if (t >= m) return;
        *reinterpret_cast<int4*>(base + t * ld + col0 + j) = make_int4(f(t, j), f(t, j + 1), f(t, j + 2), f(t, j + 3));
    } else {
        const int64_t t = lane / ncol;
        const int j = (int)(lane - t * ncol);
        if (t >= m) return;
        base[t * ld + col0 + j] = f(t, j);
    }
}

__global__ __launch_bounds__(PF_THREADS) void prefill_prepare_kernel(PrefillArgs a) {
    const int64_t b = blockIdx.y;
    const uint32_t wg = blockIdx.x;
    if (wg < a.w_k) {
        // latent block gid: rotation, then the e4m3-scale round trip
        const int64_t gid = (int64_t)wg * PF_THREADS + threadIdx.x;
        const int64_t bpr = a.D / 16;
        if (gid >= a.n_new * bpr) return;
        const uint16_t* x = a.lat_new + b * a.bs_lat_new;
        if (a.lat_codes) {
            uint8_t* c = a.lat_codes + b * a.bs_lat_codes;
            uint8_t* s = a.lat_scales + b * a.bs_lat_scales;
            if (a.rope.table)
                quant_pack_block<SCKV_FP4_E4M3_B16, true>(x, a.D, c, a.D / 2, s, bpr, bpr, gid, true, a.rope);
            else
                quant_pack_block<SCKV_FP4_E4M3_B16, false>(x, a.D, c, a.D / 2, s, bpr, bpr, gid, true, a.rope);
        } else {
            uint16_t* y = a.lat_dst + b * a.bs_lat_dst;
            if (a.rope.table)
                quant_rows_block<SCKV_FP4_E4M3_B16, true, true>(x, a.D, y, a.D, bpr, gid, a.rope);
            else
                quant_rows_block<SCKV_FP4_E4M3_B16, true, false>(x, a.D, y, a.D, bpr, gid, a.rope);
        }
    } else if (wg < a.w_win) {
        // indexer k block gid: the power-of-two-scale round trip
        const int64_t gid = (int64_t)(wg - a.w_k) * PF_THREADS + threadIdx.x;
        const int64_t bpr = a.Di / 32;
        if (gid >= a.n_new * bpr) return;
        const uint16_t* x = a.k_new + b * a.bs_k_new;
        if (a.k_codes)
            quant_pack_block<SCKV_FP4_E8M0_B32, false>(x, a.Di, a.k_codes + b * a.bs_k_codes, a.Di / 2,
                                                       a.k_scales + b * a.bs_k_scales, bpr, bpr, gid, true, a.rope);
        else
            quant_rows_block<SCKV_FP4_E8M0_B32, true, false>(x, a.Di, a.k_dst + b * a.bs_k_dst, a.Di, bpr, gid,
                                                              a.rope);
    } else if (wg < a.w_vis) {
        const int win = a.win;
        const int64_t m = a.m, sp = a.start_pos;
        idx_columns(a.idx + b * a.m * a.ld_idx, a.ld_idx, m, 0, win, (int64_t)(wg - a.w_win) * PF_THREADS + threadIdx.x,
                    a.idx_vec, [&](int64_t t, int j) { return window_col(win, m, sp, t, j); });
    } else if (wg < a.w_ring) {
        const int64_t sp = a.start_pos, n_c = a.n_c;
        const int ratio = a.ratio;
        const int32_t off = a.offset;
        idx_columns(a.idx + b * a.m * a.ld_idx, a.ld_idx, a.m, a.win, a.K,
                    (int64_t)(wg - a.w_vis) * PF_THREADS + threadIdx.x, a.idx_vec,
                    [&](int64_t t, int j) { return visible_col(sp, ratio, n_c, off, t, j); });
    } else {
        // ring row of position start_pos + t into slot (start_pos + t) mod win, 16 bytes a lane
        const int per = a.D / 8;
        const int64_t gid = (int64_t)(wg - a.w_ring) * PF_THREADS + threadIdx.x;
        const int64_t r = gid / per;
        const int piece = (int)(gid - r * per);
        const int64_t t = a.ring_first_t + r;
        if (t >= a.m) return;
        const int64_t slot = (a.start_pos + t) % a.win;
        const uint4* src = reinterpret_cast<const uint4*>(a.ring_src + b * a.bs_ring_src + t * a.D);
        uint4* dst = reinterpret_cast<uint4*>(a.ring + b * a.bs_ring + slot * a.D);
        dst[piece] = src[piece];
    }
}

bool al16(const void* p) { return ((uintptr_t)p % 16) == 0; }

// [p, p + bytes) and [q, q + qbytes) overlap
bool overlap(const void* p, int64_t bytes, const void* q, int64_t qbytes) {
    const uintptr_t ps = (uintptr_t)p, qs = (uintptr_t)q;
    return ps < qs + (uintptr_t)qbytes && qs < ps + (uintptr_t)bytes;
}

uint32_t wgs(int64_t lanes) { return (uint32_t)((lanes + PF_THREADS - 1) / PF_THREADS); }

}  // namespace
}  // namespace sckv

extern "C" int sckv_prefill_prepare(int B, int64_t m, int64_t start_pos, int win, int D, int64_t n_new,
                                    const void* lat_new, int64_t bs_lat_new, void* lat_dst, int64_t bs_lat_dst,
                                    void* lat_codes, int64_t bs_lat_codes, void* lat_scales, int64_t bs_lat_scales,
                                    const float* rope_table, int64_t n_pos, int rope_dim, int64_t pos0,
                                    int64_t pos_step, const void* k_new, int64_t bs_k_new, int Di, void* k_dst,
                                    int64_t bs_k_dst, void* k_codes, int64_t bs_k_codes, void* k_scales,
                                    int64_t bs_k_scales, const void* ring_src, int64_t bs_ring_src, void* ring,
                                    int64_t bs_ring, int32_t* idx, int64_t ld_idx, int ratio, int64_t n_c, int K,
                                    int32_t offset, void* stream) {
    using namespace sckv;
    const std::string name = "sckv_prefill_prepare";
    if (B < 0 || m < 0 || start_pos < 0 || win <= 0 || D <= 0 || n_new < 0 || K < 0)
        return fail(SCKV_EINVAL, name + ": bad sizes");
    if (D % 16 != 0) return fail(SCKV_EINVAL, name + ": D is not a multiple of 16");
    if (!idx) return fail(SCKV_EINVAL, name + ": null idx");
    if (ld_idx < (int64_t)win + K) return fail(SCKV_EINVAL, name + ": ld_idx < win + K");
    if (B > 65535) return fail(SCKV_EUNSUPPORTED, name + ": B > 65535");
    if (start_pos + m + win > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, name + ": positions past 2^31");
    const bool lat = lat_new && n_new > 0, kk = k_new && n_new > 0;
    if (lat) {
        if (lat_dst ? (lat_codes || lat_scales) : (!lat_codes || !lat_scales))
            return fail(SCKV_EINVAL, name + ": latent rows: give lat_dst, or lat_codes and lat_scales");
        if (bs_lat_new < n_new * D || (lat_dst && bs_lat_dst < n_new * D) ||
            (lat_codes && (bs_lat_codes < n_new * D / 2 || bs_lat_scales < n_new * D / 16)))
            return fail(SCKV_EINVAL, name + ": a latent batch stride is shorter than the sequence's rows");
        if (!al16(lat_new) || bs_lat_new % 8 || (lat_dst && (!al16(lat_dst) || bs_lat_dst % 8)) ||
            (lat_codes && ((uintptr_t)lat_codes % 8 || bs_lat_codes % 8)))
            return fail(SCKV_EINVAL, name + ": latent rows must be 16-byte aligned (codes 8) with such batch strides");
        if (overlap(lat_new, (n_new * D) * 2, lat_dst ? lat_dst : lat_codes, lat_dst ? n_new * D * 2 : n_new * D / 2))
            return fail(SCKV_EINVAL, name + ": latent source and destination overlap");
        if (rope_table)
            if (const int rc = rope_checks(name.c_str(), n_new, D, rope_table, n_pos, rope_dim, pos0, pos_step))
                return rc;
    }
    if (kk) {
        if (Di <= 0 || Di % 32 != 0) return fail(SCKV_EINVAL, name + ": Di must be a positive multiple of 32");
        if (k_dst ? (k_codes || k_scales) : (!k_codes || !k_scales))
            return fail(SCKV_EINVAL, name + ": k rows: give k_dst, or k_codes and k_scales");
        if (bs_k_new < n_new * Di || (k_dst && bs_k_dst < n_new * Di) ||
            (k_codes && (bs_k_codes < n_new * Di / 2 || bs_k_scales < n_new * Di / 32)))
            return fail(SCKV_EINVAL, name + ": a k batch stride is shorter than the sequence's rows");
        if (!al16(k_new) || bs_k_new % 8 || (k_dst && (!al16(k_dst) || bs_k_dst % 8)) ||
            (k_codes && (!al16(k_codes) || bs_k_codes % 16)))
            return fail(SCKV_EINVAL, name + ": k rows must be 16-byte aligned with such batch strides");
        if (overlap(k_new, n_new * Di * 2, k_dst ? k_dst : k_codes, k_dst ? n_new * Di * 2 : n_new * Di / 2))
            return fail(SCKV_EINVAL, name + ": k source and destination overlap");
    }
    if (K > 0) {
        if (ratio <= 0 || n_c < 0 || offset < 0) return fail(SCKV_EINVAL, name + ": visible columns: bad sizes");
        int64_t vmax = (start_pos + m) / ratio;
        vmax = vmax < n_c ? vmax : n_c;
        if (vmax > K) return fail(SCKV_EINVAL, name + ": more visible rows than K columns");
        if ((int64_t)offset + K > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, name + ": offset + K >= 2^31");
    }
    const int64_t first_t = (m > win) ? m - win : 0;
    if (ring_src) {
        if (!ring) return fail(SCKV_EINVAL, name + ": null ring");
        if (bs_ring_src < m * D || bs_ring < (int64_t)win * D)
            return fail(SCKV_EINVAL, name + ": a ring batch stride is shorter than one sequence");
        if (!al16(ring_src) || !al16(ring) || bs_ring_src % 8 || bs_ring % 8)
            return fail(SCKV_EINVAL, name + ": ring rows must be 16-byte aligned with 16-byte batch strides");
        if (overlap(ring_src, m * D * 2, ring, (int64_t)win * D * 2))
            return fail(SCKV_EINVAL, name + ": rows and ring overlap");
    }
    if (B == 0 || m == 0) return SCKV_OK;
    PrefillArgs a{};
    a.m = m;
    a.start_pos = start_pos;
    a.win = win;
    a.D = D;
    a.Di = Di;
    a.n_new = n_new;
    a.lat_new = (const uint16_t*)lat_new;
    a.bs_lat_new = bs_lat_new;
    a.lat_dst = (uint16_t*)lat_dst;
    a.bs_lat_dst = bs_lat_dst;
    a.lat_codes = lat_dst ? nullptr : (uint8_t*)lat_codes;
    a.bs_lat_codes = bs_lat_codes;
    a.lat_scales = (uint8_t*)lat_scales;
    a.bs_lat_scales = bs_lat_scales;
    a.rope = RopeArgs{rope_table, rope_dim, pos0, pos_step};
    a.k_new = (const uint16_t*)k_new;
    a.bs_k_new = bs_k_new;
    a.k_dst = (uint16_t*)k_dst;
    a.bs_k_dst = bs_k_dst;
    a.k_codes = k_dst ? nullptr : (uint8_t*)k_codes;
    a.bs_k_codes = bs_k_codes;
    a.k_scales = (uint8_t*)k_scales;
    a.bs_k_scales = bs_k_scales;
    a.ring_src = (const uint16_t*)ring_src;
    a.bs_ring_src = bs_ring_src;
    a.ring = (uint16_t*)ring;
    a.bs_ring = bs_ring;
    a.ring_first_t = first_t;
    a.idx = idx;
    a.ld_idx = ld_idx;
    a.ratio = ratio;
    a.n_c = n_c;
    a.K = K;
    a.offset = offset;
    a.idx_vec = al16(idx) && ld_idx % 4 == 0 && win % 4 == 0 && K % 4 == 0;
    const int64_t per_col = a.idx_vec ? 4 : 1;
    const int64_t n_lat = lat ? wgs(n_new * (D / 16)) : 0;
    const int64_t n_k = kk ? wgs(n_new * (Di / 32)) : 0;
    const int64_t n_win = wgs(m * win / per_col);
    const int64_t n_vis = K > 0 ? wgs(m * K / per_col) : 0;
    const int64_t n_ring = ring_src ? wgs((m - first_t) * (D / 8)) : 0;
    const int64_t total = n_lat + n_k + n_win + n_vis + n_ring;
    if (total > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, name + ": too many workgroups for one launch");
    a.w_k = (uint32_t)n_lat;
    a.w_win = (uint32_t)(n_lat + n_k);
    a.w_vis = (uint32_t)(n_lat + n_k + n_win);
    a.w_ring = (uint32_t)(n_lat + n_k + n_win + n_vis);
    prefill_prepare_kernel<<<dim3((unsigned)total, (unsigned)B), dim3(PF_THREADS), 0, (hipStream_t)stream>>>(a);
    return check_launch("sckv_prefill_prepare");
}

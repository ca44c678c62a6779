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
// sum follows the fixed pairwise order (stride Hi/2 first); the q rows sit in
// the MFMA rows so that strides 32, 16, 8, 4 and 2 stay inside a lane and only
// stride 1 is the lane^32 exchange.  Ordered 16-bit keys collect in LDS and leave with
// coalesced stores.  Waves take tiles as they ask for them (an LDS counter),
// so they finish together.  Short fused lists (at most 2048 rows, fp4 k) run
// in a persistent grid of 4-wave workgroups, four to a compute unit.
#include "indexer_dev.h"

namespace sckv {
namespace {

// NWV > 0: workgroups of NWV waves instead of score_waves(FP4), held to the
// registers of four waves a SIMD (four such workgroups a compute unit)
template <int MT, int DI, int KPT, bool FP4, int NWV = 0>
__global__ __launch_bounds__((NWV > 0 ? NWV : score_waves(FP4)) * 64)
__attribute__((amdgpu_waves_per_eu(NWV > 0 ? 4 : 1))) void index_score_kernel(
    const void* __restrict__ q, const void* __restrict__ k,
    const uint8_t* __restrict__ k_scales, const float* __restrict__ w, int64_t m, int Hi, int64_t n_c, int ratio,
    int64_t start_pos, int rows_per_wg, int nsplit, uint16_t* __restrict__ keys, uint16_t* __restrict__ scores, int K,
    int32_t offset, int32_t* __restrict__ idx, int64_t ld, int64_t col0, uint32_t nwork) {
    if constexpr (NWV > 0) {
        // a persistent grid: workgroup g takes work items g, g + gridDim.x, ...
        // (starting a workgroup costs more than a short query's scores)
        for (uint32_t vb = blockIdx.x; vb < nwork; vb += gridDim.x) {
            index_score_body<MT, DI, KPT, FP4, NWV>(q, k, k_scales, w, m, Hi, n_c, ratio, start_pos, rows_per_wg,
                                                    nsplit, keys, scores, K, offset, idx, ld, col0, vb);
            __syncthreads();  // the next item reuses the LDS
        }
    } else {
        index_score_body<MT, DI, KPT, FP4, NWV>(q, k, k_scales, w, m, Hi, n_c, ratio, start_pos, rows_per_wg, nsplit,
                                                keys, scores, K, offset, idx, ld, col0, blockIdx.x);
    }
}

// Compute units of the current device (cached per device; 0 if unknown).
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int KPT>
__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(const uint16_t* __restrict__ keys, int64_t n_c,
                                                            int64_t m, int ratio, int64_t start_pos, int K,
                                                            int32_t offset, int32_t* __restrict__ idx, int64_t ld,
                                                            int64_t col0) {
    topk_body<KPT>(keys, n_c, m, ratio, start_pos, K, offset, idx, ld, col0, blockIdx.x);
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
    else if (kpt <= 16)
        SCKV_TOPK(16);
    else if (kpt <= 32)
        SCKV_TOPK(32);
    else if (kpt <= 64)
        SCKV_TOPK(64);
    else
        SCKV_TOPK(128);
#undef SCKV_TOPK
}

// LDS bytes of a score launch (KPT as in index_score_kernel).
template <int MT, int DI, int KPT, bool FP4, int NWV = 0>
size_t score_lds_bytes(int rows_per_wg, bool with_scores) {
    using Sh = ScoreShape<MT, DI, KPT == 0 ? 0 : fused_ring_depth(DI, KPT, FP4, NWV), FP4, NWV>;
    return Sh::lds_bytes(rows_per_wg, with_scores);
}

// Operands of one indexer call: q (raw bf16), k (bf16 rows, or codes with
// k_scales).
struct IndexArgs {
    const void* q;
    const void* k;
    const uint8_t* k_scales;
    const float* w;
    int64_t nq, m;
    int Hi;
    int64_t n_c;
    int ratio;
    int64_t start_pos;
    int K;
    int32_t offset;
    int32_t* idx;
    int64_t ld, col0;
    uint16_t* scores;
    hipStream_t s;
};

template <int MT, int DI, int KPT, bool FP4, int NWV = 0>
int launch_scores(const IndexArgs& a, int rows_per_wg, int nsplit, uint16_t* keys) {
    const size_t lds = score_lds_bytes<MT, DI, KPT, FP4, NWV>(rows_per_wg, a.scores != nullptr);
    if (lds + SCORE_STATIC_LDS > 160 * 1024)
        return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: score tile does not fit in LDS");
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)index_score_kernel<MT, DI, KPT, FP4, NWV>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return fail(SCKV_EHIP, std::string("sckv_index_scores_topk: ") + hipGetErrorString(e));
    }
    constexpr int nw = NWV > 0 ? NWV : score_waves(FP4);
    const int64_t nwork = a.nq * nsplit;
    int64_t grid = nwork;
    if (NWV > 0) {  // persistent: four workgroups a compute unit
        const int64_t slots = 4 * (int64_t)device_cus();
        if (slots > 0 && grid > slots) grid = slots;
    }
    index_score_kernel<MT, DI, KPT, FP4, NWV><<<dim3((unsigned)grid), dim3(nw * 64), lds, a.s>>>(
        a.q, a.k, a.k_scales, a.w, a.m, a.Hi, a.n_c, a.ratio, a.start_pos, rows_per_wg, nsplit, keys,
        a.scores, a.K, a.offset, a.idx, a.ld, a.col0, (uint32_t)nwork);
    return SCKV_OK;
}

// Fused scores + top-K for one (MT, DI) with KPT keys per thread for the whole
// query; SCKV_EUNSUPPORTED (nothing launched) when it does not fit in LDS.
template <int MT, int DI, bool FP4>
int launch_fused(const IndexArgs& a) {
    const int rows = (int)((a.n_c + 127) / 128 * 128);
    const int nth = score_waves(FP4) * 64;
    const int need = (rows + nth - 1) / nth;
#define SCKV_FUSED(KPT)                                                                           \
    (score_lds_bytes<MT, DI, KPT, FP4>(rows, false) + SCORE_STATIC_LDS > 160 * 1024 ? SCKV_EUNSUPPORTED \
                                                                  : launch_scores<MT, DI, KPT, FP4>(a, rows, 1, nullptr))
    if constexpr (FP4 && DI == 128) {
        // short lists (at most 8 keys a thread at 4 waves): 4-wave workgroups,
        // four of which share a compute unit (LDS and registers allow it), so
        // twice as many queries overlap their latency-bound start and top-K
        if ((rows + 255) / 256 <= 8 && score_lds_bytes<MT, DI, 8, FP4, 4>(rows, false) + SCORE_STATIC_LDS <= 40 * 1024)
            return launch_scores<MT, DI, 8, FP4, 4>(a, rows, 1, nullptr);
    }
    if (need <= 8) return SCKV_FUSED(8);
    if (need <= 16) return SCKV_FUSED(16);
    if (need <= 32) return SCKV_FUSED(32);
    if constexpr (FP4) {  // 512 threads: 64 keys a thread cover n_c <= 32768
        if (need <= 64) return SCKV_FUSED(64);
    } else {
        if (need <= 128) return SCKV_FUSED(128);
    }
#undef SCKV_FUSED
    return SCKV_EUNSUPPORTED;
}

// Scores (+ top-K) for one Di and head tiling; the split path then runs the
// top-k kernel over the keys in the workspace.
template <int MT, int DI, bool FP4>
int run_index(const IndexArgs& a, uint16_t* keys) {
    if (!a.scores && a.nq >= FUSED_MIN_QUERIES && a.n_c <= 32768) {
        // enough queries to fill the chip with one workgroup each: scores and
        // top-K in one launch, the keys never leaving LDS
        const int rc = launch_fused<MT, DI, FP4>(a);
        if (rc != SCKV_EUNSUPPORTED) return rc ? rc : check_launch("sckv_index_scores_topk (fused)");
    }
    const int rpw = score_rows_per_wg(a.nq, a.n_c, a.scores != nullptr);
    const int nsplit = (int)((a.n_c + rpw - 1) / rpw);
    if (a.nq * nsplit > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_index_scores_topk: grid too large");
    int rc = launch_scores<MT, DI, 0, FP4>(a, rpw, nsplit, keys);
    if (rc) return rc;
    rc = check_launch("sckv_index_scores_topk (scores)");
    if (rc) return rc;
    launch_topk(keys, a.nq, a.n_c, a.m, a.ratio, a.start_pos, a.K, a.offset, a.idx, a.ld, a.col0, a.s);
    return check_launch("sckv_index_scores_topk (top-k)");
}

// Host checks shared by both entry points; returns 1 when there is work to do.
int index_checks(const char* name, int B, int64_t m, int Hi, int Di, int64_t n_c, int ratio, int64_t start_pos, int K,
                 int32_t offset, int32_t* idx, int64_t ld, int64_t col0, bool fp4) {
    if (B < 0 || m < 0 || n_c < 0 || ratio <= 0 || start_pos < 0 || K < 0 || col0 < 0 || offset < 0)
        return fail(SCKV_EINVAL, std::string(name) + ": bad sizes");
    if (Hi <= 0 || (Hi & (Hi - 1)) != 0) return fail(SCKV_EINVAL, std::string(name) + ": Hi must be a power of two");
    if (Hi > 64) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": Hi > 64");
    if (fp4 ? (Di != 128 && Di != 256) : (Di != 32 && Di != 64 && Di != 128 && Di != 256))
        return fail(SCKV_EUNSUPPORTED,
                    std::string(name) + (fp4 ? ": Di not in {128, 256}" : ": Di not in {32, 64, 128, 256}"));
    if (B == 0 || m == 0 || K == 0) return 0;
    if (!idx) return fail(SCKV_EINVAL, std::string(name) + ": null idx");
    if (ld < col0 + K) return fail(SCKV_EINVAL, std::string(name) + ": ld < col0 + K");
    if (n_c > 65536 || (int64_t)offset + n_c > 0x7fffffffLL)
        return fail(SCKV_EUNSUPPORTED, std::string(name) + ": n_c > 65536 or offset + n_c >= 2^31");
    if ((int64_t)B * m > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": too many queries");
    return 1;
}

template <bool FP4>
int dispatch_index(int Di, bool two, const IndexArgs& a, uint16_t* keys) {
    if (FP4) {
        if (Di == 128) return two ? run_index<2, 128, true>(a, keys) : run_index<1, 128, true>(a, keys);
        return two ? run_index<2, 256, true>(a, keys) : run_index<1, 256, true>(a, keys);
    }
    switch (Di) {
        case 32: return two ? run_index<2, 32, false>(a, keys) : run_index<1, 32, false>(a, keys);
        case 64: return two ? run_index<2, 64, false>(a, keys) : run_index<1, 64, false>(a, keys);
        case 128: return two ? run_index<2, 128, false>(a, keys) : run_index<1, 128, false>(a, keys);
        default: return two ? run_index<2, 256, false>(a, keys) : run_index<1, 256, false>(a, keys);
    }
}

size_t align256(size_t x) { return (x + 255u) & ~(size_t)255u; }

}  // namespace

size_t index_workspace_bytes(int B, int64_t m, int64_t n_c) {
    // one 16-bit key per (query, compressed row), 256-byte aligned
    return align256((size_t)B * (size_t)m * (size_t)n_c * 2u);
}

size_t index_fp4_workspace_bytes(int B, int64_t m, int64_t n_c) {
    // the keys only: q_hat is packed inside the score kernel
    return index_workspace_bytes(B, m, n_c);
}

}  // namespace sckv

extern "C" int sckv_index_scores_topk(const void* q, const void* k, const float* w, int B, int64_t m, int Hi, int Di,
                                      int64_t n_c, int ratio, int64_t start_pos, int K, int32_t offset,
                                      int32_t* idx, int64_t ld, int64_t col0, void* scores, void* ws,
                                      size_t ws_bytes, void* stream) {
    using namespace sckv;
    const char* name = "sckv_index_scores_topk";
    const int go = index_checks(name, B, m, Hi, Di, n_c, ratio, start_pos, K, offset, idx, ld, col0, false);
    if (go <= 0) return go;
    const int64_t nq = (int64_t)B * m;
    hipStream_t s = (hipStream_t)stream;
    // no compressed row is visible to any query: every list is K x -1 (the pages' empty selection)
    int64_t vmax = (start_pos + m) / ratio;
    vmax = vmax < n_c ? vmax : n_c;
    if (vmax == 0) {
        launch_topk(nullptr, nq, 0, m, ratio, start_pos, K, offset, idx, ld, col0, s);
        return check_launch(name);
    }
    if (!q || !k || !w) return fail(SCKV_EINVAL, "sckv_index_scores_topk: null input");
    if ((uintptr_t)q % 16 || (uintptr_t)k % 16)
        return fail(SCKV_EINVAL, "sckv_index_scores_topk: q and k must be 16-byte aligned");
    if ((uintptr_t)w % 4 || (uintptr_t)idx % 4) return fail(SCKV_EINVAL, "sckv_index_scores_topk: misaligned w/idx");
    if (scores && (uintptr_t)scores % 2) return fail(SCKV_EINVAL, "sckv_index_scores_topk: misaligned scores");
    if (!ws || ws_bytes < index_workspace_bytes(B, m, n_c))
        return fail(SCKV_EWORKSPACE, "sckv_index_scores_topk: workspace too small");
    const IndexArgs a{q, k, nullptr, w, nq, m, Hi, n_c, ratio, start_pos, K, offset, idx, ld, col0,
                      (uint16_t*)scores, s};
    return dispatch_index<false>(Di, Hi > 32, a, (uint16_t*)ws);
}

extern "C" int sckv_index_scores_topk_fp4(const void* q, const void* k_codes, const void* k_scales, const float* w,
                                          int B, int64_t m, int Hi, int Di, int64_t n_c, int ratio, int64_t start_pos,
                                          int K, int32_t offset, int32_t* idx, int64_t ld, int64_t col0,
                                          void* scores, void* ws, size_t ws_bytes, void* stream) {
    using namespace sckv;
    const char* name = "sckv_index_scores_topk_fp4";
    const int go = index_checks(name, B, m, Hi, Di, n_c, ratio, start_pos, K, offset, idx, ld, col0, true);
    if (go <= 0) return go;
    const int64_t nq = (int64_t)B * m;
    hipStream_t s = (hipStream_t)stream;
    int64_t vmax = (start_pos + m) / ratio;
    vmax = vmax < n_c ? vmax : n_c;
    if (vmax == 0) {
        launch_topk(nullptr, nq, 0, m, ratio, start_pos, K, offset, idx, ld, col0, s);
        return check_launch(name);
    }
    if (!q || !k_codes || !k_scales || !w) return fail(SCKV_EINVAL, "sckv_index_scores_topk_fp4: null input");
    if ((uintptr_t)q % 16 || (uintptr_t)k_codes % 16 || (uintptr_t)k_scales % 4)
        return fail(SCKV_EINVAL, "sckv_index_scores_topk_fp4: q / k codes must be 16-byte, k scales 4-byte aligned");
    if ((uintptr_t)w % 4 || (uintptr_t)idx % 4)
        return fail(SCKV_EINVAL, "sckv_index_scores_topk_fp4: misaligned w/idx");
    if (scores && (uintptr_t)scores % 2) return fail(SCKV_EINVAL, "sckv_index_scores_topk_fp4: misaligned scores");
    if (!ws || ws_bytes < index_fp4_workspace_bytes(B, m, n_c))
        return fail(SCKV_EWORKSPACE, "sckv_index_scores_topk_fp4: workspace too small");
    const IndexArgs a{q, k_codes, (const uint8_t*)k_scales, w, nq, m, Hi, n_c, ratio, start_pos, K, offset, idx,
                      ld, col0, (uint16_t*)scores, s};
    return dispatch_index<true>(Di, Hi > 32, a, (uint16_t*)ws);
}

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
// its index list.  Its waves form two sets that take alternate chunks; inside
// a set, wave w owns heads 16w .. 16w+15 over the whole head dim, so a wave
// never needs another wave's numbers until the very end:
//   1. a chunk's rows arrive by asynchronous global->LDS copies
//      (global_load_lds_dwordx4, one instruction per 1 KiB row, fully
//      coalesced), spread over the set's waves and requested one chunk ahead
//      into a two-stage ring per set;
//   2. S^T = R . Q^T on the matrix cores (16x16x32 bf16: rows are M, the
//      wave's 16 heads N, the head dim K; Q^T sits in registers);
//   3. the online softmax runs in the MFMA result layout (a lane holds one
//      head and 8 of the 32 rows; max and sum finish with two lane swaps), in
//      base 2, with a running max that starts at the sink logit and moves only
//      when a logit exceeds it by more than the slack;
//   4. the probabilities are already the A operand of O += P . R (16x16x32
//      again, K = the chunk's rows), whose B operand comes from the same stage
//      through the transposing LDS read (ds_read_b64_tr_b16).
// One barrier per pair of chunks (one per set).  The index slice is staged in
// LDS once (up to 64, 72 or 128 chunks, three kernel variants) with a bitmap
// of the chunks that name a valid row; empty chunks are skipped.  At the end
// the two sets exchange half of O each through LDS, each finishes half of the
// columns, and the rows leave as 16-byte pieces through an LDS staging area.
// A query's chunks may also be split over several workgroups (when the
// queries alone do not fill the chip); their partials are merged by a small
// combine kernel that adds the sink once.
//
// One-set variant (D = 512, 33..64 heads, unsplit lists of at most 72
// chunks, at least two queries per compute unit): a workgroup is one set of
// 4 waves with half the LDS, so two workgroups (two queries) share a compute
// unit and one's start and finish overlap the other's chunk loop.  In it
// P . R is split by columns: after S^T and the softmax each wave publishes
// its 16 heads' probabilities (and, when its running max moved, the rescale
// factors) in LDS, and after one more barrier every wave accumulates O for
// all 64 heads over its own 128 columns, which reads each row byte once per
// wave instead of once per head group.  It accumulates O transposed (the
// same operands in swapped roles), so a lane ends with four consecutive
// columns of one head and packs them without lane shuffles.
//
// Few queries (at most 64): the heads split too, into workgroups of 16 heads
// (grid y), over chunk ranges of at least two chunks, so that one sequence's
// attention spreads over ~40 workgroups with one round of row copies each.
#include <mutex>
#include <string>

#include "attn_dev.h"

namespace sckv {
namespace {

template <int D, int NHW, int CPS, int NS, bool CS, bool PK = false>
__global__ __launch_bounds__(NS * NHW * 64) __attribute__((amdgpu_waves_per_eu(2))) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rows_a, int64_t ra,
    const uint16_t* __restrict__ rows_b, int64_t rb, const int32_t* __restrict__ idx, int T,
    const float* __restrict__ sink, float scale_log2, int64_t m, int H, int chunks_per_split, int nsplit,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
    const uint8_t* __restrict__ rb_scales) {
    sparse_attn_body<D, NHW, CPS, NS, CS, PK>(q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, m, H, chunks_per_split, nsplit, out, part_o, part_ml, rb_scales, blockIdx.x, (int)blockIdx.y * 16 * NHW);
}

__global__ __launch_bounds__(COMBINE_THREADS) void combine_kernel(const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_ml,
                                                                  const float* __restrict__ sink, int nsplit, int H,
                                                                  int D, uint16_t* __restrict__ out) {
    combine_body<COMBINE_THREADS>(part_o, part_ml, sink, nsplit, H, D, out, blockIdx.x, blockIdx.y);
}

// Compute units of the current device (cached per device; 0 if unknown).
int compute_units() {
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

template <int D, int NHW, int CPS, int NS = 2, bool CS = false, bool PK = false>
int launch_attn(const uint16_t* q, const uint16_t* rows_a, int64_t ra, const uint16_t* rows_b, int64_t rb,
                const int32_t* idx, int T, const float* sink, float scale_log2, int64_t nq, int64_t m, int H,
                int cps, int nsplit, uint16_t* out, float* part_o, float* part_ml, hipStream_t s,
                const uint8_t* rb_scales, int hgroups = 1) {
    using Sh = AttnShape<D, NHW, CPS, NS, CS>;
    if (Sh::LDS_BYTES > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)sparse_attn_kernel<D, NHW, CPS, NS, CS, PK>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)Sh::LDS_BYTES);
        if (e != hipSuccess) return fail(SCKV_EHIP, std::string("sckv_sparse_attn_sink: ") + hipGetErrorString(e));
    }
    sparse_attn_kernel<D, NHW, CPS, NS, CS, PK><<<dim3((unsigned)(nq * nsplit), (unsigned)hgroups), dim3(Sh::WAVES * 64), Sh::LDS_BYTES,
                                                 s>>>(q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, m, H, cps,
                                                      nsplit, out, part_o, part_ml, rb_scales);
    return check_launch("sckv_sparse_attn_sink");
}

template <int D, int NHW, bool PK = false>
int launch_attn_c(const uint16_t* q, const uint16_t* rows_a, int64_t ra, const uint16_t* rows_b, int64_t rb,
                  const int32_t* idx, int T, const float* sink, float scale_log2, int64_t nq, int64_t m, int H,
                  int cps, int nsplit, uint16_t* out, float* part_o, float* part_ml, hipStream_t s,
                  const uint8_t* rb_scales, int hgroups = 1) {
    if constexpr (D == 512 && NHW == 4) {
        // unsplit lists of up to 64 chunks and at least two queries per
        // compute unit: one set of 4 waves (76 KB of LDS), so that two
        // workgroups (two queries) share a compute unit and one's start and
        // finish overlap the other's chunk loop (with fewer queries the
        // two-set workgroup keeps 8 waves on each compute unit)
        const int ncu = compute_units();
        const bool one_set = nsplit == 1 && ncu > 0 && nq >= 2 * (int64_t)ncu;
        if (cps <= 64 && one_set)
            return launch_attn<D, NHW, 64, 1, true, PK>(q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, nq, m, H,
                                                        cps, nsplit, out, part_o, part_ml, s, rb_scales);
        // (up to 72 chunks, e.g. a 128-row window plus a top-2048 list: the
        // index buffer still leaves room for two workgroups)
        if (cps <= 72 && one_set)
            return launch_attn<D, NHW, 72, 1, true, PK>(q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, nq, m, H,
                                                        cps, nsplit, out, part_o, part_ml, s, rb_scales);
    }
    if (cps <= 64)
        return launch_attn<D, NHW, 64, 2, false, PK>(q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, nq, m, H,
                                                     cps, nsplit, out, part_o, part_ml, s, rb_scales, hgroups);
    return launch_attn<D, NHW, MAX_CPS, 2, false, PK>(q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, nq, m, H,
                                                      cps, nsplit, out, part_o, part_ml, s, rb_scales, hgroups);
}

template <int D, bool PK = false>
int launch_attn_d(const uint16_t* q, const uint16_t* rows_a, int64_t ra, const uint16_t* rows_b, int64_t rb,
                  const int32_t* idx, int T, const float* sink, float scale_log2, int64_t nq, int64_t m, int H,
                  int cps, int nsplit, uint16_t* out, float* part_o, float* part_ml, hipStream_t s,
                  const uint8_t* rb_scales, int hgroups = 1) {
    // head groups of 16: one 16-head wave per set
    if (H <= 16 || hgroups > 1)
        return launch_attn_c<D, 1, PK>(q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, nq, m, H, cps, nsplit,
                                       out, part_o, part_ml, s, rb_scales, hgroups);
    if (H <= 32)
        return launch_attn_c<D, 2, PK>(q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, nq, m, H, cps, nsplit,
                                       out, part_o, part_ml, s, rb_scales);
    return launch_attn_c<D, 4, PK>(q, rows_a, ra, rows_b, rb, idx, T, sink, scale_log2, nq, m, H, cps, nsplit, out,
                                   part_o, part_ml, s, rb_scales);
}

}  // namespace

size_t attn_workspace_bytes(int B, int64_t m, int H, int D, int64_t T) {
    int cps, nsplit, hgroups;
    attn_split_groups((int64_t)B * m, (int)T, H, &cps, &nsplit, &hgroups);
    return attn_partials_bytes((int64_t)B * m, nsplit, H, D);
}

}  // namespace sckv

namespace sckv {
namespace {

// The whole call (checks, attention launch, combine of split partials) with
// the partials in ws; `name` prefixes error messages.
// rb_scales non-NULL: rows_b is the packed latent cache (codes; see the
// kernel's PK variant), D = 512 only.
int attn_run(const char* name, const void* q, const void* rows_a, int64_t ra, const void* rows_b, int64_t rb,
             const int32_t* idx, int T, const float* sink, float scale, int B, int64_t m, int H, int D, void* out,
             void* ws, size_t ws_bytes, void* stream, const void* rb_scales = nullptr) {
    if (B < 0 || m < 0 || ra < 0 || rb < 0 || H <= 0 || D <= 0 || T < 0)
        return fail(SCKV_EINVAL, std::string(name) + ": bad sizes");
    if (H > 64) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": H > 64");
    if (D != 64 && D != 128 && D != 256 && D != 512)
        return fail(SCKV_EUNSUPPORTED, std::string(name) + ": D not in {64, 128, 256, 512}");
    if (T > 65536) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": T > 65536");
    if (B == 0 || m == 0) return SCKV_OK;
    if (T == 0) return fail(SCKV_EINVAL, std::string(name) + ": T == 0");
    if (!q || !idx || !sink || !out || (ra > 0 && !rows_a) || (rb > 0 && !rows_b))
        return fail(SCKV_EINVAL, std::string(name) + ": null pointer");
    if ((uintptr_t)q % 16 || (uintptr_t)rows_a % 16 || (uintptr_t)rows_b % 16 || (uintptr_t)out % 16 ||
        (uintptr_t)idx % 4 || (uintptr_t)sink % 4)
        return fail(SCKV_EINVAL, std::string(name) + ": q / rows / out must be 16-byte aligned");
    if (ra + rb > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": ra + rb >= 2^31");
    if (!(scale > 0.0f) || !(scale < INFINITY)) return fail(SCKV_EINVAL, std::string(name) + ": bad scale");
    if (rb_scales) {
        if (D != 512) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": packed rows_b at D = 512 only");
        if ((uintptr_t)rb_scales % 16)
            return fail(SCKV_EINVAL, std::string(name) + ": packed rows_b scale bytes must be 16-byte aligned");
    }
    const int64_t nq = (int64_t)B * m;
    int cps, nsplit, hgroups;
    attn_split_groups(nq, T, H, &cps, &nsplit, &hgroups);
    if (nq * nsplit > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": grid too large");
    const size_t need = attn_workspace_bytes(B, m, H, D, T);
    if (need && (!ws || ws_bytes < need)) return fail(SCKV_EWORKSPACE, std::string(name) + ": workspace too small");
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
    const uint8_t* sc = (const uint8_t*)rb_scales;
#define SCKV_ATTN(D)                                                                                              \
    launch_attn_d<D>(qq, aa, ra, bb, rb, idx, T, sink, scale_log2, nq, m, H, cps, nsplit, oo, part_o, part_ml, s, sc, \
                     hgroups)
    if (rb_scales) {
        rc = launch_attn_d<512, true>(qq, aa, ra, bb, rb, idx, T, sink, scale_log2, nq, m, H, cps, nsplit, oo, part_o,
                                      part_ml, s, sc, hgroups);
    } else {
        switch (D) {
            case 64: rc = SCKV_ATTN(64); break;
            case 128: rc = SCKV_ATTN(128); break;
            case 256: rc = SCKV_ATTN(256); break;
            default: rc = SCKV_ATTN(512); break;
        }
    }
#undef SCKV_ATTN
    if (rc || nsplit == 1) return rc;
    if (nq > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": too many queries");
    combine_kernel<<<dim3((unsigned)nq, (unsigned)H), dim3(COMBINE_THREADS), combine_lds_bytes(COMBINE_THREADS, nsplit),
                     s>>>(part_o, part_ml, sink, nsplit, H, D, oo);
    return check_launch(name);
}

// Scratch of the no-allocation entry point: the split partials live in this
// file-scope device array (one copy per GPU, held until the process ends).
// Host code never uses the array's name as an address: it asks the runtime
// for the device address once per device (scratch_ptr) and passes that.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[64] = {nullptr};

// Device address of this device's copy of `scratch` (looked up on the first
// call on each device, with that device current).
int scratch_ptr(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SCKV_EHIP, std::string("sckv_sparse_attn_sink_noalloc: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink_noalloc: device index >= 64");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SCKV_EHIP, std::string("sckv_sparse_attn_sink_noalloc: hipGetSymbolAddress: ") +
                                       hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SCKV_OK;
}

}  // namespace
}  // namespace sckv

extern "C" int sckv_sparse_attn_sink(const void* q, const void* rows_a, int64_t ra, const void* rows_b, int64_t rb,
                                     const int32_t* idx, int T, const float* sink, float scale, int B, int64_t m,
                                     int H, int D, void* out, void* ws, size_t ws_bytes, void* stream) {
    return sckv::attn_run("sckv_sparse_attn_sink", q, rows_a, ra, rows_b, rb, idx, T, sink, scale, B, m, H, D, out,
                          ws, ws_bytes, stream);
}

extern "C" size_t sckv_sparse_attn_sink_noalloc_max_bytes(void) { return sckv::NOALLOC_SCRATCH_BYTES; }

extern "C" int sckv_sparse_attn_sink_noalloc(const void* q, const void* rows_a, int64_t ra, const void* rows_b,
                                             int64_t rb, const int32_t* idx, int T, const float* sink, float scale,
                                             int B, int64_t m, int H, int D, void* out, void* stream) {
    using namespace sckv;
    if (B < 0 || m < 0 || H <= 0 || D <= 0 || T < 0)
        return fail(SCKV_EINVAL, "sckv_sparse_attn_sink_noalloc: bad sizes");
    const size_t need = attn_workspace_bytes(B, m, H, D, T);
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink_noalloc: this shape needs " + std::to_string(need) +
                                           " bytes of split partials, more than the " +
                                           std::to_string(NOALLOC_SCRATCH_BYTES) +
                                           " bytes of static scratch; call sckv_sparse_attn_sink with a workspace");
    void* ws = nullptr;
    if (need) {
        const int rc = scratch_ptr(&ws);
        if (rc) return rc;
    }
    return attn_run("sckv_sparse_attn_sink_noalloc", q, rows_a, ra, rows_b, rb, idx, T, sink, scale, B, m, H, D, out,
                    ws, NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" int sckv_sparse_attn_sink_fp4(const void* q, const void* rows_a, int64_t ra, const void* rows_b_codes,
                                         const void* rows_b_scales, int64_t rb, const int32_t* idx, int T,
                                         const float* sink, float scale, int B, int64_t m, int H, int D, void* out,
                                         void* ws, size_t ws_bytes, void* stream) {
    using namespace sckv;
    if (rb > 0 && !rows_b_scales) return fail(SCKV_EINVAL, "sckv_sparse_attn_sink_fp4: null rows_b scale bytes");
    if (D != 512) return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink_fp4: D must be 512");
    // (no rows_b: the bf16 kernel is the same computation)
    return attn_run("sckv_sparse_attn_sink_fp4", q, rows_a, ra, rows_b_codes, rb, idx, T, sink, scale, B, m, H, D,
                    out, ws, ws_bytes, stream, rb > 0 ? rows_b_scales : nullptr);
}

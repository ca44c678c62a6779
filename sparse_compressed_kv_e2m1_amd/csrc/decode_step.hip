// decode_step.hip -- a whole decode step (m = 1) of a few sequences in one
// launch: the set-up (latent row rotation and round trip, packed indexer k
// row, ring slot, window columns), the indexer scores of every compressed row,
// the per-query top-K, the sparse attention with the sink and the combine of
// its split partials.
//
// Pages: "metrale_model_arch/attn_v41/forward.rs" (AttnV41::forward: the ring
// copy, window_topk_idxs, the indexer with offset = rows_a's length, the merge,
// attend_and_project) and "metrale_model_arch/deepseek_v41_ref/compress.rs"
// (the round trips, yarn_freqs_cis, attention_any).  The pages run this as
// graph segments split by host spans (the index top-k among them); here the
// five parts run as phases of one cooperative launch, separated by grid-wide
// barriers, with the keys, the index lists and the partials handed over in
// device memory.
//
// At small batches a decode step is latency-bound: the separate calls are five
// launches (set-up, scores, top-k, attention, combine) whose launch and drain
// gaps dominate a step that moves ~1.4 MB.  Each phase runs exactly the device
// code of its separate call (the bodies in decode_dev.h, indexer_dev.h and
// attn_dev.h) over the same work split, so the results are bit for bit those of
// sckv_decode_prepare + sckv_index_scores_topk_fp4 + sckv_sparse_attn_sink.
// Every workgroup takes the phases' work items blockIdx.x, blockIdx.x +
// gridDim.x, ...; the grid is at most one workgroup per compute unit, all
// resident (cooperative launch), so every barrier is reached by every
// workgroup.  The barriers are the library's own (grid_barrier below).
#include <mutex>
#include <string>

#include "attn_dev.h"
#include "decode_dev.h"
#include "indexer_dev.h"

namespace sckv {

size_t attn_workspace_bytes(int B, int64_t m, int H, int D, int64_t T);  // attn.hip

namespace {

constexpr int STEP_THREADS = 512;  // 8 waves: the score, top-k and two-set attention workgroups
constexpr int STEP_MAX_B = 64;     // more sequences: the separate calls are as fast
constexpr int STEP_CPS = 64;       // chunks per attention work item at most (the split keeps it far below)

// Grid barrier: workgroups count themselves in `bar` (agent scope: release
// of everything the workgroup wrote, acquire of everything the others wrote)
// and wait for the count of the barrier's generation.  The wait is bounded
// (STEP_SPIN_LIMIT sleeps, about a second): past it the workgroup raises
// `err` and goes on, so every wave always reaches the end.  The cooperative
// launch keeps every workgroup resident, so the bound is never met in a
// correct run.  bar / exitc / err sit in the first 256 bytes of the workspace,
// zero before the first launch; the last workgroup to finish puts bar and
// exitc back to zero for the next launch on the stream.
constexpr uint32_t STEP_SPIN_LIMIT = 1u << 24;

struct StepSync {
    uint32_t* bar;
    uint32_t* exitc;
    uint32_t* err;
};

__device__ __forceinline__ void grid_barrier(const StepSync& g, uint32_t target) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(g.bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t spins = 0;
        while (__hip_atomic_load(g.bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > STEP_SPIN_LIMIT) {
                __hip_atomic_store(g.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

__device__ __forceinline__ void grid_exit(const StepSync& g) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(g.exitc, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {  // every workgroup has passed every barrier
            __hip_atomic_store(g.bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(g.exitc, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

struct StepArgs {
    StepSync sync;
    PrepArgs prep;
    int B;
    // indexer (packed k cache, 64 heads x 128)
    const void* iq;
    const void* k_codes;
    const uint8_t* k_scales;
    const float* w;
    int64_t n_c;
    int ratio;
    int64_t start_pos;
    int K;
    int rows_per_wg;
    int nsplit_s;
    uint16_t* keys;
    int32_t* idx;
    int T;
    int win;
    // attention (D = 512, 33..64 heads)
    const uint16_t* q;
    const uint16_t* ring;
    const uint16_t* latent;
    const float* sink;
    float scale_log2;
    int H;
    int cps;
    int nsplit_a;
    uint16_t* out;
    float* part_o;
    float* part_ml;
};

template <int KPT>
__global__ __launch_bounds__(STEP_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void decode_step_kernel(
    StepArgs a) {
    const uint32_t G = gridDim.x;
    uint32_t gen = 0;  // barriers passed
    // phase 0: set-up, one item per sequence
    for (uint32_t vb = blockIdx.x; vb < (uint32_t)a.B; vb += G) {
        decode_prepare_body(a.prep, vb);
        __syncthreads();
    }
    grid_barrier(a.sync, G * ++gen);
    // phase 1: ordered score keys of row ranges (the split score path)
    const uint32_t n1 = (uint32_t)a.B * (uint32_t)a.nsplit_s;
    for (uint32_t vb = blockIdx.x; vb < n1; vb += G) {
        index_score_body<2, 128, 0, true>(a.iq, a.k_codes, a.k_scales, a.w, 1, 64, a.n_c, a.ratio, a.start_pos,
                                          a.rows_per_wg, a.nsplit_s, a.keys, nullptr, a.K, a.win, a.idx, a.T, a.win,
                                          vb);
        __syncthreads();
    }
    grid_barrier(a.sync, G * ++gen);
    // phase 2: top-K of each query into its index list
    for (uint32_t vb = blockIdx.x; vb < (uint32_t)a.B; vb += G) {
        topk_body<KPT>(a.keys, a.n_c, 1, a.ratio, a.start_pos, a.K, a.win, a.idx, a.T, a.win, vb);
        __syncthreads();
    }
    grid_barrier(a.sync, G * ++gen);
    // phase 3: attention over chunk ranges of the lists (the two-set workgroup);
    // at most two items a workgroup (checked at launch), as two calls: a loop
    // around this body makes the compiler spill
    const uint32_t n3 = (uint32_t)a.B * (uint32_t)a.nsplit_a;
    if (blockIdx.x < n3)
        sparse_attn_body<512, 4, STEP_CPS, 2, false, false>(a.q, a.ring, a.win, a.latent, a.n_c, a.idx, a.T, a.sink,
                                                            a.scale_log2, 1, a.H, a.cps, a.nsplit_a, a.out, a.part_o,
                                                            a.part_ml, nullptr, blockIdx.x);
    __syncthreads();
    if (blockIdx.x + G < n3)
        sparse_attn_body<512, 4, STEP_CPS, 2, false, false>(a.q, a.ring, a.win, a.latent, a.n_c, a.idx, a.T, a.sink,
                                                            a.scale_log2, 1, a.H, a.cps, a.nsplit_a, a.out, a.part_o,
                                                            a.part_ml, nullptr, blockIdx.x + G);
    if (a.nsplit_a > 1) {  // the same for every workgroup
        grid_barrier(a.sync, G * ++gen);
        // phase 4: the log-sum-exp merge of the partials, one item per (query, head)
        const uint32_t n4 = (uint32_t)a.B * (uint32_t)a.H;
        for (uint32_t vb = blockIdx.x; vb < n4; vb += G) {
            combine_body<STEP_THREADS>(a.part_o, a.part_ml, a.sink, a.nsplit_a, a.H, 512, a.out, vb / a.H,
                                       (int)(vb % a.H));
            __syncthreads();
        }
    }
    grid_exit(a.sync);
}

size_t align256(size_t x) { return (x + 255u) & ~(size_t)255u; }

// workspace: 256 bytes of barrier words, the score keys, the attention partials
constexpr size_t STEP_SYNC_BYTES = 256;
size_t step_keys_bytes(int B, int64_t n_c) { return align256((size_t)B * (size_t)n_c * 2u); }

// One launch of the cooperative kernel with the largest grid the work needs
// and the device keeps resident.
constexpr size_t STEP_LDS_MAX = 160 * 1024;  // a compute unit's LDS

// Set-up of the kernel instance on the current device, once per device: the
// compute-unit count, the cooperative-launch check, the dynamic LDS limit
// raised to what a compute unit has beside the kernel's static LDS, and the
// check that one workgroup with that much fits a compute unit (so does every
// smaller request).  Each call then only reads the cached values.
template <int KPT>
int step_device(int& ncu, size_t& lds_max, const char* name) {
    static std::mutex mu;
    static int cus[64] = {0};  // 0: not set up; -1: no cooperative launch
    static size_t dyn[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(SCKV_EHIP, std::string(name) + ": device query failed");
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0, coop = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || n <= 0)
            return fail(SCKV_EHIP, std::string(name) + ": device query failed");
        if (!coop) {
            cus[dev] = -1;
        } else {
            const void* fn = (const void*)decode_step_kernel<KPT>;
            hipFuncAttributes fa;
            hipError_t e = hipFuncGetAttributes(&fa, fn);
            if (e != hipSuccess) return fail(SCKV_EHIP, std::string(name) + ": " + hipGetErrorString(e));
            if (fa.sharedSizeBytes >= STEP_LDS_MAX)
                return fail(SCKV_EUNSUPPORTED, std::string(name) + ": no LDS left beside the static LDS");
            const size_t d = STEP_LDS_MAX - fa.sharedSizeBytes;
            e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)d);
            if (e != hipSuccess) return fail(SCKV_EHIP, std::string(name) + ": " + hipGetErrorString(e));
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, STEP_THREADS, d);
            if (e != hipSuccess || per_cu < 1)
                return fail(SCKV_EUNSUPPORTED, std::string(name) + ": the step's workgroup does not fit a compute unit");
            cus[dev] = n;
            dyn[dev] = d;
        }
    }
    if (cus[dev] < 0) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": no cooperative launch on this device");
    ncu = cus[dev];
    lds_max = dyn[dev];
    return SCKV_OK;
}

template <int KPT>
int launch_step(StepArgs& a, hipStream_t s, const char* name) {
    using SA = AttnShape<512, 4, STEP_CPS, 2, false>;
    using SS = ScoreShape<2, 128, 0, true>;
    const size_t lds_s = SS::lds_bytes(a.rows_per_wg, false);
    const size_t lds = lds_s > SA::LDS_BYTES ? lds_s : (size_t)SA::LDS_BYTES;
    const void* fn = (const void*)decode_step_kernel<KPT>;
    int ncu = 0;
    size_t lds_max = 0;
    if (const int rc = step_device<KPT>(ncu, lds_max, name)) return rc;
    if (lds > lds_max) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": the step needs more LDS than a compute unit has");
    hipError_t e;
    int64_t work = a.B;
    work = work > (int64_t)a.B * a.nsplit_s ? work : (int64_t)a.B * a.nsplit_s;
    work = work > (int64_t)a.B * a.nsplit_a ? work : (int64_t)a.B * a.nsplit_a;
    if (a.nsplit_a > 1) work = work > (int64_t)a.B * a.H ? work : (int64_t)a.B * a.H;
    int64_t G = ncu;  // one workgroup per compute unit at most (it holds ~157 KB of LDS)
    G = G < work ? G : work;
    if ((int64_t)a.B * a.nsplit_a > 2 * G)
        return fail(SCKV_EUNSUPPORTED, std::string(name) + ": more attention work items than twice the grid");
    void* args[] = {&a};
    e = hipLaunchCooperativeKernel(fn, dim3((unsigned)G), dim3(STEP_THREADS), args, (unsigned)lds, s);
    if (e != hipSuccess) return fail(SCKV_EHIP, std::string(name) + ": " + hipGetErrorString(e));
    return check_launch(name);
}

}  // namespace
}  // namespace sckv

extern "C" size_t sckv_decode_step_workspace_bytes(int B, int H, int D, int64_t n_c, int T) {
    using namespace sckv;
    if (B < 0 || H <= 0 || D <= 0 || n_c < 0 || T <= 0) return (size_t)-1;
    int cps, nsplit;
    attn_split(B, T, &cps, &nsplit);
    return STEP_SYNC_BYTES + step_keys_bytes(B, n_c) + align256(attn_partials_bytes(B, nsplit, H, D));
}

extern "C" int sckv_decode_step(const void* lat_new, const void* k_new, const void* kv_new, const float* rope_table,
                                int64_t n_pos, int rope_dim, void* latent, void* k_codes, void* k_scales, void* ring,
                                const void* iq, const float* w, int Hi, int Di, int ratio, int K, const void* q,
                                const float* sink, float scale, int H, int B, int64_t n_c, int D, int win,
                                int64_t start_pos, int32_t* idx, void* out, void* ws, size_t ws_bytes,
                                void* stream) {
    using namespace sckv;
    const char* name = "sckv_decode_step";
    if (B < 0 || n_c < 0 || win <= 0 || start_pos < 0 || K <= 0 || ratio <= 0 || H <= 0)
        return fail(SCKV_EINVAL, std::string(name) + ": bad sizes");
    if (Hi != 64 || Di != 128 || D != 512 || H < 33 || H > 64)
        return fail(SCKV_EUNSUPPORTED, std::string(name) + ": built for 64 x 128 indexer heads, D = 512, 33..64 heads");
    if (B > STEP_MAX_B) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": more than 64 sequences");
    if (n_c < 1 || n_c > 32768) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": n_c outside 1..32768");
    const int64_t T64 = (int64_t)win + K;
    if (T64 > STEP_CPS * 32 * 2) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": win + K above 4096");
    const int T = (int)T64;
    if ((start_pos + 1) / ratio < n_c)
        return fail(SCKV_EINVAL, std::string(name) + ": n_c compressed rows are not all visible at start_pos");
    if (B == 0) return SCKV_OK;
    if (!kv_new || !latent || !k_codes || !k_scales || !ring || !iq || !w || !q || !sink || !idx || !out)
        return fail(SCKV_EINVAL, std::string(name) + ": null pointer");
    if ((lat_new != nullptr) != (k_new != nullptr))
        return fail(SCKV_EINVAL, std::string(name) + ": give both new compressed rows (latent, k) or neither");
    if (lat_new && ((start_pos + 1) % ratio != 0 || (start_pos + 1) / ratio != n_c))
        return fail(SCKV_EINVAL, std::string(name) + ": new compressed rows only at the step that completes row n_c - 1");
    if (rope_table && lat_new &&
        (rope_dim <= 0 || rope_dim % 2 || rope_dim > D || (n_c - 1) * ratio >= n_pos || (uintptr_t)rope_table % 8))
        return fail(SCKV_EINVAL, std::string(name) + ": rotation table, rope_dim or position out of range");
    auto a16 = [](const void* p) { return ((uintptr_t)p % 16) == 0; };
    if (!a16(kv_new) || !a16(latent) || !a16(k_codes) || !a16(ring) || !a16(iq) || !a16(q) || !a16(out) ||
        (lat_new && (!a16(lat_new) || !a16(k_new))) || (uintptr_t)k_scales % 4 || (uintptr_t)w % 4 ||
        (uintptr_t)sink % 4 || (uintptr_t)idx % 16)
        return fail(SCKV_EINVAL, std::string(name) + ": misaligned pointer");
    if (!(scale > 0.0f) || !(scale < INFINITY)) return fail(SCKV_EINVAL, std::string(name) + ": bad scale");
    if (!ws || ws_bytes < sckv_decode_step_workspace_bytes(B, H, D, n_c, T))
        return fail(SCKV_EWORKSPACE, std::string(name) + ": workspace too small");

    StepArgs a{};
    const int64_t f = n_c - 1;  // the completed row, when there is one
    a.prep = PrepArgs{(const uint16_t*)lat_new, D, lat_new ? (uint16_t*)latent + f * D : nullptr, n_c * D,
                      (const uint16_t*)k_new, Di, (uint8_t*)k_codes + f * (Di / 2), n_c * (Di / 2),
                      (uint8_t*)k_scales + f * (Di / 32), n_c * (Di / 32), Di, (const uint16_t*)kv_new, D,
                      (uint16_t*)ring, (int64_t)win * D, D, win, start_pos, idx, T,
                      lat_new ? rope_table : nullptr, rope_dim, f * ratio, nullptr, 0, nullptr, 0};
    a.B = B;
    a.iq = iq;
    a.k_codes = k_codes;
    a.k_scales = (const uint8_t*)k_scales;
    a.w = w;
    a.n_c = n_c;
    a.ratio = ratio;
    a.start_pos = start_pos;
    a.K = K;
    a.rows_per_wg = score_rows_per_wg(B, n_c, false);
    a.nsplit_s = (int)((n_c + a.rows_per_wg - 1) / a.rows_per_wg);
    uint32_t* sw = (uint32_t*)ws;
    a.sync = StepSync{sw, sw + 1, sw + 2};
    a.keys = (uint16_t*)((char*)ws + STEP_SYNC_BYTES);
    a.idx = idx;
    a.T = T;
    a.win = win;
    a.q = (const uint16_t*)q;
    a.ring = (const uint16_t*)ring;
    a.latent = (const uint16_t*)latent;
    a.sink = sink;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    a.H = H;
    attn_split(B, T, &a.cps, &a.nsplit_a);
    if (a.cps > STEP_CPS) return fail(SCKV_EUNSUPPORTED, std::string(name) + ": list too long for one work item");
    char* pw = (char*)ws + STEP_SYNC_BYTES + step_keys_bytes(B, n_c);
    if (a.nsplit_a > 1) {
        a.part_o = (float*)pw;
        a.part_ml = (float*)(pw + align256((size_t)B * a.nsplit_a * H * D * 4u));
    }
    a.out = (uint16_t*)out;
    hipStream_t s = (hipStream_t)stream;
    const int64_t kpt = (n_c + 511) / 512;
    if (kpt <= 16) return launch_step<16>(a, s, name);
    if (kpt <= 32) return launch_step<32>(a, s, name);
    return launch_step<64>(a, s, name);
}

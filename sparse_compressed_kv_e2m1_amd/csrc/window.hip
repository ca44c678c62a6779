// window.hip -- the window ring write and the index-list columns that need no
// scores: the window rows of every query and, on a layer without an indexer,
// every causally visible compressed row.
//
// Page "metrale_model_arch/attn_v41/forward.rs": the ring's stream-ordered
// copies (slot = position mod window), window_topk_idxs (body not printed;
// reading below), offset = rows_a's length, compress_len = (start_pos + m) /
// ratio, and the [window | compressed] merge of each token's list.
#include "sckv_device.h"

namespace sckv {
namespace {

constexpr int RING_THREADS = 256;
constexpr int IDX_THREADS = 256;

// One workgroup copies one (b, position) row into its ring slot with 16-byte
// vectors when aligned.
__global__ __launch_bounds__(RING_THREADS) void ring_write_kernel(const uint16_t* __restrict__ rows,
                                                                  int64_t rows_bstride, uint16_t* __restrict__ ring,
                                                                  int64_t ring_bstride, int64_t m, int64_t first_t,
                                                                  int64_t start_pos, int win, int D, int vec) {
    const int64_t t = first_t + blockIdx.x;
    const int64_t b = blockIdx.y;
    const int64_t slot = (start_pos + t) % win;
    const uint16_t* src = rows + b * rows_bstride + t * D;
    uint16_t* dst = ring + b * ring_bstride + slot * D;
    if (vec) {
        for (int i = threadIdx.x; i < D / 8; i += RING_THREADS)
            reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    } else {
        for (int i = threadIdx.x; i < D; i += RING_THREADS) dst[i] = src[i];
    }
    (void)m;
}

// idx[b, t, j] for j < win: window_col.
__global__ __launch_bounds__(IDX_THREADS) void window_idx_kernel(int64_t m, int64_t start_pos, int win,
                                                                 int32_t* __restrict__ idx, int64_t ld) {
    const int64_t gid = (int64_t)blockIdx.x * IDX_THREADS + threadIdx.x;
    const int64_t t = gid / win;
    const int j = (int)(gid - t * win);
    if (t >= m) return;
    idx[(int64_t)blockIdx.y * m * ld + t * ld + j] = window_col(win, m, start_pos, t, j);
}

// idx[b, t, col0 + j] for j < K: visible_col.
__global__ __launch_bounds__(IDX_THREADS) void visible_idx_kernel(int64_t m, int64_t start_pos, int ratio,
                                                                  int64_t n_c, int K, int32_t offset,
                                                                  int32_t* __restrict__ idx, int64_t ld,
                                                                  int64_t col0) {
    const int64_t gid = (int64_t)blockIdx.x * IDX_THREADS + threadIdx.x;
    const int64_t t = gid / K;
    const int j = (int)(gid - t * K);
    if (t >= m) return;
    idx[(int64_t)blockIdx.y * m * ld + t * ld + col0 + j] = visible_col(start_pos, ratio, n_c, offset, t, j);
}

}  // namespace
}  // namespace sckv

extern "C" int64_t sckv_rows_a_len(int win, int64_t m, int64_t start_pos) {
    if (win <= 0 || m <= 0 || start_pos < 0) return -1;
    if (start_pos == 0) return m;
    if (m == 1) return win;
    return win + m;
}

extern "C" int sckv_ring_write(const void* rows, int64_t rows_bstride, void* ring, int64_t ring_bstride, int B,
                               int64_t m, int64_t start_pos, int win, int D, void* stream) {
    using namespace sckv;
    if (B < 0 || m < 0 || start_pos < 0 || win <= 0 || D <= 0)
        return fail(SCKV_EINVAL, "sckv_ring_write: bad sizes");
    if (B == 0 || m == 0) return SCKV_OK;
    if (!rows || !ring) return fail(SCKV_EINVAL, "sckv_ring_write: null pointer");
    if (rows_bstride < m * D || ring_bstride < (int64_t)win * D)
        return fail(SCKV_EINVAL, "sckv_ring_write: batch stride shorter than one sequence");
    if (B > 65535) return fail(SCKV_EUNSUPPORTED, "sckv_ring_write: B > 65535");
    // every written ring row and every read source row must not overlap
    for (int b = 0; b < (B < 2 ? B : 2); ++b) {
        const uintptr_t rs = (uintptr_t)rows + (uintptr_t)(b * rows_bstride * 2);
        const uintptr_t re = rs + (uintptr_t)(m * D * 2);
        const uintptr_t gs = (uintptr_t)ring + (uintptr_t)(b * ring_bstride * 2);
        const uintptr_t ge = gs + (uintptr_t)((int64_t)win * D * 2);
        if (rs < ge && gs < re) return fail(SCKV_EINVAL, "sckv_ring_write: rows and ring overlap");
    }
    const int64_t first_t = (m > win) ? m - win : 0;
    const int64_t n = m - first_t;
    const int vec = ((uintptr_t)rows % 16 == 0) && ((uintptr_t)ring % 16 == 0) && (D % 8 == 0) &&
                    (rows_bstride % 8 == 0) && (ring_bstride % 8 == 0);
    ring_write_kernel<<<dim3((unsigned)n, (unsigned)B), dim3(RING_THREADS), 0, (hipStream_t)stream>>>(
        (const uint16_t*)rows, rows_bstride, (uint16_t*)ring, ring_bstride, m, first_t, start_pos, win, D, vec);
    return check_launch("sckv_ring_write");
}

extern "C" int sckv_window_idx(int B, int64_t m, int64_t start_pos, int win, int32_t* idx, int64_t ld,
                               void* stream) {
    using namespace sckv;
    if (B < 0 || m < 0 || start_pos < 0 || win <= 0) return fail(SCKV_EINVAL, "sckv_window_idx: bad sizes");
    if (B == 0 || m == 0) return SCKV_OK;
    if (!idx) return fail(SCKV_EINVAL, "sckv_window_idx: null pointer");
    if (ld < win) return fail(SCKV_EINVAL, "sckv_window_idx: ld < win");
    if (B > 65535) return fail(SCKV_EUNSUPPORTED, "sckv_window_idx: B > 65535");
    if (start_pos + m + win > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_window_idx: positions past 2^31");
    const int64_t total = m * win;
    const int64_t grid = (total + IDX_THREADS - 1) / IDX_THREADS;
    window_idx_kernel<<<dim3((unsigned)grid, (unsigned)B), dim3(IDX_THREADS), 0, (hipStream_t)stream>>>(
        m, start_pos, win, idx, ld);
    return check_launch("sckv_window_idx");
}

extern "C" int sckv_visible_idx(int B, int64_t m, int64_t start_pos, int ratio, int64_t n_c, int K,
                                int32_t offset, int32_t* idx, int64_t ld, int64_t col0, void* stream) {
    using namespace sckv;
    if (B < 0 || m < 0 || start_pos < 0 || ratio <= 0 || n_c < 0 || K < 0 || col0 < 0 || offset < 0)
        return fail(SCKV_EINVAL, "sckv_visible_idx: bad sizes");
    if (B == 0 || m == 0 || K == 0) return SCKV_OK;
    if (!idx) return fail(SCKV_EINVAL, "sckv_visible_idx: null pointer");
    if (ld < col0 + K) return fail(SCKV_EINVAL, "sckv_visible_idx: ld < col0 + K");
    if (B > 65535) return fail(SCKV_EUNSUPPORTED, "sckv_visible_idx: B > 65535");
    // the largest visible count is that of the last query
    int64_t vmax = (start_pos + m) / ratio;
    vmax = vmax < n_c ? vmax : n_c;
    if (vmax > K) return fail(SCKV_EINVAL, "sckv_visible_idx: more visible rows than K columns");
    if ((int64_t)offset + K > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_visible_idx: offset + K >= 2^31");
    const int64_t total = m * K;
    const int64_t grid = (total + IDX_THREADS - 1) / IDX_THREADS;
    visible_idx_kernel<<<dim3((unsigned)grid, (unsigned)B), dim3(IDX_THREADS), 0, (hipStream_t)stream>>>(
        m, start_pos, ratio, n_c, K, offset, idx, ld, col0);
    return check_launch("sckv_visible_idx");
}

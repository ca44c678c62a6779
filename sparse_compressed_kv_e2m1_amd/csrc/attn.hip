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
// so every gathered row byte feeds every head.  The NW waves split the head
// dimension D: wave w owns dims [w*DW, (w+1)*DW) of Q, of every row and of O.
// Per chunk:
//   1. each lane resolves one row pointer (row = lane % 32) and loads its wave's
//      dims of that row straight from HBM in MFMA B layout (16 B per lane per
//      k-step);
//   2. S_w = Q[:, dims_w] . R[:, dims_w]^T on the matrix cores;
//   3. the NW partial S tiles meet in LDS; every wave sums them in the same
//      order, so all waves hold bit-identical logits, and reads them back in
//      MFMA A layout (head = lane % 32);
//   4. online softmax per head (running max starts at the sink logit), P in
//      bf16;
//   5. the wave's row slice goes to wave-private LDS transposed (rows along
//      the contraction) and O[:, dims_w] += P . R[:, dims_w] on the matrix cores.
// A query's chunks may be split over several workgroups; their partial
// (max, sum, O) are merged by a small combine kernel that adds the sink once.
#include "mfma.h"
#include "sckv_device.h"

namespace sckv {
namespace {

constexpr int CHUNK = 32;
constexpr int SX_STRIDE = 36;  // floats per head row of a partial S tile (32 + pad, 16-byte aligned)
constexpr int RT_STRIDE = 40;  // bf16 per dim row of a transposed chunk (32 + pad, 16-byte aligned)
constexpr float LOG2E = 1.4426950408889634f;

template <int MT, int DW, int NW>
struct AttnShape {
    static constexpr int HP = MT * 32;           // padded heads
    static constexpr int D = DW * NW;
    static constexpr int KS = DW / 16;           // k-steps of Q.R^T per wave
    static constexpr int NT = DW / 32;           // 32-wide output tiles per wave
    static constexpr int SX_FLOATS = 2 * NW * HP * SX_STRIDE;  // double-buffered partial S
    static constexpr int RT_HALVES = NW * DW * RT_STRIDE;      // transposed chunk, per wave
    static constexpr size_t LDS_BYTES = (size_t)SX_FLOATS * 4 + (size_t)RT_HALVES * 2;
};

template <int MT, int DW, int NW>
__global__ __launch_bounds__(NW * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rows_a, int64_t ra,
    const uint16_t* __restrict__ rows_b, int64_t rb, const int32_t* __restrict__ idx, int T,
    const float* __restrict__ sink, float scale_log2, int64_t m, int H, int chunks_per_split, int nsplit,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml) {
    using S = AttnShape<MT, DW, NW>;
    constexpr int D = S::D;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    float* sx = reinterpret_cast<float*>(lds_raw);
    uint16_t* rt_all = reinterpret_cast<uint16_t*>(lds_raw + (size_t)S::SX_FLOATS * 4);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r_lane = lane & 31;   // row of this lane in B layout / head in A layout
    const int half = lane >> 5;
    const int64_t qi = blockIdx.x / nsplit;
    const int split = (int)(blockIdx.x - qi * nsplit);
    const int64_t b = qi / m;
    const int dim0 = wave * DW;
    uint16_t* rt = rt_all + wave * DW * RT_STRIDE;

    const uint16_t* rows_a_b = rows_a + b * ra * D;
    const uint16_t* rows_b_b = rows_b ? rows_b + b * rb * D : nullptr;
    const int32_t* idx_q = idx + qi * (int64_t)T;

    // ---- Q slice in A layout: head mt*32 + r_lane, dims dim0 + ks*16 + half*8 + 0..7
    const uint16_t* qrow = q + qi * (int64_t)H * D;
    bf16x8 qa[MT][S::KS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int h = mt * 32 + r_lane;
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks)
            qa[mt][ks] = as_bf16x8((h < H) ? load16(qrow + (int64_t)h * D + dim0 + ks * 16 + half * 8)
                                           : u32x4{0, 0, 0, 0});
    }

    // ---- running softmax state per head (A layout: head mt*32 + r_lane)
    float m_run[MT], l_run[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int h = mt * 32 + r_lane;
        m_run[mt] = (h < H) ? sink[h] * LOG2E : 0.0f;
        l_run[mt] = (nsplit == 1) ? 1.0f : 0.0f;  // e^(sink - M) at M = sink; splits add the sink when merged
    }
    f32x16 o[MT][S::NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < S::NT; ++nt) o[mt][nt] = zero16();

    const int nchunks = (T + CHUNK - 1) / CHUNK;
    const int c_begin = split * chunks_per_split;
    int c_end = c_begin + chunks_per_split;
    c_end = c_end < nchunks ? c_end : nchunks;
    int buf = 0;

    for (int c = c_begin; c < c_end; ++c) {
        // 1. resolve this lane's row and load the wave's dims of it
        const int e = c * CHUNK + r_lane;
        const int32_t iv = (e < T) ? idx_q[e] : -1;
        const bool valid = (iv >= 0) && ((int64_t)iv < ra + rb);
        const uint64_t vmask = __ballot(valid) & 0xffffffffull;  // rows 0..31 (both halves agree)
        if (vmask == 0) continue;  // identical decision in every wave of the block
        const uint16_t* rp = nullptr;
        if (valid) rp = ((int64_t)iv < ra) ? rows_a_b + (int64_t)iv * D : rows_b_b + ((int64_t)iv - ra) * D;
        u32x4 rr[S::KS];
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks)
            rr[ks] = valid ? load16(rp + dim0 + ks * 16 + half * 8) : u32x4{0, 0, 0, 0};

        // 2. partial logits over this wave's dims
        f32x16 sp[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            sp[mt] = zero16();
#pragma unroll
            for (int ks = 0; ks < S::KS; ++ks) sp[mt] = mfma32x32x16(qa[mt][ks], as_bf16x8(rr[ks]), sp[mt]);
        }
        // 3. exchange partial tiles: sx[buf][wave][head][row]
        float* sxb = sx + buf * (NW * S::HP * SX_STRIDE);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sxb[(wave * S::HP + mt * 32 + d_row(i, lane)) * SX_STRIDE + r_lane] = sp[mt][i];
        // transposed copy of this wave's rows for P.R (wave-private)
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int d = ks * 16 + half * 8 + e2 * 2;
                rt[d * RT_STRIDE + r_lane] = (uint16_t)(rr[ks][e2] & 0xffffu);
                rt[(d + 1) * RT_STRIDE + r_lane] = (uint16_t)(rr[ks][e2] >> 16);
            }
        __syncthreads();

        // full logits in A layout: head mt*32 + r_lane, rows kr*16 + half*8 + 0..7
        float x[MT][2][8];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int kr = 0; kr < 2; ++kr) {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[mt][kr][j] = 0.0f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    const float* src = sxb + (ww * S::HP + mt * 32 + r_lane) * SX_STRIDE + kr * 16 + half * 8;
                    const float4 a0 = *reinterpret_cast<const float4*>(src);
                    const float4 a1 = *reinterpret_cast<const float4*>(src + 4);
                    x[mt][kr][0] += a0.x;
                    x[mt][kr][1] += a0.y;
                    x[mt][kr][2] += a0.z;
                    x[mt][kr][3] += a0.w;
                    x[mt][kr][4] += a1.x;
                    x[mt][kr][5] += a1.y;
                    x[mt][kr][6] += a1.z;
                    x[mt][kr][7] += a1.w;
                }
            }
        buf ^= 1;

        // 4. online softmax in base 2
        bf16x8 pa[MT][2];
        float alpha[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float cmax = -INFINITY;
#pragma unroll
            for (int kr = 0; kr < 2; ++kr)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int row = kr * 16 + half * 8 + j;
                    const float v = ((vmask >> row) & 1ull) ? x[mt][kr][j] * scale_log2 : -INFINITY;
                    x[mt][kr][j] = v;
                    cmax = fmaxf(cmax, v);
                }
            cmax = fmaxf(cmax, shfl_xor32(cmax));
            const float m_new = fmaxf(m_run[mt], cmax);
            alpha[mt] = exp2f(m_run[mt] - m_new);
            float psum = 0.0f;
#pragma unroll
            for (int kr = 0; kr < 2; ++kr) {
                u32x4 packed;
#pragma unroll
                for (int j2 = 0; j2 < 4; ++j2) {
                    const uint32_t p0 = f32_to_bf16_bits(exp2f(x[mt][kr][2 * j2] - m_new));
                    const uint32_t p1 = f32_to_bf16_bits(exp2f(x[mt][kr][2 * j2 + 1] - m_new));
                    psum += bf16_bits_to_f32(p0) + bf16_bits_to_f32(p1);
                    packed[j2] = p0 | (p1 << 16);
                }
                pa[mt][kr] = as_bf16x8(packed);
            }
            psum += shfl_xor32(psum);
            l_run[mt] = l_run[mt] * alpha[mt] + psum;
            m_run[mt] = m_new;
        }
        // rescale O rows (D layout heads) by their head's alpha
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float a = __shfl(alpha[mt], d_row(i, lane), 64);
#pragma unroll
                for (int nt = 0; nt < S::NT; ++nt) o[mt][nt][i] *= a;
            }

        // 5. O[:, dims_w] += P . R[:, dims_w]
        wave_lds_sync();
#pragma unroll
        for (int nt = 0; nt < S::NT; ++nt) {
            bf16x8 rb2[2];
#pragma unroll
            for (int kr = 0; kr < 2; ++kr)
                rb2[kr] = as_bf16x8(
                    *reinterpret_cast<const u32x4*>(rt + (nt * 32 + r_lane) * RT_STRIDE + kr * 16 + half * 8));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int kr = 0; kr < 2; ++kr) o[mt][nt] = mfma32x32x16(pa[mt][kr], rb2[kr], o[mt][nt]);
        }
        wave_lds_sync();
    }

    // ---- epilogue
    if (nsplit == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int h = mt * 32 + d_row(i, lane);
                const float inv = 1.0f / __shfl(l_run[mt], d_row(i, lane), 64);
                if (h < H) {
                    uint16_t* orow = out + (qi * H + h) * (int64_t)D + dim0;
#pragma unroll
                    for (int nt = 0; nt < S::NT; ++nt)
                        orow[nt * 32 + r_lane] = (uint16_t)f32_to_bf16_bits(o[mt][nt][i] * inv);
                }
            }
    } else {
        const int64_t pbase = (qi * nsplit + split) * (int64_t)H;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int h = mt * 32 + d_row(i, lane);
                if (h < H) {
                    float* prow = part_o + (pbase + h) * D + dim0;
#pragma unroll
                    for (int nt = 0; nt < S::NT; ++nt) prow[nt * 32 + r_lane] = o[mt][nt][i];
                }
            }
            const int h = mt * 32 + r_lane;
            if (wave == 0 && half == 0 && h < H) {
                part_ml[(pbase + h) * 2 + 0] = m_run[mt];
                part_ml[(pbase + h) * 2 + 1] = l_run[mt];
            }
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
    const int cps = (int)((nchunks + want - 1) / want);
    *chunks_per_split = cps;
    *nsplit = (nchunks + cps - 1) / cps;
}

template <int MT, int DW, int NW>
int launch_attn(const uint16_t* q, const uint16_t* rows_a, int64_t ra, const uint16_t* rows_b, int64_t rb,
                const int32_t* idx, int T, const float* sink, float scale_log2, int64_t nq, int64_t m, int H,
                int cps, int nsplit, uint16_t* out, float* part_o, float* part_ml, hipStream_t s) {
    using Sh = AttnShape<MT, DW, NW>;
    if (Sh::LDS_BYTES > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)sparse_attn_kernel<MT, DW, NW>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)Sh::LDS_BYTES);
        if (e != hipSuccess) return fail(SCKV_EHIP, std::string("sckv_sparse_attn_sink: ") + hipGetErrorString(e));
    }
    sparse_attn_kernel<MT, DW, NW><<<dim3((unsigned)(nq * nsplit)), dim3(NW * 64), Sh::LDS_BYTES, s>>>(
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
    launch_attn<MT, DW, NW>(qq, aa, ra, bb, rb, idx, T, sink, scale_log2, nq, m, H, cps, nsplit, oo, part_o, part_ml, s)
    switch (D) {
        case 64: rc = two ? SCKV_ATTN(2, 64, 1) : SCKV_ATTN(1, 64, 1); break;
        case 128: rc = two ? SCKV_ATTN(2, 128, 1) : SCKV_ATTN(1, 128, 1); break;
        case 256: rc = two ? SCKV_ATTN(2, 128, 2) : SCKV_ATTN(1, 128, 2); break;
        default: rc = two ? SCKV_ATTN(2, 128, 4) : SCKV_ATTN(1, 128, 4); break;
    }
#undef SCKV_ATTN
    if (rc || nsplit == 1) return rc;
    if (nq > 0x7fffffffLL) return fail(SCKV_EUNSUPPORTED, "sckv_sparse_attn_sink: too many queries");
    combine_kernel<<<dim3((unsigned)nq, (unsigned)H), dim3(COMBINE_THREADS), 0, s>>>(part_o, part_ml, sink, nsplit, H,
                                                                                    D, oo);
    return check_launch("sckv_sparse_attn_sink (combine)");
}

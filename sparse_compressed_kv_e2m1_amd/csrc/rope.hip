// rope.hip -- the rotation table of the compressed layers' latent rotary
// embedding (page "metrale_model_arch/deepseek_v41_ref/compress.rs":
// yarn_freqs_cis), built on the host once per model, as the pages build it,
// and copied to the device by the caller; sckv_rope_quant_rows and
// sckv_decode_prepare read it there.
//
// Host code only: binary32 arithmetic in the page's order with the host math
// library's powf / cosf / sinf (the table is an input of the hot path, not
// part of any step).
#include <math.h>

#include <string>

#include "sckv_device.h"

extern "C" int sckv_yarn_freqs_cis(float* table, int dim, int64_t seqlen, int64_t original_seq_len, float base,
                                   float factor, float beta_fast, float beta_slow) {
    using namespace sckv;
    const char* name = "sckv_yarn_freqs_cis";
    if (dim <= 0 || dim % 2 != 0 || seqlen < 0 || original_seq_len <= 0)
        return fail(SCKV_EINVAL, std::string(name) + ": dim must be even and positive, seqlen >= 0, "
                                                     "original_seq_len > 0");
    if (!(base > 1.0f) || !(factor > 0.0f) || !(beta_fast > 0.0f) || !(beta_slow > 0.0f) || !std::isfinite(base) ||
        !std::isfinite(factor))
        return fail(SCKV_EINVAL, std::string(name) + ": base must exceed 1; factor and the betas must be positive");
    if (seqlen == 0) return SCKV_OK;
    if (!table) return fail(SCKV_EINVAL, std::string(name) + ": null table");
    const int half = dim / 2;
    std::string err;
    float* freq = new float[half];
    // base frequency of pair i: 1 / base^(2i / dim), binary32 throughout
    for (int i = 0; i < half; ++i) freq[i] = 1.0f / powf(base, (float)(2 * i) / (float)dim);
    // YaRN ramp between the correction dimensions (binary64) of the two
    // rotation counts over the original context
    const double ln_base2 = 2.0 * log((double)base);
    const double pi2 = 2.0 * M_PI;
    const double d_fast = (double)dim * log((double)original_seq_len / ((double)beta_fast * pi2)) / ln_base2;
    const double d_slow = (double)dim * log((double)original_seq_len / ((double)beta_slow * pi2)) / ln_base2;
    const float low = (float)fmax(floor(d_fast), 0.0);
    const float high = (float)fmin(ceil(d_slow), (double)(dim - 1));
    const float width = fmaxf(high - low, 1e-3f);
    for (int i = 0; i < half; ++i) {
        const float ramp = fminf(fmaxf(((float)i - low) / width, 0.0f), 1.0f);
        const float keep = 1.0f - ramp;  // share of the unscaled frequency
        freq[i] = freq[i] / factor * (1.0f - keep) + freq[i] * keep;
    }
    for (int64_t p = 0; p < seqlen; ++p) {
        float* row = table + p * 2 * half;
        for (int i = 0; i < half; ++i) {
            const float angle = (float)p * freq[i];
            row[2 * i] = cosf(angle);
            row[2 * i + 1] = sinf(angle);
        }
    }
    delete[] freq;
    return SCKV_OK;
}

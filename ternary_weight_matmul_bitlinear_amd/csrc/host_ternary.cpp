// host_ternary.cpp -- host-side weight preparation: absmean ternarization and the 2-bit
// packed format of libmmf.
//
// DataCamp "MatMul-free language models", section "Replacing MatMul with ternary
// operations": each weight matrix is scaled by the mean absolute value of its elements and
// every element is rounded to the nearest of -1, 0, 1.  The scale is per matrix.
#include <cmath>
#include <cstdint>

#include "mmf.h"

namespace mmf {
int set_error(int code, const char *fmt, ...);
}

extern "C" int mmf_ternary_quantize(const float *w, int64_t n, int64_t k, int8_t *q_out,
                                    float *scale_out) {
    if (!w || !q_out || !scale_out) return mmf::set_error(MMF_EINVAL, "mmf_ternary_quantize: NULL argument");
    if (n <= 0 || k <= 0) return mmf::set_error(MMF_ESHAPE, "mmf_ternary_quantize: n=%lld k=%lld", (long long)n, (long long)k);
    // mean |w|: each row summed in double with k ascending, the row sums added in double
    // with n ascending, so the result is reproducible bit for bit.
    double total = 0.0;
    for (int64_t r = 0; r < n; ++r) {
        const float *row = w + r * k;
        double rs = 0.0;
        for (int64_t c = 0; c < k; ++c) rs += std::fabs(static_cast<double>(row[c]));
        total += rs;
    }
    const float mean_abs = static_cast<float>(total / (static_cast<double>(n) * static_cast<double>(k)));
    const float s = std::fmax(mean_abs, 1e-5f);
    const int64_t cnt = n * k;
    for (int64_t i = 0; i < cnt; ++i) {
        // fp32 division, round half to even, clamp to the ternary range
        const float v = std::nearbyint(w[i] / s);
        q_out[i] = static_cast<int8_t>(v > 1.0f ? 1.0f : (v < -1.0f ? -1.0f : v));
    }
    *scale_out = s;
    return MMF_OK;
}

// Packed format: code = q + 1; element k = 16j + 4a + b of a row in word j, bits 8b + 2a.
extern "C" int mmf_ternary_pack(const int8_t *q, int64_t n, int64_t k, uint32_t *packed) {
    if (!q || !packed) return mmf::set_error(MMF_EINVAL, "mmf_ternary_pack: NULL argument");
    if (n <= 0 || k <= 0 || k % 16) return mmf::set_error(MMF_ESHAPE, "mmf_ternary_pack: n=%lld k=%lld (k %% 16 != 0?)", (long long)n, (long long)k);
    const int64_t words = k / 16;
    for (int64_t r = 0; r < n; ++r) {
        const int8_t *row = q + r * k;
        for (int64_t j = 0; j < words; ++j) {
            uint32_t acc = 0;
            const int8_t *blk = row + 16 * j;
            for (int b = 0; b < 4; ++b) {
                uint32_t byte = 0;
                for (int a = 0; a < 4; ++a) {
                    const int v = blk[4 * a + b];
                    if (v < -1 || v > 1)
                        return mmf::set_error(MMF_EINVAL, "mmf_ternary_pack: value %d at (%lld, %lld)", v, (long long)r, (long long)(16 * j + 4 * a + b));
                    byte |= static_cast<uint32_t>(v + 1) << (2 * a);
                }
                acc |= byte << (8 * b);
            }
            packed[r * words + j] = acc;
        }
    }
    return MMF_OK;
}

extern "C" int mmf_ternary_unpack(const uint32_t *packed, int64_t n, int64_t k, int8_t *q) {
    if (!q || !packed) return mmf::set_error(MMF_EINVAL, "mmf_ternary_unpack: NULL argument");
    if (n <= 0 || k <= 0 || k % 16) return mmf::set_error(MMF_ESHAPE, "mmf_ternary_unpack: n=%lld k=%lld", (long long)n, (long long)k);
    const int64_t words = k / 16;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < words; ++j) {
            const uint32_t wv = packed[r * words + j];
            // code 3 has both bits of a pair set
            if ((wv & (wv >> 1)) & 0x55555555u)
                return mmf::set_error(MMF_EINVAL, "mmf_ternary_unpack: invalid code 3 in row %lld word %lld", (long long)r, (long long)j);
            for (int b = 0; b < 4; ++b)
                for (int a = 0; a < 4; ++a) {
                    const int code = static_cast<int>((wv >> (8 * b + 2 * a)) & 3u);
                    q[r * k + 16 * j + 4 * a + b] = static_cast<int8_t>(code - 1);
                }
        }
    return MMF_OK;
}

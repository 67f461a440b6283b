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

// HGRN forget-gate lower bounds (Hysen Labs "MatMul-Free LM", section "HGRN attention" names
// the Hierarchical Gated Recurrent Network; the bound follows HGRN's published design): per
// channel, a softmax of the per-layer logits over the layers, accumulated over the layers
// below, so the bottom layer is unbounded and higher layers forget more slowly.
extern "C" int mmf_hgrn_lower_bounds(const float *g, int64_t L, int64_t D, float *lb) {
    if (!g || !lb) return mmf::set_error(MMF_EINVAL, "mmf_hgrn_lower_bounds: NULL argument");
    if (L <= 0 || D <= 0) return mmf::set_error(MMF_ESHAPE, "mmf_hgrn_lower_bounds: L=%lld D=%lld", (long long)L, (long long)D);
    for (int64_t d = 0; d < D; ++d) {
        double top = g[d];
        for (int64_t l = 1; l < L; ++l) top = std::fmax(top, static_cast<double>(g[l * D + d]));
        double norm = 0.0;
        for (int64_t l = 0; l < L; ++l) norm += std::exp(static_cast<double>(g[l * D + d]) - top);
        double below = 0.0;  // softmax mass of the layers under layer l
        for (int64_t l = 0; l < L; ++l) {
            lb[l * D + d] = static_cast<float>(below / norm);
            below += std::exp(static_cast<double>(g[l * D + d]) - top);
        }
    }
    return MMF_OK;
}

// Base-3 packing, five ternary weights per byte (HackerPapers page on arXiv 2406.02528, HN
// discussion list: the weights are ternary digits, "trits"; 3^5 = 243 <= 256).  Codes
// c = q + 1; byte j of 4-byte word w of a row holds k = 20w + 4i + j (i = 0..4, i = 0 the
// most significant base-3 digit) as v = sum_i c_i 3^(4-i), stored as b = ceil(256 v / 243),
// so that digit i is recovered as floor(3 t_i / 256) with t_0 = b, t_{i+1} = 3 t_i mod 256.
// Rows are padded with q = 0 to whole 16-byte chunks of 80 weights.
extern "C" int64_t mmf_trit_row_bytes(int64_t k) { return k > 0 ? 16 * ((k + 79) / 80) : 0; }

extern "C" int mmf_ternary_pack_trits(const int8_t *q, int64_t n, int64_t k, uint8_t *packed) {
    if (!q || !packed) return mmf::set_error(MMF_EINVAL, "mmf_ternary_pack_trits: NULL argument");
    if (n <= 0 || k <= 0) return mmf::set_error(MMF_ESHAPE, "mmf_ternary_pack_trits: n=%lld k=%lld", (long long)n, (long long)k);
    const int64_t rb = mmf_trit_row_bytes(k);
    for (int64_t r = 0; r < n; ++r) {
        const int8_t *row = q + r * k;
        for (int64_t w = 0; w < rb / 4; ++w)
            for (int j = 0; j < 4; ++j) {
                int v = 0;
                for (int i = 0; i < 5; ++i) {
                    const int64_t kk = 20 * w + 4 * i + j;
                    int c = 1;
                    if (kk < k) {
                        if (row[kk] < -1 || row[kk] > 1)
                            return mmf::set_error(MMF_EINVAL, "mmf_ternary_pack_trits: value %d at (%lld, %lld)", row[kk], (long long)r, (long long)kk);
                        c = row[kk] + 1;
                    }
                    v = v * 3 + c;
                }
                packed[r * rb + 4 * w + j] = static_cast<uint8_t>((v * 256 + 242) / 243);
            }
    }
    return MMF_OK;
}

extern "C" int mmf_ternary_unpack_trits(const uint8_t *packed, int64_t n, int64_t k, int8_t *q) {
    if (!q || !packed) return mmf::set_error(MMF_EINVAL, "mmf_ternary_unpack_trits: NULL argument");
    if (n <= 0 || k <= 0) return mmf::set_error(MMF_ESHAPE, "mmf_ternary_unpack_trits: n=%lld k=%lld", (long long)n, (long long)k);
    const int64_t rb = mmf_trit_row_bytes(k);
    for (int64_t r = 0; r < n; ++r)
        for (int64_t by = 0; by < rb; ++by) {
            const uint32_t b = packed[r * rb + by];
            uint32_t t = b, v = 0;
            for (int i = 0; i < 5; ++i) {
                t *= 3;
                const uint32_t c = t >> 8;   // base-3 digit i, most significant first
                t &= 0xFFu;
                v = v * 3 + c;
                const int64_t kk = 20 * (by / 4) + 4 * i + by % 4;
                if (kk < k) q[r * k + kk] = static_cast<int8_t>(static_cast<int>(c) - 1);
                else if (c != 1)
                    return mmf::set_error(MMF_EINVAL, "mmf_ternary_unpack_trits: non-zero padding in row %lld byte %lld", (long long)r, (long long)by);
            }
            if ((v * 256 + 242) / 243 != b)
                return mmf::set_error(MMF_EINVAL, "mmf_ternary_unpack_trits: byte %u in row %lld is not a packed group", b, (long long)r);
        }
    return MMF_OK;
}

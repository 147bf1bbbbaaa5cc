// Device pieces shared by the matrix-core scans of the per-channel store (scan.hip) and
// of the grouped store (grouped.hip): the integer weight digits, the byte transpose
// that turns plane words into MFMA columns, and the fp32 combine of a score.
//
// Source: the blog's "Bit planes" (a t-plane prefix is the t-bit quantizer with the same
// scale) and "How each query picks its own depth": with m = p 2^(4-t) + h(t), the planes
// a channel reads contribute sum_{j<t} bit_j q s 2^(3-j) to a score, so a score is a
// constant plus the product of a token-by-plane bit matrix and a plane-by-query weight
// matrix, which the int8 matrix cores sum exactly once each weight is an integer count
// of a power-of-two unit written as signed base-256 digits.
#pragma once

#include "common.h"

namespace fathom {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;   // LDS pointers
typedef __attribute__((address_space(3))) v2i lds_v2i;

// Signed base-256 digits of M: M = sum_d 256^d digit_d, digits 0..2 in [-128, 127];
// for |M| <= 2^30 the top digit lies in [-64, 64].  With u = M + kDigitBias, bits
// 8d .. 8d+7 of u are digit_d + 128 for d < 3 (adding 128 to each lower digit makes
// it a byte, and the carries line up), and u >> 24 is the top digit.
constexpr long long kDigitBias = 128LL * (1 + 256 + 65536);
// Byte d (0..3) of an operand record: digit d of M as a two's-complement byte, from
// u = M + kDigitBias.
__device__ __forceinline__ uint32_t weight_byte(long long u, int d) {
    return d < kDigits - 1 ? ((uint32_t)(u >> (8 * d)) & 255u) ^ 128u
                           : (uint32_t)(u >> 24) & 255u;
}

// Byte transpose across a quad: lane s holds word M_s; afterwards byte p of lane s's
// result is byte s of M_p (p = 0..3).  Two butterfly stages, each one DPP move of the
// partner's word and one byte permute.
__device__ __forceinline__ uint32_t quad_byte_transpose(uint32_t m, int s) {
    const uint32_t p = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false);
    const uint32_t a = __builtin_amdgcn_perm(p, m, s < 2 ? 0x05040100u : 0x03020706u);
    const uint32_t q = (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0xB1, 0xF, 0xF, false);
    return __builtin_amdgcn_perm(q, a, (s & 1) ? 0x03070105u : 0x06020400u);
}

// One score from its query's 4 digit sums d (column of bit m of a byte): C + (D0 + 256 D1
// + 65536 (D2 + 256 D3)) * S / (byte value of bit m).  small: the head has at most 480
// planes, so D0 + 256 D1 fits int32.
template <int QS>
__device__ __forceinline__ float combined_score(const v4i &d, int m, float C, float S,
                                                bool small) {
    const float lo = small ? (float)(d[0] + d[1] * 256) : fmaf((float)d[1], 256.0f, (float)d[0]);
    const float hi = (float)(d[2] + d[3] * 256);
    const float f = fmaf(hi, 65536.0f, lo);
    const float mult = m < 7 ? S * (1.0f / (float)(1 << m)) : S * (-1.0f / 128.0f);
    return fmaf(f, mult, C);
}

}  // namespace fathom

// Per-channel arithmetic of the ancestry-gathered causal conv1d (LumoTree,
// Sec. V-C: taps in order oldest -> newest, fp32 accumulation, one cast to
// bf16 at the end).  Every kernel that convolves -- the conv kernel and the
// one-launch layer step -- calls these, so a conv output is the same bf16
// value whichever kernel produced it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_tree.h"

namespace gdn {

typedef __bf16 conv_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float conv_f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float conv_silu(float z) {
    // z * sigmoid(z) = z / (1 + 2^(-z log2 e)) on the hardware exp2 and
    // reciprocal (about 1 ulp each, far below the bf16 rounding that
    // follows).  For z below about -88 the exponential is +inf, the
    // reciprocal 0 and the result -0, which is z * sigmoid(z) rounded to
    // bf16 there (|z| e^z < 2^-133).
    const float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
    return z * __builtin_amdgcn_rcpf(1.f + e);
}

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t conv_pack_bf16x2(float a, float b) {
    const conv_bf16x2_t h = __builtin_convertvector((conv_f32x2_t){a, b}, conv_bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// One output channel.  xw[t] is the 32-bit word holding this channel (low
// half when hi == 0, high half when hi == 1) and its neighbour in tap t,
// oldest first, the node itself last (t = W - 1).  wp[p] holds the channel's
// weights (w[2p], w[2p+1] or 0) as a bf16 pair.  The sum starts from the
// bias (0 without one); taps go in pairs through v_dot2_f32_bf16 (exact bf16
// products, fp32 sums), then the activation.
template <int W>
__device__ __forceinline__ float conv_channel(const uint32_t (&xw)[W], int hi, const uint32_t* wp,
                                              bool has_bias, float bias, int act) {
    constexpr int kWP = (W + 1) / 2;
    const uint32_t sel = hi ? 0x07060302u : 0x05040100u;  // halves hi of two words
    float acc = has_bias ? bias : 0.0f;
#pragma unroll
    for (int p = 0; p < kWP; ++p) {
        const uint32_t lo_w = xw[2 * p];
        const uint32_t hi_w = (2 * p + 1 < W) ? xw[2 * p + 1] : 0u;
        const uint32_t xp = __builtin_amdgcn_perm(hi_w, lo_w, sel);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(conv_bf16x2_t, xp),
                                              __builtin_bit_cast(conv_bf16x2_t, wp[p]), acc, false);
    }
    if (act == GDN_ACT_SILU) acc = conv_silu(acc);
    return acc;
}

}  // namespace gdn

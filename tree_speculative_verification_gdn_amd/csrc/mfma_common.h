// Matrix-core helpers shared by the tree-verify kernels and the paired
// layer-step kernel: bf16 operand tiles, fp32 -> bf16 hi + lo splits, the
// conv of staged rows, and the committed state's load / store in whole
// cache-line shapes.
#pragma once

#include "conv_math.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kMfmaPath = 8;  // fused commit: paths up to this long replay on the matrix cores

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kD = 128;
constexpr int kKQStride = 264;   // bf16 row of 128 + 8 bytes pad: conflict-free 8-byte reads

__host__ __device__ inline int align_up(int x, int a) { return (x + a - 1) / a * a; }

__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }

// Conv weights of channel cb + c as tap pairs: word (c * kWP + p) of a
// 128-channel group holds (w[2p], w[2p+1] or 0); thread tid builds word tid.
template <int W>
__device__ __forceinline__ uint32_t conv_weight_word(const uint16_t* w, int cb, int tid) {
    constexpr int kWP = (W + 1) / 2;
    const int c = min(tid / kWP, kD - 1);
    const int p = tid % kWP;
    const uint16_t* row = w + static_cast<size_t>(cb + c) * W;
    const uint32_t lo = row[2 * p];
    const uint32_t hi = row[min(2 * p + 1, W - 1)];
    return lo | ((2 * p + 1 < W ? hi : 0u) << 16);
}

// Conv of 4 channels (8-byte chunk `chunk` of each row) for one node whose
// window rows, oldest first and the node itself last, start at rp[t].
template <int W>
__device__ __forceinline__ uint2 conv4_rows(const char* const (&rp)[W], int chunk, const uint32_t* wv,
                                            const float* bb, bool has_bias, int act) {
    constexpr int kWP = (W + 1) / 2;
    uint32_t xw[W][2];
#pragma unroll
    for (int t = 0; t < W; ++t) {
        const uint2 c2 = *reinterpret_cast<const uint2*>(rp[t] + chunk * 8);
        xw[t][0] = c2.x;
        xw[t][1] = c2.y;
    }
    float z[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t tw[W];
#pragma unroll
        for (int t = 0; t < W; ++t) tw[t] = xw[t][e >> 1];
        z[e] = conv_channel<W>(tw, e & 1, wv + e * kWP, has_bias, bb[e], act);
    }
    return make_uint2(conv_pack_bf16x2(z[0], z[1]), conv_pack_bf16x2(z[2], z[3]));
}

// MFMA operand: 8 bf16 of one 128-element LDS row for k-step s and lane half
// hf.  Slot e of the operand holds element 16s + 4hf + e (e < 4) or
// 16s + 8 + 4hf + (e - 4) (e >= 4).  The B operand built from the state in
// registers uses the same element order, which is all the contraction needs.
__device__ __forceinline__ bf16x8_t lds_operand(const char* base, int row, int s, int hf) {
    const char* p = base + row * kKQStride + (16 * s + 4 * hf) * 2;
    const uint2 lo = *reinterpret_cast<const uint2*>(p);
    const uint2 hi = *reinterpret_cast<const uint2*>(p + 16);
    uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
    return __builtin_bit_cast(bf16x8_t, u);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    const bf16x2_t h = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// Split 8 fp32 values into bf16 hi and lo parts: x ~= hi + lo.
__device__ __forceinline__ void split_hi_lo(const float4& x0, const float4& x1, bf16x8_t& hi,
                                            bf16x8_t& lo) {
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = cvt_pk_bf16(xs[2 * e], xs[2 * e + 1]);
        const float r0 = xs[2 * e] - __uint_as_float(h[e] << 16);
        const float r1 = xs[2 * e + 1] - __uint_as_float(h[e] & 0xffff0000u);
        l[e] = cvt_pk_bf16(r0, r1);
    }
    hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
    lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

// Root path as a bit mask of node indexes (ancestors have smaller indexes, so
// the set bits in ascending order are the path from its root-level node):
// the node at position q, for q below the path length.
template <int KMAX>
__device__ __forceinline__ int path_node(uint64_t pm, int q) {
#pragma unroll
    for (int c = 0; c < KMAX - 1; ++c)
        if (c < q) pm &= pm - 1ull;
    return __builtin_ctzll(pm | (1ull << 63));
}

__device__ __forceinline__ float sumsq_bf16x4(uint2 u) {
    const float a = __uint_as_float(u.x << 16), b = __uint_as_float(u.x & 0xffff0000u);
    const float c = __uint_as_float(u.y << 16), d = __uint_as_float(u.y & 0xffff0000u);
    return fmaf(a, a, fmaf(b, b, fmaf(c, c, d * d)));
}

__device__ __forceinline__ void store_out(void* out, size_t idx, float o, bool out_bf16) {
    if (out_bf16)
        static_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(o);
    else
        static_cast<float*>(out)[idx] = o;
}

// ---------------------------------------------------------------------------
// State traffic in whole cache lines.  The matrix-core layout gives lane
// (row r, half hf) the float4 chunks 2t + hf (t = 0..15) of one state row, so
// a load or store instruction written in that layout touches 32 rows at
// 32 bytes each; measured on this part, a 64 KiB-per-workgroup read + write
// of the state runs about 17% faster when every store instruction covers
// whole 128-byte lines and every load whole 64-byte segments.  The state is
// therefore loaded and stored in those shapes and moved into the matrix-core
// layout (and back, for the store) inside groups of lanes with DPP quad
// permutes: one exchange stage after the load, two before the store.
// ---------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]

constexpr int kDppRowMirror = 0x140;      // lane i of a 16-lane row <- lane 15 - i
constexpr int kDppRowHalfMirror = 0x141;  // lane i of an 8-lane group <- lane 7 - i

template <int CTRL>
__device__ __forceinline__ float dpp1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum of x over the 32 lanes of this lane's half-wave, in every lane of it,
// on the vector ALU (no LDS permute): quads by two quad permutes, 8-lane
// groups by the half-row mirror, 16-lane rows by the row mirror, then the
// two rows of the half-wave combined by a permlane16 swap of the register
// with itself (the even row's value in the first result, the odd row's in
// the second, in both rows).
__device__ __forceinline__ float sum_half_wave(float x) {
    x += dpp1<0xB1>(x);
    x += dpp1<0x4E>(x);
    x += dpp1<kDppRowHalfMirror>(x);
    x += dpp1<kDppRowMirror>(x);
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The value of lane SP of this lane's 8-lane group (lanes 8a .. 8a + 7),
// p = lane & 7, on DPP: the quad broadcast gives lane SP & 3 of this lane's
// own quad; lanes of the other quad take it through the half-row mirror
// (lane 8a + k <- lane 8a + 7 - k, which lies in the other quad).
template <int SP>
__device__ __forceinline__ float group8_lane(float v, int p) {
    const float t = dpp1<(SP & 3) * 0x55>(v);
    const float m = dpp1<kDppRowHalfMirror>(t);
    return ((p ^ SP) & 4) ? m : t;
}

// group8_lane for a position sp in 1 .. 7 known once loops are unrolled
__device__ __forceinline__ float group8_lane_at(float v, int sp, int p) {
    switch (sp) {
        case 1: return group8_lane<1>(v, p);
        case 2: return group8_lane<2>(v, p);
        case 3: return group8_lane<3>(v, p);
        case 4: return group8_lane<4>(v, p);
        case 5: return group8_lane<5>(v, p);
        case 6: return group8_lane<6>(v, p);
        default: return group8_lane<7>(v, p);
    }
}

// The value of lane N_ of this lane's row of 16 lanes, in every lane of the
// row (DPP row_newbcast)
template <int N_>
__device__ __forceinline__ float row16_lane(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N_, 0xF, 0xF, false));
}

// row16_lane for a lane n in 1 .. 15 known once loops are unrolled
__device__ __forceinline__ float row16_lane_at(float v, int n) {
    switch (n) {
        case 1: return row16_lane<1>(v);
        case 2: return row16_lane<2>(v);
        case 3: return row16_lane<3>(v);
        case 4: return row16_lane<4>(v);
        case 5: return row16_lane<5>(v);
        case 6: return row16_lane<6>(v);
        case 7: return row16_lane<7>(v);
        case 8: return row16_lane<8>(v);
        case 9: return row16_lane<9>(v);
        case 10: return row16_lane<10>(v);
        case 11: return row16_lane<11>(v);
        case 12: return row16_lane<12>(v);
        case 13: return row16_lane<13>(v);
        case 14: return row16_lane<14>(v);
        default: return row16_lane<15>(v);
    }
}

template <int CTRL>
__device__ __forceinline__ float4 dpp4(const float4& x) {
    auto m = [](float v) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
    };
    return make_float4(m(x.x), m(x.y), m(x.z), m(x.w));
}

__device__ __forceinline__ float4 sel4(bool c, const float4& a, const float4& b) {
    return make_float4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// Float offset of load s (0..15) of lane (l32 = 2a + i, hf) from the wave's
// 32-row block: row 2a + (s & 1), float4 chunk 4 (s >> 1) + 2i + hf, i.e.
// every instruction reads 16 rows x 64 contiguous bytes.
__device__ __forceinline__ int state_load_lane_off(int l32, int hf) {
    return (l32 >> 1) * 256 + (l32 & 1) * 8 + hf * 4;
}
constexpr int state_load_off(int s) { return (s & 1) * 128 + (s >> 1) * 16; }

// After the loads above arrived: register t of lane (2a + i, hf) must hold
// chunk 2t + hf of row 2a + i.  Load t holds it when t and i have the same
// parity; otherwise the partner lane (i ^ 1) holds it in load t ^ 1.
__device__ __forceinline__ void state_fix_loaded(float4 (&sr)[16], int l32) {
    const bool odd = (l32 & 1) != 0;
#pragma unroll
    for (int t = 0; t < 16; t += 2) {
        const float4 p0 = dpp4<kDppXor1>(sr[t + 1]);
        const float4 p1 = dpp4<kDppXor1>(sr[t]);
        sr[t] = sel4(odd, p0, sr[t]);
        sr[t + 1] = sel4(odd, sr[t + 1], p1);
    }
}

// Store of the state held in the matrix-core layout: store 4m + j of lane
// (l32 = 4a + i, hf) writes chunk 8m + 2i + hf of row 4a + j, which lane
// 4a + j holds in register 4m + i (a 4 x 4 transpose inside each lane quad,
// as two exchange stages, into temporaries: the registers stay as they are),
// so every instruction writes 8 rows' whole 128-byte lines.  One register
// group at a time (scheduling barriers keep the groups' temporaries apart).
__device__ __forceinline__ void state_store_lines(float* wave_base, const float4 (&sr)[16], int l32, int hf) {
    const int i = l32 & 3;
    float* lb = wave_base + (l32 >> 2) * 512 + i * 8 + hf * 4;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float4 y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            y[j] = sel4(((i ^ j) & 1) == 0, sr[4 * m + j], dpp4<kDppXor1>(sr[4 * m + (j ^ 1)]));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4*>(lb + j * 128 + m * 32) =
                sel4(((i ^ j) & 2) == 0, y[j], dpp4<kDppXor2>(y[j ^ 2]));
        __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ bf16x8_t lds_operand_m(const char* base, int stride, int row, int ks,
                                                  int hf) {
    const char* p = base + row * stride + (16 * ks + 4 * hf) * 2;
    const uint2 lo = *reinterpret_cast<const uint2*>(p);
    const uint2 hi = *reinterpret_cast<const uint2*>(p + 16);
    return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Layer-step inputs (kernel argument): the conv input and weights, the
// history buffers, and the previous step's path as resolved rows.
struct LayerIn {
    int C, act, Rp, Lmax;
    const uint16_t* x;
    const uint16_t* w;
    const float* bias;
    const uint16_t* hist_in;
    uint16_t* hist_out;
    uint16_t* y;
    const uint16_t* x_prev;
    const float* alpha_p;
    const float* beta_p;
    const int32_t* path_rows;
    const int32_t* path_n;
    const int32_t* parent;
};

}  // namespace gdn

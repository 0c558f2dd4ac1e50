// Ancestry-gathered causal conv1d (LumoTree, Sec. V-C).  The window of node i
// is its own ancestry (parent, grandparent, ...) continued into the request's
// conv history, exactly as listed in the descriptor's conv_src; taps are
// applied oldest -> newest with float32 accumulation and one bf16 cast at the
// end (the page's point that tap order and cast boundaries fix the recorded
// values).
//
// Layout / schedule: block = (512-channel tile, request).  Each of the 128
// lanes owns 4 consecutive channels (one 8-byte load per row).  The request's
// node rows for those channels are staged once in LDS, so every x element is
// read from HBM once however many descendants tap it; the W-1 history
// entries stay in registers.  HBM-bound: x (node rows), hist, y.
#include "gdn_internal.h"

namespace gdn {

constexpr int kConvThreads = 128;
constexpr int kConvCh = 4;

__device__ __forceinline__ float silu(float z) {
    // z * sigmoid(z), with the exponential taken of a non-positive argument
    const float e = expf(-fabsf(z));
    const float sig = (z >= 0.f) ? 1.f / (1.f + e) : e / (1.f + e);
    return z * sig;
}

template <int W>
__global__ void __launch_bounds__(kConvThreads)
    conv_gather_kernel(int N, int R, int C, int shared, const int32_t* __restrict__ node_row,
                       const int32_t* __restrict__ conv_src, const int32_t* __restrict__ status,
                       const uint16_t* __restrict__ x, const uint16_t* __restrict__ hist, int P,
                       const int32_t* __restrict__ state_idx, const uint16_t* __restrict__ w,
                       const float* __restrict__ bias, int act, uint16_t* __restrict__ y,
                       int32_t* __restrict__ err) {
    constexpr int H = W - 1;
    extern __shared__ uint2 s_x[];  // [N][kConvThreads] node inputs (4 bf16 each)
    __shared__ int32_t s_row[kMaxNodes];
    // tap sources as node indices (>= 0) or history codes -(s+1)
    __shared__ int32_t s_tap[kMaxNodes * (H > 0 ? H : 1)];

    const int b = blockIdx.y;
    const int t = shared ? 0 : b;
    if (status[t] != 0) return;
    const int slot = state_idx[b];
    if (slot < 0 || slot >= P) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, GDN_EV_STATE);
        return;
    }
    const int tid = threadIdx.x;
    int32_t* s_node_of_row = reinterpret_cast<int32_t*>(s_x + static_cast<size_t>(N) * kConvThreads);
    for (int i = tid; i < N; i += kConvThreads) {
        const int row = node_row[static_cast<size_t>(t) * N + i];
        s_row[i] = row;
        s_node_of_row[row] = i;  // rows of a valid tree are injective and < R
    }
    __syncthreads();
    // tap sources as node indices (conv_src only names rows of this tree)
    for (int e = tid; e < N * H; e += kConvThreads) {
        const int sv = conv_src[static_cast<size_t>(t) * N * H + e];
        s_tap[e] = sv >= 0 ? s_node_of_row[sv] : sv;
    }
    const int c0 = min((blockIdx.x * kConvThreads + tid) * kConvCh, C - kConvCh);
    const bool active = (blockIdx.x * kConvThreads + tid) * kConvCh < C;

    // weights w[c][0..W-1] for the 4 channels
    float wt[W][kConvCh];
#pragma unroll
    for (int j = 0; j < kConvCh; ++j)
#pragma unroll
        for (int tap = 0; tap < W; ++tap)
            wt[tap][j] = bf16_bits_to_f32(w[static_cast<size_t>(c0 + j) * W + tap]);
    float bs[kConvCh] = {0.f, 0.f, 0.f, 0.f};
    if (bias) {
#pragma unroll
        for (int j = 0; j < kConvCh; ++j) bs[j] = bias[c0 + j];
    }
    // history entries of this request's slot
    float hs[H > 0 ? H : 1][kConvCh];
#pragma unroll
    for (int m = 0; m < H; ++m) {
        const uint2 hv = *reinterpret_cast<const uint2*>(
            hist + (static_cast<size_t>(slot) * H + m) * C + c0);
        hs[m][0] = __uint_as_float(hv.x << 16);
        hs[m][1] = __uint_as_float(hv.x & 0xffff0000u);
        hs[m][2] = __uint_as_float(hv.y << 16);
        hs[m][3] = __uint_as_float(hv.y & 0xffff0000u);
    }
    // stage node inputs (each lane only ever reads its own column), eight
    // loads in flight at a time
    const size_t xb = static_cast<size_t>(b) * R;
    for (int i0 = 0; i0 < N; i0 += 8) {
        uint2 tmp[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (i0 + u < N)
                tmp[u] = *reinterpret_cast<const uint2*>(x + (xb + s_row[i0 + u]) * C + c0);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (i0 + u < N) s_x[(i0 + u) * kConvThreads + tid] = tmp[u];
    }
    __syncthreads();

    for (int i = 0; i < N; ++i) {
        float z[kConvCh];
#pragma unroll
        for (int tap = 0; tap < H; ++tap) {
            const int sv = s_tap[i * H + tap];
            float xv[kConvCh];
            if (sv >= 0) {
                const uint2 u = s_x[sv * kConvThreads + tid];
                xv[0] = __uint_as_float(u.x << 16);
                xv[1] = __uint_as_float(u.x & 0xffff0000u);
                xv[2] = __uint_as_float(u.y << 16);
                xv[3] = __uint_as_float(u.y & 0xffff0000u);
            } else {
                const int m = -sv - 1;
#pragma unroll
                for (int j = 0; j < kConvCh; ++j) {
                    float hvv = hs[0][j];
#pragma unroll
                    for (int mm = 1; mm < H; ++mm) hvv = (m == mm) ? hs[mm][j] : hvv;
                    xv[j] = hvv;
                }
            }
#pragma unroll
            for (int j = 0; j < kConvCh; ++j)
                z[j] = (tap == 0) ? wt[0][j] * xv[j] : fmaf(wt[tap][j], xv[j], z[j]);
        }
        const uint2 u = s_x[i * kConvThreads + tid];
        float xi[kConvCh] = {__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                             __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
#pragma unroll
        for (int j = 0; j < kConvCh; ++j) {
            float zz = (H == 0) ? wt[H][j] * xi[j] : fmaf(wt[H][j], xi[j], z[j]);
            if (bias) zz += bs[j];
            if (act == GDN_ACT_SILU) zz = silu(zz);
            z[j] = zz;
        }
        uint2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16_bits(z[0])) |
              (static_cast<uint32_t>(f32_to_bf16_bits(z[1])) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16_bits(z[2])) |
              (static_cast<uint32_t>(f32_to_bf16_bits(z[3])) << 16);
        if (active) *reinterpret_cast<uint2*>(y + (xb + s_row[i]) * C + c0) = o;
    }
}

hipError_t launch_conv(const gdn_tree_desc& d, const uint16_t* x, const uint16_t* hist, int P,
                       const int32_t* state_idx, const uint16_t* w, const float* bias,
                       uint16_t* y, int C, int act, int32_t* err, hipStream_t s) {
    const int tile = kConvThreads * kConvCh;
    dim3 grid((C + tile - 1) / tile, d.B);
    const size_t lds = static_cast<size_t>(d.N) * kConvThreads * sizeof(uint2) +
                       static_cast<size_t>(d.R) * sizeof(int32_t);
#define GDN_CONV_CASE(WW)                                                                     \
    case WW:                                                                                  \
        hipLaunchKernelGGL(conv_gather_kernel<WW>, grid, dim3(kConvThreads), lds, s, d.N,     \
                           d.R, C, d.shared, d.node_row, d.conv_src, d.status, x, hist, P,    \
                           state_idx, w, bias, act, y, err);                                  \
        break;
    if (lds > 160 * 1024) return hipErrorNotSupported;
    switch (d.W) {
        GDN_CONV_CASE(1)
        GDN_CONV_CASE(2)
        GDN_CONV_CASE(3)
        GDN_CONV_CASE(4)
        default:
            return hipErrorNotSupported;
    }
#undef GDN_CONV_CASE
    return hipGetLastError();
}

}  // namespace gdn

// Ancestry-gathered causal conv1d (LumoTree, Sec. V-C).  The window of node i
// is its own ancestry (parent, grandparent, ...) continued into the request's
// conv history, exactly as listed in the descriptor's conv_src; the taps are
// summed in float32 (exact bf16 products, taps paired oldest first on the
// packed dot-product instruction) with one bf16 cast at the end (the page's
// point that tap order and cast boundaries fix the recorded values: here the
// conv output is computed once and every later stage reads that bf16 value).
//
// Layout / schedule: workgroup = (channel tile, request), 256 threads.  A row
// of the tile is covered by TL lanes of CPT channels each (one 8- or 16-byte
// access per lane), so the workgroup holds 256/TL rows at a time and walks
// the request's nodes with that stride.  Two memory round trips: (1) the
// tree's rows and tap sources, the request's slot; (2) every node row of the
// tile, the W-1 history entries and the weights, all in flight together.
// Node rows are kept in LDS, so an x element is read from HBM once however
// many descendants tap it.  HBM-bound: x (node rows), hist, y.
#include <type_traits>

#include "conv_math.h"
#include "gdn_internal.h"

namespace gdn {

namespace {
constexpr int kConvThreads = 256;
constexpr int kTileLanes = 32;                          // lanes per row
constexpr int kRowsPerPass = kConvThreads / kTileLanes;  // rows in flight per pass
constexpr int kMaxPasses = (kMaxNodes + kRowsPerPass - 1) / kRowsPerPass;

template <int CPT>
struct Chunk;
template <>
struct Chunk<8> {
    uint4 u;
};
template <>
struct Chunk<4> {
    uint2 u;
};

template <int CPT>
__device__ __forceinline__ Chunk<CPT> load_chunk(const uint16_t* p) {
    Chunk<CPT> c;
    c.u = *reinterpret_cast<const decltype(c.u)*>(p);
    return c;
}

template <int CPT>
__device__ __forceinline__ void unpack(const Chunk<CPT>& c, float* f) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&c.u);
#pragma unroll
    for (int e = 0; e < CPT / 2; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
}  // namespace

// Kernel arguments (by value).  The previous-step fields are read only by
// the publishing variant.
struct ConvKArgs {
    int N, R, C, shared, P, act;
    const int32_t* node_row;
    const int32_t* conv_src;
    const int32_t* status;
    const uint16_t* x;
    uint16_t* hist;
    const int32_t* state_idx;
    const uint16_t* w;
    const float* bias;
    uint16_t* y;
    int32_t* err;
    // previous step: its accepted path resolved to rows and node counts,
    // the previous tree's R and its conv input
    int Rp, Lmax;
    const int32_t* path_rows;
    const int32_t* path_n;
    const uint16_t* x_prev;
};

// bytes of the staged rows (N node rows + W-1 history rows), 16-aligned
__host__ __device__ inline size_t conv_lds_x_bytes(int N, int W, int cpt) {
    return (static_cast<size_t>(N + W - 1) * kTileLanes * (cpt * 2) + 15) / 16 * 16;
}

template <int W, int CPT, int PASSES, bool PUB>
__global__ void __launch_bounds__(kConvThreads) conv_gather_kernel(const ConvKArgs a) {
    const int N = a.N, R = a.R, C = a.C, shared = a.shared, P = a.P, act = a.act;
    const int32_t* __restrict__ node_row = a.node_row;
    const int32_t* __restrict__ conv_src = a.conv_src;
    const int32_t* __restrict__ status = a.status;
    const uint16_t* __restrict__ x = a.x;
    uint16_t* __restrict__ hist = a.hist;
    const int32_t* __restrict__ state_idx = a.state_idx;
    const uint16_t* __restrict__ w = a.w;
    const float* __restrict__ bias = a.bias;
    uint16_t* __restrict__ y = a.y;
    int32_t* __restrict__ err = a.err;
    constexpr int H = W - 1;
    constexpr int TILE = kTileLanes * CPT;  // channels per workgroup
    constexpr int kWP = (W + 1) / 2;        // tap pairs per channel
    constexpr int kWW = CPT * kWP;          // 32-bit words of one lane's weights: tap pairs
    // LDS: x rows of the nodes, then the H history entries, as rows of
    // kTileLanes chunks; the tile's weights and bias; the row -> node map
    extern __shared__ __attribute__((aligned(16))) char lds[];
    Chunk<CPT>* s_x = reinterpret_cast<Chunk<CPT>*>(lds);  // [N + H][kTileLanes]
    // weights word-major: word e of lane chunk c at e * kTileLanes + c, so the
    // lanes of a row read consecutive words (lane-major, 16 words apart, the
    // reads of a half-wave shared a few banks)
    uint32_t* s_w = reinterpret_cast<uint32_t*>(lds + conv_lds_x_bytes(N, W, CPT));  // [kWW][kTileLanes]
    float* s_b = reinterpret_cast<float*>(reinterpret_cast<char*>(s_w) + kTileLanes * kWW * 4);  // [kTileLanes][CPT]
    int32_t* s_node_of_row = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(s_b) + TILE * 4);  // [R]
    __shared__ int32_t s_row[kMaxNodes];
    // LDS row of each tap: a node's row (< N) or history entry m (N + m)
    __shared__ int32_t s_tap[kMaxNodes * (H > 0 ? H : 1)];

    const int b = blockIdx.y;
    const int t = shared ? 0 : b;
    const int tid = threadIdx.x;

    // ---- round trip 1: tree rows, tap sources, the request's slot.  Loads
    // are unconditional, from indexes clamped into range (a load under a
    // per-lane condition becomes a branch that waits for it).
    const int32_t* rows_t = node_row + static_cast<size_t>(t) * N;
    const int32_t* src_t = conv_src + static_cast<size_t>(t) * N * (H > 0 ? H : 1);
    const int my_row = rows_t[min(tid, N - 1)];
    const int my_src = (H > 0) ? src_t[min(tid, N * H - 1)] : 0;  // N * H <= 192 < 256
    const int st = status[t];
    const int slot = state_idx[b];
    // previous step's accepted path (PUB), resolved: the node count n (-1
    // and 0 publish nothing) and the physical rows
    int n = 0, prow = 0;
    if constexpr (PUB) {
        n = min(max(a.path_n[b], -1), a.Lmax);
        prow = a.path_rows[static_cast<size_t>(b) * a.Lmax + min(tid, a.Lmax - 1)];
    }
    // the new tree is convolved only if it is well formed; the publication of
    // the previous path happens either way
    const bool conv_ok = st == 0;
    if (!PUB && !conv_ok) return;
    if (slot < 0 || slot >= P) {
        if ((PUB || conv_ok) && blockIdx.x == 0 && tid == 0) atomicOr(err, GDN_EV_STATE);
        return;
    }
    __shared__ int32_t s_prow[kMaxNodes + 1];
    if constexpr (PUB) s_prow[min(tid, a.Lmax)] = min(max(prow, 0), a.Rp - 1);  // spare entry Lmax
    if (conv_ok) {  // uniform
        for (int r = tid; r < R; r += kConvThreads) s_node_of_row[r] = -1;
    }
    __syncthreads();
    if (conv_ok && tid < N) {
        s_row[tid] = my_row;
        s_node_of_row[my_row] = tid;  // rows of a valid tree are injective and < R
    }
    __syncthreads();
    // tap sources as LDS rows; a source the descriptor build cannot have
    // produced (outside this tree's rows or history) is reported, not followed
    if (conv_ok && tid < N * H) {
        const int sv = my_src;
        int tap = (sv >= 0) ? ((sv < R) ? s_node_of_row[sv] : -1) : N + (-sv - 1);
        const bool bad = (sv >= 0) ? (tap < 0) : (sv < -H);
        if (bad) {
            atomicOr(err, GDN_EV_ROW);
            tap = 0;
        }
        s_tap[tid] = tap;
    }

    // ---- round trip 2: node rows of the tile, history, weights, bias
    const int lane = tid % kTileLanes;
    const int rs = tid / kTileLanes;  // first node of this thread
    const int c0u = blockIdx.x * TILE + lane * CPT;
    const bool active = c0u < C;  // C is a multiple of CPT
    const int c0 = active ? c0u : C - CPT;  // lanes past the end load a valid chunk, store nothing
    const size_t xb = static_cast<size_t>(b) * R;
    constexpr int kPasses = PASSES;  // kPasses * kRowsPerPass >= N
    Chunk<CPT> xin[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int i = rs + p * kRowsPerPass;
        if (conv_ok && p * kRowsPerPass < N)  // uniform: whole passes beyond N are skipped
            xin[p] = load_chunk<CPT>(x + (xb + s_row[min(i, N - 1)]) * C + c0);
    }
    // history entry m = rs (threads with rs >= H load entry H - 1 again); with
    // publication also entry n + rs, which becomes entry rs when the path
    // is shorter than the history
    Chunk<CPT> hc, hc_shift;
    const uint16_t* hs = hist + static_cast<size_t>(slot) * (H > 0 ? H : 1) * C;
    if (H > 0) hc = load_chunk<CPT>(hs + static_cast<size_t>(min(rs, H - 1)) * C + c0);
    if constexpr (PUB) {
        if (H > 0)
            hc_shift = load_chunk<CPT>(hs + static_cast<size_t>(min(max(n, 0) + rs, H - 1)) * C + c0);
    }
    // weights w[c][0..W-1] of the lane's CPT channels as tap pairs per channel,
    // (w[c][2p], w[c][2p+1] or 0).  With W even that is the memory layout:
    // 16-byte group min(rs, ...) per thread (scalar words when not 16-byte
    // aligned); with W odd, thread rs builds channel rs's pairs.
    constexpr int kWG = (kWW + 3) / 4;  // 16-byte groups
    uint4 wg4 = make_uint4(0u, 0u, 0u, 0u);
    const uint16_t* wp = w + static_cast<size_t>(c0) * W;
    if constexpr (W % 2 == 0) {
        const int grp = min(rs, kWG - 1);
        if (CPT == 8) {  // 16-byte aligned: w is, and c0 * W * 2 is a multiple of 16
            wg4 = *reinterpret_cast<const uint4*>(wp + 8 * grp);
        } else {
            uint32_t ww[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int we = min(4 * grp + e, kWW - 1);
                ww[e] = static_cast<uint32_t>(wp[2 * we]) | (static_cast<uint32_t>(wp[2 * we + 1]) << 16);
            }
            wg4 = make_uint4(ww[0], ww[1], ww[2], ww[3]);
        }
    } else {
        const int ch = min(rs, CPT - 1);
        uint32_t ww[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < W; ++t)
            ww[t >> 1] |= static_cast<uint32_t>(wp[ch * W + t]) << (16 * (t & 1));
        wg4 = make_uint4(ww[0], ww[1], ww[2], ww[3]);
    }
    float4 bq = make_float4(0.f, 0.f, 0.f, 0.f);
    if (bias)  // uniform
        bq = make_float4(bias[c0 + 4 * (rs & 1) + 0 < C ? c0 + 4 * (rs & 1) + 0 : c0],
                         bias[c0 + 4 * (rs & 1) + 1 < C ? c0 + 4 * (rs & 1) + 1 : c0],
                         bias[c0 + 4 * (rs & 1) + 2 < C ? c0 + 4 * (rs & 1) + 2 : c0],
                         bias[c0 + 4 * (rs & 1) + 3 < C ? c0 + 4 * (rs & 1) + 3 : c0]);
    // publication (the path resolution validated the path): the x row of
    // path node n + rs - H, oldest first
    const bool pub = PUB && n > 0 && H > 0;
    Chunk<CPT> xp;
    if constexpr (PUB) {
        if (pub) {  // uniform
            const int j = min(max(n + rs - H, 0), n - 1);
            xp = load_chunk<CPT>(a.x_prev + (static_cast<size_t>(b) * a.Rp + s_prow[j]) * C + c0);
        }
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int i = rs + p * kRowsPerPass;
        if (conv_ok && i < N) s_x[i * kTileLanes + lane] = xin[p];
    }
    if constexpr (PUB) {
        // the old history must be in registers before any lane overwrites it
        if (H > 0) {
            const uint32_t* h0 = reinterpret_cast<const uint32_t*>(&hc.u);
            const uint32_t* h1 = reinterpret_cast<const uint32_t*>(&hc_shift.u);
#pragma unroll
            for (int e = 0; e < CPT / 2; ++e) asm volatile("" ::"v"(h0[e]), "v"(h1[e]));
        }
        __syncthreads();
        if (pub) {  // new entry m = rs: old entry n + rs, or the x row above
            hc = (n + rs < H) ? hc_shift : xp;
            if (rs < H && active)
                *reinterpret_cast<decltype(hc.u)*>(hist + (static_cast<size_t>(slot) * H + rs) * C + c0) = hc.u;
        }
    }
    if (H > 0 && rs < H) s_x[(N + rs) * kTileLanes + lane] = hc;
    {
        const uint32_t wv[4] = {wg4.x, wg4.y, wg4.z, wg4.w};
        if constexpr (W % 2 == 0) {
            if (rs < kWG) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * rs + e < kWW) s_w[(4 * rs + e) * kTileLanes + lane] = wv[e];
            }
        } else if (rs < CPT) {
#pragma unroll
            for (int q = 0; q < kWP; ++q) s_w[(rs * kWP + q) * kTileLanes + lane] = wv[q];
        }
    }
    if (bias && rs < CPT / 4) *reinterpret_cast<float4*>(s_b + lane * CPT + 4 * rs) = bq;
    __syncthreads();
    if (!active || !conv_ok) return;

    // taps in bf16 pairs on v_dot2_f32_bf16 (exact bf16 products, fp32 sums):
    // for channel c and pair p, (x of tap 2p, x of tap 2p+1) . (w[c][2p], w[c][2p+1])
    uint32_t wr[kWW];
#pragma unroll
    for (int e = 0; e < kWW; ++e) wr[e] = s_w[e * kTileLanes + lane];
    constexpr int NW = CPT / 2;  // 32-bit words of a row chunk
    float bl[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) bl[c] = bias ? s_b[lane * CPT + c] : 0.0f;
    // one copy of the loop per (bias, activation) pair: both are uniform, and
    // fixing them outside the loop leaves only the arithmetic they need
    auto rows = [&](auto with_bias, auto silu) {
        constexpr bool kBias = decltype(with_bias)::value;
        constexpr int kAct = decltype(silu)::value ? GDN_ACT_SILU : GDN_ACT_NONE;
        for (int i = rs; i < N; i += kRowsPerPass) {
            // the node's window, oldest first: its H taps, then the node itself
            uint32_t xw[W][NW];
#pragma unroll
            for (int t = 0; t < W; ++t) {
                const int row = (t < H) ? s_tap[i * H + t] : i;
                const Chunk<CPT> ch = s_x[row * kTileLanes + lane];
                const uint32_t* cw = reinterpret_cast<const uint32_t*>(&ch.u);
#pragma unroll
                for (int q = 0; q < NW; ++q) xw[t][q] = cw[q];
            }
            float z[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                uint32_t tw[W];
#pragma unroll
                for (int t = 0; t < W; ++t) tw[t] = xw[t][c >> 1];
                z[c] = conv_channel<W>(tw, c & 1, &wr[c * kWP], kBias, bl[c], kAct);
            }
            Chunk<CPT> o;
            uint32_t* ow = reinterpret_cast<uint32_t*>(&o.u);
#pragma unroll
            for (int e = 0; e < CPT / 2; ++e) ow[e] = conv_pack_bf16x2(z[2 * e], z[2 * e + 1]);
            *reinterpret_cast<decltype(o.u)*>(y + (xb + s_row[i]) * C + c0) = o.u;
        }
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    if (act == GDN_ACT_SILU) {
        if (bias) rows(yes{}, yes{});
        else rows(no{}, yes{});
    } else {
        if (bias) rows(yes{}, no{});
        else rows(no{}, no{});
    }
}

size_t conv_lds_bytes(int N, int R, int W, int cpt) {
    return conv_lds_x_bytes(N, W, cpt) + static_cast<size_t>(kTileLanes) * (cpt * ((W + 1) / 2)) * 4 +
           static_cast<size_t>(kTileLanes) * cpt * 4 + static_cast<size_t>(R) * sizeof(int32_t);
}

hipError_t launch_conv(const gdn_tree_desc& d, const uint16_t* x, const uint16_t* hist, int P,
                       const int32_t* state_idx, const uint16_t* w, const float* bias,
                       uint16_t* y, int C, int act, int32_t* err, hipStream_t s,
                       const ConvPublish* pub) {
    // 16-byte accesses when every 8-channel group is 16-byte aligned
    const bool wide = (C % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                      (reinterpret_cast<uintptr_t>(y) % 16 == 0) &&
                      (hist == nullptr || reinterpret_cast<uintptr_t>(hist) % 16 == 0) &&
                      (reinterpret_cast<uintptr_t>(w) % 16 == 0) &&
                      (pub == nullptr || reinterpret_cast<uintptr_t>(pub->x_prev) % 16 == 0);
    const int cpt = wide ? 8 : 4;
    const int tile = kTileLanes * cpt;
    dim3 grid((C + tile - 1) / tile, d.B);
    const size_t lds = conv_lds_bytes(d.N, d.R, d.W, cpt);
    if (lds > 60 * 1024) return hipErrorNotSupported;  // plus static LDS, within the 64 KiB default
    ConvKArgs a{};
    a.N = d.N; a.R = d.R; a.C = C; a.shared = d.shared; a.P = P; a.act = act;
    a.node_row = d.node_row; a.conv_src = d.conv_src; a.status = d.status;
    a.x = x; a.hist = const_cast<uint16_t*>(hist); a.state_idx = state_idx; a.w = w; a.bias = bias;
    a.y = y; a.err = err;
    if (pub != nullptr) {
        a.Rp = pub->prev->R;
        a.Lmax = pub->Lmax;
        a.path_rows = pub->path_rows;
        a.path_n = pub->path_n;
        a.x_prev = pub->x_prev;
    }
    const bool small = d.N <= (kMaxPasses / 2) * kRowsPerPass;  // fewer row registers
#define GDN_CONV_LAUNCH(WW, CC, PP)                                                               \
    do {                                                                                          \
        if (pub)                                                                                  \
            hipLaunchKernelGGL((conv_gather_kernel<WW, CC, PP, true>), grid, dim3(kConvThreads), \
                               lds, s, a);                                                        \
        else                                                                                      \
            hipLaunchKernelGGL((conv_gather_kernel<WW, CC, PP, false>), grid, dim3(kConvThreads),\
                               lds, s, a);                                                        \
    } while (0)
#define GDN_CONV_CASE(WW)                                                   \
    case WW:                                                                \
        if (wide) {                                                         \
            if (small) GDN_CONV_LAUNCH(WW, 8, kMaxPasses / 2);              \
            else GDN_CONV_LAUNCH(WW, 8, kMaxPasses);                        \
        } else {                                                            \
            if (small) GDN_CONV_LAUNCH(WW, 4, kMaxPasses / 2);              \
            else GDN_CONV_LAUNCH(WW, 4, kMaxPasses);                        \
        }                                                                   \
        break;
    switch (d.W) {
        GDN_CONV_CASE(1)
        GDN_CONV_CASE(2)
        GDN_CONV_CASE(3)
        GDN_CONV_CASE(4)
        default:
            return hipErrorNotSupported;
    }
#undef GDN_CONV_CASE
#undef GDN_CONV_LAUNCH
    return hipGetLastError();
}

}  // namespace gdn

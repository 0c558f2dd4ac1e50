// Accepted-path commit on gfx950 (LumoTree, Sec. IV-B: the accepted path's
// recorded operands are replayed through the gated delta update in place
// into the fp32 state bank; Sec. V-A: the same device-side path drives the
// conv-history publication; Bole review, Algorithm 2 step 8: an empty path
// leaves the state as it was).
//
//   S <- S_pre;  for j < len:  u = b_j (v_j - a_j S k_j);  S <- a_j S + u k_j^T
//   hist[slot] <- last W-1 entries of (hist[slot] ++ x rows of the path)
//
// One 256-thread workgroup per (request, value head).  The 64 KiB (d = 128)
// fp32 state lives in VGPRs for the whole replay: each value row is held by
// 256/d adjacent lanes, so S k_j is a lane-local dot product plus a
// log2(256/d)-step butterfly.  The path's k/v rows are staged in LDS once.
// The kernel reads the state once and writes it once: HBM-bound.
// The workgroup of value head h also publishes the conv history for channel
// slice h of the request.
#include "gdn_internal.h"

namespace gdn {

namespace {
constexpr int kThreads = 256;

struct CommitLds {
    int K, V, al, be, rows, total;
};

__host__ __device__ inline int align16(int x) { return (x + 15) / 16 * 16; }

__host__ __device__ inline CommitLds commit_lds_layout(int Lmax, int D) {
    CommitLds L;
    int off = 0;
    const int lm = Lmax > 0 ? Lmax : 1;
    L.K = off;
    off += align16(lm * D * 4);
    L.V = off;
    off += align16(lm * D * 4);
    L.al = off;
    off += align16(lm * 4);
    L.be = off;
    off += align16(lm * 4);
    L.rows = off;
    off += align16(lm * 4);
    L.total = off;
    return L;
}
}  // namespace

size_t commit_lds_bytes(int Lmax, int D) { return static_cast<size_t>(commit_lds_layout(Lmax, D).total); }

template <typename T>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}

template <int D, typename T>
__global__ void __launch_bounds__(kThreads)
    commit_kernel(int B, int N, int R, int W, int shared, const int32_t* __restrict__ parent,
                  const int32_t* __restrict__ node_row, const int32_t* __restrict__ status,
                  const int32_t* __restrict__ path, const int32_t* __restrict__ path_len, int Lmax,
                  const T* __restrict__ k, const T* __restrict__ v, int64_t rs_qk, int64_t rs_v,
                  const float* __restrict__ alpha, const float* __restrict__ beta,
                  float* __restrict__ pool, int P, const int32_t* __restrict__ state_idx,
                  const uint16_t* __restrict__ x, uint16_t* __restrict__ hist, int C, int Hqk,
                  int Hv, int norm, int32_t* __restrict__ err) {
    constexpr int TPR = kThreads / D;  // lanes per value row
    constexpr int EPT = D / TPR;
    constexpr int NQ = EPT / 4;
    constexpr int CPR = D / 4;                                   // 4-element chunks per row
    constexpr int kItems = GDN_MAX_NODES * CPR / kThreads;       // staging chunks per thread
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const CommitLds L = commit_lds_layout(Lmax, D);
    float* s_K = reinterpret_cast<float*>(lds + L.K);
    float* s_V = reinterpret_cast<float*>(lds + L.V);
    float* s_al = reinterpret_cast<float*>(lds + L.al);
    float* s_be = reinterpret_cast<float*>(lds + L.be);
    int32_t* s_rows = reinterpret_cast<int32_t*>(lds + L.rows);
    __shared__ int s_bad;

    const uint32_t unit = xcd_local_order(blockIdx.x, gridDim.x);
    const int b = static_cast<int>(unit / Hv);
    const int h = static_cast<int>(unit % Hv);
    const int t = shared ? 0 : b;
    if (status[t] != 0) return;  // malformed tree: reported by the descriptor build
    const int tid = threadIdx.x;
    const int slot = state_idx[b];
    const int len = path_len[b];
    const int r = tid / TPR;
    const int part = tid % TPR;

    // the state load goes out first; it is only kept if the request validates
    const bool slot_ok = slot >= 0 && slot < P;
    float* Sb = pool + (static_cast<size_t>(slot_ok ? slot : 0) * Hv + h) * (D * D) +
                static_cast<size_t>(r) * D;
    float4 sv[NQ];
    if (slot_ok && len > 0) {
#pragma unroll
        for (int c = 0; c < NQ; ++c)
            sv[c] = *reinterpret_cast<const float4*>(Sb + 4 * (part + TPR * c));
    }

    // ---- validation (every workgroup of the request reaches the same verdict)
    if (tid == 0) s_bad = 0;
    __syncthreads();
    int bad = slot_ok ? 0 : GDN_EV_STATE;
    for (int b2 = tid; b2 < B; b2 += kThreads)
        if (b2 != b && state_idx[b2] == slot) bad |= GDN_EV_STATE;
    if (len < 0 || len > Lmax) {
        bad |= GDN_EV_PATH;
    } else if (tid < len) {
        const int nd = path[static_cast<size_t>(b) * Lmax + tid];
        if (nd < 0 || nd >= N) {
            bad |= GDN_EV_PATH;
        } else {
            const int want = (tid == 0) ? -1 : path[static_cast<size_t>(b) * Lmax + tid - 1];
            if (parent[static_cast<size_t>(t) * N + nd] != want) bad |= GDN_EV_PATH;
            const int row = node_row[static_cast<size_t>(t) * N + nd];
            s_rows[tid] = row;
            const size_t gi = (static_cast<size_t>(b) * R + row) * Hv + h;
            s_al[tid] = alpha[gi];
            s_be[tid] = beta[gi];
        }
    }
    if (bad) atomicOr(&s_bad, bad);
    __syncthreads();
    bad = s_bad;
    if (bad) {
        if (h == 0 && tid == 0) atomicOr(err, bad);
        return;
    }
    if (len == 0) return;  // nothing accepted: state and history stay as they are

    // ---- stage the path's k (normalised if asked) and v rows, loads batched
    const int g = static_cast<int>((static_cast<int64_t>(h) * Hqk) / Hv);
    {
        float4 kc[kItems], vc[kItems];
#pragma unroll
        for (int u = 0; u < kItems; ++u) {
            const int it = tid + u * kThreads;
            const int j = it / CPR;
            const int ch = it % CPR;
            kc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            vc[u] = kc[u];
            if (j < len) {
                const size_t rb = static_cast<size_t>(b) * R + s_rows[j];
                kc[u] = load4(k + rb * rs_qk + static_cast<size_t>(g) * D + 4 * ch);
                vc[u] = load4(v + rb * rs_v + static_cast<size_t>(h) * D + 4 * ch);
            }
        }
#pragma unroll
        for (int u = 0; u < kItems; ++u) {
            const int it = tid + u * kThreads;
            const int j = it / CPR;
            const int ch = it % CPR;
            float sc = 1.0f;
            if (norm) {  // the CPR chunks of a row sit in CPR consecutive lanes
                float ss = fmaf(kc[u].x, kc[u].x, fmaf(kc[u].y, kc[u].y,
                                fmaf(kc[u].z, kc[u].z, kc[u].w * kc[u].w)));
#pragma unroll
                for (int off = CPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
                sc = 1.0f / sqrtf(ss + 1e-6f);
            }
            if (j < len) {
                *reinterpret_cast<float4*>(s_K + j * D + 4 * ch) =
                    make_float4(kc[u].x * sc, kc[u].y * sc, kc[u].z * sc, kc[u].w * sc);
                *reinterpret_cast<float4*>(s_V + j * D + 4 * ch) = vc[u];
            }
        }
    }

    // ---- conv history of this request, channel slice h: last W-1 entries of
    //      (old history ++ x rows of the path); all loads before any store
    const int H = W - 1;
    if (x != nullptr && hist != nullptr && H > 0) {
        const int per = (C + Hv - 1) / Hv;
        const int c_begin = h * per;
        const int c_end = min(C, c_begin + per);
        for (int c = c_begin + tid; c < c_end; c += kThreads) {
            uint16_t* hp = hist + static_cast<size_t>(slot) * H * C + c;
            uint16_t nv[GDN_MAX_CONV_W - 1];
#pragma unroll
            for (int m = 0; m < GDN_MAX_CONV_W - 1; ++m) {
                if (m < H) {
                    const int pos = len + m;  // position in (old ++ path rows)
                    nv[m] = (pos < H) ? hp[static_cast<size_t>(pos) * C]
                                      : x[(static_cast<size_t>(b) * R + s_rows[pos - H]) * C + c];
                }
            }
#pragma unroll
            for (int m = 0; m < GDN_MAX_CONV_W - 1; ++m)
                if (m < H) hp[static_cast<size_t>(m) * C] = nv[m];
        }
    }
    __syncthreads();

    // ---- replay
    for (int j = 0; j < len; ++j) {
        const float* kj = s_K + j * D;
        float4 kr[NQ];
        float y = 0.f;
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            kr[c] = *reinterpret_cast<const float4*>(kj + 4 * (part + TPR * c));
            y = fmaf(sv[c].x, kr[c].x, y);
            y = fmaf(sv[c].y, kr[c].y, y);
            y = fmaf(sv[c].z, kr[c].z, y);
            y = fmaf(sv[c].w, kr[c].w, y);
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) y += __shfl_xor(y, off, 64);
        const float a = s_al[j];
        const float u = s_be[j] * (s_V[j * D + r] - a * y);
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            sv[c].x = fmaf(a, sv[c].x, u * kr[c].x);
            sv[c].y = fmaf(a, sv[c].y, u * kr[c].y);
            sv[c].z = fmaf(a, sv[c].z, u * kr[c].z);
            sv[c].w = fmaf(a, sv[c].w, u * kr[c].w);
        }
    }
#pragma unroll
    for (int c = 0; c < NQ; ++c) *reinterpret_cast<float4*>(Sb + 4 * (part + TPR * c)) = sv[c];
}

namespace {
template <int D, typename T>
hipError_t launch_commit_t(const gdn_tree_desc& d, const CommitArgs& a, int norm, size_t lds,
                           hipStream_t s) {
    auto kfn = commit_kernel<D, T>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(d.B) * static_cast<unsigned>(a.Hv));
    hipLaunchKernelGGL(kfn, grid, dim3(kThreads), lds, s, d.B, d.N, d.R, d.W, d.shared, d.parent,
                       d.node_row, d.status, a.path, a.path_len, a.Lmax,
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.rs_qk, a.rs_v,
                       a.alpha, a.beta, a.pool, a.P, a.state_idx, a.x, a.hist, a.C, a.Hqk, a.Hv,
                       norm, a.err);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_commit(const gdn_tree_desc& d, const CommitArgs& a, hipStream_t s) {
    const int norm = (a.flags & GDN_F_NORM_QK) ? 1 : 0;
    const size_t lds = commit_lds_bytes(a.Lmax, a.D);
    if (lds > 160 * 1024) return hipErrorNotSupported;
    const bool bf = a.dtype == GDN_DT_BF16;
    switch (a.D) {
        case 32:
            return bf ? launch_commit_t<32, uint16_t>(d, a, norm, lds, s)
                      : launch_commit_t<32, float>(d, a, norm, lds, s);
        case 64:
            return bf ? launch_commit_t<64, uint16_t>(d, a, norm, lds, s)
                      : launch_commit_t<64, float>(d, a, norm, lds, s);
        case 128:
            return bf ? launch_commit_t<128, uint16_t>(d, a, norm, lds, s)
                      : launch_commit_t<128, float>(d, a, norm, lds, s);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace gdn

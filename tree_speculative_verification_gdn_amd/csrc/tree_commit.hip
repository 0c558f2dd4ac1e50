// Accepted-path commit on gfx950 (LumoTree, Sec. IV-B: the accepted path's
// recorded operands are replayed through the gated delta update in place
// into the fp32 state bank; Sec. V-A: the same device-side path drives the
// conv-history publication; Bole review, Algorithm 2 step 8: an empty path
// leaves the state as it was).
//
//   S <- S_pre;  for j < len:  u = b_j (v_j - a_j S k_j);  S <- a_j S + u k_j^T
//   hist[slot] <- last W-1 entries of (hist[slot] ++ x rows of the path)
//
// One 256-thread workgroup per (request, value head).  The fp32 state (64 KiB
// at d = 128) lives in VGPRs for the whole replay: each value row is held by
// 256/d adjacent lanes, so S k_j is a lane-local dot product plus a
// log2(256/d)-step butterfly.  The kernel reads the state once and writes it
// once: HBM-bound.  Its latency is a short chain of memory round trips, kept
// to three: (1) the request's slot, path and length; (2) the state itself and
// the path nodes' parents and rows; (3) the path's k/v rows, gates and the
// conv rows.  The path's k rows stay in their input type in LDS, with the
// optional q/k normalisation applied as a per-row scale.
// The workgroup of value head h also publishes the conv history for channel
// slice h of the request.
#include "gdn_internal.h"

namespace gdn {

namespace {
constexpr int kThreads = 256;

struct CommitLds {
    int K, V, al, be, sc, rows, total;
};

__host__ __device__ inline int align16(int x) { return (x + 15) / 16 * 16; }

template <typename T>
__host__ __device__ inline CommitLds commit_lds_layout(int Lmax, int D) {
    CommitLds L;
    int off = 0;
    const int lm = Lmax > 0 ? Lmax : 1;
    // one spare row / entry past Lmax takes the stores of lanes past the path
    L.K = off;    off += align16((lm + 1) * D * static_cast<int>(sizeof(T)));
    L.V = off;    off += align16((lm + 1) * D * 4);
    L.al = off;   off += align16((lm + 1) * 4);
    L.be = off;   off += align16((lm + 1) * 4);
    L.sc = off;   off += align16((lm + 1) * 4);
    L.rows = off; off += align16(lm * 4);
    L.total = off;
    return L;
}

// four consecutive elements as fp32 (vector load when aligned)
template <typename T, bool VEC>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<uint16_t, true>(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
template <>
__device__ __forceinline__ float4 load4<float, true>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<uint16_t, false>(const uint16_t* p) {
    return make_float4(bf16_bits_to_f32(p[0]), bf16_bits_to_f32(p[1]), bf16_bits_to_f32(p[2]),
                       bf16_bits_to_f32(p[3]));
}
template <>
__device__ __forceinline__ float4 load4<float, false>(const float* p) {
    return make_float4(p[0], p[1], p[2], p[3]);
}

// the same four elements in the input type, for staging in LDS
template <typename T>
struct Raw4;
template <>
struct Raw4<uint16_t> {
    uint2 u;
    __device__ __forceinline__ float4 f() const {
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    }
};
template <>
struct Raw4<float> {
    float4 u;
    __device__ __forceinline__ float4 f() const { return u; }
};
template <typename T, bool VEC>
__device__ __forceinline__ Raw4<T> load_raw4(const T* p);
template <>
__device__ __forceinline__ Raw4<uint16_t> load_raw4<uint16_t, true>(const uint16_t* p) {
    return Raw4<uint16_t>{*reinterpret_cast<const uint2*>(p)};
}
template <>
__device__ __forceinline__ Raw4<uint16_t> load_raw4<uint16_t, false>(const uint16_t* p) {
    return Raw4<uint16_t>{make_uint2(static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 16),
                                     static_cast<uint32_t>(p[2]) | (static_cast<uint32_t>(p[3]) << 16))};
}
template <>
__device__ __forceinline__ Raw4<float> load_raw4<float, true>(const float* p) {
    return Raw4<float>{*reinterpret_cast<const float4*>(p)};
}
template <>
__device__ __forceinline__ Raw4<float> load_raw4<float, false>(const float* p) {
    return Raw4<float>{make_float4(p[0], p[1], p[2], p[3])};
}

// CW consecutive staged k elements (CW = 4 or 8) from LDS as fp32
template <typename T, int CW>
__device__ __forceinline__ void lds_k(const T* p, float* o);
template <>
__device__ __forceinline__ void lds_k<uint16_t, 8>(const uint16_t* p, float* o) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o[2 * e] = __uint_as_float(w[e] << 16);
        o[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void lds_k<uint16_t, 4>(const uint16_t* p, float* o) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(u.x << 16);
    o[1] = __uint_as_float(u.x & 0xffff0000u);
    o[2] = __uint_as_float(u.y << 16);
    o[3] = __uint_as_float(u.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void lds_k<float, 8>(const float* p, float* o) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <>
__device__ __forceinline__ void lds_k<float, 4>(const float* p, float* o) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}
}  // namespace

size_t commit_lds_bytes(int Lmax, int D, int dtype) {
    return static_cast<size_t>(dtype == GDN_DT_BF16 ? commit_lds_layout<uint16_t>(Lmax, D).total
                                                    : commit_lds_layout<float>(Lmax, D).total);
}

template <int D, typename T, bool VEC, bool RES>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
    commit_kernel(int B, int N, int R, int W, int shared, const int32_t* __restrict__ parent,
                  const int32_t* __restrict__ node_row, const int32_t* __restrict__ status,
                  const int32_t* __restrict__ path, const int32_t* __restrict__ path_len, int Lmax,
                  const T* __restrict__ k, const T* __restrict__ v, int64_t rs_qk, int64_t rs_v,
                  const float* __restrict__ alpha, const float* __restrict__ beta,
                  float* __restrict__ pool, int P, const int32_t* __restrict__ state_idx,
                  const uint16_t* __restrict__ x, uint16_t* __restrict__ hist, int C, int hvec,
                  int Hqk, int Hv, int norm, int32_t* __restrict__ err, int64_t ls_qk, int64_t ls_v,
                  int64_t ls_gate, int64_t ls_pool, const float* __restrict__ gate_params) {
    constexpr int TPR = kThreads / D;             // lanes per value row
    constexpr int EPT = D / TPR;                  // state elements per lane
    constexpr int CW = EPT >= 8 ? 8 : EPT;        // columns per chunk
    constexpr int NC = EPT / CW;                  // chunks per lane
    constexpr int CPR = D / 4;                    // 4-element staging chunks per row
    static_assert(CPR <= 64 && (64 % CPR) == 0, "a staged row must sit inside one wave");
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const CommitLds L = commit_lds_layout<T>(Lmax, D);
    T* s_K = reinterpret_cast<T*>(lds + L.K);
    float* s_V = reinterpret_cast<float*>(lds + L.V);
    float* s_al = reinterpret_cast<float*>(lds + L.al);
    float* s_be = reinterpret_cast<float*>(lds + L.be);
    float* s_sc = reinterpret_cast<float*>(lds + L.sc);
    int32_t* s_rows = reinterpret_cast<int32_t*>(lds + L.rows);
    __shared__ int s_bad;

    // workgroup -> (layer, request, head); layer l's operands and pool sit at
    // fixed element strides from the first layer's (0 for a single layer)
    const uint32_t unit_all = xcd_local_order(blockIdx.x, gridDim.x);
    const uint32_t per_layer = static_cast<uint32_t>(B) * static_cast<uint32_t>(Hv);
    const int64_t layer = static_cast<int64_t>(unit_all / per_layer);
    const uint32_t unit = unit_all % per_layer;
    const int b = static_cast<int>(unit / Hv);
    const int h = static_cast<int>(unit % Hv);
    k += layer * ls_qk;
    v += layer * ls_v;
    alpha += layer * ls_gate;
    beta += layer * ls_gate;
    pool += layer * ls_pool;
    // raw gate inputs: the head's parameters, loaded with the first round
    // trip and used when the gates are staged
    const bool raw = gate_params != nullptr;  // uniform
    float g_alog = 0.0f, g_dtb = 0.0f;
    if (raw) {
        const float* gp = gate_params + layer * 2 * Hv;
        g_alog = gp[h];
        g_dtb = gp[Hv + h];
    }
    const int t = shared ? 0 : b;
    const int tid = threadIdx.x;
    const int r = tid / TPR;
    const int part = tid % TPR;

    // ---- round trip 1: everything that depends only on (b, h); slot, path.
    //      RES: path / path_len are the resolved rows and node counts (the
    //      path resolution validated them and reported any error)
    const int st = status[t];
    const int slot = state_idx[b];
    const int len = RES ? min(path_len[b], Lmax) : path_len[b];
    // Loads are unconditional, from indexes clamped into range; what a lane
    // does not need is dropped afterwards (a load under a per-lane condition
    // becomes a branch that waits for it before anything else issues).
    const int pnode = path[static_cast<size_t>(b) * Lmax + min(tid, Lmax - 1)];
    if constexpr (RES) {
        if (st != 0 || len <= 0 || slot < 0 || slot >= P) return;  // nothing to commit
        s_rows[min(tid, Lmax - 1)] = min(max(pnode, 0), R - 1);    // lanes past Lmax repeat the last
        __syncthreads();
    } else {
        const int prev = __shfl(pnode, tid > 0 ? tid - 1 : 0, 64);  // path[tid - 1] (wave 0)
        int dup = 0;
        for (int b2 = tid; b2 < B; b2 += kThreads) dup |= (b2 != b && state_idx[b2] == slot) ? 1 : 0;
        if (st != 0) return;  // malformed tree: reported by the descriptor build
        if (tid == 0) s_bad = 0;

        // ---- round trip 2: the path nodes' parents and rows; validation
        const bool slot_ok = slot >= 0 && slot < P;
        const bool len_ok = len >= 0 && len <= Lmax;
        const size_t ti = static_cast<size_t>(t) * N + min(max(pnode, 0), N - 1);
        const int par = parent[ti];
        const int prow = node_row[ti];
        int bad = (slot_ok ? 0 : GDN_EV_STATE) | (dup ? GDN_EV_STATE : 0);
        if (!len_ok) {
            bad |= GDN_EV_PATH;
        } else if (tid < len) {  // len <= Lmax <= 64: all in wave 0
            if (pnode < 0 || pnode >= N || par != (tid == 0 ? -1 : prev)) bad |= GDN_EV_PATH;
            s_rows[tid] = prow;
        }
        __syncthreads();  // s_bad initialised
        if (bad) atomicOr(&s_bad, bad);
        __syncthreads();
        bad = s_bad;
        if (bad) {
            if (h == 0 && tid == 0) atomicOr(err, bad);
            return;
        }
        if (len == 0) return;  // nothing accepted: state and history stay as they are
    }

    // ---- round trip 3: the path's gates and k/v rows, the conv rows, then the
    //      state.  A wave's loads retire in issue order, so everything staged
    //      in LDS goes out before the 64 KiB state and is stored while the
    //      state is still arriving; only the replay waits for the state.
    const int g = static_cast<int>((static_cast<int64_t>(h) * Hqk) / Hv);
    const size_t rowb = static_cast<size_t>(b) * R;
    const int my_j = min(tid, len - 1);
    const size_t gi = (rowb + s_rows[my_j]) * Hv + h;
    const float my_al = alpha[gi], my_be = beta[gi];
    const int chunks = len * CPR;
    Raw4<T> kc[2];
    float4 vc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int it = u * kThreads + tid;
        const int j = min(it / CPR, len - 1);
        const int ch = it % CPR;
        const size_t rb = rowb + s_rows[j];
        kc[u] = load_raw4<T, VEC>(k + rb * rs_qk + static_cast<size_t>(g) * D + 4 * ch);
        vc[u] = load4<T, VEC>(v + rb * rs_v + static_cast<size_t>(h) * D + 4 * ch);
    }
    // conv history of this request, channel slice h: the last W-1 entries of
    // (old history ++ x rows of the path).  First chunk per lane loaded here.
    const int H = W - 1;
    const bool pub = x != nullptr && hist != nullptr && H > 0;
    uint16_t* hs = hist + static_cast<size_t>(slot) * (H > 0 ? H : 1) * C;
    const int cunit = hvec ? 4 : 1;  // channels per access
    const int nunits = C / cunit;
    const int per = (nunits + Hv - 1) / Hv;
    const int u_begin = h * per;
    const int u_end = min(nunits, u_begin + per);
    uint2 hv4[GDN_MAX_CONV_W - 1];
    uint16_t hv1[GDN_MAX_CONV_W - 1];
    if (pub && u_begin < u_end) {
        const int cu = min(u_begin + tid, u_end - 1);
#pragma unroll
        for (int m = 0; m < GDN_MAX_CONV_W - 1; ++m) {
            if (m < H) {
                const int pos = len + m;  // position in (old ++ path rows), uniform
                const uint16_t* src = (pos < H) ? hs + static_cast<size_t>(pos) * C
                                                : x + (rowb + s_rows[max(pos - H, 0)]) * C;
                if (hvec)
                    hv4[m] = *reinterpret_cast<const uint2*>(src + 4 * cu);
                else
                    hv1[m] = src[cu];
            }
        }
    }
    asm volatile("" ::: "memory");  // keep the state loads behind the loads above
    float* Sb = pool + (static_cast<size_t>(slot) * Hv + h) * (D * D) + static_cast<size_t>(r) * D;
    float4 sv[NC][CW / 4];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int q4 = 0; q4 < CW / 4; ++q4)
            sv[c][q4] = *reinterpret_cast<const float4*>(Sb + CW * (part + TPR * c) + 4 * q4);

    // stage gates, k (input type, per-row scale) and v in LDS; every lane
    // stores (past the end into a spare entry) so that no load above is sunk
    // into a branch behind the state loads
    if (raw) {  // uniform
        const RawGate rg = raw_gate_params(g_alog, g_dtb);
        s_al[tid < len ? tid : Lmax] = raw_gate_alpha(my_al, rg);
        s_be[tid < len ? tid : Lmax] = raw_gate_beta(my_be);
    } else {
        s_al[tid < len ? tid : Lmax] = my_al;
        s_be[tid < len ? tid : Lmax] = my_be;
    }
    for (int it0 = 0; it0 < chunks; it0 += 2 * kThreads) {
        if (it0 > 0) {  // paths longer than 2 * kThreads / CPR rows (rare)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int it = it0 + u * kThreads + tid;
                const int j = min(it / CPR, len - 1);
                const int ch = it % CPR;
                const size_t rb = rowb + s_rows[j];
                kc[u] = load_raw4<T, VEC>(k + rb * rs_qk + static_cast<size_t>(g) * D + 4 * ch);
                vc[u] = load4<T, VEC>(v + rb * rs_v + static_cast<size_t>(h) * D + 4 * ch);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int it = it0 + u * kThreads + tid;
            const int j = it / CPR;
            const int ch = it % CPR;
            // the CPR chunks of a row sit in CPR consecutive lanes of one wave;
            // whole groups of CPR lanes are either in range or not
            if (it0 + u * kThreads < chunks) {
                const float4 kf = (it < chunks) ? kc[u].f() : make_float4(0.f, 0.f, 0.f, 0.f);
                float ss = fmaf(kf.x, kf.x, fmaf(kf.y, kf.y, fmaf(kf.z, kf.z, kf.w * kf.w)));
#pragma unroll
                for (int off = CPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
                const int js = it < chunks ? j : Lmax;  // spare row past the end
                *reinterpret_cast<Raw4<T>*>(s_K + js * D + 4 * ch) = kc[u];
                *reinterpret_cast<float4*>(s_V + js * D + 4 * ch) = vc[u];
                if (ch == 0) s_sc[js] = norm ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
            }
        }
    }
    // publish the history: first chunk from the registers, the rest (slices
    // wider than the workgroup) loaded and stored here
    if (pub) {
        for (int cu = u_begin + tid; cu < u_end; cu += kThreads) {
            if (cu >= u_begin + kThreads) {
#pragma unroll
                for (int m = 0; m < GDN_MAX_CONV_W - 1; ++m) {
                    if (m < H) {
                        const int pos = len + m;
                        const uint16_t* src = (pos < H) ? hs + static_cast<size_t>(pos) * C
                                                        : x + (rowb + s_rows[max(pos - H, 0)]) * C;
                        if (hvec)
                            hv4[m] = *reinterpret_cast<const uint2*>(src + 4 * cu);
                        else
                            hv1[m] = src[cu];
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < GDN_MAX_CONV_W - 1; ++m) {
                if (m < H) {
                    if (hvec)
                        *reinterpret_cast<uint2*>(hs + static_cast<size_t>(m) * C + 4 * cu) = hv4[m];
                    else
                        hs[static_cast<size_t>(m) * C + cu] = hv1[m];
                }
            }
        }
    }
    __syncthreads();

    // ---- replay: with k^ = sc * k,  S k^ = sc (S k)  and  u k^T = (u sc) k^T
    for (int j = 0; j < len; ++j) {
        const T* kj = s_K + j * D;
        float y = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float kv[CW];
            lds_k<T, CW>(kj + CW * (part + TPR * c), kv);
#pragma unroll
            for (int q4 = 0; q4 < CW / 4; ++q4) {
                y = fmaf(sv[c][q4].x, kv[4 * q4 + 0], y);
                y = fmaf(sv[c][q4].y, kv[4 * q4 + 1], y);
                y = fmaf(sv[c][q4].z, kv[4 * q4 + 2], y);
                y = fmaf(sv[c][q4].w, kv[4 * q4 + 3], y);
            }
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) y += __shfl_xor(y, off, 64);
        const float a = s_al[j];
        const float sc = s_sc[j];
        const float us = s_be[j] * (s_V[j * D + r] - a * (y * sc)) * sc;
        // read k_j from LDS again rather than keep the unpacked copy live
        // across the reduction (it would double the registers the state needs)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            float kv[CW];
            lds_k<T, CW>(kj + CW * (part + TPR * c), kv);
#pragma unroll
            for (int q4 = 0; q4 < CW / 4; ++q4) {
                sv[c][q4].x = fmaf(a, sv[c][q4].x, us * kv[4 * q4 + 0]);
                sv[c][q4].y = fmaf(a, sv[c][q4].y, us * kv[4 * q4 + 1]);
                sv[c][q4].z = fmaf(a, sv[c][q4].z, us * kv[4 * q4 + 2]);
                sv[c][q4].w = fmaf(a, sv[c][q4].w, us * kv[4 * q4 + 3]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int q4 = 0; q4 < CW / 4; ++q4)
            *reinterpret_cast<float4*>(Sb + CW * (part + TPR * c) + 4 * q4) = sv[c][q4];
}

namespace {
template <int D, typename T, bool VEC>
hipError_t launch_commit_t(const gdn_tree_desc& d, const CommitArgs& a, int norm, size_t lds,
                           hipStream_t s) {
    // 8-byte history accesses when C is a multiple of 4 and x, hist are 8-byte aligned
    const int hvec = (a.x != nullptr && (a.C & 3) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.x) & 7) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.hist) & 7) == 0) ? 1 : 0;
    auto kfn = a.resolved ? commit_kernel<D, T, VEC, true> : commit_kernel<D, T, VEC, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(d.B) * static_cast<unsigned>(a.Hv) * static_cast<unsigned>(a.layers));
    hipLaunchKernelGGL(kfn, grid, dim3(kThreads), lds, s, d.B, d.N, d.R, d.W, d.shared, d.parent,
                       d.node_row, d.status, a.path, a.path_len, a.Lmax,
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.rs_qk, a.rs_v,
                       a.alpha, a.beta, a.pool, a.P, a.state_idx, a.x, a.hist, a.C, hvec, a.Hqk,
                       a.Hv, norm, a.err, a.ls_qk, a.ls_v, a.ls_gate, a.ls_pool,
                       (a.flags & GDN_F_RAW_GATES) ? a.gate_params : nullptr);
    return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_commit_d(const gdn_tree_desc& d, const CommitArgs& a, int norm, size_t lds,
                           hipStream_t s) {
    // vector loads need every 4-element group of k and v (in every layer)
    // aligned to 4 elements
    const bool vec = (a.rs_qk % 4 == 0) && (a.rs_v % 4 == 0) && (a.ls_qk % 4 == 0) &&
                     (a.ls_v % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.k) % (4 * sizeof(T)) == 0) &&
                     (reinterpret_cast<uintptr_t>(a.v) % (4 * sizeof(T)) == 0);
    return vec ? launch_commit_t<D, T, true>(d, a, norm, lds, s)
               : launch_commit_t<D, T, false>(d, a, norm, lds, s);
}
}  // namespace

hipError_t launch_commit(const gdn_tree_desc& d, const CommitArgs& a, hipStream_t s) {
    const int norm = (a.flags & GDN_F_NORM_QK) ? 1 : 0;
    const size_t lds = commit_lds_bytes(a.Lmax, a.D, a.dtype);
    if (lds > 160 * 1024) return hipErrorNotSupported;
    const bool bf = a.dtype == GDN_DT_BF16;
    switch (a.D) {
        case 32:
            return bf ? launch_commit_d<32, uint16_t>(d, a, norm, lds, s)
                      : launch_commit_d<32, float>(d, a, norm, lds, s);
        case 64:
            return bf ? launch_commit_d<64, uint16_t>(d, a, norm, lds, s)
                      : launch_commit_d<64, float>(d, a, norm, lds, s);
        case 128:
            return bf ? launch_commit_d<128, uint16_t>(d, a, norm, lds, s)
                      : launch_commit_d<128, float>(d, a, norm, lds, s);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace gdn

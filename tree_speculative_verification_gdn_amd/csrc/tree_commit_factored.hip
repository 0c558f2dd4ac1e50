// Commit of the accepted path from stored delta corrections (the factorised
// publish) on gfx950.
//
// What (Bole review, Sec. 5.2: Algorithm 2 keeps U from its verify and
// publishes the accepted frontier's state from it, Eq. (10); TreeWY, Sec. 3:
// the factored publish from pseudo-values):
//   S_new = P_a S_pre + sum_{j on the path} (P_a / P_j) u_j k^_j^T
// with a the path's frontier and P_x the product of the decays on the
// root-to-x path, so P_a / P_j is the product of the decays of the path nodes
// after j, and u_j = b_j (v_j - a_j S_parent(j) k^_j) the delta correction
// the verify wrote for node j.  No term depends on another: instead of
// replaying the path node by node, the kernel scales the state by P_a and adds
// one rank-8 update per 8 path nodes on the matrix cores (the k rows as the A
// operand, the coefficients (P_a / P_j) sc_j u_j[r] of this lane's value row r
// as the B operand, split into bf16 hi + lo), accumulated in the state's own
// register layout.
//
// One 256-thread workgroup per (request, value head), as the replay commit:
// round trip 1 the slot, length, path and the duplicate-slot scan, round trip
// 2 the path nodes' parents and rows (validation), round trip 3 the path's k
// and u rows and decays, then the state.
//
// The same kernel also serves the verify's debug dump (DUMP): one workgroup
// per (request, value head, node i) rebuilds S_i from node i's own root path
// (its strict ancestors from the descriptor, then i) and writes it to the dump
// instead of the pool, which it only reads.  S_i is the state the verify
// reads o_i from (o_i = S_i q^_i): the pages' verifier never materialises
// it, so the dump is what a commit of that path is compared against.
#include "mfma_common.h"

namespace gdn {

namespace {

constexpr int kFThreads = 256;

struct FacLds {
    int K, U, al, sc, rows, total;
};

__host__ __device__ inline FacLds fac_lds_layout(int Lmax) {
    const int lp = align_up(Lmax, kMfmaPath);  // whole segments; rows past the path are zero
    FacLds L{};
    int off = 0;
    L.K = off;    off += align_up(lp * kKQStride, 16);  // k rows, bf16, matrix-core operand rows
    L.U = off;    off += align_up(lp * kD * 4, 16);     // u rows, fp32
    L.al = off;   off += align_up((lp + 1) * 4, 16);    // decays (one spare entry)
    L.sc = off;   off += align_up((lp + 1) * 4, 16);    // (P_a / P_j) sc_j, zero past the path
    L.rows = off; off += align_up((lp + 1) * 4, 16);
    L.total = off;
    return L;
}

}  // namespace

size_t commit_factored_lds_bytes(int Lmax) { return static_cast<size_t>(fac_lds_layout(Lmax).total); }

template <bool RAW, bool DUMP>
__global__ void __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
    commit_factored_kernel(int B, int N, int R, int shared, const int32_t* __restrict__ parent,
                           const int32_t* __restrict__ node_row, const int32_t* __restrict__ status,
                           const uint64_t* __restrict__ anc, float* __restrict__ dump,
                           const int32_t* __restrict__ path, const int32_t* __restrict__ path_len, int Lmax,
                           const uint16_t* __restrict__ k, int64_t rs_qk, const float* __restrict__ u,
                           const float* __restrict__ alpha, float* __restrict__ pool, int P,
                           const int32_t* __restrict__ state_idx, int Hqk, int Hv, int norm,
                           int32_t* __restrict__ err, const float* __restrict__ gate_params) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const FacLds L = fac_lds_layout(Lmax);
    char* s_K = lds + L.K;
    float* s_U = reinterpret_cast<float*>(lds + L.U);
    float* s_al = reinterpret_cast<float*>(lds + L.al);
    float* s_sc = reinterpret_cast<float*>(lds + L.sc);
    int32_t* s_rows = reinterpret_cast<int32_t*>(lds + L.rows);
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5;
    const int l32 = lane & 31;
    const int r_own = wave * 32 + l32;
    const uint32_t unit = xcd_local_order(blockIdx.x, gridDim.x);
    const uint32_t bh = DUMP ? unit / static_cast<uint32_t>(N) : unit;
    const int inode = DUMP ? static_cast<int>(unit % static_cast<uint32_t>(N)) : 0;
    const int b = static_cast<int>(bh / Hv);
    const int h = static_cast<int>(bh % Hv);
    const int t = shared ? 0 : b;
    const int g = static_cast<int>((static_cast<int64_t>(h) * Hqk) / Hv);
    float g_alog = 0.0f, g_dtb = 0.0f;
    if constexpr (RAW) {
        g_alog = gate_params[h];
        g_dtb = gate_params[Hv + h];
    }
    int len;
    int slot;
    if constexpr (DUMP) {
        // node i's root path: its strict ancestors in index order (a parent
        // precedes its children), then i; lane j < N places node j's row
        const int st = status[t];
        slot = state_idx[b];
        const uint64_t path_bits = anc[static_cast<size_t>(t) * N + inode] | (1ull << inode);
        const int prow = node_row[static_cast<size_t>(t) * N + min(tid, N - 1)];
        if (st != 0) return;  // malformed tree: reported by its descriptor build
        if (slot < 0 || slot >= P) {  // the verify reports the same bit
            if (h == 0 && inode == 0 && tid == 0) atomicOr(err, GDN_EV_STATE);
            return;
        }
        len = __popcll(path_bits);
        if (tid < N && ((path_bits >> tid) & 1ull))
            s_rows[__popcll(path_bits & ((1ull << tid) - 1ull))] = min(max(prow, 0), R - 1);
        __syncthreads();
    } else {
        // round trip 1: status, slot, length, the path, the duplicate-slot
        // scan; every load unconditional from an index clamped into range
        const int st = status[t];
        slot = state_idx[b];
        len = path_len[b];
        const int pnode = path[static_cast<size_t>(b) * Lmax + min(tid, Lmax - 1)];
        const int prev = __shfl(pnode, tid > 0 ? tid - 1 : 0, 64);  // path[tid - 1] (wave 0: len <= 64)
        int dup = 0;
        for (int b2 = tid; b2 < B; b2 += kFThreads) dup |= (b2 != b && state_idx[b2] == slot) ? 1 : 0;
        if (st != 0) return;  // malformed tree: reported by its descriptor build
        if (tid == 0) s_bad = 0;

        // round trip 2: the path nodes' parents and rows; validation
        const size_t ti = static_cast<size_t>(t) * N + min(max(pnode, 0), N - 1);
        const int par = parent[ti];
        const int prow = node_row[ti];
        int bad = ((slot >= 0 && slot < P) ? 0 : GDN_EV_STATE) | (dup ? GDN_EV_STATE : 0);
        if (len < 0 || len > Lmax) {
            bad |= GDN_EV_PATH;
        } else if (tid < len) {
            if (pnode < 0 || pnode >= N || par != (tid == 0 ? -1 : prev)) bad |= GDN_EV_PATH;
        }
        s_rows[min(tid, Lmax)] = min(max(prow, 0), R - 1);  // every lane writes (spare entry Lmax)
        __syncthreads();  // s_bad initialised
        if (bad) atomicOr(&s_bad, bad);
        __syncthreads();
        bad = s_bad;
        if (bad) {
            if (h == 0 && tid == 0) atomicOr(err, bad);
            return;
        }
        if (len == 0) return;  // nothing accepted: the state stays as it is
    }

    // round trip 3: the path's k rows (qk head g), u rows (value head h) and
    // decays, zero past the path, then the state
    const size_t rowb = static_cast<size_t>(b) * R;
    const int lp = (len + kMfmaPath - 1) / kMfmaPath * kMfmaPath;
    const int c = tid & 31;  // 32 chunks per row: 8 bytes of k, 16 bytes of u
    for (int it0 = 0; it0 < lp * 32; it0 += kFThreads) {  // uniform: lp * 32 is a multiple of 256
        const int j = (it0 + tid) >> 5;
        const size_t rb = rowb + s_rows[min(j, len - 1)];
        uint2 kc = *reinterpret_cast<const uint2*>(k + rb * rs_qk + static_cast<size_t>(g) * kD + 4 * c);
        float4 uc = *reinterpret_cast<const float4*>(u + (rb * Hv + h) * kD + 4 * c);
        if (j >= len) {
            kc = make_uint2(0u, 0u);
            uc = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float ss = sumsq_bf16x4(kc);  // a row's 32 chunks sit in 32 consecutive lanes
        ss = sum_half_wave(ss);
        *reinterpret_cast<uint2*>(s_K + j * kKQStride + 8 * c) = kc;
        *reinterpret_cast<float4*>(s_U + j * kD + 4 * c) = uc;
        if (c == 0) s_sc[j] = j < len ? (norm ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f) : 0.0f;
    }
    {
        const float a_raw = alpha[(rowb + s_rows[min(tid, len - 1)]) * Hv + h];
        float a = a_raw;
        if constexpr (RAW) a = raw_gate_alpha(a_raw, raw_gate_params(g_alog, g_dtb));
        s_al[min(tid, lp)] = a;  // every lane writes (spare entry lp)
    }
    float* Sw = pool + (static_cast<size_t>(slot) * Hv + h) * (kD * kD) + static_cast<size_t>(wave) * 32 * kD;
    float* Sd = DUMP ? dump + ((static_cast<size_t>(b) * N + inode) * Hv + h) * (kD * kD) +
                           static_cast<size_t>(wave) * 32 * kD
                     : Sw;
    float4 sreg[16];
    {
        asm volatile("" ::: "memory");  // keep the state loads behind the loads above
        const float* Sl = Sw + state_load_lane_off(l32, hf);
#pragma unroll
        for (int s = 0; s < 16; ++s) sreg[s] = *reinterpret_cast<const float4*>(Sl + state_load_off(s));
    }
    __syncthreads();
    // coefficient of path node j: (P_a / P_j) = product of the decays after j, times sc_j
    if (tid < len) {
        float cf = 1.0f;
        for (int m = tid + 1; m < len; ++m) cf *= s_al[m];
        s_sc[tid] *= cf;
    }
    float Pa = 1.0f;  // P_a: the product of every decay on the path
    for (int m = 0; m < len; ++m) Pa *= s_al[m];
    __syncthreads();

    state_fix_loaded(sreg, l32);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        sreg[q].x *= Pa;
        sreg[q].y *= Pa;
        sreg[q].z *= Pa;
        sreg[q].w *= Pa;
    }
    for (int j0 = 0; j0 < len; j0 += kMfmaPath) {  // uniform
        // B operand: slot e of lane half 0 is path node j0 + e (lane half 1: zero)
        bf16x8_t uhi, ulo;
        {
            float uu[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) uu[e] = hf ? 0.0f : s_sc[j0 + e] * s_U[(j0 + e) * kD + r_own];
            split_hi_lo(make_float4(uu[0], uu[1], uu[2], uu[3]), make_float4(uu[4], uu[5], uu[6], uu[7]), uhi,
                        ulo);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            // A operand: k_m[32cb + l32] for path node j0 + 8hf + e (rows past
            // the segment's 8 are the other lane half's zeros)
            uint32_t kw[4];
            const uint16_t* col = reinterpret_cast<const uint16_t*>(s_K) + (32 * cb + l32);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int m0 = 8 * hf + 2 * e2;
                const uint32_t k0 = col[(j0 + min(m0, kMfmaPath - 1)) * (kKQStride / 2)];
                const uint32_t k1 = col[(j0 + min(m0 + 1, kMfmaPath - 1)) * (kKQStride / 2)];
                kw[e2] = (m0 < kMfmaPath ? k0 : 0u) | ((m0 + 1 < kMfmaPath ? k1 : 0u) << 16);
            }
            const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, make_uint4(kw[0], kw[1], kw[2], kw[3]));
            f32x16_t sacc;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                sacc[4 * q4 + 0] = sreg[4 * cb + q4].x;
                sacc[4 * q4 + 1] = sreg[4 * cb + q4].y;
                sacc[4 * q4 + 2] = sreg[4 * cb + q4].z;
                sacc[4 * q4 + 3] = sreg[4 * cb + q4].w;
            }
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, uhi, sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, ulo, sacc, 0, 0, 0);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                sreg[4 * cb + q4] = make_float4(sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]);
        }
    }
    state_store_lines(Sd, sreg, l32, hf);
}

namespace {

template <bool DUMP>
hipError_t launch_factored(const gdn_tree_desc& d, const FactoredCommitArgs& a, float* dump, hipStream_t s) {
    const int Lmax = DUMP ? d.N : a.Lmax;  // a node's root path has at most N nodes
    const size_t lds = commit_factored_lds_bytes(Lmax);
    if (lds > 160 * 1024) return hipErrorNotSupported;
    const int norm = (a.flags & GDN_F_NORM_QK) ? 1 : 0;
    const bool raw = (a.flags & GDN_F_RAW_GATES) != 0;
    auto kfn = raw ? commit_factored_kernel<true, DUMP> : commit_factored_kernel<false, DUMP>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kfn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(d.B) * static_cast<unsigned>(a.Hv) *
                    static_cast<unsigned>(DUMP ? d.N : 1));
    hipLaunchKernelGGL(kfn, grid, dim3(kFThreads), lds, s, d.B, d.N, d.R, d.shared, d.parent, d.node_row,
                       d.status, d.anc, dump, a.path, a.path_len, Lmax, static_cast<const uint16_t*>(a.k),
                       a.rs_qk, a.u, a.alpha, a.pool, a.P, a.state_idx, a.Hqk, a.Hv, norm, a.err,
                       raw ? a.gate_params : nullptr);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_commit_factored(const gdn_tree_desc& d, const FactoredCommitArgs& a, hipStream_t s) {
    return launch_factored<false>(d, a, nullptr, s);
}

hipError_t launch_dump_states(const gdn_tree_desc& d, const FactoredCommitArgs& a, float* dump, hipStream_t s) {
    return launch_factored<true>(d, a, dump, s);
}

}  // namespace gdn

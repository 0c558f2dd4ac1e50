// Shared tree descriptor builder (LumoTree, Sec. III-C: one logical topology
// -- parents, depth, logical->physical rows -- drives every later stage; Sec.
// V-C: static gather indices derived from the topology).
//
// One wave per tree, one lane per node (N <= 64).  Integer work only; the
// results are unique functions of parent[] and node_row[].
#include "gdn_internal.h"

namespace gdn {

// tree t of the descriptor, by one 64-lane workgroup
__device__ __forceinline__ void build_tree(int t, int N, int R, int W, const int32_t* __restrict__ parent,
                                           const int32_t* __restrict__ node_row,
                                           int32_t* __restrict__ depth, uint64_t* __restrict__ anc,
                                           int32_t* __restrict__ conv_src,
                                           int32_t* __restrict__ status, int32_t* __restrict__ err) {
    __shared__ int32_t s_par[kMaxNodes];
    __shared__ int32_t s_row[kMaxNodes];
    const int i = threadIdx.x;
    const size_t base = static_cast<size_t>(t) * N;
    if (i < N) {
        s_par[i] = parent[base + i];
        s_row[i] = node_row[base + i];
    }
    __syncthreads();
    int st = 0;
    if (i < N) {
        const int p = s_par[i];
        if (p < -1 || p >= i) st |= GDN_EV_PARENT;
        const int r = s_row[i];
        if (r < 0 || r >= R) st |= GDN_EV_ROW;
        for (int j = 0; j < i; ++j)
            if (s_row[j] == r) st |= GDN_EV_ROW;
    }
    // OR over the wave (one wave per block)
    for (int off = 32; off > 0; off >>= 1) st |= __shfl_xor(st, off, 64);
    if (i == 0) {
        status[t] = st;
        if (st) atomicOr(err, st);
    }
    if (i >= N) return;
    const int H = W - 1;
    if (st) {
        depth[base + i] = 0;
        anc[base + i] = 0ull;
        for (int m = 0; m < H; ++m) conv_src[(base + i) * H + m] = 0;
        return;
    }
    // Valid tree: parent indices strictly decrease along a chain, so the walk
    // ends within i steps.
    int dep = 1;
    uint64_t a = 0ull;
    for (int p = s_par[i]; p >= 0; p = s_par[p]) {
        a |= 1ull << p;
        ++dep;
    }
    depth[base + i] = dep;
    anc[base + i] = a;
    // Tap sources, most recent first: parent, grandparent, ...; once past the
    // root-level node, history entries H-1, H-2, ...  Stored oldest first.
    int cur = s_par[i];
    int slot = H - 1;
    for (int m = 0; m < H; ++m) {
        int32_t v;
        if (cur >= 0) {
            v = s_row[cur];
            cur = s_par[cur];
        } else {
            v = -(slot + 1);
            --slot;
        }
        conv_src[(base + i) * H + (H - 1 - m)] = v;
    }
}

__global__ void __launch_bounds__(64) desc_build_kernel(int N, int R, int W,
                                                        const int32_t* __restrict__ parent,
                                                        const int32_t* __restrict__ node_row,
                                                        int32_t* __restrict__ depth,
                                                        uint64_t* __restrict__ anc,
                                                        int32_t* __restrict__ conv_src,
                                                        int32_t* __restrict__ status,
                                                        int32_t* __restrict__ err) {
    build_tree(blockIdx.x, N, R, W, parent, node_row, depth, anc, conv_src, status, err);
}

hipError_t launch_desc_build(const gdn_tree_desc& d, int32_t* err, hipStream_t s) {
    const int T = d.shared ? 1 : d.B;
    hipLaunchKernelGGL(desc_build_kernel, dim3(T), dim3(64), 0, s, d.N, d.R, d.W, d.parent,
                       d.node_row, d.depth, d.anc, d.conv_src, d.status, err);
    return hipGetLastError();
}

// Previous step's accepted path, once per step for every layer (LumoTree,
// Sec. V-A: one device-produced path drives every publication).  One wave
// per request, lane j holds path entry j (Lmax <= 64).  The path must be a
// parent chain from a node whose parent is -1 (the same checks the commit
// makes); its rows are the previous tree's node_row of each entry.
struct ResolveArgs {
    int B, Np, shared_p, Lmax, P;
    const int32_t* parent_p;
    const int32_t* node_row_p;
    const int32_t* status_p;
    const int32_t* path;
    const int32_t* path_len;
    const int32_t* state_idx;
    int32_t* path_rows;
    int32_t* path_n;
};

__device__ __forceinline__ void resolve_path(int b, const ResolveArgs& a, int32_t* __restrict__ err) {
    const int B = a.B, Np = a.Np, shared_p = a.shared_p, Lmax = a.Lmax, P = a.P;
    const int32_t* __restrict__ parent_p = a.parent_p;
    const int32_t* __restrict__ node_row_p = a.node_row_p;
    const int32_t* __restrict__ status_p = a.status_p;
    const int32_t* __restrict__ path = a.path;
    const int32_t* __restrict__ path_len = a.path_len;
    const int32_t* __restrict__ state_idx = a.state_idx;
    int32_t* __restrict__ path_rows = a.path_rows;
    int32_t* __restrict__ path_n = a.path_n;
    const int j = threadIdx.x;
    const int tp = shared_p ? 0 : b;
    const int st_p = status_p[tp];
    const int len = path_len[b];
    const int slot = state_idx[b];
    int dup = 0;
    for (int b2 = j; b2 < B; b2 += 64) dup |= (b2 != b && state_idx[b2] == slot) ? 1 : 0;
    const int node = path[static_cast<size_t>(b) * Lmax + min(j, Lmax - 1)];
    const int prev_node = __shfl(node, j > 0 ? j - 1 : 0, 64);
    const size_t ti = static_cast<size_t>(tp) * Np + min(max(node, 0), Np - 1);
    const int par = parent_p[ti];
    const int row = node_row_p[ti];
    const bool len_ok = len >= 0 && len <= Lmax;
    const bool bad_j = len_ok && j < len && (node < 0 || node >= Np || par != (j == 0 ? -1 : prev_node));
    const bool bad = __ballot(bad_j) != 0ull;
    const bool any_dup = __ballot(dup != 0) != 0ull;
    const bool slot_bad = slot < 0 || slot >= P || any_dup;
    const bool path_bad = !len_ok || bad;
    if (j == 0) {
        int n, ev = 0;
        if (slot_bad) {
            n = -1;
            ev |= GDN_EV_STATE;
        } else {
            n = (st_p != 0 || path_bad) ? 0 : len;
        }
        if (st_p == 0 && path_bad) ev |= GDN_EV_PATH;  // a malformed tree is its own build's error
        path_n[b] = n;
        if (ev) atomicOr(err, ev);
    }
    if (st_p == 0 && !path_bad && j < len) path_rows[static_cast<size_t>(b) * Lmax + j] = row;
}

__global__ void __launch_bounds__(64) path_resolve_kernel(const ResolveArgs a, int32_t* __restrict__ err) {
    resolve_path(blockIdx.x, a, err);
}

// One launch for a step's shared work: the new tree's descriptor (workgroups
// t < T) and the previous path's rows (workgroups T + b), side by side: the
// two are independent, so neither waits for the other's memory round trips.
__global__ void __launch_bounds__(64) step_prepare_kernel(int T, int N, int R, int W,
                                                          const int32_t* __restrict__ parent,
                                                          const int32_t* __restrict__ node_row,
                                                          int32_t* __restrict__ depth,
                                                          uint64_t* __restrict__ anc,
                                                          int32_t* __restrict__ conv_src,
                                                          int32_t* __restrict__ status,
                                                          const ResolveArgs a, int32_t* __restrict__ err) {
    if (static_cast<int>(blockIdx.x) < T)  // uniform per workgroup
        build_tree(blockIdx.x, N, R, W, parent, node_row, depth, anc, conv_src, status, err);
    else
        resolve_path(static_cast<int>(blockIdx.x) - T, a, err);
}

static ResolveArgs resolve_args(const gdn_tree_desc& prev, int B, const int32_t* path,
                                const int32_t* path_len, int Lmax, const int32_t* state_idx, int P,
                                int32_t* path_rows, int32_t* path_n) {
    ResolveArgs a{};
    a.B = B;
    a.Np = prev.N;
    a.shared_p = prev.shared;
    a.Lmax = Lmax;
    a.P = P;
    a.parent_p = prev.parent;
    a.node_row_p = prev.node_row;
    a.status_p = prev.status;
    a.path = path;
    a.path_len = path_len;
    a.state_idx = state_idx;
    a.path_rows = path_rows;
    a.path_n = path_n;
    return a;
}

hipError_t launch_path_resolve(const gdn_tree_desc& prev, int B, const int32_t* path,
                               const int32_t* path_len, int Lmax, const int32_t* state_idx, int P,
                               int32_t* path_rows, int32_t* path_n, int32_t* err, hipStream_t s) {
    const ResolveArgs a = resolve_args(prev, B, path, path_len, Lmax, state_idx, P, path_rows, path_n);
    hipLaunchKernelGGL(path_resolve_kernel, dim3(B), dim3(64), 0, s, a, err);
    return hipGetLastError();
}

hipError_t launch_step_prepare(const gdn_tree_desc& d, const gdn_tree_desc& prev, const int32_t* path,
                               const int32_t* path_len, int Lmax, const int32_t* state_idx, int P,
                               int32_t* path_rows, int32_t* path_n, int32_t* err, hipStream_t s) {
    const int T = d.shared ? 1 : d.B;
    const ResolveArgs a = resolve_args(prev, d.B, path, path_len, Lmax, state_idx, P, path_rows, path_n);
    hipLaunchKernelGGL(step_prepare_kernel, dim3(T + d.B), dim3(64), 0, s, T, d.N, d.R, d.W,
                       d.parent, d.node_row, d.depth, d.anc, d.conv_src, d.status, a, err);
    return hipGetLastError();
}

}  // namespace gdn

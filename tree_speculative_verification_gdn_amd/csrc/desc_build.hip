// Shared tree descriptor builder (LumoTree, Sec. III-C: one logical topology
// -- parents, depth, logical->physical rows -- drives every later stage; Sec.
// V-C: static gather indices derived from the topology).
//
// One wave per tree, one lane per node (N <= 64).  Integer work only; the
// results are unique functions of parent[] and node_row[].
#include "gdn_internal.h"

namespace gdn {

__global__ void __launch_bounds__(64) desc_build_kernel(int N, int R, int W,
                                                        const int32_t* __restrict__ parent,
                                                        const int32_t* __restrict__ node_row,
                                                        int32_t* __restrict__ depth,
                                                        uint64_t* __restrict__ anc,
                                                        int32_t* __restrict__ conv_src,
                                                        int32_t* __restrict__ status,
                                                        int32_t* __restrict__ err) {
    __shared__ int32_t s_par[kMaxNodes];
    __shared__ int32_t s_row[kMaxNodes];
    const int t = blockIdx.x;
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

hipError_t launch_desc_build(const gdn_tree_desc& d, int32_t* err, hipStream_t s) {
    const int T = d.shared ? 1 : d.B;
    hipLaunchKernelGGL(desc_build_kernel, dim3(T), dim3(64), 0, s, d.N, d.R, d.W, d.parent,
                       d.node_row, d.depth, d.anc, d.conv_src, d.status, err);
    return hipGetLastError();
}

}  // namespace gdn

// Tree verify for the gated delta rule on gfx950.
//
// What: for every node i of every request b and value head h,
//   S~ = a_i S_pi(i);  u_i = b_i (v_i - S~ k_i);  S_i = S~ + u_i k_i^T;  o_i = S_i q_i
// with S_pi(i) = S_pre for parent -1 (TreeWY, Sec. 1; Bole review, Sec. 1 Eq. (1)
// and Sec. 3.1).
//
// How (no node state is ever formed).  Expanding S_p x one level,
//   S_p x = a_p S_pi(p) x + u_p (k_p . x),
// so S_pi(i) x for x in {k_i, q_i} is the committed-state product S_pre x
// carried down the root-to-parent path with one multiply-add per ancestor
// (the unrolled form is Lemma 1 / Eq. (3)-(4) of the Bole review).  Per
// (request, head) the kernel therefore needs
//   (1) CT = [K; Q] S_pre^T      one dense 2N x d_k x d_v contraction,
//   (2) the Gram entries k_j . k_i and k_j . q_i of ancestor pairs,
//   (3) a per-value-row scan over the nodes in index order (parent[i] < i):
//         y   = CT[k_i][r] + sum over ancestors j, root first:  y = a_j y + u_j[r] (k_j . k_i)
//         u_i = b_i (v_i[r] - a_i y)
//       and, in parallel over nodes once every u is known,
//         z   = CT[q_i][r] + same walk with (k_j . q_i)
//         o_i = a_i z + u_i[r] (k_i . q_i).
// Value rows r are independent, so the scan needs no cross-lane traffic.
// S_pre (64 KiB fp32 per head at d = 128) is read exactly once and dominates
// the bytes: the kernel is HBM-bound once (1) runs on the matrix cores.
//
// Two kernels:
//   verify_mfma_kernel<MB>  bf16 q/k/v, d = 128.  (1) and the Gram block run on
//       v_mfma_f32_32x32x16_bf16: K/Q are exact in bf16; the fp32 state is split
//       into hi + lo bf16 halves (S = hi + lo to ~2^-17 relative), two MFMAs per
//       k-step, fp32 accumulation.
//   verify_valu_kernel<D, T>  any supported d and dtype, plain fp32 FMAs.
//
// Work decomposition: one 256-thread workgroup per (request, value head); the
// two value heads that share a qk head are placed on the same XCD so their
// K/Q rows are read from HBM once (except in the commit + verify steps).
#include "mfma_common.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// LDS layout of the MFMA kernel (bytes)
// ---------------------------------------------------------------------------

// Node slots of the contraction: keys of node i at slot i, queries at slot
// NP + i, NP = 32 * NPB >= N (a whole number of 32-row blocks, so a node's key
// and query results sit in the same lane and register of different blocks).
struct MfmaLds {
    int a, v, gk, gq, nrm, sk, sq, al, be, rows, dep, anc, cidx, mh, ml, cr, cq, total;
    int mstride;  // bytes per row of the bf16 M halves
    // previous step's accepted path (fused commit): k rows (MFMA operand
    // layout), v rows, gates, k scales, rows; placed over the Gram block when
    // it fits (the Gram block is dead by the time the path is staged)
    int kp, vp, alp, bep, scp, rowp;
    // stored-U verify: hi / lo halves of W = (I + G)^-1 (the M halves' layout)
    int wh, wl;
    // one-launch layer step: conv staging (tree, path), conv weights and
    // bias, tap rows, parents, and the staging of a later path segment's conv
    int xg, pc, wts, bia, tap, par, stg, sw, sb;
};


__host__ __device__ inline MfmaLds mfma_lds_layout(int N, int NPB, int Lp = 0, bool wsolve = false) {
    MfmaLds L{};
    const int NP = 32 * NPB;
    const int MB = 2 * NPB;
    const int T = N * (N + 1) / 2;  // Gram entries j <= i (ancestors have smaller indices)
    int off = 0;
    L.mstride = NP * 2 + 8;
    // live for the whole kernel (V too while one 32-row block is staged early)
    L.a = off;    off += align_up(MB * 32 * kKQStride, 16);  // K/Q rows (bf16)
    if (NPB == 1) {
        L.v = off;  off += align_up(N * kD * 2, 16);          // V rows (bf16)
    }
    // per-node arrays written by every lane carry one spare entry (index N)
    L.be = off;   off += align_up((N + 1) * 4, 16);
    L.rows = off; off += align_up((N + 1) * 4, 16);
    if (NPB == 1) {
        L.mh = off;   off += align_up(NP * L.mstride, 16);
        L.ml = off;   off += align_up(NP * L.mstride, 16);
        if (wsolve) {
            L.wh = off;   off += align_up(NP * L.mstride, 16);
            L.wl = off;   off += align_up(NP * L.mstride, 16);
        }
    } else {
        // wide trees: M is solved in place of the q.k triangle (fp32) and read
        // from it, masked by the ancestor bits, as the readout's operand
        L.gq = off;   off += align_up(T * 4, 16);
        L.anc = off;  off += align_up((N + 1) * 8, 16);
    }
    L.cr = off;   off += align_up(N * 4, 16);      // P_i / |k_i|
    L.cq = off;   off += align_up(N * 4, 16);      // P_i / |q_i|
    // the previous path's rows are written at the start, so they get space of their own
    const int lp = Lp > 0 ? Lp : 0;
    L.rowp = off; off += align_up((lp + 1) * 4, 16);  // one spare entry
    // one region, used up to the M solve by the Gram block and the node
    // metadata, after it by the V rows (two 32-row blocks: staged late) and
    // the previous path's staged rows
    const int U = off;
    int f = U;
    L.gk = f;   f += align_up(T * 4, 16);   // k_i . k_j (raw operands), row-major lower triangle
    if (NPB == 1) {
        L.gq = f;   f += align_up(T * 4, 16);   // q_i . k_j
    }
    L.nrm = f;  f += align_up(2 * NP * 4, 16);   // squared norms by slot
    L.sk = f;   f += align_up(N * 4, 16);
    L.sq = f;   f += align_up(N * 4, 16);
    L.al = f;   f += align_up((N + 1) * 4, 16);
    L.dep = f;  f += align_up((N + 1) * 4, 16);
    if (NPB == 1) {
        L.anc = f;  f += align_up((N + 1) * 8, 16);
    }
    if (NPB == 1) {
        L.cidx = f; f += align_up(N * N, 16);    // [i][p]: node at depth p+1 on i's root path
    }
    int uend = f;
    f = U;
    if (NPB != 1) L.v = L.a;  // staged after the state contraction, the block's last use
    const int gsz = lp > 0 ? kMfmaPath * kMfmaPath * 4 : 0;
    L.kp = f;   f += align_up(lp * kKQStride, 16);
    L.vp = f;   f += align_up(lp * kD * 2, 16);
    L.alp = f;  f += align_up(lp * 4, 16);
    L.bep = f;  f += align_up(lp * 4, 16);
    L.scp = f;  f += align_up(lp * 4 + gsz, 16);  // scales, then the segment Gram
    uend = uend > f ? uend : f;
    L.total = uend;
    return L;
}


// Conv weights of the layer step in LDS: word e (tap pair e % kWP of channel
// 4c + e / kWP) of lane chunk c at e * kWtsRow + c, so the lanes of a
// half-wave read consecutive words (one word each) and a writer lane's word
// lands in its own bank too.
constexpr int kWtsRow = 33;
constexpr int kWtsGroup = 8 * kWtsRow;  // words per channel group (up to 8 words per chunk)

// Layer step (N <= 32, one 32-row block).  One region F is used in turn by
// (1) the v rows and the new history of the tree's conv, (2) the verify
// stages up to the M solve, (3) the replay of one path segment (and the
// staging of a later segment's conv); each set is dead before the next is
// written.  The previous path's conv rows sit in the key block until the
// key conv writes it; the conv weights and bias overlay the M halves,
// written only after the conv.
__host__ __device__ inline MfmaLds layer_lds_layout(int N, int H, int Lmax) {
    MfmaLds L{};
    constexpr int NP = 32;
    int off = 0;
    L.mstride = NP * 2 + 8;
    L.a = off;    off += align_up(2 * 32 * kKQStride, 16);
    L.v = off;    off += align_up(N * kD * 2, 16);
    const int F = off;
    int f = F;
    L.gk = f;   f += align_up(N * (N + 1) / 2 * 4, 16);  // lower triangle, j <= i
    L.gq = f;   f += align_up(N * (N + 1) / 2 * 4, 16);
    L.nrm = f;  f += align_up(2 * NP * 4, 16);
    L.sk = f;   f += align_up(N * 4, 16);
    L.sq = f;   f += align_up(N * 4, 16);
    L.cidx = f; f += align_up(N * N, 16);
    int fend = f;
    L.xg = F;   // v rows of the tree (N x 256 bytes), then the new history [3][H][256]
    fend = imax(fend, F + align_up((N + 3 * H) * 256, 16));
    L.pc = L.a; // (history ++ path) rows of the first segment's windows, k | v: 512 bytes
    f = F;
    L.kp = f;   f += align_up(kMfmaPath * kKQStride, 16);
    L.vp = f;   f += align_up(kMfmaPath * kD * 2, 16);
    L.scp = f;  f += align_up((kMfmaPath + kMfmaPath * kMfmaPath) * 4, 16);
    L.stg = f;  f += align_up((H + 8) * 256, 16);
    L.sw = f;   f += align_up(256 * 4, 16);
    L.sb = f;   f += align_up(kD * 4, 16);
    fend = imax(fend, f);
    off = fend;
    L.be = off;   off += align_up((N + 1) * 4, 16);
    L.rows = off; off += align_up((N + 1) * 4, 16);
    L.al = off;   off += align_up((N + 1) * 4, 16);
    L.dep = off;  off += align_up((N + 1) * 4, 16);
    L.anc = off;  off += align_up((N + 1) * 8, 16);
    L.mh = off;
    L.ml = off + align_up(NP * L.mstride, 16);
    L.wts = off;                        // [3][kWtsGroup] tap-pair words: k, q, v
    L.bia = off + 3 * kWtsGroup * 4;    // [3][128]
    off += imax(2 * align_up(NP * L.mstride, 16), 3 * kWtsGroup * 4 + 3 * kD * 4);
    L.cr = off;   off += align_up(N * 4, 16);
    L.cq = off;   off += align_up(N * 4, 16);
    L.alp = off;  off += align_up((Lmax + 1) * 4, 16);
    L.bep = off;  off += align_up((Lmax + 1) * 4, 16);
    L.tap = off;  off += align_up(N * (H > 0 ? H : 1), 16);
    L.par = off;  off += align_up((N + 1) * 4, 16);
    L.rowp = off; off += align_up((Lmax + 1) * 4, 16);
    L.total = off;
    return L;
}

// The layout's offsets as wave-uniform (scalar) values: the LDS array bases
// then live in scalar registers instead of taking vector registers the state
// kernels do not have.
__device__ __forceinline__ MfmaLds uniform_layout(MfmaLds L) {
    static_assert(sizeof(MfmaLds) % sizeof(int) == 0, "MfmaLds holds ints only");
    int* f = reinterpret_cast<int*>(&L);
#pragma unroll
    for (int i = 0; i < static_cast<int>(sizeof(MfmaLds) / sizeof(int)); ++i) f[i] = __builtin_amdgcn_readfirstlane(f[i]);
    return L;
}

// The previous step's accepted path for the fused commit, resolved to
// physical rows (kernel argument), and its recorded operands.
struct CommitPrev {
    int Rp, Lmax;
    const int32_t* path_rows;
    const int32_t* path_n;
    const uint16_t* kp;
    const uint16_t* vp;
    int64_t rs_qk_p, rs_v_p;
    const float* alpha_p;
    const float* beta_p;
};

constexpr int kModeVerify = 0;
constexpr int kModeCommitVerify = 1;
constexpr int kModeLayer = 2;      // paths of at most kMfmaPath nodes (Lmax <= kMfmaPath)
constexpr int kModeLayerLong = 3;  // any Lmax: later path segments convolved inside the replay
constexpr int kModeVerifyU = 4;    // verify that also writes every node's delta correction u_i

}  // namespace

// ===========================================================================
// MFMA kernel: bf16 q/k/v, d_k = d_v = 128, N <= 32*NPB
//
// Matrix form of the same recurrence (Bole review, Sec. 3.2-3.5, Eq. (2)-(5)),
// per (request, head), with P_i the product of the decays on the root-to-i
// path and hats for the (optionally) normalised q, k:
//   R = D_beta (V - D_P K^ S_pre^T),  G_ij = b_i (P_i/P_j) k^_i.k^_j  (j strict ancestor of i)
//   O = D_P Q^ S_pre^T + C (I + G)^-1 R,  C_ij = (P_i/P_j) q^_i.k^_j  (j ancestor of i or i)
// M = C (I + G)^-1 is formed row by row: M (I + G) = C gives, along node i's
// own root path, M_ij = C_ij - sum_{j < m <= i on the path} M_im G_mj, a solve of
// depth^2/2 multiply-adds per node (the tree's depth bounds it, as Lemma 3 of
// the Bole review bounds the Neumann series) instead of a general solve.
// The ratios P_i/P_j are taken as products of the decays strictly below j.
// ===========================================================================
template <int NPB, int MODE, int CW, bool RAW>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NPB == 1 ? 4 : 3, 8)))
    verify_mfma_kernel(int N, int R, int shared, const int32_t* __restrict__ node_row,
                       const uint64_t* __restrict__ anc_g, const int32_t* __restrict__ depth_g,
                       const int32_t* __restrict__ status, const uint16_t* __restrict__ q,
                       const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                       int64_t rs_qk, int64_t rs_v, const float* __restrict__ alpha,
                       const float* __restrict__ beta, float* __restrict__ pool, int P,
                       const int32_t* __restrict__ state_idx, void* __restrict__ out, int Hqk,
                       int Hv, int norm, int out_bf16, int32_t* __restrict__ err,
                       const float* __restrict__ gate_params, const CommitPrev cp, const LayerIn li,
                       float* __restrict__ u_out) {
    constexpr bool FUSED = MODE == kModeCommitVerify;  // commit of a path given as k/v rows
    constexpr bool LAYER = MODE == kModeLayer || MODE == kModeLayerLong;  // the whole layer step
    constexpr bool LONGP = MODE == kModeLayerLong;
    constexpr bool COMMIT = FUSED || LAYER;
    // stored-U mode (Bole review, Sec. 5.2, Algorithm 2 steps 5-7): besides
    // M = C (I + G)^-1 the path solve forms W = (I + G)^-1 (the same
    // elimination from the identity), and U = W R, every node's u_i, is
    // written out for a later factorised commit
    constexpr bool STOREU = MODE == kModeVerifyU;
    static_assert(!STOREU || NPB == 1, "stored-U verify: N <= 32 on the matrix cores");
    constexpr int H = CW > 0 ? CW - 1 : 0;             // conv history entries (layer step)
    constexpr int kWP = (CW + 1) / 2;                  // conv tap pairs per channel
    static_assert(!LAYER || (NPB == 1 && CW >= 1 && CW <= 4), "layer step: N <= 32, 1 <= W <= 4");
    constexpr int NP = 32 * NPB;
    constexpr int MB = 2 * NPB;                              // key blocks, then query blocks
    constexpr int kKQItems = MB * 32 * 32 / kThreads;       // 8-byte K/Q chunks per thread
    constexpr int kVItems = (NP * 32 + kThreads - 1) / kThreads;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const MfmaLds L = uniform_layout(LAYER ? layer_lds_layout(N, H, li.Lmax)
                                           : mfma_lds_layout(N, NPB, FUSED ? cp.Lmax : 0, STOREU));
    char* s_a = lds + L.a;
    uint16_t* s_v = reinterpret_cast<uint16_t*>(lds + L.v);
    float* s_gk = reinterpret_cast<float*>(lds + L.gk);
    float* s_gq = reinterpret_cast<float*>(lds + L.gq);
    float* s_nrm = reinterpret_cast<float*>(lds + L.nrm);
    float* s_sk = reinterpret_cast<float*>(lds + L.sk);
    float* s_sq = reinterpret_cast<float*>(lds + L.sq);
    float* s_al = reinterpret_cast<float*>(lds + L.al);
    float* s_be = reinterpret_cast<float*>(lds + L.be);
    int32_t* s_rows = reinterpret_cast<int32_t*>(lds + L.rows);
    int32_t* s_dep = reinterpret_cast<int32_t*>(lds + L.dep);
    uint64_t* s_anc = reinterpret_cast<uint64_t*>(lds + L.anc);
    uint8_t* s_cidx = reinterpret_cast<uint8_t*>(lds + L.cidx);
    char* s_mh = lds + L.mh;
    char* s_ml = lds + L.ml;
    float* s_cr = reinterpret_cast<float*>(lds + L.cr);
    float* s_cq = reinterpret_cast<float*>(lds + L.cq);
    const int mstride = L.mstride;

    constexpr int kSlots = NP / 8;      // node slots per thread: node tid/32 + 8u
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addressing
    const int hf = lane >> 5;
    const int l32 = lane & 31;
    const int r_own = wave * 32 + l32;  // value row this lane owns in every MFMA

    // the steady-state steps (commit + verify) take units in plain workgroup
    // order: measured faster than keeping a request's qk-sharing heads on one
    // XCD on the 27-node, B = 128 workload (layer step 145-148 against
    // 150-151 us per launch, commit + verify 127 against 129 us; 64-node
    // trees unchanged), although the two heads of a qk group then fetch
    // their shared rows on two XCDs
    const uint32_t unit = COMMIT ? blockIdx.x : xcd_local_order(blockIdx.x, gridDim.x);
    const int b = static_cast<int>(unit / Hv);
    const int h = static_cast<int>(unit % Hv);
    const int t = shared ? 0 : b;
    const int g = static_cast<int>((static_cast<int64_t>(h) * Hqk) / Hv);
    const size_t tb = static_cast<size_t>(t) * N;
    const size_t rowb = static_cast<size_t>(b) * R;
    // layer step: this unit's q and k (qk head g) and v (head h) channels in
    // the conv input, order [q | k | v], head-major
    const int cq0 = g * kD, ck0 = Hqk * kD + g * kD, cv0 = 2 * Hqk * kD + h * kD;
    const uint16_t* kbase = LAYER ? li.x + ck0 : k + static_cast<size_t>(g) * kD;
    const uint16_t* qbase = LAYER ? li.x + cq0 : q + static_cast<size_t>(g) * kD;
    const uint16_t* vbase = LAYER ? li.x + cv0 : v + static_cast<size_t>(h) * kD;
    const int64_t rsq = LAYER ? static_cast<int64_t>(li.C) : rs_qk;
    const int64_t rsv = LAYER ? static_cast<int64_t>(li.C) : rs_v;

    // (a) Memory, in three waves of loads.  A wave's vector loads retire in
    //     issue order, so the K/Q/V rows go out before the 64 KiB state: the
    //     Gram block and the M solve below run on them while the state is
    //     still arriving, and only the state contraction waits for it.
    //   (a1) the tree's rows per node slot, this lane's node's row, ancestors
    //   and depth; status and slot.  Every load here and below is
    //   unconditional, from an index clamped into range, and unused results
    //   are dropped afterwards: a load under a per-lane condition becomes a
    //   branch that waits for it before the next one issues.
    const int st = status[t];
    const int slot = state_idx[b];
    int nrow[kSlots];
#pragma unroll
    for (int x = 0; x < kSlots; ++x) nrow[x] = node_row[tb + min(tid / 32 + 8 * x, N - 1)];
    const int my_node = min(tid, N - 1);
    const int my_row = node_row[tb + my_node];
    const uint64_t my_anc = anc_g[tb + my_node];
    const int my_dep = depth_g[tb + my_node];
    //   raw gate inputs: the head's gate parameters (used when the gates are
    //   staged)
    float g_alog = 0.0f, g_dtb = 0.0f;
    if constexpr (RAW) {
        g_alog = gate_params[h];
        g_dtb = gate_params[Hv + h];
    }
    //   (a1') the previous step's accepted path, resolved to its node count
    //   (-1: neither state nor history is written) and physical rows
    const int LmaxP = LAYER ? li.Lmax : (FUSED ? cp.Lmax : 1);
    const int RpP = LAYER ? li.Rp : (FUSED ? cp.Rp : 1);
    int pn = 0, prow = 0, my_par = -1;
    if constexpr (FUSED) {
        pn = cp.path_n[b];
        prow = cp.path_rows[static_cast<size_t>(b) * cp.Lmax + min(tid, cp.Lmax - 1)];
    }
    //   (a1'') layer step: the tree's parents (conv taps), the conv weights
    //   (as tap pairs) and bias of the unit's channels
    uint32_t wq[3] = {0u, 0u, 0u};
    float bq[3] = {0.f, 0.f, 0.f};
    if constexpr (LAYER) {
        pn = li.path_n[b];
        prow = li.path_rows[static_cast<size_t>(b) * li.Lmax + min(tid, li.Lmax - 1)];
        my_par = li.parent[tb + my_node];
#pragma unroll
        for (int u = 0; u < 3; ++u) {  // groups k, q, v
            const int cb = u == 0 ? ck0 : (u == 1 ? cq0 : cv0);
            wq[u] = conv_weight_word<CW>(li.w, cb, tid);
            if (li.bias) bq[u] = li.bias[cb + (tid & (kD - 1))];
        }
    }
    if (slot < 0 || slot >= P) {
        if ((COMMIT || st == 0) && h == 0 && tid == 0) atomicOr(err, GDN_EV_STATE);
        return;
    }
    // the new tree is verified only if it is well formed; the fused commit of
    // the previous path happens either way
    const bool vok = st == 0;
    if (!COMMIT && !vok) return;
    float* s_alp = reinterpret_cast<float*>(lds + L.alp);
    float* s_bep = reinterpret_cast<float*>(lds + L.bep);
    float* s_scp = reinterpret_cast<float*>(lds + L.scp);
    int32_t* s_rowp = reinterpret_cast<int32_t*>(lds + L.rowp);
    char* s_kp = lds + L.kp;
    uint16_t* s_vp = reinterpret_cast<uint16_t*>(lds + L.vp);
    uint32_t* s_wts = reinterpret_cast<uint32_t*>(lds + L.wts);
    float* s_bia = reinterpret_cast<float*>(lds + L.bia);
    int32_t* s_par = reinterpret_cast<int32_t*>(lds + L.par);
    uint8_t* s_tap = reinterpret_cast<uint8_t*>(lds + L.tap);
    // n = -1 writes neither state nor history; nc path nodes commit
    const int n_res = COMMIT ? min(max(pn, -1), LmaxP) : 0;
    const int nc = n_res > 0 ? n_res : 0;
    if constexpr (FUSED) {
        s_rowp[min(tid, cp.Lmax)] = prow;  // every lane writes (spare entry Lmax)
        __syncthreads();
    }
    if constexpr (LAYER) {
        // every lane writes (spare entries Lmax and N)
        s_rowp[min(tid, li.Lmax)] = prow;
        s_par[min(tid, N)] = my_par;
        s_rows[min(tid, N)] = my_row;
        s_anc[min(tid, N)] = my_anc;
        s_dep[min(tid, N)] = my_dep;
#pragma unroll
        for (int u = 0; u < 3; ++u)
            if (tid < kD * kWP) s_wts[u * kWtsGroup + (tid % (4 * kWP)) * kWtsRow + tid / (4 * kWP)] = wq[u];
        if (li.bias) {
#pragma unroll
            for (int u = 0; u < 3; ++u) s_bia[u * kD + (tid & (kD - 1))] = bq[u];
        }
        __syncthreads();
    }
    // physical row of path node j of the previous tree, clamped into range
    auto prow_at = [&](int j) -> int {
        const int r = s_rowp[min(max(j, 0), LmaxP - 1)];
        return min(max(r, 0), RpP - 1);
    };
    //   (a2) K/Q/V chunks and the gates of every node (rows of a valid tree are
    //        in range, so the clamped loads are too)
    static_assert(kKQItems == 2 * kSlots && kVItems == kSlots, "item u uses node slot u mod kSlots");
    uint2 kq_val[kKQItems];
    uint2 v_val[kVItems];
    float my_al = 0.f, my_be = 0.f;
    if (vok) {  // uniform
#pragma unroll
        for (int u = 0; u < kKQItems; ++u) {
            const int sl = (tid + u * kThreads) >> 5;
            const uint16_t* src = (sl < NP ? kbase : qbase) + (rowb + nrow[u % kSlots]) * rsq + (tid & 31) * 4;
            kq_val[u] = *reinterpret_cast<const uint2*>(src);
        }
#pragma unroll
        for (int u = 0; u < kVItems; ++u)
            v_val[u] = *reinterpret_cast<const uint2*>(vbase + (rowb + nrow[u]) * rsv + (tid & 31) * 4);
        const size_t my_gi = (rowb + my_row) * Hv + h;
        my_al = alpha[my_gi];
        my_be = beta[my_gi];
    }
    //   (a2'') layer step: the previous path's conv input -- the old history
    //   and the path's rows as the rows (history ++ path) of its first
    //   segment's windows, k | v channels, plus the q channels of the new
    //   history -- and the path's gates
    constexpr int kPC = (H + 8) * 32;  // 16-byte items: H + 8 rows x (k | v)
    constexpr int kNH = H * 16;        // 16-byte items: H rows x q
    constexpr int kPItems = LAYER ? (kPC + kNH + kThreads - 1) / kThreads : 1;
    uint4 pc_val[kPItems];
    uint4 nh_kv = make_uint4(0u, 0u, 0u, 0u);
    uint2 pk_val = make_uint2(0u, 0u), pv_val = make_uint2(0u, 0u);
    float p_al = 0.f, p_be = 0.f;
    if constexpr (LAYER) {
#pragma unroll
        for (int u = 0; u < kPItems; ++u) {
            const int it = min(tid + u * kThreads, kPC + kNH - 1);
            int ci, col;  // row of (history ++ path) and channel
            if (it < kPC) {
                const int c16 = it & 31;
                ci = it >> 5;
                col = c16 < 16 ? ck0 + 8 * c16 : cv0 + 8 * (c16 - 16);
            } else {
                ci = nc + ((it - kPC) >> 4);
                col = cq0 + 8 * ((it - kPC) & 15);
            }
            const uint16_t* src = li.x_prev + (static_cast<size_t>(b) * li.Rp + prow_at(ci - H)) * li.C + col;
            if constexpr (H > 0) {
                if (ci < H) src = li.hist_in + (static_cast<size_t>(slot) * H + ci) * li.C + col;
            }
            pc_val[u] = *reinterpret_cast<const uint4*>(src);
        }
        const size_t gi = (static_cast<size_t>(b) * li.Rp + prow_at(min(tid, nc - 1))) * Hv + h;
        p_al = li.alpha_p[gi];
        p_be = li.beta_p[gi];
    }
    //   (a2') fused: the previous path's k/v rows (its first kMfmaPath rows)
    //   and gates
    if constexpr (FUSED) {
        const size_t rbp = static_cast<size_t>(b) * cp.Rp + prow_at(min(tid >> 5, nc - 1));
        pk_val = *reinterpret_cast<const uint2*>(cp.kp + rbp * cp.rs_qk_p + static_cast<size_t>(g) * kD +
                                                 (tid & 31) * 4);
        pv_val = *reinterpret_cast<const uint2*>(cp.vp + rbp * cp.rs_v_p + static_cast<size_t>(h) * kD +
                                                 (tid & 31) * 4);
        const size_t gi = (static_cast<size_t>(b) * cp.Rp + prow_at(min(tid, nc - 1))) * Hv + h;
        p_al = cp.alpha_p[gi];
        p_be = cp.beta_p[gi];
    }
    //   (a3) the committed state, loaded in 64-byte row segments; after the
    //        fix-up at its first use, lane (r_own, hf) holds chunks 2t + hf of
    //        row r_own in register t.  The layer step issues it only once its
    //        conv input is staged in LDS (below): the input rows then do not
    //        queue behind every unit's state, the registers that held them
    //        are free, and the conv, Gram block and M solve still cover the
    //        state's latency.
    float* Sw = pool + (static_cast<size_t>(slot) * Hv + h) * (kD * kD) + static_cast<size_t>(wave) * 32 * kD;
    float4 sreg[16];
    // the state's loads, in four chunks of four (chunk c: loads 4c .. 4c+3):
    // a wave whose memory requests the CU cannot take yet stalls at issue,
    // so the layer step spreads the chunks over its conv phases
    auto issue_state_chunk = [&](int c) {
        asm volatile("" ::: "memory");  // keep the state loads behind the loads above
        const float* Sl = Sw + state_load_lane_off(l32, hf);
#pragma unroll
        for (int s = 0; s < 16; ++s)
            if ((s >> 2) == c) sreg[s] = *reinterpret_cast<const float4*>(Sl + state_load_off(s));
    };
    if constexpr (!LAYER) {
#pragma unroll
        for (int c = 0; c < 4; ++c) issue_state_chunk(c);
    }
    bool sfixed = false;  // uniform: the state is in the matrix-core layout

    if constexpr (FUSED) {
        // used under per-lane conditions after the M solve: take delivery
        // here (the state, issued after them, stays in flight)
        asm volatile("" ::"v"(pk_val.x), "v"(pk_val.y), "v"(pv_val.x), "v"(pv_val.y), "v"(p_al), "v"(p_be));
    }

    // layer step: publish the new conv history, convolve the previous path's
    // first segment into k/v chunks held in registers and the new tree into
    // the K/Q/V rows (LumoTree, Sec. V-A: the accepted path's conv rows
    // become the history; Sec. V-C: each window follows the node's ancestry,
    // then the history)
    if constexpr (LAYER) {
        // the loads above are used under per-lane conditions below: take
        // delivery here (the state is issued once they are staged)
#pragma unroll
        for (int u = 0; u < kPItems; ++u)
            asm volatile("" ::"v"(pc_val[u].x), "v"(pc_val[u].y), "v"(pc_val[u].z), "v"(pc_val[u].w));
        asm volatile("" ::"v"(p_al), "v"(p_be));
        if (LONGP && H > 0 && nc > kMfmaPath) {  // uniform: the new history lies past the first segment
            // (paths longer than one segment only: this waits for the state too)
            const int e = min(tid, H * 32 - 1);
            const int c16 = e & 31;
            const int col = c16 < 16 ? ck0 + 8 * c16 : cv0 + 8 * (c16 - 16);
            nh_kv = *reinterpret_cast<const uint4*>(
                li.x_prev + (static_cast<size_t>(b) * li.Rp + prow_at(nc - H + (e >> 5))) * li.C + col);
        }
#pragma unroll
        for (int u = 0; u < kKQItems; ++u) asm volatile("" ::"v"(kq_val[u].x), "v"(kq_val[u].y));
#pragma unroll
        for (int u = 0; u < kVItems; ++u) asm volatile("" ::"v"(v_val[u].x), "v"(v_val[u].y));
        const bool qk_writer = (h % (Hv / Hqk)) == 0;  // one head per qk group writes q/k channels
        const bool has_bias = li.bias != nullptr;
        // stage everything in LDS at once.  Each conv group's output
        // overwrites only input already used: the path's rows in the key
        // block (the path conv runs first), k rows in the query block, q rows
        // in the V rows, v rows and the new history (groups k, q, v) in F
        char* xk = s_a + NP * kKQStride;
        char* xq = reinterpret_cast<char*>(s_v);
        char* xv = lds + L.xg;
        char* hg = xv + N * 256;
        const int nl = tid >> 5;
        const int c4 = tid & 31;
        if (nc > 0) {  // uniform
            // the path's gates (nc <= Lmax <= 64: wave 0; spare entry Lmax)
            if constexpr (RAW) {
                s_alp[min(tid, li.Lmax)] = raw_gate_alpha(p_al, raw_gate_params(g_alog, g_dtb));
                s_bep[min(tid, li.Lmax)] = raw_gate_beta(p_be);
            } else {
                s_alp[min(tid, li.Lmax)] = p_al;
                s_bep[min(tid, li.Lmax)] = p_be;
            }
            uint4* s_pc = reinterpret_cast<uint4*>(lds + L.pc);  // [H + 8][32]: k half, v half
#pragma unroll
            for (int u = 0; u < kPItems; ++u) {
                const int it = tid + u * kThreads;
                if (it < kPC) s_pc[it] = pc_val[u];
            }
        }
        if (vok) {  // uniform
            {
                const int slot_i = tid < N ? tid : N;  // lanes past N write the spare entry
                if constexpr (RAW) {
                    s_al[slot_i] = raw_gate_alpha(my_al, raw_gate_params(g_alog, g_dtb));
                    s_be[slot_i] = raw_gate_beta(my_be);
                } else {
                    s_al[slot_i] = my_al;
                    s_be[slot_i] = my_be;
                }
            }
#pragma unroll
            for (int u = 0; u < kSlots; ++u) {
                const int node = nl + 8 * u;
                if (node < N) {
                    *reinterpret_cast<uint2*>(xk + node * 256 + c4 * 8) = kq_val[u];
                    *reinterpret_cast<uint2*>(xq + node * 256 + c4 * 8) = kq_val[kSlots + u];
                    *reinterpret_cast<uint2*>(xv + node * 256 + c4 * 8) = v_val[u];
                }
            }
            if constexpr (H > 0) {
#pragma unroll
                for (int u = 0; u < kPItems; ++u) {
                    const int it = tid + u * kThreads;
                    if (it < kPC) {
                        const int c16 = it & 31;
                        const int m = (it >> 5) - nc;
                        if ((!LONGP || nc <= kMfmaPath) && m >= 0 && m < H)
                            *reinterpret_cast<uint4*>(hg + ((c16 < 16 ? 0 : 2) * H + m) * 256 + (c16 & 15) * 16) =
                                pc_val[u];
                    } else if (it < kPC + kNH) {
                        const int e = it - kPC;
                        *reinterpret_cast<uint4*>(hg + (H + (e >> 4)) * 256 + (e & 15) * 16) = pc_val[u];
                    }
                }
                if (LONGP && nc > kMfmaPath && tid < H * 32) {
                    const int c16 = tid & 31;
                    *reinterpret_cast<uint4*>(hg + ((c16 < 16 ? 0 : 2) * H + (tid >> 5)) * 256 + (c16 & 15) * 16) =
                        nh_kv;
                }
                // the new tree's conv taps as staged rows: node j < N, or
                // history entry s at N + s (s = W-2 the most recent); oldest first
                if (tid < N) {
                    int cur = s_par[tid];
                    int hs = H - 1;
#pragma unroll
                    for (int m = 0; m < H; ++m) {
                        int tap;
                        if (cur >= 0) {
                            tap = cur;
                            cur = s_par[cur];
                        } else {
                            tap = N + hs;
                            --hs;
                        }
                        s_tap[tid * H + (H - 1 - m)] = static_cast<uint8_t>(tap);
                    }
                }
            }
        }
        // publish: new history entry m = (old history ++ path rows)[nc + m]
        if constexpr (H > 0) {
            if (n_res >= 0) {  // uniform
                uint16_t* ho = li.hist_out + static_cast<size_t>(slot) * H * li.C;
#pragma unroll
                for (int u = 0; u < kPItems; ++u) {
                    const int it = tid + u * kThreads;
                    int m = 0, col = 0;
                    bool wr = false;
                    if (it < kPC) {
                        const int c16 = it & 31;
                        m = (it >> 5) - nc;
                        col = c16 < 16 ? ck0 + 8 * c16 : cv0 + 8 * (c16 - 16);
                        wr = (!LONGP || nc <= kMfmaPath) && m >= 0 && m < H && (c16 >= 16 || qk_writer);
                    } else if (it < kPC + kNH) {
                        m = (it - kPC) >> 4;
                        col = cq0 + 8 * ((it - kPC) & 15);
                        wr = qk_writer;
                    }
                    if (wr) *reinterpret_cast<uint4*>(ho + static_cast<size_t>(m) * li.C + col) = pc_val[u];
                }
                if (LONGP && nc > kMfmaPath && tid < H * 32) {
                    const int c16 = tid & 31;
                    const int col = c16 < 16 ? ck0 + 8 * c16 : cv0 + 8 * (c16 - 16);
                    if (c16 >= 16 || qk_writer)
                        *reinterpret_cast<uint4*>(ho + static_cast<size_t>(tid >> 5) * li.C + col) = nh_kv;
                }
            }
        }
        __syncthreads();
        // the conv input is in LDS now: the state's first chunk, the others
        // with the tree's conv groups (all of them now if there is no tree)
        issue_state_chunk(0);
        if (nc > 0) {  // uniform: the previous path's first segment, k and v channels
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int grp = half == 0 ? 0 : 2;
                uint32_t wv[4 * kWP];
#pragma unroll
                for (int e = 0; e < 4 * kWP; ++e) wv[e] = s_wts[grp * kWtsGroup + e * kWtsRow + c4];
                float bb[4] = {0.f, 0.f, 0.f, 0.f};
                if (has_bias) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) bb[e] = s_bia[grp * kD + 4 * c4 + e];
                }
                const char* rp[CW];
#pragma unroll
                for (int t = 0; t <= H; ++t) rp[t] = lds + L.pc + (nl + t) * 512 + half * 256;
                const uint2 o = conv4_rows<CW>(rp, c4, wv, bb, has_bias, li.act);
                if (half == 0)
                    pk_val = o;
                else
                    pv_val = o;
            }
            __syncthreads();
        }
        // the new tree's conv, groups k, q, v (a malformed tree has none; the
        // state's chunks are issued on every path, so no path leaves loads
        // pending on registers another path reuses)
#pragma unroll
        for (int grp = 0; grp < 3; ++grp) {
            issue_state_chunk(grp + 1);
            if (vok) {  // uniform
                const char* src = grp == 0 ? xk : (grp == 1 ? xq : xv);
                const int cb = grp == 0 ? ck0 : (grp == 1 ? cq0 : cv0);
                uint32_t wv[4 * kWP];
#pragma unroll
                for (int e = 0; e < 4 * kWP; ++e) wv[e] = s_wts[grp * kWtsGroup + e * kWtsRow + c4];
                float bb[4] = {0.f, 0.f, 0.f, 0.f};
                if (has_bias) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) bb[e] = s_bia[grp * kD + 4 * c4 + e];
                }
#pragma unroll 2
                for (int x = 0; x < kSlots; ++x) {
                    const int i = nl + 8 * x;
                    if (i < N) {
                        const char* rp[CW];
#pragma unroll
                        for (int t = 0; t < H; ++t) {
                            const int r = s_tap[i * H + t];
                            rp[t] = r < N ? src + r * 256 : hg + (grp * H + r - N) * 256;
                        }
                        rp[H] = src + i * 256;
                        const uint2 o = conv4_rows<CW>(rp, c4, wv, bb, has_bias, li.act);
                        char* dst = grp == 2 ? reinterpret_cast<char*>(s_v) + i * (kD * 2)
                                             : s_a + (grp == 1 ? NP + i : i) * kKQStride;
                        *reinterpret_cast<uint2*>(dst + c4 * 8) = o;
                        if (li.y && (grp == 2 || qk_writer))
                            *reinterpret_cast<uint2*>(li.y + (rowb + s_rows[i]) * li.C + cb + 4 * c4) = o;
                    } else if (grp < 2) {  // zero pad rows of the MFMA blocks
                        *reinterpret_cast<uint2*>(s_a + (grp == 1 ? NP + i : i) * kKQStride + c4 * 8) =
                            make_uint2(0u, 0u);
                    }
                }
            }
            __syncthreads();
        }
    }

    if (vok) {  // uniform: stages (a)-(e) of the new tree
        // stage the metadata, K/Q (with squared norms) and V in LDS.  Every lane
        // writes (lanes past N into the spare entry): a store under a per-lane
        // condition would let the compiler sink the loads above into its branch,
        // behind the state loads, where using them waits for the whole state.
        if constexpr (!LAYER) {  // (the layer step staged these with its conv input)
            const int slot_i = tid < N ? tid : N;
            s_rows[slot_i] = my_row;
            s_anc[slot_i] = my_anc;
            s_dep[slot_i] = my_dep;
            if constexpr (RAW) {
                s_al[slot_i] = raw_gate_alpha(my_al, raw_gate_params(g_alog, g_dtb));
                s_be[slot_i] = raw_gate_beta(my_be);
            } else {
                s_al[slot_i] = my_al;
                s_be[slot_i] = my_be;
            }
        }
        if constexpr (NPB == 1) {
            // M halves start as zero (entries off the ancestor pattern stay zero)
            for (int e = tid; e < NP * mstride / 4; e += kThreads) {
                reinterpret_cast<uint32_t*>(s_mh)[e] = 0u;
                reinterpret_cast<uint32_t*>(s_ml)[e] = 0u;
                if constexpr (STOREU) {
                    reinterpret_cast<uint32_t*>(lds + L.wh)[e] = 0u;
                    reinterpret_cast<uint32_t*>(lds + L.wl)[e] = 0u;
                }
            }
        }
        if constexpr (LAYER) {  // K/Q/V rows are staged; squared norms from them
    #pragma unroll
            for (int u = 0; u < kKQItems; ++u) {
                const int it = tid + u * kThreads;
                const int sl = it >> 5;
                const int ch = it & 31;
                float ss = sumsq_bf16x4(*reinterpret_cast<const uint2*>(s_a + sl * kKQStride + ch * 8));
                ss = sum_half_wave(ss);
                if (ch == 0) s_nrm[sl] = ss;
            }
        } else {
    #pragma unroll
        for (int u = 0; u < kKQItems; ++u) {
            const int it = tid + u * kThreads;
            const int sl = it >> 5;
            const int ch = it & 31;
            const int node = sl < NP ? sl : sl - NP;
            if (node >= N) kq_val[u] = make_uint2(0u, 0u);  // zero pad rows of the MFMA blocks
            *reinterpret_cast<uint2*>(s_a + sl * kKQStride + ch * 8) = kq_val[u];
            float ss = sumsq_bf16x4(kq_val[u]);  // a row's 32 chunks sit in 32 consecutive lanes
            ss = sum_half_wave(ss);
            if (ch == 0) s_nrm[sl] = ss;
        }
        if constexpr (NPB == 1) {  // two blocks: staged after the M solve, over the Gram block
    #pragma unroll
            for (int u = 0; u < kVItems; ++u) {
                const int it = tid + u * kThreads;
                const int node = it >> 5;
                if (node < N) *reinterpret_cast<uint2*>(s_v + node * kD + (it & 31) * 4) = v_val[u];
            }
        }
        }
        __syncthreads();

        // (b) per node: normalisation scales and the root path list
        if (tid < N) {
            s_sk[tid] = norm ? 1.0f / sqrtf(s_nrm[tid] + 1e-6f) : 1.0f;
            s_sq[tid] = norm ? 1.0f / sqrtf(s_nrm[NP + tid] + 1e-6f) : 1.0f;
            if constexpr (NPB == 1) {  // wide trees read the paths from the ancestor bits
                uint64_t m = s_anc[tid];
                int p = 0;
                while (m) {  // ancestors in index order are root first
                    const int j = __builtin_ctzll(m);
                    m &= m - 1ull;
                    s_cidx[tid * N + p++] = static_cast<uint8_t>(j);
                }
                s_cidx[tid * N + p] = static_cast<uint8_t>(tid);
            }
        }

        // (c) Gram block on the matrix cores (exact bf16 products, fp32 sums):
        //     k_i . k_j and q_i . k_j for j <= i (every ancestor has a smaller
        //     index), stored as row-major lower triangles
        {
            constexpr int kTiles = MB * NPB;  // all query/key row blocks x key column blocks
            for (int tile = wave; tile < kTiles; tile += kThreads / 64) {
                const int ta = tile / NPB;
                const int tcol = tile % NPB;
                if (tcol > ta % NPB) continue;  // wholly above the diagonal (uniform per wave)
                f32x16_t acc = {};
    #pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const bf16x8_t a = lds_operand(s_a, ta * 32 + l32, s, hf);
                    const bf16x8_t bb = lds_operand(s_a, tcol * 32 + l32, s, hf);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
                }
                float* gdst = (ta < NPB) ? s_gk : s_gq;
                const int col = tcol * 32 + l32;
    #pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = (ta % NPB) * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
                    if (row < N && col <= row) gdst[row * (row + 1) / 2 + col] = acc[e];
                }
            }
        }
        __syncthreads();

        // (e) M = C (I + G)^-1, row by row: along node i's root path n_0 .. n_(d-1) = i,
        //       M_(i,n_p) = C_(i,n_p) - sum_(s > p) M_(i,n_s) G_(n_s,n_p)
        //     with C_(i,j) = (P_i/P_j) q^_i.k^_j and G_(m,j) = b_m (P_m/P_j) k^_m.k^_j, the
        //     decay ratios taken as products of the decays strictly below j.  A group
        //     of kLP lanes holds one node, lane p its path position p: each lane forms
        //     its G column, then the deepest position is final and is eliminated from
        //     the shallower ones, one position per step.  In trees of more than
        //     32 nodes, nodes of depth 9..16 go through the same in groups of 16
        //     lanes; deeper ones are solved one thread per node afterwards.
        {
            constexpr int kLP = 8;
            // wide trees only: at N <= 32 the 16-lane groups' registers would
            // spill in the kernels capped at 128 VGPRs
            constexpr int kLP2 = NPB == 1 ? kLP : 16;
            const int p = tid & (kLP - 1);
            for (int i0 = 0; i0 < N; i0 += kThreads / kLP) {
                const int i = i0 + tid / kLP;
                const int ii = min(i, N - 1);
                const int d0 = s_dep[ii];
                // wide trees: a node one deeper than the lanes (depth 9) is
                // solved here too: the lanes take path positions 1 .. 8
                // exactly as a depth-8 path, and position 0 follows at the end
                const int sh = (NPB != 1 && d0 == kLP + 1) ? 1 : 0;  // uniform in the group
                const int d = d0 - sh;  // positions on the lanes
                const bool act = i < N && d <= kLP && p < d;
                const uint8_t* path = s_cidx + ii * N;
                // wide trees: the path from the ancestor bits
                const uint64_t pm = (NPB == 1) ? 0ull : (s_anc[ii] | (1ull << ii));
                int j;  // the node at this lane's position
                if constexpr (NPB == 1) j = path[min(p, d - 1)];
                else j = path_node<kLP + 1>(pm, min(p + sh, d0 - 1));
                const float sk_j = s_sk[j];
                // the path's nodes first (lane sp of the group holds position
                // sp's), then every LDS read at once (each index is a valid
                // node, whether or not the position is in use), then the
                // products: one LDS round trip, not one per position
                int mm[kLP];
    #pragma unroll
                for (int sp = 1; sp < kLP; ++sp) {
                    const int js = __float_as_int(group8_lane_at(__int_as_float(j), sp, p));
                    mm[sp] = sp < d ? js : ii;
                }
                float al[kLP], bs[kLP], gk[kLP];
    #pragma unroll
                for (int sp = 1; sp < kLP; ++sp) {
                    const int m = mm[sp];
                    al[sp] = s_al[m];
                    bs[sp] = s_be[m] * s_sk[m];
                    gk[sp] = s_gk[m * (m + 1) / 2 + j];
                }
                float gco[kLP];
                float r = 1.0f;  // decays of positions p+1 .. s
    #pragma unroll
                for (int sp = 1; sp < kLP; ++sp) {
                    const bool in = sp > p && sp < d;
                    r *= in ? al[sp] : 1.0f;
                    gco[sp] = in ? bs[sp] * sk_j * gk[sp] * r : 0.0f;
                }
                // r = P_i / P_j now
                float val = r * s_sq[ii] * sk_j * s_gq[ii * (ii + 1) / 2 + j];
                float wval = p == d - 1 ? 1.0f : 0.0f;  // W row i starts as the identity's
    #pragma unroll
                for (int sp = kLP - 1; sp >= 1; --sp) {
                    const float ms = group8_lane_at(val, sp, p);  // final M at position sp
                    val = (sp < d && p < sp) ? fmaf(-ms, gco[sp], val) : val;
                    if constexpr (STOREU) {
                        const float ws = group8_lane_at(wval, sp, p);
                        wval = (sp < d && p < sp) ? fmaf(-ws, gco[sp], wval) : wval;
                    }
                }
                if (act) {
                    if constexpr (NPB == 1) {
                        const uint32_t hv = cvt_pk_bf16(val, 0.0f) & 0xffffu;
                        const float rest = val - __uint_as_float(hv << 16);
                        const uint32_t lv = cvt_pk_bf16(rest, 0.0f) & 0xffffu;
                        reinterpret_cast<uint16_t*>(s_mh + i * mstride)[j] = static_cast<uint16_t>(hv);
                        reinterpret_cast<uint16_t*>(s_ml + i * mstride)[j] = static_cast<uint16_t>(lv);
                        if constexpr (STOREU) {
                            const uint32_t hw = cvt_pk_bf16(wval, 0.0f) & 0xffffu;
                            const uint32_t lw2 = cvt_pk_bf16(wval - __uint_as_float(hw << 16), 0.0f) & 0xffffu;
                            reinterpret_cast<uint16_t*>(lds + L.wh + i * mstride)[j] = static_cast<uint16_t>(hw);
                            reinterpret_cast<uint16_t*>(lds + L.wl + i * mstride)[j] = static_cast<uint16_t>(lw2);
                        }
                    } else {
                        s_gq[i * (i + 1) / 2 + j] = val;  // only this lane reads that entry
                    }
                    if (p == 0 && !sh) {
                        const float P_i = r * s_al[j];  // j = n_0: times the root-level decay
                        s_cr[i] = P_i * s_sk[i];
                        s_cq[i] = P_i * s_sq[i];
                    }
                }
                if constexpr (NPB != 1) {
                    if (sh) {  // the group's node has depth 9 (uniform in the group)
                        // position 0 (node j0, the lowest index on the path):
                        //   M_i,j0 = (P_i / P_j0) q^_i . k^_j0 - sum_s M_i,n_s G_n_s,j0
                        // over positions s = 1 .. 8, lane p holding s = p + 1;
                        // G_m,j0 carries the decays of positions 1 .. s, an
                        // inclusive prefix product over the lanes
                        const int j0 = __builtin_ctzll(pm);
                        float pref = s_al[j];
                        {
                            const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                0, __builtin_bit_cast(int, pref), 0x111, 0xF, 0xF, false));  // row_shr:1
                            pref = p >= 1 ? pref * t1 : pref;
                            const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                0, __builtin_bit_cast(int, pref), 0x112, 0xF, 0xF, false));  // row_shr:2
                            pref = p >= 2 ? pref * t2 : pref;
                            const float t4 = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                0, __builtin_bit_cast(int, pref), 0x114, 0xF, 0xF, false));  // row_shr:4
                            pref = p >= 4 ? pref * t4 : pref;
                        }
                        const float sk_j0 = s_sk[j0];
                        float term = val * (s_be[j] * s_sk[j] * sk_j0 * s_gk[j * (j + 1) / 2 + j0] * pref);
                        term += dpp1<0xB1>(term);
                        term += dpp1<0x4E>(term);
                        term += dpp1<kDppRowHalfMirror>(term);
                        const float r0 = group8_lane<7>(pref, p);  // P_i / P_j0
                        const float v0 = r0 * s_sq[ii] * sk_j0 * s_gq[ii * (ii + 1) / 2 + j0] - term;
                        if (i < N && p == 0) {
                            s_gq[i * (i + 1) / 2 + j0] = v0;
                            const float P_i = r0 * s_al[j0];
                            s_cr[i] = P_i * s_sk[i];
                            s_cq[i] = P_i * s_sq[i];
                        }
                    }
                }
            }
            if constexpr (kLP2 > kLP) {
                // the nodes of depth kLP+2 .. kLP2 (a mask every wave forms
                // alike), one per group of kLP2 lanes, as above
                const int dl = s_dep[min(lane, N - 1)];
                const uint64_t deep = __ballot(lane < N && dl > kLP + 1 && dl <= kLP2);  // depth 9: above
                const int ndeep = __popcll(deep);
                const int p2 = tid & (kLP2 - 1);
                for (int q0 = 0; q0 < ndeep; q0 += kThreads / kLP2) {  // uniform
                    const int qi = q0 + tid / kLP2;
                    uint64_t dm = deep;
                    for (int c = 0; c < min(qi, ndeep - 1); ++c) dm &= dm - 1ull;
                    const int i = __builtin_ctzll(dm);  // the qi-th deep node
                    const int d = s_dep[i];
                    const bool act = qi < ndeep && p2 < d;
                    const uint64_t pm = s_anc[i] | (1ull << i);
                    const int j = path_node<kLP2>(pm, min(p2, d - 1));
                    const float sk_j = s_sk[j];
                    // as above: the nodes from the group's lanes, then all LDS
                    // reads, then products
                    // (in chunks of five positions, to bound the registers held)
                    float gco[kLP2];
                    float r = 1.0f;
    #pragma unroll
                    for (int s0 = 1; s0 < kLP2; s0 += 5) {
                        float al[5], bs[5], gk[5];
    #pragma unroll
                        for (int c = 0; c < 5; ++c) {
                            const int sp = s0 + c;
                            const int js = __float_as_int(row16_lane_at(__int_as_float(j), sp));
                            const int m = sp < d ? js : i;
                            al[c] = s_al[m];
                            bs[c] = s_be[m] * s_sk[m];
                            gk[c] = s_gk[m * (m + 1) / 2 + j];
                        }
    #pragma unroll
                        for (int c = 0; c < 5; ++c) {
                            const int sp = s0 + c;
                            const bool in = sp > p2 && sp < d;
                            r *= in ? al[c] : 1.0f;
                            gco[sp] = in ? bs[c] * sk_j * gk[c] * r : 0.0f;
                        }
                    }
                    float val = r * s_sq[i] * sk_j * s_gq[i * (i + 1) / 2 + j];
    #pragma unroll
                    for (int sp = kLP2 - 1; sp >= 1; --sp) {
                        const float ms = row16_lane_at(val, sp);  // lane sp of the 16-lane group
                        val = (sp < d && p2 < sp) ? fmaf(-ms, gco[sp], val) : val;
                    }
                    if (act) {
                        s_gq[i * (i + 1) / 2 + j] = val;
                        if (p2 == 0) {
                            const float P_i = r * s_al[j];
                            s_cr[i] = P_i * s_sk[i];
                            s_cq[i] = P_i * s_sq[i];
                        }
                    }
                }
            }
            // nodes deeper than kLP2: one thread per node, the same elimination in
            // place (M values so far read back from their hi + lo halves, or in
            // wide trees from the fp32 row that holds them)
            if (tid < N && s_dep[tid] > kLP2) {
                const int i = tid;
                const int d = s_dep[i];
                const uint8_t* path = s_cidx + i * N;
                const float sq_i = s_sq[i];
                uint16_t* mh = reinterpret_cast<uint16_t*>(s_mh + i * mstride);
                uint16_t* ml = reinterpret_cast<uint16_t*>(s_ml + i * mstride);
                float* mrow = s_gq + i * (i + 1) / 2;
                // wide trees: positions from the ancestor bits, deepest first
                const uint64_t pm = (NPB == 1) ? 0ull : (s_anc[i] | (1ull << i));
                uint64_t rem = pm;
                float wq = 1.0f;  // decays of the positions below p
                for (int pp = d - 1; pp >= 0; --pp) {
                    int jj;
                    uint64_t deeper = 0ull;  // wide trees: the positions below jj
                    if constexpr (NPB == 1) {
                        jj = path[pp];
                    } else {
                        jj = 63 - __builtin_clzll(rem);
                        rem &= ~(1ull << jj);
                        deeper = pm & ~(((1ull << jj) << 1) - 1ull);
                    }
                    const float sk_j = s_sk[jj];
                    float val = wq * sq_i * sk_j * mrow[jj];
                    float wval = pp == d - 1 ? 1.0f : 0.0f;  // W row i: the identity's
                    float wg = 1.0f;
                    for (int sp = pp + 1; sp < d; ++sp) {
                        int m;
                        if constexpr (NPB == 1) {
                            m = path[sp];
                        } else {
                            m = __builtin_ctzll(deeper | (1ull << 63));
                            deeper &= deeper - 1ull;
                        }
                        wg *= s_al[m];
                        const float gmj = s_be[m] * wg * s_sk[m] * sk_j * s_gk[m * (m + 1) / 2 + jj];
                        float msv;
                        if constexpr (NPB == 1)
                            msv = bf16_bits_to_f32(mh[m]) + bf16_bits_to_f32(ml[m]);
                        else
                            msv = mrow[m];
                        val = fmaf(-msv, gmj, val);
                        if constexpr (STOREU) {
                            const uint16_t* wh = reinterpret_cast<const uint16_t*>(lds + L.wh + i * mstride);
                            const uint16_t* wl = reinterpret_cast<const uint16_t*>(lds + L.wl + i * mstride);
                            wval = fmaf(-(bf16_bits_to_f32(wh[m]) + bf16_bits_to_f32(wl[m])), gmj, wval);
                        }
                    }
                    if constexpr (NPB == 1) {
                        const uint32_t hv = cvt_pk_bf16(val, 0.0f) & 0xffffu;
                        const float rest = val - __uint_as_float(hv << 16);
                        const uint32_t lv = cvt_pk_bf16(rest, 0.0f) & 0xffffu;
                        mh[jj] = static_cast<uint16_t>(hv);
                        ml[jj] = static_cast<uint16_t>(lv);
                        if constexpr (STOREU) {
                            const uint32_t hw = cvt_pk_bf16(wval, 0.0f) & 0xffffu;
                            const uint32_t lw2 = cvt_pk_bf16(wval - __uint_as_float(hw << 16), 0.0f) & 0xffffu;
                            reinterpret_cast<uint16_t*>(lds + L.wh + i * mstride)[jj] = static_cast<uint16_t>(hw);
                            reinterpret_cast<uint16_t*>(lds + L.wl + i * mstride)[jj] = static_cast<uint16_t>(lw2);
                        }
                    } else {
                        mrow[jj] = val;
                    }
                    wq *= s_al[jj];
                }
                s_cr[i] = wq * s_sk[i];
                s_cq[i] = wq * sq_i;
            }
        }
        __syncthreads();
    }

    // fused: replay the previous path into the state in registers, in this
    // kernel's layout (lane (r_own, hf) holds columns 16s + 4hf + e and
    // 16s + 8 + 4hf + e of row r_own; its partner hf ^ 1 is lane ^ 32), and
    // publish the state (LumoTree, Sec. IV-B):
    //   u = b_j (v_j - a_j S k^_j),  S <- a_j S + u k^_j^T,  k^_j = sc_j k_j
    if constexpr (COMMIT) {
        const bool do_commit = nc > 0;
        const int plen = nc;
        if (do_commit) {  // uniform
            const int jj = tid >> 5;
            const int chp = tid & 31;
          if constexpr (FUSED) {
            // the staged path overlays the Gram block, dead after the M solve
            const int cpl = nc * 32;  // 8-byte chunks of the path's k (and of v)
            float ss = sumsq_bf16x4(pk_val);
            ss = sum_half_wave(ss);
            if (tid < cpl) {
                *reinterpret_cast<uint2*>(s_kp + jj * kKQStride + chp * 8) = pk_val;
                *reinterpret_cast<uint2*>(s_vp + jj * kD + chp * 4) = pv_val;
                if (chp == 0) s_scp[jj] = norm ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
            }
            for (int it0 = kThreads; it0 < cpl; it0 += kThreads) {  // paths longer than 8 rows
                const int it = it0 + tid;
                const size_t rbp = static_cast<size_t>(b) * cp.Rp + prow_at(min(it >> 5, nc - 1));
                const uint2 kc = *reinterpret_cast<const uint2*>(
                    cp.kp + rbp * cp.rs_qk_p + static_cast<size_t>(g) * kD + chp * 4);
                const uint2 vc = *reinterpret_cast<const uint2*>(
                    cp.vp + rbp * cp.rs_v_p + static_cast<size_t>(h) * kD + chp * 4);
                float s2 = sumsq_bf16x4(kc);
                s2 = sum_half_wave(s2);
                if (it < cpl) {
                    *reinterpret_cast<uint2*>(s_kp + (it >> 5) * kKQStride + chp * 8) = kc;
                    *reinterpret_cast<uint2*>(s_vp + (it >> 5) * kD + chp * 4) = vc;
                    if (chp == 0) s_scp[it >> 5] = norm ? 1.0f / sqrtf(s2 + 1e-6f) : 1.0f;
                }
            }
            if (tid < nc) {
                if constexpr (RAW) {
                    s_alp[tid] = raw_gate_alpha(p_al, raw_gate_params(g_alog, g_dtb));
                    s_bep[tid] = raw_gate_beta(p_be);
                } else {
                    s_alp[tid] = p_al;
                    s_bep[tid] = p_be;
                }
            }
          } else {
            // the first segment's k/v rows (their conv ran with the tree's)
            *reinterpret_cast<uint2*>(s_kp + jj * kKQStride + chp * 8) = pk_val;
            *reinterpret_cast<uint2*>(s_vp + jj * kD + chp * 4) = pv_val;
            float ss = sumsq_bf16x4(pk_val);
            ss = sum_half_wave(ss);
            if (chp == 0) s_scp[jj] = norm ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
          }
            __syncthreads();
            // On the matrix cores, kMfmaPath path nodes at a time (segment
            // j0 .. j0 + n - 1 of the path, from the state the previous segment
            // left), with A = product of the segment's decays so far and
            // w_m = u_m times the decays after m:
            //   z_j = (S_(j-1) k^_j)_r = A sc_j (S k_j)_r + sum_(m<j) w_m (k^_m . k^_j)
            //   u_j = b_j (v_j,r - a_j z_j)
            //   S  <- A S + sum_m (w_m sc_m) k_m^T   (a rank-n update)
            // S k_j for every j of the segment is one contraction like (d); the
            // rank-n update is four 32-column contractions whose output layout
            // is this lane's own state layout.
            float* s_gp = s_scp + (FUSED ? cp.Lmax : kMfmaPath);  // [kMfmaPath][kMfmaPath] scaled segment Gram
            state_fix_loaded(sreg, l32);
            sfixed = true;
            for (int j0 = 0; j0 < plen; j0 += kMfmaPath) {
                const int n = min(plen - j0, kMfmaPath);
                const int kr0 = FUSED ? j0 : 0;  // staged row of the segment's first node
                if constexpr (LAYER) {
                    // a later segment's k/v rows: the conv of its path rows
                    if (LONGP && j0 > 0) {  // uniform: paths longer than one segment
                        uint2 kc = make_uint2(0u, 0u), vc = make_uint2(0u, 0u);
                        uint4* s_stg = reinterpret_cast<uint4*>(lds + L.stg);  // [H + 8][16]
                        uint32_t* s_sw = reinterpret_cast<uint32_t*>(lds + L.sw);
                        float* s_sb = reinterpret_cast<float*>(lds + L.sb);
#pragma unroll 1
                        for (int half = 0; half < 2; ++half) {
                            int colb = half == 0 ? ck0 : cv0;
                            asm volatile("" : "+s"(colb));  // keep these loads inside the loop
                            const int e = min(tid, (H + 8) * 16 - 1);
                            const uint4 xv4 = *reinterpret_cast<const uint4*>(
                                li.x_prev + (static_cast<size_t>(b) * li.Rp + prow_at(j0 + (e >> 4) - H)) * li.C +
                                colb + 8 * (e & 15));
                            const uint32_t wword = conv_weight_word<CW>(li.w, colb, tid);
                            float bword = 0.0f;
                            if (li.bias) bword = li.bias[colb + (tid & (kD - 1))];
                            s_stg[e] = xv4;
                            s_sw[tid] = wword;
                            s_sb[tid & (kD - 1)] = bword;
                            __syncthreads();
                            // two channels at a time: this runs with the whole state live
                            const char* st0 = reinterpret_cast<const char*>(s_stg) + jj * 256 + chp * 8;
                            uint2 o;
#pragma unroll 1
                            for (int pr = 0; pr < 2; ++pr) {
                                uint32_t tw[CW];
#pragma unroll
                                for (int t = 0; t <= H; ++t)
                                    tw[t] = *reinterpret_cast<const uint32_t*>(st0 + t * 256 + pr * 4);
                                const int c0 = 4 * chp + 2 * pr;
                                const float z0 = conv_channel<CW>(tw, 0, s_sw + c0 * kWP, li.bias != nullptr,
                                                                  s_sb[c0], li.act);
                                const float z1 = conv_channel<CW>(tw, 1, s_sw + (c0 + 1) * kWP,
                                                                  li.bias != nullptr, s_sb[c0 + 1], li.act);
                                const uint32_t wd = conv_pack_bf16x2(z0, z1);
                                if (pr == 0)
                                    o.x = wd;
                                else
                                    o.y = wd;
                            }
                            if (half == 0)
                                kc = o;
                            else
                                vc = o;
                            __syncthreads();
                        }
                        *reinterpret_cast<uint2*>(s_kp + jj * kKQStride + chp * 8) = kc;
                        *reinterpret_cast<uint2*>(s_vp + jj * kD + chp * 4) = vc;
                        float ss = sumsq_bf16x4(kc);
                        ss = sum_half_wave(ss);
                        if (chp == 0) s_scp[jj] = norm ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
                        __syncthreads();
                    }
                }
                auto path_row = [&](int row, int ks) -> bf16x8_t {  // zero past the segment
                    const bf16x8_t a = lds_operand(s_kp, kr0 + min(row, n - 1), ks, hf);
                    return row < n ? a : bf16x8_t{};
                };
                if (wave == 0 && n > 1) {
                    f32x16_t gacc = {};
#pragma unroll
                    for (int ks = 0; ks < 8; ++ks)
                        gacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(path_row(l32, ks), path_row(l32, ks),
                                                                       gacc, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < kMfmaPath / 2; ++e) {  // rows m < kMfmaPath sit in these e
                        const int m = 8 * (e >> 2) + 4 * hf + (e & 3);
                        if (l32 < n && m < n)
                            s_gp[m * kMfmaPath + l32] = gacc[e] * s_scp[kr0 + m] * s_scp[kr0 + l32];
                    }
                }
                f32x16_t pacc = {};
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    bf16x8_t shi, slo;
                    split_hi_lo(sreg[2 * ks], sreg[2 * ks + 1], shi, slo);
                    const bf16x8_t a = path_row(l32, ks);
                    pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, shi, pacc, 0, 0, 0);
                    pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, slo, pacc, 0, 0, 0);
                }
                __syncthreads();  // segment Gram in LDS
                // S k_j of this lane's row: this lane holds j in {4hf .. 4hf+3,
                // 8+4hf .. 8+4hf+3}, its partner (lane ^ 32) the rest
                float ctp[kMfmaPath];
#pragma unroll
                for (int e = 0; e < kMfmaPath / 2; ++e) {
                    // the two halves' values in every lane (a permlane32
                    // swap of the register with itself: the hf = 0 lane's
                    // value first, the hf = 1 lane's second)
                    const auto pr2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pacc[e]),
                                                                      __float_as_uint(pacc[e]), false, false);
                    const int jo = 8 * (e >> 2) + (e & 3);  // j held by the hf = 0 lane
                    ctp[jo] = __uint_as_float(pr2[0]);
                    ctp[jo + 4] = __uint_as_float(pr2[1]);
                }
                float w[kMfmaPath];
                float A = 1.0f;
#pragma unroll
                for (int j = 0; j < kMfmaPath; ++j) {
                    w[j] = 0.0f;
                    if (j < n) {  // uniform
                        const float a = s_alp[j0 + j];
                        float z = A * s_scp[kr0 + j] * ctp[j];
#pragma unroll
                        for (int m = 0; m < j; ++m) z = fmaf(w[m], s_gp[m * kMfmaPath + j], z);
                        const float u = s_bep[j0 + j] * (bf16_bits_to_f32(s_vp[(kr0 + j) * kD + r_own]) - a * z);
#pragma unroll
                        for (int m = 0; m < j; ++m) w[m] *= a;
                        w[j] = u;
                        A *= a;
                    }
                }
                // B operand of the update: slot e of lane half hf is segment row 8hf + e
                bf16x8_t uhi, ulo;
                {
                    float uu[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float w0 = w[e] * s_scp[kr0 + min(e, n - 1)];
                        float w1 = 0.0f;
                        if constexpr (kMfmaPath > 8)
                            w1 = w[min(8 + e, kMfmaPath - 1)] * s_scp[kr0 + min(8 + e, n - 1)];
                        uu[e] = hf ? w1 : w0;
                    }
                    split_hi_lo(make_float4(uu[0], uu[1], uu[2], uu[3]), make_float4(uu[4], uu[5], uu[6], uu[7]),
                                uhi, ulo);
                }
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    // A operand: k_m[32cb + l32] for segment row m = 8hf + e (zero past it)
                    uint32_t kw[4];
                    const uint16_t* col = reinterpret_cast<const uint16_t*>(s_kp) + (32 * cb + l32);
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const int m0 = 8 * hf + 2 * e2;
                        const uint32_t k0 = col[(kr0 + min(m0, n - 1)) * (kKQStride / 2)];
                        const uint32_t k1 = col[(kr0 + min(m0 + 1, n - 1)) * (kKQStride / 2)];
                        kw[e2] = (m0 < n ? k0 : 0u) | ((m0 + 1 < n ? k1 : 0u) << 16);
                    }
                    const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, make_uint4(kw[0], kw[1], kw[2], kw[3]));
                    f32x16_t sacc;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        sacc[4 * q4 + 0] = A * sreg[4 * cb + q4].x;
                        sacc[4 * q4 + 1] = A * sreg[4 * cb + q4].y;
                        sacc[4 * q4 + 2] = A * sreg[4 * cb + q4].z;
                        sacc[4 * q4 + 3] = A * sreg[4 * cb + q4].w;
                    }
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, uhi, sacc, 0, 0, 0);
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, ulo, sacc, 0, 0, 0);
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        sreg[4 * cb + q4] = make_float4(sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2],
                                                        sacc[4 * q4 + 3]);
                }
                __syncthreads();  // the segment Gram is rewritten by the next segment
            }
        }
        // one 32-row block: the state goes out after the contraction below,
        // its last use (a wave's vector memory counter covers stores, so a
        // later wait for a load would also wait for these 16 KB per wave);
        // two blocks: here, as the contraction's four accumulator blocks
        // leave no registers to keep the state any longer
        if (do_commit && (NPB != 1 || !vok)) state_store_lines(Sw, sreg, l32, hf);  // uniform
        if (!vok) return;
    }

    // (d) CT = [K;Q] S_pre^T on the matrix cores, state split into bf16 hi + lo
    //     (the first use of the state when nothing was replayed: the only wait
    //     for it)
    if (!sfixed) state_fix_loaded(sreg, l32);
    f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        bf16x8_t shi, slo;
        split_hi_lo(sreg[2 * s], sreg[2 * s + 1], shi, slo);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const bf16x8_t a = lds_operand(s_a, mb * 32 + l32, s, hf);
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, shi, acc[mb], 0, 0, 0);
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, slo, acc[mb], 0, 0, 0);
        }
    }
    if constexpr (COMMIT && NPB == 1) {  // the committed state, after its last use
        if (nc > 0) state_store_lines(Sw, sreg, l32, hf);  // uniform
    }
    if constexpr (NPB != 1) {
        // V rows, over the key/query block once every wave has read it
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kVItems; ++u) {
            const int it = tid + u * kThreads;
            const int node = it >> 5;
            if (node < N) *reinterpret_cast<uint2*>(s_v + node * kD + (it & 31) * 4) = v_val[u];
        }
        __syncthreads();
    }

    // this lane's indices again, from a fresh copy of the thread id: kept
    // live from the start of the kernel they would be spilled, and their
    // reload would wait for the state stores above (the vector memory
    // counter covers stores)
    int tid_o = tid;
    asm volatile("" : "+v"(tid_o));
    const int hfo = (tid_o >> 5) & 1;
    const int l32o = tid_o & 31;
    const int r_owno = wave * 32 + l32o;

    // (f) R = beta (v - P k^ S_pre) from the key blocks, as bf16 hi/lo MFMA
    //     operands (a key block's output layout is a permutation of the
    //     contraction index that the M operand reads in the same order)
    // (a lane's 16 entries of a block are four runs of four consecutive
    // nodes: the per-node scalars are read four at a time; entries past N
    // read padding or the next array and are masked)
    bf16x8_t rhi[2 * NPB], rlo[2 * NPB];
#pragma unroll
    for (int kb = 0; kb < NPB; ++kb) {
        float rv[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int i0 = kb * 32 + 8 * g4 + 4 * hfo;
            const float4 be4 = *reinterpret_cast<const float4*>(s_be + i0);
            const float4 cr4 = *reinterpret_cast<const float4*>(s_cr + i0);
            const float bev[4] = {be4.x, be4.y, be4.z, be4.w};
            const float crv[4] = {cr4.x, cr4.y, cr4.z, cr4.w};
#pragma unroll
            for (int e3 = 0; e3 < 4; ++e3) {
                const int e = 4 * g4 + e3;
                float val = 0.0f;
                if (i0 + e3 < N)
                    val = bev[e3] * (bf16_bits_to_f32(s_v[(i0 + e3) * kD + r_owno]) - crv[e3] * acc[kb][e]);
                rv[e] = val;
            }
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint32_t hh[4], ll[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float x0 = rv[8 * half + 2 * e2], x1 = rv[8 * half + 2 * e2 + 1];
                hh[e2] = cvt_pk_bf16(x0, x1);
                ll[e2] = cvt_pk_bf16(x0 - __uint_as_float(hh[e2] << 16),
                                     x1 - __uint_as_float(hh[e2] & 0xffff0000u));
            }
            rhi[2 * kb + half] = __builtin_bit_cast(bf16x8_t, make_uint4(hh[0], hh[1], hh[2], hh[3]));
            rlo[2 * kb + half] = __builtin_bit_cast(bf16x8_t, make_uint4(ll[0], ll[1], ll[2], ll[3]));
        }
    }
    // (g) O = P q^ S_pre + M R, accumulated onto the query blocks; write out
#pragma unroll
    for (int ob = 0; ob < NPB; ++ob) {
        f32x16_t o = acc[NPB + ob];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int i0 = ob * 32 + 8 * g4 + 4 * hfo;
            const float4 cq4 = *reinterpret_cast<const float4*>(s_cq + i0);
            const float cqv[4] = {cq4.x, cq4.y, cq4.z, cq4.w};
#pragma unroll
            for (int e3 = 0; e3 < 4; ++e3) o[4 * g4 + e3] *= (i0 + e3 < N) ? cqv[e3] : 0.0f;
        }
        // wide trees: row ob*32 + l32o of M from the triangle, zero off its root path
        const int mr = min(ob * 32 + l32o, N - 1);
        const uint64_t mpath = (ob * 32 + l32o < N) ? (s_anc[mr] | (1ull << mr)) : 0ull;
#pragma unroll
        for (int ks = 0; ks < 2 * NPB; ++ks) {
            if (ks > 2 * ob + 1) break;  // M is zero right of the diagonal block
            bf16x8_t mh, ml;
            if constexpr (NPB == 1) {
                mh = lds_operand_m(s_mh, mstride, ob * 32 + l32o, ks, hfo);
                ml = lds_operand_m(s_ml, mstride, ob * 32 + l32o, ks, hfo);
            } else {
                float mv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int col = 16 * ks + 4 * hfo + (e & 3) + 8 * (e >> 2);
                    // unclamped: past the row's end (col > mr) the read lands in
                    // the next rows or the ancestor masks that follow the
                    // triangle in LDS, and the mask drops it; consecutive
                    // columns stay consecutive reads
                    const float x = s_gq[mr * (mr + 1) / 2 + col];
                    mv[e] = ((mpath >> col) & 1ull) ? x : 0.0f;
                }
                split_hi_lo(make_float4(mv[0], mv[1], mv[2], mv[3]), make_float4(mv[4], mv[5], mv[6], mv[7]),
                            mh, ml);
            }
            o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mh, rhi[ks], o, 0, 0, 0);
            o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mh, rlo[ks], o, 0, 0, 0);
            o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ml, rhi[ks], o, 0, 0, 0);
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int i0 = ob * 32 + 8 * g4 + 4 * hfo;
            const int4 rw4 = *reinterpret_cast<const int4*>(s_rows + i0);
            const int rwv[4] = {rw4.x, rw4.y, rw4.z, rw4.w};
#pragma unroll
            for (int e3 = 0; e3 < 4; ++e3)
                if (i0 + e3 < N)
                    store_out(out, ((rowb + rwv[e3]) * Hv + h) * kD + r_owno, o[4 * g4 + e3], out_bf16 != 0);
        }
    }
    if constexpr (STOREU) {  // U = W R: row i of U is node i's delta correction
        f32x16_t uacc = {};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8_t wh = lds_operand_m(lds + L.wh, mstride, l32o, ks, hfo);
            const bf16x8_t wl = lds_operand_m(lds + L.wl, mstride, l32o, ks, hfo);
            uacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh, rhi[ks], uacc, 0, 0, 0);
            uacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh, rlo[ks], uacc, 0, 0, 0);
            uacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wl, rhi[ks], uacc, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = 8 * (e >> 2) + 4 * hfo + (e & 3);
            if (i < N) u_out[((rowb + s_rows[i]) * Hv + h) * kD + r_owno] = uacc[e];
        }
    }
}

// ===========================================================================
// Vector-ALU kernel: any d in {32, 64, 128}, bf16 or fp32 operands
// ===========================================================================
struct ValuLds {
    int K, Q, V, U, kk, kq, al, be, anc, rows, scale, total;
};

__host__ __device__ inline ValuLds valu_lds_layout(int N, int D) {
    ValuLds L;
    int off = 0;
    const int nd = align_up(N * D * 4, 16);
    L.K = off;
    off += nd;
    L.Q = off;
    off += nd;
    L.V = off;
    off += nd;
    L.U = off;
    off += nd;
    // Gram entries of ancestor pairs only (j <= i): row-major lower triangles
    L.kk = off;
    off += align_up(N * (N + 1) / 2 * 4, 16);
    L.kq = off;
    off += align_up(N * (N + 1) / 2 * 4, 16);
    L.al = off;
    off += align_up(N * 4, 16);
    L.be = off;
    off += align_up(N * 4, 16);
    L.anc = off;
    off += align_up(N * 8, 16);
    L.rows = off;
    off += align_up(N * 4, 16);
    L.scale = off;
    off += align_up(2 * N * 4, 16);
    L.total = off;
    return L;
}

size_t verify_valu_lds_bytes(int N, int D) { return static_cast<size_t>(valu_lds_layout(N, D).total); }

template <int D, typename T>
__global__ void __launch_bounds__(kThreads)
    verify_valu_kernel(int N, int R, int shared, const int32_t* __restrict__ node_row,
                       const uint64_t* __restrict__ anc_g, const int32_t* __restrict__ status,
                       const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                       int64_t rs_qk, int64_t rs_v, const float* __restrict__ alpha,
                       const float* __restrict__ beta, const float* __restrict__ pool, int P,
                       const int32_t* __restrict__ state_idx, void* __restrict__ out, int Hqk,
                       int Hv, int norm, int out_bf16, int32_t* __restrict__ err,
                       const float* __restrict__ gate_params, float* __restrict__ u_out) {
    constexpr int TPR = kThreads / D;  // lanes per value row
    constexpr int EPT = D / TPR;       // state elements per lane
    constexpr int NQ = EPT / 4;        // float4 chunks per lane
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const ValuLds L = valu_lds_layout(N, D);
    float* s_K = reinterpret_cast<float*>(lds + L.K);
    float* s_Q = reinterpret_cast<float*>(lds + L.Q);
    float* s_V = reinterpret_cast<float*>(lds + L.V);
    float* s_U = reinterpret_cast<float*>(lds + L.U);
    float* s_kk = reinterpret_cast<float*>(lds + L.kk);
    float* s_kq = reinterpret_cast<float*>(lds + L.kq);
    float* s_al = reinterpret_cast<float*>(lds + L.al);
    float* s_be = reinterpret_cast<float*>(lds + L.be);
    uint64_t* s_anc = reinterpret_cast<uint64_t*>(lds + L.anc);
    int32_t* s_rows = reinterpret_cast<int32_t*>(lds + L.rows);
    float* s_scale = reinterpret_cast<float*>(lds + L.scale);

    const uint32_t unit = xcd_local_order(blockIdx.x, gridDim.x);
    const int b = static_cast<int>(unit / Hv);
    const int h = static_cast<int>(unit % Hv);
    const int t = shared ? 0 : b;
    if (status[t] != 0) return;
    const int slot = state_idx[b];
    if (slot < 0 || slot >= P) {
        if (h == 0 && threadIdx.x == 0) atomicOr(err, GDN_EV_STATE);
        return;
    }
    const int g = static_cast<int>((static_cast<int64_t>(h) * Hqk) / Hv);
    const int tid = threadIdx.x;
    const int r = tid / TPR;
    const int part = tid % TPR;

    float4 sv[NQ];
    const float* Sb = pool + (static_cast<size_t>(slot) * Hv + h) * (D * D) +
                      static_cast<size_t>(r) * D;
#pragma unroll
    for (int c = 0; c < NQ; ++c)
        sv[c] = *reinterpret_cast<const float4*>(Sb + 4 * (part + TPR * c));

    const size_t tb = static_cast<size_t>(t) * N;
    if (tid < N) {
        const int row = node_row[tb + tid];
        s_rows[tid] = row;
        s_anc[tid] = anc_g[tb + tid];
        const size_t gi = (static_cast<size_t>(b) * R + row) * Hv + h;
        if (gate_params) {  // uniform: raw gate inputs
            s_al[tid] = raw_gate_alpha(alpha[gi], raw_gate_params(gate_params[h], gate_params[Hv + h]));
            s_be[tid] = raw_gate_beta(beta[gi]);
        } else {
            s_al[tid] = alpha[gi];
            s_be[tid] = beta[gi];
        }
    }
    __syncthreads();
    for (int e = tid; e < N * D; e += kThreads) {
        const int i = e / D, c = e % D;
        const size_t rqk = (static_cast<size_t>(b) * R + s_rows[i]) * rs_qk + static_cast<size_t>(g) * D + c;
        s_K[e] = load_elem(k + rqk);
        s_Q[e] = load_elem(q + rqk);
        s_V[e] = load_elem(v + (static_cast<size_t>(b) * R + s_rows[i]) * rs_v +
                           static_cast<size_t>(h) * D + c);
    }
    __syncthreads();
    if (norm) {
        if (tid < 2 * N) {
            const float* rowp = (tid < N) ? s_K + tid * D : s_Q + (tid - N) * D;
            float ss = 0.f;
            for (int c = 0; c < D; ++c) {
                const float xv = rowp[(c + tid) % D];
                ss = fmaf(xv, xv, ss);
            }
            s_scale[tid] = 1.0f / sqrtf(ss + 1e-6f);
        }
        __syncthreads();
        for (int e = tid; e < N * D; e += kThreads) {
            const int i = e / D;
            s_K[e] *= s_scale[i];
            s_Q[e] *= s_scale[N + i];
        }
        __syncthreads();
    }
    // Gram entries of ancestor pairs (and k_i . q_i)
    for (int e = tid; e < N * N; e += kThreads) {
        const int i = e / N, j = e % N;
        if (j > i) continue;
        const bool is_anc = ((s_anc[i] >> j) & 1ull) != 0ull;
        if (!is_anc && j != i) continue;
        const float* ki = s_K + i * D;
        const float* qi = s_Q + i * D;
        const float* kj = s_K + j * D;
        float dkk = 0.f, dkq = 0.f;
        for (int c0 = 0; c0 < D; ++c0) {
            const int c = (c0 + e) % D;
            dkk = fmaf(ki[c], kj[c], dkk);
            dkq = fmaf(qi[c], kj[c], dkq);
        }
        s_kk[i * (i + 1) / 2 + j] = dkk;
        s_kq[i * (i + 1) / 2 + j] = dkq;
    }
    __syncthreads();

    for (int i = 0; i < N; ++i) {
        const float* ki = s_K + i * D;
        const float* qi = s_Q + i * D;
        float yk = 0.f, yq = 0.f;
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const int col = 4 * (part + TPR * c);
            const float4 kv = *reinterpret_cast<const float4*>(ki + col);
            const float4 qv = *reinterpret_cast<const float4*>(qi + col);
            yk = fmaf(sv[c].x, kv.x, yk);
            yk = fmaf(sv[c].y, kv.y, yk);
            yk = fmaf(sv[c].z, kv.z, yk);
            yk = fmaf(sv[c].w, kv.w, yk);
            yq = fmaf(sv[c].x, qv.x, yq);
            yq = fmaf(sv[c].y, qv.y, yq);
            yq = fmaf(sv[c].z, qv.z, yq);
            yq = fmaf(sv[c].w, qv.w, yq);
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) {
            yk += __shfl_xor(yk, off, 64);
            yq += __shfl_xor(yq, off, 64);
        }
        uint64_t am = s_anc[i];
        while (am) {
            const int j = __builtin_ctzll(am);
            am &= am - 1ull;
            const float uj = s_U[j * D + r];
            yk = fmaf(s_al[j], yk, uj * s_kk[i * (i + 1) / 2 + j]);
            yq = fmaf(s_al[j], yq, uj * s_kq[i * (i + 1) / 2 + j]);
        }
        const float u = s_be[i] * (s_V[i * D + r] - s_al[i] * yk);
        const float o = fmaf(s_al[i], yq, u * s_kq[i * (i + 1) / 2 + i]);
        if (part == 0) {
            s_U[i * D + r] = u;
            const size_t oi = ((static_cast<size_t>(b) * R + s_rows[i]) * Hv + h) * D + r;
            store_out(out, oi, o, out_bf16 != 0);
            if (u_out) u_out[oi] = u;  // stored-U mode
        }
    }
}

// ===========================================================================
// dispatch
// ===========================================================================
namespace {
constexpr size_t kMaxLds = 160 * 1024;

template <typename K>
hipError_t set_lds(K kernel, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

template <int NPB, int MODE, int CW, bool RAW>
hipError_t launch_mfma_raw(const gdn_tree_desc& d, const VerifyArgs& a, float* pool, int norm,
                           int obf, size_t lds, const CommitPrev& cp, hipStream_t s,
                           const LayerIn& li) {
    auto kfn = verify_mfma_kernel<NPB, MODE, CW, RAW>;
    hipError_t e = set_lds(kfn, lds);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(d.B) * static_cast<unsigned>(a.Hv));
    hipLaunchKernelGGL(kfn, grid, dim3(kThreads), lds, s, d.N, d.R, d.shared, d.node_row, d.anc,
                       d.depth, d.status, static_cast<const uint16_t*>(a.q),
                       static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                       a.rs_qk, a.rs_v, a.alpha, a.beta, pool, a.P, a.state_idx, a.out, a.Hqk,
                       a.Hv, norm, obf, a.err, a.gate_params, cp, li, a.u);
    return hipGetLastError();
}

// raw gate inputs select their own instantiation, so the plain kernels keep
// their register allocation
template <int NPB, int MODE, int CW = 0>
hipError_t launch_mfma_t(const gdn_tree_desc& d, const VerifyArgs& a, float* pool, int norm,
                         int obf, size_t lds, const CommitPrev& cp, hipStream_t s,
                         const LayerIn& li = LayerIn{}) {
    if (a.flags & GDN_F_RAW_GATES)
        return launch_mfma_raw<NPB, MODE, CW, true>(d, a, pool, norm, obf, lds, cp, s, li);
    return launch_mfma_raw<NPB, MODE, CW, false>(d, a, pool, norm, obf, lds, cp, s, li);
}

template <int D, typename T>
hipError_t launch_valu_t(const gdn_tree_desc& d, const VerifyArgs& a, int norm, int obf,
                         size_t lds, hipStream_t s) {
    auto kfn = verify_valu_kernel<D, T>;
    hipError_t e = set_lds(kfn, lds);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(d.B) * static_cast<unsigned>(a.Hv));
    hipLaunchKernelGGL(kfn, grid, dim3(kThreads), lds, s, d.N, d.R, d.shared, d.node_row, d.anc,
                       d.status, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.rs_qk, a.rs_v, a.alpha, a.beta, a.pool, a.P,
                       a.state_idx, a.out, a.Hqk, a.Hv, norm, obf, a.err,
                       (a.flags & GDN_F_RAW_GATES) ? a.gate_params : nullptr, a.u);
    return hipGetLastError();
}
}  // namespace

bool verify_uses_mfma(const gdn_tree_desc& d, const VerifyArgs& a) {
    const bool aligned = (a.rs_qk % 4 == 0) && (a.rs_v % 4 == 0) &&
                         (reinterpret_cast<uintptr_t>(a.q) % 8 == 0) &&
                         (reinterpret_cast<uintptr_t>(a.k) % 8 == 0) &&
                         (reinterpret_cast<uintptr_t>(a.v) % 8 == 0);
    return a.dtype == GDN_DT_BF16 && a.D == kD && !(a.flags & GDN_F_VALU) && aligned && d.N >= 1;
}

// Whether launch_verify has a kernel for these arguments (checked by the
// fused call before it launches anything).
bool verify_supported(const gdn_tree_desc& d, const VerifyArgs& a) {
    const int NPB = (d.N + 31) / 32;
    if (verify_uses_mfma(d, a) && (a.u == nullptr || NPB == 1)) {
        return NPB <= 2 && static_cast<size_t>(mfma_lds_layout(d.N, NPB, 0, a.u != nullptr).total) <= kMaxLds;
    }
    return (a.D == 32 || a.D == 64 || a.D == 128) && verify_valu_lds_bytes(d.N, a.D) <= kMaxLds;
}

hipError_t launch_verify(const gdn_tree_desc& d, const VerifyArgs& a, hipStream_t s) {
    const int norm = (a.flags & GDN_F_NORM_QK) ? 1 : 0;
    const int obf = (a.flags & GDN_F_OUT_BF16) ? 1 : 0;
    const int NPB = (d.N + 31) / 32;
    // the stored-U mode runs on the matrix cores for N <= 32, on the vector
    // ALU otherwise
    if (verify_uses_mfma(d, a) && (a.u == nullptr || NPB == 1)) {
        const size_t lds = static_cast<size_t>(mfma_lds_layout(d.N, NPB, 0, a.u != nullptr).total);
        if (lds > kMaxLds) return hipErrorNotSupported;
        const CommitPrev none{};
        // the non-fused kernel only reads the state
        float* pool = const_cast<float*>(a.pool);
        if (a.u != nullptr) return launch_mfma_t<1, kModeVerifyU>(d, a, pool, norm, obf, lds, none, s);
        switch (NPB) {
            case 1: return launch_mfma_t<1, kModeVerify>(d, a, pool, norm, obf, lds, none, s);
            case 2: return launch_mfma_t<2, kModeVerify>(d, a, pool, norm, obf, lds, none, s);
            default: return hipErrorNotSupported;
        }
    }
    const size_t lds = verify_valu_lds_bytes(d.N, a.D);
    if (lds > kMaxLds) return hipErrorNotSupported;
    const bool bf = a.dtype == GDN_DT_BF16;
    switch (a.D) {
        case 32:
            return bf ? launch_valu_t<32, uint16_t>(d, a, norm, obf, lds, s)
                      : launch_valu_t<32, float>(d, a, norm, obf, lds, s);
        case 64:
            return bf ? launch_valu_t<64, uint16_t>(d, a, norm, obf, lds, s)
                      : launch_valu_t<64, float>(d, a, norm, obf, lds, s);
        case 128:
            return bf ? launch_valu_t<128, uint16_t>(d, a, norm, obf, lds, s)
                      : launch_valu_t<128, float>(d, a, norm, obf, lds, s);
        default:
            return hipErrorNotSupported;
    }
}

hipError_t launch_commit_verify(const gdn_tree_desc& d, const CommitVerifyArgs& a, hipStream_t s) {
    const VerifyArgs& va = a.verify;
    const gdn_tree_desc& dp = *a.prev;
    const bool prev_aligned = (a.rs_qk_prev % 4 == 0) && (a.rs_v_prev % 4 == 0) &&
                              (reinterpret_cast<uintptr_t>(a.k_prev) % 8 == 0) &&
                              (reinterpret_cast<uintptr_t>(a.v_prev) % 8 == 0);
    if (verify_uses_mfma(d, va) && prev_aligned) {
        const int NPB = (d.N + 31) / 32;
        const size_t lds = static_cast<size_t>(mfma_lds_layout(d.N, NPB, a.Lmax).total);
        if (lds <= kMaxLds) {
            CommitPrev cp{};
            cp.Rp = dp.R;
            cp.Lmax = a.Lmax;
            cp.path_rows = a.path_rows;
            cp.path_n = a.path_n;
            cp.kp = static_cast<const uint16_t*>(a.k_prev);
            cp.vp = static_cast<const uint16_t*>(a.v_prev);
            cp.rs_qk_p = a.rs_qk_prev;
            cp.rs_v_p = a.rs_v_prev;
            cp.alpha_p = a.alpha_prev;
            cp.beta_p = a.beta_prev;
            const int norm = (va.flags & GDN_F_NORM_QK) ? 1 : 0;
            const int obf = (va.flags & GDN_F_OUT_BF16) ? 1 : 0;
            switch (NPB) {
                case 1: return launch_mfma_t<1, kModeCommitVerify>(d, va, a.pool, norm, obf, lds, cp, s);
                case 2: return launch_mfma_t<2, kModeCommitVerify>(d, va, a.pool, norm, obf, lds, cp, s);
                default: break;
            }
        }
    }
    // other shapes: the commit, then the verify (the same result in two
    // launches).  Nothing is launched unless both have a kernel: the commit
    // writes the pool in place, so a verify refused after it would leave
    // the call half done.
    if (!verify_supported(d, va)) return hipErrorNotSupported;
    CommitArgs ca{a.path_rows, a.path_n, a.Lmax, a.k_prev, a.v_prev, a.rs_qk_prev, a.rs_v_prev,
                  a.alpha_prev, a.beta_prev, a.pool, va.P, va.state_idx, nullptr, nullptr, 0,
                  va.Hqk, va.Hv, va.D, va.dtype, va.flags & (GDN_F_NORM_QK | GDN_F_RAW_GATES), va.err, 1};
    ca.gate_params = va.gate_params;
    hipError_t e = launch_commit(dp, ca, s);
    if (e != hipSuccess) return e;
    return launch_verify(d, va, s);
}

hipError_t launch_layer_step(const gdn_tree_desc& d, const LayerArgs& a, hipStream_t s) {
    if (d.N > 32 || d.W < 1 || d.W > 4) return hipErrorNotSupported;
    const size_t lds = static_cast<size_t>(layer_lds_layout(d.N, d.W - 1, a.Lmax).total);
    if (lds > kMaxLds) return hipErrorNotSupported;
    LayerIn li{};
    li.C = 2 * a.Hqk * kD + a.Hv * kD;
    li.act = a.act;
    li.Rp = a.prev->R;
    li.Lmax = a.Lmax;
    li.x = a.x;
    li.w = a.w;
    li.bias = a.bias;
    li.hist_in = a.hist_in;
    li.hist_out = a.hist_out;
    li.y = a.y;
    li.x_prev = a.x_prev;
    li.alpha_p = a.alpha_prev;
    li.beta_p = a.beta_prev;
    li.path_rows = a.path_rows;
    li.path_n = a.path_n;
    li.parent = d.parent;
    const VerifyArgs va{nullptr, nullptr, nullptr, 0, 0, a.alpha, a.beta, a.pool, a.P, a.state_idx,
                        a.out, a.Hqk, a.Hv, kD, GDN_DT_BF16, a.flags, a.err, a.gate_params};
    const int norm = (a.flags & GDN_F_NORM_QK) ? 1 : 0;
    const int obf = (a.flags & GDN_F_OUT_BF16) ? 1 : 0;
    const CommitPrev none{};
    const bool longp = a.Lmax > kMfmaPath;
#define GDN_LAYER_CASE(WW)                                                                          \
    case WW:                                                                                        \
        return longp ? launch_mfma_t<1, kModeLayerLong, WW>(d, va, a.pool, norm, obf, lds, none, s, li) \
                     : launch_mfma_t<1, kModeLayer, WW>(d, va, a.pool, norm, obf, lds, none, s, li);
    switch (d.W) {
        GDN_LAYER_CASE(1)
        GDN_LAYER_CASE(2)
        GDN_LAYER_CASE(3)
        GDN_LAYER_CASE(4)
        default:
            return hipErrorNotSupported;
    }
#undef GDN_LAYER_CASE
}

}  // namespace gdn

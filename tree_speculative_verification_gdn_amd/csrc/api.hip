// C ABI of libgdntree (declared in include/gdn_tree.h): synchronous argument
// validation, then one asynchronous launch on the caller's stream.  No
// allocation, no host synchronisation, no global mutable state.
#include "gdn_internal.h"

namespace {

int32_t map_launch(hipError_t e) {
    if (e == hipSuccess) return GDN_OK;
    if (e == hipErrorNotSupported) return GDN_ERR_UNSUPPORTED;
    return GDN_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t check_desc(const gdn_tree_desc* d) {
    if (d == nullptr) return GDN_ERR_ARG;
    if (d->B < 1 || d->R < 1 || d->W < 1 || (d->shared != 0 && d->shared != 1)) return GDN_ERR_ARG;
    if (d->N < 1 || d->N > GDN_MAX_NODES || d->W > GDN_MAX_CONV_W) return GDN_ERR_UNSUPPORTED;
    if (d->R < d->N) return GDN_ERR_ARG;
    if (!d->parent || !d->node_row || !d->depth || !d->anc || !d->status) return GDN_ERR_ARG;
    if (d->W > 1 && !d->conv_src) return GDN_ERR_ARG;
    if (!aligned(d->anc, 8)) return GDN_ERR_ARG;
    return GDN_OK;
}

int32_t check_heads(int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, int32_t dtype) {
    if (Hqk < 1 || Hv < 1 || Hv % Hqk != 0) return GDN_ERR_ARG;
    if (dtype != GDN_DT_BF16 && dtype != GDN_DT_F32) return GDN_ERR_ARG;
    if (dk != dv) return GDN_ERR_UNSUPPORTED;
    if (dk != 32 && dk != 64 && dk != 128) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

}  // namespace

extern "C" {

// GDN_F_RAW_GATES needs the per-head gate parameters (4-byte aligned floats)
static int32_t check_gates(int32_t flags, const float* gate_params) {
    if ((flags & GDN_F_RAW_GATES) == 0) return GDN_OK;
    return (gate_params != nullptr && aligned(gate_params, 4)) ? GDN_OK : GDN_ERR_ARG;
}

int32_t gdn_abi_version(void) { return 8; }

const char* gdn_status_string(int32_t status) {
    switch (status) {
        case GDN_OK:
            return "ok";
        case GDN_ERR_ARG:
            return "invalid argument";
        case GDN_ERR_UNSUPPORTED:
            return "unsupported size";
        case GDN_ERR_HIP:
            return "kernel launch failed";
        default:
            return "unknown status";
    }
}

int32_t gdn_tree_desc_build(const gdn_tree_desc* d, int32_t* err, void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    if (!err) return GDN_ERR_ARG;
    return map_launch(gdn::launch_desc_build(*d, err, static_cast<hipStream_t>(stream)));
}

int32_t conv_ancestry_gather(const gdn_tree_desc* d, const void* x, const void* hist, int32_t P,
                             const int32_t* state_idx, const void* w, const float* bias, void* y,
                             int32_t C, int32_t act, int32_t* err, void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    if (!x || !state_idx || !w || !y || !err || P < 1) return GDN_ERR_ARG;
    if (d->W > 1 && !hist) return GDN_ERR_ARG;
    if (C < 4 || C % 4 != 0) return GDN_ERR_UNSUPPORTED;
    if (act != GDN_ACT_NONE && act != GDN_ACT_SILU) return GDN_ERR_ARG;
    if (!aligned(x, 8) || !aligned(y, 8) || (hist && !aligned(hist, 8))) return GDN_ERR_ARG;
    return map_launch(gdn::launch_conv(*d, static_cast<const uint16_t*>(x),
                                       static_cast<const uint16_t*>(hist), P, state_idx,
                                       static_cast<const uint16_t*>(w), bias,
                                       static_cast<uint16_t*>(y), C, act, err,
                                       static_cast<hipStream_t>(stream)));
}

int32_t gdn_tree_verify(const gdn_tree_desc* d, const void* q, const void* k, const void* v,
                        int64_t row_stride_qk, int64_t row_stride_v, const float* alpha,
                        const float* beta, const float* state_pool, int32_t P,
                        const int32_t* state_idx, void* out, int32_t Hqk, int32_t Hv, int32_t dk,
                        int32_t dv, int32_t dtype, int32_t flags, const float* gate_params,
                        int32_t* err, void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    st = check_heads(Hqk, Hv, dk, dv, dtype);
    if (st != GDN_OK) return st;
    if (!q || !k || !v || !alpha || !beta || !state_pool || !state_idx || !out || !err || P < 1)
        return GDN_ERR_ARG;
    if ((flags & ~(GDN_F_NORM_QK | GDN_F_OUT_BF16 | GDN_F_VALU | GDN_F_RAW_GATES)) != 0) return GDN_ERR_ARG;
    if (check_gates(flags, gate_params) != GDN_OK) return GDN_ERR_ARG;
    if (row_stride_qk < static_cast<int64_t>(Hqk) * dk || row_stride_v < static_cast<int64_t>(Hv) * dv)
        return GDN_ERR_ARG;
    if (!aligned(state_pool, 16)) return GDN_ERR_ARG;
    gdn::VerifyArgs a{q, k, v, row_stride_qk, row_stride_v, alpha, beta, state_pool, P,
                      state_idx, out, Hqk, Hv, dk, dtype, flags, err, gate_params};
    return map_launch(gdn::launch_verify(*d, a, static_cast<hipStream_t>(stream)));
}

int32_t gdn_tree_verify_store_u(const gdn_tree_desc* d, const void* q, const void* k, const void* v,
                                int64_t row_stride_qk, int64_t row_stride_v, const float* alpha,
                                const float* beta, const float* state_pool, int32_t P,
                                const int32_t* state_idx, void* out, float* u, float* dump, int32_t Hqk,
                                int32_t Hv, int32_t dk, int32_t dv, int32_t dtype, int32_t flags,
                                const float* gate_params, int32_t* err, void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    st = check_heads(Hqk, Hv, dk, dv, dtype);
    if (st != GDN_OK) return st;
    if (!q || !k || !v || !alpha || !beta || !state_pool || !state_idx || !out || !u || !err || P < 1)
        return GDN_ERR_ARG;
    if ((flags & ~(GDN_F_NORM_QK | GDN_F_OUT_BF16 | GDN_F_VALU | GDN_F_RAW_GATES | GDN_F_DUMP_STATES)) != 0)
        return GDN_ERR_ARG;
    if (check_gates(flags, gate_params) != GDN_OK) return GDN_ERR_ARG;
    if (row_stride_qk < static_cast<int64_t>(Hqk) * dk || row_stride_v < static_cast<int64_t>(Hv) * dv)
        return GDN_ERR_ARG;
    if (!aligned(state_pool, 16) || !aligned(u, 4)) return GDN_ERR_ARG;
    const bool want_dump = (flags & GDN_F_DUMP_STATES) != 0;
    if (want_dump) {
        // the dump rebuilds each node's state on the factored commit's kernel
        if (dump == nullptr) return GDN_ERR_ARG;
        if (dk != 128 || dtype != GDN_DT_BF16) return GDN_ERR_UNSUPPORTED;
        if (row_stride_qk % 4 != 0 || !aligned(k, 8) || !aligned(u, 16) || !aligned(dump, 16))
            return GDN_ERR_ARG;
    }
    const int vflags = flags & ~GDN_F_DUMP_STATES;
    gdn::VerifyArgs a{q, k, v, row_stride_qk, row_stride_v, alpha, beta, state_pool, P,
                      state_idx, out, Hqk, Hv, dk, dtype, vflags, err, gate_params, u};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = map_launch(gdn::launch_verify(*d, a, s));
    if (st != GDN_OK || !want_dump) return st;
    gdn::FactoredCommitArgs fa{nullptr, nullptr, 0, k, row_stride_qk, u, alpha, const_cast<float*>(state_pool),
                               P, state_idx, Hqk, Hv, vflags & (GDN_F_NORM_QK | GDN_F_RAW_GATES), err,
                               gate_params};
    return map_launch(gdn::launch_dump_states(*d, fa, dump, s));
}

int32_t gdn_tree_commit_factored(const gdn_tree_desc* d, const int32_t* path, const int32_t* path_len,
                                 int32_t Lmax, const void* k, int64_t row_stride_qk, const float* u,
                                 const float* alpha, float* state_pool, int32_t P, const int32_t* state_idx,
                                 int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, int32_t flags,
                                 const float* gate_params, int32_t* err, void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    st = check_heads(Hqk, Hv, dk, dv, GDN_DT_BF16);
    if (st != GDN_OK) return st;
    if (dk != 128) return GDN_ERR_UNSUPPORTED;
    if (!path || !path_len || !k || !u || !alpha || !state_pool || !state_idx || !err || P < 1)
        return GDN_ERR_ARG;
    if (Lmax < 1 || Lmax > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    if ((flags & ~(GDN_F_NORM_QK | GDN_F_RAW_GATES)) != 0) return GDN_ERR_ARG;
    if (check_gates(flags, gate_params) != GDN_OK) return GDN_ERR_ARG;
    if (row_stride_qk < static_cast<int64_t>(Hqk) * dk || row_stride_qk % 4 != 0) return GDN_ERR_ARG;
    if (!aligned(k, 8) || !aligned(u, 16) || !aligned(state_pool, 16)) return GDN_ERR_ARG;
    gdn::FactoredCommitArgs a{path, path_len, Lmax, k, row_stride_qk, u, alpha, state_pool, P, state_idx,
                              Hqk, Hv, flags, err, gate_params};
    return map_launch(gdn::launch_commit_factored(*d, a, static_cast<hipStream_t>(stream)));
}

int32_t gdn_tree_commit(const gdn_tree_desc* d, const int32_t* path, const int32_t* path_len,
                        int32_t Lmax, const void* k, const void* v, int64_t row_stride_qk,
                        int64_t row_stride_v, const float* alpha, const float* beta,
                        float* state_pool, int32_t P, const int32_t* state_idx, const void* x,
                        void* hist, int32_t C, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                        int32_t dtype, int32_t flags, const float* gate_params, int32_t* err,
                        void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    st = check_heads(Hqk, Hv, dk, dv, dtype);
    if (st != GDN_OK) return st;
    if (!path || !path_len || !k || !v || !alpha || !beta || !state_pool || !state_idx || !err ||
        P < 1)
        return GDN_ERR_ARG;
    if (check_gates(flags, gate_params) != GDN_OK) return GDN_ERR_ARG;
    if (Lmax < 1 || Lmax > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    // the conv history exists only for W > 1; with W == 1 x and hist are ignored
    if (d->W == 1) {
        x = nullptr;
        hist = nullptr;
    }
    if ((x == nullptr) != (hist == nullptr)) return GDN_ERR_ARG;
    if (x != nullptr && C < 1) return GDN_ERR_ARG;
    if (x != nullptr && (!aligned(x, 2) || !aligned(hist, 2))) return GDN_ERR_ARG;
    if ((flags & ~(GDN_F_NORM_QK | GDN_F_RAW_GATES)) != 0) return GDN_ERR_ARG;
    if (row_stride_qk < static_cast<int64_t>(Hqk) * dk || row_stride_v < static_cast<int64_t>(Hv) * dv)
        return GDN_ERR_ARG;
    if (!aligned(state_pool, 16)) return GDN_ERR_ARG;
    gdn::CommitArgs a{path, path_len, Lmax, k, v, row_stride_qk, row_stride_v, alpha, beta,
                      state_pool, P, state_idx, static_cast<const uint16_t*>(x),
                      static_cast<uint16_t*>(hist), x ? C : 0, Hqk, Hv, dk, dtype, flags, err, 0};
    a.gate_params = gate_params;
    return map_launch(gdn::launch_commit(*d, a, static_cast<hipStream_t>(stream)));
}

int32_t gdn_tree_commit_layers(const gdn_tree_desc* d, const int32_t* path, const int32_t* path_len,
                               int32_t Lmax, int32_t layers, const void* k, const void* v,
                               int64_t row_stride_qk, int64_t row_stride_v, int64_t layer_stride_qk,
                               int64_t layer_stride_v, const float* alpha, const float* beta,
                               int64_t layer_stride_gate, float* state_pool,
                               int64_t layer_stride_pool, int32_t P, const int32_t* state_idx,
                               int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, int32_t dtype,
                               int32_t flags, const float* gate_params, int32_t* err, void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    st = check_heads(Hqk, Hv, dk, dv, dtype);
    if (st != GDN_OK) return st;
    if (!path || !path_len || !k || !v || !alpha || !beta || !state_pool || !state_idx || !err ||
        P < 1 || layers < 1)
        return GDN_ERR_ARG;
    if (Lmax < 1 || Lmax > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    if ((flags & ~(GDN_F_NORM_QK | GDN_F_RAW_GATES)) != 0) return GDN_ERR_ARG;
    if (check_gates(flags, gate_params) != GDN_OK) return GDN_ERR_ARG;
    if (row_stride_qk < static_cast<int64_t>(Hqk) * dk || row_stride_v < static_cast<int64_t>(Hv) * dv)
        return GDN_ERR_ARG;
    // a layer's buffers must not overlap the next layer's
    const int64_t rows = static_cast<int64_t>(d->B) * d->R;
    if (layers > 1 && (layer_stride_qk < rows * row_stride_qk || layer_stride_v < rows * row_stride_v ||
                       layer_stride_gate < rows * Hv ||
                       layer_stride_pool < static_cast<int64_t>(P) * Hv * dk * dv))
        return GDN_ERR_ARG;
    if (static_cast<int64_t>(d->B) * Hv * layers > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;
    if (!aligned(state_pool, 16) || (layer_stride_pool % 4) != 0) return GDN_ERR_ARG;
    gdn::CommitArgs a{path, path_len, Lmax, k, v, row_stride_qk, row_stride_v, alpha, beta,
                      state_pool, P, state_idx, nullptr, nullptr, 0, Hqk, Hv, dk, dtype, flags, err, 0};
    a.layers = layers;
    a.ls_qk = layer_stride_qk;
    a.ls_v = layer_stride_v;
    a.ls_gate = layer_stride_gate;
    a.ls_pool = layer_stride_pool;
    a.gate_params = gate_params;
    return map_launch(gdn::launch_commit(*d, a, static_cast<hipStream_t>(stream)));
}

int32_t conv_ancestry_gather_publish(const gdn_tree_desc* d, const void* x, void* hist, int32_t P,
                                     const int32_t* state_idx, const void* w, const float* bias,
                                     void* y, int32_t C, int32_t act, const gdn_tree_desc* d_prev,
                                     const int32_t* path_rows, const int32_t* path_n, int32_t Lmax,
                                     const void* x_prev, int32_t* err, void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    st = check_desc(d_prev);
    if (st != GDN_OK) return st;
    if (d_prev->B != d->B || d_prev->W != d->W) return GDN_ERR_ARG;
    if (!x || !state_idx || !w || !y || !err || !path_rows || !path_n || !x_prev || P < 1)
        return GDN_ERR_ARG;
    if (d->W > 1 && !hist) return GDN_ERR_ARG;
    if (Lmax < 1 || Lmax > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    if (C < 4 || C % 4 != 0) return GDN_ERR_UNSUPPORTED;
    if (act != GDN_ACT_NONE && act != GDN_ACT_SILU) return GDN_ERR_ARG;
    if (!aligned(x, 8) || !aligned(y, 8) || !aligned(x_prev, 8) || (hist && !aligned(hist, 8)))
        return GDN_ERR_ARG;
    const gdn::ConvPublish pub{d_prev, path_rows, path_n, Lmax, static_cast<const uint16_t*>(x_prev)};
    return map_launch(gdn::launch_conv(*d, static_cast<const uint16_t*>(x),
                                       static_cast<const uint16_t*>(hist), P, state_idx,
                                       static_cast<const uint16_t*>(w), bias,
                                       static_cast<uint16_t*>(y), C, act, err,
                                       static_cast<hipStream_t>(stream), &pub));
}

int32_t gdn_tree_commit_verify(const gdn_tree_desc* d, const void* q, const void* k, const void* v,
                               int64_t row_stride_qk, int64_t row_stride_v, const float* alpha,
                               const float* beta, float* state_pool, int32_t P,
                               const int32_t* state_idx, void* out, const gdn_tree_desc* d_prev,
                               const int32_t* path_rows, const int32_t* path_n, int32_t Lmax,
                               const void* k_prev, const void* v_prev, int64_t row_stride_qk_prev,
                               int64_t row_stride_v_prev, const float* alpha_prev,
                               const float* beta_prev, int32_t Hqk, int32_t Hv, int32_t dk,
                               int32_t dv, int32_t dtype, int32_t flags, const float* gate_params,
                               int32_t* err, void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    st = check_desc(d_prev);
    if (st != GDN_OK) return st;
    if (d_prev->B != d->B) return GDN_ERR_ARG;
    st = check_heads(Hqk, Hv, dk, dv, dtype);
    if (st != GDN_OK) return st;
    if (!q || !k || !v || !alpha || !beta || !state_pool || !state_idx || !out || !err || P < 1 ||
        !path_rows || !path_n || !k_prev || !v_prev || !alpha_prev || !beta_prev)
        return GDN_ERR_ARG;
    if (Lmax < 1 || Lmax > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    if ((flags & ~(GDN_F_NORM_QK | GDN_F_OUT_BF16 | GDN_F_VALU | GDN_F_RAW_GATES)) != 0) return GDN_ERR_ARG;
    if (check_gates(flags, gate_params) != GDN_OK) return GDN_ERR_ARG;
    if (row_stride_qk < static_cast<int64_t>(Hqk) * dk || row_stride_v < static_cast<int64_t>(Hv) * dv ||
        row_stride_qk_prev < static_cast<int64_t>(Hqk) * dk ||
        row_stride_v_prev < static_cast<int64_t>(Hv) * dv)
        return GDN_ERR_ARG;
    if (!aligned(state_pool, 16)) return GDN_ERR_ARG;
    gdn::CommitVerifyArgs a{};
    a.verify = gdn::VerifyArgs{q, k, v, row_stride_qk, row_stride_v, alpha, beta, state_pool, P,
                               state_idx, out, Hqk, Hv, dk, dtype, flags, err, gate_params};
    a.pool = state_pool;
    a.prev = d_prev;
    a.path_rows = path_rows;
    a.path_n = path_n;
    a.Lmax = Lmax;
    a.k_prev = k_prev;
    a.v_prev = v_prev;
    a.rs_qk_prev = row_stride_qk_prev;
    a.rs_v_prev = row_stride_v_prev;
    a.alpha_prev = alpha_prev;
    a.beta_prev = beta_prev;
    return map_launch(gdn::launch_commit_verify(*d, a, static_cast<hipStream_t>(stream)));
}

int32_t gdn_path_resolve(const gdn_tree_desc* d_prev, const int32_t* path, const int32_t* path_len,
                         int32_t Lmax, const int32_t* state_idx, int32_t P, int32_t* path_rows,
                         int32_t* path_n, int32_t* err, void* stream) {
    int32_t st = check_desc(d_prev);
    if (st != GDN_OK) return st;
    if (!path || !path_len || !state_idx || !path_rows || !path_n || !err || P < 1) return GDN_ERR_ARG;
    if (Lmax < 1 || Lmax > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    return map_launch(gdn::launch_path_resolve(*d_prev, d_prev->B, path, path_len, Lmax, state_idx, P,
                                               path_rows, path_n, err,
                                               static_cast<hipStream_t>(stream)));
}

int32_t gdn_step_prepare(const gdn_tree_desc* d, const gdn_tree_desc* d_prev, const int32_t* path,
                         const int32_t* path_len, int32_t Lmax, const int32_t* state_idx, int32_t P,
                         int32_t* path_rows, int32_t* path_n, int32_t* err, void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    st = check_desc(d_prev);
    if (st != GDN_OK) return st;
    if (d_prev->B != d->B) return GDN_ERR_ARG;
    if (!path || !path_len || !state_idx || !path_rows || !path_n || !err || P < 1) return GDN_ERR_ARG;
    if (Lmax < 1 || Lmax > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    return map_launch(gdn::launch_step_prepare(*d, *d_prev, path, path_len, Lmax, state_idx, P, path_rows,
                                               path_n, err, static_cast<hipStream_t>(stream)));
}

int32_t gdn_layer_step(const gdn_tree_desc* d, const void* x, const void* w, const float* bias,
                       int32_t act, const void* hist_in, void* hist_out, const float* alpha,
                       const float* beta, float* state_pool, int32_t P, const int32_t* state_idx,
                       void* out, void* y, const gdn_tree_desc* d_prev, const void* x_prev,
                       const float* alpha_prev, const float* beta_prev, const int32_t* path_rows,
                       const int32_t* path_n, int32_t Lmax, int32_t Hqk, int32_t Hv, int32_t dk,
                       int32_t dv, int32_t flags, const float* gate_params, int32_t* err,
                       void* stream) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    st = check_desc(d_prev);
    if (st != GDN_OK) return st;
    if (d_prev->B != d->B) return GDN_ERR_ARG;
    st = check_heads(Hqk, Hv, dk, dv, GDN_DT_BF16);
    if (st != GDN_OK) return st;
    if (dk != 128 || d->N > 32) return GDN_ERR_UNSUPPORTED;
    if (!x || !w || !alpha || !beta || !state_pool || !state_idx || !out || !x_prev ||
        !alpha_prev || !beta_prev || !path_rows || !path_n || !err || P < 1)
        return GDN_ERR_ARG;
    if (Lmax < 1 || Lmax > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    if (act != GDN_ACT_NONE && act != GDN_ACT_SILU) return GDN_ERR_ARG;
    if ((flags & ~(GDN_F_NORM_QK | GDN_F_OUT_BF16 | GDN_F_RAW_GATES)) != 0) return GDN_ERR_ARG;
    if (check_gates(flags, gate_params) != GDN_OK) return GDN_ERR_ARG;
    const int64_t C = 2 * static_cast<int64_t>(Hqk) * dk + static_cast<int64_t>(Hv) * dv;
    if (d->W > 1) {
        if (!hist_in || !hist_out) return GDN_ERR_ARG;
        // the two history buffers must not overlap: both heads of a qk group
        // read the old q/k history that one of them writes
        const uintptr_t bytes = static_cast<uintptr_t>(P) * static_cast<uintptr_t>(d->W - 1) *
                                static_cast<uintptr_t>(C) * 2u;
        const uintptr_t i0 = reinterpret_cast<uintptr_t>(hist_in), o0 = reinterpret_cast<uintptr_t>(hist_out);
        if (i0 < o0 + bytes && o0 < i0 + bytes) return GDN_ERR_ARG;
        if (!aligned(hist_in, 16) || !aligned(hist_out, 16)) return GDN_ERR_ARG;
    } else {
        hist_in = nullptr;
        hist_out = nullptr;
    }
    if (!aligned(x, 16) || !aligned(x_prev, 16) || !aligned(state_pool, 16) || (y && !aligned(y, 8)))
        return GDN_ERR_ARG;
    gdn::LayerArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.w = static_cast<const uint16_t*>(w);
    a.bias = bias;
    a.act = act;
    a.hist_in = static_cast<const uint16_t*>(hist_in);
    a.hist_out = static_cast<uint16_t*>(hist_out);
    a.alpha = alpha;
    a.beta = beta;
    a.pool = state_pool;
    a.P = P;
    a.state_idx = state_idx;
    a.out = out;
    a.y = static_cast<uint16_t*>(y);
    a.prev = d_prev;
    a.x_prev = static_cast<const uint16_t*>(x_prev);
    a.alpha_prev = alpha_prev;
    a.beta_prev = beta_prev;
    a.path_rows = path_rows;
    a.path_n = path_n;
    a.Lmax = Lmax;
    a.Hqk = Hqk;
    a.Hv = Hv;
    a.flags = flags;
    a.err = err;
    a.gate_params = gate_params;
    return map_launch(gdn::launch_layer_step(*d, a, static_cast<hipStream_t>(stream)));
}

size_t gdn_tree_attention_workspace_bytes(int32_t B, int32_t N, int32_t Hq, int32_t D,
                                          int32_t splits) {
    if (B < 1 || N < 1 || Hq < 1 || D < 1 || splits < 1) return 0;
    return gdn::tree_attention_workspace_bytes(B, N, Hq, D, splits);
}

namespace {

// Argument checks shared by the two attention entry points (all but the
// workspace).
int32_t check_attention(const gdn_tree_desc* d, const void* q, const void* k_cache, const void* v_cache,
                        int32_t S, const int32_t* ctx_len, const void* out, int32_t splits, int32_t Hq,
                        int32_t Hkv, int32_t D, float scale, int32_t flags, const int32_t* err) {
    int32_t st = check_desc(d);
    if (st != GDN_OK) return st;
    if (!q || !k_cache || !v_cache || !ctx_len || !out || !err) return GDN_ERR_ARG;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return GDN_ERR_ARG;
    if (D != 128 && D != 256) return GDN_ERR_UNSUPPORTED;
    if (d->R > 64) return GDN_ERR_UNSUPPORTED;
    if (splits < 1 || splits > 1024) return GDN_ERR_UNSUPPORTED;
    if (S < d->R) return GDN_ERR_ARG;
    // the kernels work with scale * log2(e) (the exponent base 2): it must
    // be a finite positive number
    const float scale2 = scale * 1.4426950408889634f;
    if (!(scale > 0.0f) || !(scale2 <= 3.40282347e38f) || (flags & ~GDN_F_OUT_BF16) != 0) return GDN_ERR_ARG;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(out, (flags & GDN_F_OUT_BF16) ? 2 : 4))
        return GDN_ERR_ARG;
    const int64_t units = static_cast<int64_t>(d->B) * Hkv * (splits + 1) * Hq;
    if (units > 0x7fffffffLL || static_cast<int64_t>(d->B) * S * Hkv * D > (int64_t{1} << 40))
        return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

}  // namespace

int32_t gdn_tree_attention(const gdn_tree_desc* d, const void* q, const void* k_cache,
                           const void* v_cache, int32_t S, const int32_t* ctx_len, void* out,
                           void* workspace, size_t workspace_bytes, int32_t splits, int32_t Hq,
                           int32_t Hkv, int32_t D, float scale, int32_t flags, int32_t* err,
                           void* stream) {
    const int32_t st = check_attention(d, q, k_cache, v_cache, S, ctx_len, out, splits, Hq, Hkv, D, scale,
                                       flags, err);
    if (st != GDN_OK) return st;
    if (!workspace || !aligned(workspace, 16)) return GDN_ERR_ARG;
    if (workspace_bytes < gdn::tree_attention_workspace_bytes(d->B, d->N, Hq, D, splits)) return GDN_ERR_ARG;
    gdn::TreeAttnArgs a{q, k_cache, v_cache, S, ctx_len, out, workspace, splits, Hq, Hkv, D,
                        scale, flags, err};
    return map_launch(gdn::launch_tree_attention(*d, a, static_cast<hipStream_t>(stream)));
}

int32_t gdn_tree_attention_noalloc(const gdn_tree_desc* d, const void* q, const void* k_cache,
                                   const void* v_cache, int32_t S, const int32_t* ctx_len, void* out,
                                   int32_t splits, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                                   int32_t flags, int32_t* err, void* stream) {
    const int32_t st = check_attention(d, q, k_cache, v_cache, S, ctx_len, out, splits, Hq, Hkv, D, scale,
                                       flags, err);
    if (st != GDN_OK) return st;
    if (gdn::tree_attention_workspace_bytes(d->B, d->N, Hq, D, splits) > gdn::kNoAllocScratchBytes)
        return GDN_ERR_UNSUPPORTED;
    hipError_t e = hipSuccess;
    void* ws = gdn::noalloc_scratch(&e);
    if (ws == nullptr) return GDN_ERR_HIP;
    gdn::TreeAttnArgs a{q, k_cache, v_cache, S, ctx_len, out, ws, splits, Hq, Hkv, D,
                        scale, flags, err};
    return map_launch(gdn::launch_tree_attention(*d, a, static_cast<hipStream_t>(stream)));
}

int32_t gdn_tree_kv_publish(const gdn_tree_desc* d_prev, const int32_t* path_rows,
                            const int32_t* path_n, int32_t Lmax, void* k_cache, void* v_cache,
                            int32_t S, const int32_t* ctx_len, int32_t Hkv, int32_t D,
                            int32_t* err, void* stream) {
    int32_t st = check_desc(d_prev);
    if (st != GDN_OK) return st;
    if (!path_rows || !path_n || !k_cache || !v_cache || !ctx_len || !err || Hkv < 1) return GDN_ERR_ARG;
    if (Lmax < 1 || Lmax > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    if (D != 128 && D != 256) return GDN_ERR_UNSUPPORTED;
    if (S < d_prev->R) return GDN_ERR_ARG;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return GDN_ERR_ARG;
    return map_launch(gdn::launch_kv_publish(*d_prev, path_rows, path_n, Lmax, k_cache, v_cache, S, ctx_len,
                                             Hkv, D, err, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

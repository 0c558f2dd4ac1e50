// Internal helpers shared by the gfx950 kernels of libgdntree (not part of
// the ABI).  Host launchers declared here are defined in the kernel files
// and called by api.hip after argument validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_tree.h"

namespace gdn {

constexpr int kMaxNodes = GDN_MAX_NODES;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) {
    return bf16_bits_to_f32(*p);
}
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) {
    return *p;
}

// Gates from raw inputs (GDN_F_RAW_GATES; LumoTree, Sec. IV-B: the verifier
// takes raw gate inputs and evaluates the gates itself).  Per value head the
// parameters A_log and dt_bias, per node the raw inputs a and b:
//   alpha = exp(-exp(A_log) * softplus(a + dt_bias)),  beta = 1 / (1 + exp(-b)),
// softplus(x) = max(x, 0) + log(1 + exp(-|x|)) (no overflow for any x), on
// the hardware exp2 / log2 / reciprocal (about 1 ulp each; the log of
// 1 + e loses e below 2^-24, an absolute error under 6e-8 in softplus).
struct RawGate {
    float A2;   // exp(A_log) * log2(e)
    float dtb;  // dt_bias
};
__device__ __forceinline__ RawGate raw_gate_params(float A_log, float dt_bias) {
    return RawGate{__builtin_amdgcn_exp2f(A_log * 1.4426950408889634f) * 1.4426950408889634f, dt_bias};
}
__device__ __forceinline__ float raw_gate_alpha(float a, RawGate g) {
    const float x = a + g.dtb;
    const float e = __builtin_amdgcn_exp2f(fabsf(x) * -1.4426950408889634f);  // exp(-|x|) in (0, 1]
    const float sp = fmaxf(x, 0.0f) + __builtin_amdgcn_logf(1.0f + e) * 0.6931471805599453f;
    return __builtin_amdgcn_exp2f(-g.A2 * sp);
}
__device__ __forceinline__ float raw_gate_beta(float b) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(b * -1.4426950408889634f));
}

// Make a wave-uniform value scalar (all lanes hold the same value).
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}

// Map a hardware workgroup id to a logical work item so that logical
// neighbours run on the same XCD (gfx950 deals consecutive workgroup ids out
// round-robin over its 8 XCDs, each with its own L2).  Identity when the grid
// is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_local_order(uint32_t hw_id, uint32_t n) {
    if ((n & 7u) != 0u) return hw_id;
    return (hw_id & 7u) * (n >> 3) + (hw_id >> 3);
}

// ---- launchers (host) -------------------------------------------------
hipError_t launch_desc_build(const gdn_tree_desc& d, int32_t* err, hipStream_t s);
// Conv-history publication of the previous step's accepted path, done by the
// conv of the next step before its taps read the history.
struct ConvPublish {
    const gdn_tree_desc* prev;  // previous step's tree (its R)
    const int32_t* path_rows;   // [B][Lmax] physical rows of the accepted path (resolved)
    const int32_t* path_n;      // [B] nodes to publish; -1 / 0: none
    int Lmax;
    const uint16_t* x_prev;     // previous step's conv input [B][prev R][C]
};
hipError_t launch_conv(const gdn_tree_desc& d, const uint16_t* x, const uint16_t* hist, int P,
                       const int32_t* state_idx, const uint16_t* w, const float* bias,
                       uint16_t* y, int C, int act, int32_t* err, hipStream_t s,
                       const ConvPublish* pub = nullptr);

struct VerifyArgs {
    const void* q;
    const void* k;
    const void* v;
    int64_t rs_qk, rs_v;
    const float* alpha;
    const float* beta;
    const float* pool;
    int P;
    const int32_t* state_idx;
    void* out;
    int Hqk, Hv, D;
    int dtype, flags;
    int32_t* err;
    const float* gate_params = nullptr;  // [2][Hv] A_log, dt_bias with GDN_F_RAW_GATES
    float* u = nullptr;  // stored-U mode: every node's delta correction [B][R][Hv][D], or none
};
// Returns hipErrorNotSupported (without launching) when no kernel covers the
// shape; the API maps that to GDN_ERR_UNSUPPORTED.
hipError_t launch_verify(const gdn_tree_desc& d, const VerifyArgs& a, hipStream_t s);
bool verify_uses_mfma(const gdn_tree_desc& d, const VerifyArgs& a);
size_t verify_valu_lds_bytes(int N, int D);

struct CommitArgs {
    const int32_t* path;      // logical ids [B][Lmax], or physical rows when resolved
    const int32_t* path_len;  // [B], or the resolved node counts (-1: nothing written)
    int Lmax;
    const void* k;
    const void* v;
    int64_t rs_qk, rs_v;
    const float* alpha;
    const float* beta;
    float* pool;
    int P;
    const int32_t* state_idx;
    const uint16_t* x;
    uint16_t* hist;
    int C;
    int Hqk, Hv, D;
    int dtype, flags;
    int32_t* err;
    int resolved;  // 1: path / path_len come from the path resolution (no validation here)
    // several layers in one launch: layer l's k, v, gates and pool at these
    // element strides from the first layer's (layers = 1: one layer)
    int layers = 1;
    int64_t ls_qk = 0, ls_v = 0, ls_gate = 0, ls_pool = 0;
    const float* gate_params = nullptr;  // [layers][2][Hv] with GDN_F_RAW_GATES
};
hipError_t launch_commit(const gdn_tree_desc& d, const CommitArgs& a, hipStream_t s);
size_t commit_lds_bytes(int Lmax, int D, int dtype);

// Commit from the delta corrections a stored-U verify wrote (bf16 k, d = 128).
struct FactoredCommitArgs {
    const int32_t* path;      // logical ids [B][Lmax]
    const int32_t* path_len;  // [B]
    int Lmax;
    const void* k;            // bf16 k rows, row stride rs_qk
    int64_t rs_qk;
    const float* u;           // [B][R][Hv][128]
    const float* alpha;       // [B][R][Hv] (raw inputs with GDN_F_RAW_GATES)
    float* pool;
    int P;
    const int32_t* state_idx;
    int Hqk, Hv, flags;
    int32_t* err;
    const float* gate_params;
};
hipError_t launch_commit_factored(const gdn_tree_desc& d, const FactoredCommitArgs& a, hipStream_t s);
// Every node's state S_i rebuilt from its root path's stored corrections into
// dump [B][N][Hv][128][128] (a.path, a.path_len and a.Lmax unused; the pool
// only read).
hipError_t launch_dump_states(const gdn_tree_desc& d, const FactoredCommitArgs& a, float* dump, hipStream_t s);
size_t commit_factored_lds_bytes(int Lmax);

// Commit of the previous step's accepted path followed by the verify of the
// next tree, from the committed state (one launch on the matrix-core path).
struct CommitVerifyArgs {
    VerifyArgs verify;          // the next tree; verify.pool is the pool below
    float* pool;                // written: the committed states
    const gdn_tree_desc* prev;  // the previous step's tree
    const int32_t* path_rows;   // resolved accepted path: rows [B][Lmax] and node counts [B]
    const int32_t* path_n;
    int Lmax;
    const void* k_prev;
    const void* v_prev;
    int64_t rs_qk_prev, rs_v_prev;
    const float* alpha_prev;
    const float* beta_prev;
};
hipError_t launch_commit_verify(const gdn_tree_desc& d, const CommitVerifyArgs& a, hipStream_t s);

// One launch per layer and step: commit of the previous path (its k/v
// recomputed from its conv input), conv-history publication, conv and verify
// of the new tree (bf16, d = 128, N <= 32).
struct LayerArgs {
    const uint16_t* x;
    const uint16_t* w;
    const float* bias;
    int act;
    const uint16_t* hist_in;
    uint16_t* hist_out;
    const float* alpha;
    const float* beta;
    float* pool;
    int P;
    const int32_t* state_idx;
    void* out;
    uint16_t* y;
    const gdn_tree_desc* prev;
    const uint16_t* x_prev;
    const float* alpha_prev;
    const float* beta_prev;
    const int32_t* path_rows;
    const int32_t* path_n;
    int Lmax;
    int Hqk, Hv, flags;
    int32_t* err;
    const float* gate_params = nullptr;  // [2][Hv] with GDN_F_RAW_GATES
};
hipError_t launch_layer_step(const gdn_tree_desc& d, const LayerArgs& a, hipStream_t s);

// Tree attention over the committed prefix and the candidate suffix, and
// the accepted path's KV publication (bf16, D = 128 or 256).
struct TreeAttnArgs {
    const void* q;
    const void* k;
    const void* v;
    int S;
    const int32_t* ctx_len;
    void* out;
    void* workspace;
    int splits, Hq, Hkv, D;
    float scale;
    int flags;
    int32_t* err;
};
size_t tree_attention_workspace_bytes(int B, int N, int Hq, int D, int splits);
// The no-alloc attention's scratch: its size, and its device address on the
// current device (nullptr and *status set if that address cannot be had).
constexpr size_t kNoAllocScratchBytes = GDN_ATTN_NOALLOC_SCRATCH_BYTES;
void* noalloc_scratch(hipError_t* status);
hipError_t launch_tree_attention(const gdn_tree_desc& d, const TreeAttnArgs& a, hipStream_t s);
hipError_t launch_kv_publish(const gdn_tree_desc& prev, const int32_t* path_rows, const int32_t* path_n,
                             int Lmax, void* k, void* v, int S, const int32_t* ctx_len, int Hkv, int D,
                             int32_t* err, hipStream_t s);

// Validation of the previous step's path and its physical rows, once per step.
hipError_t launch_path_resolve(const gdn_tree_desc& prev, int B, const int32_t* path,
                               const int32_t* path_len, int Lmax, const int32_t* state_idx, int P,
                               int32_t* path_rows, int32_t* path_n, int32_t* err, hipStream_t s);
// The new tree's descriptor and the previous path's resolution in one launch.
hipError_t launch_step_prepare(const gdn_tree_desc& d, const gdn_tree_desc& prev, const int32_t* path,
                               const int32_t* path_len, int Lmax, const int32_t* state_idx, int P,
                               int32_t* path_rows, int32_t* path_n, int32_t* err, hipStream_t s);

}  // namespace gdn

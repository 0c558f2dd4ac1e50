// Ancestry-aware tree attention over a physically placed candidate suffix,
// and the accepted path's KV publication (LumoTree, Sec. III-C and V-B: one
// slot map places the candidates' keys/values after the committed prefix and
// names the mask's key columns; grouped query heads share staged KV tiles;
// the context is split into partitions for parallel work at small batch).
//
// Attention: one 512-thread workgroup per (request, kv head, group of query
// heads, key partition).  Partitions 0..splits-1 cover the committed prefix
// in equal ranges; partition `splits` covers the R candidate slots under the
// ancestry mask.  A workgroup holds up to 128 query rows (the N nodes of four
// heads, or of two heads when N > 32), 16 per wave, and walks its keys in
// tiles of 32: the tile's keys and values go to LDS row-major (the values
// are read back with the transposing LDS read), S^T = K Q^T runs on
// v_mfma_f32_16x16x32_bf16 (a wave's lane holds one query
// row's scores for four keys per 16-key block), an online softmax keeps each
// row's reference maximum and sum in the log2 domain (the reference moves
// only when a score exceeds it by more than 2^8), and O += P V on the same
// instruction with P split into bf16 hi + lo (P's rounding error stays near
// 2^-17 of a weight).  Each partition writes its unnormalised O, reference
// maximum and sum; a second kernel merges the partitions (the standard
// split-softmax merge) into the output.
//
// Layouts: q [B][N][Hq][D] logical node rows; k, v [B][S][Hkv][D] bf16, the
// prefix at positions [0, ctx_len[b]), candidate physical row r at
// ctx_len[b] + r.
#include <mutex>

#include "gdn_internal.h"

namespace gdn {

namespace {
typedef __bf16 abf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 abf16x2_t __attribute__((ext_vector_type(2)));
typedef float af32x2_t __attribute__((ext_vector_type(2)));
typedef float af32x4_t __attribute__((ext_vector_type(4)));

constexpr int kAThreads = 512;  // 8 waves of 16 query rows
constexpr int kRows = 128;      // query rows per workgroup
constexpr int kTileKeys = 32;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.f;  // log2 units a score may exceed the reference maximum by
// word 3 of a buffer descriptor for raw 32-bit-element loads (a nonzero
// data format; no swizzle, no index stride)
constexpr int kRawBufferFlags = 0x00020000;

struct AttnArgs {
    int B, N, R, S, Hq, Hkv, splits, HPW, pairs, chunk, shared;
    const int32_t* node_row;
    const uint64_t* anc;
    const int32_t* status;
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* ctx_len;
    float scale2;   // softmax scale * log2(e)
    int kv_cap;     // positions one buffer descriptor may span (its byte range fits 32 bits)
    float* ws_o;    // [splits + 1][B][Hq][N][D] unnormalised partial outputs
    float* ws_ml;   // [splits + 1][B][Hq][N][2] running maximum (log2 domain) and sum
    void* out;      // [B][N][Hq][D]
    int out_bf16;
    int32_t* err;
};

template <int D>
struct AttnLds {
    // bf16 per staged key, value or query row: D + 16 (a 32-byte pad) puts
    // the rows of a key block 8 banks apart, which keeps the 16-byte fragment
    // reads of keys and queries free of bank conflicts (a 16-byte pad cost 10%
    // of the launch in them), and the transposing 8-byte reads of values too
    // (the eight keys one read of 32 lanes touches fall on distinct 32-byte
    // bank groups)
    static constexpr int kKStride = D + 16;
    static constexpr int Q = 0;  // the workgroup's query rows
    static constexpr int kKBytes = kTileKeys * kKStride * 2;
    static constexpr int kVBytes = kKBytes;
    static constexpr int K = Q + kRows * kKStride * 2;  // two buffers: K, V, K, V
    static constexpr int V = K + kKBytes;
    static constexpr int kBuf = kKBytes + kVBytes;      // offset of the second buffer
    static constexpr int ROW = K + 2 * kBuf;            // int32 node_row[64]
    static constexpr int VIS = ROW + 64 * 4;           // uint64 visible rows [64]
    static constexpr int total = VIS + 64 * 8;
};

// two finite fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16_pack_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((af32x2_t){a, b}, abf16x2_t));
}

typedef short ai16x4_t __attribute__((ext_vector_type(4)));
typedef short ai16x8_t __attribute__((ext_vector_type(8)));

// the transposing 8-byte LDS read (ds_read_b64_tr_b16) at an LDS address p
// (8-byte aligned; each lane addresses four 16-bit values): within each row
// of 16 lanes, lane 4 a + c receives value c of the pieces that lanes a,
// 4 + a, 8 + a and 12 + a address, one from each, in that order
__device__ __forceinline__ ai16x4_t lds_read_tr16x4(const uint16_t* p) {
    typedef __attribute__((address_space(3))) ai16x4_t lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);  // generic -> LDS address
}

// x combined with the x of lane l ^ 16 (rows of 16 lanes swapped in pairs)
// or of lane l ^ 32 (the two halves of the wave swapped) on the vector ALU:
// a permlane swap of a register with itself leaves the value of the pair's
// lower row (half) in the first result and the upper one's in the second,
// in every lane of the pair.  Sums are exact in either order; the maximum
// is the same value up to the sign of a zero.
__device__ __forceinline__ float pair16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Is request b skipped (malformed tree or context out of range)?  Uniform.
__device__ __forceinline__ bool attn_skip(const AttnArgs& a, int b, int& L) {
    const int t = a.shared ? 0 : b;
    L = a.ctx_len[b];
    return a.status[t] != 0 || L < 0 || L + a.R > a.S;
}
}  // namespace

template <int D>
__global__ void __launch_bounds__(kAThreads) tree_attn_kernel(const AttnArgs a) {
    using Lds = AttnLds<D>;
    constexpr int kDS = D / 32;   // 32-wide d steps of S^T
    constexpr int kDB = D / 16;   // 16-wide d blocks of O
    extern __shared__ __attribute__((aligned(16))) char lds[];
    uint16_t* s_q = reinterpret_cast<uint16_t*>(lds + Lds::Q);
    uint16_t* s_k = reinterpret_cast<uint16_t*>(lds + Lds::K);
    uint16_t* s_v = reinterpret_cast<uint16_t*>(lds + Lds::V);
    int32_t* s_row = reinterpret_cast<int32_t*>(lds + Lds::ROW);
    uint64_t* s_vis = reinterpret_cast<uint64_t*>(lds + Lds::VIS);

    // workgroup -> (request, kv head, key partition, head group); the groups
    // of one kv head and partition are neighbours (same XCD: shared KV tiles)
    const int nsp = a.splits + 1;
    const uint32_t unit = xcd_local_order(blockIdx.x, gridDim.x);
    const int p = static_cast<int>(unit % a.pairs);
    const int sp = static_cast<int>((unit / a.pairs) % nsp);
    const int g = static_cast<int>((unit / (a.pairs * nsp)) % a.Hkv);
    const int b = static_cast<int>(unit / (a.pairs * nsp * a.Hkv));
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lg = l >> 4, l16 = l & 15;
    const int G = a.Hq / a.Hkv;
    const int h0 = g * G + p * a.HPW;
    const int nh = min(a.HPW, G - p * a.HPW);
    const int NPH = kRows / a.HPW;  // rows per head in the workgroup (N <= NPH)
    const int N = a.N;
    const int t = a.shared ? 0 : b;

    int L;
    if (attn_skip(a, b, L)) {
        if (a.status[t] == 0 && tid == 0 && sp == 0 && p == 0 && g == 0) atomicOr(a.err, GDN_EV_CTX);
        return;
    }
    const bool tree = sp == a.splits;
    const int lo = tree ? L : min(sp * a.chunk, L);
    const int hi = tree ? L + a.R : min((sp + 1) * a.chunk, L);

    // the query rows (row r = head r / NPH, node r % NPH; rows past the
    // nodes or heads are zeros) staged in LDS once
#pragma unroll
    for (int u = 0; u < kRows * D / 8 / kAThreads; ++u) {
        const int c = tid + u * kAThreads;
        const int r = c / (D / 8), d8 = (c % (D / 8)) * 8;
        const int ir = r % NPH, hr = r / NPH;
        const uint16_t* qp = a.q + ((static_cast<size_t>(b) * N + min(ir, N - 1)) * a.Hq + h0 + min(hr, nh - 1)) * D;
        uint4 qc = *reinterpret_cast<const uint4*>(qp + d8);
        if (!(ir < N && hr < nh)) qc = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(s_q + r * Lds::kKStride + d8) = qc;
    }
    // this lane's query row (S^T column): row r = 16 w + l16
    const int rq = 16 * w + l16;
    const int iq = rq % NPH, hq = rq / NPH;
    const bool vq = iq < N && hq < nh;
    // the candidates visible to each node: its own row and its ancestors';
    // the rows some node occupies (the others may hold anything)
    uint64_t my_vis = 0ull, used = ~0ull;
    if (tree) {  // uniform
        if (tid < 64) s_row[tid] = a.node_row[static_cast<size_t>(t) * N + min(tid, N - 1)];
        __syncthreads();
        used = 0ull;
        for (int i = 0; i < N; ++i) used |= 1ull << s_row[i];
        if (tid < N) {
            uint64_t anc = a.anc[static_cast<size_t>(t) * N + tid];
            uint64_t vis = 1ull << s_row[tid];
            while (anc) {
                const int j = __builtin_ctzll(anc);
                anc &= anc - 1;
                vis |= 1ull << s_row[j];
            }
            s_vis[tid] = vis;
        }
        __syncthreads();
        my_vis = s_vis[min(iq, N - 1)];
    }

    const uint64_t vis_or = tree ? my_vis : ~0ull;  // context keys: every row sees them
    af32x4_t o[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) o[db] = af32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    // kept with m_run: the exponent offset (0 while nothing was seen) and the
    // threshold a raw (unscaled) score must pass to move the reference
    float m_use = 0.f, thr_raw = -INFINITY;

    const int ntiles = (hi - lo + kTileKeys - 1) / kTileKeys;
    constexpr int kChunks = kTileKeys * D / 8;  // 16-byte chunks of a K (or V) tile
    constexpr int kU = kChunks / kAThreads;     // chunks of each per lane
    // The cache is read with buffer loads: one descriptor per tile (scalar
    // registers) covers request b's kv head g from the tile's first position
    // to the end of the request's cache, so a lane's offset inside the tile
    // is fixed for the whole loop and a read at or past position S returns
    // zeros (the descriptor's range check) instead of needing a clamp.
    const int rowb = a.Hkv * D * 2;  // bytes from one position to the next
    auto cache_rsrc = [&](const uint16_t* cache, int key0) {
        const int k0 = min(key0, a.S);
        const int nrec = static_cast<int>(static_cast<uint32_t>(min(a.S - k0, a.kv_cap)) * static_cast<uint32_t>(rowb) -
                                          static_cast<uint32_t>(k0 < a.S ? g * D * 2 : 0));
        const uint16_t* p = cache + ((static_cast<size_t>(b) * a.S + k0) * a.Hkv + g) * D;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), static_cast<short>(0), nrec,
                                                 kRawBufferFlags);
    };
    // chunk c of a tile: key c / (D/8), values 8 (c % (D/8)) .. + 7, the
    // same for keys and values
    uint32_t koff[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int c = tid + u * kAThreads;
        koff[u] = static_cast<uint32_t>((c / (D / 8)) * rowb + (c % (D / 8)) * 16);
    }
    // a tile's keys and values in registers: the next tile's loads are issued
    // before the current tile's matrix work, so the two overlap
    uint4 kc[kU], vc[kU];
    auto load_tile = [&](int key0) {
        const auto rk = cache_rsrc(a.k, key0);
        const auto rv = cache_rsrc(a.v, key0);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            kc[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff[u], 0, 0));
            vc[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, koff[u], 0, 0));
        }
    };
    // bit j: key key0 + j of a tile exists in the partition (below hi), and
    // (candidates) lies in a row some node occupies (`rows`, uniform) or on
    // this lane's query row's root path (`vis_or`, per lane)
    auto tile_bits = [&](int key0, uint64_t rows) {
        const int sh = tree ? ((key0 - L) & 63) : 0;  // uniform: 0 or 32 for the candidates
        const int rem = hi - key0;
        const uint32_t below = rem >= kTileKeys ? 0xffffffffu : (rem <= 0 ? 0u : (1u << rem) - 1u);
        return static_cast<uint32_t>(rows >> sh) & below;
    };
    // stage a tile from the registers into LDS buffer `buf`, keys and values
    // alike row-major (one row per key).  Keys are staged as they are (the
    // scores of keys a row may not see are masked); the values of keys no row
    // may see (past the partition, candidate rows no node occupies, positions
    // past S) are staged as zeros, since their weight 0 times whatever the
    // cache holds there must not reach the output
    auto stage = [&](int key0, int buf) {
        uint16_t* sk = s_k + buf * (Lds::kBuf / 2);
        uint16_t* sv = s_v + buf * (Lds::kBuf / 2);
        const uint32_t keepb = tile_bits(key0, used);  // uniform
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int c = tid + u * kAThreads;
            const int kk = c / (D / 8), d8 = (c % (D / 8)) * 8;
            *reinterpret_cast<uint4*>(sk + kk * Lds::kKStride + d8) = kc[u];
            uint4 vw = vc[u];
            if (keepb != 0xffffffffu) {  // uniform: a tile with keys to drop
                const uint32_t keep = 0u - ((keepb >> kk) & 1u);  // all ones or zeros
                vw = make_uint4(vw.x & keep, vw.y & keep, vw.z & keep, vw.w & keep);
            }
            *reinterpret_cast<uint4*>(sv + kk * Lds::kKStride + d8) = vw;
        }
    };
    // two LDS buffers: while the waves work on tile t in one, tile t + 1 is
    // staged into the other and tile t + 2 is on its way into registers
    if (ntiles > 0) {
        load_tile(lo);
        stage(lo, 0);
        load_tile(lo + kTileKeys);
    }
    __syncthreads();  // queries and the first tile staged
    abf16x8_t qreg[kDS];  // this lane's query row, as the B operand of S^T
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds)
        qreg[ds] = *reinterpret_cast<const abf16x8_t*>(s_q + rq * Lds::kKStride + ds * 32 + 8 * lg);
    const float scale2 = a.scale2;  // positive and finite (checked on the host)
    for (int tile = 0; tile < ntiles; ++tile) {
        const int key0 = lo + tile * kTileKeys;
        const int cur = tile & 1;
        // (uniform.)  Past the last tile the loads read zeros and are never
        // staged
        if (tile + 1 < ntiles) stage(key0 + kTileKeys, cur ^ 1);
        load_tile(key0 + 2 * kTileKeys);
        const uint16_t* s_kc = s_k + cur * (Lds::kBuf / 2);
        const uint16_t* s_vc = s_v + cur * (Lds::kBuf / 2);

        // S^T blocks: lane (lg, l16) holds keys 16 kb + 4 lg + i of query row rq
        // four independent accumulation chains (block x even/odd d step) keep
        // the matrix pipeline busy instead of waiting on one chain
        af32x4_t acc4[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc4[kb][0] = acc4[kb][1] = af32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < kDS; ++ds)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const abf16x8_t ka = *reinterpret_cast<const abf16x8_t*>(
                    s_kc + (kb * 16 + l16) * Lds::kKStride + ds * 32 + 8 * lg);
                acc4[kb][ds & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[ds], acc4[kb][ds & 1], 0, 0, 0);
            }
        // raw scores: the matrix-core results are first read right after
        // the contraction, in its basic block (a read in a later block after
        // a branch got stale results here)
        float sr[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const af32x4_t acc = acc4[kb][0] + acc4[kb][1];
#pragma unroll
            for (int i = 0; i < 4; ++i) sr[kb][i] = acc[i];
        }
        // masked, unless every key of the tile is visible to every row (a
        // whole tile of a prefix partition): a key row q may not see gets
        // -inf; bit 16 kb + i of `vis` is this lane's key 16 kb + 4 lg + i
        if (tree || hi - key0 < kTileKeys) {  // uniform
            const uint32_t vis = tile_bits(key0, vis_or) >> (4 * lg);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int bit = 16 * kb + i;
                    const uint32_t okm = static_cast<uint32_t>(static_cast<int32_t>(vis << (31 - bit)) >> 31);
                    sr[kb][i] = __uint_as_float((__float_as_uint(sr[kb][i]) & okm) | (0xff800000u & ~okm));
                }
        }
        // online softmax per query row (the row's scores sit in lanes l16,
        // l16 + 16, l16 + 32, l16 + 48), in the log2 domain: the scale is
        // positive, so the row maximum of the scaled scores is the scaled
        // maximum of the raw ones, and -inf stays -inf
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sr[kb][i]);  // this lane's raw maximum
        // The row's reference maximum m_run (the same in the row's four
        // lanes) moves only when a score exceeds it by more than
        // kRescaleSlack (log2 units): weights then stay below 2^kRescaleSlack,
        // far inside fp32 and the hi + lo split, and the output rows are
        // rescaled a few times per partition instead of at almost every
        // tile.  The first finite score always moves it.  A row moves only
        // when one of its lanes' raw maxima passes thr_raw, so the row
        // maximum is formed only on tiles where some lane of the wave does
        // (the test is wave-uniform).
        if (__ballot(mt > thr_raw) != 0ull) {
            const float mrow = pair32_max(pair16_max(mt)) * scale2;
            const bool grow = mrow > m_run + kRescaleSlack;
            const float m_old = m_run;
            if (grow) m_run = mrow;
            m_use = m_run == -INFINITY ? 0.f : m_run;
            thr_raw = (m_run + kRescaleSlack) / scale2;
            // rescale this lane's share of the row's sum and the output rows
            // 4 lg + i of this lane's blocks
            const float factor = grow ? __builtin_amdgcn_exp2f(m_old - m_run) : 1.f;  // 0 while nothing was seen
            l_run *= factor;
            float fr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) fr[i] = __shfl(factor, 4 * lg + i, 64);
#pragma unroll
            for (int db = 0; db < kDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[db][i] *= fr[i];
        }
        float pr[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[kb][i], scale2, -m_use));
        // this lane's share of the row's sum: its eight weights summed
        // pairwise (a chain three deep); the four shares are added at the end
        l_run += ((pr[0][0] + pr[0][1]) + (pr[0][2] + pr[0][3])) + ((pr[1][0] + pr[1][1]) + (pr[1][2] + pr[1][3]));
        // P as the A operand (row rq; k slots: keys 4 lg + j of block 0, then
        // of block 1), split into bf16 hi + lo
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int kb = e >> 1, i0 = 2 * (e & 1);
            const float x0 = pr[kb][i0], x1 = pr[kb][i0 + 1];
            ph[e] = bf16_pack_rne(x0, x1);
            const float h0f = bf16_bits_to_f32(static_cast<uint16_t>(ph[e] & 0xffffu));
            const float h1f = bf16_bits_to_f32(static_cast<uint16_t>(ph[e] >> 16));
            pl[e] = bf16_pack_rne(x0 - h0f, x1 - h1f);
        }
        const abf16x8_t pa_hi = __builtin_bit_cast(abf16x8_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
        const abf16x8_t pa_lo = __builtin_bit_cast(abf16x8_t, make_uint4(pl[0], pl[1], pl[2], pl[3]));
        // value operands for eight d blocks at a time, then the hi products
        // of all eight, then the lo products (independent accumulators back
        // to back).  Lane (lg, l16) needs value column 16 db + l16 of keys
        // 4 lg .. + 3 and 16 + 4 lg .. + 3.  The transposing LDS read hands
        // lane 4 a + c of each 16-lane row element c of the 4-value pieces
        // that the row's lanes a, 4 + a, 8 + a, 12 + a address: so lane
        // (lg, l16) addresses key 4 lg + l16 / 4, columns 16 db + 4 (l16 % 4)
        // .. + 3, and 16 keys further for the second half
        const uint16_t* vrow = s_vc + (4 * lg + (l16 >> 2)) * Lds::kKStride + 4 * (l16 & 3);
        constexpr int kDBH = kDB < 8 ? kDB : 8;
#pragma unroll
        for (int d0 = 0; d0 < kDB; d0 += kDBH) {
            abf16x8_t vb[kDBH];
#pragma unroll
            for (int j = 0; j < kDBH; ++j) {
                const uint16_t* vr = vrow + (d0 + j) * 16;
                const ai16x4_t v0 = lds_read_tr16x4(vr);
                const ai16x4_t v1 = lds_read_tr16x4(vr + 16 * Lds::kKStride);
                vb[j] = __builtin_bit_cast(abf16x8_t, (ai16x8_t){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
            }
#pragma unroll
            for (int j = 0; j < kDBH; ++j)
                o[d0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, vb[j], o[d0 + j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kDBH; ++j)
                o[d0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vb[j], o[d0 + j], 0, 0, 0);
        }
        __syncthreads();  // tile t + 1 staged; tile t's buffer free for tile t + 2
    }

    // partial results: O rows 4 lg + i of this wave, maximum and sum of row rq
    const size_t base = (static_cast<size_t>(sp) * a.B + b) * a.Hq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * lg + i;
        const int ir = r % NPH, hr = r / NPH;
        if (ir < N && hr < nh) {
            float* dst = a.ws_o + ((base + h0 + hr) * N + ir) * D + l16;
#pragma unroll
            for (int db = 0; db < kDB; ++db) dst[db * 16] = o[db][i];
        }
    }
    l_run = pair32_sum(pair16_sum(l_run));  // the row's sum from its four lanes' shares
    if (lg == 0 && vq) {
        float* ml = a.ws_ml + ((base + h0 + hq) * N + iq) * 2;
        ml[0] = m_run;
        ml[1] = l_run;
    }
}

// Merge of the key partitions (the standard split-softmax merge): one
// workgroup per (request, head, node) row, one thread per output element.
// The partitions' maxima, weights exp2(m_s - M) and the denominator are
// formed once per row, cooperatively, with the weights kept in LDS; then each
// thread sums its element over the partitions with many loads in flight.
constexpr int kMaxPartitions = 1025;  // splits <= 1024, plus the candidates'
template <int D>
__global__ void __launch_bounds__(D) tree_attn_merge_kernel(const AttnArgs a) {
    __shared__ float s_w[kMaxPartitions];
    __shared__ float s_red[D / 64];
    const int row = blockIdx.x;  // ((b * Hq) + h) * N + i
    const int N = a.N;
    const int i = row % N;
    const int h = (row / N) % a.Hq;
    const int b = row / (N * a.Hq);
    int L;
    if (attn_skip(a, b, L)) return;  // uniform
    const int d = threadIdx.x;
    const int wv = d >> 6;
    const size_t per_split = static_cast<size_t>(a.B) * a.Hq * N;
    const int nsp = a.splits + 1;
    float M = -INFINITY;
    for (int s = d; s < nsp; s += D) {
        const float m = a.ws_ml[(s * per_split + row) * 2];
        s_w[s] = m;
        M = fmaxf(M, m);
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x, 64));
    if ((d & 63) == 0) s_red[wv] = M;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < D / 64; ++k) M = fmaxf(M, s_red[k]);
    float den = 0.f;
    for (int s = d; s < nsp; s += D) {
        const float wgt = __builtin_amdgcn_exp2f(s_w[s] - M);  // 0 for an empty partition
        s_w[s] = wgt;
        den += wgt * a.ws_ml[(s * per_split + row) * 2 + 1];
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) den += __shfl_xor(den, x, 64);
    __syncthreads();  // every lane has read s_red (the maxima)
    if ((d & 63) == 0) s_red[wv] = den;
    __syncthreads();  // the weights and the partial denominators
    den = 0.f;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) den += s_red[k];
    float acc = 0.f;
#pragma unroll 16
    for (int s = 0; s < nsp; ++s) acc += s_w[s] * a.ws_o[(s * per_split + row) * D + d];
    const float val = acc / den;
    const size_t oi = ((static_cast<size_t>(b) * N + i) * a.Hq + h) * D + d;
    if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_bits(val);
    else
        static_cast<float*>(a.out)[oi] = val;
}

// ---- scratch of the no-alloc entry point ---------------------------------
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the split partial results
// go to this file-scope array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy until the process ends; calls that
// overlap on one GPU share it and race.  In host code its name is only a
// stand-in: the device address comes from hipGetSymbolAddress, taken once
// per device with that device current.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void* noalloc_scratch(hipError_t* status) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    if (e != hipSuccess) {
        *status = e;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            *status = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        addr[dev] = ptr;
    }
    *status = hipSuccess;
    return addr[dev];
}

size_t tree_attention_workspace_bytes(int B, int N, int Hq, int D, int splits) {
    const size_t rows = static_cast<size_t>(splits + 1) * B * Hq * N;
    return rows * (static_cast<size_t>(D) + 2) * sizeof(float);
}

hipError_t launch_tree_attention(const gdn_tree_desc& d, const TreeAttnArgs& ta, hipStream_t s) {
    AttnArgs a{};
    a.B = d.B;
    a.N = d.N;
    a.R = d.R;
    a.S = ta.S;
    a.Hq = ta.Hq;
    a.Hkv = ta.Hkv;
    a.splits = ta.splits;
    a.HPW = d.N <= 32 ? 4 : 2;  // query heads per workgroup (kRows rows)
    const int G = ta.Hq / ta.Hkv;
    a.pairs = (G + a.HPW - 1) / a.HPW;
    a.shared = d.shared;
    a.node_row = d.node_row;
    a.anc = d.anc;
    a.status = d.status;
    a.q = static_cast<const uint16_t*>(ta.q);
    a.k = static_cast<const uint16_t*>(ta.k);
    a.v = static_cast<const uint16_t*>(ta.v);
    a.ctx_len = ta.ctx_len;
    a.scale2 = ta.scale * kLog2e;
    a.kv_cap = static_cast<int>(0xffffffffu / (static_cast<uint32_t>(ta.Hkv) * ta.D * 2u));
    const size_t rows = static_cast<size_t>(ta.splits + 1) * d.B * ta.Hq * d.N;
    a.ws_o = static_cast<float*>(ta.workspace);
    a.ws_ml = a.ws_o + rows * ta.D;
    a.out = ta.out;
    a.out_bf16 = (ta.flags & GDN_F_OUT_BF16) ? 1 : 0;
    a.err = ta.err;
    // context keys per partition: the longest context the cache can hold
    // (S - R) split evenly, in whole tiles
    const int max_ctx = ta.S - d.R;
    a.chunk = ((max_ctx + ta.splits - 1) / ta.splits + kTileKeys - 1) / kTileKeys * kTileKeys;
    if (a.chunk < kTileKeys) a.chunk = kTileKeys;
    const unsigned units = static_cast<unsigned>(d.B) * ta.Hkv * (ta.splits + 1) * a.pairs;
    const unsigned mrows = static_cast<unsigned>(d.B) * ta.Hq * d.N;
    if (ta.D == 128) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(tree_attn_kernel<128>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(AttnLds<128>::total));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(tree_attn_kernel<128>, dim3(units), dim3(kAThreads), AttnLds<128>::total, s, a);
        hipLaunchKernelGGL(tree_attn_merge_kernel<128>, dim3(mrows), dim3(128), 0, s, a);
    } else if (ta.D == 256) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(tree_attn_kernel<256>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(AttnLds<256>::total));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(tree_attn_kernel<256>, dim3(units), dim3(kAThreads), AttnLds<256>::total, s, a);
        hipLaunchKernelGGL(tree_attn_merge_kernel<256>, dim3(mrows), dim3(256), 0, s, a);
    } else {
        return hipErrorNotSupported;
    }
    return hipGetLastError();
}

// ---- KV publication ----------------------------------------------------
// One workgroup per (request, kv head): every source entry of the accepted
// path is read into LDS before any destination is written (sources and
// destinations overlap inside the candidate suffix).
template <int D>
__global__ void __launch_bounds__(256) kv_publish_kernel(int B, int R, int S, int Hkv, int Lmax,
                                                         const int32_t* __restrict__ path_rows,
                                                         const int32_t* __restrict__ path_n,
                                                         uint16_t* __restrict__ k, uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ ctx_len,
                                                         int32_t* __restrict__ err) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    uint4* s_k = reinterpret_cast<uint4*>(lds);                          // [Lmax][D / 8]
    uint4* s_v = s_k + static_cast<size_t>(Lmax) * (D / 8);
    const int b = blockIdx.x / Hkv;
    const int g = blockIdx.x % Hkv;
    const int n = min(min(path_n[b], Lmax), R);  // a path has at most R distinct nodes
    if (n <= 0) return;
    const int L = ctx_len[b];
    if (L < 0 || L + R > S) {
        if (g == 0 && threadIdx.x == 0) atomicOr(err, GDN_EV_CTX);
        return;
    }
    constexpr int C8 = D / 8;  // 16-byte chunks per entry
    for (int c = threadIdx.x; c < n * C8; c += blockDim.x) {
        const int j = c / C8, e = c % C8;
        const int r = min(max(path_rows[static_cast<size_t>(b) * Lmax + j], 0), R - 1);
        const size_t src = ((static_cast<size_t>(b) * S + L + r) * Hkv + g) * D / 8 + e;
        s_k[c] = reinterpret_cast<const uint4*>(k)[src];
        s_v[c] = reinterpret_cast<const uint4*>(v)[src];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < n * C8; c += blockDim.x) {
        const int j = c / C8, e = c % C8;
        const size_t dst = ((static_cast<size_t>(b) * S + L + j) * Hkv + g) * D / 8 + e;
        reinterpret_cast<uint4*>(k)[dst] = s_k[c];
        reinterpret_cast<uint4*>(v)[dst] = s_v[c];
    }
}

hipError_t launch_kv_publish(const gdn_tree_desc& prev, const int32_t* path_rows, const int32_t* path_n,
                             int Lmax, void* k, void* v, int S, const int32_t* ctx_len, int Hkv, int D,
                             int32_t* err, hipStream_t s) {
    const size_t lds = static_cast<size_t>(Lmax) * D * 2 * 2;
    const dim3 grid(static_cast<unsigned>(prev.B) * Hkv);
    if (D == 128) {
        hipLaunchKernelGGL(kv_publish_kernel<128>, grid, dim3(256), lds, s, prev.B, prev.R, S, Hkv, Lmax,
                           path_rows, path_n, static_cast<uint16_t*>(k), static_cast<uint16_t*>(v), ctx_len,
                           err);
    } else if (D == 256) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kv_publish_kernel<256>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kv_publish_kernel<256>, grid, dim3(256), lds, s, prev.B, prev.R, S, Hkv, Lmax,
                           path_rows, path_n, static_cast<uint16_t*>(k), static_cast<uint16_t*>(v), ctx_len,
                           err);
    } else {
        return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace gdn

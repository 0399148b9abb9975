// gdn_fast.hip -- tree verify and accepted-path replay on the matrix cores for
// D in {64, 128} with bf16 or fp32 q/k/v (fp32 keys and queries enter the
// products split into bf16 hi + lo, fp32 values enter the vector arithmetic
// as they are).
//
// Unrolling the gated delta rule along a root-to-node path gives, for node n
// with path p_0 (root) ... p_{d-1} = n and G_n = a_{p_0} ... a_{p_{d-1}}:
//     S^n = G_n S0 + sum_e R(n,e) c_{p_e} k_{p_e}^T,   R(n,e) = a_{p_{e+1}} ... a_{p_{d-1}}
//     c_n = b_n v_n - b_n G_n (S0 k_n) - sum_{e<d-1} b_n R(n,e) (k_{p_e} . k_n) c_{p_e}
//     o_n = G_n (S0 q_n) + sum_{e<=d-1} R(n,e) (k_{p_e} . q_n) c_{p_e}
// where c_n = b_n (v_n - a_n S^{parent} k_n) is the row vector of the rule
// written as S' = a S + c k^T.  A whole tree therefore needs only the dense
// products S0 K^T and S0 Q^T over its nodes -- one contraction per (sequence,
// value head), done on the matrix cores -- plus, per state row, a short
// recurrence over each node's ancestors.  Verify never materializes a state.
// Replay (persist) needs S^m for one root-to-node path of <= 16 nodes: it
// reads S0 once, forms S0 k_e for the path keys on the matrix cores, runs the
// same recurrence per row and writes G_m S0 + sum_e R(m,e) c_e k_e^T in place
// as a rank-16 update accumulated onto the scaled state.  The fused persist + verify
// runs both on one load of S: the replay's update in registers, stored in
// place, then the next tree's products S K^T and S Q^T from the same registers.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 32;             // nodes per MFMA block
constexpr int kPath = GDN_MAX_DEPTH;  // max ancestors per node (incl. itself)
constexpr int kFastMaxNodes = GDN_MAX_NODES;  // largest tree the MFMA verify takes (8 node blocks)
constexpr int kMaskWords = GDN_MAX_NODES / 32;  // 32-node ancestor mask words per node
constexpr size_t kLdsBudget = 160 * 1024;       // LDS of one compute unit

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
__device__ __forceinline__ float qnan_f() { return __int_as_float(0x7fc00000); }

// q/k/v element: bf16 bits, or fp32 (F32)
template <bool F32>
using InT = typename std::conditional<F32, float, uint16_t>::type;
__device__ __forceinline__ float in2f(uint16_t x) { return bf2f(x); }
__device__ __forceinline__ float in2f(float x) { return x; }

// fp32 keys and queries enter the matrix cores as bf16 hi + lo (hi the nearest
// bf16, lo the nearest bf16 to the remainder: about 16 significant bits).
__device__ __forceinline__ uint32_t split_pair(float x, float y, uint32_t &lo) {
    const __bf16 hx = static_cast<__bf16>(x), hy = static_cast<__bf16>(y);
    const __bf16 lx = static_cast<__bf16>(x - static_cast<float>(hx));
    const __bf16 ly = static_cast<__bf16>(y - static_cast<float>(hy));
    lo = (uint32_t)__builtin_bit_cast(uint16_t, lx) | (uint32_t)__builtin_bit_cast(uint16_t, ly) << 16;
    return (uint32_t)__builtin_bit_cast(uint16_t, hx) | (uint32_t)__builtin_bit_cast(uint16_t, hy) << 16;
}
__device__ __forceinline__ void split4(const float4 x, uint2 &hi, uint2 &lo) {
    hi.x = split_pair(x.x, x.y, lo.x);
    hi.y = split_pair(x.z, x.w, lo.y);
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Buffer resource over `bytes` bytes from `base`: loads past the end return zero and
// stores past the end are dropped by the hardware's range check (the byte offset is
// the VGPR offset; it must hold all of it, the scalar offset is not range-checked).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}


// ===========================================================================
// Verify
// ===========================================================================
template <int D>
struct VG {
    static constexpr int WAVES = D / 32;      // wave w owns state rows [32w, 32w+32)
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int KS = D / 16;         // MFMA 32x32x16 k-steps
};

__device__ __forceinline__ bf16x8 frag_of(const uint16_t *vec, int s, int hf) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(vec + 16 * s + 8 * hf);
    return __builtin_bit_cast(bf16x8, raw);
}
__device__ __forceinline__ bf16x8 zero_frag() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// acc + A B for operands split hi + lo: hi*hi + hi*lo + lo*hi (the lo*lo term, at
// most ~2^-16 of the product, is dropped)
__device__ __forceinline__ f32x16 mfma_split(bf16x8 ahi, bf16x8 alo, bf16x8 bhi, bf16x8 blo, f32x16 acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bhi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, blo, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bhi, acc, 0, 0, 0);
}

// k-step s fragment (8 values, 16s + 8*half onwards) of an fp32 row, split hi + lo
__device__ __forceinline__ void frag_split(const float *vec, int s, int hf, bf16x8 &hi, bf16x8 &lo) {
    const float4 x0 = *reinterpret_cast<const float4 *>(vec + 16 * s + 8 * hf);
    const float4 x1 = *reinterpret_cast<const float4 *>(vec + 16 * s + 8 * hf + 4);
    uint2 h0, l0, h1, l1;
    split4(x0, h0, l0);
    split4(x1, h1, l1);
    hi = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
    lo = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
}

// Sequence view shared by the two verify kernels.  CHAIN: sequence b is the
// chain of nodes [cu[b], cu[b+1]) (validated here); else the plan's verdict.
struct SeqView {
    int lo, n, status, slot;
};

template <bool CHAIN>
__device__ __forceinline__ SeqView seq_view(const Params &P, int b) {
    SeqView v;
    if (CHAIN) {
        const int c0 = P.cu_nodes[b], c1 = P.cu_nodes[b + 1];
        const bool in_bounds = 0 <= c0 && c0 <= c1 && c1 <= P.T;
        v.lo = in_bounds ? c0 : 0;
        v.n = in_bounds ? c1 - c0 : 0;
        v.status = (in_bounds && v.n <= P.max_nodes) ? GDN_SEQ_OK : GDN_SEQ_BAD_NODES;
        v.slot = (v.status == GDN_SEQ_OK && v.n > 0) ? P.slot_idx[b] : 0;
        if (v.status == GDN_SEQ_OK && v.n > 0 && (v.slot < 0 || v.slot >= P.num_slots)) v.status = GDN_SEQ_BAD_SLOT;
    } else {
        const int4 info = *reinterpret_cast<const int4 *>(P.ws.seq_info + b * kSeqInfoInts);
        v.lo = info.x;
        v.n = info.y;
        v.status = info.z;
        v.slot = info.w;
    }
    return v;
}

// Ancestor e (root first) of local node i: the plan's path, or e for a chain.
template <bool CHAIN>
__device__ __forceinline__ int anc_of(const Params &P, int lo, int i, int e) {
    if (CHAIN) return e <= i ? e : 0;
    const int a = P.ws.nodepath[(size_t)(lo + i) * GDN_MAX_DEPTH + e];
    return a < 0 ? 0 : a;
}

// ===========================================================================
// Verify, part 1: coefficients.  One workgroup per (sequence, key head); the
// value heads of the group share the tree, the keys/queries and the Gram
// entries k_anc . k_i and k_anc . q_i.  Per (node i, value head) it writes
//   y_i[e] (e < 16), gamma_i, alpha_i = b_i gamma_i, b_i, depth_i
// into the workspace, where, with R(i,e) = a_{anc_{e+1}} ... a_{anc_{d-1}},
//   Lc[i][e] = b_i R(i,e) (k_{anc_e} . k_i)      (e < d-1)
//   m_i[e]   = R(i,e) (k_{anc_e} . q_i)           (e < d-1),   m_i[d-1] = k_i . q_i
//   y_i      = m_i (I + Lc_path(i))^-1, by back substitution over i's path:
//   y_{d-1} = m_i[d-1],   y_e = m_i[e] - sum_{f>e} y_f Lc[anc_f][e].
// Then o_i = gamma_i (S0 q_i) + sum_e y_i[e] r_{anc_e(i)} with
// r_j = b_j v_j - alpha_j (S0 k_j): see the main kernel.
// ===========================================================================
constexpr int kCoefThreads = 256;
constexpr int kCoefMaxHeadsPerPass = 8;

struct CTab {
    int *anc;        // [cap][16]
    int *depth;      // [cap rounded up to whole node blocks]
    uint32_t *amask; // [cap][kMaskWords]
    float *gk, *gq;  // [cap][16] path-indexed Gram entries
    float *a, *b;    // [grp][cap]
    float *coefL;    // [hpp][cap][16]
};

__host__ __device__ inline size_t ctab_bytes(int cap, int grp, int hpp) {
    const size_t c = (size_t)cap;
    const size_t depth = (c + kTile - 1) / kTile * kTile;  // whole node blocks, read four at a time
    return c * kPath * 4 + depth * 4 + c * kMaskWords * 4 + 2 * c * kPath * 4 + 2 * (size_t)grp * c * 4 +
           (size_t)hpp * c * kPath * 4;
}

// Most value heads one coefficient pass takes for trees of up to cap nodes: what
// the LDS holds, at most kCoefMaxHeadsPerPass (0: not even one fits)
__host__ __device__ inline int coef_heads_per_pass(int cap, int grp) {
    int h = grp < kCoefMaxHeadsPerPass ? grp : kCoefMaxHeadsPerPass;
    while (h > 0 && ctab_bytes(cap, grp, h) > kLdsBudget) --h;
    return h;
}

__device__ inline CTab ctab_carve(char *base, int cap, int grp, int hpp) {
    CTab L;
    const size_t c = (size_t)cap;
    L.anc = reinterpret_cast<int *>(base);        base += c * kPath * 4;
    L.gk = reinterpret_cast<float *>(base);       base += c * kPath * 4;
    L.gq = reinterpret_cast<float *>(base);       base += c * kPath * 4;
    L.coefL = reinterpret_cast<float *>(base);    base += (size_t)hpp * c * kPath * 4;
    L.amask = reinterpret_cast<uint32_t *>(base); base += c * kMaskWords * 4;
    L.depth = reinterpret_cast<int *>(base);      base += (c + kTile - 1) / kTile * kTile * 4;
    L.a = reinterpret_cast<float *>(base);        base += (size_t)grp * c * 4;
    L.b = reinterpret_cast<float *>(base);
    return L;
}

template <int D, bool CHAIN, bool F32>
__global__ __launch_bounds__(kCoefThreads) void coef_kernel(Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    constexpr int KS = D / 16;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int grp = P.Hv / P.Hk;
    const int b = blockIdx.x / P.Hk, g = blockIdx.x % P.Hk;
    const SeqView sv = seq_view<CHAIN>(P, b);
    if (!CHAIN && !ws_plan_matches(P)) return;
    if (sv.status != GDN_SEQ_OK || sv.n == 0) return;
    const int lo = sv.lo, n = sv.n;
    const int cap = CHAIN ? kPath : P.max_nodes;
    const int hpp = max(1, min(coef_heads_per_pass(cap, grp), kCoefThreads / n));  // value heads per pass
    const CTab L = ctab_carve(lds_raw, cap, grp, hpp);

    // tree tables and ancestor masks, gates of every head of the group
    for (int i = tid; i < n; i += kCoefThreads) {
        int an[kPath];
#pragma unroll
        for (int e = 0; e < kPath; ++e) an[e] = anc_of<CHAIN>(P, lo, i, e);
        const int d = CHAIN ? i + 1 : P.ws.depth[lo + i];
#pragma unroll
        for (int e = 0; e < kPath; ++e) L.anc[i * kPath + e] = an[e];
        // one mask word at a time, so the word index stays a constant
#pragma unroll
        for (int t = 0; t < kMaskWords; ++t) {
            uint32_t m = 0u;
#pragma unroll
            for (int e = 0; e < kPath; ++e)
                if (e < d && (an[e] >> 5) == t) m |= 1u << (an[e] & 31);
            L.amask[i * kMaskWords + t] = m;
        }
        L.depth[i] = d;
    }
    for (int idx = tid; idx < grp * n; idx += kCoefThreads) {
        const int hh = idx / n, i = idx % n;
        const size_t at = (size_t)(lo + i) * P.Hv + g * grp + hh;
        L.a[hh * cap + i] = P.a[at];
        L.b[hh * cap + i] = P.b[at];
    }
    __syncthreads();

    // Gram entries for every (ancestor, node) pair on the matrix cores
    const InT<F32> *kb = static_cast<const InT<F32> *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const InT<F32> *qb = static_cast<const InT<F32> *>(P.q) + ((size_t)lo * P.Hk + g) * D;
    const size_t kq_stride = (size_t)P.Hk * D;
    const int ntiles = (n + kTile - 1) / kTile;
    for (int pair = w; pair < ntiles * ntiles; pair += kCoefThreads / 64) {
        const int ti = pair % ntiles, tj = pair / ntiles;
        const int pi = ti * kTile + l32, pj = tj * kTile + l32;
        f32x16 gkk = {}, gkq = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if constexpr (F32) {
                bf16x8 A = zero_frag(), Al = zero_frag(), Bk = zero_frag(), Bkl = zero_frag(), Bq = zero_frag(),
                       Bql = zero_frag();
                if (pi < n) frag_split(kb + (size_t)pi * kq_stride, s, hf, A, Al);
                if (pj < n) {
                    frag_split(kb + (size_t)pj * kq_stride, s, hf, Bk, Bkl);
                    frag_split(qb + (size_t)pj * kq_stride, s, hf, Bq, Bql);
                }
                gkk = mfma_split(A, Al, Bk, Bkl, gkk);
                gkq = mfma_split(A, Al, Bq, Bql, gkq);
            } else {
                const bf16x8 A = pi < n ? frag_of(kb + (size_t)pi * kq_stride, s, hf) : zero_frag();
                const bf16x8 Bk = pj < n ? frag_of(kb + (size_t)pj * kq_stride, s, hf) : zero_frag();
                const bf16x8 Bq = pj < n ? frag_of(qb + (size_t)pj * kq_stride, s, hf) : zero_frag();
                gkk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bk, gkk, 0, 0, 0);
                gkq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bq, gkq, 0, 0, 0);
            }
        }
        if (pj < n) {  // accumulator r: (candidate ancestor ti*32 + il, node pj)
            const uint32_t mask = L.amask[pj * kMaskWords + ti];
            // the candidates' depths four at a time, read before any write (past the last node
            // the depths are never used)
            int4 dq[4];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) dq[g4] = *reinterpret_cast<const int4 *>(L.depth + ti * kTile + 8 * g4 + 4 * hf);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int il = 8 * (r / 4) + 4 * hf + (r % 4);
                const int4 q4 = dq[r / 4];
                const int dep = r % 4 == 0 ? q4.x : r % 4 == 1 ? q4.y : r % 4 == 2 ? q4.z : q4.w;
                if ((mask >> il) & 1u) {
                    L.gk[pj * kPath + dep - 1] = gkk[r];
                    L.gq[pj * kPath + dep - 1] = gkq[r];
                }
            }
        }
    }
    __syncthreads();

    for (int h0 = 0; h0 < grp; h0 += hpp) {
        const int hh = h0 + tid / n, i = tid % n;
        const bool act = tid < hpp * n && hh < grp;
        const int slot_h = tid / n;
        float mrow[kPath], gamma = 0.0f, bi = 0.0f;
        int an[kPath], d = 0;
        if (act) {
            d = L.depth[i];
            bi = L.b[hh * cap + i];
            // every table entry of the row, read before the first coefficient is written
            float av[kPath], gk[kPath], gq[kPath];
#pragma unroll
            for (int e = 0; e < kPath; ++e) an[e] = L.anc[i * kPath + e];
#pragma unroll
            for (int e = 0; e < kPath; ++e) {
                const float ae = L.a[hh * cap + max(an[e], 0)];
                av[e] = e < d ? ae : 1.0f;
                gk[e] = L.gk[i * kPath + e];
                gq[e] = L.gq[i * kPath + e];
            }
            float r = 1.0f;
#pragma unroll
            for (int e = kPath - 1; e >= 0; --e) {
                const bool on = e < d - 1;
                L.coefL[(slot_h * cap + i) * kPath + e] = on ? bi * r * gk[e] : 0.0f;
                mrow[e] = on ? r * gq[e] : (e == d - 1 ? gq[e] : 0.0f);
                r *= av[e];
            }
            gamma = r;
        }
        __syncthreads();
        if (act) {
            float y[kPath];
#pragma unroll
            for (int e = kPath - 1; e >= 0; --e) {
                float acc = mrow[e];
                // deepest terms first: y_{e+1}, the last one known, enters last
#pragma unroll
                for (int f = kPath - 1; f > e; --f)
                    acc = fmaf(-y[f], L.coefL[(slot_h * cap + an[f]) * kPath + e], acc);
                y[e] = e < d ? acc : 0.0f;
            }
            float4 *rec = reinterpret_cast<float4 *>(P.ws.coef + ((size_t)(lo + i) * P.Hv + g * grp + hh) * kCoefFloats);
#pragma unroll
            for (int e = 0; e < kPath; e += 4) rec[e / 4] = make_float4(y[e], y[e + 1], y[e + 2], y[e + 3]);
            rec[4] = make_float4(gamma, bi * gamma, bi, __int_as_float(d));
        }
        __syncthreads();
    }
}

// ===========================================================================
// Verify, part 2: one workgroup per (sequence, value head), D/32 waves; wave
// w owns state rows [32w, 32w+32).  With the records of part 1:
//   X = S0 K^T, Y = S0 Q^T          bf16 MFMA (state split hi + lo; keys exact)
//   r_j = b_j v_j - alpha_j X_j     in the MFMA accumulator layout
//   O = diag(gamma) Y + MT R        MT[i][anc_e(i)] = y_i[e]
// MT tiles: node blocks of 32 (1: trees of <= 32 nodes; the product then
// runs on fp32 MFMA straight from the accumulators of the first product).
// ===========================================================================
struct VTab {
    uint16_t *kq;   // [2][32][D] bf16 keys / queries (single-block trees); fp32 inputs: hi, then [2][32][D] lo
    float *mt;      // [32][32] dense MT (single-block trees)
    float *rbuf;    // [cap][D] r rows (multi-block trees)
    float *y;       // [cap][16] path weights
    uint8_t *anc;   // [cap][16] (local node ids, < 256)
    float4 *gabd;   // [cap] gamma, alpha, b, depth
};

__host__ __device__ inline size_t vtab_bytes(int cap, int D, bool single, bool f32 = false) {
    const size_t c = (size_t)cap;
    const size_t kq = (size_t)(f32 ? 4 : 2) * kTile * D * 2;
    return (single ? kq + (size_t)kTile * kTile * 4 : c * D * 4) + c * kPath * 4 + c * kPath + c * 16;
}

__device__ inline VTab vtab_carve(char *base, int cap, int D, bool single, bool f32 = false) {
    VTab L;
    const size_t c = (size_t)cap;
    L.gabd = reinterpret_cast<float4 *>(base);  base += c * 16;
    L.kq = reinterpret_cast<uint16_t *>(base);  base += single ? (size_t)(f32 ? 4 : 2) * kTile * D * 2 : 0;
    L.mt = reinterpret_cast<float *>(base);     base += single ? (size_t)kTile * kTile * 4 : 0;
    L.rbuf = reinterpret_cast<float *>(base);   base += single ? 0 : c * D * 4;
    L.y = reinterpret_cast<float *>(base);      base += c * kPath * 4;
    L.anc = reinterpret_cast<uint8_t *>(base);
    return L;
}

template <int D, bool CHAIN, int MT, bool F32>
__global__ __launch_bounds__(VG<D>::THREADS) __attribute__((amdgpu_waves_per_eu(3))) void verify_kernel(Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int row = w * 32 + l32;
    const int b = blockIdx.x / P.Hv, h = blockIdx.x % P.Hv;
    const int g = h / (P.Hv / P.Hk);
    const size_t out_stride = (size_t)P.Hv * D;
    const SeqView sv = seq_view<CHAIN>(P, b);  // loaded together with the header check below
    if (!CHAIN && !ws_plan_matches(P)) return;
    if (CHAIN && P.has_ws && h == 0 && tid == 0) {
        if (b == 0) {
            P.ws.header[0] = kChainMagic;
            P.ws.header[1] = P.B;
            P.ws.header[2] = P.T;
            P.ws.header[kHdrMisuse] = 0;
        }
        P.ws.seq_status[b] = sv.status;
    }
    if (!P.out) return;
    const int lo = sv.lo, n = sv.n;
    float *out_base = P.out + ((size_t)lo * P.Hv + h) * D + row;
    if (sv.status != GDN_SEQ_OK) {
        if (hf == 0)
            for (int i = 0; i < n; ++i) out_base[i * out_stride] = qnan_f();
        return;
    }
    if (n == 0) return;

    constexpr bool kSingle = MT == 1;
    const int cap = CHAIN ? kPath : P.max_nodes;
    const VTab L = vtab_carve(lds_raw, cap, D, kSingle, F32);
    const InT<F32> *kb = static_cast<const InT<F32> *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const InT<F32> *qb = static_cast<const InT<F32> *>(P.q) + ((size_t)lo * P.Hk + g) * D;
    const InT<F32> *vb = static_cast<const InT<F32> *>(P.v) + ((size_t)lo * P.Hv + h) * D + row;
    constexpr int EPC = F32 ? 4 : 8;  // values per 16-byte chunk
    const size_t kq_stride = (size_t)P.Hk * D, v_stride = (size_t)P.Hv * D;

    // ---- one round trip: every load is issued before any result is used
    const float *srow = P.state_in + (((size_t)sv.slot * P.Hv + h) * D + row) * D;
    float sf[VG<D>::KS][8];
#pragma unroll
    for (int s = 0; s < VG<D>::KS; ++s) {
        const float4 x0 = *reinterpret_cast<const float4 *>(srow + 16 * s + 8 * hf);
        const float4 x1 = *reinterpret_cast<const float4 *>(srow + 16 * s + 8 * hf + 4);
        sf[s][0] = x0.x; sf[s][1] = x0.y; sf[s][2] = x0.z; sf[s][3] = x0.w;
        sf[s][4] = x1.x; sf[s][5] = x1.y; sf[s][6] = x1.z; sf[s][7] = x1.w;
    }
    constexpr int KQ_PER = kSingle ? (2 * kTile * D / EPC + VG<D>::THREADS - 1) / VG<D>::THREADS : 1;
    uint4 kqv[KQ_PER];
    if (kSingle) {
#pragma unroll
        for (int u = 0; u < KQ_PER; ++u) {
            const int idx = tid + u * VG<D>::THREADS;
            const int which = idx / (kTile * (D / EPC)), rem = idx % (kTile * (D / EPC));
            const int i = rem / (D / EPC), c8 = rem % (D / EPC);
            kqv[u] = (which < 2 && i < n)
                         ? *reinterpret_cast<const uint4 *>((which ? qb : kb) + (size_t)i * kq_stride + EPC * c8)
                         : make_uint4(0, 0, 0, 0);
        }
    }
    InT<F32> vraw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r / 4) + 4 * hf + (r % 4);
        vraw[r] = i < n ? vb[(size_t)i * v_stride] : InT<F32>(0);
    }
    const float *coef = P.ws.coef + ((size_t)lo * P.Hv + h) * kCoefFloats;
    for (int i = tid; i < n; i += VG<D>::THREADS) {
        const float4 *rec = reinterpret_cast<const float4 *>(coef + (size_t)i * P.Hv * kCoefFloats);
        const float4 y0 = rec[0], y1 = rec[1], y2 = rec[2], y3 = rec[3], gabd = rec[4];
        int an[kPath];
#pragma unroll
        for (int e = 0; e < kPath; ++e) an[e] = anc_of<CHAIN>(P, lo, i, e);
        float4 *ydst = reinterpret_cast<float4 *>(L.y + i * kPath);
        ydst[0] = y0;
        ydst[1] = y1;
        ydst[2] = y2;
        ydst[3] = y3;
        uint32_t packed[kPath / 4];
#pragma unroll
        for (int e = 0; e < kPath; e += 4)
            packed[e / 4] = (uint32_t)an[e] | (uint32_t)an[e + 1] << 8 | (uint32_t)an[e + 2] << 16 |
                            (uint32_t)an[e + 3] << 24;
        *reinterpret_cast<uint4 *>(L.anc + i * kPath) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        L.gabd[i] = gabd;
    }
    if (kSingle) {
#pragma unroll
        for (int u = 0; u < KQ_PER; ++u) {
            const int idx = tid + u * VG<D>::THREADS;
            if (idx < 2 * kTile * (D / EPC)) {
                if constexpr (F32) {  // hi rows as the bf16 layout, lo rows 2*32 rows further
                    uint2 hi, lo2;
                    split4(__builtin_bit_cast(float4, kqv[u]), hi, lo2);
                    reinterpret_cast<uint2 *>(L.kq)[idx] = hi;
                    reinterpret_cast<uint2 *>(L.kq + 2 * kTile * D)[idx] = lo2;
                } else {
                    reinterpret_cast<uint4 *>(L.kq)[idx] = kqv[u];
                }
            }
        }
        for (int idx = tid; idx < kTile * kTile; idx += VG<D>::THREADS) L.mt[idx] = 0.0f;
    }
    bf16x8 shi[VG<D>::KS], slo[VG<D>::KS];
#pragma unroll
    for (int s = 0; s < VG<D>::KS; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const __bf16 hb = static_cast<__bf16>(sf[s][e]);
            shi[s][e] = hb;
            slo[s][e] = static_cast<__bf16>(sf[s][e] - static_cast<float>(hb));
        }
    }
    __syncthreads();

    if (kSingle) {
        // dense MT from the path weights
        for (int idx = tid; idx < n * kPath; idx += VG<D>::THREADS) {
            const int i = idx / kPath, e = idx % kPath;
            if (e < __float_as_int(L.gabd[i].w)) L.mt[i * kTile + L.anc[idx]] = L.y[idx];
        }
        const uint16_t *kr = L.kq + (size_t)l32 * D;
        const uint16_t *qr = L.kq + (size_t)(kTile + l32) * D;
        f32x16 ax = {}, ay = {};
#pragma unroll
        for (int s = 0; s < VG<D>::KS; ++s) {
            const bf16x8 Ak = frag_of(kr, s, hf);
            const bf16x8 Aq = frag_of(qr, s, hf);
            if constexpr (F32) {
                const bf16x8 Akl = frag_of(kr + 2 * kTile * D, s, hf);
                const bf16x8 Aql = frag_of(qr + 2 * kTile * D, s, hf);
                ax = mfma_split(Ak, Akl, shi[s], slo[s], ax);
                ay = mfma_split(Aq, Aql, shi[s], slo[s], ay);
            } else {
                ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, shi[s], ax, 0, 0, 0);
                ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, slo[s], ax, 0, 0, 0);
                ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, shi[s], ay, 0, 0, 0);
                ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, slo[s], ay, 0, 0, 0);
            }
        }
        f32x16 rr, oo;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r / 4) + 4 * hf + (r % 4);
            const float4 gabd = L.gabd[min(i, n - 1)];
            rr[r] = i < n ? fmaf(-gabd.y, ax[r], gabd.z * in2f(vraw[r])) : 0.0f;
            oo[r] = i < n ? gabd.x * ay[r] : 0.0f;
        }
        __syncthreads();
        // O += MT R: k-step s pairs the nodes held in accumulator slot s by the two half-waves
        const float *mrow = L.mt + l32 * kTile;
#pragma unroll
        for (int s = 0; s < 16; ++s)
            oo = __builtin_amdgcn_mfma_f32_32x32x2f32(mrow[8 * (s / 4) + 4 * hf + (s % 4)], rr[s], oo, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r / 4) + 4 * hf + (r % 4);
            if (i < n) out_base[(size_t)i * out_stride] = oo[r];
        }
        return;
    }

    // ---- multi-block trees: r rows through LDS, output on VALU
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t * kTile < n) {
            if (t > 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = t * kTile + 8 * (r / 4) + 4 * hf + (r % 4);
                    vraw[r] = i < n ? vb[(size_t)i * v_stride] : InT<F32>(0);
                }
            }
            const int pi = t * kTile + l32;
            f32x16 ax = {};
#pragma unroll
            for (int s = 0; s < VG<D>::KS; ++s) {
                if constexpr (F32) {
                    bf16x8 Ak = zero_frag(), Akl = zero_frag();
                    if (pi < n) frag_split(kb + (size_t)pi * kq_stride, s, hf, Ak, Akl);
                    ax = mfma_split(Ak, Akl, shi[s], slo[s], ax);
                } else {
                    const bf16x8 Ak = pi < n ? frag_of(kb + (size_t)pi * kq_stride, s, hf) : zero_frag();
                    ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, shi[s], ax, 0, 0, 0);
                    ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, slo[s], ax, 0, 0, 0);
                }
            }
            // the gates of the lane's 16 nodes are read before any r row is written (a read under
            // the store's branch would wait for its data once per node)
            float gy[16], gz[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float4 gabd = L.gabd[min(t * kTile + 8 * (r / 4) + 4 * hf + (r % 4), n - 1)];
                gy[r] = gabd.y;
                gz[r] = gabd.z;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = t * kTile + 8 * (r / 4) + 4 * hf + (r % 4);
                const float rv = fmaf(-gy[r], ax[r], gz[r] * in2f(vraw[r]));
                if (i < n) L.rbuf[(size_t)i * D + row] = rv;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t * kTile < n) {
            const int pi = t * kTile + l32;
            f32x16 ay = {};
#pragma unroll
            for (int s = 0; s < VG<D>::KS; ++s) {
                if constexpr (F32) {
                    bf16x8 Aq = zero_frag(), Aql = zero_frag();
                    if (pi < n) frag_split(qb + (size_t)pi * kq_stride, s, hf, Aq, Aql);
                    ay = mfma_split(Aq, Aql, shi[s], slo[s], ay);
                } else {
                    const bf16x8 Aq = pi < n ? frag_of(qb + (size_t)pi * kq_stride, s, hf) : zero_frag();
                    ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, shi[s], ay, 0, 0, 0);
                    ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, slo[s], ay, 0, 0, 0);
                }
            }
            // 16 nodes per lane; weights are zero past each node's depth
            float o[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = min(t * kTile + 8 * (r / 4) + 4 * hf + (r % 4), n - 1);
                o[r] = L.gabd[i].x * ay[r];
            }
#pragma unroll 1
            for (int e = 0; e < kPath; ++e) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = min(t * kTile + 8 * (r / 4) + 4 * hf + (r % 4), n - 1);
                    o[r] = fmaf(L.y[i * kPath + e], L.rbuf[(size_t)L.anc[i * kPath + e] * D + row], o[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = t * kTile + 8 * (r / 4) + 4 * hf + (r % 4);
                if (i < n) out_base[(size_t)i * out_stride] = o[r];
            }
        }
    }
}

// ===========================================================================
// Verify for trees of at most 32 nodes: one workgroup per (sequence, group of
// HPW value heads of one key head), D/32 waves; HPW is all of the key head's
// value heads, or one when a small batch leaves room for a workgroup per head.
// One round trip brings the keys, queries, values, gates and paths into LDS.
// Then wave 0 alone forms the coefficients once for all the heads (the Gram
// entries are shared through the key head), with no barrier inside that phase,
// while the other waves issue their first two heads' states; wave 0 issues its
// own after one barrier that publishes the output operator.  Each head's
// products are taken as its state lands, and a register set takes the next
// head's state as soon as its products are done.  Same algebra as the
// two-kernel path (coef_kernel + verify_kernel).
// ===========================================================================
constexpr int kGroupMaxHeads = 4;  // value heads per key head this kernel takes

// LDS row strides padded so that lanes walking consecutive rows hit distinct banks.
template <int D>
struct GPad {
    static constexpr int KQ = D + 8;       // bf16 per key/query row
    static constexpr int PS = kPath + 1;   // per-node path tables
    static constexpr int MT = kTile + 8;   // output-operator rows, bf16 (80 bytes: conflict-free 8-byte reads)
};

template <int D>
struct GTab {
    uint16_t *kq;     // [2][32][KQ] keys / queries (bf16); fp32 inputs: their hi parts, then [2][32][KQ] lo parts
    uint16_t *v;      // [32][grp][D] values of the group's heads (bf16), node-major as in memory;
                      // fp32 values are not staged (each head reads its own from memory)
    float4 *gab;      // [grp][32] gamma, alpha, b
    uint16_t *mth, *mtl;  // [grp][32][MT] dense output operator, bf16 hi and lo parts
    float *coefL;     // [grp][32][PS]
    float *gk, *gq;   // [32][PS] path-indexed Gram entries
    int *anc;         // [32][PS] root-to-node path, -1 past the depth
    float *a, *b;     // [grp][32]
    int *depth;       // [32]
};

template <int D>
__host__ __device__ inline size_t gtab_bytes(int grp, bool f32 = false) {
    using Q = GPad<D>;
    const size_t vb = f32 ? 0 : (size_t)kTile * grp * D * 2;  // fp32 keys/queries take two bf16 rows each
    return (size_t)(f32 ? 4 : 2) * kTile * Q::KQ * 2 + vb + (size_t)grp * kTile * 16 +
           (size_t)grp * kTile * Q::MT * 4 + (size_t)grp * kTile * Q::PS * 4 + 3 * kTile * Q::PS * 4 +
           2 * (size_t)grp * kTile * 4 + kTile * 4;
}

template <int D>
__device__ inline GTab<D> gtab_carve(char *base, int grp, bool f32 = false) {
    using Q = GPad<D>;
    GTab<D> L;
    L.kq = reinterpret_cast<uint16_t *>(base);     base += (size_t)(f32 ? 4 : 2) * kTile * Q::KQ * 2;
    L.v = reinterpret_cast<uint16_t *>(base);      base += f32 ? 0 : (size_t)kTile * grp * D * 2;
    L.gab = reinterpret_cast<float4 *>(base);      base += (size_t)grp * kTile * 16;
    L.mth = reinterpret_cast<uint16_t *>(base);    base += (size_t)grp * kTile * Q::MT * 2;
    L.mtl = reinterpret_cast<uint16_t *>(base);    base += (size_t)grp * kTile * Q::MT * 2;
    L.coefL = reinterpret_cast<float *>(base);     base += (size_t)grp * kTile * Q::PS * 4;
    L.gk = reinterpret_cast<float *>(base);        base += kTile * Q::PS * 4;
    L.gq = reinterpret_cast<float *>(base);        base += kTile * Q::PS * 4;
    L.anc = reinterpret_cast<int *>(base);         base += kTile * Q::PS * 4;
    L.a = reinterpret_cast<float *>(base);         base += (size_t)grp * kTile * 4;
    L.b = reinterpret_cast<float *>(base);         base += (size_t)grp * kTile * 4;
    L.depth = reinterpret_cast<int *>(base);
    return L;
}

// Loads lane's state fragments: uniform head base + one 32-bit lane offset, so
// the 2*KS loads share a single address register.
template <int D>
__device__ __forceinline__ void load_state_frags(const float *head, unsigned lane_off, float (&sf)[VG<D>::KS][8]) {
    const float *p = head + lane_off;
#pragma unroll
    for (int s = 0; s < VG<D>::KS; ++s) {
        const float4 x0 = *reinterpret_cast<const float4 *>(p + 16 * s);
        const float4 x1 = *reinterpret_cast<const float4 *>(p + 16 * s + 4);
        sf[s][0] = x0.x; sf[s][1] = x0.y; sf[s][2] = x0.z; sf[s][3] = x0.w;
        sf[s][4] = x1.x; sf[s][5] = x1.y; sf[s][6] = x1.z; sf[s][7] = x1.w;
    }
}

// The group verify's coefficient phase, run by one wave (lanes `lane`, halves `hf`,
// rows `l32`) on tables already in LDS: the Gram entries k.k and k.q of the block
// scattered into path order, then per (value head, node) pair the ratios, the
// coefficients and the back substitution that gives the output operator's rows
// (bf16 hi + lo) and the gates gamma, alpha, b.
template <int D, bool F32, int GRP>
__device__ __forceinline__ void group_coefficients(const GTab<D> &L, int n, int lane, int hf, int l32) {
    constexpr int KS = VG<D>::KS;
    constexpr int grp = GRP;
    using Q = GPad<D>;
    // Gram entries of the block: k . k, then k . q
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const int bro = which == 0 ? 0 : kTile;  // B operand rows: the keys or the queries
        f32x16 gacc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 A = frag_of(L.kq + l32 * Q::KQ, s, hf);
            const bf16x8 B = frag_of(L.kq + (bro + l32) * Q::KQ, s, hf);
            if constexpr (F32) {
                const bf16x8 Al = frag_of(L.kq + (2 * kTile + l32) * Q::KQ, s, hf);
                const bf16x8 Bl = frag_of(L.kq + (2 * kTile + bro + l32) * Q::KQ, s, hf);
                gacc = mfma_split(A, Al, B, Bl, gacc);
            } else {
                gacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, gacc, 0, 0, 0);
            }
        }
        if (l32 < n) {  // accumulator r: (candidate ancestor il, node l32)
            // ancestors of node l32 within the block: its path entries (-1 past its depth),
            // all read before any is tested, so no read waits under a branch
            int anl[kPath];
#pragma unroll
            for (int e = 0; e < kPath; ++e) anl[e] = L.anc[l32 * Q::PS + e];
            uint32_t mask = 0u;
#pragma unroll
            for (int e = 0; e < kPath; ++e) mask |= anl[e] >= 0 ? 1u << (anl[e] & 31) : 0u;
            float *gdst = (which == 0 ? L.gk : L.gq) + l32 * Q::PS;
            // the candidates' depths four at a time, all read before any write; a candidate
            // that is not an ancestor writes to the row's pad column, which nothing reads
            int4 dq[4];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                dq[g4] = *reinterpret_cast<const int4 *>(L.depth + 8 * g4 + 4 * hf);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int il = 8 * (r / 4) + 4 * hf + (r % 4);
                const int4 q4 = dq[r / 4];
                const int dep = r % 4 == 0 ? q4.x : r % 4 == 1 ? q4.y : r % 4 == 2 ? q4.z : q4.w;
                gdst[((mask >> il) & 1u) ? dep - 1 : kPath] = gacc[r];
            }
        }
    }
    // one wave's LDS accesses take effect in program order: only the compiler must keep them
    __builtin_amdgcn_wave_barrier();

    // per (value head, node) pair, lane (and lane + 64 for more than two heads): ratios,
    // coefficients, output weights
    constexpr int RND = (GRP * kTile + 63) / 64;  // rounds of 64 (head, node) pairs
    float mrow[RND][kPath];
    int an_t[RND][kPath];
    int d_t[RND], hh_t[RND], i_t[RND];
    bool act[RND];
#pragma unroll
    for (int rd = 0; rd < RND; ++rd) {
        const int pr = lane + 64 * rd;
        act[rd] = pr < grp * n;
        hh_t[rd] = act[rd] ? pr / n : 0;
        i_t[rd] = act[rd] ? pr % n : 0;
        d_t[rd] = 0;
        if (act[rd]) {
            const int hh = hh_t[rd], i = i_t[rd];
            const int di = L.depth[i];
            d_t[rd] = di;
            const float bi = L.b[hh * kTile + i];
            // every table entry of the row, read before the first result is written (the
            // writes would otherwise order each step's reads behind the previous step's)
            float av[kPath], gk[kPath], gq[kPath];
#pragma unroll
            for (int e = 0; e < kPath; ++e) an_t[rd][e] = max(L.anc[i * Q::PS + e], 0);
#pragma unroll
            for (int e = 0; e < kPath; ++e) {
                const float ae = L.a[hh * kTile + an_t[rd][e]];
                av[e] = e < di ? ae : 1.0f;
                gk[e] = L.gk[i * Q::PS + e];
                gq[e] = L.gq[i * Q::PS + e];
            }
            float r = 1.0f;
#pragma unroll
            for (int e = kPath - 1; e >= 0; --e) {
                const bool on = e < di - 1;
                L.coefL[(hh * kTile + i) * Q::PS + e] = on ? bi * r * gk[e] : 0.0f;
                mrow[rd][e] = on ? r * gq[e] : (e == di - 1 ? gq[e] : 0.0f);
                r *= av[e];
            }
            L.gab[hh * kTile + i] = make_float4(r, bi * r, bi, 0.0f);
        }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int rd = 0; rd < RND; ++rd) {
        if (act[rd]) {
            const int hh = hh_t[rd], i = i_t[rd];
            float y[kPath];
#pragma unroll
            for (int e = kPath - 1; e >= 0; --e) {
                float acc = mrow[rd][e];
                // deepest terms first: y_{e+1}, the last one known, enters last
#pragma unroll
                for (int f = kPath - 1; f > e; --f)
                    acc = fmaf(-y[f], L.coefL[(hh * kTile + an_t[rd][f]) * Q::PS + e], acc);
                y[e] = e < d_t[rd] ? acc : 0.0f;
            }
            uint16_t *mh = L.mth + (hh * kTile + i) * Q::MT, *ml = L.mtl + (hh * kTile + i) * Q::MT;
#pragma unroll
            for (int e = 0; e < kPath; ++e)
                if (e < d_t[rd]) {  // stored as bf16 hi + lo for the matrix cores
                    const __bf16 yh = static_cast<__bf16>(y[e]);
                    mh[an_t[rd][e]] = __builtin_bit_cast(uint16_t, yh);
                    ml[an_t[rd][e]] =
                        __builtin_bit_cast(uint16_t, static_cast<__bf16>(y[e] - static_cast<float>(yh)));
                }
        }
    }
}

template <int D, bool CHAIN, int HPW, bool F32>
__global__ __launch_bounds__(VG<D>::THREADS) __attribute__((amdgpu_waves_per_eu(HPW == 1 ? 3 : 2))) void
verify_group_kernel(Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    constexpr int KS = VG<D>::KS, NT = VG<D>::THREADS;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int row = w * 32 + l32;
    constexpr int grp = HPW;  // value heads of this workgroup, all reading one key head
    const int nhg = P.Hv / grp;
    const int b = blockIdx.x / nhg, h0 = blockIdx.x % nhg * grp;
    const int g = h0 / (P.Hv / P.Hk);
    const SeqView sv = seq_view<CHAIN>(P, b);
    const bool planned = CHAIN || ws_plan_matches(P);
    const int lo = sv.lo, n = sv.n;
    // out[node][h0 + hh][row]: uniform base per (node, head) + this lane's offset
    const unsigned out_lane = (unsigned)(4 * hf * P.Hv * D + row);
    // a planned tree's common case is tested on the plan check and the sequence's record
    // at once, so the two loads are issued together
    if (CHAIN || !(planned & (sv.status == GDN_SEQ_OK) & (n > 0) & (P.out != nullptr))) {
        if (!planned) return;
        if (CHAIN && P.has_ws && h0 == 0 && tid == 0) {
            if (b == 0) {
                P.ws.header[0] = kChainMagic;
                P.ws.header[1] = P.B;
                P.ws.header[2] = P.T;
                P.ws.header[kHdrMisuse] = 0;
            }
            P.ws.seq_status[b] = sv.status;
        }
        if (!P.out) return;
        if (sv.status != GDN_SEQ_OK) {
            for (int t = tid; t < n * grp * D; t += NT)
                P.out[((size_t)(lo + t / (grp * D)) * P.Hv + h0) * D + t % (grp * D)] = qnan_f();
            return;
        }
        if (n == 0) return;
    }
    using Q = GPad<D>;
    const GTab<D> L = gtab_carve<D>(lds_raw, grp, F32);
    const InT<F32> *kb = static_cast<const InT<F32> *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const InT<F32> *qb = static_cast<const InT<F32> *>(P.q) + ((size_t)lo * P.Hk + g) * D;
    const size_t kq_stride = (size_t)P.Hk * D;
    const float *s0 = P.state_in + ((size_t)sv.slot * P.Hv + h0) * D * D;
    const unsigned s_lane = (unsigned)(row * D + 8 * hf);

    // ---- one round trip: keys/queries, all heads' values, tree, gates (16-byte chunks:
    // 8 bf16 or 4 fp32 values)
    constexpr int EPC = F32 ? 4 : 8;  // values per 16-byte chunk
    constexpr int KQ_PER = (2 * kTile * D / EPC + NT - 1) / NT;
    uint4 kqv[KQ_PER];
#pragma unroll
    for (int u = 0; u < KQ_PER; ++u) {
        const int idx = tid + u * NT;
        const int which = idx / (kTile * (D / EPC)), rem = idx % (kTile * (D / EPC));
        const int i = rem / (D / EPC), c8 = rem % (D / EPC);
        kqv[u] = (which < 2 && i < n)
                     ? *reinterpret_cast<const uint4 *>((which ? qb : kb) + (size_t)i * kq_stride + EPC * c8)
                     : make_uint4(0, 0, 0, 0);
    }
    // values: node i's group heads are contiguous (grp*D values)
    const InT<F32> *vg = static_cast<const InT<F32> *>(P.v) + ((size_t)lo * P.Hv + h0) * D;
    const int vchunks = grp * D / EPC;  // 16-byte chunks per node
    // bf16 values are staged; fp32 values are read per head as it runs
    constexpr int V_PER = F32 ? 0 : (kGroupMaxHeads * kTile * D / 8 + NT - 1) / NT;
    static_assert(kGroupMaxHeads * kTile <= NT, "one thread per (head, node) gate");
    uint4 vv[V_PER > 0 ? V_PER : 1];
#pragma unroll
    for (int u = 0; u < V_PER; ++u) {
        const int idx = tid + u * NT;
        const int i = idx / vchunks, c = idx % vchunks;
        vv[u] = i < n ? *reinterpret_cast<const uint4 *>(vg + (size_t)i * P.Hv * D + EPC * c) : make_uint4(0, 0, 0, 0);
    }
    float ga = 0.0f, gb = 0.0f;  // gates of (head tid / n, node tid % n); grp * n <= NT
    if (tid < grp * n) {
        const size_t at = (size_t)(lo + tid % n) * P.Hv + h0 + tid / n;
        ga = P.a[at];
        gb = P.b[at];
    }
    // the path rows last: whatever waits on them waits on the loads above as well
    int an[kPath], d = 0;  // path entries, -1 past the depth
    if (tid < n) {
        d = CHAIN ? tid + 1 : P.ws.depth[lo + tid];
#pragma unroll
        for (int e = 0; e < kPath; ++e)
            an[e] = CHAIN ? (e <= tid ? e : -1) : P.ws.nodepath[(size_t)(lo + tid) * GDN_MAX_DEPTH + e];
    }
    if (tid < n) {  // stored as loaded: no arithmetic on them before the states are out
#pragma unroll
        for (int e = 0; e < kPath; ++e) L.anc[tid * Q::PS + e] = an[e];
        L.depth[tid] = d;
    }
    if (tid < grp * n) {
        L.a[(tid / n) * kTile + tid % n] = ga;
        L.b[(tid / n) * kTile + tid % n] = gb;
    }
#pragma unroll
    for (int u = 0; u < KQ_PER; ++u) {
        const int idx = tid + u * NT;
        if (idx < 2 * kTile * (D / EPC)) {
            if constexpr (F32) {  // hi rows as the bf16 layout, lo rows 2*32 rows further
                uint2 hi, lo2;
                split4(__builtin_bit_cast(float4, kqv[u]), hi, lo2);
                uint16_t *dst = L.kq + (idx / (D / 4)) * Q::KQ + 4 * (idx % (D / 4));
                *reinterpret_cast<uint2 *>(dst) = hi;
                *reinterpret_cast<uint2 *>(dst + 2 * kTile * Q::KQ) = lo2;
            } else {
                *reinterpret_cast<uint4 *>(L.kq + (idx / (D / 8)) * Q::KQ + 8 * (idx % (D / 8))) = kqv[u];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < V_PER; ++u) {
        const int idx = tid + u * NT;
        if (idx < kTile * vchunks) reinterpret_cast<uint4 *>(L.v)[idx] = vv[u];
    }
    for (int idx = tid; idx < grp * kTile * Q::MT / 2; idx += NT) {
        reinterpret_cast<uint32_t *>(L.mth)[idx] = 0u;
        reinterpret_cast<uint32_t *>(L.mtl)[idx] = 0u;
    }
    float sA[KS][8], sB[KS][8];
    __syncthreads();  // the tables are in LDS

    // ---- the coefficient phase runs on wave 0 alone, with no barrier inside it, while the
    // other waves issue their first two heads' states.  A wave that issues loads into a
    // saturated memory system stalls until they are taken; with a barrier inside the phase
    // every such stall would hold back the coefficients, which gate every output.  Wave 0
    // issues its own states once the phase is done.
    if (uni(w) == 0) {
        group_coefficients<D, F32, grp>(L, n, lane, hf, l32);
    } else {
        load_state_frags<D>(s0, s_lane, sA);
        if (grp > 1) load_state_frags<D>(s0 + (size_t)D * D, s_lane, sB);
    }
    __syncthreads();  // the output operator and the gates are in LDS
    if (uni(w) == 0) {
        load_state_frags<D>(s0, s_lane, sA);
        if (grp > 1) load_state_frags<D>(s0 + (size_t)D * D, s_lane, sB);
    }

    // ---- value heads: X, Y from the state and K/Q; outputs from X, Y and the coefficients
    // fp32 values of head hh at this lane's row for the 16 nodes of its accumulator slots,
    // through a buffer resource over the sequence's value rows: past the last node the
    // hardware returns zero, so no load is guarded
    auto load_vf = [&](int hh, float (&vf)[16]) {
        if constexpr (F32) {
            const __amdgpu_buffer_rsrc_t rv =
                buffer_rsrc(reinterpret_cast<const float *>(vg) + (size_t)hh * D, (unsigned)(n * P.Hv * D) * 4u);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r / 4) + 4 * hf + (r % 4);
                vf[r] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rv, (unsigned)(i * P.Hv * D + row) * 4u, 0, 0));
            }
        }
    };
    auto xy = [&](const float (&st)[KS][8], f32x16 &ax, f32x16 &ay) {
        ax = f32x16{};
        ay = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {  // the state as bf16 hi + lo, split one k-step at a time
            bf16x8 shi, slo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 hb = static_cast<__bf16>(st[s][e]);
                shi[e] = hb;
                slo[e] = static_cast<__bf16>(st[s][e] - static_cast<float>(hb));
            }
            const bf16x8 Ak = frag_of(L.kq + l32 * Q::KQ, s, hf);
            const bf16x8 Aq = frag_of(L.kq + (kTile + l32) * Q::KQ, s, hf);
            if constexpr (F32) {
                const bf16x8 Akl = frag_of(L.kq + (2 * kTile + l32) * Q::KQ, s, hf);
                const bf16x8 Aql = frag_of(L.kq + (3 * kTile + l32) * Q::KQ, s, hf);
                ax = mfma_split(Ak, Akl, shi, slo, ax);
                ay = mfma_split(Aq, Aql, shi, slo, ay);
            } else {
                ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, shi, ax, 0, 0, 0);
                ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, slo, ax, 0, 0, 0);
                ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, shi, ay, 0, 0, 0);
                ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, slo, ay, 0, 0, 0);
            }
        }
    };
    auto finish = [&](f32x16 ax, f32x16 ay, int hh, const float (&vf)[16]) {
        const float4 *gab = L.gab + hh * kTile;
        const uint16_t *vh = L.v + hh * D + row;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r / 4) + 4 * hf + (r % 4);
            const float4 q4 = gab[min(i, n - 1)];
            const float vi = F32 ? vf[r] : bf2f(vh[i * grp * D]);
            ax[r] = i < n ? fmaf(-q4.y, ax[r], q4.z * vi) : 0.0f;  // r = b v - alpha x
            ay[r] = i < n ? q4.x * ay[r] : 0.0f;                   // gamma y
        }
        // O = gamma y + MT R on bf16 MFMA with both operands split hi + lo (the lo x lo
        // term is dropped: each lo is at most 2^-8 of its value, so the term is up to
        // ~2^-16 of the product, the order of the state's own split).  k-step u takes R from accumulator slots
        // 8u .. 8u+7, i.e. nodes 16u + 8(e/4) + 4*half + e%4, and MT's columns in that order.
        const uint16_t *mh = L.mth + (hh * kTile + l32) * Q::MT, *ml = L.mtl + (hh * kTile + l32) * Q::MT;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint2 h0 = *reinterpret_cast<const uint2 *>(mh + 16 * u + 4 * hf);
            const uint2 h1 = *reinterpret_cast<const uint2 *>(mh + 16 * u + 8 + 4 * hf);
            const uint2 l0 = *reinterpret_cast<const uint2 *>(ml + 16 * u + 4 * hf);
            const uint2 l1 = *reinterpret_cast<const uint2 *>(ml + 16 * u + 8 + 4 * hf);
            const bf16x8 ahi = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
            const bf16x8 alo = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
            bf16x8 bhi, blo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float rv = ax[8 * u + e];
                const __bf16 rb = static_cast<__bf16>(rv);
                bhi[e] = rb;
                blo[e] = static_cast<__bf16>(rv - static_cast<float>(rb));
            }
            ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bhi, ay, 0, 0, 0);
            ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, blo, ay, 0, 0, 0);
            ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bhi, ay, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ir = 8 * (r / 4) + (r % 4);  // node of half-wave 0; half-wave 1 adds 4
            if (ir + 4 * hf < n) {
                float *ob = P.out + ((size_t)(lo + ir) * P.Hv + h0 + hh) * D;
                ob[out_lane] = ay[r];
            }
        }
    };
    // each register set is refilled as soon as its products are taken
    float vf[16];  // fp32 inputs: the running head's values
    f32x16 x0, y0;
    load_vf(0, vf);
    xy(sA, x0, y0);
    finish(x0, y0, 0, vf);
    if (grp > 2) load_state_frags<D>(s0 + (size_t)2 * D * D, s_lane, sA);
    if (grp > 1) {
        f32x16 x1, y1;
        load_vf(1, vf);
        xy(sB, x1, y1);
        finish(x1, y1, 1, vf);
        if (grp > 3) load_state_frags<D>(s0 + (size_t)3 * D * D, s_lane, sB);
    }
    if (grp > 2) {
        f32x16 x2, y2;
        load_vf(2, vf);
        xy(sA, x2, y2);
        finish(x2, y2, 2, vf);
    }
    if (grp > 3) {
        f32x16 x3, y3;
        load_vf(3, vf);
        xy(sB, x3, y3);
        finish(x3, y3, 3, vf);
    }
}

// ===========================================================================
// Verify for trees of 33 .. 96 nodes: NB node blocks of 32, one workgroup per
// (sequence, group of GRP value heads of one key head: all of them, or one for a
// small batch).  The Gram entries k.k and k.q of every block pair and the
// per-(head, node) coefficients are formed once; ancestors may sit in any block,
// so each head takes Y_t = Q_t S0^T and X_j = K_j S0^T for all blocks, then
// R_j = diag(b)V_j - diag(alpha)X_j and O_t = diag(gamma)Y_t + sum_j MT_tj R_j
// with MT (the output operator, rows from the 16-step back substitution) dense
// in LDS: cleared once, its entries (the same places, the ancestors, for every
// head) rewritten per head.  All products run on bf16 MFMA with fp32 operands
// split hi + lo.  LDS and registers are kept small enough that two workgroups
// share a CU (a 65-node tree: 79 KB, at most 256 registers), so one's table,
// Gram and coefficient phases run under the other's state stream:
//  - keys and queries are staged for the tree's own nodes only (max_nodes rows;
//    rows past the last node enter the products as zero fragments);
//  - the values are read from memory into registers per head, not staged;
//  - the dense output operator has max_nodes rows and as many columns, rounded
//    up to the 16 of one k-step, and shares its LDS with the Gram entries,
//    coefficients and gates, which are dead once the path weights are formed;
//  - one state register set: the first head's state streams in under the
//    coefficients and back substitution, each later head's is issued with its
//    values right after that head's operator entries are written (the other
//    workgroup on the CU keeps the memory system busy meanwhile);
//  - k-steps and node blocks past the last node are skipped.
// ===========================================================================
template <int D>
struct BPad {
    static constexpr int KQ = D + 8;      // bf16 per key/query row
    static constexpr int PS = kPath + 1;  // per-node path tables
};

struct BLayout {
    size_t kq, gab, ysp, anc, depth, gk, gq, coefL, a, b, mth, mtl, total;
    int ms;  // bf16 per output-operator row
};

template <int D>
__host__ __device__ inline BLayout blocks_layout(int cap, int grp) {
    using Q = BPad<D>;
    const size_t c = (size_t)cap;
    BLayout L;
    L.ms = (cap + 15) / 16 * 16 + 8;
    size_t off = 0;
    L.kq = off;    off += 2 * c * Q::KQ * 2;
    L.gab = off;   off += (size_t)grp * c * 16;
    L.ysp = off;   off += (size_t)grp * c * kPath * 4;
    L.anc = off;   off += c * Q::PS * 4;
    off = (off + 15) & ~size_t(15);
    L.depth = off; off += (c + kTile - 1) / kTile * kTile * 4;  // whole node blocks, read four at a time
    off = (off + 15) & ~size_t(15);
    // the coefficient phase's tables and the output operator share one region
    L.gk = off;
    L.gq = L.gk + c * Q::PS * 4;
    L.coefL = L.gq + c * Q::PS * 4;
    L.a = L.coefL + (size_t)grp * c * Q::PS * 4;
    L.b = L.a + (size_t)grp * c * 4;
    const size_t u1 = L.b + (size_t)grp * c * 4 - off;
    L.mth = off;
    L.mtl = L.mth + c * L.ms * 2;
    const size_t u2 = 2 * c * L.ms * 2;
    off += u1 > u2 ? u1 : u2;
    L.total = off;
    return L;
}

template <int D, int NB, int GRP>
__global__ __launch_bounds__(VG<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2))) void verify_blocks_kernel(
    Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    using Q = BPad<D>;
    constexpr int KS = VG<D>::KS, NT = VG<D>::THREADS, WAVES = VG<D>::WAVES, NN = NB * kTile;
    constexpr int grp = GRP;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int row = w * 32 + l32;
    const int nhg = P.Hv / grp;  // workgroups per sequence
    const int b = blockIdx.x / nhg, h0 = blockIdx.x % nhg * grp;
    const int g = h0 / (P.Hv / P.Hk);
    const SeqView sv = seq_view<false>(P, b);
    if (!ws_plan_matches(P)) return;
    const int lo = sv.lo, n = sv.n;
    if (sv.status != GDN_SEQ_OK) {
        for (int t = tid; t < n * grp * D; t += NT)
            P.out[((size_t)(lo + t / (grp * D)) * P.Hv + h0) * D + t % (grp * D)] = qnan_f();
        return;
    }
    if (n == 0) return;
    // n <= max_nodes <= NN: the plan rejects longer sequences, and its max_nodes is ours
    const int cap = P.max_nodes;
    const int nb = (n + kTile - 1) / kTile;  // node blocks in use
    const BLayout SL = blocks_layout<D>(cap, grp);
    uint16_t *const Lkq = reinterpret_cast<uint16_t *>(lds_raw + SL.kq);
    float4 *const Lgab = reinterpret_cast<float4 *>(lds_raw + SL.gab);
    float *const Lysp = reinterpret_cast<float *>(lds_raw + SL.ysp);
    int *const Lanc = reinterpret_cast<int *>(lds_raw + SL.anc);
    int *const Ldepth = reinterpret_cast<int *>(lds_raw + SL.depth);
    float *const Lgk = reinterpret_cast<float *>(lds_raw + SL.gk);
    float *const Lgq = reinterpret_cast<float *>(lds_raw + SL.gq);
    float *const LcoefL = reinterpret_cast<float *>(lds_raw + SL.coefL);
    float *const La = reinterpret_cast<float *>(lds_raw + SL.a);
    float *const Lb = reinterpret_cast<float *>(lds_raw + SL.b);
    uint16_t *const Lmth = reinterpret_cast<uint16_t *>(lds_raw + SL.mth);
    uint16_t *const Lmtl = reinterpret_cast<uint16_t *>(lds_raw + SL.mtl);
    const int MS = SL.ms;
    const uint16_t *kb = static_cast<const uint16_t *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const uint16_t *qb = static_cast<const uint16_t *>(P.q) + ((size_t)lo * P.Hk + g) * D;
    const size_t kq_stride = (size_t)P.Hk * D;
    const float *s0 = P.state_in + ((size_t)sv.slot * P.Hv + h0) * D * D;
    // out[node][h0 + hh][row] and v[node][h0 + hh][row]: a uniform base per (node, head)
    // plus this lane's offset
    const unsigned out_lane = (unsigned)(4 * hf * P.Hv * D + row);
    const unsigned s_lane = (unsigned)(row * D + 8 * hf);
    const uint16_t *vb = static_cast<const uint16_t *>(P.v) + ((size_t)lo * P.Hv + h0) * D;
    const int hvd = P.Hv * D;  // elements between consecutive nodes' rows of out and v

    // ---- one round trip: keys/queries of the tree's nodes, gates, paths
    constexpr int KQ_PER = 2 * NN * (D / 8) / NT;
    static_assert(2 * NN * (D / 8) % NT == 0, "whole key/query rounds");
    uint4 kqv[KQ_PER];
#pragma unroll
    for (int u = 0; u < KQ_PER; ++u) {
        const int idx = tid + u * NT;
        const int which = idx / (NN * (D / 8)), rem = idx % (NN * (D / 8));
        const int i = rem / (D / 8), c8 = rem % (D / 8);
        kqv[u] = i < n ? *reinterpret_cast<const uint4 *>((which ? qb : kb) + (size_t)i * kq_stride + 8 * c8)
                       : make_uint4(0, 0, 0, 0);
    }
    constexpr int GA_PER = (GRP * NN + NT - 1) / NT;
    float ga[GA_PER], gb[GA_PER];
#pragma unroll
    for (int u = 0; u < GA_PER; ++u) {
        const int t = tid + u * NT;
        ga[u] = 1.0f;
        gb[u] = 0.0f;
        if (t < grp * n) {
            const size_t at = (size_t)(lo + t % n) * P.Hv + h0 + t / n;
            ga[u] = P.a[at];
            gb[u] = P.b[at];
        }
    }
    static_assert(NN <= NT, "one thread per node");
    int4 an4[kPath / 4];
    int d = 0;
    if (tid < n) {
        d = P.ws.depth[lo + tid];
        const int4 *np = reinterpret_cast<const int4 *>(P.ws.nodepath + (size_t)(lo + tid) * GDN_MAX_DEPTH);
#pragma unroll
        for (int e = 0; e < kPath / 4; ++e) an4[e] = np[e];
    }
    if (tid < n) {
#pragma unroll
        for (int e = 0; e < kPath / 4; ++e) {
            Lanc[tid * Q::PS + 4 * e + 0] = an4[e].x;
            Lanc[tid * Q::PS + 4 * e + 1] = an4[e].y;
            Lanc[tid * Q::PS + 4 * e + 2] = an4[e].z;
            Lanc[tid * Q::PS + 4 * e + 3] = an4[e].w;
        }
        Ldepth[tid] = d;
    }
#pragma unroll
    for (int u = 0; u < GA_PER; ++u) {
        const int t = tid + u * NT;
        if (t < grp * n) {
            La[(t / n) * cap + t % n] = ga[u];
            Lb[(t / n) * cap + t % n] = gb[u];
        }
    }
#pragma unroll
    for (int u = 0; u < KQ_PER; ++u) {
        const int idx = tid + u * NT;
        const int which = idx / (NN * (D / 8)), rem = idx % (NN * (D / 8));
        const int i = rem / (D / 8), c8 = rem % (D / 8);
        if (i < n) *reinterpret_cast<uint4 *>(Lkq + (which * cap + i) * Q::KQ + 8 * c8) = kqv[u];
    }
    float st[KS][8];
    // values of head hh in the R layout: block jb, accumulator slot r holds node
    // jb*32 + 8(r/4) + 4*half + r%4 at this lane's row; two bf16 per register.  Read
    // through a buffer resource over the sequence's nodes: past the last node the
    // hardware returns zero, so no load is clamped or guarded and all are in flight at once.
    uint32_t vv[NB][8];
    auto load_v = [&](int hh, int nn, unsigned lane_v) {
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vb + (size_t)hh * D, (unsigned)(nn * hvd) * 2u);
#pragma unroll
        for (int jb = 0; jb < NB; ++jb)
#pragma unroll
            for (int r2 = 0; r2 < 8; ++r2) {
                uint32_t x[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int ir = jb * kTile + 8 * (r2 / 2) + 2 * (r2 % 2) + q;  // node of half-wave 0
                    x[q] = __builtin_amdgcn_raw_buffer_load_b16(rv, (unsigned)(ir * hvd) * 2u + lane_v, 0, 0);
                }
                vv[jb][r2] = x[0] | (x[1] << 16);
            }
    };
    __syncthreads();

    // key / query fragments of node block jb, k-step s.  A row past the last node reads
    // the last node's row: what it produces lands only in accumulator rows of nodes that
    // do not exist, which are masked (R) or never stored (outputs, Gram entries).
    auto kfrag = [&](int jb, int s) { return frag_of(Lkq + min(jb * kTile + l32, n - 1) * Q::KQ, s, hf); };
    auto qfrag = [&](int jb, int s) {
        return frag_of(Lkq + (cap + min(jb * kTile + l32, n - 1)) * Q::KQ, s, hf);
    };

    // a wave with no Gram block (w >= nb) issues its first-head state now
    const bool early = w >= nb;
    if (early) load_state_frags<D>(s0, s_lane, st);
    // ---- Gram entries: wave w takes the nodes of block w (column block tj = w) against
    // every block ti; node j's ancestor i, at path position depth(i) - 1, gets k_i . k_j
    // and k_i . q_j.  The ancestors of j are a bit mask over node ids, so a candidate
    // needs no path lookup, and the nb products of a wave are independent MFMA chains.
    for (int tj = w; tj < nb; tj += WAVES) {
        const int j = tj * kTile + l32;
        uint32_t amask[NB];  // ancestors of node j (itself included), by block
#pragma unroll
        for (int t = 0; t < NB; ++t) amask[t] = 0u;
        if (j < n) {
            const int dj = Ldepth[j];
#pragma unroll
            for (int e = 0; e < kPath; ++e) {
                const int an = Lanc[j * Q::PS + e];
#pragma unroll
                for (int t = 0; t < NB; ++t)
                    if (e < dj && (an >> 5) == t) amask[t] |= 1u << (an & 31);
            }
        }
        f32x16 gkk[NB], gkq[NB];
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            gkk[t] = f32x16{};
            gkq[t] = f32x16{};
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 Bk = kfrag(tj, s);
            const bf16x8 Bq = qfrag(tj, s);
#pragma unroll
            for (int ti = 0; ti < NB; ++ti) {
                const bf16x8 A = kfrag(ti, s);
                gkk[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bk, gkk[ti], 0, 0, 0);
                gkq[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bq, gkq[ti], 0, 0, 0);
            }
        }
        if (j < n) {
#pragma unroll
            for (int ti = 0; ti < NB; ++ti) {
                if (ti < nb) {
                    // the depths of the lane's 16 candidates ti * 32 + il, four consecutive nodes
                    // per read, all read before any write; a candidate that is not an ancestor
                    // writes to the row's pad column, which nothing reads, so no write waits on a
                    // branch (past the last node the depths are never used)
                    int4 dq[4];
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        dq[g4] = *reinterpret_cast<const int4 *>(Ldepth + ti * kTile + 8 * g4 + 4 * hf);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int il = 8 * (r / 4) + 4 * hf + (r % 4);
                        const int4 q4 = dq[r / 4];
                        const int dep = r % 4 == 0 ? q4.x : r % 4 == 1 ? q4.y : r % 4 == 2 ? q4.z : q4.w;
                        const int e = ((amask[ti] >> il) & 1u) ? dep - 1 : kPath;
                        Lgk[j * Q::PS + e] = gkk[ti][r];
                        Lgq[j * Q::PS + e] = gkq[ti][r];
                    }
                }
            }
        }
    }
    __syncthreads();
    // the first head's state streams in under the coefficients and back substitution
    // (issued earlier, it would have to share the registers of the Gram products)
    if (!early) load_state_frags<D>(s0, s_lane, st);

    // ---- per (head, node): ratios, coefficients, the output weights' right-hand sides
#pragma unroll 1
    for (int t = tid; t < grp * n; t += NT) {
        const int hh = t / n, i = t % n;
        const int di = Ldepth[i];
        const float bi = Lb[hh * cap + i];
        // every table entry of the row, read before the first result is written (the writes
        // would otherwise order each step's reads behind the previous step's)
        float gk[kPath], gq[kPath], av[kPath];
#pragma unroll
        for (int e = 0; e < kPath; ++e) {
            gk[e] = Lgk[i * Q::PS + e];
            gq[e] = Lgq[i * Q::PS + e];
            av[e] = La[hh * cap + max(Lanc[i * Q::PS + e], 0)];
        }
        float r = 1.0f;
#pragma unroll
        for (int e = kPath - 1; e >= 0; --e) {
            const bool on = e < di - 1;
            LcoefL[(hh * cap + i) * Q::PS + e] = on ? bi * r * gk[e] : 0.0f;
            Lysp[(hh * cap + i) * kPath + e] = on ? r * gq[e] : (e == di - 1 ? gq[e] : 0.0f);
            if (e < di) r *= av[e];
        }
        Lgab[hh * cap + i] = make_float4(r, bi * r, bi, 0.0f);
    }
    __syncthreads();
    // back substitution, deepest weight first, in place
#pragma unroll 1
    for (int t = tid; t < grp * n; t += NT) {
        const int hh = t / n, i = t % n;
        const int di = Ldepth[i];
        int an_t[kPath];
#pragma unroll
        for (int e = 0; e < kPath; ++e) an_t[e] = max(Lanc[i * Q::PS + e], 0);
        float *yr = Lysp + (hh * cap + i) * kPath;
        float y[kPath];
#pragma unroll
        for (int e = kPath - 1; e >= 0; --e) {
            float acc = yr[e];
#pragma unroll
            for (int f = kPath - 1; f > e; --f) acc = fmaf(-y[f], LcoefL[(hh * cap + an_t[f]) * Q::PS + e], acc);
            y[e] = e < di ? acc : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < kPath; ++e) yr[e] = y[e];
    }
    __syncthreads();  // the coefficient tables are dead: their region becomes the output operator
    // every head's operator has its nonzeros at the same places (the ancestors), so clearing
    // once leaves each head's scatter a complete operator
    for (int c = tid; c < cap * MS / 8; c += NT) {
        reinterpret_cast<uint4 *>(Lmth)[c] = make_uint4(0u, 0u, 0u, 0u);
        reinterpret_cast<uint4 *>(Lmtl)[c] = make_uint4(0u, 0u, 0u, 0u);
    }

    // ---- value heads (unrolled: a loop would carry its values across heads and spill)
#pragma unroll
    for (int hh = 0; hh < grp; ++hh) {
        // the loop's own copies of the node count and the lane's output offset: what is
        // derived from them is recomputed per head instead of being hoisted out of the
        // loop and held (dozens of per-node indices and addresses) across it
        int n_h = n;
        unsigned lane_b = out_lane * 4u;  // byte offset of this lane's element in a (node, head) row
        int hf4 = 4 * hf, l32_h = l32;    // the lane's node offset within an accumulator slot, its row
        asm volatile("" : "+s"(n_h));
        asm volatile("" : "+v"(lane_b));
        asm volatile("" : "+v"(hf4));
        asm volatile("" : "+v"(l32_h));
        __syncthreads();  // the operator is cleared, or the previous head's products are done with it
        for (int t = tid; t < n_h * kPath; t += NT) {
            const int i = t / kPath, e = t % kPath;
            if (e < Ldepth[i]) {
                const int col = Lanc[i * Q::PS + e];
                const float y = Lysp[(hh * cap + i) * kPath + e];
                const __bf16 yh = static_cast<__bf16>(y);
                Lmth[i * MS + col] = __builtin_bit_cast(uint16_t, yh);
                Lmtl[i * MS + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(y - static_cast<float>(yh)));
            }
        }
        __syncthreads();
        // this head's values (its state is already in flight)
        load_v(hh, n_h, lane_b >> 1);
        // Y_t = Q_t S0^T and X_j = K_j S0^T for every block, one product at a time (NB
        // independent MFMA chains each), the state split into bf16 hi + lo one k-step at a
        // time (only the fp32 state is held); blocks past the last node multiply zeros
        auto state_products = [&](bool queries, f32x16 (&acc)[NB]) {
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) acc[jb] = f32x16{};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 shi, slo;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const __bf16 hb = static_cast<__bf16>(st[s][e]);
                    shi[e] = hb;
                    slo[e] = static_cast<__bf16>(st[s][e] - static_cast<float>(hb));
                }
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) {
                    const bf16x8 A = queries ? qfrag(jb, s) : kfrag(jb, s);
                    acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, shi, acc[jb], 0, 0, 0);
                    acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, slo, acc[jb], 0, 0, 0);
                }
            }
        };
        f32x16 Y[NB], X[NB];
        state_products(true, Y);
        state_products(false, X);
        // per accumulator slot (node i of block jb): gamma Y and R_j = b v - alpha X_j, the
        // latter as bf16 hi + lo in the k-order of the output products (k-step u of block j:
        // slots 8u .. 8u+7)
        const float4 *gab = Lgab + hh * cap;
        bf16x8 rhi[NB][2], rlo[NB][2];
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = jb * kTile + 8 * (r / 4) + hf4 + (r % 4);
                const float4 q4 = gab[min(i, n_h - 1)];
                const float vi = __uint_as_float((vv[jb][r / 2] >> (16 * (r % 2))) << 16);
                // past the last node: zero (its X comes from a repeated key row)
                const float rv = __uint_as_float(__float_as_uint(fmaf(-q4.y, X[jb][r], q4.z * vi)) &
                                                 (i < n_h ? 0xffffffffu : 0u));
                const __bf16 rb = static_cast<__bf16>(rv);
                rhi[jb][r / 8][r % 8] = rb;
                rlo[jb][r / 8][r % 8] = static_cast<__bf16>(rv - static_cast<float>(rb));
                Y[jb][r] = q4.x * Y[jb][r];
            }
        }
        // per output block t: O_t = gamma Y_t + sum_j MT_tj R_j over the k-steps that hold
        // nodes, then its stores
        // outputs through a buffer resource over the sequence's rows of this head: stores
        // past the last node are dropped by the hardware, so none is guarded
        const __amdgpu_buffer_rsrc_t ro =
            buffer_rsrc(P.out + ((size_t)lo * P.Hv + h0 + hh) * D, (unsigned)(n_h * hvd) * 4u);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            if (t < nb) {
                f32x16 Yt = Y[t];
                // rows past the last node repeat the last operator row; they are not stored
                const int it = min(t * kTile + l32_h, n_h - 1);
                const uint16_t *mh = Lmth + it * MS + hf4;
                const uint16_t *ml = Lmtl + it * MS + hf4;
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) {
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        if (jb * kTile + 16 * u < n_h) {  // operand nodes past the last: zero weights
                            const int c0 = jb * kTile + 16 * u;
                            const uint2 x0 = *reinterpret_cast<const uint2 *>(mh + c0);
                            const uint2 x1 = *reinterpret_cast<const uint2 *>(mh + c0 + 8);
                            const uint2 y0 = *reinterpret_cast<const uint2 *>(ml + c0);
                            const uint2 y1 = *reinterpret_cast<const uint2 *>(ml + c0 + 8);
                            const bf16x8 ahi = __builtin_bit_cast(bf16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
                            const bf16x8 alo = __builtin_bit_cast(bf16x8, make_uint4(y0.x, y0.y, y1.x, y1.y));
                            Yt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, rhi[jb][u], Yt, 0, 0, 0);
                            Yt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, rlo[jb][u], Yt, 0, 0, 0);
                            Yt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, rhi[jb][u], Yt, 0, 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // node of half-wave 0 (uniform; half-wave 1 adds 4)
                    const int ir = t * kTile + 8 * (r / 4) + (r % 4);
                    // (the builtin takes the 32 bits as an integer: pass the bits, not the value)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Yt[r]), ro, (unsigned)(ir * hvd) * 4u + lane_b,
                                                          0, 0);
                }
            }
            // one output block's operator fragments live at a time
            __builtin_amdgcn_sched_barrier(0);
        }
        // the next head's state: its registers, Y and R are all spent here, and it streams
        // in under the next head's operator scatter
        if (hh + 1 < grp) load_state_frags<D>(s0 + (size_t)(hh + 1) * D * D, s_lane, st);
    }
}

// ===========================================================================
// Replay on the matrix cores: one workgroup per (sequence, value head), D/32
// waves, wave w owning state rows [32w, 32w+32).  Four workgroups fit a CU,
// so one's table and state loads overlap another's arithmetic and stores.
// With L path tokens (keys k_e, L <= 16):
//   x_e   = S0 k_e                                   (X = S0 K^T, MFMA)
//   c_p   = b_p v_p - alpha_p x_p - sum_{e<p} Lc[p][e] c_e   (per row, VALU)
//   S_new = gamma_{L-1} S0 + sum_e w_e c_e k_e^T     (rank-L update, MFMA
//                                                     accumulating onto the
//                                                     scaled state in place)
// with Lc[p][e] = b_p R(p,e) (k_e . k_p), R(p,e) = a_{e+1} ... a_p,
// gamma_p = a_0 ... a_p, alpha_p = b_p gamma_p, w_e = R(L-1, e).
// The lane's state registers follow the 32x32 accumulator layout of the
// transposed tile (lane: one row; register r of tile t: column
// 32t + 8(r/4) + 4*half + r%4), which is also a valid k-ordering of the B
// operand of X, so the state is loaded once and updated in place.
// ===========================================================================
template <int D>
struct PTab {
    uint16_t *k;      // [16][KP] path keys (bf16), rows >= L zero
    uint16_t *kt;     // [D][KT] the same keys transposed
    uint16_t *klo, *ktlo;  // fp32 keys: the lo parts, laid out as k and kt (k, kt hold the hi parts)
    uint16_t *v;      // [16][grp][D] path values of the workgroup's heads
    float *vf;        // the same for fp32 values
    float *gram;      // [16][17] k_e . k_p
    float *coefL;     // [grp][16][17]
    float4 *gaw;      // [grp][16] gamma, alpha, b, w
    float *a, *b;     // [grp][16]
    static constexpr int KP = D + 8;
    static constexpr int KT = kPath + 8;
};

template <int D>
__host__ __device__ inline size_t ptab_bytes(int grp, bool f32 = false) {
    const size_t keys = (size_t)kPath * PTab<D>::KP * 2 + (size_t)D * PTab<D>::KT * 2;
    return keys * (f32 ? 2 : 1) + (size_t)kPath * grp * D * (f32 ? 4 : 2) + kPath * (kPath + 1) * 4 +
           (size_t)grp * kPath * (kPath + 1) * 4 + (size_t)grp * kPath * 16 + 2 * (size_t)grp * kPath * 4;
}

template <int D>
__device__ inline PTab<D> ptab_carve(char *base, int grp, bool f32 = false) {
    PTab<D> L;
    L.gaw = reinterpret_cast<float4 *>(base);      base += (size_t)grp * kPath * 16;
    L.k = reinterpret_cast<uint16_t *>(base);      base += (size_t)kPath * PTab<D>::KP * 2;
    L.kt = reinterpret_cast<uint16_t *>(base);     base += (size_t)D * PTab<D>::KT * 2;
    L.klo = L.k;
    L.ktlo = L.kt;
    if (f32) {
        L.klo = reinterpret_cast<uint16_t *>(base);  base += (size_t)kPath * PTab<D>::KP * 2;
        L.ktlo = reinterpret_cast<uint16_t *>(base); base += (size_t)D * PTab<D>::KT * 2;
    }
    L.v = reinterpret_cast<uint16_t *>(base);
    L.vf = reinterpret_cast<float *>(base);        base += (size_t)kPath * grp * D * (f32 ? 4 : 2);
    L.gram = reinterpret_cast<float *>(base);      base += kPath * (kPath + 1) * 4;
    L.coefL = reinterpret_cast<float *>(base);     base += (size_t)grp * kPath * (kPath + 1) * 4;
    L.a = reinterpret_cast<float *>(base);         base += (size_t)grp * kPath * 4;
    L.b = reinterpret_cast<float *>(base);
    return L;
}

// the lane's state tiles: S[t][r] = state[row][32t + 8(r/4) + 4*half + r%4]
template <int D>
__device__ __forceinline__ void load_state_tiles(const float *head, unsigned lane_off, f32x16 (&S)[D / 32]) {
    const float *p = head + lane_off;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 x = *reinterpret_cast<const float4 *>(p + 32 * t + 8 * q);
            S[t][4 * q + 0] = x.x; S[t][4 * q + 1] = x.y; S[t][4 * q + 2] = x.z; S[t][4 * q + 3] = x.w;
        }
}

// Gram entries k_e . k_p of the path keys in LDS, formed by one wave (one 32x32
// tile, 16 rows used) and written to L.gram.
template <int D, bool F32>
__device__ __forceinline__ void replay_gram(const PTab<D> &L, int l32, int hf) {
    f32x16 gk = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const bf16x8 A = l32 < kPath ? frag_of(L.k + l32 * PTab<D>::KP, s, hf) : zero_frag();
        if constexpr (F32) {
            const bf16x8 Al = l32 < kPath ? frag_of(L.klo + l32 * PTab<D>::KP, s, hf) : zero_frag();
            gk = mfma_split(A, Al, A, Al, gk);
        } else {
            gk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, A, gk, 0, 0, 0);
        }
    }
    if (l32 < kPath) {
#pragma unroll
        for (int r = 0; r < 8; ++r) L.gram[l32 * (kPath + 1) + 8 * (r / 4) + 4 * hf + (r % 4)] = gk[r];
    }
}

// The replay's coefficient phase for (head hh, path entry p): the ratios R(p, e),
// the row Lc[p][.] of the recurrence and the gates gamma_p, alpha_p, b_p, w_p, from
// the gates and Gram entries in LDS.
template <int D>
__device__ __forceinline__ void replay_coef_entry(const PTab<D> &L, int len, int hh, int p) {
    const int tid = hh * kPath + p;
    const float *ah = L.a + hh * kPath;
    const float bp = L.b[tid];
    // the gates and the row's Gram entries, read before the first coefficient is written
    float av[kPath], gr[kPath];
#pragma unroll
    for (int e = 0; e < kPath; ++e) {
        av[e] = ah[e];
        gr[e] = L.gram[p * (kPath + 1) + e];
    }
    float r = 1.0f;  // R(p, e), e from p-1 down
#pragma unroll
    for (int e = kPath - 1; e >= 0; --e) {
        float v = 0.0f;
        if (e < p) {
            r *= av[min(e + 1, kPath - 1)];
            v = p < len ? bp * r * gr[e] : 0.0f;
        }
        L.coefL[(hh * kPath + p) * (kPath + 1) + e] = v;
    }
    float gm = 1.0f, wr = 1.0f;
#pragma unroll
    for (int t = 0; t < kPath; ++t) {
        if (t <= p) gm *= av[t];
        if (t > p && t < len) wr *= av[t];
    }
    L.gaw[tid] = make_float4(gm, bp * gm, bp, p < len ? wr : 0.0f);
}

// One value head of the replay, on the path tables in LDS: X = S0 K^T for the path
// keys (MFMA, the state split hi + lo), the per-row recurrence for c, then
// S <- gamma_{L-1} S + sum_e w_e c_e k_e^T accumulated onto the lane's state tiles
// and stored from them to dst's head hh (s_lane: the lane's first element of a head).
template <int D, bool F32>
__device__ __forceinline__ void replay_head(f32x16 (&S)[D / 32], const PTab<D> &L, int grp, int hh, int len, int l32,
                                            int hf, int row, float *dst, unsigned s_lane) {
    constexpr int NTILE = D / 32;
    // X = S0 K^T: k-step s takes tile s/2, registers 8(s%2) .. 8(s%2)+7 (columns
    // 32t + 16u + 8(e/4) + 4*half + e%4), the keys read in the same column order
    f32x16 ax = {};
    const uint16_t *krow = L.k + l32 * PTab<D>::KP;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const int t = s / 2, u = s % 2;
        bf16x8 shi, slo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = S[t][8 * u + e];
            const __bf16 hb = static_cast<__bf16>(x);
            shi[e] = hb;
            slo[e] = static_cast<__bf16>(x - static_cast<float>(hb));
        }
        bf16x8 A = zero_frag();
        if (l32 < kPath) {
            const uint2 k0 = *reinterpret_cast<const uint2 *>(krow + 32 * t + 16 * u + 4 * hf);
            const uint2 k1 = *reinterpret_cast<const uint2 *>(krow + 32 * t + 16 * u + 8 + 4 * hf);
            A = __builtin_bit_cast(bf16x8, make_uint4(k0.x, k0.y, k1.x, k1.y));
        }
        if constexpr (F32) {
            bf16x8 Al = zero_frag();
            if (l32 < kPath) {
                const uint16_t *klrow = L.klo + l32 * PTab<D>::KP;
                const uint2 k0 = *reinterpret_cast<const uint2 *>(klrow + 32 * t + 16 * u + 4 * hf);
                const uint2 k1 = *reinterpret_cast<const uint2 *>(klrow + 32 * t + 16 * u + 8 + 4 * hf);
                Al = __builtin_bit_cast(bf16x8, make_uint4(k0.x, k0.y, k1.x, k1.y));
            }
            ax = mfma_split(A, Al, shi, slo, ax);
        } else {
            ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, shi, ax, 0, 0, 0);
            ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, slo, ax, 0, 0, 0);
        }
    }
    // x_e of this row: accumulator r < 8 holds e = 8(r/4) + 4*half + r%4, the other
    // half-wave the rest
    float x[kPath];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const float mine = ax[r];
        const float other = __shfl_xor(mine, 32);
        const int e_mine = 8 * (r / 4) + (r % 4);  // + 4*half
        x[e_mine] = hf ? other : mine;
        x[e_mine + 4] = hf ? mine : other;
    }
    // c_p = b_p v_p - alpha_p x_p - sum_{e<p} Lc[p][e] c_e
    const float4 *gaw = L.gaw + hh * kPath;
    const float *cl = L.coefL + hh * kPath * (kPath + 1);
    const uint16_t *vh = L.v + hh * D + row;
    const float *vhf = L.vf + hh * D + row;
    float c[kPath];
#pragma unroll
    for (int p = 0; p < kPath; ++p) {
        const float4 q4 = gaw[p];
        float acc = fmaf(-q4.y, x[p], q4.z * (F32 ? vhf[p * grp * D] : bf2f(vh[p * grp * D])));
#pragma unroll
        for (int e = 0; e < p; ++e) acc = fmaf(-cl[p * (kPath + 1) + e], c[e], acc);
        c[p] = p < len ? acc : 0.0f;
    }
    // B operand of the update: this half-wave's entries w_e c_e, e = 8*half .. 8*half+7
    bf16x8 whi, wlo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int ee = e;  // entry 8*half + e
        const float wc = (hf ? gaw[8 + ee].w * c[8 + ee] : gaw[ee].w * c[ee]);
        const __bf16 hb = static_cast<__bf16>(wc);
        whi[e] = hb;
        wlo[e] = static_cast<__bf16>(wc - static_cast<float>(hb));
    }
    const float gl = gaw[len - 1].x;
    float *dh = dst + (size_t)hh * D * D + s_lane;
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
        // A: k_e[32t + l32] for e = 8*half .. 8*half+7 (transposed keys)
        const bf16x8 A = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4 *>(L.kt + (32 * t + l32) * PTab<D>::KT + 8 * hf));
#pragma unroll
        for (int r = 0; r < 16; ++r) S[t][r] *= gl;
        if constexpr (F32) {
            const bf16x8 Al = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(L.ktlo + (32 * t + l32) * PTab<D>::KT + 8 * hf));
            S[t] = mfma_split(A, Al, whi, wlo, S[t]);
        } else {
            S[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, whi, S[t], 0, 0, 0);
            S[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wlo, S[t], 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4 *>(dh + 32 * t + 8 * q) =
                make_float4(S[t][4 * q], S[t][4 * q + 1], S[t][4 * q + 2], S[t][4 * q + 3]);
    }
}

template <int D, bool CHAIN, bool F32>
__global__ __launch_bounds__(VG<D>::THREADS) __attribute__((amdgpu_waves_per_eu(3))) void replay_kernel(
    Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    constexpr int NT = VG<D>::THREADS, NTILE = D / 32;
    constexpr int grp = 1;  // value heads of this workgroup
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int row = w * 32 + l32;
    const int nhg = P.Hv / grp;
    const int b = blockIdx.x / nhg, h0 = blockIdx.x % nhg * grp;
    const int g = h0 / (P.Hv / P.Hk);

    // ---- the path: lane e < 16 of every wave holds path entry e (local id, root first);
    // its length, source and destination.  Each step's loads are issued before any test.
    int lo, len, slot, pl;
    float *dst;
    if (CHAIN) {
        const int c0 = P.cu_nodes[b], c1 = P.cu_nodes[b + 1];
        len = P.final_len[b];
        slot = P.slot_idx[b];
        if (!(0 <= c0 && c0 <= c1 && c1 <= P.T) || c1 - c0 > P.max_nodes) return;
        if (len < 0 || len > c1 - c0 || len > kPath) return;
        if (slot < 0 || slot >= P.num_slots) return;
        lo = c0;
        pl = lane % kPath;
        dst = P.final_state + (size_t)b * P.Hv * D * D;
    } else {
        const bool planned = ws_plan_matches(P);
        const int4 info = *reinterpret_cast<const int4 *>(P.ws.seq_info + b * kSeqInfoInts);
        const int m = P.accepted[b];
        // the common case is tested on all three loads at once, so they are issued together
        // instead of each waiting for the test on the one before
        if (!(planned & (info.z == GDN_SEQ_OK) & (m >= 0) & (m < info.y))) {
            if (!planned) {  // no slot is written; gdn_tree_status reports the misuse
                if (blockIdx.x == 0 && tid == 0) P.ws.header[kHdrMisuse] = 1;
                return;
            }
            if (info.z != GDN_SEQ_OK || info.y == 0) return;
            if ((m < -1 || m >= info.y) && g == 0 && tid == 0) P.ws.seq_status[b] = GDN_SEQ_BAD_ACCEPT;
            return;  // a rejected accepted node, or m = -1: nothing to persist
        }
        lo = uni(info.x);
        slot = uni(info.w);
        const int mu = uni(m);
        pl = P.ws.nodepath[(size_t)(lo + mu) * GDN_MAX_DEPTH + lane % kPath];
        len = P.ws.depth[lo + mu];
        if (g == 0 && tid < GDN_MAX_DEPTH) {
            P.ws.path[b * GDN_MAX_DEPTH + tid] = pl;
            if (tid == 0) P.ws.path_len[b] = len;
        }
        dst = P.state_out + (size_t)slot * P.Hv * D * D;
    }
    len = uni(len);
    const float *s0 = P.state_in + ((size_t)slot * P.Hv + h0) * D * D;
    dst += (size_t)h0 * D * D;
    const unsigned s_lane = (unsigned)(row * D + 4 * hf);

    f32x16 SA[NTILE];
    if (len == 0) {  // chain final state after zero tokens: the committed state
#pragma unroll 1
        for (int hh = 0; hh < grp; ++hh) {
            load_state_tiles<D>(s0 + (size_t)hh * D * D, s_lane, SA);
#pragma unroll
            for (int t = 0; t < NTILE; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<float4 *>(dst + (size_t)hh * D * D + s_lane + 32 * t + 8 * q) =
                        make_float4(SA[t][4 * q], SA[t][4 * q + 1], SA[t][4 * q + 2], SA[t][4 * q + 3]);
        }
        return;
    }

    // ---- tables: path keys (both ways), values and gates of the workgroup's head
    const PTab<D> L = ptab_carve<D>(lds_raw, grp, F32);
    const InT<F32> *kb = static_cast<const InT<F32> *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const InT<F32> *vg = static_cast<const InT<F32> *>(P.v) + ((size_t)lo * P.Hv + h0) * D;
    constexpr int EPC = F32 ? 4 : 8;   // values per 16-byte chunk
    constexpr int KC = kPath * D / EPC;  // 16-byte chunks of the path keys
    constexpr int K_PER = (KC + NT - 1) / NT;
    constexpr int VC = kPath * grp * D / EPC;
    constexpr int V_PER = (VC + NT - 1) / NT;
    // the nodes each thread fetches for, looked up before any fetch is issued; every
    // fetch is unconditional (entries past the path read node 0 and are dropped), so
    // nothing waits for one before the states are issued
    static_assert(KC % NT == 0 && VC % NT == 0, "whole table rounds");
    // node of path entry e, and node 0 for every e >= len: a chain shorter than 16
    // tokens may end its buffers right after its last token
    auto node_of = [&](int e) {
        const int x = __shfl(pl, e);  // every lane takes part in the shuffle
        return e < len ? max(x, 0) : 0;
    };
    int nk[K_PER], nv[V_PER];
#pragma unroll
    for (int u = 0; u < K_PER; ++u) nk[u] = node_of(((tid + u * NT) / (D / EPC)) % kPath);
#pragma unroll
    for (int u = 0; u < V_PER; ++u) nv[u] = node_of(((tid + u * NT) / (grp * D / EPC)) % kPath);
    const int ng = node_of(tid % kPath);
    uint4 kr[K_PER], vr[V_PER];
#pragma unroll
    for (int u = 0; u < K_PER; ++u)
        kr[u] = *reinterpret_cast<const uint4 *>(kb + (size_t)nk[u] * P.Hk * D + EPC * ((tid + u * NT) % (D / EPC)));
#pragma unroll
    for (int u = 0; u < V_PER; ++u)
        vr[u] = *reinterpret_cast<const uint4 *>(vg + (size_t)nv[u] * P.Hv * D +
                                                 EPC * ((tid + u * NT) % (grp * D / EPC)));
    const bool gate_t = tid < grp * kPath;
    const size_t at = (size_t)(lo + ng) * P.Hv + h0 + (gate_t ? tid / kPath : 0);
    float ga = P.a[at], gb = P.b[at];
    // the state, issued after the tables so that waiting for the tables does not wait for it
    load_state_tiles<D>(s0, s_lane, SA);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < K_PER; ++u) {
        const int idx = tid + u * NT, e = idx / (D / EPC), c8 = idx % (D / EPC);
        const uint4 kv = e < len ? kr[u] : make_uint4(0, 0, 0, 0);
        if constexpr (F32) {  // four keys' values, split hi + lo, both ways
            uint2 hi, lo2;
            split4(__builtin_bit_cast(float4, kv), hi, lo2);
            *reinterpret_cast<uint2 *>(L.k + e * PTab<D>::KP + 4 * c8) = hi;
            *reinterpret_cast<uint2 *>(L.klo + e * PTab<D>::KP + 4 * c8) = lo2;
            const uint16_t *hh2 = reinterpret_cast<const uint16_t *>(&hi);
            const uint16_t *ll2 = reinterpret_cast<const uint16_t *>(&lo2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                L.kt[(4 * c8 + i) * PTab<D>::KT + e] = hh2[i];
                L.ktlo[(4 * c8 + i) * PTab<D>::KT + e] = ll2[i];
            }
        } else {
            *reinterpret_cast<uint4 *>(L.k + e * PTab<D>::KP + 8 * c8) = kv;
            const uint16_t *hv = reinterpret_cast<const uint16_t *>(&kv);
#pragma unroll
            for (int i = 0; i < 8; ++i) L.kt[(8 * c8 + i) * PTab<D>::KT + e] = hv[i];
        }
    }
#pragma unroll
    for (int u = 0; u < V_PER; ++u) {
        const int idx = tid + u * NT;
        reinterpret_cast<uint4 *>(L.v)[idx] = idx / (grp * D / EPC) < len ? vr[u] : make_uint4(0, 0, 0, 0);
    }
    if (gate_t) {
        const bool on = tid % kPath < len;
        L.a[tid] = on ? ga : 1.0f;
        L.b[tid] = on ? gb : 0.0f;
    }
    __syncthreads();

    // ---- Gram entries of the path keys (one wave, one 32x32 tile, 16 rows used)
    if (w == 0) replay_gram<D, F32>(L, l32, hf);
    __syncthreads();
    // ---- per (head, path entry p): ratios, coefficients
    if (tid < grp * kPath) replay_coef_entry<D>(L, len, tid / kPath, tid % kPath);
    __syncthreads();

    // ---- value heads
    replay_head<D, F32>(SA, L, grp, 0, len, l32, hf, row, dst, s_lane);
}

// ===========================================================================
// Chains longer than one drafting block (prefill-style gdn_chain_verify): one
// workgroup per (sequence, value head), D/32 waves, the state held in
// registers in the replay's tile layout for the whole chain and walked in
// chunks of 16 tokens.  Per chunk, from the state S at its start, with
// G_p = a_0 ... a_p and R(p,e) = a_{e+1} ... a_p inside the chunk:
//   X = S K^T, Y = S Q^T                                  (MFMA, S split hi + lo)
//   c_p = b_p v_p - b_p G_p x_p - sum_{e<p} b_p R(p,e) (k_e . k_p) c_e  (per row)
//   o_p = G_p y_p + sum_{e<=p} R(p,e) (k_e . q_p) c_e                  (per row)
//   S  <- G_{L-1} S + sum_e R(L-1,e) c_e k_e^T            (rank-16 MFMA update)
// The state after final_len tokens, when that falls inside a chunk, is the same
// update truncated to the chunk's first tokens.  The next chunk's keys, queries,
// values and gates are loaded into registers while this chunk computes.
// ===========================================================================
template <int D>
struct CkTab {
    uint16_t *k, *kt, *q;        // [16][KP], [D][KT], [16][KP] bf16 (fp32 inputs: hi parts)
    uint16_t *klo, *ktlo, *qlo;  // fp32 inputs: lo parts, same layouts
    float *v;                    // [16][D] this head's values
    float *gram, *gq;            // [16][17]: row p, column e: k_e . k_p and k_e . q_p
    float *coefL;                // [16][17]: b_p R(p,e) (k_e . k_p) (e < p)
    float *coefM;                // [16][MS]: R(p,e) (k_e . q_p) (e <= p), rows 16-byte aligned
    float4 *gaw;                 // [16] G_p, b_p G_p, b_p, R(L-1, p)
    float *wf;                   // [16] R(f-1, p) for the final state f tokens into the chunk
    float *a, *b;                // [16]
    static constexpr int KP = D + 8;
    static constexpr int KT = kPath + 8;
    static constexpr int PS = kPath + 1;
    static constexpr int MS = kPath + 4;
};

template <int D>
__host__ __device__ inline size_t cktab_bytes(bool f32) {
    using Q = CkTab<D>;
    const size_t keys = (size_t)2 * kPath * Q::KP * 2 + (size_t)D * Q::KT * 2;
    return keys * (f32 ? 2 : 1) + (size_t)kPath * D * 4 + 3 * (size_t)kPath * Q::PS * 4 + (size_t)kPath * Q::MS * 4 +
           kPath * 16 + 3 * kPath * 4;
}

template <int D>
__device__ inline CkTab<D> cktab_carve(char *base, bool f32) {
    using Q = CkTab<D>;
    CkTab<D> L;
    L.gaw = reinterpret_cast<float4 *>(base);      base += kPath * 16;
    L.v = reinterpret_cast<float *>(base);         base += (size_t)kPath * D * 4;
    L.k = reinterpret_cast<uint16_t *>(base);      base += (size_t)kPath * Q::KP * 2;
    L.q = reinterpret_cast<uint16_t *>(base);      base += (size_t)kPath * Q::KP * 2;
    L.kt = reinterpret_cast<uint16_t *>(base);     base += (size_t)D * Q::KT * 2;
    L.klo = L.k;
    L.qlo = L.q;
    L.ktlo = L.kt;
    if (f32) {
        L.klo = reinterpret_cast<uint16_t *>(base);  base += (size_t)kPath * Q::KP * 2;
        L.qlo = reinterpret_cast<uint16_t *>(base);  base += (size_t)kPath * Q::KP * 2;
        L.ktlo = reinterpret_cast<uint16_t *>(base); base += (size_t)D * Q::KT * 2;
    }
    L.coefM = reinterpret_cast<float *>(base);     base += kPath * Q::MS * 4;
    L.gram = reinterpret_cast<float *>(base);      base += kPath * Q::PS * 4;
    L.gq = reinterpret_cast<float *>(base);        base += kPath * Q::PS * 4;
    L.coefL = reinterpret_cast<float *>(base);     base += kPath * Q::PS * 4;
    L.wf = reinterpret_cast<float *>(base);        base += kPath * 4;
    L.a = reinterpret_cast<float *>(base);         base += kPath * 4;
    L.b = reinterpret_cast<float *>(base);
    return L;
}

// the lane's state tiles stored in the replay layout
template <int D>
__device__ __forceinline__ void store_state_tiles(float *head, unsigned lane_off, const f32x16 (&S)[D / 32]) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4 *>(head + lane_off + 32 * t + 8 * q) =
                make_float4(S[t][4 * q], S[t][4 * q + 1], S[t][4 * q + 2], S[t][4 * q + 3]);
}

template <int D, bool F32>
__global__ __launch_bounds__(VG<D>::THREADS) __attribute__((amdgpu_waves_per_eu(2))) void chain_chunks_kernel(
    Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    using Q = CkTab<D>;
    constexpr int NT = VG<D>::THREADS, NTILE = D / 32;
    constexpr int EPC = F32 ? 4 : 8;               // values per 16-byte chunk
    constexpr int RC = kPath * D / EPC;            // 16-byte chunks of one chunk's keys (queries, values)
    constexpr int R_PER = RC / NT;
    static_assert(RC % NT == 0, "whole rounds of chunk loads");
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int row = w * 32 + l32;
    const int b = blockIdx.x / P.Hv, h = blockIdx.x % P.Hv;
    const int g = h / (P.Hv / P.Hk);
    const SeqView sv = seq_view<true>(P, b);
    if (P.has_ws && h == 0 && tid == 0) {
        if (b == 0) {
            P.ws.header[0] = kChainMagic;
            P.ws.header[1] = P.B;
            P.ws.header[2] = P.T;
            P.ws.header[kHdrMisuse] = 0;
        }
        P.ws.seq_status[b] = sv.status;
    }
    const int lo = sv.lo, n = sv.n;
    const bool want_out = P.q != nullptr && P.out != nullptr;
    if (sv.status != GDN_SEQ_OK) {
        if (P.out)
            for (int t = tid; t < n * D; t += NT) P.out[((size_t)(lo + t / D) * P.Hv + h) * D + t % D] = qnan_f();
        return;
    }
    const int flen = P.final_len ? P.final_len[b] : -1;
    float *fin = (P.final_state && flen >= 0 && flen <= n) ? P.final_state + ((size_t)b * P.Hv + h) * D * D
                                                            : nullptr;
    if (!fin && !(want_out && n > 0)) return;
    // an empty chain leaves its slot unchecked in the sequence view: only the committed
    // state is wanted, from a valid slot
    int slot = sv.slot;
    if (n == 0) {
        slot = P.slot_idx[b];
        if (slot < 0 || slot >= P.num_slots) return;
    }
    const unsigned s_lane = (unsigned)(row * D + 4 * hf);
    f32x16 S[NTILE];
    load_state_tiles<D>(P.state_in + ((size_t)slot * P.Hv + h) * D * D, s_lane, S);
    if (fin && flen == 0) store_state_tiles<D>(fin, s_lane, S);
    // only the chunks up to the last output or the final state are walked
    const int n_walk = want_out ? n : flen;
    if (n_walk <= 0) return;

    const CkTab<D> L = cktab_carve<D>(lds_raw, F32);
    const InT<F32> *kb = static_cast<const InT<F32> *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const InT<F32> *qb = want_out ? static_cast<const InT<F32> *>(P.q) + ((size_t)lo * P.Hk + g) * D : kb;
    const InT<F32> *vb = static_cast<const InT<F32> *>(P.v) + ((size_t)lo * P.Hv + h) * D;
    const size_t kq_stride = (size_t)P.Hk * D, v_stride = (size_t)P.Hv * D;
    // one chunk's raw inputs: this thread's 16-byte pieces of keys, queries and values, and
    // (threads < 16) a gate pair; entries past the chain read its last token and are dropped
    uint4 rk[R_PER], rq[R_PER], rv[R_PER];
    float ra = 1.0f, rb = 0.0f;
    auto fetch = [&](int c0) {
        const int len = min(kPath, n_walk - c0);
#pragma unroll
        for (int u = 0; u < R_PER; ++u) {
            const int idx = tid + u * NT, e = min(idx / (D / EPC), len - 1), c8 = idx % (D / EPC);
            rk[u] = *reinterpret_cast<const uint4 *>(kb + (size_t)(c0 + e) * kq_stride + EPC * c8);
            rq[u] = *reinterpret_cast<const uint4 *>(qb + (size_t)(c0 + e) * kq_stride + EPC * c8);
            rv[u] = *reinterpret_cast<const uint4 *>(vb + (size_t)(c0 + e) * v_stride + EPC * c8);
        }
        if (tid < kPath) {
            const size_t at = (size_t)(lo + c0 + min(tid, len - 1)) * P.Hv + h;
            ra = P.a[at];
            rb = P.b[at];
        }
    };
    fetch(0);

#pragma unroll 1
    for (int c0 = 0; c0 < n_walk; c0 += kPath) {
        const int len = min(kPath, n_walk - c0);
        __syncthreads();  // the previous chunk's tables are spent
        // ---- stage the chunk: keys and queries both ways (hi + lo for fp32), values as fp32
#pragma unroll
        for (int u = 0; u < R_PER; ++u) {
            const int idx = tid + u * NT, e = idx / (D / EPC), c8 = idx % (D / EPC);
            const bool on = e < len;
            const uint4 kv = on ? rk[u] : make_uint4(0, 0, 0, 0);
            const uint4 qv = on ? rq[u] : make_uint4(0, 0, 0, 0);
            const uint4 vw = on ? rv[u] : make_uint4(0, 0, 0, 0);
            if constexpr (F32) {
                uint2 kh, kl, qh, ql;
                split4(__builtin_bit_cast(float4, kv), kh, kl);
                split4(__builtin_bit_cast(float4, qv), qh, ql);
                *reinterpret_cast<uint2 *>(L.k + e * Q::KP + 4 * c8) = kh;
                *reinterpret_cast<uint2 *>(L.klo + e * Q::KP + 4 * c8) = kl;
                *reinterpret_cast<uint2 *>(L.q + e * Q::KP + 4 * c8) = qh;
                *reinterpret_cast<uint2 *>(L.qlo + e * Q::KP + 4 * c8) = ql;
                const uint16_t *h2 = reinterpret_cast<const uint16_t *>(&kh);
                const uint16_t *l2 = reinterpret_cast<const uint16_t *>(&kl);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    L.kt[(4 * c8 + i) * Q::KT + e] = h2[i];
                    L.ktlo[(4 * c8 + i) * Q::KT + e] = l2[i];
                }
                *reinterpret_cast<uint4 *>(L.v + e * D + 4 * c8) = vw;
            } else {
                *reinterpret_cast<uint4 *>(L.k + e * Q::KP + 8 * c8) = kv;
                *reinterpret_cast<uint4 *>(L.q + e * Q::KP + 8 * c8) = qv;
                const uint16_t *k8 = reinterpret_cast<const uint16_t *>(&kv);
                const uint16_t *v8 = reinterpret_cast<const uint16_t *>(&vw);
#pragma unroll
                for (int i = 0; i < 8; ++i) L.kt[(8 * c8 + i) * Q::KT + e] = k8[i];
                float4 *vd = reinterpret_cast<float4 *>(L.v + e * D + 8 * c8);
                vd[0] = make_float4(bf2f(v8[0]), bf2f(v8[1]), bf2f(v8[2]), bf2f(v8[3]));
                vd[1] = make_float4(bf2f(v8[4]), bf2f(v8[5]), bf2f(v8[6]), bf2f(v8[7]));
            }
        }
        if (tid < kPath) {
            L.a[tid] = tid < len ? ra : 1.0f;
            L.b[tid] = tid < len ? rb : 0.0f;
        }
        // the next chunk's inputs stream in under this chunk's arithmetic
        if (c0 + kPath < n_walk) fetch(c0 + kPath);
        __syncthreads();

        // ---- Gram entries: wave 0 k . k, wave 1 k . q (16 rows of one 32x32 tile)
        if (w < 2) {
            f32x16 acc = {};
            // rows 16..31 of the tile read row 15 and are zeroed (no branch around the reads)
            const int rl = min(l32, kPath - 1);
            const bool live = l32 < kPath;
            const uint16_t *br = (w == 0 ? L.k : L.q) + rl * Q::KP;
            const uint16_t *brl = (w == 0 ? L.klo : L.qlo) + rl * Q::KP;
            auto keep = [&](bf16x8 x) { return live ? x : zero_frag(); };
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const bf16x8 A = keep(frag_of(L.k + rl * Q::KP, s, hf));
                const bf16x8 B = keep(frag_of(br, s, hf));
                if constexpr (F32) {
                    const bf16x8 Al = keep(frag_of(L.klo + rl * Q::KP, s, hf));
                    const bf16x8 Bl = keep(frag_of(brl, s, hf));
                    acc = mfma_split(A, Al, B, Bl, acc);
                } else {
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc, 0, 0, 0);
                }
            }
            // accumulator r < 8: (key e = 8(r/4) + 4*half + r%4, column p = l32)
            if (l32 < kPath) {
                float *dst = (w == 0 ? L.gram : L.gq) + l32 * Q::PS;
#pragma unroll
                for (int r = 0; r < 8; ++r) dst[8 * (r / 4) + 4 * hf + (r % 4)] = acc[r];
            }
        }
        __syncthreads();
        // ---- per token p of the chunk: ratios and coefficients
        const int f = fin ? flen - c0 : 0;  // the final state's token count inside this chunk, if in (0, len]
        if (tid < kPath) {
            const int p = tid;
            const float bp = L.b[p];
            // the gates and the row's Gram entries, read before the first coefficient is
            // written (the writes would otherwise order each step's reads behind the last's)
            float av[kPath], gkr[kPath], gqr[kPath];
#pragma unroll
            for (int e = 0; e < kPath; ++e) {
                av[e] = L.a[e];
                gkr[e] = L.gram[p * Q::PS + e];
                gqr[e] = L.gq[p * Q::PS + e];
            }
            float r = 1.0f;  // R(p, e), e from p - 1 down
#pragma unroll
            for (int e = kPath - 1; e >= 0; --e) {
                const bool lt = e < p;
                const float ae = av[min(e + 1, kPath - 1)];
                const float gk = gkr[e], gqe = gqr[e];
                r = lt ? r * ae : r;
                L.coefL[p * Q::PS + e] = lt ? bp * r * gk : 0.0f;
                L.coefM[p * Q::MS + e] = lt ? r * gqe : (e == p ? gqe : 0.0f);
            }
            float gm = 1.0f, wr = 1.0f, wfr = 1.0f;
#pragma unroll
            for (int t = 0; t < kPath; ++t) {
                const float at = av[t];
                gm = t <= p ? gm * at : gm;
                wr = (t > p && t < len) ? wr * at : wr;
                wfr = (t > p && t < f) ? wfr * at : wfr;
            }
            L.gaw[p] = make_float4(gm, bp * gm, bp, p < len ? wr : 0.0f);
            L.wf[p] = p < f ? wfr : 0.0f;
        }
        __syncthreads();

        // ---- X = S K^T and Y = S Q^T (k-step s: tile s/2, registers 8(s%2) .. +7)
        f32x16 ax = {}, ay = {};
        const int rl = min(l32, kPath - 1);
        const uint16_t *krow = L.k + rl * Q::KP, *qrow = L.q + rl * Q::KP;
        const uint16_t *klrow = L.klo + rl * Q::KP, *qlrow = L.qlo + rl * Q::KP;
        // rows past the chunk's 16 read row 15 and are zeroed (no branch around the reads)
        auto row_frag = [&](const uint16_t *rowp, int t, int u) {
            const uint2 x0 = *reinterpret_cast<const uint2 *>(rowp + 32 * t + 16 * u + 4 * hf);
            const uint2 x1 = *reinterpret_cast<const uint2 *>(rowp + 32 * t + 16 * u + 8 + 4 * hf);
            const bf16x8 A = __builtin_bit_cast(bf16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
            return l32 < kPath ? A : zero_frag();
        };
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const int t = s / 2, u = s % 2;
            bf16x8 shi, slo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = S[t][8 * u + e];
                const __bf16 hb = static_cast<__bf16>(x);
                shi[e] = hb;
                slo[e] = static_cast<__bf16>(x - static_cast<float>(hb));
            }
            const bf16x8 Ak = row_frag(krow, t, u), Aq = row_frag(qrow, t, u);
            if constexpr (F32) {
                ax = mfma_split(Ak, row_frag(klrow, t, u), shi, slo, ax);
                if (want_out) ay = mfma_split(Aq, row_frag(qlrow, t, u), shi, slo, ay);
            } else {
                ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, shi, ax, 0, 0, 0);
                ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, slo, ax, 0, 0, 0);
                if (want_out) {
                    ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, shi, ay, 0, 0, 0);
                    ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, slo, ay, 0, 0, 0);
                }
            }
        }
        // x_e, y_e of this row: accumulator r < 8 holds e = 8(r/4) + 4*half + r%4, the
        // other half-wave the rest
        float x[kPath], y[kPath];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int e_mine = 8 * (r / 4) + (r % 4);  // + 4*half
            const float mx = ax[r], ox = __shfl_xor(mx, 32);
            const float my = ay[r], oy = __shfl_xor(my, 32);
            x[e_mine] = hf ? ox : mx;
            x[e_mine + 4] = hf ? mx : ox;
            y[e_mine] = hf ? oy : my;
            y[e_mine + 4] = hf ? my : oy;
        }
        // ---- c_p per row
        float c[kPath];
#pragma unroll
        for (int p = 0; p < kPath; ++p) {
            const float4 q4 = L.gaw[p];
            float acc = fmaf(-q4.y, x[p], q4.z * L.v[p * D + row]);
#pragma unroll
            for (int e = 0; e < p; ++e) acc = fmaf(-L.coefL[p * Q::PS + e], c[e], acc);
            c[p] = p < len ? acc : 0.0f;
        }
        // ---- outputs: half-wave 0 tokens 0..7, half-wave 1 tokens 8..15
        if (want_out) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int p = 8 * hf + j;
                // this half-wave's token p: the terms e > p are selected away (their weights
                // are zero; a select keeps a non-finite later c_e out of this output)
                const float yp = hf ? y[8 + j] : y[j];
                float o = L.gaw[p].x * yp;
                const float4 *mrow = reinterpret_cast<const float4 *>(L.coefM + p * Q::MS);
#pragma unroll
                for (int e4 = 0; e4 < kPath / 4; ++e4) {
                    const float4 m4 = mrow[e4];
                    const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 4 * e4 + i;
                        o = fmaf(e <= p ? mv[i] : 0.0f, e <= p ? c[e] : 0.0f, o);
                    }
                }
                if (p < len) P.out[((size_t)(lo + c0 + p) * P.Hv + h) * D + row] = o;
            }
        }
        // ---- the state after f tokens of this chunk, and the state after the chunk
        auto rank16 = [&](const float *wsrc, float gam, bool final_out) {
            bf16x8 whi, wlo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float wc = (hf ? wsrc[8 + e] * c[8 + e] : wsrc[e] * c[e]);
                const __bf16 hb = static_cast<__bf16>(wc);
                whi[e] = hb;
                wlo[e] = static_cast<__bf16>(wc - static_cast<float>(hb));
            }
#pragma unroll
            for (int t = 0; t < NTILE; ++t) {
                const bf16x8 A = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const uint4 *>(L.kt + (32 * t + l32) * Q::KT + 8 * hf));
                f32x16 T = S[t];
#pragma unroll
                for (int r = 0; r < 16; ++r) T[r] *= gam;
                if constexpr (F32) {
                    const bf16x8 Al = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4 *>(L.ktlo + (32 * t + l32) * Q::KT + 8 * hf));
                    T = mfma_split(A, Al, whi, wlo, T);
                } else {
                    T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, whi, T, 0, 0, 0);
                    T = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wlo, T, 0, 0, 0);
                }
                if (final_out) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<float4 *>(fin + s_lane + 32 * t + 8 * q) =
                            make_float4(T[4 * q], T[4 * q + 1], T[4 * q + 2], T[4 * q + 3]);
                } else {
                    S[t] = T;
                }
            }
        };
        if (f > 0 && f <= len) rank16(L.wf, L.gaw[f - 1].x, true);
        if (c0 + kPath < n_walk) {
            float wv[kPath];
#pragma unroll
            for (int e = 0; e < kPath; ++e) wv[e] = L.gaw[e].w;
            rank16(wv, L.gaw[len - 1].x, false);
        }
    }
}

// ===========================================================================
// Persist fused with the next verify (trees of at most 32 nodes, bf16 inputs).
// In a decode loop a layer's state is read by that layer's verify and read and
// written by its persist.  Deferring step t's persist to the layer's verify of
// step t+1 lets one pass over the state serve both: the workgroup of (sequence,
// value head) loads S once, replays step t's accepted path in registers with
// the replay's own tables and arithmetic, writes the result in place, and forms
// step t+1's products X = S K^T and Y = S Q^T from the same registers, reading
// the tree's keys and queries in the column order of the state tiles (the order
// the replay uses for its path keys).  Coefficients and outputs follow the group
// verify.  Pp holds the previous step (plan, inputs, accepted nodes), Pn the new
// one (plan, inputs, outputs); both address the same state cache.
// Slots.  Sequence b is persisted into its previous slot and verified from its
// new slot.  When the two are equal and the new tree is verified here, the new
// plan guarantees no other verified sequence reads that slot.  Otherwise the
// workgroup checks every sequence's new record: if another verified sequence
// reads the slot it would write, the persist is skipped and the sequence is
// marked GDN_SEQ_NOT_PERSISTED in the previous workspace, so no slot is ever
// written by one workgroup while another reads it.
// ===========================================================================
// LDS of the fused kernel, 39 KiB at D = 128 (three workgroups share a CU, as many as
// its registers allow; 49 KiB kept the same three and measured 2 us slower per call):
//  - the replay's tables that its coefficient phase needs (path keys, gates, Gram
//    entries, coefficients);
//  - the new tree's keys and queries, gates and output operator;
//  - one region used twice: first the new tree's coefficient scratch (Gram entries in
//    path order, coefficients, paths, gates, depths), then, once those are spent, the
//    replay's transposed path keys and path values.
template <int D>
struct FusedLayout {
    using Q = GPad<D>;
    static constexpr size_t P_GAW = 0;
    static constexpr size_t P_K = P_GAW + (size_t)kPath * 16;
    static constexpr size_t P_GRAM = P_K + (size_t)kPath * PTab<D>::KP * 2;
    static constexpr size_t P_COEF = P_GRAM + (size_t)kPath * (kPath + 1) * 4;
    static constexpr size_t P_A = P_COEF + (size_t)kPath * (kPath + 1) * 4;
    static constexpr size_t P_B = P_A + (size_t)kPath * 4;
    static constexpr size_t N_KQ = P_B + (size_t)kPath * 4;
    static constexpr size_t N_GAB = N_KQ + (size_t)2 * kTile * Q::KQ * 2;
    static constexpr size_t N_MTH = N_GAB + (size_t)kTile * 16;
    static constexpr size_t N_MTL = N_MTH + (size_t)kTile * Q::MT * 2;
    static constexpr size_t U = N_MTL + (size_t)kTile * Q::MT * 2;  // the shared region
    // first use: the new tree's coefficient scratch
    static constexpr size_t N_COEF = U;
    static constexpr size_t N_GK = N_COEF + (size_t)kTile * Q::PS * 4;
    static constexpr size_t N_GQ = N_GK + (size_t)kTile * Q::PS * 4;
    static constexpr size_t N_ANC = N_GQ + (size_t)kTile * Q::PS * 4;
    static constexpr size_t N_A = N_ANC + (size_t)kTile * Q::PS * 4;
    static constexpr size_t N_B = N_A + (size_t)kTile * 4;
    static constexpr size_t N_DEPTH = N_B + (size_t)kTile * 4;
    static constexpr size_t N_END = N_DEPTH + (size_t)kTile * 4;
    // second use: the replay's transposed keys and values
    static constexpr size_t P_KT = U;
    static constexpr size_t P_V = P_KT + (size_t)D * PTab<D>::KT * 2;
    static constexpr size_t P_END = P_V + (size_t)kPath * D * 2;
    static constexpr size_t BYTES = N_END > P_END ? N_END : P_END;
    static_assert(P_K % 16 == 0 && N_KQ % 16 == 0 && N_GAB % 16 == 0 && N_MTH % 8 == 0 && U % 16 == 0 &&
                      N_DEPTH % 16 == 0 && P_V % 16 == 0,
                  "16-byte aligned tables");
};

template <int D>
__device__ inline PTab<D> fused_prev_carve(char *base) {
    using F = FusedLayout<D>;
    PTab<D> L;
    L.gaw = reinterpret_cast<float4 *>(base + F::P_GAW);
    L.k = L.klo = reinterpret_cast<uint16_t *>(base + F::P_K);
    L.kt = L.ktlo = reinterpret_cast<uint16_t *>(base + F::P_KT);
    L.v = reinterpret_cast<uint16_t *>(base + F::P_V);
    L.vf = reinterpret_cast<float *>(base + F::P_V);
    L.gram = reinterpret_cast<float *>(base + F::P_GRAM);
    L.coefL = reinterpret_cast<float *>(base + F::P_COEF);
    L.a = reinterpret_cast<float *>(base + F::P_A);
    L.b = reinterpret_cast<float *>(base + F::P_B);
    return L;
}

// the group verify's tables for one value head, without the staged values
template <int D>
__device__ inline GTab<D> fused_new_carve(char *base) {
    using F = FusedLayout<D>;
    GTab<D> L;
    L.kq = reinterpret_cast<uint16_t *>(base + F::N_KQ);
    L.v = nullptr;
    L.gab = reinterpret_cast<float4 *>(base + F::N_GAB);
    L.mth = reinterpret_cast<uint16_t *>(base + F::N_MTH);
    L.mtl = reinterpret_cast<uint16_t *>(base + F::N_MTL);
    L.coefL = reinterpret_cast<float *>(base + F::N_COEF);
    L.gk = reinterpret_cast<float *>(base + F::N_GK);
    L.gq = reinterpret_cast<float *>(base + F::N_GQ);
    L.anc = reinterpret_cast<int *>(base + F::N_ANC);
    L.a = reinterpret_cast<float *>(base + F::N_A);
    L.b = reinterpret_cast<float *>(base + F::N_B);
    L.depth = reinterpret_cast<int *>(base + F::N_DEPTH);
    return L;
}

template <int D>
size_t fused_lds_bytes() {
    return FusedLayout<D>::BYTES;
}

template <int D>
__global__ __launch_bounds__(VG<D>::THREADS) __attribute__((amdgpu_waves_per_eu(3))) void persist_verify_kernel(
    Params Pp, Params Pn) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    constexpr int NT = VG<D>::THREADS, KS = VG<D>::KS;
    using Q = GPad<D>;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int row = w * 32 + l32;
    const int b = blockIdx.x / Pn.Hv, h = blockIdx.x % Pn.Hv;
    const int g = h / (Pn.Hv / Pn.Hk);

    // ---- both plans' checks and records and the accepted node, loaded together
    const bool plan_p = ws_plan_matches(Pp), plan_n = ws_plan_matches(Pn);
    const int4 ip = *reinterpret_cast<const int4 *>(Pp.ws.seq_info + b * kSeqInfoInts);
    const int4 in4 = *reinterpret_cast<const int4 *>(Pn.ws.seq_info + b * kSeqInfoInts);
    const int m = Pp.accepted[b];
    if (!(plan_p & plan_n)) {  // nothing is written; gdn_tree_status reports the misuse
        if (blockIdx.x == 0 && tid == 0) {
            if (!plan_p) Pp.ws.header[kHdrMisuse] = 1;
            if (!plan_n) Pn.ws.header[kHdrMisuse] = 1;
        }
        return;
    }
    const int lo = uni(in4.x), n = uni(in4.y), slot = uni(in4.w);
    const bool new_ok = in4.z == GDN_SEQ_OK;
    const bool verified = new_ok & (n > 0);
    // what gdn_tree_persist would do for this sequence: replay the path to m
    const bool prev_live = (ip.z == GDN_SEQ_OK) & (ip.y > 0);
    const bool want = prev_live & (m >= 0) & (m < ip.y);
    const int pslot = uni(ip.w);
    bool persist = want;
    if (want && !(verified && pslot == slot)) {
        // the slot it would write must not be another verified sequence's source
        int clash = 0;
        for (int j = tid; j < Pn.B; j += NT) {
            const int4 r = *reinterpret_cast<const int4 *>(Pn.ws.seq_info + j * kSeqInfoInts);
            clash |= (j != b) & (r.z == GDN_SEQ_OK) & (r.y > 0) & (r.w == pslot);
        }
        persist = !__syncthreads_or(clash);
    }
    if (h == 0 && tid == 0 && prev_live) {
        if (m < -1 || m >= ip.y) Pp.ws.seq_status[b] = GDN_SEQ_BAD_ACCEPT;
        else if (want && !persist) Pp.ws.seq_status[b] = GDN_SEQ_NOT_PERSISTED;
    }
    if (!new_ok) {  // a rejected new tree: NaN outputs, as verify writes them
        if (hf == 0)
            for (int i = 0; i < n; ++i) Pn.out[((size_t)(lo + i) * Pn.Hv + h) * D + row] = qnan_f();
    }
    if (!persist && !verified) return;

    // ---- the accepted path (lane e < 16 of every wave: entry e, root first) and the
    // new tree's path rows; each table's loads are issued before any test
    int pl = 0, len = 0;
    if (persist) {
        const int mu = uni(m), pl0 = uni(ip.x);
        pl = Pp.ws.nodepath[(size_t)(pl0 + mu) * GDN_MAX_DEPTH + lane % kPath];
        len = Pp.ws.depth[pl0 + mu];
    }
    int an[kPath], d = 0;
    if (verified && tid < n) {
        d = Pn.ws.depth[lo + tid];
#pragma unroll
        for (int e = 0; e < kPath; ++e) an[e] = Pn.ws.nodepath[(size_t)(lo + tid) * GDN_MAX_DEPTH + e];
    }
    len = uni(len);
    if (persist && h == 0 && tid < GDN_MAX_DEPTH) {
        Pp.ws.path[b * GDN_MAX_DEPTH + tid] = pl;
        if (tid == 0) Pp.ws.path_len[b] = len;
    }

    const PTab<D> Lp = fused_prev_carve<D>(lds_raw);
    const GTab<D> Ln = fused_new_carve<D>(lds_raw);
    const size_t kq_stride = (size_t)Pn.Hk * D;

    // previous step: path keys, values and gates (as the replay stages them), loaded below
    const uint16_t *kbp = static_cast<const uint16_t *>(Pp.k) + ((size_t)ip.x * Pp.Hk + g) * D;
    const uint16_t *vgp = static_cast<const uint16_t *>(Pp.v) + ((size_t)ip.x * Pp.Hv + h) * D;
    constexpr int KC = kPath * D / 8, K_PER = KC / NT;  // 16-byte chunks of the path keys
    constexpr int VC = kPath * D / 8;                    // and of the path values
    static_assert(KC % NT == 0 && KC % 64 == 0 && VC % 64 == 0, "whole table rounds");
    auto node_of = [&](int e) {
        const int x = __shfl(pl, e);  // every lane of the wave takes part in the shuffle
        return e < len ? max(x, 0) : 0;
    };
    // new step: keys and queries of the tree, the head's gates, the lane's values
    const uint16_t *kbn = static_cast<const uint16_t *>(Pn.k) + ((size_t)lo * Pn.Hk + g) * D;
    const uint16_t *qbn = static_cast<const uint16_t *>(Pn.q) + ((size_t)lo * Pn.Hk + g) * D;
    constexpr int KQ_PER = (2 * kTile * D / 8 + NT - 1) / NT;
    uint4 kqv[KQ_PER];
    uint16_t vraw[16];
    float nga = 0.0f, ngb = 0.0f;
    if (verified) {
#pragma unroll
        for (int u = 0; u < KQ_PER; ++u) {
            const int idx = tid + u * NT;
            const int which = idx / (kTile * (D / 8)), rem = idx % (kTile * (D / 8));
            const int i = rem / (D / 8), c8 = rem % (D / 8);
            kqv[u] = (which < 2 && i < n)
                         ? *reinterpret_cast<const uint4 *>((which ? qbn : kbn) + (size_t)i * kq_stride + 8 * c8)
                         : make_uint4(0, 0, 0, 0);
        }
        if (tid < n) {
            const size_t at = (size_t)(lo + tid) * Pn.Hv + h;
            nga = Pn.a[at];
            ngb = Pn.b[at];
        }
    }
    // previous step, wave 1 alone: it stages the path's keys, values and gates and forms
    // their Gram entries and coefficients, so no other wave waits for this round trip
    constexpr int K1 = KC / 64, V1 = VC / 64;  // 16-byte chunks per lane of wave 1
    uint4 kr[K1], vr[V1];
    float pga = 0.0f, pgb = 0.0f;
    if (persist && uni(w) == 1) {
        int nk[K1], nv[V1];
#pragma unroll
        for (int u = 0; u < K1; ++u) nk[u] = node_of(((lane + u * 64) / (D / 8)) % kPath);
#pragma unroll
        for (int u = 0; u < V1; ++u) nv[u] = node_of(((lane + u * 64) / (D / 8)) % kPath);
        const int ng = node_of(lane % kPath);
#pragma unroll
        for (int u = 0; u < K1; ++u)
            kr[u] = *reinterpret_cast<const uint4 *>(kbp + (size_t)nk[u] * Pp.Hk * D + 8 * ((lane + u * 64) % (D / 8)));
#pragma unroll
        for (int u = 0; u < V1; ++u)
            vr[u] = *reinterpret_cast<const uint4 *>(vgp + (size_t)nv[u] * Pp.Hv * D + 8 * ((lane + u * 64) % (D / 8)));
        const size_t at = (size_t)(ip.x + ng) * Pp.Hv + h;
        pga = Pp.a[at];
        pgb = Pp.b[at];
    }
    // the state (the persist's source: its previous slot) and the lane's values of the new
    // tree, issued right behind the tables so that waiting for the tables does not wait for them
    const float *s0 = Pn.state_in + ((size_t)slot * Pn.Hv + h) * D * D;
    const float *sp = Pn.state_in + ((size_t)(persist ? pslot : slot) * Pn.Hv + h) * D * D;
    const unsigned s_lane = (unsigned)(row * D + 4 * hf);
    const uint16_t *vl = static_cast<const uint16_t *>(Pn.v) + ((size_t)lo * Pn.Hv + h) * D + row;
    f32x16 SA[D / 32];
    auto issue_values = [&]() {
        if (verified) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r / 4) + 4 * hf + (r % 4);
                vraw[r] = i < n ? vl[(size_t)i * Pn.Hv * D] : (uint16_t)0;
            }
        }
    };

    // ---- the new tree's tables into LDS
    if (verified) {
        if (tid < n) {
#pragma unroll
            for (int e = 0; e < kPath; ++e) Ln.anc[tid * Q::PS + e] = an[e];
            Ln.depth[tid] = d;
            Ln.a[tid] = nga;
            Ln.b[tid] = ngb;
        }
#pragma unroll
        for (int u = 0; u < KQ_PER; ++u) {
            const int idx = tid + u * NT;
            if (idx < 2 * kTile * (D / 8))
                *reinterpret_cast<uint4 *>(Ln.kq + (idx / (D / 8)) * Q::KQ + 8 * (idx % (D / 8))) = kqv[u];
        }
        for (int idx = tid; idx < kTile * Q::MT / 2; idx += NT) {
            reinterpret_cast<uint32_t *>(Ln.mth)[idx] = 0u;
            reinterpret_cast<uint32_t *>(Ln.mtl)[idx] = 0u;
        }
    }
    __syncthreads();

    // ---- coefficients, while the states stream in: the new tree's on wave 0, the accepted
    // path's on wave 1 (after staging its tables), no barrier inside either (one wave's LDS
    // accesses take effect in program order)
    if (uni(w) == 0) {
        if (verified) group_coefficients<D, false, 1>(Ln, n, lane, hf, l32);
    } else {
        load_state_tiles<D>(sp, s_lane, SA);
        issue_values();
        if (uni(w) == 1 && persist) {
#pragma unroll
            for (int u = 0; u < K1; ++u) {
                const int idx = lane + u * 64, e = idx / (D / 8), c8 = idx % (D / 8);
                const uint4 kv = e < len ? kr[u] : make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(Lp.k + e * PTab<D>::KP + 8 * c8) = kv;
            }
            if (lane < kPath) {
                const bool on = lane < len;
                Lp.a[lane] = on ? pga : 1.0f;
                Lp.b[lane] = on ? pgb : 0.0f;
            }
            __builtin_amdgcn_wave_barrier();
            replay_gram<D, false>(Lp, l32, hf);
            __builtin_amdgcn_wave_barrier();
            if (lane < kPath) replay_coef_entry<D>(Lp, len, 0, lane);
        }
    }
    __syncthreads();
    if (uni(w) == 0) {
        load_state_tiles<D>(sp, s_lane, SA);
        issue_values();
    }
    if (persist) {
        // the coefficient scratch is spent: the replay's transposed keys (from the keys in
        // LDS) and its values take its place
#pragma unroll
        for (int u = 0; u < K_PER; ++u) {
            const int idx = tid + u * NT, e = idx / (D / 8), c8 = idx % (D / 8);
            const uint4 kv = *reinterpret_cast<const uint4 *>(Lp.k + e * PTab<D>::KP + 8 * c8);
            const uint16_t *hv = reinterpret_cast<const uint16_t *>(&kv);
#pragma unroll
            for (int i = 0; i < 8; ++i) Lp.kt[(8 * c8 + i) * PTab<D>::KT + e] = hv[i];
        }
        if (uni(w) == 1) {
#pragma unroll
            for (int u = 0; u < V1; ++u) {
                const int idx = lane + u * 64;
                reinterpret_cast<uint4 *>(Lp.v)[idx] = idx / (D / 8) < len ? vr[u] : make_uint4(0, 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- the persist: S <- the state after the accepted path, written in place
    if (persist) replay_head<D, false>(SA, Lp, 1, 0, len, l32, hf, row,
                                       Pn.state_out + ((size_t)pslot * Pn.Hv + h) * D * D, s_lane);
    if (!verified) return;
    if (persist && pslot != slot) load_state_tiles<D>(s0, s_lane, SA);  // the verify's own source

    // ---- the verify from the registers: X = S K^T, Y = S Q^T, k-step s over tile s/2,
    // registers 8(s%2) .. 8(s%2)+7 (columns 32t + 16u + 8(e/4) + 4*half + e%4)
    f32x16 ax = {}, ay = {};
    const uint16_t *krow = Ln.kq + l32 * Q::KQ, *qrow = Ln.kq + (kTile + l32) * Q::KQ;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int t = s / 2, u = s % 2;
        bf16x8 shi, slo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = SA[t][8 * u + e];
            const __bf16 hb = static_cast<__bf16>(x);
            shi[e] = hb;
            slo[e] = static_cast<__bf16>(x - static_cast<float>(hb));
        }
        const uint2 k0 = *reinterpret_cast<const uint2 *>(krow + 32 * t + 16 * u + 4 * hf);
        const uint2 k1 = *reinterpret_cast<const uint2 *>(krow + 32 * t + 16 * u + 8 + 4 * hf);
        const uint2 q0 = *reinterpret_cast<const uint2 *>(qrow + 32 * t + 16 * u + 4 * hf);
        const uint2 q1 = *reinterpret_cast<const uint2 *>(qrow + 32 * t + 16 * u + 8 + 4 * hf);
        const bf16x8 Ak = __builtin_bit_cast(bf16x8, make_uint4(k0.x, k0.y, k1.x, k1.y));
        const bf16x8 Aq = __builtin_bit_cast(bf16x8, make_uint4(q0.x, q0.y, q1.x, q1.y));
        ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, shi, ax, 0, 0, 0);
        ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, slo, ax, 0, 0, 0);
        ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, shi, ay, 0, 0, 0);
        ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, slo, ay, 0, 0, 0);
    }
    // r = b v - alpha x and gamma y in the accumulator layout (node 8(r/4) + 4*half + r%4)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r / 4) + 4 * hf + (r % 4);
        const float4 q4 = Ln.gab[min(i, n - 1)];
        ax[r] = i < n ? fmaf(-q4.y, ax[r], q4.z * bf2f(vraw[r])) : 0.0f;
        ay[r] = i < n ? q4.x * ay[r] : 0.0f;
    }
    // O = gamma y + MT R on bf16 MFMA, both operands split hi + lo (lo x lo dropped)
    const uint16_t *mh = Ln.mth + l32 * Q::MT, *ml = Ln.mtl + l32 * Q::MT;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const uint2 h0 = *reinterpret_cast<const uint2 *>(mh + 16 * u + 4 * hf);
        const uint2 h1 = *reinterpret_cast<const uint2 *>(mh + 16 * u + 8 + 4 * hf);
        const uint2 l0 = *reinterpret_cast<const uint2 *>(ml + 16 * u + 4 * hf);
        const uint2 l1 = *reinterpret_cast<const uint2 *>(ml + 16 * u + 8 + 4 * hf);
        const bf16x8 ahi = __builtin_bit_cast(bf16x8, make_uint4(h0.x, h0.y, h1.x, h1.y));
        const bf16x8 alo = __builtin_bit_cast(bf16x8, make_uint4(l0.x, l0.y, l1.x, l1.y));
        bf16x8 bhi, blo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float rv = ax[8 * u + e];
            const __bf16 rb = static_cast<__bf16>(rv);
            bhi[e] = rb;
            blo[e] = static_cast<__bf16>(rv - static_cast<float>(rb));
        }
        ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bhi, ay, 0, 0, 0);
        ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, blo, ay, 0, 0, 0);
        ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bhi, ay, 0, 0, 0);
    }
    const unsigned out_lane = (unsigned)(4 * hf * Pn.Hv * D + row);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int ir = 8 * (r / 4) + (r % 4);  // node of half-wave 0; half-wave 1 adds 4
        if (ir + 4 * hf < n) {
            float *ob = Pn.out + ((size_t)(lo + ir) * Pn.Hv + h) * D;
            ob[out_lane] = ay[r];
        }
    }
}

template <int D>
hipError_t launch_fused_d(const Params &pp, const Params &pn, hipStream_t s) {
    const size_t lds = fused_lds_bytes<D>();
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(persist_verify_kernel<D>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(persist_verify_kernel<D>, dim3(pn.B * pn.Hv), dim3(VG<D>::THREADS), lds, s, pp, pn);
    return hipGetLastError();
}

template <typename K>
hipError_t launch_with_lds(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, const Params &p) {
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kernel, grid, block, lds, s, p);
    return hipGetLastError();
}

// Workgroups of Kernel (threads, dynamic LDS) resident at once on the current device:
// compute units x workgroups per unit, queried once per (kernel, device, LDS size in
// KiB).  0 when unknown.
constexpr int kMaxDevices = 64;
constexpr int kLdsBuckets = 161;  // 0 .. 160 KiB
template <void (*Kernel)(Params)>
int resident_workgroups(int threads, size_t lds) {
    const auto kernel = Kernel;
    // one table per kernel; threads that race store the same value
    static std::atomic<int> cache[kMaxDevices][kLdsBuckets];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    const size_t kib = (lds + 1023) / 1024;
    if (kib >= (size_t)kLdsBuckets) return 0;
    std::atomic<int> &slot = cache[dev][kib];
    int known = slot.load(std::memory_order_relaxed);
    if (known == 0) {
        int cus = 0, per_cu = 0;
        if (lds > 65536 && hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kernel), threads,
                                                         lds) != hipSuccess)
            return 0;
        known = cus * per_cu;
        slot.store(known, std::memory_order_relaxed);
    }
    return known;
}

// Value heads per verify workgroup.  A key head's value heads share its Gram entries and
// coefficient tables, so a workgroup normally takes all of them; when a batch is small
// enough that one workgroup per value head are all resident at once, the heads run side by
// side instead of one after another (the shared tables are then formed once per head).
// GDN_VERIFY_HEADS=shared or =split fixes the choice (read on each call).
template <void (*OneHeadKernel)(Params)>
int heads_per_workgroup(const Params &p, int threads, size_t lds) {
    const int grp = p.Hv / p.Hk;
    if (grp == 1) return 1;
    const char *env = std::getenv("GDN_VERIFY_HEADS");
    if (env && std::strcmp(env, "shared") == 0) return grp;
    if (env && std::strcmp(env, "split") == 0) return 1;
    const int resident = resident_workgroups<OneHeadKernel>(threads, lds);
    return resident > 0 && (long long)p.B * p.Hv <= resident ? 1 : grp;
}

// trees of at most 32 nodes (and chains): one workgroup per key head and its value
// heads, which share the coefficients' Gram entries; trees of up to 96 nodes: the same
// over node blocks (bf16 inputs); else (larger trees, fp32 inputs past 32 nodes, or more
// than 4 value heads per key head at a batch too large to split them) coefficients + verify
template <int D, bool F32>
hipError_t launch_verify_d(const Params &p, bool chain, hipStream_t s) {
    const int grp = p.Hv / p.Hk;
    const int hpw = chain ? heads_per_workgroup<verify_group_kernel<D, true, 1, F32>>(p, VG<D>::THREADS,
                                                                                     gtab_bytes<D>(1, F32))
                          : heads_per_workgroup<verify_group_kernel<D, false, 1, F32>>(p, VG<D>::THREADS,
                                                                                      gtab_bytes<D>(1, F32));
    if ((chain || p.max_nodes <= kTile) && hpw <= kGroupMaxHeads) {
        const dim3 grid(p.B * (p.Hv / hpw)), block(VG<D>::THREADS);
        const size_t lds = gtab_bytes<D>(hpw, F32);
        switch (hpw) {
#define GDN_GROUP_CASE(G)                                                                         \
    case G:                                                                                       \
        return chain ? launch_with_lds(verify_group_kernel<D, true, G, F32>, grid, block, lds, s, p) \
                     : launch_with_lds(verify_group_kernel<D, false, G, F32>, grid, block, lds, s, p);
            GDN_GROUP_CASE(1)
            GDN_GROUP_CASE(2)
            GDN_GROUP_CASE(3)
            GDN_GROUP_CASE(4)
#undef GDN_GROUP_CASE
        }
    }
    if constexpr (!F32) {
        const bool two = p.max_nodes <= 2 * kTile;
        const int gb = !chain && p.max_nodes <= 3 * kTile
                           ? (two ? heads_per_workgroup<verify_blocks_kernel<D, 2, 1>>(
                                        p, VG<D>::THREADS, blocks_layout<D>(p.max_nodes, 1).total)
                                  : heads_per_workgroup<verify_blocks_kernel<D, 3, 1>>(
                                        p, VG<D>::THREADS, blocks_layout<D>(p.max_nodes, 1).total))
                           : grp;
        if (!chain && p.max_nodes <= 3 * kTile && gb <= kGroupMaxHeads) {
            const dim3 grid(p.B * (p.Hv / gb)), block(VG<D>::THREADS);
            const size_t lds = blocks_layout<D>(p.max_nodes, gb).total;
            switch (gb) {
#define GDN_BLOCKS_CASE(G)                                                                      \
    case G:                                                                                     \
        return two ? launch_with_lds(verify_blocks_kernel<D, 2, G>, grid, block, lds, s, p) \
                   : launch_with_lds(verify_blocks_kernel<D, 3, G>, grid, block, lds, s, p);
                GDN_BLOCKS_CASE(1)
                GDN_BLOCKS_CASE(2)
                GDN_BLOCKS_CASE(3)
                GDN_BLOCKS_CASE(4)
#undef GDN_BLOCKS_CASE
            }
        }
    }
    const int cap = chain ? kPath : p.max_nodes;
    // LDS for the most value heads a pass can take (a one-node sequence)
    const size_t clds = ctab_bytes(cap, grp, coef_heads_per_pass(cap, grp));
    hipError_t e = chain ? launch_with_lds(coef_kernel<D, true, F32>, dim3(p.B * p.Hk), dim3(kCoefThreads), clds, s, p)
                         : launch_with_lds(coef_kernel<D, false, F32>, dim3(p.B * p.Hk), dim3(kCoefThreads), clds, s, p);
    if (e != hipSuccess) return e;
    const dim3 grid(p.B * p.Hv), block(VG<D>::THREADS);
    if (chain)
        return launch_with_lds(verify_kernel<D, true, 1, F32>, grid, block, vtab_bytes(kPath, D, true, F32), s, p);
    if (p.max_nodes <= kTile)
        return launch_with_lds(verify_kernel<D, false, 1, F32>, grid, block, vtab_bytes(p.max_nodes, D, true, F32), s,
                               p);
    if (p.max_nodes <= 3 * kTile)
        return launch_with_lds(verify_kernel<D, false, 3, F32>, grid, block, vtab_bytes(p.max_nodes, D, false), s, p);
    return launch_with_lds(verify_kernel<D, false, kFastMaxNodes / kTile, F32>, grid, block,
                           vtab_bytes(p.max_nodes, D, false), s, p);
}

// one workgroup per value head: four fit a CU, and their independent rounds overlap
// reading and writing better than a key head's workgroup walking its value heads
template <int D, bool F32>
hipError_t launch_replay_d(const Params &p, bool chain, hipStream_t s) {
    const dim3 grid(p.B * p.Hv), block(VG<D>::THREADS);
    return chain ? launch_with_lds(replay_kernel<D, true, F32>, grid, block, ptab_bytes<D>(1, F32), s, p)
                 : launch_with_lds(replay_kernel<D, false, F32>, grid, block, ptab_bytes<D>(1, F32), s, p);
}

template <int D, bool F32>
hipError_t launch_chunks_d(const Params &p, hipStream_t s) {
    return launch_with_lds(chain_chunks_kernel<D, F32>, dim3(p.B * p.Hv), dim3(VG<D>::THREADS), cktab_bytes<D>(F32), s,
                           p);
}
hipError_t chunks_any(const Params &p, hipStream_t s) {
    if (p.f32_in) return p.D == 64 ? launch_chunks_d<64, true>(p, s) : launch_chunks_d<128, true>(p, s);
    return p.D == 64 ? launch_chunks_d<64, false>(p, s) : launch_chunks_d<128, false>(p, s);
}

template <bool F32>
hipError_t verify_any_d(const Params &p, bool chain, hipStream_t s) {
    return p.D == 64 ? launch_verify_d<64, F32>(p, chain, s) : launch_verify_d<128, F32>(p, chain, s);
}
hipError_t verify_any(const Params &p, bool chain, hipStream_t s) {
    return p.f32_in ? verify_any_d<true>(p, chain, s) : verify_any_d<false>(p, chain, s);
}
template <bool F32>
hipError_t replay_any_d(const Params &p, bool chain, hipStream_t s) {
    return p.D == 64 ? launch_replay_d<64, F32>(p, chain, s) : launch_replay_d<128, F32>(p, chain, s);
}
hipError_t replay_any(const Params &p, bool chain, hipStream_t s) {
    return p.f32_in ? replay_any_d<true>(p, chain, s) : replay_any_d<false>(p, chain, s);
}

}  // namespace

bool fast_path_supported(int D, int dtype) { return (D == 64 || D == 128) && (dtype == GDN_BF16 || dtype == GDN_F32); }
// Trees of up to 96 nodes run the group or block kernels, larger ones the coefficient
// + verify pair, whose tables must fit one compute unit's LDS (fp32 inputs take the pair
// from 33 nodes on)
bool fast_tree_supported(int D, int dtype, int max_nodes, int heads_per_key) {
    if (!fast_path_supported(D, dtype) || max_nodes > kFastMaxNodes) return false;
    return coef_heads_per_pass(max_nodes, heads_per_key) > 0 && vtab_bytes(max_nodes, D, false) <= kLdsBudget;
}

hipError_t launch_tree_verify_fast(const Params &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    return verify_any(p, false, s);
}
hipError_t launch_persist_fast(const Params &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    return replay_any(p, false, s);
}
// The fused persist + verify: bf16 inputs, D 64 or 128, new trees of at most 32 nodes.
bool fused_supported(int D, int dtype, int max_nodes) {
    return (D == 64 || D == 128) && dtype == GDN_BF16 && max_nodes <= kTile;
}
hipError_t launch_persist_verify_fast(const Params &prev, const Params &next, hipStream_t s) {
    if (next.B == 0) return hipSuccess;
    return next.D == 64 ? launch_fused_d<64>(prev, next, s) : launch_fused_d<128>(prev, next, s);
}
// Chains of at most 16 nodes: outputs from the verify kernel in chain order
// (so a chain-shaped tree and a chain give the same bits) and the final state
// from the replay kernel (so persist and chain give the same bits).  Longer
// chains: the chunked chain kernel, state in registers across chunks.
hipError_t launch_chain_verify_fast(const Params &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    if (p.max_nodes > kPath) return chunks_any(p, s);
    hipError_t e = hipSuccess;
    if (p.out || p.has_ws) e = verify_any(p, true, s);
    if (e != hipSuccess) return e;
    if (p.final_state) e = replay_any(p, true, s);
    return e;
}

}  // namespace gdn

// gdn_fast.hip -- tree verify and accepted-path replay on the matrix cores for
// D in {64, 128} with bf16 q/k/v.
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
// as a rank-16 update accumulated onto the scaled state.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 32;             // nodes per MFMA block
constexpr int kPath = GDN_MAX_DEPTH;  // max ancestors per node (incl. itself)
constexpr int kFastMaxNodes = 96;     // largest tree the MFMA verify takes (3 node blocks)

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
__device__ __forceinline__ float qnan_f() { return __int_as_float(0x7fc00000); }
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// one load, no short-circuit: the test does not hold back the loads issued next to it
__device__ __forceinline__ bool ws_planned(const Params &P) {
    const int4 h = *reinterpret_cast<const int4 *>(P.ws.header);
    return (h.x == (int)kMagic) & (h.y == P.B) & (h.z == P.T);
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
    int *depth;      // [cap]
    uint32_t *amask; // [cap][4]
    float *gk, *gq;  // [cap][16] path-indexed Gram entries
    float *a, *b;    // [grp][cap]
    float *coefL;    // [hpp][cap][16]
};

__host__ __device__ inline size_t ctab_bytes(int cap, int grp, int hpp) {
    const size_t c = (size_t)cap;
    return c * kPath * 4 + c * 4 + c * 16 + 2 * c * kPath * 4 + 2 * (size_t)grp * c * 4 + (size_t)hpp * c * kPath * 4;
}

__device__ inline CTab ctab_carve(char *base, int cap, int grp, int hpp) {
    CTab L;
    const size_t c = (size_t)cap;
    L.anc = reinterpret_cast<int *>(base);        base += c * kPath * 4;
    L.gk = reinterpret_cast<float *>(base);       base += c * kPath * 4;
    L.gq = reinterpret_cast<float *>(base);       base += c * kPath * 4;
    L.coefL = reinterpret_cast<float *>(base);    base += (size_t)hpp * c * kPath * 4;
    L.amask = reinterpret_cast<uint32_t *>(base); base += c * 16;
    L.depth = reinterpret_cast<int *>(base);      base += c * 4;
    L.a = reinterpret_cast<float *>(base);        base += (size_t)grp * c * 4;
    L.b = reinterpret_cast<float *>(base);
    return L;
}

template <int D, bool CHAIN>
__global__ __launch_bounds__(kCoefThreads) void coef_kernel(Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    constexpr int KS = D / 16;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int grp = P.Hv / P.Hk;
    const int b = blockIdx.x / P.Hk, g = blockIdx.x % P.Hk;
    const SeqView sv = seq_view<CHAIN>(P, b);
    if (!CHAIN && !ws_planned(P)) return;
    if (sv.status != GDN_SEQ_OK || sv.n == 0) return;
    const int lo = sv.lo, n = sv.n;
    const int cap = CHAIN ? kPath : P.max_nodes;
    const int hpp = max(1, min(min(grp, kCoefMaxHeadsPerPass), kCoefThreads / n));  // value heads per pass
    const CTab L = ctab_carve(lds_raw, cap, grp, hpp);

    // tree tables and ancestor masks, gates of every head of the group
    for (int i = tid; i < n; i += kCoefThreads) {
        int an[kPath];
#pragma unroll
        for (int e = 0; e < kPath; ++e) an[e] = anc_of<CHAIN>(P, lo, i, e);
        const int d = CHAIN ? i + 1 : P.ws.depth[lo + i];
        uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < kPath; ++e) {
            L.anc[i * kPath + e] = an[e];
            if (e < d) m[an[e] >> 5] |= 1u << (an[e] & 31);
        }
        L.depth[i] = d;
        *reinterpret_cast<uint4 *>(L.amask + i * 4) = make_uint4(m[0], m[1], m[2], m[3]);
    }
    for (int idx = tid; idx < grp * n; idx += kCoefThreads) {
        const int hh = idx / n, i = idx % n;
        const size_t at = (size_t)(lo + i) * P.Hv + g * grp + hh;
        L.a[hh * cap + i] = P.a[at];
        L.b[hh * cap + i] = P.b[at];
    }
    __syncthreads();

    // Gram entries for every (ancestor, node) pair on the matrix cores
    const uint16_t *kb = static_cast<const uint16_t *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const uint16_t *qb = static_cast<const uint16_t *>(P.q) + ((size_t)lo * P.Hk + g) * D;
    const size_t kq_stride = (size_t)P.Hk * D;
    const int ntiles = (n + kTile - 1) / kTile;
    for (int pair = w; pair < ntiles * ntiles; pair += kCoefThreads / 64) {
        const int ti = pair % ntiles, tj = pair / ntiles;
        const int pi = ti * kTile + l32, pj = tj * kTile + l32;
        f32x16 gkk = {}, gkq = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 A = pi < n ? frag_of(kb + (size_t)pi * kq_stride, s, hf) : zero_frag();
            const bf16x8 Bk = pj < n ? frag_of(kb + (size_t)pj * kq_stride, s, hf) : zero_frag();
            const bf16x8 Bq = pj < n ? frag_of(qb + (size_t)pj * kq_stride, s, hf) : zero_frag();
            gkk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bk, gkk, 0, 0, 0);
            gkq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bq, gkq, 0, 0, 0);
        }
        if (pj < n) {  // accumulator r: (candidate ancestor ti*32 + il, node pj)
            const uint32_t mask = L.amask[pj * 4 + ti];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int il = 8 * (r / 4) + 4 * hf + (r % 4);
                if ((mask >> il) & 1u) {
                    const int e = L.depth[ti * kTile + il] - 1;
                    L.gk[pj * kPath + e] = gkk[r];
                    L.gq[pj * kPath + e] = gkq[r];
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
            float av[kPath];
#pragma unroll
            for (int e = 0; e < kPath; ++e) an[e] = L.anc[i * kPath + e];
#pragma unroll
            for (int e = 0; e < kPath; ++e) av[e] = e < d ? L.a[hh * cap + an[e]] : 1.0f;
            float r = 1.0f;
#pragma unroll
            for (int e = kPath - 1; e >= 0; --e) {
                const bool on = e < d - 1;
                L.coefL[(slot_h * cap + i) * kPath + e] = on ? bi * r * L.gk[i * kPath + e] : 0.0f;
                mrow[e] = on ? r * L.gq[i * kPath + e] : (e == d - 1 ? L.gq[i * kPath + e] : 0.0f);
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
    uint16_t *kq;   // [2][32][D] bf16 keys / queries (single-block trees)
    float *mt;      // [32][32] dense MT (single-block trees)
    float *rbuf;    // [cap][D] r rows (multi-block trees)
    float *y;       // [cap][16] path weights
    int *anc;       // [cap][16]
    float4 *gabd;   // [cap] gamma, alpha, b, depth
};

__host__ __device__ inline size_t vtab_bytes(int cap, int D, bool single) {
    const size_t c = (size_t)cap;
    return (single ? (size_t)2 * kTile * D * 2 + (size_t)kTile * kTile * 4 : c * D * 4) + 2 * c * kPath * 4 + c * 16;
}

__device__ inline VTab vtab_carve(char *base, int cap, int D, bool single) {
    VTab L;
    const size_t c = (size_t)cap;
    L.gabd = reinterpret_cast<float4 *>(base);  base += c * 16;
    L.kq = reinterpret_cast<uint16_t *>(base);  base += single ? (size_t)2 * kTile * D * 2 : 0;
    L.mt = reinterpret_cast<float *>(base);     base += single ? (size_t)kTile * kTile * 4 : 0;
    L.rbuf = reinterpret_cast<float *>(base);   base += single ? 0 : c * D * 4;
    L.y = reinterpret_cast<float *>(base);      base += c * kPath * 4;
    L.anc = reinterpret_cast<int *>(base);
    return L;
}

template <int D, bool CHAIN, int MT>
__global__ __launch_bounds__(VG<D>::THREADS) __attribute__((amdgpu_waves_per_eu(3))) void verify_kernel(Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int row = w * 32 + l32;
    const int b = blockIdx.x / P.Hv, h = blockIdx.x % P.Hv;
    const int g = h / (P.Hv / P.Hk);
    const size_t out_stride = (size_t)P.Hv * D;
    const SeqView sv = seq_view<CHAIN>(P, b);  // loaded together with the header check below
    if (!CHAIN && !ws_planned(P)) return;
    if (CHAIN && P.has_ws && h == 0 && tid == 0) {
        if (b == 0) {
            P.ws.header[0] = kMagic;
            P.ws.header[1] = P.B;
            P.ws.header[2] = P.T;
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
    const VTab L = vtab_carve(lds_raw, cap, D, kSingle);
    const uint16_t *kb = static_cast<const uint16_t *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const uint16_t *qb = static_cast<const uint16_t *>(P.q) + ((size_t)lo * P.Hk + g) * D;
    const uint16_t *vb = static_cast<const uint16_t *>(P.v) + ((size_t)lo * P.Hv + h) * D + row;
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
    constexpr int KQ_PER = kSingle ? (2 * kTile * D / 8 + VG<D>::THREADS - 1) / VG<D>::THREADS : 1;
    uint4 kqv[KQ_PER];
    if (kSingle) {
#pragma unroll
        for (int u = 0; u < KQ_PER; ++u) {
            const int idx = tid + u * VG<D>::THREADS;
            const int which = idx / (kTile * (D / 8)), rem = idx % (kTile * (D / 8));
            const int i = rem / (D / 8), c8 = rem % (D / 8);
            kqv[u] = (which < 2 && i < n)
                         ? *reinterpret_cast<const uint4 *>((which ? qb : kb) + (size_t)i * kq_stride + 8 * c8)
                         : make_uint4(0, 0, 0, 0);
        }
    }
    uint16_t vraw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r / 4) + 4 * hf + (r % 4);
        vraw[r] = i < n ? vb[(size_t)i * v_stride] : uint16_t(0);
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
#pragma unroll
        for (int e = 0; e < kPath; e += 4)
            *reinterpret_cast<int4 *>(L.anc + i * kPath + e) = make_int4(an[e], an[e + 1], an[e + 2], an[e + 3]);
        L.gabd[i] = gabd;
    }
    if (kSingle) {
#pragma unroll
        for (int u = 0; u < KQ_PER; ++u) {
            const int idx = tid + u * VG<D>::THREADS;
            if (idx < 2 * kTile * (D / 8)) reinterpret_cast<uint4 *>(L.kq)[idx] = kqv[u];
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
            ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, shi[s], ax, 0, 0, 0);
            ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, slo[s], ax, 0, 0, 0);
            ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, shi[s], ay, 0, 0, 0);
            ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, slo[s], ay, 0, 0, 0);
        }
        f32x16 rr, oo;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r / 4) + 4 * hf + (r % 4);
            const float4 gabd = L.gabd[min(i, n - 1)];
            rr[r] = i < n ? fmaf(-gabd.y, ax[r], gabd.z * bf2f(vraw[r])) : 0.0f;
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
                    vraw[r] = i < n ? vb[(size_t)i * v_stride] : uint16_t(0);
                }
            }
            const int pi = t * kTile + l32;
            f32x16 ax = {};
#pragma unroll
            for (int s = 0; s < VG<D>::KS; ++s) {
                const bf16x8 Ak = pi < n ? frag_of(kb + (size_t)pi * kq_stride, s, hf) : zero_frag();
                ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, shi[s], ax, 0, 0, 0);
                ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, slo[s], ax, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = t * kTile + 8 * (r / 4) + 4 * hf + (r % 4);
                if (i < n) {
                    const float4 gabd = L.gabd[i];
                    L.rbuf[(size_t)i * D + row] = fmaf(-gabd.y, ax[r], gabd.z * bf2f(vraw[r]));
                }
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
                const bf16x8 Aq = pi < n ? frag_of(qb + (size_t)pi * kq_stride, s, hf) : zero_frag();
                ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, shi[s], ay, 0, 0, 0);
                ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, slo[s], ay, 0, 0, 0);
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
// value heads, or one when a small batch leaves room for a workgroup per head.  One round trip brings the keys,
// queries, values, gates and paths into LDS; the first two heads' states are
// issued as soon as those have landed (issued with them they would queue ahead
// of them).  While the states arrive the workgroup forms the coefficients once
// for all its heads (the Gram entries are shared through the key head); then
// each head's products are taken as its state lands, and a register set takes
// the next head's state as soon as its products are done.  No barrier after
// the coefficients.  Same algebra as the two-kernel path (coef_kernel +
// verify_kernel).
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
    uint16_t *kq;     // [2][32][KQ] keys / queries (bf16)
    uint16_t *v;      // [32][grp][D] values of the group's heads (bf16), node-major as in memory
    float4 *gab;      // [grp][32] gamma, alpha, b
    uint16_t *mth, *mtl;  // [grp][32][MT] dense output operator, bf16 hi and lo parts
    float *coefL;     // [grp][32][PS]
    float *gk, *gq;   // [32][PS] path-indexed Gram entries
    int *anc;         // [32][PS] root-to-node path, -1 past the depth
    float *a, *b;     // [grp][32]
    int *depth;       // [32]
};

template <int D>
__host__ __device__ inline size_t gtab_bytes(int grp) {
    using Q = GPad<D>;
    return (size_t)2 * kTile * Q::KQ * 2 + (size_t)kTile * grp * D * 2 + (size_t)grp * kTile * 16 +
           (size_t)grp * kTile * Q::MT * 4 + (size_t)grp * kTile * Q::PS * 4 + 3 * kTile * Q::PS * 4 +
           2 * (size_t)grp * kTile * 4 + kTile * 4;
}

template <int D>
__device__ inline GTab<D> gtab_carve(char *base, int grp) {
    using Q = GPad<D>;
    GTab<D> L;
    L.kq = reinterpret_cast<uint16_t *>(base);     base += (size_t)2 * kTile * Q::KQ * 2;
    L.v = reinterpret_cast<uint16_t *>(base);      base += (size_t)kTile * grp * D * 2;
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

template <int D, bool CHAIN, int HPW>
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
    if (!CHAIN && !ws_planned(P)) return;
    if (CHAIN && P.has_ws && h0 == 0 && tid == 0) {
        if (b == 0) {
            P.ws.header[0] = kMagic;
            P.ws.header[1] = P.B;
            P.ws.header[2] = P.T;
        }
        P.ws.seq_status[b] = sv.status;
    }
    if (!P.out) return;
    const int lo = sv.lo, n = sv.n;
    // out[node][h0 + hh][row]: uniform base per (node, head) + this lane's offset
    const unsigned out_lane = (unsigned)(4 * hf * P.Hv * D + row);
    if (sv.status != GDN_SEQ_OK) {
        for (int t = tid; t < n * grp * D; t += NT)
            P.out[((size_t)(lo + t / (grp * D)) * P.Hv + h0) * D + t % (grp * D)] = qnan_f();
        return;
    }
    if (n == 0) return;
    using Q = GPad<D>;
    const GTab<D> L = gtab_carve<D>(lds_raw, grp);
    const uint16_t *kb = static_cast<const uint16_t *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const uint16_t *qb = static_cast<const uint16_t *>(P.q) + ((size_t)lo * P.Hk + g) * D;
    const size_t kq_stride = (size_t)P.Hk * D;
    const float *s0 = P.state_in + ((size_t)sv.slot * P.Hv + h0) * D * D;
    const unsigned s_lane = (unsigned)(row * D + 8 * hf);

    // ---- one round trip: keys/queries, all heads' values, tree, gates
    constexpr int KQ_PER = (2 * kTile * D / 8 + NT - 1) / NT;
    uint4 kqv[KQ_PER];
#pragma unroll
    for (int u = 0; u < KQ_PER; ++u) {
        const int idx = tid + u * NT;
        const int which = idx / (kTile * (D / 8)), rem = idx % (kTile * (D / 8));
        const int i = rem / (D / 8), c8 = rem % (D / 8);
        kqv[u] = (which < 2 && i < n)
                     ? *reinterpret_cast<const uint4 *>((which ? qb : kb) + (size_t)i * kq_stride + 8 * c8)
                     : make_uint4(0, 0, 0, 0);
    }
    // values: node i's group heads are contiguous (grp*D bf16); kGroupMaxHeads*32*D/8/NT chunks at most
    const uint16_t *vg = static_cast<const uint16_t *>(P.v) + ((size_t)lo * P.Hv + h0) * D;
    const int vchunks = grp * D / 8;  // 16-byte chunks per node
    constexpr int V_PER = (kGroupMaxHeads * kTile * D / 8 + NT - 1) / NT;
    static_assert(kGroupMaxHeads * kTile <= NT, "one thread per (head, node) gate");
    uint4 vv[V_PER];
#pragma unroll
    for (int u = 0; u < V_PER; ++u) {
        const int idx = tid + u * NT;
        const int i = idx / vchunks, c = idx % vchunks;
        vv[u] = i < n ? *reinterpret_cast<const uint4 *>(vg + (size_t)i * P.Hv * D + 8 * c) : make_uint4(0, 0, 0, 0);
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
        if (idx < 2 * kTile * (D / 8))
            *reinterpret_cast<uint4 *>(L.kq + (idx / (D / 8)) * Q::KQ + 8 * (idx % (D / 8))) = kqv[u];
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
    // the states go out only now: issued together with the small loads above they would queue
    // ahead of them and hold back the coefficients, which gate every output
    float sA[KS][8], sB[KS][8];
    load_state_frags<D>(s0, s_lane, sA);
    if (grp > 1) load_state_frags<D>(s0 + (size_t)D * D, s_lane, sB);
    __syncthreads();

    // ---- Gram entries of the block (one wave)
    if (w == 0) {
        f32x16 gkk = {}, gkq = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 A = frag_of(L.kq + l32 * Q::KQ, s, hf);
            const bf16x8 Bq = frag_of(L.kq + (kTile + l32) * Q::KQ, s, hf);
            gkk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, A, gkk, 0, 0, 0);
            gkq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bq, gkq, 0, 0, 0);
        }
        if (l32 < n) {  // accumulator r: (candidate ancestor il, node l32)
            const int dl = L.depth[l32];
            uint32_t mask = 0u;  // ancestors of node l32 within the block
#pragma unroll
            for (int e = 0; e < kPath; ++e)
                if (e < dl) mask |= 1u << (L.anc[l32 * Q::PS + e] & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int il = 8 * (r / 4) + 4 * hf + (r % 4);
                if ((mask >> il) & 1u) {
                    const int e = L.depth[il] - 1;
                    L.gk[l32 * Q::PS + e] = gkk[r];
                    L.gq[l32 * Q::PS + e] = gkq[r];
                }
            }
        }
    }
    __syncthreads();

    // ---- per (value head, node): ratios, coefficients, output weights
    const bool act = tid < grp * n;
    const int hh_t = act ? tid / n : 0, i_t = act ? tid % n : 0;
    float mrow[kPath];
    int an_t[kPath];
    int d_t = 0;
    if (act) {
        d_t = L.depth[i_t];
        const float bi = L.b[hh_t * kTile + i_t];
        float av[kPath];
#pragma unroll
        for (int e = 0; e < kPath; ++e) an_t[e] = max(L.anc[i_t * Q::PS + e], 0);
#pragma unroll
        for (int e = 0; e < kPath; ++e) av[e] = e < d_t ? L.a[hh_t * kTile + an_t[e]] : 1.0f;
        float r = 1.0f;
#pragma unroll
        for (int e = kPath - 1; e >= 0; --e) {
            const bool on = e < d_t - 1;
            L.coefL[(hh_t * kTile + i_t) * Q::PS + e] = on ? bi * r * L.gk[i_t * Q::PS + e] : 0.0f;
            mrow[e] = on ? r * L.gq[i_t * Q::PS + e] : (e == d_t - 1 ? L.gq[i_t * Q::PS + e] : 0.0f);
            r *= av[e];
        }
        L.gab[hh_t * kTile + i_t] = make_float4(r, bi * r, bi, 0.0f);
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
                acc = fmaf(-y[f], L.coefL[(hh_t * kTile + an_t[f]) * Q::PS + e], acc);
            y[e] = e < d_t ? acc : 0.0f;
        }
        uint16_t *mh = L.mth + (hh_t * kTile + i_t) * Q::MT, *ml = L.mtl + (hh_t * kTile + i_t) * Q::MT;
#pragma unroll
        for (int e = 0; e < kPath; ++e)
            if (e < d_t) {  // stored as bf16 hi + lo for the matrix cores
                const __bf16 yh = static_cast<__bf16>(y[e]);
                mh[an_t[e]] = __builtin_bit_cast(uint16_t, yh);
                ml[an_t[e]] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(y[e] - static_cast<float>(yh)));
            }
    }
    __syncthreads();

    // ---- value heads: X, Y from the state and K/Q; outputs from X, Y and the coefficients
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
            ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, shi, ax, 0, 0, 0);
            ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, slo, ax, 0, 0, 0);
            ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, shi, ay, 0, 0, 0);
            ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, slo, ay, 0, 0, 0);
        }
    };
    auto finish = [&](f32x16 ax, f32x16 ay, int hh) {
        const float4 *gab = L.gab + hh * kTile;
        const uint16_t *vh = L.v + hh * D + row;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 8 * (r / 4) + 4 * hf + (r % 4);
            const float4 q4 = gab[min(i, n - 1)];
            const float vi = bf2f(vh[i * grp * D]);
            ax[r] = i < n ? fmaf(-q4.y, ax[r], q4.z * vi) : 0.0f;  // r = b v - alpha x
            ay[r] = i < n ? q4.x * ay[r] : 0.0f;                   // gamma y
        }
        // O = gamma y + MT R on bf16 MFMA with both operands split hi + lo (the lo x lo
        // term, ~2^-32 relative, is dropped).  k-step u takes R from accumulator slots
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
    f32x16 x0, y0;
    xy(sA, x0, y0);
    finish(x0, y0, 0);
    if (grp > 2) load_state_frags<D>(s0 + (size_t)2 * D * D, s_lane, sA);
    if (grp > 1) {
        f32x16 x1, y1;
        xy(sB, x1, y1);
        finish(x1, y1, 1);
        if (grp > 3) load_state_frags<D>(s0 + (size_t)3 * D * D, s_lane, sB);
    }
    if (grp > 2) {
        f32x16 x2, y2;
        xy(sA, x2, y2);
        finish(x2, y2, 2);
    }
    if (grp > 3) {
        f32x16 x3, y3;
        xy(sB, x3, y3);
        finish(x3, y3, 3);
    }
}

// ===========================================================================
// Verify for trees of 33 .. 96 nodes: NB node blocks of 32, one workgroup per
// (sequence, group of GRP value heads of one key head: all of them, or one for a
// small batch), one workgroup per CU (the keys and queries of all blocks stay in
// LDS).  The Gram entries k.k and k.q of every
// block pair and the per-(head, node) coefficients are formed once; ancestors
// may sit in any block, so each head first takes X_j = K_j S0^T for all blocks
// (R_j = diag(b)V_j - diag(alpha)X_j kept in registers), then per block t
// O_t = diag(gamma)Y_t + sum_j MT_tj R_j, with MT (the output operator, rows
// from the 16-step back substitution) dense in LDS: cleared once, its entries
// (the same places, the ancestors, for every head) rewritten per head.
// All products run on bf16 MFMA with fp32 operands split hi + lo.
// ===========================================================================
template <int D, int NB>
struct BPad {
    static constexpr int NN = NB * kTile;  // node slots
    static constexpr int KQ = D + 8;       // bf16 per key/query row
    static constexpr int PS = kPath + 1;   // per-node path tables
    static constexpr int MS = NN + 8;      // bf16 per output-operator row
};

template <int D, int NB>
struct BTab {
    uint16_t *kq;         // [2][NN][KQ] keys, queries
    uint16_t *vst;        // [NN][D] values of the current head
    float4 *gab;          // [grp][NN] gamma, alpha, b
    float *ysp;           // [grp][NN][16] output weights by path position
    float *gk, *gq;       // [NN][PS]       (these three and the next share one region:
    float *coefL;         // [grp][NN][PS]   the Gram entries and coefficients die before
    uint16_t *mth, *mtl;  // [NN][MS]        the output operator is built)
    int *anc;             // [NN][PS] root-to-node path, -1 past the depth
    float *a, *b;         // [grp][NN]
    int *depth;           // [NN]
};

template <int D, int NB>
__host__ __device__ inline size_t btab_bytes(int grp) {
    using Q = BPad<D, NB>;
    const size_t u1 = (size_t)2 * Q::NN * Q::PS * 4 + (size_t)grp * Q::NN * Q::PS * 4;
    const size_t u2 = (size_t)2 * Q::NN * Q::MS * 2;
    return (size_t)2 * Q::NN * Q::KQ * 2 + (size_t)Q::NN * D * 2 + (size_t)grp * Q::NN * 16 +
           (size_t)grp * Q::NN * kPath * 4 + (u1 > u2 ? u1 : u2) + (size_t)Q::NN * Q::PS * 4 +
           2 * (size_t)grp * Q::NN * 4 + (size_t)Q::NN * 4;
}

template <int D, int NB>
__device__ inline BTab<D, NB> btab_carve(char *base, int grp) {
    using Q = BPad<D, NB>;
    BTab<D, NB> L;
    L.kq = reinterpret_cast<uint16_t *>(base);   base += (size_t)2 * Q::NN * Q::KQ * 2;
    L.vst = reinterpret_cast<uint16_t *>(base);  base += (size_t)Q::NN * D * 2;
    L.gab = reinterpret_cast<float4 *>(base);    base += (size_t)grp * Q::NN * 16;
    L.ysp = reinterpret_cast<float *>(base);     base += (size_t)grp * Q::NN * kPath * 4;
    char *u = base;
    const size_t u1 = (size_t)2 * Q::NN * Q::PS * 4 + (size_t)grp * Q::NN * Q::PS * 4;
    const size_t u2 = (size_t)2 * Q::NN * Q::MS * 2;
    base += u1 > u2 ? u1 : u2;
    L.gk = reinterpret_cast<float *>(u);
    L.gq = L.gk + Q::NN * Q::PS;
    L.coefL = L.gq + Q::NN * Q::PS;
    L.mth = reinterpret_cast<uint16_t *>(u);
    L.mtl = L.mth + Q::NN * Q::MS;
    L.anc = reinterpret_cast<int *>(base);       base += (size_t)Q::NN * Q::PS * 4;
    L.a = reinterpret_cast<float *>(base);       base += (size_t)grp * Q::NN * 4;
    L.b = reinterpret_cast<float *>(base);       base += (size_t)grp * Q::NN * 4;
    L.depth = reinterpret_cast<int *>(base);
    return L;
}

template <int D, int NB, int GRP>
__global__ __launch_bounds__(VG<D>::THREADS) __attribute__((amdgpu_waves_per_eu(1))) void verify_blocks_kernel(
    Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    using Q = BPad<D, NB>;
    constexpr int KS = VG<D>::KS, NT = VG<D>::THREADS, WAVES = VG<D>::WAVES, NN = Q::NN;
    constexpr int grp = GRP;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64, hf = lane / 32, l32 = lane % 32;
    const int row = w * 32 + l32;
    const int nhg = P.Hv / grp;  // workgroups per sequence
    const int b = blockIdx.x / nhg, h0 = blockIdx.x % nhg * grp;
    const int g = h0 / (P.Hv / P.Hk);
    const SeqView sv = seq_view<false>(P, b);
    if (!ws_planned(P)) return;
    const int lo = sv.lo, n = sv.n;
    if (sv.status != GDN_SEQ_OK) {
        for (int t = tid; t < n * grp * D; t += NT)
            P.out[((size_t)(lo + t / (grp * D)) * P.Hv + h0) * D + t % (grp * D)] = qnan_f();
        return;
    }
    if (n == 0) return;
    const int nb = (n + kTile - 1) / kTile;  // node blocks in use (n <= NN)
    const BTab<D, NB> L = btab_carve<D, NB>(lds_raw, grp);
    const uint16_t *kb = static_cast<const uint16_t *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const uint16_t *qb = static_cast<const uint16_t *>(P.q) + ((size_t)lo * P.Hk + g) * D;
    const uint16_t *vg = static_cast<const uint16_t *>(P.v) + ((size_t)lo * P.Hv + h0) * D;
    const size_t kq_stride = (size_t)P.Hk * D;
    const float *s0 = P.state_in + ((size_t)sv.slot * P.Hv + h0) * D * D;
    // out[node][h0 + hh][row]: uniform base per (node, head) + this lane's offset
    const unsigned out_lane = (unsigned)(4 * hf * P.Hv * D + row);
    const unsigned s_lane = (unsigned)(row * D + 8 * hf);
    constexpr int V_PER = (NN * (D / 8) + NT - 1) / NT;  // 16-byte chunks of one head's values
    auto fetch_v = [&](int hh, uint4 (&vr)[V_PER]) {
#pragma unroll
        for (int u = 0; u < V_PER; ++u) {
            const int c = tid + u * NT;
            vr[u] = c < n * (D / 8) ? *reinterpret_cast<const uint4 *>(vg + (size_t)(c / (D / 8)) * P.Hv * D + hh * D +
                                                                        8 * (c % (D / 8)))
                                    : make_uint4(0, 0, 0, 0);
        }
    };

    // ---- one round trip: keys/queries of all blocks, gates, paths
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
    int an[kPath], d = 0;
    if (tid < n) {
        d = P.ws.depth[lo + tid];
#pragma unroll
        for (int e = 0; e < kPath; ++e) an[e] = P.ws.nodepath[(size_t)(lo + tid) * GDN_MAX_DEPTH + e];
    }
    if (tid < n) {
#pragma unroll
        for (int e = 0; e < kPath; ++e) L.anc[tid * Q::PS + e] = an[e];
        L.depth[tid] = d;
    }
#pragma unroll
    for (int u = 0; u < GA_PER; ++u) {
        const int t = tid + u * NT;
        if (t < grp * n) {
            L.a[(t / n) * NN + t % n] = ga[u];
            L.b[(t / n) * NN + t % n] = gb[u];
        }
    }
#pragma unroll
    for (int u = 0; u < KQ_PER; ++u) {
        const int idx = tid + u * NT;
        *reinterpret_cast<uint4 *>(L.kq + (idx / (D / 8)) * Q::KQ + 8 * (idx % (D / 8))) = kqv[u];
    }
    // the first head's state and values go out once the tables have landed; the second
    // head's after the coefficients (registers are scarce while those are formed)
    float sA[KS][8], sB[KS][8];
    uint4 vA[V_PER], vB[V_PER];
    load_state_frags<D>(s0, s_lane, sA);
    fetch_v(0, vA);
    __syncthreads();

    // ---- Gram entries of every block pair: node j's ancestor i at path position
    // depth(i) - 1 gets k_i . k_j and k_i . q_j
    for (int pr = w; pr < nb * nb; pr += WAVES) {
        const int ti = pr / nb, tj = pr % nb;
        f32x16 gkk = {}, gkq = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 A = frag_of(L.kq + (ti * kTile + l32) * Q::KQ, s, hf);
            const bf16x8 Bk = frag_of(L.kq + (tj * kTile + l32) * Q::KQ, s, hf);
            const bf16x8 Bq = frag_of(L.kq + (NN + tj * kTile + l32) * Q::KQ, s, hf);
            gkk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bk, gkk, 0, 0, 0);
            gkq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bq, gkq, 0, 0, 0);
        }
        const int j = tj * kTile + l32;
        if (j < n) {
            const int dj = L.depth[j];
            int er[16], ar[16];  // candidate i's path position in j's path, and who sits there
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ti * kTile + 8 * (r / 4) + 4 * hf + (r % 4);
                er[r] = i < n ? L.depth[i] - 1 : kPath;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) ar[r] = L.anc[j * Q::PS + min(er[r], kPath - 1)];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ti * kTile + 8 * (r / 4) + 4 * hf + (r % 4);
                if (er[r] < dj && ar[r] == i) {
                    L.gk[j * Q::PS + er[r]] = gkk[r];
                    L.gq[j * Q::PS + er[r]] = gkq[r];
                }
            }
        }
    }
    __syncthreads();

    // ---- per (head, node): ratios, coefficients, the output weights' right-hand sides
    for (int t = tid; t < grp * n; t += NT) {
        const int hh = t / n, i = t % n;
        const int di = L.depth[i];
        const float bi = L.b[hh * NN + i];
        float r = 1.0f;
#pragma unroll
        for (int e = kPath - 1; e >= 0; --e) {
            const bool on = e < di - 1;
            L.coefL[(hh * NN + i) * Q::PS + e] = on ? bi * r * L.gk[i * Q::PS + e] : 0.0f;
            L.ysp[(hh * NN + i) * kPath + e] =
                on ? r * L.gq[i * Q::PS + e] : (e == di - 1 ? L.gq[i * Q::PS + e] : 0.0f);
            if (e < di) r *= L.a[hh * NN + max(L.anc[i * Q::PS + e], 0)];
        }
        L.gab[hh * NN + i] = make_float4(r, bi * r, bi, 0.0f);
    }
    __syncthreads();
    // back substitution, deepest weight first, in place
    for (int t = tid; t < grp * n; t += NT) {
        const int hh = t / n, i = t % n;
        const int di = L.depth[i];
        int an_t[kPath];
#pragma unroll
        for (int e = 0; e < kPath; ++e) an_t[e] = max(L.anc[i * Q::PS + e], 0);
        float *yr = L.ysp + (hh * NN + i) * kPath;
        float y[kPath];
#pragma unroll
        for (int e = kPath - 1; e >= 0; --e) {
            float acc = yr[e];
#pragma unroll
            for (int f = kPath - 1; f > e; --f) acc = fmaf(-y[f], L.coefL[(hh * NN + an_t[f]) * Q::PS + e], acc);
            y[e] = e < di ? acc : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < kPath; ++e) yr[e] = y[e];
    }

    // ---- value heads
    auto head = [&](const float (&st)[KS][8], int hh, const uint4 (&vr)[V_PER]) {
        __syncthreads();  // the previous head is done with the operator and the values
        // this head's values, and its dense output operator (bf16 hi + lo)
#pragma unroll
        for (int u = 0; u < V_PER; ++u) {
            const int c = tid + u * NT;
            if (c < NN * (D / 8)) reinterpret_cast<uint4 *>(L.vst)[c] = vr[u];
        }
        if (hh == 0) {
            // every head's operator has its nonzeros at the same places (the ancestors), so
            // clearing once, before the first head, leaves each later head's scatter a
            // complete operator
            static_assert(Q::MS % 8 == 0, "16-byte operator rows");
            for (int c = tid; c < nb * kTile * Q::MS / 8; c += NT) {
                reinterpret_cast<uint4 *>(L.mth)[c] = make_uint4(0u, 0u, 0u, 0u);
                reinterpret_cast<uint4 *>(L.mtl)[c] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        __syncthreads();
        for (int t = tid; t < n * kPath; t += NT) {
            const int i = t / kPath, e = t % kPath;
            if (e < L.depth[i]) {
                const int col = L.anc[i * Q::PS + e];
                const float y = L.ysp[(hh * NN + i) * kPath + e];
                const __bf16 yh = static_cast<__bf16>(y);
                L.mth[i * Q::MS + col] = __builtin_bit_cast(uint16_t, yh);
                L.mtl[i * Q::MS + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(y - static_cast<float>(yh)));
            }
        }
        __syncthreads();
        // X_j = K_j S0^T and Y_t = Q_t S0^T for every block in one pass over the state:
        // the state is split once per k-step and the 2 NB accumulations are independent
        // MFMA chains
        f32x16 X[NB], Y[NB];
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            X[jb] = f32x16{};
            Y[jb] = f32x16{};
        }
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
                if (jb < nb) {
                    const bf16x8 Ak = frag_of(L.kq + (jb * kTile + l32) * Q::KQ, s, hf);
                    const bf16x8 Aq = frag_of(L.kq + (NN + jb * kTile + l32) * Q::KQ, s, hf);
                    X[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, shi, X[jb], 0, 0, 0);
                    Y[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, shi, Y[jb], 0, 0, 0);
                    X[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ak, slo, X[jb], 0, 0, 0);
                    Y[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, slo, Y[jb], 0, 0, 0);
                }
            }
        }
        // R_j = b v - alpha X_j, kept as bf16 hi + lo in the k-order of the output products
        // (k-step u of block j: accumulator slots 8u .. 8u+7)
        const float4 *gab = L.gab + hh * NN;
        bf16x8 rhi[NB][2], rlo[NB][2];
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = jb * kTile + 8 * (r / 4) + 4 * hf + (r % 4);
                const float4 q4 = gab[min(i, n - 1)];
                const float vi = bf2f(L.vst[min(i, NN - 1) * D + row]);
                const float rv = i < n ? fmaf(-q4.y, X[jb][r], q4.z * vi) : 0.0f;
                const __bf16 rb = static_cast<__bf16>(rv);
                rhi[jb][r / 8][r % 8] = rb;
                rlo[jb][r / 8][r % 8] = static_cast<__bf16>(rv - static_cast<float>(rb));
                // gamma Y_t, the start of block t's outputs
                Y[jb][r] = i < n ? q4.x * Y[jb][r] : 0.0f;
            }
        }
        // O_t = gamma Y_t + sum_j MT_tj R_j: for each operand block j, the NB output
        // blocks' accumulations are independent chains
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            if (jb < nb) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int t = 0; t < NB; ++t) {
                        if (t < nb) {
                            const uint16_t *mh = L.mth + (t * kTile + l32) * Q::MS;
                            const uint16_t *ml = L.mtl + (t * kTile + l32) * Q::MS;
                            const int c0 = jb * kTile + 16 * u + 4 * hf;
                            const uint2 x0 = *reinterpret_cast<const uint2 *>(mh + c0);
                            const uint2 x1 = *reinterpret_cast<const uint2 *>(mh + c0 + 8);
                            const uint2 y0 = *reinterpret_cast<const uint2 *>(ml + c0);
                            const uint2 y1 = *reinterpret_cast<const uint2 *>(ml + c0 + 8);
                            const bf16x8 ahi = __builtin_bit_cast(bf16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
                            const bf16x8 alo = __builtin_bit_cast(bf16x8, make_uint4(y0.x, y0.y, y1.x, y1.y));
                            Y[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, rhi[jb][u], Y[t], 0, 0, 0);
                            Y[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, rlo[jb][u], Y[t], 0, 0, 0);
                            Y[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, rhi[jb][u], Y[t], 0, 0, 0);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            if (t < nb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // node of half-wave 0 (uniform; half-wave 1 adds 4): a uniform base
                    // per (node, head) plus the lane's fixed offset
                    const int ir = t * kTile + 8 * (r / 4) + (r % 4);
                    if (ir + 4 * hf < n) {
                        float *ob = P.out + ((size_t)(lo + ir) * P.Hv + h0 + hh) * D;
                        ob[out_lane] = Y[t][r];
                    }
                }
            }
        }
    };
    if (grp > 1) {
        load_state_frags<D>(s0 + (size_t)D * D, s_lane, sB);
        fetch_v(1, vB);
    }
    head(sA, 0, vA);
    if (grp > 2) {
        load_state_frags<D>(s0 + (size_t)2 * D * D, s_lane, sA);
        fetch_v(2, vA);
    }
    if (grp > 1) head(sB, 1, vB);
    if (grp > 3) {
        load_state_frags<D>(s0 + (size_t)3 * D * D, s_lane, sB);
        fetch_v(3, vB);
    }
    if (grp > 2) head(sA, 2, vA);
    if (grp > 3) head(sB, 3, vB);
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
    uint16_t *v;      // [16][grp][D] path values of the workgroup's heads
    float *gram;      // [16][17] k_e . k_p
    float *coefL;     // [grp][16][17]
    float4 *gaw;      // [grp][16] gamma, alpha, b, w
    float *a, *b;     // [grp][16]
    static constexpr int KP = D + 8;
    static constexpr int KT = kPath + 8;
};

template <int D>
__host__ __device__ inline size_t ptab_bytes(int grp) {
    return (size_t)kPath * PTab<D>::KP * 2 + (size_t)D * PTab<D>::KT * 2 + (size_t)kPath * grp * D * 2 +
           kPath * (kPath + 1) * 4 + (size_t)grp * kPath * (kPath + 1) * 4 + (size_t)grp * kPath * 16 +
           2 * (size_t)grp * kPath * 4;
}

template <int D>
__device__ inline PTab<D> ptab_carve(char *base, int grp) {
    PTab<D> L;
    L.gaw = reinterpret_cast<float4 *>(base);      base += (size_t)grp * kPath * 16;
    L.k = reinterpret_cast<uint16_t *>(base);      base += (size_t)kPath * PTab<D>::KP * 2;
    L.kt = reinterpret_cast<uint16_t *>(base);     base += (size_t)D * PTab<D>::KT * 2;
    L.v = reinterpret_cast<uint16_t *>(base);      base += (size_t)kPath * grp * D * 2;
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

template <int D, bool CHAIN>
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
        const bool planned = ws_planned(P);
        const int4 info = *reinterpret_cast<const int4 *>(P.ws.seq_info + b * kSeqInfoInts);
        const int m = P.accepted[b];
        if (!planned) return;
        if (info.z != GDN_SEQ_OK || info.y == 0) return;
        if (m < -1 || m >= info.y) {
            if (g == 0 && tid == 0) P.ws.seq_status[b] = GDN_SEQ_BAD_ACCEPT;
            return;
        }
        if (m == -1) return;
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
    const PTab<D> L = ptab_carve<D>(lds_raw, grp);
    const uint16_t *kb = static_cast<const uint16_t *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    const uint16_t *vg = static_cast<const uint16_t *>(P.v) + ((size_t)lo * P.Hv + h0) * D;
    constexpr int KC = kPath * D / 8;  // 16-byte chunks of the path keys
    constexpr int K_PER = (KC + NT - 1) / NT;
    constexpr int VC = kPath * grp * D / 8;
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
    for (int u = 0; u < K_PER; ++u) nk[u] = node_of(((tid + u * NT) / (D / 8)) % kPath);
#pragma unroll
    for (int u = 0; u < V_PER; ++u) nv[u] = node_of(((tid + u * NT) / (grp * D / 8)) % kPath);
    const int ng = node_of(tid % kPath);
    uint4 kr[K_PER], vr[V_PER];
#pragma unroll
    for (int u = 0; u < K_PER; ++u)
        kr[u] = *reinterpret_cast<const uint4 *>(kb + (size_t)nk[u] * P.Hk * D + 8 * ((tid + u * NT) % (D / 8)));
#pragma unroll
    for (int u = 0; u < V_PER; ++u)
        vr[u] = *reinterpret_cast<const uint4 *>(vg + (size_t)nv[u] * P.Hv * D + 8 * ((tid + u * NT) % (grp * D / 8)));
    const bool gate_t = tid < grp * kPath;
    const size_t at = (size_t)(lo + ng) * P.Hv + h0 + (gate_t ? tid / kPath : 0);
    float ga = P.a[at], gb = P.b[at];
    // the state, issued after the tables so that waiting for the tables does not wait for it
    load_state_tiles<D>(s0, s_lane, SA);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < K_PER; ++u) {
        const int idx = tid + u * NT, e = idx / (D / 8), c8 = idx % (D / 8);
        const uint4 kv = e < len ? kr[u] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(L.k + e * PTab<D>::KP + 8 * c8) = kv;
        const uint16_t *hv = reinterpret_cast<const uint16_t *>(&kv);
#pragma unroll
        for (int i = 0; i < 8; ++i) L.kt[(8 * c8 + i) * PTab<D>::KT + e] = hv[i];
    }
#pragma unroll
    for (int u = 0; u < V_PER; ++u) {
        const int idx = tid + u * NT;
        reinterpret_cast<uint4 *>(L.v)[idx] = idx / (grp * D / 8) < len ? vr[u] : make_uint4(0, 0, 0, 0);
    }
    if (gate_t) {
        const bool on = tid % kPath < len;
        L.a[tid] = on ? ga : 1.0f;
        L.b[tid] = on ? gb : 0.0f;
    }
    __syncthreads();

    // ---- Gram entries of the path keys (one wave, one 32x32 tile, 16 rows used)
    if (w == 0) {
        f32x16 gk = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const bf16x8 A = l32 < kPath ? frag_of(L.k + l32 * PTab<D>::KP, s, hf) : zero_frag();
            gk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, A, gk, 0, 0, 0);
        }
        if (l32 < kPath) {
#pragma unroll
            for (int r = 0; r < 8; ++r) L.gram[l32 * (kPath + 1) + 8 * (r / 4) + 4 * hf + (r % 4)] = gk[r];
        }
    }
    __syncthreads();
    // ---- per (head, path entry p): ratios, coefficients
    if (tid < grp * kPath) {
        const int hh = tid / kPath, p = tid % kPath;
        const float *ah = L.a + hh * kPath;
        const float bp = L.b[tid];
        float r = 1.0f;  // R(p, e), e from p-1 down
#pragma unroll
        for (int e = kPath - 1; e >= 0; --e) {
            float v = 0.0f;
            if (e < p) {
                r *= ah[e + 1];
                v = p < len ? bp * r * L.gram[p * (kPath + 1) + e] : 0.0f;
            }
            L.coefL[(hh * kPath + p) * (kPath + 1) + e] = v;
        }
        float gm = 1.0f, wr = 1.0f;
#pragma unroll
        for (int t = 0; t < kPath; ++t) {
            if (t <= p) gm *= ah[t];
            if (t > p && t < len) wr *= ah[t];
        }
        L.gaw[tid] = make_float4(gm, bp * gm, bp, p < len ? wr : 0.0f);
    }
    __syncthreads();

    // ---- value heads
    auto head = [&](f32x16 (&S)[NTILE], int hh) {
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
            ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, shi, ax, 0, 0, 0);
            ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, slo, ax, 0, 0, 0);
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
        float c[kPath];
#pragma unroll
        for (int p = 0; p < kPath; ++p) {
            const float4 q4 = gaw[p];
            float acc = fmaf(-q4.y, x[p], q4.z * bf2f(vh[p * grp * D]));
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
            S[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, whi, S[t], 0, 0, 0);
            S[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, wlo, S[t], 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4 *>(dh + 32 * t + 8 * q) =
                    make_float4(S[t][4 * q], S[t][4 * q + 1], S[t][4 * q + 2], S[t][4 * q + 3]);
        }
    };
    head(SA, 0);
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
// compute units x workgroups per unit, queried once per (kernel, device).  0 when unknown.
constexpr int kMaxDevices = 64;
template <void (*Kernel)(Params)>
int resident_workgroups(int threads, size_t lds) {
    const auto kernel = Kernel;
    static std::atomic<int> cache[kMaxDevices];  // one per kernel; threads that race store the same value
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int known = cache[dev].load(std::memory_order_relaxed);
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
        cache[dev].store(known, std::memory_order_relaxed);
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
// over node blocks; else coefficients + verify
template <int D>
hipError_t launch_verify_d(const Params &p, bool chain, hipStream_t s) {
    const int grp = p.Hv / p.Hk;
    const int hpw = chain ? heads_per_workgroup<verify_group_kernel<D, true, 1>>(p, VG<D>::THREADS, gtab_bytes<D>(1))
                          : heads_per_workgroup<verify_group_kernel<D, false, 1>>(p, VG<D>::THREADS, gtab_bytes<D>(1));
    if ((chain || p.max_nodes <= kTile) && hpw <= kGroupMaxHeads) {
        const dim3 grid(p.B * (p.Hv / hpw)), block(VG<D>::THREADS);
        switch (hpw) {
#define GDN_GROUP_CASE(G)                                                                                    \
    case G:                                                                                                  \
        return chain ? launch_with_lds(verify_group_kernel<D, true, G>, grid, block, gtab_bytes<D>(G), s, p) \
                     : launch_with_lds(verify_group_kernel<D, false, G>, grid, block, gtab_bytes<D>(G), s, p);
            GDN_GROUP_CASE(1)
            GDN_GROUP_CASE(2)
            GDN_GROUP_CASE(3)
            GDN_GROUP_CASE(4)
#undef GDN_GROUP_CASE
        }
    }
    const bool two = p.max_nodes <= 2 * kTile;
    const int gb = !chain && p.max_nodes <= 3 * kTile
                       ? (two ? heads_per_workgroup<verify_blocks_kernel<D, 2, 1>>(p, VG<D>::THREADS, btab_bytes<D, 2>(1))
                              : heads_per_workgroup<verify_blocks_kernel<D, 3, 1>>(p, VG<D>::THREADS, btab_bytes<D, 3>(1)))
                       : grp;
    if (!chain && p.max_nodes <= 3 * kTile && gb <= kGroupMaxHeads) {
        const dim3 grid(p.B * (p.Hv / gb)), block(VG<D>::THREADS);
        switch (gb) {
#define GDN_BLOCKS_CASE(G)                                                                                          \
    case G:                                                                                                         \
        return two ? launch_with_lds(verify_blocks_kernel<D, 2, G>, grid, block, btab_bytes<D, 2>(G), s, p) \
                   : launch_with_lds(verify_blocks_kernel<D, 3, G>, grid, block, btab_bytes<D, 3>(G), s, p);
            GDN_BLOCKS_CASE(1)
            GDN_BLOCKS_CASE(2)
            GDN_BLOCKS_CASE(3)
            GDN_BLOCKS_CASE(4)
#undef GDN_BLOCKS_CASE
        }
    }
    const int cap = chain ? kPath : p.max_nodes;
    // LDS for the most value heads a pass can take (a one-node sequence)
    const size_t clds = ctab_bytes(cap, grp, std::min(grp, kCoefMaxHeadsPerPass));
    hipError_t e = chain ? launch_with_lds(coef_kernel<D, true>, dim3(p.B * p.Hk), dim3(kCoefThreads), clds, s, p)
                         : launch_with_lds(coef_kernel<D, false>, dim3(p.B * p.Hk), dim3(kCoefThreads), clds, s, p);
    if (e != hipSuccess) return e;
    const dim3 grid(p.B * p.Hv), block(VG<D>::THREADS);
    if (chain) return launch_with_lds(verify_kernel<D, true, 1>, grid, block, vtab_bytes(kPath, D, true), s, p);
    if (p.max_nodes <= kTile)
        return launch_with_lds(verify_kernel<D, false, 1>, grid, block, vtab_bytes(p.max_nodes, D, true), s, p);
    return launch_with_lds(verify_kernel<D, false, 3>, grid, block, vtab_bytes(p.max_nodes, D, false), s, p);
}

// one workgroup per value head: four fit a CU, and their independent rounds overlap
// reading and writing better than a key head's workgroup walking its value heads
template <int D>
hipError_t launch_replay_d(const Params &p, bool chain, hipStream_t s) {
    const dim3 grid(p.B * p.Hv), block(VG<D>::THREADS);
    return chain ? launch_with_lds(replay_kernel<D, true>, grid, block, ptab_bytes<D>(1), s, p)
                 : launch_with_lds(replay_kernel<D, false>, grid, block, ptab_bytes<D>(1), s, p);
}

}  // namespace

bool fast_path_supported(int D, int dtype) { return (D == 64 || D == 128) && dtype == GDN_BF16; }
bool fast_tree_supported(int D, int dtype, int max_nodes) {
    return fast_path_supported(D, dtype) && max_nodes <= kFastMaxNodes;
}

hipError_t launch_tree_verify_fast(const Params &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    return p.D == 64 ? launch_verify_d<64>(p, false, s) : launch_verify_d<128>(p, false, s);
}
hipError_t launch_persist_fast(const Params &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    return p.D == 64 ? launch_replay_d<64>(p, false, s) : launch_replay_d<128>(p, false, s);
}
// Chains of at most 16 nodes: outputs from the verify kernel in chain order
// (so a chain-shaped tree and a chain give the same bits) and the final state
// from the replay kernel (so persist and chain give the same bits).
hipError_t launch_chain_verify_fast(const Params &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    hipError_t e = hipSuccess;
    if (p.out || p.has_ws) e = p.D == 64 ? launch_verify_d<64>(p, true, s) : launch_verify_d<128>(p, true, s);
    if (e != hipSuccess) return e;
    if (p.final_state) e = p.D == 64 ? launch_replay_d<64>(p, true, s) : launch_replay_d<128>(p, true, s);
    return e;
}

}  // namespace gdn

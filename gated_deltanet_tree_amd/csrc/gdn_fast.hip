// gdn_fast.hip -- tree verify, chain verify and persist for D in {64, 128}
// with bf16 q/k/v, built on MFMA.
//
// Unrolling the gated delta rule along a root-to-node path gives, for node n
// with path p_0 (root) ... p_{d-1} = n and G_n = a_{p_0} ... a_{p_{d-1}}:
//     S^n = G_n S0 + sum_e R(n,e) c_{p_e} k_{p_e}^T,   R(n,e) = a_{p_{e+1}} ... a_{p_{d-1}}
//     c_n = b_n v_n - b_n G_n (S0 k_n) - sum_{e<d-1} b_n R(n,e) (k_{p_e} . k_n) c_{p_e}
//     o_n = G_n (S0 q_n) + sum_{e<=d-1} R(n,e) (k_{p_e} . q_n) c_{p_e}
// (c_n is the row vector b (v - a S^{parent} k) of the rule written as
// S' = a S + c k^T.)  So a whole tree needs only the dense products S0 K^T
// and S0 Q^T over all of its nodes -- one contraction per (sequence, head),
// done on the matrix cores -- plus, per state row, a short recurrence over
// each node's ancestors.  The state itself is never materialized in verify.
// Persist materializes S^m for the accepted node m from the same pieces.
//
// Precision: S0 is fp32; it enters the bf16 MFMA as hi + lo with
// hi = bf16(S0) and lo = bf16(S0 - hi) (two passes, ~2^-16 relative), while
// k and q are bf16 already, so the products are exact and accumulate in fp32.
//
// Geometry: one workgroup per (sequence, value head), D/32 waves, wave w owns
// state rows [32w, 32w+32).  MFMA 32x32x16: the node block (32 nodes in tree
// preorder) is the A operand, the state rows are the B operand, so lane l of
// a wave ends with state row l%32 for 16 of the 32 nodes; the accumulators go
// through LDS once so each lane then walks the nodes of the block in order
// for its row.  Both 32-lane halves of a wave run that walk for the same row
// (half 0 writes the outputs).
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 32;                 // nodes per MFMA block
constexpr int kPath = GDN_MAX_DEPTH;      // ancestors per node, chain chunk length

template <int D>
struct FG {
    static constexpr int WAVES = D / 32;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int KS = D / 16;     // MFMA k-steps over the key dimension
};

// ---- LDS carve-up -----------------------------------------------------------
struct FastLds {
    int *order;    // [cap]      position -> local node id
    int *pos_of;   // [cap]      local node id -> position
    int *depth;    // [cap]
    int *anc;      // [cap][16]  ancestor positions, root first; anc[p][d-1] = p
    float *a, *b, *gamma, *alpha;  // [cap]
    float *coefL;  // [cap][16]  b_p R(p,e) (k_anc . k_p)
    float *coefM;  // [cap][16]  R(p,e) (k_anc . q_p)
    float *xt;     // [WAVES][2][32][32]  S0 K^T / S0 Q^T blocks, node-major
    uint16_t *kpath;  // [16][D] bf16 keys of the chunk being materialized
};

__host__ __device__ inline size_t fast_lds_bytes(int cap, int D) {
    const size_t c = (size_t)cap;
    return c * 4 * 3 + c * kPath * 4 + c * 4 * 4 + 2 * c * kPath * 4 + (size_t)(D / 32) * 2 * kTile * 32 * 4 +
           (size_t)kPath * D * 2;
}

__device__ inline FastLds carve(char *base, int cap, int D) {
    FastLds L;
    L.xt = reinterpret_cast<float *>(base);
    base += (size_t)(D / 32) * 2 * kTile * 32 * 4;
    L.kpath = reinterpret_cast<uint16_t *>(base);  // 16-byte aligned: follows the float blocks
    base += (size_t)kPath * D * 2;
    L.coefL = reinterpret_cast<float *>(base); base += (size_t)cap * kPath * 4;
    L.coefM = reinterpret_cast<float *>(base); base += (size_t)cap * kPath * 4;
    L.anc = reinterpret_cast<int *>(base);     base += (size_t)cap * kPath * 4;
    L.order = reinterpret_cast<int *>(base);   base += (size_t)cap * 4;
    L.pos_of = reinterpret_cast<int *>(base);  base += (size_t)cap * 4;
    L.depth = reinterpret_cast<int *>(base);   base += (size_t)cap * 4;
    L.a = reinterpret_cast<float *>(base);     base += (size_t)cap * 4;
    L.b = reinterpret_cast<float *>(base);     base += (size_t)cap * 4;
    L.gamma = reinterpret_cast<float *>(base); base += (size_t)cap * 4;
    L.alpha = reinterpret_cast<float *>(base);
    return L;
}

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }
__device__ __forceinline__ float qnan_f() { return __int_as_float(0x7fc00000); }

// Per-lane view of one workgroup.
struct Lane {
    int tid, w, lane, hf, l32, row;
};
template <int D>
__device__ __forceinline__ Lane lane_of() {
    Lane L;
    L.tid = threadIdx.x;
    L.w = L.tid / 64;
    L.lane = L.tid % 64;
    L.hf = L.lane / 32;
    L.l32 = L.lane % 32;
    L.row = L.w * 32 + L.l32;
    return L;
}

// Everything the block routines need about the current sequence/head.
struct Seq {
    const uint16_t *k, *q, *v;  // base of node 0 of the sequence, this key / value head
    size_t kq_stride, v_stride; // elements between consecutive nodes
    int n;                      // positions in the current topology
};

// R(p, e) = a_{anc[e+1]} * ... * a_{anc[d-1]} (ascending, 1 when e = d-1)
__device__ __forceinline__ float ratio(const FastLds &L, int p, int e) {
    const int d = L.depth[p];
    float r = 1.0f;
    for (int t = e + 1; t < d; ++t) r *= L.a[L.anc[p * kPath + t]];
    return r;
}

// gamma_p = a_{anc[0]} * ... * a_{anc[d-1]},  alpha_p = b_p gamma_p
__device__ __forceinline__ void finish_tables(const FastLds &L, int n, int tid, int nthreads) {
    for (int p = tid; p < n; p += nthreads) {
        const int d = L.depth[p];
        float g = 1.0f;
        for (int t = 0; t < d; ++t) g *= L.a[L.anc[p * kPath + t]];
        L.gamma[p] = g;
        L.alpha[p] = L.b[p] * g;
    }
}

// MFMA fragment: 8 bf16 of the key dimension [16 s + 8 hf, +8) of a node vector.
__device__ __forceinline__ bf16x8 frag_of(const uint16_t *vec, int s, int hf) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(vec + 16 * s + 8 * hf);
    return __builtin_bit_cast(bf16x8, raw);
}

__device__ __forceinline__ bf16x8 zero_frag() {
    return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}

// State rows as B fragments: fp32 values and their bf16 hi/lo split.
template <int D>
struct StateFrags {
    float f[FG<D>::KS][8];
    bf16x8 hi[FG<D>::KS], lo[FG<D>::KS];

    __device__ __forceinline__ void load(const float *row_ptr, int hf) {
#pragma unroll
        for (int s = 0; s < FG<D>::KS; ++s) {
            const float4 x0 = *reinterpret_cast<const float4 *>(row_ptr + 16 * s + 8 * hf);
            const float4 x1 = *reinterpret_cast<const float4 *>(row_ptr + 16 * s + 8 * hf + 4);
            f[s][0] = x0.x; f[s][1] = x0.y; f[s][2] = x0.z; f[s][3] = x0.w;
            f[s][4] = x1.x; f[s][5] = x1.y; f[s][6] = x1.z; f[s][7] = x1.w;
        }
    }
    __device__ __forceinline__ void split() {
#pragma unroll
        for (int s = 0; s < FG<D>::KS; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 h = static_cast<__bf16>(f[s][e]);
                hi[s][e] = h;
                lo[s][e] = static_cast<__bf16>(f[s][e] - static_cast<float>(h));
            }
        }
    }
    __device__ __forceinline__ void store(float *row_ptr, int hf) const {
#pragma unroll
        for (int s = 0; s < FG<D>::KS; ++s) {
            *reinterpret_cast<float4 *>(row_ptr + 16 * s + 8 * hf) = make_float4(f[s][0], f[s][1], f[s][2], f[s][3]);
            *reinterpret_cast<float4 *>(row_ptr + 16 * s + 8 * hf + 4) =
                make_float4(f[s][4], f[s][5], f[s][6], f[s][7]);
        }
    }
};

// Gram entries k_anc . k_p (and k_anc . q_p) for every (ancestor, node) pair,
// turned into the recurrence coefficients.  Block pairs (ti <= tj) are spread
// over the waves; node blocks follow preorder so ancestors never come later.
template <int D>
__device__ void gram_coefficients(const FastLds &L, const Seq &S, const Lane &ln, bool want_m) {
    const int ntiles = (S.n + kTile - 1) / kTile;
    int pair = 0;
    for (int tj = 0; tj < ntiles; ++tj) {
        for (int ti = 0; ti <= tj; ++ti, ++pair) {
            if (pair % FG<D>::WAVES != ln.w) continue;
            const int pi = ti * kTile + ln.l32, pj = tj * kTile + ln.l32;
            const uint16_t *ki = pi < S.n ? S.k + (size_t)L.order[pi] * S.kq_stride : nullptr;
            const uint16_t *kj = pj < S.n ? S.k + (size_t)L.order[pj] * S.kq_stride : nullptr;
            const uint16_t *qj = pj < S.n ? S.q + (size_t)L.order[pj] * S.kq_stride : nullptr;
            f32x16 gkk = {}, gkq = {};
#pragma unroll
            for (int s = 0; s < FG<D>::KS; ++s) {
                const bf16x8 A = ki ? frag_of(ki, s, ln.hf) : zero_frag();
                const bf16x8 Bk = kj ? frag_of(kj, s, ln.hf) : zero_frag();
                gkk = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bk, gkk, 0, 0, 0);
                if (want_m) {
                    const bf16x8 Bq = qj ? frag_of(qj, s, ln.hf) : zero_frag();
                    gkq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bq, gkq, 0, 0, 0);
                }
            }
            // accumulator r holds (ancestor candidate i, node j = pj)
            if (pj < S.n) {
                const int dj = L.depth[pj];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = ti * kTile + 8 * (r / 4) + 4 * ln.hf + (r % 4);
                    if (i >= S.n) continue;
                    const int di = L.depth[i];
                    if (di > dj || L.anc[pj * kPath + di - 1] != i) continue;
                    const int e = di - 1;
                    const float R = ratio(L, pj, e);
                    if (e < dj - 1) L.coefL[pj * kPath + e] = L.b[pj] * R * gkk[r];
                    if (want_m) L.coefM[pj * kPath + e] = R * gkq[r];
                }
            }
        }
    }
}

// For node block t: S0 K^T (and S0 Q^T) on the matrix cores, parked in LDS
// node-major, then each lane walks the block's nodes for its state row.
// cpath[e] holds c of the current node's ancestor at depth e+1 (preorder
// keeps exactly the current path in it).
template <int D, bool WANT_OUT>
__device__ void block_walk(const FastLds &L, const Seq &S, const Lane &ln, const StateFrags<D> &st, int t,
                           float (&cpath)[kPath], float *out_base, size_t out_stride) {
    const int p0 = t * kTile;
    const int cnt = min(kTile, S.n - p0);
    // prefetch this row's v for the block
    float vv[kTile];
#pragma unroll
    for (int i = 0; i < kTile; ++i)
        vv[i] = i < cnt ? bf2f(S.v[(size_t)L.order[p0 + i] * S.v_stride]) : 0.0f;

    const int pi = p0 + ln.l32;
    const uint16_t *kr = pi < S.n ? S.k + (size_t)L.order[pi] * S.kq_stride : nullptr;
    const uint16_t *qr = (WANT_OUT && pi < S.n) ? S.q + (size_t)L.order[pi] * S.kq_stride : nullptr;
    f32x16 ax = {}, ay = {};
#pragma unroll
    for (int s = 0; s < FG<D>::KS; ++s) {
        const bf16x8 A = kr ? frag_of(kr, s, ln.hf) : zero_frag();
        ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, st.hi[s], ax, 0, 0, 0);
        ax = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, st.lo[s], ax, 0, 0, 0);
        if (WANT_OUT) {
            const bf16x8 Aq = qr ? frag_of(qr, s, ln.hf) : zero_frag();
            ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, st.hi[s], ay, 0, 0, 0);
            ay = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aq, st.lo[s], ay, 0, 0, 0);
        }
    }
    float *xw = L.xt + (size_t)ln.w * 2 * kTile * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r / 4) + 4 * ln.hf + (r % 4);
        xw[i * 32 + ln.l32] = ax[r];
        if (WANT_OUT) xw[kTile * 32 + i * 32 + ln.l32] = ay[r];
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < kTile; ++i) {
        if (i >= cnt) break;
        const int p = p0 + i;
        const int d = L.depth[p];
        const float x = xw[i * 32 + ln.l32];
        const float *cl = L.coefL + p * kPath;
        float c = fmaf(-L.alpha[p], x, L.b[p] * vv[i]);
#pragma unroll
        for (int e = 0; e < kPath - 1; ++e) {
            if (e >= d - 1) break;
            c = fmaf(-cl[e], cpath[e], c);
        }
        if (WANT_OUT) {
            const float y = xw[kTile * 32 + i * 32 + ln.l32];
            const float *cm = L.coefM + p * kPath;
            float o = L.gamma[p] * y;
#pragma unroll
            for (int e = 0; e < kPath - 1; ++e) {
                if (e >= d - 1) break;
                o = fmaf(cm[e], cpath[e], o);
            }
            o = fmaf(cm[d - 1], c, o);
            if (ln.hf == 0) out_base[(size_t)L.order[p] * out_stride] = o;
        }
#pragma unroll
        for (int e = 0; e < kPath; ++e)
            if (e == d - 1) cpath[e] = c;
    }
    __syncthreads();
}

// State after the first `len` positions of a chain-shaped chunk (positions
// 0..len-1, each the parent of the next):
//     S = G_{len-1} S0 + sum_{e < len} R(len-1, e) c_e k_e^T
// kpath holds the chunk's keys; cpath the chunk's c values for this row.
template <int D>
__device__ void materialize(const FastLds &L, const Lane &ln, const float (&cpath)[kPath], int len,
                            const StateFrags<D> &src, float (&dst)[FG<D>::KS][8]) {
    float w[kPath];
#pragma unroll
    for (int e = 0; e < kPath; ++e) {
        w[e] = 0.0f;
        if (e < len) w[e] = ratio(L, len - 1, e) * cpath[e];
    }
    const float g = L.gamma[len - 1];
#pragma unroll
    for (int s = 0; s < FG<D>::KS; ++s) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = 16 * s + 8 * ln.hf + j;
            float acc = g * src.f[s][j];
#pragma unroll
            for (int e = 0; e < kPath; ++e) {
                if (e >= len) break;
                acc = fmaf(w[e], bf2f(L.kpath[e * D + col]), acc);
            }
            dst[s][j] = acc;
        }
    }
}

// Chain-shaped tables for positions [0, cnt) = nodes first_node + pos_map(p).
__device__ void chain_tables(const FastLds &L, const int32_t *nodes, int first, int cnt, const float *a,
                             const float *b, size_t ab_stride, int tid, int nthreads) {
    for (int p = tid; p < cnt; p += nthreads) {
        const int node = nodes ? nodes[p] : first + p;
        L.order[p] = node;
        L.depth[p] = p + 1;
        L.a[p] = a[(size_t)node * ab_stride];
        L.b[p] = b[(size_t)node * ab_stride];
        for (int e = 0; e < kPath; ++e) L.anc[p * kPath + e] = e <= p ? e : -1;
    }
}

template <int D>
__device__ void stage_kpath(const FastLds &L, const Seq &S, int cnt, int tid, int nthreads) {
    for (int idx = tid; idx < kPath * D / 8; idx += nthreads) {
        const int e = idx / (D / 8), c8 = idx % (D / 8);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (e < cnt) v = *reinterpret_cast<const uint4 *>(S.k + (size_t)L.order[e] * S.kq_stride + 8 * c8);
        *reinterpret_cast<uint4 *>(L.kpath + e * D + 8 * c8) = v;
    }
}

__device__ __forceinline__ bool ws_planned(const Params &P) {
    return P.ws.header[0] == kMagic && P.ws.header[1] == P.B && P.ws.header[2] == P.T;
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(FG<D>::THREADS) void fast_tree_verify(Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    const Lane ln = lane_of<D>();
    const int b = blockIdx.x / P.Hv, h = blockIdx.x % P.Hv;
    const int g = h / (P.Hv / P.Hk);
    if (!ws_planned(P)) return;
    const int lo = P.ws.seq_info[b * kSeqInfoInts + 0];
    const int n = P.ws.seq_info[b * kSeqInfoInts + 1];
    const size_t out_stride = (size_t)P.Hv * D;
    float *out_base = P.out + ((size_t)lo * P.Hv + h) * D + ln.row;
    if (P.ws.seq_status[b] != GDN_SEQ_OK) {
        if (ln.hf == 0)
            for (int i = 0; i < n; ++i) out_base[i * out_stride] = qnan_f();
        return;
    }
    if (n == 0) return;
    const FastLds L = carve(lds_raw, P.max_nodes, D);

    // tables in preorder positions
    for (int p = ln.tid; p < n; p += FG<D>::THREADS) {
        const int node = P.ws.order[lo + p];
        L.order[p] = node;
        L.pos_of[node] = p;
        L.depth[p] = P.ws.depth[lo + node];
        L.a[p] = P.a[(size_t)(lo + node) * P.Hv + h];
        L.b[p] = P.b[(size_t)(lo + node) * P.Hv + h];
    }
    __syncthreads();
    for (int idx = ln.tid; idx < n * kPath; idx += FG<D>::THREADS) {
        const int p = idx / kPath, e = idx % kPath;
        const int node = L.order[p];
        L.anc[idx] = e < L.depth[p] ? L.pos_of[P.ws.nodepath[(size_t)(lo + node) * GDN_MAX_DEPTH + e]] : -1;
    }
    __syncthreads();
    finish_tables(L, n, ln.tid, FG<D>::THREADS);

    Seq S;
    S.k = static_cast<const uint16_t *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    S.q = static_cast<const uint16_t *>(P.q) + ((size_t)lo * P.Hk + g) * D;
    S.v = static_cast<const uint16_t *>(P.v) + ((size_t)lo * P.Hv + h) * D + ln.row;
    S.kq_stride = (size_t)P.Hk * D;
    S.v_stride = (size_t)P.Hv * D;
    S.n = n;

    StateFrags<D> st;
    const int slot = P.slot_idx[b];
    st.load(P.state_in + (((size_t)slot * P.Hv + h) * D + ln.row) * D, ln.hf);
    st.split();
    __syncthreads();
    gram_coefficients<D>(L, S, ln, true);
    __syncthreads();

    float cpath[kPath];
#pragma unroll
    for (int e = 0; e < kPath; ++e) cpath[e] = 0.0f;
    const int ntiles = (n + kTile - 1) / kTile;
    for (int t = 0; t < ntiles; ++t) block_walk<D, true>(L, S, ln, st, t, cpath, out_base, out_stride);
}

// ---------------------------------------------------------------------------
// Chain verify: chunks of up to 16 nodes; between chunks the state is
// materialized exactly like persist does for an accepted path.
template <int D>
__global__ __launch_bounds__(FG<D>::THREADS) void fast_chain_verify(Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    const Lane ln = lane_of<D>();
    const int b = blockIdx.x / P.Hv, h = blockIdx.x % P.Hv;
    const int g = h / (P.Hv / P.Hk);
    const int lo = P.cu_nodes[b], hi = P.cu_nodes[b + 1];
    const bool in_bounds = 0 <= lo && lo <= hi && hi <= P.T;
    const bool range_ok = in_bounds && hi - lo <= P.max_nodes;
    const int n = in_bounds ? hi - lo : 0;
    const int slot = (range_ok && n > 0) ? P.slot_idx[b] : 0;
    int status = GDN_SEQ_OK;
    if (!range_ok) status = GDN_SEQ_BAD_NODES;
    else if (n > 0 && (slot < 0 || slot >= P.num_slots)) status = GDN_SEQ_BAD_SLOT;
    if (P.has_ws && h == 0 && ln.tid == 0) {
        if (b == 0) {
            P.ws.header[0] = kMagic;
            P.ws.header[1] = P.B;
            P.ws.header[2] = P.T;
        }
        P.ws.seq_status[b] = status;
    }
    const bool want_out = P.q != nullptr && P.out != nullptr;
    const size_t out_stride = (size_t)P.Hv * D;
    float *out_base = want_out ? P.out + ((size_t)lo * P.Hv + h) * D + ln.row : nullptr;
    if (status != GDN_SEQ_OK) {
        if (out_base && ln.hf == 0)
            for (int i = 0; i < n; ++i) out_base[i * out_stride] = qnan_f();
        return;
    }
    const int flen = P.final_len ? P.final_len[b] : -1;
    float *fin = (P.final_state && flen >= 0 && flen <= n)
                     ? P.final_state + (((size_t)b * P.Hv + h) * D + ln.row) * D
                     : nullptr;
    if (n == 0 && !fin) return;
    const FastLds L = carve(lds_raw, kPath, D);

    StateFrags<D> st;
    st.load(P.state_in + (((size_t)slot * P.Hv + h) * D + ln.row) * D, ln.hf);
    if (fin && flen == 0) st.store(fin, ln.hf);

    Seq S;
    S.kq_stride = (size_t)P.Hk * D;
    S.v_stride = (size_t)P.Hv * D;
    for (int c0 = 0; c0 < n; c0 += kPath) {
        const int cnt = min(kPath, n - c0);
        const bool need_fin = fin && flen > c0 && flen <= c0 + cnt;
        const bool need_next = c0 + cnt < n && (want_out || (fin && flen > c0 + cnt));
        if (!want_out && !need_fin && !need_next) break;
        S.k = static_cast<const uint16_t *>(P.k) + ((size_t)(lo + c0) * P.Hk + g) * D;
        S.q = want_out ? static_cast<const uint16_t *>(P.q) + ((size_t)(lo + c0) * P.Hk + g) * D : nullptr;
        S.v = static_cast<const uint16_t *>(P.v) + ((size_t)(lo + c0) * P.Hv + h) * D + ln.row;
        S.n = cnt;
        __syncthreads();
        chain_tables(L, nullptr, 0, cnt, P.a + (size_t)(lo + c0) * P.Hv + h, P.b + (size_t)(lo + c0) * P.Hv + h,
                     P.Hv, ln.tid, FG<D>::THREADS);
        __syncthreads();
        finish_tables(L, cnt, ln.tid, FG<D>::THREADS);
        stage_kpath<D>(L, S, cnt, ln.tid, FG<D>::THREADS);
        st.split();
        __syncthreads();
        gram_coefficients<D>(L, S, ln, want_out);
        __syncthreads();
        float cpath[kPath];
#pragma unroll
        for (int e = 0; e < kPath; ++e) cpath[e] = 0.0f;
        float *ob = want_out ? out_base + (size_t)c0 * out_stride : nullptr;
        if (want_out) block_walk<D, true>(L, S, ln, st, 0, cpath, ob, out_stride);
        else block_walk<D, false>(L, S, ln, st, 0, cpath, ob, out_stride);
        if (need_fin) {
            float f[FG<D>::KS][8];
            materialize<D>(L, ln, cpath, flen - c0, st, f);
            float *dst = fin;
#pragma unroll
            for (int s = 0; s < FG<D>::KS; ++s) {
                *reinterpret_cast<float4 *>(dst + 16 * s + 8 * ln.hf) = make_float4(f[s][0], f[s][1], f[s][2], f[s][3]);
                *reinterpret_cast<float4 *>(dst + 16 * s + 8 * ln.hf + 4) =
                    make_float4(f[s][4], f[s][5], f[s][6], f[s][7]);
            }
        }
        if (need_next) {
            float f[FG<D>::KS][8];
            materialize<D>(L, ln, cpath, cnt, st, f);
#pragma unroll
            for (int s = 0; s < FG<D>::KS; ++s)
#pragma unroll
                for (int j = 0; j < 8; ++j) st.f[s][j] = f[s][j];
        }
    }
}

// ---------------------------------------------------------------------------
// Persist: the accepted root-to-node path as a chain chunk, materialized in place.
template <int D>
__global__ __launch_bounds__(FG<D>::THREADS) void fast_persist(Params P) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    const Lane ln = lane_of<D>();
    const int b = blockIdx.x / P.Hv, h = blockIdx.x % P.Hv;
    const int g = h / (P.Hv / P.Hk);
    if (!ws_planned(P)) return;
    const int status = P.ws.seq_status[b];
    const int lo = P.ws.seq_info[b * kSeqInfoInts + 0];
    const int n = P.ws.seq_info[b * kSeqInfoInts + 1];
    if (status != GDN_SEQ_OK || n == 0) return;
    const int m = P.accepted[b];
    if (m < -1 || m >= n) {
        if (h == 0 && ln.tid == 0) P.ws.seq_status[b] = GDN_SEQ_BAD_ACCEPT;
        return;
    }
    if (m == -1) return;
    const int len = P.ws.depth[lo + m];
    const int32_t *np = P.ws.nodepath + (size_t)(lo + m) * GDN_MAX_DEPTH;
    if (h == 0) {
        if (ln.tid < GDN_MAX_DEPTH) P.ws.path[b * GDN_MAX_DEPTH + ln.tid] = np[ln.tid];
        if (ln.tid == 0) P.ws.path_len[b] = len;
    }
    const FastLds L = carve(lds_raw, kPath, D);
    chain_tables(L, np, 0, len, P.a + (size_t)lo * P.Hv + h, P.b + (size_t)lo * P.Hv + h, P.Hv, ln.tid,
                 FG<D>::THREADS);
    __syncthreads();
    finish_tables(L, len, ln.tid, FG<D>::THREADS);

    Seq S;
    S.k = static_cast<const uint16_t *>(P.k) + ((size_t)lo * P.Hk + g) * D;
    S.q = nullptr;
    S.v = static_cast<const uint16_t *>(P.v) + ((size_t)lo * P.Hv + h) * D + ln.row;
    S.kq_stride = (size_t)P.Hk * D;
    S.v_stride = (size_t)P.Hv * D;
    S.n = len;
    stage_kpath<D>(L, S, len, ln.tid, FG<D>::THREADS);

    float *row_ptr = P.state_out + (((size_t)P.slot_idx[b] * P.Hv + h) * D + ln.row) * D;
    StateFrags<D> st;
    st.load(row_ptr, ln.hf);
    st.split();
    __syncthreads();
    gram_coefficients<D>(L, S, ln, false);
    __syncthreads();
    float cpath[kPath];
#pragma unroll
    for (int e = 0; e < kPath; ++e) cpath[e] = 0.0f;
    block_walk<D, false>(L, S, ln, st, 0, cpath, nullptr, 0);
    float f[FG<D>::KS][8];
    materialize<D>(L, ln, cpath, len, st, f);
#pragma unroll
    for (int s = 0; s < FG<D>::KS; ++s) {
        *reinterpret_cast<float4 *>(row_ptr + 16 * s + 8 * ln.hf) = make_float4(f[s][0], f[s][1], f[s][2], f[s][3]);
        *reinterpret_cast<float4 *>(row_ptr + 16 * s + 8 * ln.hf + 4) = make_float4(f[s][4], f[s][5], f[s][6], f[s][7]);
    }
}

template <int D>
hipError_t launch_fast(int which, const Params &p, hipStream_t s) {
    const int cap = which == 0 ? (p.max_nodes > 0 ? p.max_nodes : 1) : kPath;
    const size_t lds = fast_lds_bytes(cap, D);
    const dim3 grid(p.B * p.Hv), block(FG<D>::THREADS);
    const void *fn = which == 0 ? reinterpret_cast<const void *>(&fast_tree_verify<D>)
                   : which == 1 ? reinterpret_cast<const void *>(&fast_chain_verify<D>)
                                : reinterpret_cast<const void *>(&fast_persist<D>);
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (which == 0) hipLaunchKernelGGL(fast_tree_verify<D>, grid, block, lds, s, p);
    else if (which == 1) hipLaunchKernelGGL(fast_chain_verify<D>, grid, block, lds, s, p);
    else hipLaunchKernelGGL(fast_persist<D>, grid, block, lds, s, p);
    return hipGetLastError();
}

hipError_t launch_fast_any(int which, const Params &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    switch (p.D) {
        case 64: return launch_fast<64>(which, p, s);
        case 128: return launch_fast<128>(which, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool fast_path_supported(int D, int dtype) { return (D == 64 || D == 128) && dtype == GDN_BF16; }
size_t fast_tree_lds_bytes(int max_nodes, int D) { return fast_lds_bytes(max_nodes > 0 ? max_nodes : 1, D); }
hipError_t launch_tree_verify_fast(const Params &p, hipStream_t s) { return launch_fast_any(0, p, s); }
hipError_t launch_chain_verify_fast(const Params &p, hipStream_t s) { return launch_fast_any(1, p, s); }
hipError_t launch_persist_fast(const Params &p, hipStream_t s) { return launch_fast_any(2, p, s); }

}  // namespace gdn

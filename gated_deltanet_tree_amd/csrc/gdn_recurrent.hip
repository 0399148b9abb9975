// gdn_recurrent.hip -- recurrent kernels: chain verify, tree verify (depth-first
// with a state stack: its top in registers, the rest in LDS) and accepted-path
// persist.
//
// One 64-lane workgroup owns one (sequence, value head, slice of RPW state
// rows).  Each state row of D fp32 values is spread over LPR lanes (LPR*4
// consecutive floats per load, so a row slice is read with 16*LPR-byte
// coalesced accesses) and lives in VGPRs for the whole kernel.  Per node, with
// the state S of the node's parent:
//     u = S k,  w = S q          (row dot products: per-lane FMAs + DPP sums)
//     c = b (v - a u)            (per row)
//     o = a w + c (k . q)        (= S' q with S' below)
//     S' = a S + c k^T           (the gated delta rule: a S (I - b k k^T) + b v k^T)
// The three kernels call the same step helpers in the same order, so a chain
// verified by the tree kernel, by the chain kernel, and the state the persist
// kernel writes for a path are bitwise identical.  Compiled without FP
// contraction; every fused multiply-add is an explicit fmaf.
#include <hip/hip_fp16.h>

#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace {

template <int D>
struct Geo {
    static constexpr int LPR = D >= 64 ? 8 : 4;  // lanes per state row
    static constexpr int CPL = D / LPR;          // columns per lane
    static constexpr int NCH = CPL / 4;          // float4 chunks per lane
    static constexpr int RPW = 64 / LPR;         // rows per workgroup
    static constexpr int SLICES = D / RPW;       // workgroups per (sequence, value head)
    static_assert(CPL % 4 == 0, "columns per lane must be a multiple of 4");
};

// column of element e of chunk c held by lane j of a row group
template <int D>
__device__ __forceinline__ int col_of(int j, int c) {
    return c * 4 * Geo<D>::LPR + j * 4;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Load the lane's CPL columns of a length-D vector stored as fp32 or bf16.
template <int D, typename Tin>
__device__ __forceinline__ void load_cols(const Tin *base, int j, float (&x)[Geo<D>::CPL]) {
#pragma unroll
    for (int c = 0; c < Geo<D>::NCH; ++c) {
        const int col = col_of<D>(j, c);
        if constexpr (sizeof(Tin) == 4) {
            const float4 f = *reinterpret_cast<const float4 *>(base + col);
            x[4 * c + 0] = f.x; x[4 * c + 1] = f.y; x[4 * c + 2] = f.z; x[4 * c + 3] = f.w;
        } else {
            const uint2 w = *reinterpret_cast<const uint2 *>(base + col);
            x[4 * c + 0] = bf16_lo(w.x); x[4 * c + 1] = bf16_hi(w.x);
            x[4 * c + 2] = bf16_lo(w.y); x[4 * c + 3] = bf16_hi(w.y);
        }
    }
}

// A lane's CPL columns of a length-D vector as loaded: bf16 stays packed two
// to a register until unpack_cols, so a prefetched node costs half the
// registers of its fp32 form.
template <int D, typename Tin>
struct RawCols {
    using W = std::conditional_t<sizeof(Tin) == 4, float4, uint2>;
    W w[Geo<D>::NCH];
};

template <int D, typename Tin>
__device__ __forceinline__ void load_raw(const Tin *base, int j, RawCols<D, Tin> &r) {
#pragma unroll
    for (int c = 0; c < Geo<D>::NCH; ++c)
        r.w[c] = *reinterpret_cast<const typename RawCols<D, Tin>::W *>(base + col_of<D>(j, c));
}

template <int D, typename Tin>
__device__ __forceinline__ void unpack_cols(const RawCols<D, Tin> &r, float (&x)[Geo<D>::CPL]) {
#pragma unroll
    for (int c = 0; c < Geo<D>::NCH; ++c) {
        if constexpr (sizeof(Tin) == 4) {
            x[4 * c + 0] = r.w[c].x; x[4 * c + 1] = r.w[c].y; x[4 * c + 2] = r.w[c].z; x[4 * c + 3] = r.w[c].w;
        } else {
            x[4 * c + 0] = bf16_lo(r.w[c].x); x[4 * c + 1] = bf16_hi(r.w[c].x);
            x[4 * c + 2] = bf16_lo(r.w[c].y); x[4 * c + 3] = bf16_hi(r.w[c].y);
        }
    }
}

template <typename Tin>
__device__ __forceinline__ float load_one(const Tin *p) {
    if constexpr (sizeof(Tin) == 4) return *p;
    else return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

template <int D>
__device__ __forceinline__ void load_state(const float *row_base, int j, float (&S)[Geo<D>::CPL]) {
#pragma unroll
    for (int c = 0; c < Geo<D>::NCH; ++c) {
        const float4 f = *reinterpret_cast<const float4 *>(row_base + col_of<D>(j, c));
        S[4 * c + 0] = f.x; S[4 * c + 1] = f.y; S[4 * c + 2] = f.z; S[4 * c + 3] = f.w;
    }
}

template <int D>
__device__ __forceinline__ void store_state(float *row_base, int j, const float (&S)[Geo<D>::CPL]) {
#pragma unroll
    for (int c = 0; c < Geo<D>::NCH; ++c)
        *reinterpret_cast<float4 *>(row_base + col_of<D>(j, c)) =
            make_float4(S[4 * c + 0], S[4 * c + 1], S[4 * c + 2], S[4 * c + 3]);
}

// the lane's columns of a state row, rounded to fp16 (nearest, ties to even)
template <int D>
__device__ __forceinline__ void store_state_f16(uint16_t *row_base, int j, const float (&S)[Geo<D>::CPL]) {
#pragma unroll
    for (int c = 0; c < Geo<D>::NCH; ++c) {
        const __half2 lo = __floats2half2_rn(S[4 * c + 0], S[4 * c + 1]);
        const __half2 hi = __floats2half2_rn(S[4 * c + 2], S[4 * c + 3]);
        *reinterpret_cast<uint2 *>(row_base + col_of<D>(j, c)) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
}

// DPP lane exchange inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each half row

// Sum over the LPR lanes of a row group.  Every lane ends with the same bits
// (each step adds a pair in both orders, and fp addition is commutative).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    x = x + dpp<kQuadXor1>(x);
    x = x + dpp<kQuadXor2>(x);
    if constexpr (LPR == 8) x = x + dpp<kRowHalfMirror>(x);
    return x;
}

// partial dot product of the lane's columns, fixed accumulation order
template <int CPL>
__device__ __forceinline__ float lane_dot(const float (&x)[CPL], const float (&y)[CPL]) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc = fmaf(x[i], y[i], acc);
    return acc;
}

// c = b (v - a u): the row's write coefficient
__device__ __forceinline__ float write_coef(float v, float a, float b, float u) {
    const float au = a * u;
    const float r = v - au;
    return b * r;
}

// S <- a S + c k^T (row part)
template <int CPL>
__device__ __forceinline__ void update_row(float (&S)[CPL], const float (&k)[CPL], float a, float c) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) S[i] = fmaf(c, k[i], a * S[i]);
}

__device__ __forceinline__ float qnan() { return __int_as_float(0x7fc00000); }

// state stack entries the tree kernel keeps in LDS: all but the top
__host__ __device__ __forceinline__ int lds_stack_entries(const Params &P) {
    return P.stack_slots > 1 ? P.stack_slots - 1 : 0;
}

// the plan was made for these dims, including the stack size its preorder assumes
__device__ __forceinline__ bool planned(const Params &P) {
    return ws_plan_matches(P) && P.ws.header[5] == P.stack_slots;
}

struct Tile {
    int b, h, g, slice, lane, j, rloc, row;
};

template <int D>
__device__ __forceinline__ Tile tile_of(const Params &P) {
    using G = Geo<D>;
    Tile t;
    const int wg = blockIdx.x;
    t.slice = wg % G::SLICES;
    t.h = (wg / G::SLICES) % P.Hv;
    t.b = wg / (G::SLICES * P.Hv);
    t.g = t.h / (P.Hv / P.Hk);
    t.lane = threadIdx.x;
    t.j = t.lane % G::LPR;
    t.rloc = t.lane / G::LPR;
    t.row = t.slice * G::RPW + t.rloc;
    return t;
}

// ---------------------------------------------------------------------------
// Tree verify: walk the plan's preorder, keep the state in VGPRs, save
// states that later siblings need on a stack (top entry in VGPRs, the rest in
// LDS).  STORE also writes every
// node's state (leaves included) in fp16 to P.node_states: the pages' own
// tree path, which keeps per-node states for the later commit (GreenGames
// page, "Key wins": the f16 intermediate cache).
// ---------------------------------------------------------------------------
template <int D, typename Tin, bool STORE>
__global__ __launch_bounds__(64) void tree_verify_kernel(Params P) {
    using G = Geo<D>;
    // The state stack's top entry is held in registers; the entries below it
    // are [stack_slots - 1][NCH][64 lanes] float4 in LDS, followed by the
    // preorder, actions and gates of up to max_nodes nodes (tree_lds_bytes).
    extern __shared__ float4 lds_stack[];
    int *s_order = reinterpret_cast<int *>(lds_stack + (size_t)lds_stack_entries(P) * G::NCH * 64);
    int *s_act = s_order + P.max_nodes;
    float *s_a = reinterpret_cast<float *>(s_act + P.max_nodes);
    float *s_b = s_a + P.max_nodes;

    const Tile t = tile_of<D>(P);
    if (!planned(P)) return;  // a planned workspace bounds every tree by max_nodes
    const int lo = P.ws.seq_info[t.b * kSeqInfoInts + 0];
    const int n = P.ws.seq_info[t.b * kSeqInfoInts + 1];
    const int status = P.ws.seq_status[t.b];
    const size_t out_stride = (size_t)P.Hv * D;
    float *out = P.out + ((size_t)lo * P.Hv + t.h) * D + t.row;
    if (status != GDN_SEQ_OK) {
        if (t.j == 0)
            for (int i = 0; i < n; ++i) out[i * out_stride] = qnan();
        return;
    }
    if (n == 0) return;

    for (int i = t.lane; i < n; i += 64) {
        s_order[i] = P.ws.order[lo + i];
        s_act[i] = P.ws.action[lo + i];
        const int node = P.ws.order[lo + i];
        s_a[i] = P.a[(size_t)(lo + node) * P.Hv + t.h];
        s_b[i] = P.b[(size_t)(lo + node) * P.Hv + t.h];
    }
    __syncthreads();

    const int slot = P.slot_idx[t.b];
    const float *S0 = P.state_in + (((size_t)slot * P.Hv + t.h) * D + t.row) * D;
    const Tin *kbase = static_cast<const Tin *>(P.k) + ((size_t)lo * P.Hk + t.g) * D;
    const Tin *qbase = static_cast<const Tin *>(P.q) + ((size_t)lo * P.Hk + t.g) * D;
    const Tin *vbase = static_cast<const Tin *>(P.v) + ((size_t)lo * P.Hv + t.h) * D + t.row;
    const size_t kq_stride = (size_t)P.Hk * D;
    const size_t v_stride = (size_t)P.Hv * D;

    float S[G::CPL];
    load_state<D>(S0, t.j, S);
    float top[G::CPL];  // the stack's top entry when sp > 0
#pragma unroll
    for (int i = 0; i < G::CPL; ++i) top[i] = 0.0f;
    int sp = 0;

    RawCols<D, Tin> kn, qn;
    int node = s_order[0];
    load_raw<D, Tin>(kbase + node * kq_stride, t.j, kn);
    load_raw<D, Tin>(qbase + node * kq_stride, t.j, qn);
    float vn = load_one<Tin>(vbase + node * v_stride);

    for (int p = 0; p < n; ++p) {
        const int act = s_act[p];
        const float a = s_a[p], bb = s_b[p];
        const int cur = node;
        float k[G::CPL], q[G::CPL];
        unpack_cols<D, Tin>(kn, k);
        unpack_cols<D, Tin>(qn, q);
        const float v = vn;
        if (p + 1 < n) {  // prefetch the next node's inputs
            node = s_order[p + 1];
            load_raw<D, Tin>(kbase + node * kq_stride, t.j, kn);
            load_raw<D, Tin>(qbase + node * kq_stride, t.j, qn);
            vn = load_one<Tin>(vbase + node * v_stride);
        }
        // parent state
        const int kind = act & 3;
        if (kind == GDN_ACT_INIT) {
            if (p > 0) load_state<D>(S0, t.j, S);
        } else if (kind != GDN_ACT_CONTINUE && sp > 0) {  // the plan never restores from an empty stack
#pragma unroll
            for (int i = 0; i < G::CPL; ++i) S[i] = top[i];
            if (kind == GDN_ACT_POP && --sp > 0) {  // the entry below becomes the top
                const float4 *src = lds_stack + (size_t)(sp - 1) * G::NCH * 64;
#pragma unroll
                for (int c = 0; c < G::NCH; ++c) {
                    const float4 f = src[c * 64 + t.lane];
                    top[4 * c + 0] = f.x; top[4 * c + 1] = f.y; top[4 * c + 2] = f.z; top[4 * c + 3] = f.w;
                }
            }
        }
        // node step
        const float u = group_sum<G::LPR>(lane_dot<G::CPL>(S, k));
        const float w = group_sum<G::LPR>(lane_dot<G::CPL>(S, q));
        const float kq = group_sum<G::LPR>(lane_dot<G::CPL>(k, q));
        const float c = write_coef(v, a, bb, u);
        const float o = fmaf(c, kq, a * w);
        if (t.j == 0) out[cur * out_stride] = o;
        // a leaf's state is never a parent state (the next position restores
        // or reloads), so updating it for the store changes nothing else
        if (STORE || !(act & GDN_ACT_LEAF)) {
            update_row<G::CPL>(S, k, a, c);
            if (STORE)
                store_state_f16<D>(P.node_states + (((size_t)(lo + cur) * P.Hv + t.h) * D + t.row) * D, t.j, S);
            if ((act & GDN_ACT_PUSH) && sp < P.stack_slots) {  // the plan's order never exceeds the bound
                __syncthreads();
                if (sp > 0) {  // the old top moves to LDS entry sp - 1 <= stack_slots - 2
                    float4 *dst = lds_stack + (size_t)(sp - 1) * G::NCH * 64;
#pragma unroll
                    for (int c4 = 0; c4 < G::NCH; ++c4)
                        dst[c4 * 64 + t.lane] =
                            make_float4(top[4 * c4 + 0], top[4 * c4 + 1], top[4 * c4 + 2], top[4 * c4 + 3]);
                }
#pragma unroll
                for (int i = 0; i < G::CPL; ++i) top[i] = S[i];
                ++sp;
                __syncthreads();
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Chain verify: nodes in index order, each the parent of the next.
// ---------------------------------------------------------------------------
template <int D, typename Tin>
__global__ __launch_bounds__(64) void chain_verify_kernel(Params P) {
    using G = Geo<D>;
    const Tile t = tile_of<D>(P);
    const int lo = P.cu_nodes[t.b], hi = P.cu_nodes[t.b + 1];
    const bool in_bounds = 0 <= lo && lo <= hi && hi <= P.T;
    const bool range_ok = in_bounds && hi - lo <= P.max_nodes;
    const int n = in_bounds ? hi - lo : 0;
    const int slot = range_ok ? P.slot_idx[t.b] : 0;
    const bool slot_ok = slot >= 0 && slot < P.num_slots;
    int status = GDN_SEQ_OK;
    if (!range_ok) status = GDN_SEQ_BAD_NODES;
    else if (n > 0 && !slot_ok) status = GDN_SEQ_BAD_SLOT;
    if (P.has_ws && t.h == 0 && t.slice == 0 && t.lane == 0) {
        if (t.b == 0) {
            P.ws.header[0] = kChainMagic;
            P.ws.header[1] = P.B;
            P.ws.header[2] = P.T;
            P.ws.header[kHdrMisuse] = 0;
        }
        P.ws.seq_status[t.b] = status;
    }
    const size_t out_stride = (size_t)P.Hv * D;
    float *out = P.out ? P.out + ((size_t)lo * P.Hv + t.h) * D + t.row : nullptr;
    if (status != GDN_SEQ_OK) {
        if (out && t.j == 0)
            for (int i = 0; i < n; ++i) out[i * out_stride] = qnan();
        return;
    }
    const int flen = P.final_len ? P.final_len[t.b] : -1;
    float *fin = (P.final_state && slot_ok && flen >= 0 && flen <= n)
                     ? P.final_state + (((size_t)t.b * P.Hv + t.h) * D + t.row) * D
                     : nullptr;

    const float *S0 = P.state_in + (((size_t)slot * P.Hv + t.h) * D + t.row) * D;
    float S[G::CPL];
    if (n == 0 && !fin) return;
    load_state<D>(S0, t.j, S);
    if (fin && flen == 0) store_state<D>(fin, t.j, S);

    const Tin *kbase = static_cast<const Tin *>(P.k) + ((size_t)lo * P.Hk + t.g) * D;
    const Tin *qbase = P.q ? static_cast<const Tin *>(P.q) + ((size_t)lo * P.Hk + t.g) * D : nullptr;
    const Tin *vbase = static_cast<const Tin *>(P.v) + ((size_t)lo * P.Hv + t.h) * D + t.row;
    const float *abase = P.a + (size_t)lo * P.Hv + t.h;
    const float *bbase = P.b + (size_t)lo * P.Hv + t.h;
    const size_t kq_stride = (size_t)P.Hk * D;
    const size_t v_stride = (size_t)P.Hv * D;
    const bool want_out = qbase && out;

    float kn[G::CPL], qn[G::CPL];
    float vn = 0.f, an = 0.f, bn = 0.f;
    if (n > 0) {
        load_cols<D, Tin>(kbase, t.j, kn);
        if (want_out) load_cols<D, Tin>(qbase, t.j, qn);
        vn = load_one<Tin>(vbase);
        an = abase[0];
        bn = bbase[0];
    }
    for (int i = 0; i < n; ++i) {
        float k[G::CPL], q[G::CPL];
#pragma unroll
        for (int e = 0; e < G::CPL; ++e) { k[e] = kn[e]; q[e] = want_out ? qn[e] : 0.f; }
        const float v = vn, a = an, bb = bn;
        if (i + 1 < n) {
            load_cols<D, Tin>(kbase + (i + 1) * kq_stride, t.j, kn);
            if (want_out) load_cols<D, Tin>(qbase + (i + 1) * kq_stride, t.j, qn);
            vn = load_one<Tin>(vbase + (i + 1) * v_stride);
            an = abase[(size_t)(i + 1) * P.Hv];
            bn = bbase[(size_t)(i + 1) * P.Hv];
        }
        const float u = group_sum<G::LPR>(lane_dot<G::CPL>(S, k));
        const float c = write_coef(v, a, bb, u);
        if (want_out) {
            const float w = group_sum<G::LPR>(lane_dot<G::CPL>(S, q));
            const float kq = group_sum<G::LPR>(lane_dot<G::CPL>(k, q));
            const float o = fmaf(c, kq, a * w);
            if (t.j == 0) out[i * out_stride] = o;
        }
        if (i + 1 < n || fin) update_row<G::CPL>(S, k, a, c);
        if (fin && i + 1 == flen) store_state<D>(fin, t.j, S);
    }
}

// ---------------------------------------------------------------------------
// Persist: replay the accepted root-to-node path, store the state in place.
// ---------------------------------------------------------------------------
template <int D, typename Tin>
__global__ __launch_bounds__(64) void persist_kernel(Params P) {
    using G = Geo<D>;
    const Tile t = tile_of<D>(P);
    if (!planned(P)) {  // no slot is written; gdn_tree_status reports the misuse
        if (blockIdx.x == 0 && t.lane == 0) P.ws.header[kHdrMisuse] = 1;
        return;
    }
    const int status = P.ws.seq_status[t.b];
    const int lo = P.ws.seq_info[t.b * kSeqInfoInts + 0];
    const int n = P.ws.seq_info[t.b * kSeqInfoInts + 1];
    if (status != GDN_SEQ_OK || n == 0) return;
    const int m = P.accepted[t.b];
    const bool lead = t.h == 0 && t.slice == 0;
    if (m < -1 || m >= n) {
        if (lead && t.lane == 0) P.ws.seq_status[t.b] = GDN_SEQ_BAD_ACCEPT;
        return;
    }
    if (m == -1) return;
    const int len = P.ws.depth[lo + m];
    const int32_t *np = P.ws.nodepath + (size_t)(lo + m) * GDN_MAX_DEPTH;
    if (lead) {
        if (t.lane < GDN_MAX_DEPTH) P.ws.path[t.b * GDN_MAX_DEPTH + t.lane] = np[t.lane];
        if (t.lane == 0) P.ws.path_len[t.b] = len;
    }
    const int slot = P.slot_idx[t.b];
    float *Srow = P.state_out + (((size_t)slot * P.Hv + t.h) * D + t.row) * D;
    const Tin *kbase = static_cast<const Tin *>(P.k) + ((size_t)lo * P.Hk + t.g) * D;
    const Tin *vbase = static_cast<const Tin *>(P.v) + ((size_t)lo * P.Hv + t.h) * D + t.row;
    const size_t kq_stride = (size_t)P.Hk * D;
    const size_t v_stride = (size_t)P.Hv * D;

    float S[G::CPL];
    load_state<D>(Srow, t.j, S);
    float kn[G::CPL];
    int node = np[0];
    load_cols<D, Tin>(kbase + node * kq_stride, t.j, kn);
    float vn = load_one<Tin>(vbase + node * v_stride);
    float an = P.a[(size_t)(lo + node) * P.Hv + t.h], bn = P.b[(size_t)(lo + node) * P.Hv + t.h];
    for (int s = 0; s < len; ++s) {
        float k[G::CPL];
#pragma unroll
        for (int e = 0; e < G::CPL; ++e) k[e] = kn[e];
        const float v = vn, a = an, bb = bn;
        if (s + 1 < len) {
            node = np[s + 1];
            load_cols<D, Tin>(kbase + node * kq_stride, t.j, kn);
            vn = load_one<Tin>(vbase + node * v_stride);
            an = P.a[(size_t)(lo + node) * P.Hv + t.h];
            bn = P.b[(size_t)(lo + node) * P.Hv + t.h];
        }
        const float u = group_sum<G::LPR>(lane_dot<G::CPL>(S, k));
        const float c = write_coef(v, a, bb, u);
        update_row<G::CPL>(S, k, a, c);
    }
    store_state<D>(Srow, t.j, S);
}

template <int D>
int grid_of(const Params &p) {
    return p.B * p.Hv * Geo<D>::SLICES;
}

// the tree kernel's LDS: the stack entries below the top and four per-node tables
template <int D>
size_t tree_lds_bytes(const Params &p) {
    return (size_t)lds_stack_entries(p) * Geo<D>::NCH * 64 * sizeof(float4) + (size_t)4 * p.max_nodes * sizeof(int);
}

template <int D, typename Tin>
hipError_t launch_tree_d(const Params &p, hipStream_t s) {
    hipLaunchKernelGGL((tree_verify_kernel<D, Tin, false>), dim3(grid_of<D>(p)), dim3(64), tree_lds_bytes<D>(p), s,
                       p);
    return hipGetLastError();
}
template <int D, typename Tin>
hipError_t launch_tree_store_d(const Params &p, hipStream_t s) {
    hipLaunchKernelGGL((tree_verify_kernel<D, Tin, true>), dim3(grid_of<D>(p)), dim3(64), tree_lds_bytes<D>(p), s,
                       p);
    return hipGetLastError();
}

// Persist by copy: the accepted node's stored fp16 state, widened exactly to
// fp32, into the sequence's slot; one workgroup per (sequence, value head)
constexpr int kCopyThreads = 256;
__global__ __launch_bounds__(kCopyThreads) void persist_copy_kernel(Params P) {
    const int b = blockIdx.x / P.Hv, h = blockIdx.x % P.Hv;
    if (!planned(P)) {  // no slot is written; gdn_tree_status reports the misuse
        if (blockIdx.x == 0 && threadIdx.x == 0) P.ws.header[kHdrMisuse] = 1;
        return;
    }
    const int lo = P.ws.seq_info[b * kSeqInfoInts + 0];
    const int n = P.ws.seq_info[b * kSeqInfoInts + 1];
    if (P.ws.seq_status[b] != GDN_SEQ_OK || n == 0) return;
    const int m = P.accepted[b];
    if (m < -1 || m >= n) {
        if (h == 0 && threadIdx.x == 0) P.ws.seq_status[b] = GDN_SEQ_BAD_ACCEPT;
        return;
    }
    if (m == -1) return;
    const int slot = P.slot_idx[b];
    const size_t dd = (size_t)P.D * P.D;
    const uint4 *src = reinterpret_cast<const uint4 *>(P.node_states + ((size_t)(lo + m) * P.Hv + h) * dd);
    float4 *dst = reinterpret_cast<float4 *>(P.state_out + ((size_t)slot * P.Hv + h) * dd);
    for (size_t i = threadIdx.x; i < dd / 8; i += kCopyThreads) {  // 8 values per step
        const uint4 w = src[i];
        const uint32_t e[4] = {w.x, w.y, w.z, w.w};
        float f[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float2 two = __half22float2(__builtin_bit_cast(__half2, e[k]));
            f[2 * k] = two.x;
            f[2 * k + 1] = two.y;
        }
        dst[2 * i] = make_float4(f[0], f[1], f[2], f[3]);
        dst[2 * i + 1] = make_float4(f[4], f[5], f[6], f[7]);
    }
}
template <int D, typename Tin>
hipError_t launch_chain_d(const Params &p, hipStream_t s) {
    hipLaunchKernelGGL((chain_verify_kernel<D, Tin>), dim3(grid_of<D>(p)), dim3(64), 0, s, p);
    return hipGetLastError();
}
template <int D, typename Tin>
hipError_t launch_persist_d(const Params &p, hipStream_t s) {
    hipLaunchKernelGGL((persist_kernel<D, Tin>), dim3(grid_of<D>(p)), dim3(64), 0, s, p);
    return hipGetLastError();
}

#define GDN_DISPATCH(FN, p, dtype, s)                                                   \
    do {                                                                                \
        const bool bf = (dtype) == GDN_BF16;                                            \
        switch ((p).D) {                                                                \
            case 16: return bf ? FN<16, uint16_t>(p, s) : FN<16, float>(p, s);          \
            case 32: return bf ? FN<32, uint16_t>(p, s) : FN<32, float>(p, s);          \
            case 64: return bf ? FN<64, uint16_t>(p, s) : FN<64, float>(p, s);          \
            case 128: return bf ? FN<128, uint16_t>(p, s) : FN<128, float>(p, s);       \
            default: return hipErrorInvalidValue;                                       \
        }                                                                               \
    } while (0)

}  // namespace

hipError_t launch_tree_verify_recurrent(const Params &p, int dtype, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    GDN_DISPATCH(launch_tree_d, p, dtype, s);
}
hipError_t launch_chain_verify_recurrent(const Params &p, int dtype, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    GDN_DISPATCH(launch_chain_d, p, dtype, s);
}
hipError_t launch_persist_recurrent(const Params &p, int dtype, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    GDN_DISPATCH(launch_persist_d, p, dtype, s);
}
hipError_t launch_tree_verify_store(const Params &p, int dtype, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    GDN_DISPATCH(launch_tree_store_d, p, dtype, s);
}
hipError_t launch_persist_copy(const Params &p, hipStream_t s) {
    if (p.B == 0) return hipSuccess;
    hipLaunchKernelGGL(persist_copy_kernel, dim3(p.B * p.Hv), dim3(kCopyThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace gdn

// gdn_ddtree.hip -- the drafter's top-k candidates and the DDTree builder.
//
// The drafter scores the whole vocabulary at each position of its block; the
// tree builder keeps each position's W best candidates in descending order
// (rank 1 first: the GreenGames page, "Key wins", traces a slowdown to that
// order being reversed, which put the worst candidate at the tree root) with
// their log-probabilities, pre-seeds the rank-1 chain ("From autoregressive to
// DDTree") and grows the rest of the budget best first by path score.
//
//   topk_kernel   one workgroup per row: streams the row once (16-byte loads
//                 when the layout allows) with a running (max, sum of
//                 exp(x - max)) for the log-softmax; entries at or above a
//                 wave-wide floor go through an LDS candidate buffer into
//                 per-lane lists of the WT best in argmax order (a NaN counts
//                 as largest, equal values keep the smaller id), which the
//                 waves merge by repeated wave-wide extraction.  HBM-bound.
//   build_kernel  one wave per sequence: the chain, then one candidate per
//                 node (its next unused rank) and a wave-wide extraction of
//                 the best candidate per added node.  Latency-bound.
#include <algorithm>
#include <cfloat>
#include <climits>

#include "gdn_internal.h"

namespace gdn {
namespace {

// argmax order: a NaN before any number (smaller id first among NaNs), else the
// larger value, then the smaller id; (-inf, INT_MAX) is an empty slot
__device__ __forceinline__ bool before(float v1, int i1, float v2, int i2) {
    const bool n1 = v1 != v1, n2 = v2 != v2;
    if (n1 | n2) return n1 && (!n2 || i1 < i2);
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

// threads per row: 1024 for the short lists (more loads in flight per row), 512 from
// W = 8 on, where the lists' own work grows with the wave count
template <int WT>
constexpr int topk_threads() { return WT <= 4 ? 1024 : 512; }
// 16-byte loads in flight per thread: 4 for the short lists (1024 threads), 8 at W = 8,
// 6 at W = 16 (8 there spills the larger lists)
template <int WT>
constexpr int topk_unroll() { return WT <= 4 ? 4 : WT <= 8 ? 8 : 6; }

template <int WT>
struct TopList {
    float v[WT];
    int i[WT];
    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int k = 0; k < WT; ++k) {
            v[k] = -INFINITY;
            i[k] = INT_MAX;
        }
    }
    // keeps the WT best offers in argmax order, whatever the order of offers
    __device__ __forceinline__ void offer(float x, int id) {
        if (before(x, id, v[WT - 1], i[WT - 1])) {
            float cv = x;
            int ci = id;
#pragma unroll
            for (int k = 0; k < WT; ++k) {
                const bool sw = before(cv, ci, v[k], i[k]);
                const float tv = v[k];
                const int ti = i[k];
                v[k] = sw ? cv : tv;
                i[k] = sw ? ci : ti;
                cv = sw ? tv : cv;
                ci = sw ? ti : ci;
            }
        }
    }
    __device__ __forceinline__ void pop() {
#pragma unroll
        for (int k = 0; k < WT - 1; ++k) {
            v[k] = v[k + 1];
            i[k] = i[k + 1];
        }
        v[WT - 1] = -INFINITY;
        i[WT - 1] = INT_MAX;
    }
};

// running log-sum-exp state: m starts at -FLT_MAX (finite) so that -inf
// entries add exp(-inf) = 0; a NaN or a +inf entry makes s NaN
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
    const float mm = fmaxf(m, m2);
    s = s * __expf(m - mm) + s2 * __expf(m2 - mm);
    m = mm;
}

// the best entry among the wave's list heads; its owner pops it
template <int WT>
__device__ __forceinline__ void wave_take(TopList<WT> &L, float &bv, int &bi) {
    bv = L.v[0];
    bi = L.i[0];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (before(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (bi != INT_MAX && L.i[0] == bi) L.pop();
}

// A wave-wide lower bound of the row's W-th best value: the largest of the
// lanes' own W-th best entries (that lane holds W entries at least as good).
// Entries below it can never enter the row's top W.
template <int WT>
__device__ __forceinline__ float wave_floor(const TopList<WT> &L) {
    float t = L.v[WT - 1];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t = fmaxf(t, __shfl_xor(t, off));
    return t;
}

constexpr int kCandBuf = 512;  // per-wave candidate buffer (LDS entries)

template <int WT, bool VEC, int kTopkThreads = topk_threads<WT>()>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(int vocab, int width, const float *logits,
                                                             int32_t *tokens, float *logp) {
    constexpr int NW = kTopkThreads / 64;
    constexpr int kTopkUnroll = topk_unroll<WT>();
    __shared__ float s_v[NW][WT];
    __shared__ int s_i[NW][WT];
    __shared__ float s_m[NW], s_s[NW];
    __shared__ float c_v[NW][kCandBuf];
    __shared__ int c_i[NW][kCandBuf];
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
    const float *x = logits + (size_t)row * vocab;
    TopList<WT> L;
    L.clear();
    float m = -FLT_MAX, s = 0.0f;
    // Entries at or above the wave's floor (and NaNs) are appended to the wave's
    // candidate buffer; a full buffer is folded into the lanes' lists (each lane
    // takes every 64th entry; the lists compare ids on equal values, so the
    // order of offers does not matter) and the floor is raised.  With a good
    // floor almost every entry is dismissed by one comparison.
    // floor_v is the same on every lane except after a lane saw only NaNs, when at
    // least W NaNs lead the row and any floor keeps them (a NaN always passes)
    float floor_v = -INFINITY;
    int cnt = 0;  // wave-uniform
    const unsigned long long below = (1ull << lane) - 1ull;
    auto fold = [&]() {
        for (int k = lane; k < cnt; k += 64) L.offer(c_v[w][k], c_i[w][k]);
        cnt = 0;
        floor_v = wave_floor(L);
    };
    // every lane runs the same number of steps (the buffer count and the floor
    // must stay uniform across the wave); entries past the row are not offered
    auto take = [&](float e, int id, bool valid) {
        const bool pass = valid && !(e < floor_v);
        const unsigned long long mask = __ballot(pass);
        if (mask) {
            if (pass) {
                const int pos = cnt + __popcll(mask & below);
                c_v[w][pos] = e;
                c_i[w][pos] = id;
            }
            cnt += __popcll(mask);
            if (cnt > kCandBuf - 64) fold();
        }
    };
    if (VEC) {
        const float4 *x4 = reinterpret_cast<const float4 *>(x);
        const int n4 = vocab / 4;
        auto eat = [&](const float4 r, int j, bool valid) {
            const float g = fmaxf(fmaxf(r.x, r.y), fmaxf(r.z, r.w));
            if (g > m) {
                s *= __expf(m - g);
                m = g;
            }
            s += (__expf(r.x - m) + __expf(r.y - m)) + (__expf(r.z - m) + __expf(r.w - m));
            take(r.x, 4 * j, valid);
            take(r.y, 4 * j + 1, valid);
            take(r.z, 4 * j + 2, valid);
            take(r.w, 4 * j + 3, valid);
        };
        constexpr int step = kTopkUnroll * kTopkThreads;
        int base = 0;
        for (; base + step <= n4; base += step) {  // whole blocks: no lane idles
            float4 r[kTopkUnroll];
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) r[u] = x4[base + u * kTopkThreads + tid];
            if (base == 0) {
                // a first floor from the first block: the WT-th largest of the lanes' own
                // maxima (WT distinct entries at least that large)
                float lm = -INFINITY;
#pragma unroll
                for (int u = 0; u < kTopkUnroll; ++u)
                    lm = fmaxf(lm, fmaxf(fmaxf(r[u].x, r[u].y), fmaxf(r[u].z, r[u].w)));
                float f = -INFINITY;
                bool taken = false;
#pragma unroll 1
                for (int k = 0; k < WT; ++k) {
                    float bv = taken ? -INFINITY : lm;
                    int bl = taken ? 64 : lane;
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1) {
                        const float ov = __shfl_xor(bv, off);
                        const int ol = __shfl_xor(bl, off);
                        if (ov > bv || (ov == bv && ol < bl)) {
                            bv = ov;
                            bl = ol;
                        }
                    }
                    taken = taken || bl == lane;
                    f = bv;
                }
                floor_v = f;
            }
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) eat(r[u], base + u * kTopkThreads + tid, true);
        }
        for (int u = 0; u < kTopkUnroll; ++u) {  // the ragged last block, one load at a time
            const int j = base + u * kTopkThreads + tid;
            const bool valid = j < n4;
            eat(valid ? x4[j] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY), j, valid);
        }
    } else {
        auto eat = [&](float r, int j, bool valid) {
            if (r > m) {
                s *= __expf(m - r);
                m = r;
            }
            s += __expf(r - m);
            take(r, j, valid);
        };
        constexpr int step = kTopkUnroll * kTopkThreads;
        int base = 0;
        for (; base + step <= vocab; base += step) {
            float r[kTopkUnroll];
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) r[u] = x[base + u * kTopkThreads + tid];
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) eat(r[u], base + u * kTopkThreads + tid, true);
        }
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int j = base + u * kTopkThreads + tid;
            const bool valid = j < vocab;
            eat(valid ? x[j] : -INFINITY, j, valid);
        }
    }
    fold();
    // log-sum-exp over the wave, then the workgroup
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lse_merge(m, s, __shfl_xor(m, off), __shfl_xor(s, off));
    // each wave's best WT entries, in order
#pragma unroll 1
    for (int r = 0; r < WT; ++r) {
        float bv;
        int bi;
        wave_take(L, bv, bi);
        if (lane == 0) {
            s_v[w][r] = bv;
            s_i[w][r] = bi;
        }
    }
    if (lane == 0) {
        s_m[w] = m;
        s_s[w] = s;
    }
    __syncthreads();
    if (w != 0) return;
    // wave 0 merges the NW lists (lane k < NW holds wave k's list)
    TopList<WT> M;
    M.clear();
    if (lane < NW) {
#pragma unroll
        for (int k = 0; k < WT; ++k) {
            M.v[k] = s_v[lane][k];
            M.i[k] = s_i[lane][k];
        }
    }
    float gm = s_m[0], gs = s_s[0];
    for (int k = 1; k < NW; ++k) lse_merge(gm, gs, s_m[k], s_s[k]);
    // every entry equal to -inf: no finite mass (all log p -inf); NaN mass: no distribution
    const float lse = gm + logf(gs);
#pragma unroll 1
    for (int r = 0; r < width; ++r) {
        float bv;
        int bi;
        wave_take(M, bv, bi);
        if (lane == 0) {
            const bool none = bi == INT_MAX;
            tokens[(size_t)row * width + r] = none ? -1 : bi;
            float lp;
            if (none || gs == 0.0f) lp = -INFINITY;
            else if (gs != gs) lp = __int_as_float(0x7fc00000);
            else lp = bv - lse;
            logp[(size_t)row * width + r] = lp;
        }
    }
}

// ---------------------------------------------------------------------------
// Builder
// ---------------------------------------------------------------------------
constexpr int kSlots = GDN_MAX_NODES / 64;  // nodes per lane

struct BuildArgs {
    int B, levels, width, budget, depth_cap, nodes;
    const int32_t *root_token, *tokens;
    const float *logp;
    int32_t *parent, *node_token, *cu_nodes;
};

// candidate key: higher score first, then (child depth, rank, parent id) packed
// ascending; an exhausted node offers (-inf, INT_MAX)
__device__ __forceinline__ bool cand_before(float s1, int k1, float s2, int k2) {
    return s1 > s2 || (s1 == s2 && k1 < k2);
}

__global__ __launch_bounds__(64) void build_kernel(BuildArgs A) {
    __shared__ float s_lp[GDN_MAX_DEPTH][kMaxDraftWidth];
    __shared__ int s_tok[GDN_MAX_DEPTH][kMaxDraftWidth];
    __shared__ int s_par[GDN_MAX_NODES], s_ntok[GDN_MAX_NODES];
    const int lane = threadIdx.x, b = blockIdx.x;
    const int W = A.width, cap = A.depth_cap, N = A.nodes;
    const int rows = min(A.levels, cap - 1);  // levels a node can occupy
    for (int e = lane; e < rows * W; e += 64) {
        const int l = e / W, r = e % W;
        const size_t at = ((size_t)b * A.levels + l) * W + r;
        const float v = A.logp[at];
        s_lp[l][r] = v != v ? -INFINITY : v;
        s_tok[l][r] = A.tokens[at];
    }
    __syncthreads();

    // node state, node = lane + 64 k: score, depth, children taken; and its candidate
    float sc[kSlots], cs[kSlots];
    int dp[kSlots], nc[kSlots], ck[kSlots];
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
        sc[k] = 0.0f;
        dp[k] = 0;
        nc[k] = 0;
        cs[k] = -INFINITY;
        ck[k] = INT_MAX;
    }
    auto refresh = [&](int k, int node) {
        const bool open = dp[k] > 0 && dp[k] < cap && nc[k] < W;
        cs[k] = open ? sc[k] + s_lp[open ? dp[k] - 1 : 0][open ? nc[k] : 0] : -INFINITY;
        ck[k] = open ? ((dp[k] + 1) << 14) | (nc[k] << 9) | node : INT_MAX;
    };
    // the root, then the rank-1 chain: node i is the first child of node i - 1
    const int chain = min(A.budget, cap - 1);
    float score = 0.0f;
    if (lane == 0) {
        s_par[0] = -1;
        s_ntok[0] = A.root_token ? A.root_token[b] : -1;
    }
    for (int i = 0; i <= chain; ++i) {
        if (i > 0) {
            score = score + s_lp[i - 1][0];
            if (lane == 0) {
                s_par[i] = i - 1;
                s_ntok[i] = s_tok[i - 1][0];
            }
        }
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            if (lane + 64 * k == i) {
                sc[k] = score;
                dp[k] = i + 1;
                nc[k] = i < chain ? 1 : 0;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kSlots; ++k) refresh(k, lane + 64 * k);

    // best first: one node per round
    for (int n = chain + 1; n < N; ++n) {
        float bs = cs[0];
        int bk = ck[0];
#pragma unroll
        for (int k = 1; k < kSlots; ++k)
            if (cand_before(cs[k], ck[k], bs, bk)) {
                bs = cs[k];
                bk = ck[k];
            }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float os = __shfl_xor(bs, off);
            const int ok = __shfl_xor(bk, off);
            if (cand_before(os, ok, bs, bk)) {
                bs = os;
                bk = ok;
            }
        }
        if (bk == INT_MAX) break;  // cannot happen: the node count is what the limits allow
        const int d = bk >> 14, r = (bk >> 9) & 31, p = bk & 511;
        if (lane == 0) {
            s_par[n] = p;
            s_ntok[n] = s_tok[d - 2][r];
        }
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            const int node = lane + 64 * k;
            if (node == p) {
                nc[k] += 1;
                refresh(k, node);
            }
            if (node == n) {
                sc[k] = bs;
                dp[k] = d;
                nc[k] = 0;
                refresh(k, node);
            }
        }
    }
    __syncthreads();
    for (int i = lane; i < N; i += 64) {
        A.parent[(size_t)b * N + i] = s_par[i];
        A.node_token[(size_t)b * N + i] = s_ntok[i];
    }
    if (lane == 0) {
        A.cu_nodes[b] = b * N;
        if (b == A.B - 1) A.cu_nodes[A.B] = A.B * N;
    }
}

__global__ void cu_zero_kernel(int32_t *cu_nodes) { cu_nodes[0] = 0; }

}  // namespace

int ddtree_nodes(int levels, int width, int budget, int max_depth) {
    const int cap = std::min(levels + 1, max_depth);
    long long total = 0, layer = 1;
    for (int d = 1; d < cap && total < budget; ++d) {
        layer *= width;
        total += layer;
    }
    return 1 + (int)std::min<long long>(budget, total);
}

hipError_t launch_draft_topk(int rows, int vocab, int width, const float *logits, int32_t *tokens, float *logp,
                             hipStream_t s) {
    const bool vec = vocab % 4 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0;
    const dim3 grid(rows);
#define GDN_TOPK_CASE(WT)                                                                                     \
    if (width <= WT) {                                                                                        \
        const dim3 block(topk_threads<WT>());                                                                 \
        if (vec)                                                                                              \
            hipLaunchKernelGGL((topk_kernel<WT, true>), grid, block, 0, s, vocab, width, logits, tokens, logp);  \
        else                                                                                                  \
            hipLaunchKernelGGL((topk_kernel<WT, false>), grid, block, 0, s, vocab, width, logits, tokens, logp); \
        return hipGetLastError();                                                                             \
    }
    GDN_TOPK_CASE(1)
    GDN_TOPK_CASE(2)
    GDN_TOPK_CASE(4)
    GDN_TOPK_CASE(8)
    GDN_TOPK_CASE(16)
#undef GDN_TOPK_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_ddtree_build(int B, int levels, int width, int budget, int max_depth, const int32_t *root_token,
                               const int32_t *tokens, const float *logp, int32_t *parent, int32_t *node_token,
                               int32_t *cu_nodes, hipStream_t s) {
    BuildArgs A;
    A.B = B;
    A.levels = levels;
    A.width = width;
    A.budget = budget;
    A.depth_cap = std::min(levels + 1, max_depth);
    A.nodes = ddtree_nodes(levels, width, budget, max_depth);
    A.root_token = root_token;
    A.tokens = tokens;
    A.logp = logp;
    A.parent = parent;
    A.node_token = node_token;
    A.cu_nodes = cu_nodes;
    if (B == 0) {  // no trees: cu_nodes = {0}
        hipLaunchKernelGGL(cu_zero_kernel, dim3(1), dim3(1), 0, s, cu_nodes);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(build_kernel, dim3(B), dim3(64), 0, s, A);
    return hipGetLastError();
}

}  // namespace gdn

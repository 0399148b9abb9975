// gdn_accept.hip -- greedy (temperature-0) acceptance of each draft tree
// against the target's verify logits.
//
// The verify forward yields one vocabulary-wide logits row per tree node
// (GreenGames page, "Key wins": the verify logits buffer has budget + 1 rows);
// the target's token after node n is the first index of the largest entry of
// row n (a NaN counts as largest).  Starting at the root, the walk moves to
// the smallest-id child whose draft token equals the target's token after the
// current node, and stops where no child does: the stop node is the accepted
// node, its depth the accept length, and its row's argmax the next token
// (greedy-only verification, GreenGames "What comes next"; lossless at
// temperature 0, dflash-caddtree-integrations README "The shared method").
//
// Two launches:
//   argmax_kernel  one workgroup per (node, slice of the row): streams the
//                  slice once with 16-byte loads and writes (value, index)
//                  of its first largest entry into the workspace.  This is
//                  the HBM-bound part: T x vocab x 4 bytes.
//   walk_kernel    one wave per sequence: merges the slices of its nodes,
//                  then walks down the tree with ballots (<= 15 steps).
#include <climits>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kArgThreads = 256;
constexpr int kArgUnroll = 4;  // 16-byte loads in flight per thread

// (v1, i1) comes before (v2, i2) in argmax order: a NaN before any number
// (the smaller index among NaNs), else the larger value, then the smaller
// index (+0 and -0 are equal)
__device__ __forceinline__ bool beats(float v1, int i1, float v2, int i2) {
    const bool n1 = v1 != v1, n2 = v2 != v2;
    if (n1 | n2) return n1 && (!n2 || i1 < i2);
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

__device__ __forceinline__ void take(float v, int i, float &bv, int &bi) {
    if (beats(v, i, bv, bi)) {
        bv = v;
        bi = i;
    }
}

// One slice [beg, end) of one row.  The scan keeps, per thread, the first
// index of its largest entry above -inf (strict >, indices visited in
// increasing order); NaNs are invisible to it and are caught through a
// running sum that a NaN turns into NaN, which sends the slice through an
// exact rescan for its first NaN.
template <bool VEC>
__global__ __launch_bounds__(kArgThreads) void argmax_kernel(Params P) {
    __shared__ float s_v[kArgThreads / 64];
    __shared__ int s_i[kArgThreads / 64];
    const int row = blockIdx.x / P.chunks, c = blockIdx.x % P.chunks;
    const int tid = threadIdx.x, lane = tid % 64, w = tid / 64;
    const int beg = c * P.chunk_len;
    const int end = min(P.vocab, beg + P.chunk_len);
    const float *x = P.logits + (size_t)row * P.vocab;
    float bv = -INFINITY, sum = 0.0f;
    int bi = INT_MAX;
    if (VEC) {  // beg, end and the row start are multiples of 4 floats
        const float4 *x4 = reinterpret_cast<const float4 *>(x);
        const int e4 = end / 4;
        float cv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        int ci[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};  // 16-byte group of each component's best
        int j = beg / 4 + tid;
        for (; j + (kArgUnroll - 1) * kArgThreads < e4; j += kArgUnroll * kArgThreads) {
            float4 r[kArgUnroll];
#pragma unroll
            for (int u = 0; u < kArgUnroll; ++u) r[u] = x4[j + u * kArgThreads];
#pragma unroll
            for (int u = 0; u < kArgUnroll; ++u) {
                const int g = j + u * kArgThreads;
                const float e[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const bool up = e[q] > cv[q];
                    cv[q] = up ? e[q] : cv[q];
                    ci[q] = up ? g : ci[q];
                }
                sum += (e[0] + e[1]) + (e[2] + e[3]);
            }
        }
        for (; j < e4; j += kArgThreads) {
            const float4 r = x4[j];
            const float e[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool up = e[q] > cv[q];
                cv[q] = up ? e[q] : cv[q];
                ci[q] = up ? j : ci[q];
            }
            sum += (e[0] + e[1]) + (e[2] + e[3]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) take(cv[q], ci[q] == INT_MAX ? INT_MAX : 4 * ci[q] + q, bv, bi);
    } else {
        int i = beg + tid;
        for (; i + (kArgUnroll - 1) * kArgThreads < end; i += kArgUnroll * kArgThreads) {
            float r[kArgUnroll];
#pragma unroll
            for (int u = 0; u < kArgUnroll; ++u) r[u] = x[i + u * kArgThreads];
#pragma unroll
            for (int u = 0; u < kArgUnroll; ++u) {
                if (r[u] > bv) {
                    bv = r[u];
                    bi = i + u * kArgThreads;
                }
                sum += r[u];
            }
        }
        for (; i < end; i += kArgThreads) {
            const float r = x[i];
            if (r > bv) {
                bv = r;
                bi = i;
            }
            sum += r;
        }
    }
    // a NaN anywhere in the slice (or +inf meeting -inf): find the first NaN exactly
    if (__syncthreads_or(sum != sum)) {
        int first = INT_MAX;
        for (int i = beg + tid; i < end; i += kArgThreads) {
            const float r = x[i];
            if (r != r) {
                first = i;
                break;
            }
        }
        if (first != INT_MAX) {
            bv = __int_as_float(0x7fc00000);
            bi = first;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        take(ov, oi, bv, bi);
    }
    if (lane == 0) {
        s_v[w] = bv;
        s_i[w] = bi;
    }
    __syncthreads();
    if (tid == 0) {
#pragma unroll
        for (int k = 1; k < kArgThreads / 64; ++k) take(s_v[k], s_i[k], bv, bi);
        // nothing above -inf and no NaN: every entry is -inf, the first one wins
        if (bi == INT_MAX && end > beg) bi = beg;
        P.ws.amax[(size_t)row * kAcceptChunks + c] = make_int2(__float_as_int(bv), bi);
    }
}

// argmax of a whole row from its slices (slices past the row end hold
// (-inf, INT_MAX), which never wins); all slice loads are issued before the
// first comparison
__device__ __forceinline__ int row_argmax(const Params &P, int row) {
    const int2 *pr = P.ws.amax + (size_t)row * kAcceptChunks;
    int2 e[kAcceptChunks];
#pragma unroll
    for (int c = 0; c < kAcceptChunks; ++c) e[c] = c < P.chunks ? pr[c] : make_int2(0, INT_MAX);
    float bv = __int_as_float(e[0].x);
    int bi = e[0].y;
#pragma unroll
    for (int c = 1; c < kAcceptChunks; ++c)
        if (c < P.chunks) take(__int_as_float(e[c].x), e[c].y, bv, bi);
    return bi;
}

constexpr int kNodesPerLane = GDN_MAX_NODES / 64;

// blocks [0, B): one sequence each; blocks [B, ...): 64 rows each of the
// optional per-node target_out
__global__ __launch_bounds__(64) void walk_kernel(Params P) {
    __shared__ int s_tgt[GDN_MAX_NODES];
    const int lane = threadIdx.x;
    const int b = blockIdx.x;
    if (b >= P.B) {
        const int row = (b - P.B) * 64 + lane;
        if (row < P.T) P.target_out[row] = row_argmax(P, row);
        return;
    }
    const bool planned = ws_plan_matches(P);
    const int4 info = *reinterpret_cast<const int4 *>(P.ws.seq_info + b * kSeqInfoInts);
    if (!planned || info.z != GDN_SEQ_OK || info.y <= 0 || info.y > GDN_MAX_NODES) {
        // a plan made for other dims: nothing is accepted, and gdn_tree_status reports the misuse
        if (!planned && b == 0 && lane == 0) P.ws.header[kHdrMisuse] = 1;
        if (lane == 0) {
            P.accepted_out[b] = -1;
            P.accept_len_out[b] = 0;
            P.next_token_out[b] = -1;
        }
        return;
    }
    const int lo = info.x, n = info.y;
    // node t = lane + 64 k: its parent (from the plan's path row, fetched whole
    // next to its depth) and draft token
    int par[kNodesPerLane], tok[kNodesPerLane];
#pragma unroll
    for (int k = 0; k < kNodesPerLane; ++k) {
        const int t = lane + 64 * k;
        par[k] = -2;
        tok[k] = 0;
        if (64 * k < n) {  // uniform: the whole wave takes part in this group
            const int tt = t < n ? t : n - 1;
            const int4 *np = reinterpret_cast<const int4 *>(P.ws.nodepath + (size_t)(lo + tt) * GDN_MAX_DEPTH);
            int4 row[GDN_MAX_DEPTH / 4];
#pragma unroll
            for (int q = 0; q < GDN_MAX_DEPTH / 4; ++q) row[q] = np[q];
            const int d = P.ws.depth[lo + tt];
            const int tk = P.draft_token[lo + tt];
            const int tg = row_argmax(P, lo + tt);
            // the parent is path entry d - 2 (root first); a root has none
            int pp = -1;
#pragma unroll
            for (int q = 0; q < GDN_MAX_DEPTH / 4; ++q) {
                pp = (4 * q + 0 == d - 2) ? row[q].x : pp;
                pp = (4 * q + 1 == d - 2) ? row[q].y : pp;
                pp = (4 * q + 2 == d - 2) ? row[q].z : pp;
                pp = (4 * q + 3 == d - 2) ? row[q].w : pp;
            }
            if (t < n) {
                par[k] = pp;
                tok[k] = tk;
                s_tgt[t] = tg;
            }
        }
    }
    __syncthreads();
    // smallest-id root, then down while a child carries the target's token
    auto first_of = [&](auto pred) {
        int found = -1;
#pragma unroll
        for (int k = 0; k < kNodesPerLane; ++k) {
            const unsigned long long m = __ballot(pred(k));
            if (found < 0 && m != 0ull) found = 64 * k + __ffsll((long long)m) - 1;
        }
        return found;
    };
    int cur = first_of([&](int k) { return par[k] == -1; });
    int len = 1;
    for (int step = 1; step < GDN_MAX_DEPTH; ++step) {
        const int want = s_tgt[cur];
        const int nxt = first_of([&](int k) { return par[k] == cur && tok[k] == want; });
        if (nxt < 0) break;
        cur = nxt;
        ++len;
    }
    if (lane == 0) {
        P.accepted_out[b] = cur;
        P.accept_len_out[b] = len;
        P.next_token_out[b] = s_tgt[cur];
    }
}

}  // namespace

hipError_t launch_accept(const Params &p, hipStream_t s) {
    if (p.T > 0) {
        const bool vec = p.vocab % 4 == 0 && reinterpret_cast<uintptr_t>(p.logits) % 16 == 0;
        const dim3 grid(p.T * p.chunks), block(kArgThreads);
        if (vec)
            hipLaunchKernelGGL(argmax_kernel<true>, grid, block, 0, s, p);
        else
            hipLaunchKernelGGL(argmax_kernel<false>, grid, block, 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int extra = p.target_out ? (p.T + 63) / 64 : 0;
    if (p.B + extra > 0) hipLaunchKernelGGL(walk_kernel, dim3(p.B + extra), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace gdn

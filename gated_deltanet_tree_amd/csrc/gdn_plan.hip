// gdn_plan.hip -- device-side validation and traversal metadata of the draft
// trees (one workgroup per sequence, one thread per node).
//
// The trees arrive in parent-pointer form from DDTree's tree builder
// (GreenGames page, "From autoregressive to DDTree"), depth bounded by the
// 16-token drafting block (GreenGames, "Prefill").  For each sequence the
// plan writes: its verdict, each node's depth and root-to-node path, and a
// depth-first preorder in which children are visited by increasing (subtree
// size, id) -- the largest child last -- with one action word per position.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kPlanDupPer = 2;  // other sequences checked per thread from registers

// workgroup-wide "any": a ballot when the workgroup is one wave (no LDS round trip)
template <int NT>
__device__ __forceinline__ bool wg_any(bool pred) {
    if constexpr (NT == 64) return __ballot(pred) != 0ull;
    else return __syncthreads_or(pred) != 0;
}

// NT threads, one per node: NT = 64 (a single wave, whose barriers cost nothing)
// when every tree fits, else NT = GDN_MAX_NODES
template <int NT>
__global__ __launch_bounds__(NT) void plan_kernel(Params P) {
    constexpr int kPlanThreads = NT;
    __shared__ int s_par[kPlanThreads];
    __shared__ int s_size[kPlanThreads];
    __shared__ int s_nchild[kPlanThreads];
    __shared__ int s_off[kPlanThreads];
    __shared__ int s_later[kPlanThreads];

    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const WsPtrs W = P.ws;
    if (b == 0 && t == 0) {
        W.header[0] = kMagic;
        W.header[1] = P.B;
        W.header[2] = P.T;
        W.header[3] = P.max_nodes;
        W.header[4] = P.max_depth;
        W.header[5] = P.stack_slots;
        W.header[kHdrMisuse] = 0;
    }
    if (b >= P.B) return;

    // ---- node range (the other sequences' ranges and slots are fetched in the
    // same round trip, for the duplicate-slot check) --------------------------
    const int lo = P.cu_nodes[b], hi = P.cu_nodes[b + 1];
    const int my_slot = P.slot_idx[b];
    int o_lo[kPlanDupPer], o_hi[kPlanDupPer], o_slot[kPlanDupPer];
#pragma unroll
    for (int u = 0; u < kPlanDupPer; ++u) {
        const int o = t + u * kPlanThreads;
        o_lo[u] = o < P.B ? P.cu_nodes[o] : 0;
        o_hi[u] = o < P.B ? P.cu_nodes[o + 1] : 0;
        o_slot[u] = o < P.B ? P.slot_idx[o] : -1;
    }
    int status = GDN_SEQ_OK;
    // in_bounds: the range lies inside [0, T] (its outputs can be NaN-filled);
    // range_ok: additionally no longer than max_nodes
    const bool in_bounds = 0 <= lo && lo <= hi && hi <= P.T;
    const bool range_ok = in_bounds && hi - lo <= P.max_nodes;
    if (!range_ok) status = GDN_SEQ_BAD_NODES;
    const int n = range_ok ? hi - lo : 0;

    // ---- slot: in range and not shared with another non-empty sequence ------
    if (status == GDN_SEQ_OK && n > 0) {
        const int slot = my_slot;
        if (slot < 0 || slot >= P.num_slots) {
            status = GDN_SEQ_BAD_SLOT;
        } else {
            int dup = 0;
#pragma unroll
            for (int u = 0; u < kPlanDupPer; ++u) {
                const int o = t + u * kPlanThreads;
                const int lo2 = o_lo[u], hi2 = o_hi[u];
                const bool ok2 = 0 <= lo2 && lo2 <= hi2 && hi2 <= P.T && hi2 - lo2 <= P.max_nodes;
                if (o < P.B && o != b && ok2 && hi2 > lo2 && o_slot[u] == slot) dup = 1;
            }
            for (int o = t + kPlanDupPer * kPlanThreads; o < P.B; o += kPlanThreads) {  // very large batches
                const int lo2 = P.cu_nodes[o], hi2 = P.cu_nodes[o + 1];
                const bool ok2 = 0 <= lo2 && lo2 <= hi2 && hi2 <= P.T && hi2 - lo2 <= P.max_nodes;
                if (o != b && ok2 && hi2 > lo2 && P.slot_idx[o] == slot) dup = 1;
            }
            if (wg_any<NT>(dup)) status = GDN_SEQ_DUP_SLOT;
        }
    }

    // ---- parent ids ------------------------------------------------------------
    int par = -1;
    if (status == GDN_SEQ_OK && n > 0) {
        if (t < n) par = P.parent[lo + t];
        const bool bad = t < n && !(par == -1 || (par >= 0 && par < n && par != t));
        if (wg_any<NT>(bad)) status = GDN_SEQ_BAD_PARENT;
    }

    // ---- depth: every ancestor walk must reach a root within max_depth nodes -----
    // anc[j] is the ancestor j steps up from this node (anc[0] = the node), j < depth
    int depth = 0;
    int anc[GDN_MAX_DEPTH];
    if (status == GDN_SEQ_OK && n > 0) {
        s_par[t] = par;
        s_size[t] = 0;
        s_nchild[t] = 0;
        __syncthreads();
        bool deep = false;
        if (t < n) {
            int x = t;
#pragma unroll
            for (int j = 0; j < GDN_MAX_DEPTH; ++j) {
                anc[j] = x;
                const bool step = x != -1 && depth < P.max_depth;
                depth += step ? 1 : 0;
                x = step ? s_par[x < 0 ? 0 : x] : x;
            }
            deep = x != -1;
        }
        if (wg_any<NT>(deep)) status = GDN_SEQ_CYCLE_OR_DEPTH;
    }

    if (status == GDN_SEQ_OK && n > 0) {
        // subtree sizes (each node counts itself into every ancestor) and child counts
        if (t < n) {
#pragma unroll
            for (int j = 0; j < GDN_MAX_DEPTH; ++j)
                if (j < depth) atomicAdd(&s_size[anc[j]], 1);
            if (par >= 0) atomicAdd(&s_nchild[par], 1);
        }
        __syncthreads();
        // siblings visited before this node (smaller (size, id)) and after it
        if constexpr (NT == 64) {
            // one wave: node s2's parent and size come from lane s2's registers
            const int my = s_size[t];
            int off = 0, later = 0;
            for (int s2 = 0; s2 < n; ++s2) {
                const int ps = __builtin_amdgcn_readlane(par, s2), ss = __builtin_amdgcn_readlane(my, s2);
                const bool sib = ps == par && s2 != t;
                const bool before = ss < my || (ss == my && s2 < t);
                off += (sib && before) ? ss : 0;
                later += (sib && !before) ? 1 : 0;
            }
            if (t < n) {
                s_off[t] = off;
                s_later[t] = later;
            }
        } else if (t < n) {
            const int my = s_size[t];
            int off = 0, later = 0;
#pragma unroll 8
            for (int s2 = 0; s2 < n; ++s2) {
                const int ps = s_par[s2], ss = s_size[s2];
                const bool sib = ps == par && s2 != t;
                const bool before = ss < my || (ss == my && s2 < t);
                off += (sib && before) ? ss : 0;
                later += (sib && !before) ? 1 : 0;
            }
            s_off[t] = off;
            s_later[t] = later;
        }
        __syncthreads();
        int pos = 0, act = 0;
        if (t < n) {
            // preorder position: every ancestor's offset plus one per non-root node on the path
            pos = depth - 1;
#pragma unroll
            for (int j = 0; j < GDN_MAX_DEPTH; ++j)
                if (j < depth) pos += s_off[anc[j]];
            if (par == -1) act = GDN_ACT_INIT;
            else if (s_off[t] == 0) act = GDN_ACT_CONTINUE;  // first child: follows its parent
            else if (s_later[t] == 0) act = GDN_ACT_POP;     // last child
            else act = GDN_ACT_TOP;
            if (s_nchild[t] >= 2) act |= GDN_ACT_PUSH;
            if (s_nchild[t] == 0) act |= GDN_ACT_LEAF;
            W.order[lo + pos] = t;
            W.action[lo + pos] = act;
            W.depth[lo + t] = depth;
            int32_t *np = W.nodepath + (size_t)(lo + t) * GDN_MAX_DEPTH;  // root first
#pragma unroll
            for (int j = 0; j < GDN_MAX_DEPTH; ++j)
                if (j < depth) np[depth - 1 - j] = anc[j];
#pragma unroll
            for (int s2 = 0; s2 < GDN_MAX_DEPTH; ++s2)
                if (s2 >= depth) np[s2] = -1;
        }
    } else if (in_bounds) {
        // rejected (or empty) sequence: defined metadata
        for (int i = t; i < hi - lo; i += kPlanThreads) {
            W.order[lo + i] = -1;
            W.action[lo + i] = 0;
            W.depth[lo + i] = 0;
            for (int s = 0; s < GDN_MAX_DEPTH; ++s) W.nodepath[(size_t)(lo + i) * GDN_MAX_DEPTH + s] = -1;
        }
    }
    if (t == 0) {
        W.seq_status[b] = status;
        W.seq_info[b * kSeqInfoInts + 0] = in_bounds ? lo : 0;
        W.seq_info[b * kSeqInfoInts + 1] = in_bounds ? hi - lo : 0;
        W.seq_info[b * kSeqInfoInts + 2] = status;
        W.seq_info[b * kSeqInfoInts + 3] = (status == GDN_SEQ_OK && n > 0) ? my_slot : 0;
        for (int r = 4; r < kSeqInfoInts; ++r) W.seq_info[b * kSeqInfoInts + r] = 0;
        W.path_len[b] = 0;
    }
    if (t < GDN_MAX_DEPTH) W.path[b * GDN_MAX_DEPTH + t] = -1;
}

}  // namespace

hipError_t launch_plan(const Params &p, hipStream_t s) {
    const int grid = p.B > 0 ? p.B : 1;
    if (p.max_nodes <= 64)
        hipLaunchKernelGGL(plan_kernel<64>, dim3(grid), dim3(64), 0, s, p);
    else
        hipLaunchKernelGGL(plan_kernel<GDN_MAX_NODES>, dim3(grid), dim3(GDN_MAX_NODES), 0, s, p);
    return hipGetLastError();
}

}  // namespace gdn

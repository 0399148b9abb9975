// gdn_internal.h -- workspace layout, kernel parameter block and small device
// helpers shared by the kernels and the C-ABI layer of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn_tree.h"

namespace gdn {

constexpr int32_t kMagic = 0x67646e74;       // written by the plan into the workspace header
constexpr int32_t kChainMagic = 0x67646e63;  // written by gdn_chain_verify instead: no plan in it
constexpr int kHeaderInts = 16;  // magic, B, T, max_nodes, max_depth, stack slots, misuse flag, ...
constexpr int kHdrMisuse = 6;    // set when a persist or accept found the plan made for other dims
constexpr int kSeqInfoInts = 8;          // node offset, node count, verdict, slot, reserved x4

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kCoefFloats = 20;         // per (node, value head): 16 path weights, gamma, alpha, b, depth
constexpr int kAcceptChunks = 8;        // most slices one logits row is split into for the argmax
constexpr int kMaxDraftWidth = GDN_MAX_DRAFT_WIDTH;  // candidates per drafted position

// Byte offsets of the workspace regions (each 256-byte aligned).  The
// per-(node, head) coefficient records come last, so the other offsets do
// not depend on the head count.
struct WsLayout {
    size_t header, seq_status, seq_info, depth, order, action, nodepath, path, path_len, amax, coef, total;
};

__host__ __device__ inline WsLayout ws_layout(int B, int T, int Hv = 0) {
    const size_t b = B > 0 ? (size_t)B : 1, t = T > 0 ? (size_t)T : 1;
    WsLayout L;
    size_t off = 0;
    L.header = off;     off += align256(kHeaderInts * 4);
    L.seq_status = off; off += align256(b * 4);
    L.seq_info = off;   off += align256(b * kSeqInfoInts * 4);
    L.depth = off;      off += align256(t * 4);
    L.order = off;      off += align256(t * 4);
    L.action = off;     off += align256(t * 4);
    L.nodepath = off;   off += align256(t * GDN_MAX_DEPTH * 4);
    L.path = off;       off += align256(b * GDN_MAX_DEPTH * 4);
    L.path_len = off;   off += align256(b * 4);
    L.amax = off;       off += align256(t * kAcceptChunks * 8);
    L.coef = off;       off += align256(t * (size_t)(Hv > 0 ? Hv : 0) * kCoefFloats * 4);
    L.total = off;
    return L;
}

struct WsPtrs {
    int32_t *header, *seq_status, *seq_info, *depth, *order, *action, *nodepath, *path, *path_len;
    int2 *amax;  // per (node, row slice): largest logit (bits) and its index
    float *coef;
};

inline WsPtrs ws_ptrs(void *ws, int B, int T, int Hv = 0) {
    const WsLayout L = ws_layout(B, T, Hv);
    char *base = static_cast<char *>(ws);
    WsPtrs p;
    p.header = reinterpret_cast<int32_t *>(base + L.header);
    p.seq_status = reinterpret_cast<int32_t *>(base + L.seq_status);
    p.seq_info = reinterpret_cast<int32_t *>(base + L.seq_info);
    p.depth = reinterpret_cast<int32_t *>(base + L.depth);
    p.order = reinterpret_cast<int32_t *>(base + L.order);
    p.action = reinterpret_cast<int32_t *>(base + L.action);
    p.nodepath = reinterpret_cast<int32_t *>(base + L.nodepath);
    p.path = reinterpret_cast<int32_t *>(base + L.path);
    p.path_len = reinterpret_cast<int32_t *>(base + L.path_len);
    p.amax = reinterpret_cast<int2 *>(base + L.amax);
    p.coef = reinterpret_cast<float *>(base + L.coef);
    return p;
}

// Everything a kernel needs; passed by value.
struct Params {
    int B, T, max_nodes, max_depth, Hk, Hv, D, num_slots;
    int stack_slots;             // LDS stack entries of the recurrent tree kernel
    int f32_in;                  // q/k/v are fp32 (else bf16 bits)
    const int32_t *parent;       // plan
    const int32_t *cu_nodes;     // plan, chain
    const int32_t *slot_idx;
    const void *q, *k, *v;       // bf16 bits (uint16) or fp32
    const float *a, *b;
    const float *state_in;       // committed states (verify, chain, persist)
    float *state_out;            // persist: same slots, written in place
    float *out;                  // [T][Hv][D]
    const int32_t *accepted;     // persist
    const int32_t *final_len;    // chain
    float *final_state;          // chain
    WsPtrs ws;
    int has_ws;
    // greedy acceptance
    const float *logits;         // [T][vocab]
    const int32_t *draft_token;  // [T]
    int32_t *accepted_out, *accept_len_out, *next_token_out, *target_out;
    int vocab, chunks, chunk_len;
    // per-node states stored in fp16 (verify-and-store / persist-by-copy)
    uint16_t *node_states;       // [T][Hv][D][D] fp16 bits
};

// The plan in the workspace was made for exactly these dims: the header's magic,
// B, T, max_nodes and max_depth match.  A workspace last written by a chain call
// (kChainMagic) holds no tree metadata and fails; so does a plan for a larger
// max_nodes, whose trees could overflow tables sized from these dims.  Two
// vector loads, no short-circuit, so the test does not hold back loads issued
// next to it.
__device__ __forceinline__ bool ws_plan_matches(const Params &P) {
    const int4 h = *reinterpret_cast<const int4 *>(P.ws.header);
    const int4 e = *reinterpret_cast<const int4 *>(P.ws.header + 4);
    return (h.x == kMagic) & (h.y == P.B) & (h.z == P.T) & (h.w == P.max_nodes) & (e.x == P.max_depth);
}

// ---- kernel launchers (defined in the .hip files) --------------------------
hipError_t launch_plan(const Params &p, hipStream_t s);
hipError_t launch_tree_verify_recurrent(const Params &p, int dtype, hipStream_t s);
hipError_t launch_chain_verify_recurrent(const Params &p, int dtype, hipStream_t s);
hipError_t launch_persist_recurrent(const Params &p, int dtype, hipStream_t s);
// the per-node-state design: recurrent verify that also stores every node's
// state in fp16, and a persist that copies the accepted node's stored state
hipError_t launch_tree_verify_store(const Params &p, int dtype, hipStream_t s);
hipError_t launch_persist_copy(const Params &p, hipStream_t s);
// MFMA path (D in {64, 128}, bf16 or fp32 q/k/v)
bool fast_path_supported(int D, int dtype);
bool fast_tree_supported(int D, int dtype, int max_nodes, int heads_per_key);
hipError_t launch_tree_verify_fast(const Params &p, hipStream_t s);
hipError_t launch_chain_verify_fast(const Params &p, hipStream_t s);
hipError_t launch_persist_fast(const Params &p, hipStream_t s);
bool fused_supported(int D, int dtype, int max_nodes);
hipError_t launch_persist_verify_fast(const Params &prev, const Params &next, hipStream_t s);
// greedy acceptance over the verify logits
hipError_t launch_accept(const Params &p, hipStream_t s);
// draft candidates and the DDTree builder
int ddtree_nodes(int levels, int width, int budget, int max_depth);
hipError_t launch_draft_topk(int rows, int vocab, int width, const float *logits, int32_t *tokens, float *logp,
                             hipStream_t s);
hipError_t launch_ddtree_build(int B, int levels, int width, int budget, int max_depth, const int32_t *root_token,
                               const int32_t *tokens, const float *logp, int32_t *parent, int32_t *node_token,
                               int32_t *cu_nodes, hipStream_t s);
// streaming diagnostic: mode 0 reads `bytes` (one partial sum per wave into dst),
// mode 1 copies them
size_t probe_partials_bytes(size_t bytes);
hipError_t launch_probe(int mode, const void *src, void *dst, size_t bytes, hipStream_t s);
// the static scratch of gdn_tree_verify_static: its size, and this GPU's device
// address of it (looked up on the first call on each device)
size_t static_scratch_bytes();
hipError_t static_scratch(void **out);
// prefix-cache snapshots
hipError_t launch_state_copy(const float *src, int src_total, const int32_t *src_slot, float *dst, int dst_total,
                             const int32_t *dst_slot, int count, size_t slot_floats, hipStream_t s);

// Largest LDS stack the heavy-last preorder can need for trees of n nodes:
// k nested pushes need a subtree of at least 2^(k+1) - 1 nodes.
inline int stack_bound(int max_nodes, int max_depth) {
    int k = 0;
    while ((1 << (k + 2)) - 1 <= max_nodes) ++k;
    return k < max_depth - 1 ? k : (max_depth > 1 ? max_depth - 1 : 0);
}

}  // namespace gdn

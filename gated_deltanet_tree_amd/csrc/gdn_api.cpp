// gdn_api.cpp -- the C ABI: host-side argument checks, workspace sizing and
// kernel launches.  Nothing here allocates device memory or synchronizes,
// except gdn_tree_status.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gdn_internal.h"

using gdn::Params;

namespace {

bool dims_ok(const gdn_dims *d, int max_nodes_limit) {
    if (!d) return false;
    if (d->num_seqs < 0 || d->total_nodes < 0) return false;
    if (d->max_nodes < 0 || d->max_nodes > max_nodes_limit) return false;
    if (d->max_depth < 1 || d->max_depth > GDN_MAX_DEPTH) return false;
    if (d->num_k_heads < 1 || d->num_v_heads < 1 || d->num_v_heads % d->num_k_heads != 0) return false;
    if (d->num_seqs > 0 && d->num_slots < 1) return false;
    if (d->num_slots < 0) return false;
    // index arithmetic inside the kernels stays in 64 bits, but per-launch grid sizes are int
    if ((long long)d->num_seqs * d->num_v_heads * 16 > INT_MAX) return false;
    return true;
}

int check_dims(const gdn_dims *d, int max_nodes_limit) {
    if (!d) return GDN_ERR_NULL;
    if (!dims_ok(d, max_nodes_limit)) return GDN_ERR_SHAPE;
    if (d->head_dim != 16 && d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128)
        return GDN_ERR_UNSUPPORTED;
    if (d->qkv_dtype != GDN_BF16 && d->qkv_dtype != GDN_F32) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

Params base_params(const gdn_dims *d) {
    Params p;
    std::memset(&p, 0, sizeof(p));
    p.B = d->num_seqs;
    p.T = d->total_nodes;
    p.max_nodes = d->max_nodes;
    p.max_depth = d->max_depth;
    p.Hk = d->num_k_heads;
    p.Hv = d->num_v_heads;
    p.D = d->head_dim;
    p.num_slots = d->num_slots;
    p.stack_slots = gdn::stack_bound(d->max_nodes, d->max_depth);
    p.f32_in = d->qkv_dtype == GDN_F32;
    return p;
}

int launched(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

// GDN_KERNEL_PATH=recurrent selects the per-node recurrent kernels for every call
bool recurrent_forced() {
    const char *v = std::getenv("GDN_KERNEL_PATH");
    return v && std::strcmp(v, "recurrent") == 0;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

size_t gdn_workspace_bytes(const gdn_dims *dims) {
    if (!dims || !dims_ok(dims, GDN_MAX_CHAIN)) return 0;
    return gdn::ws_layout(dims->num_seqs, dims->total_nodes, dims->num_v_heads).total;
}

int gdn_tree_plan(const gdn_dims *dims, const int32_t *parent, const int32_t *cu_nodes,
                  const int32_t *slot_idx, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_dims(dims, GDN_MAX_NODES);
    if (rc) return rc;
    if (!ws || !cu_nodes) return GDN_ERR_NULL;
    if (dims->num_seqs > 0 && !slot_idx) return GDN_ERR_NULL;
    if (dims->total_nodes > 0 && !parent) return GDN_ERR_NULL;
    if (ws_bytes < gdn_workspace_bytes(dims)) return GDN_ERR_WORKSPACE;
    Params p = base_params(dims);
    p.parent = parent;
    p.cu_nodes = cu_nodes;
    p.slot_idx = slot_idx;
    p.ws = gdn::ws_ptrs(ws, p.B, p.T, p.Hv);
    p.has_ws = 1;
    return launched(gdn::launch_plan(p, as_stream(stream)));
}

int gdn_tree_verify(const gdn_dims *dims, const void *q, const void *k, const void *v,
                    const float *a, const float *b, const float *state_cache,
                    const int32_t *slot_idx, float *out, const void *ws, size_t ws_bytes,
                    void *stream) {
    int rc = check_dims(dims, GDN_MAX_NODES);
    if (rc) return rc;
    if (!ws) return GDN_ERR_NULL;
    if (dims->total_nodes > 0 && (!q || !k || !v || !a || !b || !out)) return GDN_ERR_NULL;
    if (dims->num_seqs > 0 && (!state_cache || !slot_idx)) return GDN_ERR_NULL;
    if (ws_bytes < gdn_workspace_bytes(dims)) return GDN_ERR_WORKSPACE;
    if (dims->num_seqs == 0 || dims->total_nodes == 0) return GDN_OK;
    Params p = base_params(dims);
    p.q = q;
    p.k = k;
    p.v = v;
    p.a = a;
    p.b = b;
    p.state_in = state_cache;
    p.slot_idx = slot_idx;
    p.out = out;
    p.ws = gdn::ws_ptrs(const_cast<void *>(ws), p.B, p.T, p.Hv);
    p.has_ws = 1;
    // the MFMA verify covers every tree size a call takes, unless the coefficient
    // tables of a very wide key-head group would not fit the LDS
    if (!recurrent_forced() && gdn::fast_tree_supported(p.D, dims->qkv_dtype, dims->max_nodes, p.Hv / p.Hk))
        return launched(gdn::launch_tree_verify_fast(p, as_stream(stream)));
    return launched(gdn::launch_tree_verify_recurrent(p, dims->qkv_dtype, as_stream(stream)));
}

int gdn_tree_verify_static(const gdn_dims *dims, const int32_t *parent, const int32_t *cu_nodes,
                           const int32_t *slot_idx, const void *q, const void *k, const void *v, const float *a,
                           const float *b, const float *state_cache, float *out, int32_t *seq_status,
                           void *stream) {
    int rc = check_dims(dims, GDN_MAX_NODES);
    if (rc) return rc;
    if (!cu_nodes) return GDN_ERR_NULL;
    if (dims->total_nodes > 0 && (!parent || !q || !k || !v || !a || !b || !out)) return GDN_ERR_NULL;
    if (dims->num_seqs > 0 && (!state_cache || !slot_idx)) return GDN_ERR_NULL;
    // the plan's metadata must fit the library's static scratch
    if (gdn_workspace_bytes(dims) > gdn::static_scratch_bytes()) return GDN_ERR_WORKSPACE;
    if (dims->num_seqs == 0) return GDN_OK;
    void *ws = nullptr;
    if (gdn::static_scratch(&ws) != hipSuccess) return GDN_ERR_LAUNCH;
    Params p = base_params(dims);
    p.parent = parent;
    p.cu_nodes = cu_nodes;
    p.slot_idx = slot_idx;
    p.ws = gdn::ws_ptrs(ws, p.B, p.T, p.Hv);
    if (seq_status) p.ws.seq_status = seq_status;  // the verdicts go to the caller
    p.has_ws = 1;
    hipStream_t s = as_stream(stream);
    if (gdn::launch_plan(p, s) != hipSuccess) return GDN_ERR_LAUNCH;
    if (dims->total_nodes == 0) return GDN_OK;
    p.q = q;
    p.k = k;
    p.v = v;
    p.a = a;
    p.b = b;
    p.state_in = state_cache;
    p.out = out;
    if (!recurrent_forced() && gdn::fast_tree_supported(p.D, dims->qkv_dtype, dims->max_nodes, p.Hv / p.Hk))
        return launched(gdn::launch_tree_verify_fast(p, s));
    return launched(gdn::launch_tree_verify_recurrent(p, dims->qkv_dtype, s));
}

int gdn_tree_persist(const gdn_dims *dims, const void *k, const void *v, const float *a,
                     const float *b, const int32_t *accepted_node, float *state_cache,
                     const int32_t *slot_idx, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_dims(dims, GDN_MAX_NODES);
    if (rc) return rc;
    if (!ws) return GDN_ERR_NULL;
    if (dims->total_nodes > 0 && (!k || !v || !a || !b)) return GDN_ERR_NULL;
    if (dims->num_seqs > 0 && (!state_cache || !slot_idx || !accepted_node)) return GDN_ERR_NULL;
    if (ws_bytes < gdn_workspace_bytes(dims)) return GDN_ERR_WORKSPACE;
    if (dims->num_seqs == 0 || dims->total_nodes == 0) return GDN_OK;
    Params p = base_params(dims);
    p.k = k;
    p.v = v;
    p.a = a;
    p.b = b;
    p.accepted = accepted_node;
    p.state_in = state_cache;
    p.state_out = state_cache;
    p.slot_idx = slot_idx;
    p.ws = gdn::ws_ptrs(ws, p.B, p.T, p.Hv);
    p.has_ws = 1;
    if (!recurrent_forced() && gdn::fast_path_supported(p.D, dims->qkv_dtype))
        return launched(gdn::launch_persist_fast(p, as_stream(stream)));
    return launched(gdn::launch_persist_recurrent(p, dims->qkv_dtype, as_stream(stream)));
}

int gdn_tree_persist_verify(const gdn_dims *prev_dims, const void *prev_k, const void *prev_v,
                            const float *prev_a, const float *prev_b, const int32_t *accepted_node,
                            void *prev_ws, size_t prev_ws_bytes, const gdn_dims *dims, const void *q,
                            const void *k, const void *v, const float *a, const float *b,
                            float *state_cache, const int32_t *slot_idx, float *out, void *ws,
                            size_t ws_bytes, void *stream) {
    int rc = check_dims(prev_dims, GDN_MAX_NODES);
    if (rc) return rc;
    rc = check_dims(dims, GDN_MAX_NODES);
    if (rc) return rc;
    if (prev_dims->num_seqs != dims->num_seqs || prev_dims->num_k_heads != dims->num_k_heads ||
        prev_dims->num_v_heads != dims->num_v_heads || prev_dims->head_dim != dims->head_dim ||
        prev_dims->num_slots != dims->num_slots || prev_dims->qkv_dtype != dims->qkv_dtype)
        return GDN_ERR_SHAPE;
    if (!prev_ws || !ws) return GDN_ERR_NULL;
    if (prev_dims->total_nodes > 0 && (!prev_k || !prev_v || !prev_a || !prev_b)) return GDN_ERR_NULL;
    if (dims->total_nodes > 0 && (!q || !k || !v || !a || !b || !out)) return GDN_ERR_NULL;
    if (dims->num_seqs > 0 && (!state_cache || !slot_idx || !accepted_node)) return GDN_ERR_NULL;
    if (prev_ws_bytes < gdn_workspace_bytes(prev_dims) || ws_bytes < gdn_workspace_bytes(dims))
        return GDN_ERR_WORKSPACE;
    // Step t's plan and path records and step t+1's plan live side by side:
    // one workspace for both would let one step's tables overwrite the other's.
    const uintptr_t wp = reinterpret_cast<uintptr_t>(prev_ws), wn = reinterpret_cast<uintptr_t>(ws);
    if (wp < wn + gdn_workspace_bytes(dims) && wn < wp + gdn_workspace_bytes(prev_dims)) return GDN_ERR_WORKSPACE;
    if (dims->num_seqs == 0) return GDN_OK;
    const bool fused = !recurrent_forced() && dims->total_nodes > 0 && prev_dims->total_nodes > 0 &&
                       gdn::fused_supported(dims->head_dim, dims->qkv_dtype, dims->max_nodes);
    if (!fused) {
        rc = gdn_tree_persist(prev_dims, prev_k, prev_v, prev_a, prev_b, accepted_node, state_cache, slot_idx,
                              prev_ws, prev_ws_bytes, stream);
        if (rc) return rc;
        return gdn_tree_verify(dims, q, k, v, a, b, state_cache, slot_idx, out, ws, ws_bytes, stream);
    }
    Params pp = base_params(prev_dims);
    pp.k = prev_k;
    pp.v = prev_v;
    pp.a = prev_a;
    pp.b = prev_b;
    pp.accepted = accepted_node;
    pp.state_in = state_cache;
    pp.state_out = state_cache;
    pp.slot_idx = slot_idx;
    pp.ws = gdn::ws_ptrs(prev_ws, pp.B, pp.T, pp.Hv);
    pp.has_ws = 1;
    Params pn = base_params(dims);
    pn.q = q;
    pn.k = k;
    pn.v = v;
    pn.a = a;
    pn.b = b;
    pn.state_in = state_cache;
    pn.state_out = state_cache;
    pn.slot_idx = slot_idx;
    pn.out = out;
    pn.ws = gdn::ws_ptrs(ws, pn.B, pn.T, pn.Hv);
    pn.has_ws = 1;
    return launched(gdn::launch_persist_verify_fast(pp, pn, as_stream(stream)));
}

int gdn_tree_verify_store(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *a,
                          const float *b, const float *state_cache, const int32_t *slot_idx, float *out,
                          uint16_t *node_states, const void *ws, size_t ws_bytes, void *stream) {
    int rc = check_dims(dims, GDN_MAX_NODES);
    if (rc) return rc;
    if (!ws) return GDN_ERR_NULL;
    if (dims->total_nodes > 0 && (!q || !k || !v || !a || !b || !out || !node_states)) return GDN_ERR_NULL;
    if (dims->num_seqs > 0 && (!state_cache || !slot_idx)) return GDN_ERR_NULL;
    if (ws_bytes < gdn_workspace_bytes(dims)) return GDN_ERR_WORKSPACE;
    if (dims->num_seqs == 0 || dims->total_nodes == 0) return GDN_OK;
    Params p = base_params(dims);
    p.q = q;
    p.k = k;
    p.v = v;
    p.a = a;
    p.b = b;
    p.state_in = state_cache;
    p.slot_idx = slot_idx;
    p.out = out;
    p.node_states = node_states;
    p.ws = gdn::ws_ptrs(const_cast<void *>(ws), p.B, p.T, p.Hv);
    p.has_ws = 1;
    return launched(gdn::launch_tree_verify_store(p, dims->qkv_dtype, as_stream(stream)));
}

int gdn_tree_persist_copy(const gdn_dims *dims, const int32_t *accepted_node, const uint16_t *node_states,
                          float *state_cache, const int32_t *slot_idx, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_dims(dims, GDN_MAX_NODES);
    if (rc) return rc;
    if (!ws) return GDN_ERR_NULL;
    if (dims->num_seqs > 0 && (!accepted_node || !state_cache || !slot_idx)) return GDN_ERR_NULL;
    if (dims->total_nodes > 0 && !node_states) return GDN_ERR_NULL;
    if (ws_bytes < gdn_workspace_bytes(dims)) return GDN_ERR_WORKSPACE;
    if (dims->num_seqs == 0 || dims->total_nodes == 0) return GDN_OK;
    Params p = base_params(dims);
    p.accepted = accepted_node;
    p.node_states = const_cast<uint16_t *>(node_states);
    p.state_out = state_cache;
    p.slot_idx = slot_idx;
    p.ws = gdn::ws_ptrs(ws, p.B, p.T, p.Hv);
    p.has_ws = 1;
    return launched(gdn::launch_persist_copy(p, as_stream(stream)));
}

int gdn_chain_verify(const gdn_dims *dims, const int32_t *cu_nodes, const void *q, const void *k,
                     const void *v, const float *a, const float *b, const float *state_cache,
                     const int32_t *slot_idx, float *out, const int32_t *final_len,
                     float *final_state, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_dims(dims, GDN_MAX_CHAIN);
    if (rc) return rc;
    if (!cu_nodes) return GDN_ERR_NULL;
    if ((q == nullptr) != (out == nullptr)) return GDN_ERR_NULL;
    if ((final_len == nullptr) != (final_state == nullptr)) return GDN_ERR_NULL;
    if (dims->total_nodes > 0 && (!k || !v || !a || !b)) return GDN_ERR_NULL;
    if (dims->num_seqs > 0 && (!state_cache || !slot_idx)) return GDN_ERR_NULL;
    if (ws && ws_bytes < gdn_workspace_bytes(dims)) return GDN_ERR_WORKSPACE;
    const bool fast = !recurrent_forced() && gdn::fast_path_supported(dims->head_dim, dims->qkv_dtype);
    // chains of one drafting block keep per-node coefficients in the workspace
    if (fast && dims->max_nodes <= GDN_MAX_DEPTH && q && !ws) return GDN_ERR_NULL;
    if (dims->num_seqs == 0) return GDN_OK;
    Params p = base_params(dims);
    p.cu_nodes = cu_nodes;
    p.q = q;
    p.k = k;
    p.v = v;
    p.a = a;
    p.b = b;
    p.state_in = state_cache;
    p.slot_idx = slot_idx;
    p.out = out;
    p.final_len = final_len;
    p.final_state = final_state;
    if (ws) {
        p.ws = gdn::ws_ptrs(ws, p.B, p.T, p.Hv);
        p.has_ws = 1;
    }
    // chains that fit one drafting block share the tree kernels' arithmetic;
    // longer chains (e.g. prefill) run in chunks of one block on the matrix cores
    if (fast) return launched(gdn::launch_chain_verify_fast(p, as_stream(stream)));
    return launched(gdn::launch_chain_verify_recurrent(p, dims->qkv_dtype, as_stream(stream)));
}

int gdn_tree_accept(const gdn_dims *dims, const float *logits, int32_t vocab, const int32_t *draft_token,
                    int32_t *accepted_node, int32_t *accept_len, int32_t *next_token, int32_t *target_token,
                    void *ws, size_t ws_bytes, void *stream) {
    if (!dims) return GDN_ERR_NULL;
    if (!dims_ok(dims, GDN_MAX_NODES)) return GDN_ERR_SHAPE;
    if (vocab < 1) return GDN_ERR_SHAPE;
    if ((long long)dims->total_nodes * gdn::kAcceptChunks > INT_MAX) return GDN_ERR_SHAPE;
    if (!ws) return GDN_ERR_NULL;
    if (dims->total_nodes > 0 && (!logits || !draft_token)) return GDN_ERR_NULL;
    if (dims->num_seqs > 0 && (!accepted_node || !accept_len || !next_token)) return GDN_ERR_NULL;
    if (ws_bytes < gdn_workspace_bytes(dims)) return GDN_ERR_WORKSPACE;
    Params p = base_params(dims);
    p.logits = logits;
    p.vocab = vocab;
    p.draft_token = draft_token;
    p.accepted_out = accepted_node;
    p.accept_len_out = accept_len;
    p.next_token_out = next_token;
    p.target_out = target_token;
    // a row is cut into up to kAcceptChunks slices of >= 8192 entries (a multiple
    // of 4, so 16-byte loads stay inside their slice)
    p.chunks = std::min(gdn::kAcceptChunks, std::max(1, (vocab + 8191) / 8192));
    p.chunk_len = ((vocab + p.chunks - 1) / p.chunks + 3) & ~3;
    p.ws = gdn::ws_ptrs(ws, p.B, p.T, p.Hv);
    p.has_ws = 1;
    return launched(gdn::launch_accept(p, as_stream(stream)));
}

int gdn_draft_topk(int32_t rows, int32_t vocab, int32_t width, const float *logits, int32_t *tokens,
                   float *logp, void *stream) {
    if (rows < 0 || vocab < 1 || width < 1 || width > GDN_MAX_DRAFT_WIDTH) return GDN_ERR_SHAPE;
    if (rows == 0) return GDN_OK;
    if (!logits || !tokens || !logp) return GDN_ERR_NULL;
    return launched(gdn::launch_draft_topk(rows, vocab, width, logits, tokens, logp, as_stream(stream)));
}

int32_t gdn_ddtree_nodes(int32_t levels, int32_t width, int32_t budget, int32_t max_depth) {
    if (levels < 1 || width < 1 || width > GDN_MAX_DRAFT_WIDTH || budget < 0 || max_depth < 1 ||
        max_depth > GDN_MAX_DEPTH)
        return 0;
    return gdn::ddtree_nodes(levels, width, budget, max_depth);
}

int gdn_ddtree_build(int32_t num_seqs, int32_t levels, int32_t width, int32_t budget, int32_t max_depth,
                     const int32_t *root_token, const int32_t *tokens, const float *logp, int32_t *parent,
                     int32_t *node_token, int32_t *cu_nodes, void *stream) {
    const int32_t n = gdn_ddtree_nodes(levels, width, budget, max_depth);
    if (num_seqs < 0 || n < 1 || n > GDN_MAX_NODES) return GDN_ERR_SHAPE;
    if (!cu_nodes) return GDN_ERR_NULL;
    if (num_seqs > 0 && (!tokens || !logp || !parent || !node_token)) return GDN_ERR_NULL;
    if ((long long)num_seqs * n > INT_MAX) return GDN_ERR_SHAPE;
    return launched(gdn::launch_ddtree_build(num_seqs, levels, width, budget, max_depth, root_token, tokens, logp,
                                             parent, node_token, cu_nodes, as_stream(stream)));
}

int gdn_state_copy(int32_t num_v_heads, int32_t head_dim, const float *src_cache, int32_t src_slots_total,
                   const int32_t *src_slot, float *dst_cache, int32_t dst_slots_total, const int32_t *dst_slot,
                   int32_t count, void *stream) {
    if (num_v_heads < 1 || head_dim < 1 || (head_dim & 3) || count < 0 || count > 65535 || src_slots_total < 0 ||
        dst_slots_total < 0)
        return GDN_ERR_SHAPE;
    if (count == 0) return GDN_OK;
    if (!src_cache || !src_slot || !dst_cache || !dst_slot) return GDN_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(src_cache) % 16 || reinterpret_cast<uintptr_t>(dst_cache) % 16)
        return GDN_ERR_SHAPE;
    const size_t slot_floats = (size_t)num_v_heads * head_dim * head_dim;
    return launched(gdn::launch_state_copy(src_cache, src_slots_total, src_slot, dst_cache, dst_slots_total,
                                           dst_slot, count, slot_floats, as_stream(stream)));
}

int gdn_probe_stream(int32_t mode, const void *src, void *dst, size_t bytes, size_t dst_bytes, void *stream) {
    if (mode != 0 && mode != 1) return GDN_ERR_SHAPE;
    if (bytes == 0) return GDN_OK;
    if (!src || !dst) return GDN_ERR_NULL;
    if (bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
        return GDN_ERR_SHAPE;
    if (bytes / (64 * 1024) >= (size_t)INT_MAX) return GDN_ERR_SHAPE;
    if (dst_bytes < (mode == 0 ? gdn::probe_partials_bytes(bytes) : bytes)) return GDN_ERR_WORKSPACE;
    return launched(gdn::launch_probe(mode, src, dst, bytes, as_stream(stream)));
}

int gdn_tree_read_metadata(const gdn_dims *dims, const void *ws, size_t ws_bytes, int32_t *depth,
                           int32_t *order, int32_t *action, int32_t *path, int32_t *path_len,
                           int32_t *seq_status, void *stream) {
    int rc = check_dims(dims, GDN_MAX_NODES);
    if (rc) return rc;
    if (!ws) return GDN_ERR_NULL;
    if (ws_bytes < gdn_workspace_bytes(dims)) return GDN_ERR_WORKSPACE;
    const gdn::WsPtrs w = gdn::ws_ptrs(const_cast<void *>(ws), dims->num_seqs, dims->total_nodes);
    const size_t T = (size_t)dims->total_nodes, B = (size_t)dims->num_seqs;
    hipStream_t s = as_stream(stream);
    struct Copy {
        void *dst;
        const void *src;
        size_t bytes;
    } copies[] = {
        {depth, w.depth, T * 4},       {order, w.order, T * 4},
        {action, w.action, T * 4},     {path, w.path, B * GDN_MAX_DEPTH * 4},
        {path_len, w.path_len, B * 4}, {seq_status, w.seq_status, B * 4},
    };
    for (const Copy &c : copies) {
        if (!c.dst || c.bytes == 0) continue;
        if (hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return GDN_ERR_LAUNCH;
    }
    return GDN_OK;
}

int gdn_tree_status(const void *ws, size_t ws_bytes, void *stream, int32_t *first_bad_seq,
                    int32_t *first_bad_code) {
    if (first_bad_seq) *first_bad_seq = -1;
    if (first_bad_code) *first_bad_code = 0;
    if (!ws) return GDN_ERR_NULL;
    if (ws_bytes < gdn::ws_layout(0, 0).total) return GDN_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    if (hipStreamSynchronize(s) != hipSuccess) return GDN_ERR_DEVICE;
    int32_t header[gdn::kHeaderInts];
    if (hipMemcpy(header, ws, sizeof(header), hipMemcpyDeviceToHost) != hipSuccess) return GDN_ERR_DEVICE;
    if ((header[0] != gdn::kMagic && header[0] != gdn::kChainMagic) || header[1] < 0 || header[2] < 0)
        return GDN_ERR_WORKSPACE;
    // a persist or accept call that found the plan made for other dims wrote nothing else
    if (header[gdn::kHdrMisuse] != 0) return GDN_ERR_WORKSPACE;
    const int B = header[1], T = header[2];
    if (ws_bytes < gdn::ws_layout(B, T).total) return GDN_ERR_WORKSPACE;
    if (B == 0) return GDN_OK;
    std::vector<int32_t> st(B);
    const gdn::WsPtrs w = gdn::ws_ptrs(const_cast<void *>(ws), B, T);
    if (hipMemcpy(st.data(), w.seq_status, (size_t)B * 4, hipMemcpyDeviceToHost) != hipSuccess)
        return GDN_ERR_DEVICE;
    for (int i = 0; i < B; ++i) {
        if (st[i] != GDN_SEQ_OK) {
            if (first_bad_seq) *first_bad_seq = i;
            if (first_bad_code) *first_bad_code = st[i];
            return GDN_ERR_TREE;
        }
    }
    return GDN_OK;
}

const char *gdn_strerror(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "dims out of range or inconsistent";
        case GDN_ERR_UNSUPPORTED: return "head dim or dtype not supported";
        case GDN_ERR_WORKSPACE: return "workspace too small or not planned for these dims";
        case GDN_ERR_LAUNCH: return "kernel launch failed";
        case GDN_ERR_TREE: return "a sequence was rejected (bad tree, slot or accepted node)";
        case GDN_ERR_DEVICE: return "HIP error while synchronizing";
        default: return "unknown gdn status";
    }
}

}  // extern "C"

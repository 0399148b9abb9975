/*
 * gdn_tree.h -- C ABI of the Gated DeltaNet tree-verify / persist library
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  A Gated DeltaNet layer keeps, per sequence and
 * value head, a recurrent state S of D_v x D_k fp32 values next to the KV
 * cache (GreenGames page, "Why the experiment exists": the SSM state cache of
 * the 48 Gated DeltaNet layers of a 64-layer hybrid).  One token with key k,
 * value v, decay a and write strength b updates it by the gated delta rule
 *
 *         S' = a * S * (I - b k k^T) + b * v k^T ,       o = S' q .
 *
 * (The pages name the kernel -- ggml_gated_delta_net, GreenGames "TL;DR" --
 * but do not print the rule; this is the reading the library implements.)
 *
 * Speculative decoding with DDTree (magik.net page, "The Broader Context";
 * GreenGames, "From autoregressive to DDTree") verifies a whole tree of draft
 * tokens in one target forward: every node's state is the rule applied to its
 * parent's state, the committed state for a root, so each node sees exactly
 * the tokens on its root-to-node path.  gdn_tree_verify produces o for every
 * node without touching the committed state.  After acceptance,
 * gdn_tree_persist replays the accepted root-to-node path and writes its
 * final state in place into the state cache (GreenGames, "Key wins": the
 * persist-write kernel that replaced a per-step state copy).
 *
 * Conventions shared by every entry point
 *  - Every pointer except `dims` (and the host outputs of gdn_tree_status) is
 *    a DEVICE pointer to contiguous memory in the layouts below.  The caller
 *    owns all memory, including the workspace; the library allocates nothing
 *    and keeps no mutable global state (apart from a per-device count of how
 *    many verify workgroups fit the device at once, a fixed property of the
 *    part), so calls with distinct workspaces are independent.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns without synchronizing, except
 *    gdn_tree_status, which synchronizes `stream`.
 *  - Errors the host can see (bad dims, NULL pointers, small workspace)
 *    return a negative gdn_status BEFORE anything is enqueued.  Errors only
 *    the device can see (malformed tree, bad slot, bad accepted node) mark the
 *    sequence in the workspace; such a sequence is skipped: its verify
 *    outputs are NaN and its cache slot is not written.  gdn_tree_status
 *    reports them.
 *  - Stream order per decode step: gdn_tree_plan once, then gdn_tree_verify
 *    for each layer, then (after acceptance) gdn_tree_persist for each layer.
 *    k, v, a and b of the step must stay alive until persist has run.
 *  - Kernel choice is automatic: bf16 or fp32 inputs with head_dim 64 or 128
 *    run the matrix-core kernels (every tree size a call takes, unless the value
 *    heads of one key head are so many that the coefficient tables of a tree
 *    over 96 nodes would not fit one compute unit's LDS), everything else the
 *    per-node recurrent kernels.  Setting the environment variable
 *    GDN_KERNEL_PATH=recurrent makes every call use the recurrent kernels
 *    (read on each call); both agree to within the stated tolerance.  The
 *    matrix-core verify gives one workgroup all value heads of a key head,
 *    or, when a batch is small enough that one workgroup per value head all
 *    fit the device at once, one value head each; GDN_VERIFY_HEADS=shared or
 *    =split fixes that choice (read on each call; the results are identical
 *    bit for bit).
 *
 * Layouts (row-major, T = total nodes, B = sequences):
 *   parent       int32 [T]        local node id of the parent inside its own
 *                                  sequence, -1 for a root (a forest is allowed)
 *   cu_nodes     int32 [B+1]      sequence b owns nodes [cu_nodes[b], cu_nodes[b+1])
 *   slot_idx     int32 [B]        state-cache slot of sequence b
 *   q, k         [T][H_k][D_k]    bf16 or fp32 (dims.qkv_dtype)
 *   v            [T][H_v][D_v]    bf16 or fp32
 *   a, b         fp32 [T][H_v]    decay and write strength, already activated
 *   state_cache  fp32 [num_slots][H_v][D_v][D_k]   (row = value index)
 *   out          fp32 [T][H_v][D_v]
 *   Value head h reads key head h / (H_v / H_k).
 */
#ifndef GDN_TREE_H
#define GDN_TREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Longest root-to-node path, in nodes: the 16-token drafting block
   (GreenGames, "Prefill"). */
#define GDN_MAX_DEPTH 16
/* Largest tree (nodes per sequence) one verify call accepts. */
#define GDN_MAX_NODES 256
/* Longest chain gdn_chain_verify accepts (it has no depth limit). */
#define GDN_MAX_CHAIN 65536
/* Most draft candidates kept per drafted position (gdn_draft_topk, gdn_ddtree_build). */
#define GDN_MAX_DRAFT_WIDTH 16

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = -2,       /* dims out of range or inconsistent */
    GDN_ERR_UNSUPPORTED = -3, /* head dim / dtype without a kernel */
    GDN_ERR_WORKSPACE = -4,   /* workspace too small, or not planned for these dims */
    GDN_ERR_LAUNCH = -5,      /* the HIP runtime refused a launch */
    GDN_ERR_TREE = -6,        /* (gdn_tree_status) at least one sequence was skipped */
    GDN_ERR_DEVICE = -7       /* (gdn_tree_status) a HIP error while synchronizing */
} gdn_status;

typedef enum gdn_dtype { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* Per-sequence verdicts written into the workspace (first failing check wins). */
typedef enum gdn_seq_status {
    GDN_SEQ_OK = 0,
    GDN_SEQ_BAD_NODES = 1,      /* [cu[b], cu[b+1]) not inside [0, T], or longer than max_nodes */
    GDN_SEQ_BAD_SLOT = 2,       /* slot_idx[b] outside [0, num_slots) (non-empty sequences only) */
    GDN_SEQ_DUP_SLOT = 3,       /* slot shared by two non-empty sequences (both flagged) */
    GDN_SEQ_BAD_PARENT = 4,     /* parent outside {-1} U [0, n) or a node's own id */
    GDN_SEQ_CYCLE_OR_DEPTH = 5, /* an ancestor walk does not reach a root within max_depth nodes */
    GDN_SEQ_BAD_ACCEPT = 6,     /* accepted_node outside {-1} U [0, n) (set by persist) */
    GDN_SEQ_NOT_PERSISTED = 7   /* (gdn_tree_persist_verify, in the previous step's workspace) the
                                   slot the accepted path would be written to is read by another
                                   sequence's verify in the same call; the slot was not written */
} gdn_seq_status;

/* Traversal action word (one per visited position, see gdn_tree_plan). */
enum {
    GDN_ACT_CONTINUE = 0, /* parent state = the state just produced */
    GDN_ACT_TOP = 1,      /* parent state = copy of the stack top */
    GDN_ACT_POP = 2,      /* parent state = stack top, popped */
    GDN_ACT_INIT = 3,     /* parent state = committed state (a root) */
    GDN_ACT_PUSH = 4,     /* push this node's state (it has >= 2 children) */
    GDN_ACT_LEAF = 8      /* no children: its state is never needed again */
};

typedef struct gdn_dims {
    int32_t num_seqs;    /* B >= 0 */
    int32_t total_nodes; /* T >= 0; must equal cu_nodes[B] */
    int32_t max_nodes;   /* upper bound on nodes per sequence, <= GDN_MAX_NODES (trees) */
    int32_t max_depth;   /* depth limit in nodes, 1 .. GDN_MAX_DEPTH */
    int32_t num_k_heads; /* H_k >= 1 */
    int32_t num_v_heads; /* H_v, a multiple of H_k */
    int32_t head_dim;    /* D = D_k = D_v, one of 16, 32, 64, 128 */
    int32_t num_slots;   /* slots in state_cache, >= 1 when B > 0 */
    int32_t qkv_dtype;   /* gdn_dtype of q, k, v */
} gdn_dims;

/* Bytes of workspace gdn_tree_plan/verify/persist/accept need for these dims
   (0 if the dims are invalid).  The caller allocates it (device memory, no
   initialization needed); one workspace serves one decode step. */
size_t gdn_workspace_bytes(const gdn_dims *dims);

/*
 * gdn_tree_plan -- validate the draft trees and build traversal metadata on
 * the device (one workgroup per sequence).  The trees are the parent-pointer
 * trees DDTree's builder grows from the drafter's candidates (GreenGames page,
 * "From autoregressive to DDTree": the budgeted tree of build_ddtree, seeded
 * with a chain), at most one drafting block deep (GreenGames, "Prefill": 16
 * tokens).  Per node: depth (root = 1) and the
 * root-to-node path.  Per sequence: a depth-first preorder in which the
 * children of a node (and the roots of a forest) are visited by increasing
 * (subtree size, node id), so the largest child comes last and is entered
 * without saving the parent's state; the per-position action words tell the
 * recurrent verify how to obtain each node's parent state.  Also writes each
 * sequence's verdict.  Reads parent, cu_nodes, slot_idx; writes only `ws`.
 */
int gdn_tree_plan(const gdn_dims *dims, const int32_t *parent, const int32_t *cu_nodes,
                  const int32_t *slot_idx, void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_tree_verify -- for every node n of every valid sequence and every value
 * head, o_n = S^n q_n where S^n is the gated delta rule applied along n's
 * root-to-node path starting from state_cache[slot_idx[b]].  state_cache is
 * only read.  Sequences the plan rejected get NaN outputs.  `ws` must come
 * from gdn_tree_plan with the same dims on the same stream; a workspace planned
 * for other dims (B, T, max_nodes or max_depth differ), or last written by
 * gdn_chain_verify, makes the call write nothing at all.
 */
int gdn_tree_verify(const gdn_dims *dims, const void *q, const void *k, const void *v,
                    const float *a, const float *b, const float *state_cache,
                    const int32_t *slot_idx, float *out, const void *ws, size_t ws_bytes,
                    void *stream);

/*
 * gdn_tree_verify_static -- gdn_tree_plan followed by gdn_tree_verify in one
 * call with no caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The plan's metadata goes to a scratch array of
 * 32 MiB in device memory that the library holds per GPU until the process
 * ends; dims whose gdn_workspace_bytes exceed it return GDN_ERR_WORKSPACE
 * before anything is enqueued.  The call allocates nothing (the first call on
 * each device looks up that device's scratch address; make it outside graph
 * capture).  Arguments are those of the two calls it replaces; the outputs are
 * the same bits gdn_tree_verify writes after gdn_tree_plan.  seq_status
 * (device int32 [B], may be NULL) receives the per-sequence verdicts that
 * gdn_tree_status would report.  Every call on one GPU uses that GPU's single
 * scratch array: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialized by the caller.  The scratch is not readable
 * through gdn_tree_status, gdn_tree_read_metadata or gdn_tree_persist; a
 * decode step that persists plans into a workspace of its own.
 */
int gdn_tree_verify_static(const gdn_dims *dims, const int32_t *parent, const int32_t *cu_nodes,
                           const int32_t *slot_idx, const void *q, const void *k, const void *v, const float *a,
                           const float *b, const float *state_cache, float *out, int32_t *seq_status,
                           void *stream);

/*
 * gdn_tree_persist -- for each sequence b with accepted_node[b] = m >= 0,
 * replay the rule over the root-to-m path from state_cache[slot_idx[b]] and
 * write the result in place into that slot.  accepted_node[b] = -1 skips the
 * sequence.  Only the slots of valid, accepted sequences are written.  Also
 * records the accepted path (root first) and its length in the workspace.  On a
 * workspace planned for other dims (or last written by gdn_chain_verify) no
 * slot is written and the workspace is marked so that gdn_tree_status returns
 * GDN_ERR_WORKSPACE.
 */
int gdn_tree_persist(const gdn_dims *dims, const void *k, const void *v, const float *a,
                     const float *b, const int32_t *accepted_node, float *state_cache,
                     const int32_t *slot_idx, void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_tree_persist_verify -- gdn_tree_persist of one decode step followed by
 * gdn_tree_verify of the next, on one layer, in one pass over the state.  A
 * layer's state is read by its verify and read and written by its persist
 * (GreenGames page, "Key wins": the persist-write kernel writes the accepted
 * node's state in place after acceptance; magik.net page, "The Broader
 * Context": the tree of the next step is verified from that committed state).
 * Deferring step t's persist until the layer's verify of step t+1 lets each
 * (sequence, value head) load its state once, replay the accepted path of
 * step t in registers, write the result in place and take step t+1's outputs
 * from the same registers: two state passes per layer call instead of three.
 *
 * prev_dims, prev_k/v/a/b, accepted_node and prev_ws are exactly the
 * arguments gdn_tree_persist would take for step t (prev_ws from
 * gdn_tree_plan of step t; it receives the accepted path and the per-sequence
 * verdicts of the persist).  dims, q/k/v/a/b, slot_idx, out and ws are those of
 * gdn_tree_verify for step t+1 (ws from gdn_tree_plan of step t+1 with
 * slot_idx); state_cache is the one cache both steps address, written in
 * place.  The two dims must agree in num_seqs, heads, head_dim, num_slots and
 * qkv_dtype (GDN_ERR_SHAPE otherwise); total_nodes, max_nodes and max_depth
 * may differ.  prev_ws and ws are two workspaces: their first
 * gdn_workspace_bytes(prev_dims) and gdn_workspace_bytes(dims) bytes must not
 * overlap (GDN_ERR_WORKSPACE otherwise).  Sequence b of one step is sequence b
 * of the other; its slot in each step is the one that step's plan recorded.
 *
 * Results: out equals what gdn_tree_verify writes after gdn_tree_persist, to
 * within the verify's rounding (the products sum the state's columns in
 * another order), and every persisted slot holds the same bits gdn_tree_persist
 * writes.  One exception keeps the call free of races: a sequence whose
 * accepted path would be written to a slot that another sequence of step t+1
 * verifies from is not persisted and is marked GDN_SEQ_NOT_PERSISTED in
 * prev_ws (gdn_tree_status on prev_ws reports it); the caller may persist it
 * with gdn_tree_persist and accepted_node = -1 for every other sequence.  A
 * sequence whose step t+1 tree is rejected gets NaN outputs, as in verify.
 * Either workspace planned for other dims makes the call write nothing and
 * marks that workspace, as persist does.  Bf16 inputs with head_dim 64 or 128
 * and step t+1 trees of at most 32 nodes run the fused kernel; every other
 * shape runs gdn_tree_persist then gdn_tree_verify on `stream` (which never
 * marks GDN_SEQ_NOT_PERSISTED: it persists before any verify reads).
 */
int gdn_tree_persist_verify(const gdn_dims *prev_dims, const void *prev_k, const void *prev_v,
                            const float *prev_a, const float *prev_b, const int32_t *accepted_node,
                            void *prev_ws, size_t prev_ws_bytes, const gdn_dims *dims, const void *q,
                            const void *k, const void *v, const float *a, const float *b,
                            float *state_cache, const int32_t *slot_idx, float *out, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * gdn_tree_verify_store and gdn_tree_persist_copy -- the pages' own tree path,
 * kept for comparison (GreenGames page, "Key wins": verify writes every node's
 * state to an f16 intermediate cache and the commit copies the accepted one;
 * "half the bandwidth" of fp32 states, about 1.5 MiB per node per layer at
 * 48 value heads of 128 x 128).  gdn_tree_verify_store computes the same
 * outputs as gdn_tree_verify with the per-node recurrent kernel (any head dim
 * and dtype) and also writes each node's post-update state, rounded to fp16
 * (nearest, ties to even), into node_states (fp16 bits, [T][H_v][D_v][D_k]).
 * gdn_tree_persist_copy then writes, for each sequence b with
 * accepted_node[b] = m >= 0, the stored state of node m widened to fp32 into
 * state_cache[slot_idx[b]] (-1 skips; an out-of-range m marks the sequence
 * GDN_SEQ_BAD_ACCEPT).  The fp16 rounding makes the persisted state differ
 * from gdn_tree_persist's fp32 replay (relative error up to 2^-11 per value),
 * so the chain bit-identity of the replay path does not hold here.  Both
 * calls need `ws` from gdn_tree_plan with the same dims (otherwise neither
 * writes anything, and after persist_copy gdn_tree_status returns
 * GDN_ERR_WORKSPACE); persist_copy does not record the path.
 */
int gdn_tree_verify_store(const gdn_dims *dims, const void *q, const void *k, const void *v, const float *a,
                          const float *b, const float *state_cache, const int32_t *slot_idx, float *out,
                          uint16_t *node_states, const void *ws, size_t ws_bytes, void *stream);
int gdn_tree_persist_copy(const gdn_dims *dims, const int32_t *accepted_node, const uint16_t *node_states,
                          float *state_cache, const int32_t *slot_idx, void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_chain_verify -- the W = 1 case, linear DFlash verification of one
 * drafted block (dflash-caddtree-integrations README, "What's in here": a tree
 * of width 1 must reproduce the chain path byte for byte; GreenGames page,
 * "From autoregressive to DDTree": chain DFlash, the baseline DDTree is
 * measured against).  A chain-shaped tree given to gdn_tree_verify and
 * gdn_tree_persist gives the same bits as this call.  Sequence b is the linear chain of nodes
 * [cu_nodes[b], cu_nodes[b+1]) (no parent array, no plan, no depth limit;
 * lengths up to dims.max_nodes <= GDN_MAX_CHAIN).  Writes o for every node
 * (q and out may both be NULL to skip outputs) and, when final_len and
 * final_state are given, the state after the first final_len[b] nodes into
 * final_state [B][H_v][D_v][D_k] (final_len[b] = 0 writes the committed state;
 * a value outside [0, n_b] writes nothing).  state_cache is only read and
 * final_state must not overlap it.  `ws` (sized by gdn_workspace_bytes for
 * the same dims) receives the per-sequence verdicts for gdn_tree_status; it
 * is required when outputs are requested for inputs with head_dim 64 or 128
 * and chains of at most GDN_MAX_DEPTH nodes (the kernels keep per-node
 * coefficients there), and may be NULL otherwise.  Longer chains at head_dim
 * 64 or 128 run in chunks of GDN_MAX_DEPTH tokens on the matrix cores, the
 * state kept in registers from chunk to chunk.  The call marks the
 * workspace as a chain workspace: gdn_tree_status reads its verdicts, and the
 * tree calls reject it until gdn_tree_plan runs on it again.
 */
int gdn_chain_verify(const gdn_dims *dims, const int32_t *cu_nodes, const void *q, const void *k,
                     const void *v, const float *a, const float *b, const float *state_cache,
                     const int32_t *slot_idx, float *out, const int32_t *final_len,
                     float *final_state, void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_tree_accept -- greedy (temperature-0) acceptance of each planned tree
 * against the target's verify logits.  Row n of `logits` (fp32 [T][vocab],
 * one row per node, the verify logits buffer of the GreenGames page, "Key
 * wins") is the target's prediction for the token after node n; the target's
 * token there is the first index of the row's largest entry, a NaN counting
 * as largest (numpy argmax order; +0 equals -0).  From the sequence's root
 * (the smallest-id root of a forest) the walk moves to the smallest-id child
 * c with draft_token[c] equal to the target's token after the current node,
 * until no child qualifies.  Outputs per sequence: accepted_node[b] (local id
 * of the stop node; feed it to gdn_tree_persist), accept_len[b] (its depth,
 * root = 1) and next_token[b] (the target's token after it).  A sequence the
 * plan rejected, or an empty one, gets -1, 0, -1.  target_token (int32 [T],
 * may be NULL) receives every row's argmax.  Draft tokens outside [0, vocab)
 * never match; the roots' draft tokens are not read.  Verification at
 * temperature 0 must reproduce plain greedy decoding token for token
 * (dflash-caddtree-integrations README, "The shared method"; greedy-only
 * verify, GreenGames "What comes next").  `ws` comes from gdn_tree_plan with
 * the same dims on the same stream; the call reuses a per-node region of it.
 * On a workspace planned for other dims every sequence gets -1, 0, -1 and
 * gdn_tree_status returns GDN_ERR_WORKSPACE.
 * logits may be any 4-byte-aligned address; 16-byte alignment and vocab % 4
 * == 0 take the vector loads.
 */
int gdn_tree_accept(const gdn_dims *dims, const float *logits, int32_t vocab, const int32_t *draft_token,
                    int32_t *accepted_node, int32_t *accept_len, int32_t *next_token, int32_t *target_token,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_draft_topk -- the drafter's candidates per drafted position: for each of
 * `rows` rows of fp32 logits [rows][vocab], the `width` (1 .. 16) best entries
 * in argmax order (a NaN counts as largest, equal values keep the smaller id,
 * +0 equals -0) into tokens [rows][width], and their log-softmax values
 * x - log(sum(exp(row))) into logp [rows][width] (fp32; all NaN when the row
 * holds a NaN or +inf, all -inf when every entry is -inf; ranks past the
 * vocabulary get token -1 and log p -inf).  The descending order is the one
 * DDTree's builder expects: rank 1 first (GreenGames page, "Key wins": a
 * reversed order sent the worst candidate to the tree root).  One workgroup
 * per row; logits may be any 4-byte-aligned address.  No workspace.
 */
int gdn_draft_topk(int32_t rows, int32_t vocab, int32_t width, const float *logits, int32_t *tokens,
                   float *logp, void *stream);

/*
 * gdn_ddtree_nodes -- nodes of every tree gdn_ddtree_build grows: 1 + min(budget,
 * all nodes a depth of min(levels + 1, max_depth) and `width` children per node
 * allow); 0 for arguments out of range.
 */
int32_t gdn_ddtree_nodes(int32_t levels, int32_t width, int32_t budget, int32_t max_depth);

/*
 * gdn_ddtree_build -- grow one draft tree per sequence (GreenGames page, "From
 * autoregressive to DDTree": budgeted best-first trees with a chain pre-seed).
 * tokens/logp [B][levels][width] hold each drafted position's candidates in
 * rank order (as gdn_draft_topk writes them); position l (1-based) is tree
 * level l, the children of a depth-l node (root depth 1).  Node 0 is the root
 * carrying root_token[b] (NULL: -1).  Nodes 1 .. min(budget, levels,
 * max_depth - 1) form the rank-1 chain; then, until budget drafts exist, the
 * next node is the best candidate among every node's next unused rank r <
 * width at the node's level (child depth <= min(levels + 1, max_depth)): the
 * higher path score (the fp32 sum of log p along the path, parent's score
 * plus the candidate's log p; NaN log p counts as -inf), then the smaller
 * depth, the smaller rank, the smaller parent id.  Node ids are insertion
 * order, so parent ids precede their children.  Outputs (N =
 * gdn_ddtree_nodes(...), at most GDN_MAX_NODES): parent [B*N] (local ids, -1
 * for the root), node_token [B*N] and cu_nodes [B+1] = b*N -- the inputs of
 * gdn_tree_plan and the draft tokens of gdn_tree_accept.  log p values are
 * log-probabilities (<= 0) or -inf.  One wave per sequence.
 */
int gdn_ddtree_build(int32_t num_seqs, int32_t levels, int32_t width, int32_t budget, int32_t max_depth,
                     const int32_t *root_token, const int32_t *tokens, const float *logp, int32_t *parent,
                     int32_t *node_token, int32_t *cu_nodes, void *stream);

/*
 * gdn_state_copy -- prefix-cache snapshots (dflash-caddtree-integrations
 * README, "What's in here": gdn_apc, automatic prefix caching under
 * speculative decoding, warm start bitwise equal to a cold one).  For each
 * entry i < count: dst_cache[dst_slot[i]] = src_cache[src_slot[i]], a whole
 * slot of num_v_heads x head_dim x head_dim fp32 values, copied exactly.  Save
 * a sequence's committed state into a prefix pool, or restore it from the pool
 * into a new sequence's slot.  src_slots_total / dst_slots_total are the slot
 * counts of the two caches; an entry with a slot outside its cache is skipped.
 * The destination slots must be distinct, and when both caches are the same
 * memory no destination slot may be another entry's source (such calls race).
 * Slot arrays are device int32 [count]; caches are 16-byte aligned.
 */
int gdn_state_copy(int32_t num_v_heads, int32_t head_dim, const float *src_cache, int32_t src_slots_total,
                   const int32_t *src_slot, float *dst_cache, int32_t dst_slots_total, const int32_t *dst_slot,
                   int32_t count, void *stream);

/*
 * gdn_tree_read_metadata -- device-to-device copies of what the plan (and the
 * last persist) stored: depth [T], order [T] (node ids by visit position,
 * offset by cu_nodes), action [T], path [B][GDN_MAX_DEPTH] (root first,
 * padded with -1), path_len [B], seq_status [B].  Any output may be NULL.
 */
int gdn_tree_read_metadata(const gdn_dims *dims, const void *ws, size_t ws_bytes, int32_t *depth,
                           int32_t *order, int32_t *action, int32_t *path, int32_t *path_len,
                           int32_t *seq_status, void *stream);

/*
 * gdn_tree_status -- synchronizes `stream`, then reads the verdicts in `ws`.
 * Returns GDN_OK, GDN_ERR_TREE (some sequence was skipped; *first_bad_seq and
 * *first_bad_code name the lowest such sequence and its gdn_seq_status),
 * GDN_ERR_WORKSPACE (ws was never planned, or a persist or accept call found
 * it planned for other dims) or GDN_ERR_DEVICE.  Workspaces written by
 * gdn_chain_verify are read the same way.  The two outputs are HOST pointers
 * and may be NULL.
 */
int gdn_tree_status(const void *ws, size_t ws_bytes, void *stream, int32_t *first_bad_seq,
                    int32_t *first_bad_code);

/*
 * gdn_probe_stream -- diagnostic, not part of a decode step: the plain
 * streaming rates of the device, the practical ceilings the state streams of
 * verify and persist are measured against.  mode 0 reads `bytes` of src and
 * writes one partial sum per 64 lanes of each 64 KiB block into dst (dst_bytes
 * >= 16 * ceil(bytes / 65536)); mode 1 copies `bytes` from src to dst
 * (dst_bytes >= bytes).  bytes and both addresses are multiples of 16.
 */
int gdn_probe_stream(int32_t mode, const void *src, void *dst, size_t bytes, size_t dst_bytes, void *stream);

/* Static string for a gdn_status value. */
const char *gdn_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* GDN_TREE_H */

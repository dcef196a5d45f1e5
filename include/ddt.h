/*
 * ddt.h -- C ABI of the dynamic draft-tree library for MI355X (gfx950).
 *
 * One speculative-decoding round over a batch of requests: expand a draft
 * tree layer by layer from draft logits, rerank its nodes, flatten the chosen
 * subtree into a token list with an ancestor-only attention mask, and run the
 * accept walk against target logits; optionally with CAST's cost-aware width,
 * depth and verify-count rules, or with Graft's checkpoint gate, retrieval
 * graft and successor-matrix refresh.
 *
 * Sources of the operations (the three public pages the method is defined on):
 *   [E2]   "EAGLE-2 完全拆解：动态草稿树如何让投机解码上下文感知"
 *          (pinghaoyang.com.cn): confidence as an acceptance proxy, path value,
 *          expansion, reranking, flattening/mask, accept rule, decode-step flow.
 *   [CAST] "Inference-Cost-Aware Dynamic Tree Construction for Efficient
 *          Inference in Large Language Models" notes (papernotes.org, ICLR
 *          2026): key designs 1-4 (cost table, width, depth, verify count).
 *   [GR]   "Draft Less, Retrieve More: Hybrid Tree Construction for
 *          Speculative Decoding" review (paper.rainbus.top): execution-flow
 *          paragraph, steps (1) pruning, (2) retrieval graft, (3) hybrid verify
 *          and online update.
 *
 * Conventions for every call:
 *   - Ownership: the caller allocates every buffer; all pointers are device
 *     pointers unless marked "host".  The library never allocates or frees
 *     memory and keeps no pointer between calls.
 *   - Execution: a call only enqueues kernels on `stream` (a hipStream_t, NULL
 *     = the default stream) and returns; results are valid once the stream is
 *     synchronised.  No call synchronises the stream.
 *   - Errors: every call returns DDT_OK (0) or a DDT_E* code.  Arguments are
 *     checked on the host before anything is launched; on an error nothing is
 *     enqueued.  DDT_ELAUNCH reports a failed kernel launch.  There is no
 *     device-side error channel.
 *   - Determinism: identical inputs give bitwise-identical outputs.
 *   - Logits are float32 (DDT_F32) or bfloat16 (DDT_BF16), must be finite,
 *     and are addressed through element strides.
 *   - Ties: vocabulary top-k by (logit desc, token id asc); tree orderings by
 *     (path value desc, canonical key asc); argmax takes the lowest id.
 */
#ifndef DDT_H
#define DDT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DDT_OK 0
#define DDT_EINVAL 1      /* null pointer or inconsistent size/stride */
#define DDT_EDTYPE 2      /* unknown logit dtype */
#define DDT_ECAPACITY 3   /* a size exceeds a documented limit */
#define DDT_EWORKSPACE 4  /* workspace too small */
#define DDT_ELAUNCH 5     /* a kernel launch failed */

/* logit dtypes */
#define DDT_F32 0
#define DDT_BF16 1

/* T > 0 proposal of draft children in ddt_tree_verify */
#define DDT_PROPOSAL_DRAFT 0  /* q = softmax(draft/T): children drawn i.i.d. from the draft */
#define DDT_PROPOSAL_POINT 1  /* q = delta_x: children chosen deterministically (top-k trees) */

/* documented limits */
#define DDT_MAX_K 32        /* children per node, vocab top-k, refresh k */
#define DDT_MAX_DEPTH 11    /* draft layers (canonical key holds 11 rank fields) */
#define DDT_MAX_FRONT 32    /* frontier width */
#define DDT_MAX_NODES 4096  /* nodes per row (draft + retrieval, root included) */
#define DDT_MAX_VERIFY 255  /* draft nodes sent to verification per row */
#define DDT_MAX_CHUNKS 64   /* vocab chunks per row: V <= 64*8192 (bf16), 64*4096 (f32) */
#define DDT_WALK_STRIDE 2176 /* doubles per request in walk_buf: 2 x 32 x 2 pass sums + 2048 tile sums */

/*
 * Canonical node key (uint64): bits 62..59 depth, bit 58 source (0 draft,
 * 1 retrieval), then one 5-bit rank per depth level from bit 57 down
 * (level d at bits 57-5(d-1) .. 53-5(d-1)).  Ascending key order is
 * breadth-first, draft before retrieval at equal depth, then lexicographic in
 * the rank path; it is the flat order of a flattened tree.
 */

/* ------------------------------------------------------------------------ */
/* Logit tensor descriptor                                                   */
/* ------------------------------------------------------------------------ */
typedef struct ddt_logits {
    const void* data;    /* device; element (i0, i1, v) at data + i0*s0 + i1*s1 + v */
    int dtype;           /* DDT_F32 or DDT_BF16 */
    int V;               /* vocabulary size (elements per row, contiguous) */
    int64_t s0, s1;      /* strides in elements of the two outer indices */
} ddt_logits;

/* ------------------------------------------------------------------------ */
/* Tree state: caller-allocated device memory, carved by ddt_tree_bind        */
/* ------------------------------------------------------------------------ */
/*
 * Per batch row b, nodes are numbered: 0 = root; layer d's children follow in
 * (frontier slot j, rank r) order; retrieval nodes (Graft) after every draft
 * node, in template order.  S is the path value as a sum of log confidences,
 * V = exp(S) = product of confidences along the path ([E2] value formula;
 * [GR] step 1 S_{d,j} recursion).
 */
typedef struct ddt_tree {
    int32_t B, cap, D_max, R_max;
    int32_t* token;      /* [B][cap] token id (root: the last accepted token) */
    int32_t* parent;     /* [B][cap] parent node, -1 for the root */
    int32_t* depth;      /* [B][cap] 0 for the root */
    int32_t* eslot;      /* [B][cap] frontier slot the node was expanded with, -1 if never */
    uint64_t* key;       /* [B][cap] canonical key */
    float* S;            /* [B][cap] summed log confidence; -inf for retrieval nodes */
    float* logc;         /* [B][cap] log confidence of the node's own token */
    float* rmax;         /* [B][D_max][R_max] max of the draft row of (layer, slot) */
    float* rsp;          /* [B][D_max][R_max] sum_{v != argmax} exp(l_v - max) of that row */
    int32_t* n_nodes;    /* [B] */
    int32_t* layer_base; /* [B] first node of the most recent layer */
    int32_t* n_front;    /* [B] frontier width the next layer expands (0: row stopped) */
    int32_t* frontier;   /* [B][R_max] latest layer's nodes by (S desc, key asc) */
    float* front_S;      /* [B][R_max] S of those nodes */
    uint64_t* front_key; /* [B][R_max] canonical key of those nodes */
    int32_t* active;     /* [B] Graft: 1 until the row is pruned */
    int32_t* k_draft;    /* [B] Graft: draft nodes the row keeps (K_max if never pruned) */
    int32_t* cont;       /* [1] CAST: 1 while the batch keeps growing */
    int32_t* widths;     /* [D_max] CAST: width n_i chosen at layer i (0 for layers not built) */
    double* cast_state;  /* [16] CAST per-round state (gain FIFO, utility, context) */
    uint32_t* ticket;    /* [1] CAST: workgroups of a layer done so far (back to 0 after each layer) */
    double* walk_buf;    /* [B][DDT_WALK_STRIDE] T>0 verify: partial sums shared by a request's workgroups */
    uint32_t* walk_sync; /* [B][2] T>0 verify: arrival and exit counters (back to 0 after each call) */
    uint32_t* layer_sync; /* [B*R_max + B] expand: per-row and per-request arrival counters (back to 0) */
} ddt_tree;

/* Bytes of device memory a tree of these sizes needs (256-byte aligned base). */
size_t ddt_tree_bytes(int B, int cap, int D_max, int R_max);

/*
 * Fill *t with pointers into `base` (device, >= ddt_tree_bytes, 256-byte
 * aligned).  Host-only: touches no device memory.  The memory must be
 * zero-filled once before its first use (the layer counters of
 * ddt_tree_expand, the CAST layer counter and the T>0 walk counters start at
 * 0 and every call leaves them at 0); the tree itself is (re)initialised by
 * ddt_tree_expand with layer = 1.
 */
int ddt_tree_bind(ddt_tree* t /*host*/, void* base, size_t bytes, int B, int cap, int D_max,
                  int R_max);

/* ------------------------------------------------------------------------ */
/* Flattened tree: caller-allocated, carved by ddt_flat_bind                  */
/* ------------------------------------------------------------------------ */
/*
 * P = m_max + 1 positions per row (root at 0), W = ceil(P/32) mask words,
 * Dp = longest path length (depths 0..Dp).  Positions past a row's selection
 * are padding: node -1, token -1, parent -1, pos = prefix, self-only mask bit.
 */
typedef struct ddt_flat {
    int32_t B, P, W, Dp, L;
    int32_t* node;       /* [B][P] tree node at each flat position */
    int32_t* token;      /* [B][P] */
    int32_t* parent;     /* [B][P] flat index of the parent, -1 for root/padding */
    int32_t* pos;        /* [B][P] position id = prefix_len + depth ([GR] step 3) */
    uint32_t* mask;      /* [B][P][W] bit j of row i: position i may attend to tree position j */
    int32_t* retrieve;   /* [B][L][Dp+1] root-to-leaf flat indices per leaf, -1 padded; L = max(P-1,1) */
    int32_t* n_leaves;   /* [B] */
    int32_t* m;          /* [B] selected draft (+retrieval) nodes, root excluded */
} ddt_flat;

size_t ddt_flat_bytes(int B, int m_max, int Dp);
int ddt_flat_bind(ddt_flat* f /*host*/, void* base, size_t bytes, int B, int m_max, int Dp);

/* ------------------------------------------------------------------------ */
/* Mode parameters                                                           */
/* ------------------------------------------------------------------------ */

/*
 * CAST ([CAST] key designs 1-4).  Cost tables S_T (target) and S_D (draft) are
 * fp32 [M][N+1] device arrays, column n = time for n tokens (column 0 unused),
 * row r = context grid point (r+1)*L.  select(c) clamps to the last row (the
 * printed formula's max is read as min).  Width at layer i keeps n_i of the
 * layer's nodes by the anchor scan on the batch-averaged cumulative utility of
 * the sorted values e^S, cost c_k = S_D[sel(ctx)][k]/S_T[sel(ctx)][1] with ctx
 * = sum of earlier widths, threshold C1[i-1].  Depth: a FIFO of the last R
 * gain ratios (initially {1}); the batch grows another layer iff
 * mean(FIFO) * u_n / c_n >= C2.  Verify count per row: anchor scan over the
 * row's sorted node values with cost S_T[sel(ctx_verify)][k]/S_T[..][1] and
 * threshold C3[b].  "Anchor scan": keep 1; move the anchor a to k whenever
 * (u_k - u_a)/(c_k - c_a) >= C.  Batches of more than 64 rows are refused
 * (DDT_ECAPACITY).
 */
typedef struct ddt_cast {
    const float* S_T;    /* [M][N+1] */
    const float* S_D;    /* [M][N+1] */
    int L, M, N;         /* grid step; rows 1..64 (DDT_ECAPACITY above); columns */
    const float* C1;     /* [D_max] width threshold per layer (device) */
    float C2;            /* depth threshold */
    const float* C3;     /* [B] verify-count threshold per row (device) */
    int R;               /* FIFO length, 1..8 */
    int ctx_verify;      /* n0: context length for the verify cost lookup */
} ddt_cast;

/*
 * Graft checkpoint gate ([GR] step 1).  After building tree depth ck_depth[s],
 * c = exp(max S over that depth's nodes); the row is pruned (no deeper layers,
 * keeps k_draft[s] draft nodes) unless c > tau[s].  Rows never pruned keep
 * K_max draft nodes.
 */
typedef struct ddt_graft_gate {
    int n_ck;            /* 0..4 */
    int ck_depth[4];
    float tau[4];
    int k_draft[4];
    int K_max;
} ddt_graft_gate;

/* ------------------------------------------------------------------------ */
/* Workspace                                                                 */
/* ------------------------------------------------------------------------ */
/*
 * Scratch for the vocabulary-wide row reductions of ddt_tree_expand,
 * ddt_tree_verify, ddt_row_topk and ddt_succ_update: rows x ceil(V/chunk) x
 * (2 + 2K) x 4 bytes.  `rows` is the number of logit rows one call reduces:
 * B*R_max for expand, B*P for verify, the row count for ddt_row_topk.
 */
size_t ddt_workspace_bytes(int rows, int V, int dtype, int K);

/* ------------------------------------------------------------------------ */
/* The calls                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * ddt_tree_expand -- one draft layer ([E2] expansion section and decode-step
 * flow; [GR] step 1).
 *
 * layer = 1 resets every row: root token root_tok[b], V = 1 (S = 0), and
 * expands the root with row (b, 0) of `logits`.  layer = d >= 2 expands the
 * n_front[b] frontier nodes of layer d-1, frontier slot j with row (b, j).
 * Row (b, j) of `logits` is element (b, j, .) of the descriptor.
 *
 * For each expanded row: max, sigma' and the top-K_n tokens by (logit desc,
 * id asc); each becomes a child with log confidence (l - max) - log1p(sigma')
 * and S = S_parent + log confidence.  The new layer's nodes are then ordered
 * by (S desc, key asc); the next frontier is the first min(K_e, nodes) of
 * them (CAST: the first n_i), unless the row stops (Graft prune, CAST depth
 * gate, or layer = D_max where no frontier is formed).
 *
 * cast and gate are host pointers or NULL (not both).  With cast, the
 * widths/cont/n_front of the whole batch are updated within the call.
 * One kernel per call: the chunks of every row are reduced in parallel, and
 * the last chunk of a row, then the last row of a request, then (CAST) the
 * last request carry on with the merge, the children and frontier, and the
 * batch rule, counting themselves in on t->layer_sync and t->ticket.
 * Rows reduced per call: B*1 for layer 1, B*R_max after; ws must hold
 * ddt_workspace_bytes(B*R_max, V, dtype, K_n).
 */
int ddt_tree_expand(const ddt_tree* t /*host*/, int layer, const int32_t* root_tok /*[B]*/,
                    const ddt_logits* logits /*host*/, int K_n, int K_e,
                    const ddt_cast* cast /*host or NULL*/, const ddt_graft_gate* gate /*host or NULL*/,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * ddt_tree_rerank -- global top-m over every non-root node by (S desc, key
 * asc), i.e. shallower first on equal value ([E2] reranking section).  Because
 * a child never outranks its parent the selection is parent-closed.
 *
 * m per row: min(m_max, nodes) by default; with cast (host, may be NULL) the
 * CAST verify count; with use_k_draft the row's Graft k_draft.
 * sel: [B][m_max+1] node ids, root first then rerank order, -1 padded.
 * m_out: [B].
 */
int ddt_tree_rerank(const ddt_tree* t /*host*/, int m_max, const ddt_cast* cast, int use_k_draft,
                    int32_t* sel, int32_t* m_out, void* stream);

/*
 * ddt_succ_gather -- Graft retrieval graft ([GR] step 2).  For each row,
 * K_ret = K_max - m_out[b] nodes from the root-centred template: `width`
 * chains of length `depth`; chain c starts at M[b][root token][c] and
 * continues with successor 0 of its own last token (x_u = M[x_parent(u),
 * r_u]); level-major then chain order, first K_ret kept.  They are appended to
 * the tree (key source bit 1, S = -inf) and to sel after the draft nodes;
 * m_out becomes K_max.  M: int32 [B][V][k_succ] at M + b*M_bstride (M_bstride
 * = 0: one matrix shared by the batch).  sel has m_max + 1 entries per row
 * (m_max >= K_max, the value given to ddt_tree_rerank); tpl_width <= k_succ.
 */
int ddt_succ_gather(const ddt_tree* t /*host*/, const int32_t* M, int64_t M_bstride, int V,
                    int k_succ, int tpl_depth, int tpl_width, int K_max, int m_max, int32_t* sel,
                    int32_t* m_out, void* stream);

/*
 * ddt_succ_gather_at -- the same graft with the template hung off another
 * node, for the two grafts Graft's prune-then-graft is compared with ([GR]
 * technical-novelty point (2), Fig. 2): anchor DDT_GRAFT_ROOT is
 * ddt_succ_gather; DDT_GRAFT_TAIL hangs it off the tail of the row's selected
 * draft tree: the deepest node of sel[1 .. m_out[b]], ties to the higher S,
 * then the smaller canonical key (the root if nothing is selected).  Chain c
 * then starts at M[anchor token][c]; template node depths continue from the
 * anchor's, and levels that would pass DDT_MAX_DEPTH are not built (the flat
 * layout's Dp must cover the deepest node).  A fixed draft budget without
 * checkpoints (root-only and tail-only grafting) is a ddt_graft_gate with
 * n_ck = 0 and K_max = that budget, then this call with the full K_max.
 */
#define DDT_GRAFT_ROOT 0
#define DDT_GRAFT_TAIL 1
int ddt_succ_gather_at(const ddt_tree* t /*host*/, const int32_t* M, int64_t M_bstride, int V,
                       int k_succ, int tpl_depth, int tpl_width, int K_max, int m_max, int anchor,
                       int32_t* sel, int32_t* m_out, void* stream);

/*
 * ddt_tree_build_mask -- flatten {root} + selection in ascending canonical key
 * order; tokens, flat parents, position ids prefix_len + depth, ancestor-only
 * bitmask (self and ancestors visible, never siblings; prefix columns are
 * implicit), and one root-to-leaf path per leaf in flat order ([E2] reranking
 * section and engineering difficulty one; [GR] step 3).
 * sel/m as written by ddt_tree_rerank (+ ddt_succ_gather); m_max + 1 = f->P.
 * dense: optional uint8 [B][P][prefix_len + P] full mask (1 = visible), or NULL.
 */
int ddt_tree_build_mask(const ddt_tree* t /*host*/, const int32_t* sel, const int32_t* m,
                        int prefix_len, const ddt_flat* f /*host*/, uint8_t* dense,
                        void* stream);

/*
 * ddt_tree_select -- ddt_tree_rerank followed by ddt_tree_build_mask, for a
 * round with no Graft template between them, in one launch: the selection
 * goes from the rerank to the flattening in on-chip memory.  sel and m_out
 * are written as ddt_tree_rerank writes them, and f (and dense) as
 * ddt_tree_build_mask writes them from those; the results are the same as
 * calling the two in turn.  Arguments and errors are those of the two calls
 * ([E2] reranking section and engineering difficulty one; [CAST] key
 * design 4).
 */
int ddt_tree_select(const ddt_tree* t /*host*/, int m_max, const ddt_cast* cast, int use_k_draft,
                    int32_t* sel, int32_t* m_out, int prefix_len, const ddt_flat* f /*host*/,
                    uint8_t* dense, void* stream);

/*
 * ddt_tree_verify -- accept walk over the flattened tree ([E2] ledger and
 * losslessness sections, decode-step flow step 3).
 *
 * target: row (b, i) = target logits at flat position i (next-token logits
 * after that position's token), i = 0..f->m[b].
 * temperature[b] == 0: greedy -- the accept length is the longest prefix of a
 * root-to-leaf path whose every token equals the target argmax at its parent
 * (first path on ties); next_token = argmax at the last accepted position.
 * temperature[b] > 0: p = softmax(target/T); children are tried in flat
 * order, each accepted with probability min(1, p_k(x)/q(x)) under the
 * residual p_k left by the rejected siblings before it, with q the proposal
 * of that child (uniforms[b][c][0] < p_k(x_c)/q(x_c) accepts child c):
 *   proposal = DDT_PROPOSAL_POINT: q = delta_x for every child, the proposal
 *     of a deterministically chosen token such as the top-k children that
 *     ddt_tree_expand attaches.  Accepted iff uniforms < p_k(x); a rejection
 *     leaves norm(max(0, p_k - delta_x)) = p_k with x removed and
 *     renormalised.  Exactly lossless for any tree ([E2] losslessness
 *     section: the draft distribution only shapes which candidates are
 *     proposed).  The draft rows are not read (draft may be NULL).
 *   proposal = DDT_PROPOSAL_DRAFT: q = softmax(draft/T) of the row that
 *     expanded the node, and a rejection leaves norm(max(0, p_k - q)) (kept
 *     as it was if all zero).  The proposal of children drawn i.i.d. from the
 *     draft; on top-k children it is not exactly lossless.  Retrieval
 *     children (key source bit 1, and any child of a node without a draft
 *     row) still take point-mass proposals, after the draft children.
 * When no child is accepted, or at a leaf, next_token is the smallest v with
 * prefix sum of p_k > u * sum(p_k), u = uniforms[b][pos][1], tokens removed by
 * point-mass rejections excluded.
 * draft: the draft arena; the row that expanded a node of depth d - 1 from
 * frontier slot j of batch row b (i.e. layer d's slice) starts at
 * draft->data + (d-1)*draft_layer_stride + b*draft->s0 + j*draft->s1
 * elements.  Read only with DDT_PROPOSAL_DRAFT when some temperature > 0.
 * row_argmax: [B][P] or NULL.  k_top > 0 with row_topk [B][P][k_top]: top-k
 * ids of every verified row from the same pass (feeds ddt_succ_update).
 * Both hold -1 at padding positions (past f->m[b]).
 * accept_len [B]; accept_path [B][Dp+1] flat indices root first, -1 padded;
 * next_token [B].  ws >= ddt_workspace_bytes(B*P, V, dtype, max(1,k_top)).
 * A T > 0 request's vocabulary passes may be split over several workgroups
 * that exchange partial sums through t->walk_buf / t->walk_sync and wait for
 * each other with a bounded spin.  If a wait runs out (the workgroups were
 * not resident together), workgroup 0 finishes the walk alone over the whole
 * vocabulary: the outcome is the same, only slower.
 * Errors: DDT_EINVAL also for a proposal other than the two above.
 */
int ddt_tree_verify(const ddt_tree* t /*host*/, const ddt_flat* f /*host*/,
                    const ddt_logits* target /*host*/, const ddt_logits* draft /*host or NULL*/,
                    int64_t draft_layer_stride, const float* temperature /*[B]*/,
                    const float* uniforms /*[B][P][2]*/, int proposal, int k_top, int32_t* row_topk,
                    int32_t* row_argmax, int32_t* accept_len, int32_t* accept_path,
                    int32_t* next_token, void* ws, size_t ws_bytes, void* stream);

/*
 * ddt_succ_update -- Graft online refresh ([GR] step 3): for every verified
 * flat position i = 1..f->m[b] (accepted or not) with token x,
 * M[b][x][0..k_succ) <- the top-k_succ ids of target row i; when two positions
 * carry the same token the later one wins.  Ids come from row_topk
 * ([B][P][k_top], k_top >= k_succ, as written by ddt_tree_verify) or, if
 * row_topk is NULL, from a pass over `target` (ws as for ddt_tree_verify).
 */
int ddt_succ_update(int32_t* M, int64_t M_bstride, int V, int k_succ, const ddt_flat* f /*host*/,
                    const int32_t* row_topk, int k_top, const ddt_logits* target /*host or NULL*/,
                    void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Tree attention: the verify forward's attention over prefix and tree        */
/* ------------------------------------------------------------------------ */
/*
 * ddt_tree_attention -- scaled dot-product attention of every verified flat
 * position over the context prefix and its own ancestors, itself included;
 * siblings are never visible ([E2] reranking section and engineering
 * difficulty one; [GR] step (3): the hybrid tree is flattened with the same
 * mask before the one verify forward).  The tree positions visible to flat
 * position i are the set bits of f->mask row i (as ddt_tree_build_mask
 * writes it); every prefix position is visible.  Query head h reads
 * key/value head h / (Hq / Hkv).
 *
 * Tensors are bf16 and contiguous (element strides follow from the sizes):
 *   q               [B][P][Hq][D]    queries of the flat positions, P = f->P
 *   k_pre, v_pre    [B][L][Hkv][D]   the context's keys and values (may be NULL if L = 0)
 *   k_tree, v_tree  [B][P][Hkv][D]   keys and values of the flat positions
 * out: fp32 [B][P][Hq][D], device; positions past f->m[b] are written as 0.
 * The softmax uses scale * q.k; P (the attention weights) enters the value
 * product rounded to bf16, everything else accumulates in fp32.
 * Limits: D = 128; Hq a multiple of Hkv with Hq / Hkv <= 16.
 * Errors: DDT_EINVAL for null or inconsistent arguments (B or P differing from
 * f, scale not positive and finite), DDT_ECAPACITY for other D, larger groups,
 * or tensors past 2^31 elements.
 */
typedef struct ddt_attn {
    const void* q;
    const void* k_pre;
    const void* v_pre;
    const void* k_tree;
    const void* v_tree;
    int32_t B, P, Hq, Hkv, D, L;
    float scale;
} ddt_attn;

int ddt_tree_attention(const ddt_flat* f /*host*/, const ddt_attn* a /*host*/, float* out,
                       void* stream);

/*
 * ddt_tree_attention_split -- the same attention with each (request,
 * key/value head, tile of 128 query rows) split over `splits` contiguous
 * ranges of its 64-key blocks (prefix blocks first, then tree blocks), for
 * shapes whose tiles alone do not fill the GPU: few requests, few flat
 * positions, a long context.  Each split writes its rows' unnormalised
 * outputs and softmax statistics (running maximum, weight total) to ws; a
 * second kernel combines them, so out holds the same softmax up to fp32
 * rounding of the combination.  Same tensors, limits and errors as
 * ddt_tree_attention.
 *   splits  requested splits; 0 lets the library choose for the shape (one
 *           split once the tiles fill the device, otherwise as many as fit
 *           one resident round of 512 workgroups, with at least two key
 *           blocks each).  The count
 *           is capped at 32 and at the number of key blocks (ceil(L / 64) +
 *           ceil(P / 64)), and lowered so that every split but the last has
 *           the same number of blocks; ddt_tree_attention_splits returns the
 *           count used.  One split runs ddt_tree_attention.
 *   ws      device workspace of at least ddt_tree_attention_ws_bytes(...)
 *           bytes (256-byte aligned), owned by the caller, overwritten.
 * Errors additionally: DDT_EWORKSPACE if ws is NULL or too small while more
 * than one split is used.
 */
int ddt_tree_attention_split(const ddt_flat* f /*host*/, const ddt_attn* a /*host*/, float* out,
                             int splits, void* ws, size_t ws_bytes, void* stream);

/* The split count ddt_tree_attention_split uses for these sizes and request
 * (0 = the library's choice), and the workspace bytes it needs then (0 when
 * one split is used); both return 0 on invalid sizes. */
int ddt_tree_attention_splits(int B, int P, int Hq, int Hkv, int L, int splits);
size_t ddt_tree_attention_ws_bytes(int B, int P, int Hq, int Hkv, int L, int splits);

/* ------------------------------------------------------------------------ */
/* Paged KV cache: committing the accepted path, sharing, release            */
/* ------------------------------------------------------------------------ */
/*
 * Candidate KV is kept apart from the committed context; after the verify
 * the accepted tokens' KV is committed and the rejected candidates' KV is
 * dropped; with block-paged storage, block allocation, reference counts,
 * reclamation and copy-on-write are part of that step ([E2] engineering
 * difficulty two, and the decode-step flow: commit accepted tokens and their
 * KV, discard rejected candidate KV).
 *
 * Reading: the candidates' KV is the round's contiguous tree buffer
 * (k_tree, v_tree [B][P][Hkv][D], written by the verify forward and read by
 * ddt_tree_attention), so dropping a rejected candidate costs nothing.  The
 * committed context is a pool of fixed-size blocks:
 *   k, v        bf16 [n_blocks][block][Hkv][D]   token t of request b sits at
 *               slot t % block of block table[b][t / block]
 *   table       [B][max_blocks]  block ids of each request, -1 past its end
 *   len         [B]              tokens committed per request
 *   ref         [n_blocks]       number of tables holding each block
 *   free_ids    [n_blocks]       stack of free block ids: free_ids[0 .. *n_free)
 *   n_free      [1]
 *   plan        [B][4] int32     scratch written by ddt_kv_commit
 * All arrays are device memory owned by the caller; the library only reads
 * and writes them.  A consistent state has ref[x] = the number of table rows
 * holding x, and free_ids[0 .. n_free) = the blocks with ref 0, each once.
 * Calls on one cache must be ordered on one stream (they are not atomic with
 * respect to each other).
 */
typedef struct ddt_kv_cache {
    void* k;
    void* v;
    int32_t* table;
    int32_t* len;
    int32_t* ref;
    int32_t* free_ids;
    int32_t* n_free;
    int32_t* plan;
    int32_t B, max_blocks, n_blocks, block, Hkv, D;
} ddt_kv_cache;

/*
 * ddt_kv_commit -- append each request's accepted path to its context.
 * For request b with accept_len[b] = a >= 0, the n = a + 1 flat positions
 * accept_path[b][0 .. a] (root first, as ddt_tree_verify writes them) are
 * appended in path order: k_tree[b][accept_path[b][j]] becomes context token
 * len[b] + j, likewise for v.  Only the block holding token len[b] can be
 * partly filled; if it is and it is shared (ref > 1 when the call starts),
 * it is copied first (copy-on-write): a new block takes its committed slots
 * and replaces it in this table, and the old block loses one holder.  Every
 * other token goes to a new block.  need[b] = new blocks (+1 for a copy).
 * Requests are admitted in index order while the free stack lasts: b is
 * admitted iff need[0] + .. + need[b] (over requests that got this far) <=
 * *n_free, so a request that does not fit, and every later one, is left
 * unchanged.  Admitted requests take their blocks from the top of the stack
 * in index order, the copy first, then the new blocks in table order.  Old
 * blocks left with no holder are then pushed, ordered by the lowest index of
 * the requests that copied them.  The outcome is deterministic.
 * status[b]: n (tokens committed); 0 if accept_len[b] < 0 (nothing done);
 * -1 if the context would pass max_blocks * block tokens; -2 if the free
 * stack ran out; -3 if a path entry is outside [0, P).
 * k_tree, v_tree: bf16 [B][P][Hkv][D] (device), Dp = the path row length - 1.
 * Errors: DDT_EINVAL for null or inconsistent arguments ((Hkv*D) % 8 != 0
 * included); DDT_ECAPACITY for B > 1024, max_blocks > 4096 or Dp >
 * DDT_MAX_DEPTH.
 */
int ddt_kv_commit(const ddt_kv_cache* c /*host struct*/, const int32_t* accept_len /*[B]*/,
                  const int32_t* accept_path /*[B][Dp+1]*/, int Dp, const void* k_tree,
                  const void* v_tree, int P, int32_t* status /*[B]*/, void* stream);

/*
 * ddt_kv_fork -- request dst[i] takes the context of src[i] (for i < n):
 * it shares src's blocks (each gains a holder) and its length.  dst[i] must
 * hold no blocks (len 0, table row all -1) and differ from every src; pairs
 * that break this are skipped with status[i] = -1, otherwise status[i] = 0.
 * src, dst, status: device [n].  Pairs are applied in order.
 */
int ddt_kv_fork(const ddt_kv_cache* c /*host struct*/, const int32_t* src, const int32_t* dst, int n,
                int32_t* status, void* stream);

/*
 * ddt_kv_release -- drop the context of requests req[0 .. n) (device), in
 * order: every block of the request loses one holder, the blocks left with
 * none are pushed on the free stack in table order, and the request's table
 * row and length are cleared.  A request listed twice is released once.
 */
int ddt_kv_release(const ddt_kv_cache* c /*host struct*/, const int32_t* req, int n, void* stream);

/*
 * ddt_row_topk -- the vocabulary-wide row reduction on its own: for rows
 * (i0, i1) in [n0) x [n1), max, sigma' and the top-K ids with their log
 * confidences.  ids/logc: [n0*n1][K]; rmax/rsp: [n0*n1] (any may be NULL).
 * ws >= ddt_workspace_bytes(n0*n1, V, dtype, K).
 */
int ddt_row_topk(const ddt_logits* x /*host*/, int n0, int n1, int K, int32_t* ids, float* logc,
                 float* rmax, float* rsp, void* ws, size_t ws_bytes, void* stream);

/*
 * ddt_row_topk_noalloc -- ddt_row_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the chunk partials go to a fixed array of
 * DDT_NOALLOC_SCRATCH_BYTES inside the library, one per device, held until
 * the process ends, instead of a caller workspace.  Same arguments, outputs
 * and kernels as ddt_row_topk without ws.  The caller still owns x and the
 * outputs.  Nothing is allocated or freed; the array's device address is
 * looked up once per device, on the first call (DDT_ELAUNCH if that fails).
 * Errors as ddt_row_topk, and DDT_ECAPACITY when the partials would exceed
 * the array: ddt_workspace_bytes(n0*n1, V, dtype, K) > DDT_NOALLOC_SCRATCH_BYTES
 * (e.g. 1024 rows of 128256 bf16 logits fit up to K = 32).  All calls on one
 * device share the array: calls that overlap in time on a device (on
 * different streams, or from several threads) race and must be ordered by
 * the caller.
 */
#define DDT_NOALLOC_SCRATCH_BYTES (8u << 20)
int ddt_row_topk_noalloc(const ddt_logits* x /*host*/, int n0, int n1, int K, int32_t* ids,
                         float* logc, float* rmax, float* rsp, void* stream);

/*
 * ddt_set_reduce_events -- timing hook for the kernels that reduce vocabulary
 * rows: the layer kernel of ddt_tree_expand and the row reduction of
 * ddt_tree_verify, ddt_row_topk and ddt_succ_update.  While set, the i-th
 * launch of those (any call, any stream, in launch order), i <
 * n_pairs, is launched with events[2i] and events[2i+1] as its start and stop
 * events (hipExtLaunchKernelGGL: the runtime stamps them when the kernel
 * itself starts and ends); later launches are not timed.  events are
 * hipEvent_t handles created by the caller.
 * NULL / 0 clears the hook.  Returns the number of launches bracketed since
 * the previous call.  Process-wide host state; not thread-safe.
 */
int ddt_set_reduce_events(void* const* events, int n_pairs);

/*
 * ddt_set_walk_spin_limit -- test and diagnostic hook: the number of polls
 * after which a T > 0 walk's cross-workgroup wait in ddt_tree_verify gives up
 * (workgroup 0 then finishes that request alone; see ddt_tree_verify).  0
 * restores the default (2^22 polls).  Returns the previous value.
 * Process-wide host state read when a verify is enqueued; not thread-safe.
 */
unsigned ddt_set_walk_spin_limit(unsigned polls);

/* Text for a status code. */
const char* ddt_strerror(int status);

/* Chunk length (elements) of the row reduction for a dtype, for launches of
 * fewer than 256 rows (8192 bf16, 4096 fp32).  Launches of 256 rows or more
 * use chunks twice as long.  Returns -1 for an unknown dtype. */
int ddt_chunk_elems(int dtype);

#ifdef __cplusplus
}
#endif
#endif /* DDT_H */

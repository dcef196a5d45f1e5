"""CPU oracle for one dynamic draft-tree round.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the bench's CPU-baseline leg
may import or run this module.  The HIP product path never calls it, and the
two share no code: this file imports numpy and the standard library only.

It is a plain, slow, single-threaded restatement of what the three pages
describe, written in float64, following the pages' steps in their order:

  * EAGLE-2 explainer (pinghaoyang.com.cn, "EAGLE-2 完全拆解"): confidence as
    draft probability (section on why confidence approximates acceptance),
    path value as a product of confidences (value-formula section), the
    expansion loop with the incremental value update (expansion section), the
    global top-m rerank with shallow-first ties (reranking section), the
    flattening and ancestor-only mask (reranking section and the
    engineering-difficulties section), and the accept/reject rule with the
    residual distribution (ledger section and losslessness section).
  * CAST notes (papernotes.org, ICLR 2026): cost table and select(), width
    pruning, depth pruning and the cost-aware verify count (key designs 1-4).
  * Graft review (paper.rainbus.top): checkpoint gate and budget release,
    retrieval graft from the successor matrix, hybrid verification and the
    online top-k refresh (execution-flow paragraph, steps 1-3).

Where the pages are silent or garbled this module takes one reading and says
so at the point of use.

Each function a parity test relies on is pinned, in tests/test_oracle_pins.py,
by something other than itself:
  * row statistics and top-k: exact sums and brute-force orderings;
  * path values: the product of confidences recomputed along parent chains;
  * frontier and rerank: invariants, and brute force over every connected
    subtree of tiny trees;
  * flatten, mask, positions, paths: hand-listed visibility and path rules;
  * greedy verify: the noise-free rank-0-chain closed form;
  * stochastic verify: the textbook one-child rule, hand-computed thresholds
    for q- and point-mass proposals (duplicate siblings and T != 1 included),
    and chi-square losslessness on a 16-token vocabulary;
  * CAST: the Theorem 4.1 reduction to fixed top-K, a hand-worked round whose
    cost lookups move through a 4-row grid (context row, verify context,
    S_T versus S_D, the zero-cost step), and a hand-worked depth-gate FIFO;
  * Graft: the gather recomputed directly, stages forced by thresholds, and
    the refresh as a full sort of each target row.

Conventions shared with the library's documented layout (not with its code):
  * node 0 of a row is the root; layer d's children are appended slot-major
    (frontier slot j, then rank r), retrieval nodes after all draft nodes;
  * a canonical key packs (depth, source, rank path) so that ascending key
    order is breadth-first, draft before retrieval, then lexicographic ranks.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# canonical node key
# ---------------------------------------------------------------------------
KEY_DEPTH_SHIFT = 59
KEY_SRC_SHIFT = 58
RANK_BITS = 5
MAX_DEPTH = 11          # 11 rank fields of 5 bits fit under the source bit
MAX_RANK = (1 << RANK_BITS) - 1


def key_child(parent_key: int, parent_depth: int, rank: int, src: int = 0) -> int:
    """Key of the child at `rank` under a parent: depth+1, same rank path + rank."""
    d = parent_depth + 1
    assert 1 <= d <= MAX_DEPTH and 0 <= rank <= MAX_RANK
    path = parent_key & ((1 << KEY_SRC_SHIFT) - 1)
    path |= rank << (KEY_SRC_SHIFT - RANK_BITS * d)
    srcbit = (src << KEY_SRC_SHIFT) | (parent_key & (1 << KEY_SRC_SHIFT))
    return (d << KEY_DEPTH_SHIFT) | srcbit | path


def key_depth(key: int) -> int:
    return key >> KEY_DEPTH_SHIFT


def key_as_i64(key: int) -> int:
    """Keys stay below 2**63 (depth <= 11), so they fit a signed 64-bit slot."""
    assert 0 <= key < (1 << 63)
    return key


# ---------------------------------------------------------------------------
# O1: draft-row statistics and per-node vocabulary top-k
# ---------------------------------------------------------------------------

def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Input logits as float64; bf16 is decoded exactly from its bit pattern."""
    if dtype == "bf16":
        return (np.asarray(raw).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(raw, dtype=np.float32).astype(np.float64)


def row_stats(l: np.ndarray):
    """(max, argmax, sigma') of one logit row.

    The confidence of a token is its draft softmax probability (EAGLE-2
    explainer, section on confidence as an acceptance proxy).  sigma' is the
    softmax normaliser relative to the max with one instance of the max left
    out, so that log-confidence of the top token, -log1p(sigma'), keeps full
    relative precision (reading: summed log-probabilities, Graft step 1).
    """
    mx = float(np.max(l))
    vstar = int(np.argmax(l))                 # first occurrence = lowest id
    e = np.exp(l - mx)
    e[vstar] = 0.0
    return mx, vstar, float(np.sum(e))


def topk_ids(l: np.ndarray, K: int) -> np.ndarray:
    """The K largest entries by (value desc, id asc) -- an exact total order."""
    K = min(K, l.shape[0])
    thr = np.partition(l, l.shape[0] - K)[l.shape[0] - K]   # K-th largest value
    cand = np.nonzero(l >= thr)[0]
    order = np.lexsort((cand, -l[cand]))
    return cand[order[:K]].astype(np.int64)


def log_conf(l: np.ndarray, ids: np.ndarray, mx: float, sp: float) -> np.ndarray:
    """log c_x = (l_x - max) - log1p(sigma'):  the log of the draft softmax probability."""
    return (l[ids] - mx) - math.log1p(sp)


# ---------------------------------------------------------------------------
# per-row tree
# ---------------------------------------------------------------------------

@dataclass
class RowTree:
    token: List[int] = field(default_factory=list)
    parent: List[int] = field(default_factory=list)
    depth: List[int] = field(default_factory=list)
    S: List[float] = field(default_factory=list)       # summed log confidence (fp64)
    logc: List[float] = field(default_factory=list)
    key: List[int] = field(default_factory=list)
    eslot: List[int] = field(default_factory=list)     # frontier slot used to expand it, -1 if never
    src: List[int] = field(default_factory=list)       # 0 draft, 1 retrieval
    # statistics of the draft row that expanded each node: (layer, slot) -> (max, sigma')
    rstats: dict = field(default_factory=dict)
    layers_built: int = 0

    def add(self, token, parent, depth, S, logc, key, src=0) -> int:
        self.token.append(int(token)); self.parent.append(int(parent))
        self.depth.append(int(depth)); self.S.append(float(S)); self.logc.append(float(logc))
        self.key.append(int(key)); self.eslot.append(-1); self.src.append(int(src))
        return len(self.token) - 1

    @property
    def n(self) -> int:
        return len(self.token)


def new_tree(root_token: int) -> RowTree:
    t = RowTree()
    t.add(root_token, -1, 0, 0.0, 0.0, 0)       # V(root) = 1, i.e. S = 0
    return t


def order_by_value(t: RowTree, nodes: Sequence[int]) -> List[int]:
    """Nodes sorted by (S desc, key asc).  Since the key leads with depth this is
    also (S desc, depth asc, key asc): on equal value the shallower node wins
    (EAGLE-2 explainer, reranking section)."""
    return sorted(nodes, key=lambda i: (-t.S[i], t.key[i]))


# ---------------------------------------------------------------------------
# O2 / O3: one expansion layer
# ---------------------------------------------------------------------------

def expand_layer(t: RowTree, layer: int, frontier: Sequence[int], rows: Sequence[np.ndarray],
                 K_n: int) -> List[int]:
    """Expand each frontier node with its draft row and attach K_n children.

    Children are the draft row's top-K_n tokens; each child's value is its
    parent's value times its own confidence, kept as a sum of logs
    (EAGLE-2 explainer, expansion section; Graft step 1's S_{d,j} recursion).
    Frontier slot j is expanded with rows[j].
    """
    new = []
    for j, u in enumerate(frontier):
        l = rows[j]
        mx, _, sp = row_stats(l)
        t.eslot[u] = j
        t.rstats[(layer, j)] = (mx, sp)
        ids = topk_ids(l, K_n)
        lc = log_conf(l, ids, mx, sp)
        for r, (x, c) in enumerate(zip(ids, lc)):
            new.append(t.add(x, u, t.depth[u] + 1, t.S[u] + c, c,
                             key_child(t.key[u], t.depth[u], r)))
    t.layers_built = layer
    return new


# ---------------------------------------------------------------------------
# O9: CAST (cost table, select(), width, depth, verify count)
# ---------------------------------------------------------------------------

def cast_select_row(c: int, L: int, M: int) -> int:
    """Grid row of context length c.

    The notes print select(c) = (max(floor(c/L), M-1) + 1) L, which maps every c
    to the last grid point; reading: min (clamp to the last row).  The row index
    is select(c)/L - 1 = min(floor(c/L), M-1).  (CAST notes, key design 1.)
    """
    return min(c // L, M - 1)


def cast_width_costs(S_T: np.ndarray, S_D: np.ndarray, ctx: int, L: int, M: int, kmax: int):
    """c_k = S_D[select(ctx)][k] / S_T[select(ctx)][1] for k = 1..kmax (index 0 unused)."""
    r = cast_select_row(ctx, L, M)
    c = np.zeros(kmax + 1)
    c[1:] = S_D[r, 1:kmax + 1].astype(np.float64) / float(S_T[r, 1])
    return c


def cast_verify_costs(S_T: np.ndarray, ctx: int, L: int, M: int, kmax: int):
    """c_k = S_T[select(n0)][k] / S_T[select(n0)][1] (CAST notes, key design 4)."""
    r = cast_select_row(ctx, L, M)
    c = np.zeros(kmax + 1)
    c[1:] = S_T[r, 1:kmax + 1].astype(np.float64) / float(S_T[r, 1])
    return c


def anchor_scan(u: np.ndarray, c: np.ndarray, C: float, kmax: int, margins=None) -> int:
    """Number of items to keep from cumulative utility u[1..kmax] and cost c[1..kmax].

    The notes keep items while the marginal utility (u_k - u_k')/(c_k - c_k')
    stays above the threshold and defer the discrete, non-concave case to an
    "Algorithm 1" whose text is not on the page.  Reading: start with one item
    (anchor a = 1); for k = 2..kmax, move the anchor to k when the average
    marginal from the anchor reaches C (>=, so that the fixed top-K special case
    of Theorem 4.1 holds with equality).  On concave u this is "stop at the
    first marginal below C"; on a plateau it looks past it.  A non-increasing
    cost step counts as infinite marginal when utility grows.
    """
    if kmax <= 0:
        return 0
    a = 1
    for k in range(2, kmax + 1):
        du, dc = u[k] - u[a], c[k] - c[a]
        if dc > 0:
            g = du / dc
            if margins is not None and math.isfinite(C):
                margins.append(("cast", abs(g - C) / max(1.0, abs(C))))
            if g >= C:
                a = k
        elif du > 0:
            a = k
    return a


def cast_width(sorted_v: Sequence[np.ndarray], c: np.ndarray, C1: float, K_e_max: int,
               margins=None):
    """Width n_i of layer i from the batch-averaged cumulative utility (key design 2).

    sorted_v[b] holds row b's layer-i candidate values e^S in frontier order.
    u_k = (1/B) sum_b sum_{s<=k} v_b(s); K_cap = min(K_e_max, candidates).
    Returns (n_i, u) with u[k] for k = 0..K_cap.
    """
    B = len(sorted_v)
    kcap = min([K_e_max] + [len(v) for v in sorted_v])
    u = np.zeros(kcap + 1)
    for k in range(1, kcap + 1):
        u[k] = sum(float(np.sum(v[:k])) for v in sorted_v) / B
    return anchor_scan(u, c, C1, kcap, margins), u


def cast_verify_count(t: RowTree, c: np.ndarray, C3: float, m_max: int, margins=None) -> int:
    """Per-row verify count m_b over all nodes' values, sorted (key design 4).

    u_k = sum_{j<=k} v_(j) with v = e^S of the k best non-root nodes.  The
    formula has no batch average, so the count is per row (reading).
    """
    order = order_by_value(t, range(1, t.n))
    kmax = min(m_max, len(order))
    v = np.exp(np.array([t.S[i] for i in order[:kmax]]))
    u = np.concatenate([[0.0], np.cumsum(v)])
    return anchor_scan(u, c, C3, kmax, margins)


# ---------------------------------------------------------------------------
# draft phase for a batch: EAGLE-2 expansion, optionally with CAST or the Graft gate
# ---------------------------------------------------------------------------

@dataclass
class DraftResult:
    trees: List[RowTree]
    frontiers: List[List[List[int]]]        # [b][layer-1] -> frontier node list
    widths: List[int]                       # per built layer: frontier width used next
    depth_built: int
    active: List[bool]
    k_draft: List[int]
    margins: list


def draft_phase(draft_rows, B: int, root_tok: Sequence[int], D: int, K_e: int, K_n: int,
                cast: Optional[dict] = None, graft: Optional[dict] = None) -> DraftResult:
    """Build every row's tree, layer by layer.

    draft_rows(layer, b, slot) -> float64 row: the stand-in for the draft
    forward of frontier slot `slot` at layer `layer` (1-based).  Layer 1
    expands the root; layers 2..D expand the previous layer's frontier, which is
    the top-K_e of that layer's nodes by value (EAGLE-2 explainer, expansion
    section and the decode-step flow); layer-D nodes are never expanded.

    cast: dict(S_T, S_D, L, M, C1[D], C2, R) switches width and depth to CAST.
    graft: dict(ck_depth, tau, k_draft, K_max) turns on the Graft gate; an
    optional draft_cap (default K_max) is the draft budget of rows never pruned
    (root-only and tail-only grafting keep a fixed budget and no checkpoints).
    """
    assert not (cast and graft)
    trees = [new_tree(root_tok[b]) for b in range(B)]
    fronts = [[[0]] for _ in range(B)]        # "layer 0" frontier: the root
    active = [True] * B
    k_draft = [graft.get("draft_cap", graft["K_max"]) if graft else 0] * B
    margins: list = []
    widths: List[int] = []
    fifo = [1.0]                              # CAST gain buffer, initial {1}
    ctx = 0                                   # tree tokens fed to the draft so far
    u_prev = None
    depth_built = 0
    for d in range(1, D + 1):
        new_nodes = [[] for _ in range(B)]
        for b in range(B):
            if not active[b]:
                continue
            fr = fronts[b][-1]
            rows = [draft_rows(d, b, j) for j in range(len(fr))]
            new_nodes[b] = expand_layer(trees[b], d, fr, rows, K_n)
        depth_built = d
        ordered = [order_by_value(trees[b], new_nodes[b]) for b in range(B)]

        if cast is not None:
            cw = cast_width_costs(cast["S_T"], cast["S_D"], ctx, cast["L"], cast["M"],
                                  min(K_e, min(len(o) for o in ordered)))
            sv = [np.exp(np.array([trees[b].S[i] for i in ordered[b]])) for b in range(B)]
            wm: list = []
            n_i, u = cast_width(sv, cw, float(cast["C1"][d - 1]), K_e, wm)
            margins.extend((k, v, -1) for k, v in wm)
            _frontier_margins(trees, ordered, n_i, margins)
            widths.append(n_i)
            for b in range(B):
                fronts[b].append(ordered[b][:n_i])
            # depth gate (key design 3): push the previous layer's gain ratio,
            # then grow iff mean(A) * u_n / c_n >= C2 and the depth cap allows it.
            if u_prev is not None:
                fifo.append(u[n_i] / u_prev if u_prev > 0 else 0.0)
                if len(fifo) > cast["R"]:
                    fifo.pop(0)
            score = float(np.mean(fifo)) * u[n_i] / cw[n_i]
            if d < D and math.isfinite(cast["C2"]):
                margins.append(("cast", abs(score - cast["C2"]) / max(1.0, abs(cast["C2"])), -1))
            u_prev = u[n_i]
            ctx += n_i
            if d == D or score < cast["C2"]:
                break
            continue

        widths.append(K_e)
        _frontier_margins(trees, ordered, K_e, margins)
        for b in range(B):
            fronts[b].append(ordered[b][:K_e] if active[b] else [])
        if graft is not None and d in graft["ck_depth"]:
            s = graft["ck_depth"].index(d)
            for b in range(B):
                if not active[b]:
                    continue
                cmax = math.exp(max(trees[b].S[i] for i in new_nodes[b]))
                margins.append(("gate", abs(cmax - graft["tau"][s]), b))
                if not cmax > graft["tau"][s]:          # g_d = 1[c_d > tau_d]
                    active[b] = False
                    k_draft[b] = graft["k_draft"][s]
    return DraftResult(trees, fronts, widths, depth_built, active, k_draft, margins)


def _frontier_margins(trees, ordered, n, margins):
    """Gaps between consecutive values that decide the frontier slots: every pair
    inside the first n+1 positions.  Exact ties between siblings expanded from
    the same row with equal logits are resolved identically by key and carry no
    risk, so they are skipped."""
    for b, o in enumerate(ordered):
        t = trees[b]
        for i in range(min(n, len(o) - 1)):
            x, y = o[i], o[i + 1]
            if t.S[x] == t.S[y] and t.parent[x] == t.parent[y]:
                continue
            margins.append(("value", abs(t.S[x] - t.S[y]), b))


# ---------------------------------------------------------------------------
# O5: rerank
# ---------------------------------------------------------------------------

def rerank(t: RowTree, m: int, margins=None) -> List[int]:
    """Top-m non-root nodes by (value desc, depth asc, key asc).

    All nodes of the tree are candidates, expanded or not (EAGLE-2 explainer,
    reranking section).  Because a child's value never exceeds its parent's and
    ties prefer the shallower node, the selection is parent-closed; asserted.
    """
    order = order_by_value(t, range(1, t.n))
    sel = order[:min(m, len(order))]
    if margins is not None and 0 < len(sel) < len(order):
        x, y = order[len(sel) - 1], order[len(sel)]
        if not (t.S[x] == t.S[y] and t.parent[x] == t.parent[y]):
            margins.append(("value", abs(t.S[x] - t.S[y])))
    chosen = set(sel) | {0}
    for i in sel:
        assert t.parent[i] in chosen, "rerank selection is not parent-closed"
    return sel


# ---------------------------------------------------------------------------
# O10: Graft retrieval graft and successor-matrix refresh
# ---------------------------------------------------------------------------

def graft_template(t: RowTree, M_b: np.ndarray, k_ret: int, depth: int, width: int,
                   anchor: int = 0) -> List[int]:
    """Append the first k_ret nodes of the retrieval template hung off `anchor`
    (the root for Graft's prune-then-graft).

    Each retrieved node's token is a successor-matrix lookup of its parent's
    token, x_u = M[x_parent(u), r_u] (Graft step 2).  Reading of the template
    (depth x width): `width` chains hang off the anchor; chain c starts with
    successor c of the anchor's token and continues with successor 0 of its
    own last token.  Template order is level-major, then chain; truncating a
    prefix keeps it parent-closed.  Retrieved nodes have no draft value
    (S = -inf).  Levels that would pass MAX_DEPTH (the canonical key's limit)
    are not built.
    """
    added = []
    prev = [anchor] * width
    depth = min(depth, MAX_DEPTH - t.depth[anchor])
    for lvl in range(1, depth + 1):
        for c in range(width):
            idx = (lvl - 1) * width + c
            if idx >= k_ret:
                return added
            p = prev[c]
            tok = int(M_b[t.token[p], c if lvl == 1 else 0])
            key = key_child(t.key[p], t.depth[p], c if lvl == 1 else 0, src=1)
            n = t.add(tok, p, t.depth[p] + 1, -math.inf, -math.inf, key, src=1)
            prev[c] = n
            added.append(n)
    return added


def graft_tail_anchor(t: RowTree, sel: Sequence[int]) -> int:
    """The tail of the selected draft tree, for tail-only grafting (Graft
    review, the Fig. 2 comparison; reading): the deepest selected node, ties
    to the higher value, then the smaller canonical key; the root if nothing
    is selected."""
    best = 0
    for i in sel:
        if best == 0 or (t.depth[i], t.S[i], -t.key[i]) > (t.depth[best], t.S[best], -t.key[best]):
            best = i
    return best


def succ_update(M_b: np.ndarray, flat_token: Sequence[int], n_flat: int, target_rows, k: int):
    """Refresh M rows after verification (Graft step 3).

    For every verified flat position i >= 1 (accepted or not), the row of its
    token becomes the top-k ids of the target's next-token distribution at i.
    A later flat position wins when two positions carry the same token.
    """
    for i in range(1, n_flat):
        tok = int(flat_token[i])
        if tok < 0:
            continue
        M_b[tok, :] = topk_ids(target_rows(i), k)[:k]


# ---------------------------------------------------------------------------
# O6: flatten, mask, positions, retrieve paths
# ---------------------------------------------------------------------------

@dataclass
class Flat:
    node: List[int]
    token: List[int]
    parent: List[int]
    pos: List[int]
    mask: np.ndarray          # [P][W] uint32, bit j of row i: j is i or an ancestor of i
    retrieve: np.ndarray      # [n_leaves][Dp+1] flat indices, -1 padded
    n_leaves: int
    depth: List[int]


def flatten(t: RowTree, sel: Sequence[int], P: int, prefix: int, Dp: int) -> Flat:
    """Linearise {root} + selected into flat order, with the ancestor-only mask.

    Flat order is ascending canonical key (root first, breadth-first, draft
    before retrieval): a function of the selected set alone (reading; the
    pages only require a linear order).  Each position attends to itself, its
    ancestors and the whole prefix, never to siblings (EAGLE-2 explainer,
    reranking section and engineering difficulty one).  Positions are
    prefix + depth (reading of Graft step 3's tree position ids).  Candidate
    paths are root-to-leaf flat indices, one per leaf in flat order.
    Positions past the selection are padding: token -1, parent -1,
    pos = prefix, self-only mask bit, on no path.
    """
    nodes = sorted(set(sel) | {0}, key=lambda i: t.key[i])
    n = len(nodes)
    assert n <= P
    where = {v: i for i, v in enumerate(nodes)}
    W = (P + 31) // 32
    node = nodes + [-1] * (P - n)
    token = [t.token[v] for v in nodes] + [-1] * (P - n)
    parent = [where[t.parent[v]] if t.parent[v] >= 0 else -1 for v in nodes] + [-1] * (P - n)
    depth = [t.depth[v] for v in nodes] + [0] * (P - n)
    pos = [prefix + d for d in depth]
    mask = np.zeros((P, W), np.uint32)
    for i in range(P):
        j = i
        while j >= 0:
            mask[i, j // 32] |= np.uint32(1 << (j % 32))
            j = parent[j] if i < n else -1
    has_child = [False] * n
    for i in range(1, n):
        has_child[parent[i]] = True
    leaves = [i for i in range(n) if not has_child[i]]
    retrieve = np.full((max(1, len(leaves)), Dp + 1), -1, np.int32)
    for li, leaf in enumerate(leaves):
        chain = []
        j = leaf
        while j >= 0:
            chain.append(j)
            j = parent[j]
        chain.reverse()
        retrieve[li, :len(chain)] = chain
    return Flat(node, token, parent, pos, mask, retrieve, len(leaves), depth)


# ---------------------------------------------------------------------------
# O7: greedy verification
# ---------------------------------------------------------------------------

def verify_greedy(f: Flat, argmax_of) -> tuple:
    """Longest accepted candidate path at temperature 0.

    At T = 0 acceptance is deterministic: a child is accepted iff its token is
    the target's argmax (lowest id on ties) at its parent (EAGLE-2 explainer,
    losslessness section; the decode-step flow applies the rule along candidate
    paths).  The accept length of a path is its longest matching prefix; the
    first path with the greatest length wins.  Returns (accept_len,
    accept_path (root first), next_token).
    """
    best_len, best_path = -1, None
    for li in range(f.n_leaves):
        path = [int(x) for x in f.retrieve[li] if x >= 0]
        ell = 0
        for s in range(1, len(path)):
            if f.token[path[s]] == argmax_of(path[s - 1]):
                ell = s
            else:
                break
        if ell > best_len:
            best_len, best_path = ell, path[:ell + 1]
    return best_len, best_path, int(argmax_of(best_path[-1]))


# ---------------------------------------------------------------------------
# O8: stochastic verification (T > 0)
# ---------------------------------------------------------------------------

def softmax_T(l: np.ndarray, T: float) -> np.ndarray:
    z = l / T
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def sample_inverse_cdf(p: np.ndarray, u: float, margins=None) -> int:
    """Smallest id v with sum_{w<=v} p_w > u * sum(p), by ascending-id prefix sums."""
    cs = np.cumsum(p)
    thr = u * cs[-1]
    v = int(np.searchsorted(cs, thr, side="right"))
    if v >= p.shape[0]:
        v = int(np.nonzero(p > 0)[0][-1])
    if margins is not None:
        lo = cs[v - 1] if v > 0 else 0.0
        margins.append(("cdf", min(thr - lo, cs[v] - thr) / cs[-1]))
    return v


def verify_stochastic(f: Flat, target_row, draft_row_of, T: float, U: np.ndarray,
                      margins=None, retrieval=None, proposal: str = "draft") -> tuple:
    """Speculative sampling over the flattened tree.

    Chain rule (EAGLE-2 explainer, ledger section): accept a drafted token x
    with probability min(1, p(x)/q(x)), q being the distribution x was
    proposed from; on rejection draw from norm(max(0, p - q)).  Reading for a
    tree (the pages apply the rule "along candidate paths"): at node u, with p
    the target distribution at u, try u's selected children in flat order;
    child c is accepted when U[c,0] < p(x_c)/q(x_c) (min(1, .) is implicit),
    and a rejection replaces p by norm(max(0, p - q)) (kept as it was if that
    residual is all zero) before the next sibling.  When no child is accepted,
    or u has no selected child, the next token is drawn from the current p by
    inverse CDF with U[u,1].  p = softmax(target/T).

    Which q (reading; the losslessness section says the draft distribution
    only shapes which candidates are proposed, never the output distribution):
      proposal = "draft": q = softmax(draft/T) of the row u was expanded with.
        This is the proposal of children drawn i.i.d. from the draft, and the
        walk is then exactly lossless; on children picked deterministically
        (top-K) it is not.
      proposal = "point": every child is a point-mass proposal q = delta_x,
        the proposal of a deterministically chosen token: accepted with
        probability p(x), and a rejection leaves norm(max(0, p - delta_x)),
        i.e. p with x removed and renormalised.  Exactly lossless for any
        tree, top-K trees included; the draft rows are not read.

    Retrieval children (retrieval[c] true: Graft grafted nodes, which no draft
    row proposed) are point-mass proposals in both modes (Graft review, step
    (3): the acceptance rule is the standard one).  Draft children come first
    in flat order, then retrieval children.
    """
    assert proposal in ("draft", "point")
    n = len([x for x in f.node if x >= 0])
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[f.parent[i]].append(i)
    u = 0
    path = [0]
    while True:
        p = softmax_T(target_row(u), T)
        if not children[u]:
            nxt = sample_inverse_cdf(p, float(U[u, 1]), margins)
            break
        q = None
        acc = None
        for c in children[u]:
            x = f.token[c]
            if proposal == "point" or (retrieval is not None and retrieval[c]):
                ratio = float(p[x])
                if margins is not None:
                    margins.append(("accept", abs(float(U[c, 0]) - ratio)))
                if float(U[c, 0]) < ratio:
                    acc = c
                    break
                r = p.copy()
                r[x] = 0.0
                Z = float(np.sum(r))
                if margins is not None:
                    margins.append(("residual", Z))
                if Z > 0.0:
                    p = r / Z
                continue
            if q is None:
                q = softmax_T(draft_row_of(u), T)
            ratio = p[x] / q[x] if q[x] > 0 else math.inf
            if margins is not None and math.isfinite(ratio):
                margins.append(("accept", abs(float(U[c, 0]) - ratio) / max(1.0, ratio)))
            if float(U[c, 0]) < ratio:
                acc = c
                break
            r = np.maximum(0.0, p - q)
            Z = float(np.sum(r))
            if margins is not None:
                margins.append(("residual", Z))
            if Z > 0.0:
                p = r / Z
        if acc is None:
            nxt = sample_inverse_cdf(p, float(U[u, 1]), margins)
            break
        path.append(acc)
        u = acc
    return len(path) - 1, path, nxt


# ---------------------------------------------------------------------------
# whole round for a batch: the layout the library's outputs are compared against
# ---------------------------------------------------------------------------

def tree_arrays(trees: Sequence[RowTree], cap: int, D: int, R: int) -> dict:
    """Per-row tree state as [B][cap] arrays (fp32 values, int32/int64 ids)."""
    B = len(trees)
    out = {
        "token": np.full((B, cap), -1, np.int32), "parent": np.full((B, cap), -1, np.int32),
        "depth": np.full((B, cap), -1, np.int32), "S": np.zeros((B, cap), np.float32),
        "logc": np.zeros((B, cap), np.float32), "key": np.full((B, cap), -1, np.int64),
        "eslot": np.full((B, cap), -1, np.int32), "n_nodes": np.zeros(B, np.int32),
        "rmax": np.zeros((B, D, R), np.float32), "rsp": np.zeros((B, D, R), np.float32),
    }
    for b, t in enumerate(trees):
        n = t.n
        assert n <= cap
        out["token"][b, :n] = t.token; out["parent"][b, :n] = t.parent
        out["depth"][b, :n] = t.depth
        out["S"][b, :n] = np.array(t.S, np.float64).astype(np.float32)
        out["logc"][b, :n] = np.array(t.logc, np.float64).astype(np.float32)
        out["key"][b, :n] = [key_as_i64(k) for k in t.key]
        out["eslot"][b, :n] = t.eslot; out["n_nodes"][b] = n
        for (layer, j), (mx, sp) in t.rstats.items():
            out["rmax"][b, layer - 1, j] = mx
            out["rsp"][b, layer - 1, j] = sp
    return out


def run_round(*, B, V, dtype, D, K_e, K_n, m_max, root_tok, draft_raw, target_raw_fn,
              temperature, U, prefix=0, cast=None, graft=None, M=None, k_succ=8,
              tpl=(8, 8), proposal="point") -> dict:
    """One full round on the CPU.

    draft_raw: [D][B][R][V] raw logits; target_raw_fn(flat) -> [B][P][V] raw
    target rows for the flattened tree (the stand-in for the target forward,
    built by the caller from the returned flat layout); temperature [B]
    (0 = greedy); U [B][P][2]; proposal: the T > 0 walk's proposal for draft
    children ("point" or "draft", see verify_stochastic).
    cast: dict(S_T, S_D, L, M, C1[D], C2, C3[B], R).
    graft: dict(ck_depth, tau, k_draft, K_max).  M: [B][V][k] successor matrix,
    updated in place when graft is given.  Returns every output of the round.
    """
    def drow(layer, b, j):
        return decode(draft_raw[layer - 1, b, j], dtype)

    dr = draft_phase(drow, B, root_tok, D, K_e, K_n, cast=cast, graft=graft)
    margins = dr.margins
    P = m_max + 1
    tail = graft is not None and graft.get("anchor") == "tail"
    Dp = (min(D + tpl[0], MAX_DEPTH) if tail else max(D, tpl[0])) if graft else D
    sels, m_rows, flats = [], [], []
    for b in range(B):
        t = dr.trees[b]
        mb: list = []
        if cast is not None:
            cv = cast_verify_costs(cast["S_T"], prefix, cast["L"], cast["M"], m_max)
            m_b = cast_verify_count(t, cv, float(cast["C3"][b]), m_max, mb)
        elif graft is not None:
            m_b = dr.k_draft[b]
        else:
            m_b = m_max
        sel = rerank(t, m_b, mb)
        margins.extend((k, v, b) for k, v in mb)
        if graft is not None:
            k_ret = graft["K_max"] - len(sel)
            anchor = graft_tail_anchor(t, sel) if tail else 0
            sel = sel + graft_template(t, M[b], k_ret, tpl[0], tpl[1], anchor)
        sels.append(sel)
        m_rows.append(len(sel))
        flats.append(flatten(t, sel, P, prefix, Dp))

    target_raw = target_raw_fn(dr, flats)
    acc_len = np.zeros(B, np.int32)
    acc_path = np.full((B, Dp + 1), -1, np.int32)
    nxt = np.zeros(B, np.int32)
    amax = np.full((B, P), -1, np.int32)
    for b in range(B):
        f = flats[b]
        rows = {}

        def trow(i, b=b, rows=rows):
            if i not in rows:
                rows[i] = decode(target_raw[b, i], dtype)
            return rows[i]

        n = len([x for x in f.node if x >= 0])
        for i in range(n):
            amax[b, i] = int(np.argmax(trow(i)))
        if float(temperature[b]) == 0.0:
            L_, path, tok = verify_greedy(f, lambda i: amax[b, i])
        else:
            t = dr.trees[b]

            def qrow(i, b=b, t=t, f=f):
                v = f.node[i]
                return drow(t.depth[v] + 1, b, t.eslot[v])

            ret = [t.src[v] == 1 if v >= 0 else False for v in f.node]
            mb = []
            L_, path, tok = verify_stochastic(f, trow, qrow, float(temperature[b]), U[b], mb, ret,
                                              proposal)
            margins.extend((k, v, b) for k, v in mb)
        acc_len[b] = L_
        acc_path[b, :len(path)] = path
        nxt[b] = tok
        if graft is not None:
            succ_update(M[b], f.token, n, trow, k_succ)

    cap = max(t.n for t in dr.trees)
    out = {
        "draft": dr, "flats": flats, "sels": sels, "m_rows": np.array(m_rows, np.int32),
        "accept_len": acc_len, "accept_path": acc_path, "next_token": nxt, "argmax": amax,
        "margins": margins, "Dp": Dp,
    }
    out["tree"] = tree_arrays(dr.trees, cap, D, K_e)
    return out


def min_margins(margins) -> dict:
    """Smallest margin of each kind of float-driven decision.

    Entries are (kind, margin, row); row -1 marks a decision shared by the
    whole batch (CAST width and depth)."""
    res: dict = {}
    for kind, v, _ in margins:
        res[kind] = min(res.get(kind, math.inf), v)
    return res


# Smallest gap between a float-driven decision and its threshold for which an
# fp32 implementation is expected to take the same decision as this fp64 one.
MARGIN_FLOOR = {"value": 1e-4, "cast": 1e-4, "gate": 1e-4, "accept": 1e-5,
                "residual": 1e-6, "cdf": 1e-8}


def margin_failures(margins) -> set:
    """Rows (or -1 for the whole batch) with a decision closer than its floor."""
    return {row for kind, v, row in margins if not v > MARGIN_FLOOR[kind]}

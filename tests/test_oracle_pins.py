"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Nothing here compares the oracle with itself.  Each test ties one oracle step
to a closed form, an invariant, brute force on tiny inputs, a special case
that reduces to a textbook rule, a hand-computed example, or a statistical
property (losslessness) -- chosen so that a dropped term, a wrong sign or
index, or a swapped operand in the oracle fails at least one of them.
"""
import functools
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import special, stats

from gen import synth
from gen.configs import CastSpec, GraftSpec, Workload
from oracle import ddt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers: small random batches from the seeded generator
# ---------------------------------------------------------------------------

def small_workload(V=64, B=2, D=3, K_e=3, K_n=4, m=10, dtype="f32", **kw):
    return Workload(f"pin_V{V}", B=B, V=V, dtype=dtype, D=D, K_e=K_e, K_n=K_n, m=m,
                    verify=kw.pop("verify", "greedy"), sigma=0.5, **kw)


def build(w, seed=7, rnd=0, cast=None, graft=None):
    arena = synth.draft_arena(w, seed, rnd)
    roots = synth.root_tokens(w, seed, rnd)

    def drow(layer, b, j):
        return O.decode(arena[layer - 1, b, j], w.dtype)

    dr = O.draft_phase(drow, w.B, roots, w.D, w.K_e, w.K_n, cast=cast, graft=graft)
    return dr, drow, arena, roots


def brute_sorted_ids(l):
    return sorted(range(len(l)), key=lambda v: (-l[v], v))


# ---------------------------------------------------------------------------
# O1: row statistics, top-k, log-confidence
# ---------------------------------------------------------------------------

def test_bf16_decode_known_bits():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0000, 0x7F7F], np.uint16)
    got = O.decode(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 3.140625 and got[3] == 0.0
    assert got[4] == float(np.float32(3.3895313892515355e38))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_stats_against_exact_sum(dtype):
    g = np.random.default_rng(1)
    for _ in range(20):
        V = int(g.integers(2, 400))
        x = (g.standard_normal(V) * g.uniform(0.1, 4)).astype(np.float32)
        raw = synth.cast_row(x, dtype)
        l = O.decode(raw, dtype)
        mx, vstar, sp = O.row_stats(l)
        # brute force: first index holding the maximum, exact sum of the rest
        assert mx == max(l.tolist())
        assert vstar == l.tolist().index(mx)
        rest = [math.exp(v - mx) for i, v in enumerate(l.tolist()) if i != vstar]
        assert sp == pytest.approx(math.fsum(rest), rel=1e-13, abs=0.0)


def test_row_stats_repeated_max_counts_once():
    l = np.array([1.0, 3.0, 3.0, 0.0])
    mx, vstar, sp = O.row_stats(l)
    assert (mx, vstar) == (3.0, 1)
    assert sp == pytest.approx(1.0 + math.exp(-2.0) + math.exp(-3.0), rel=1e-15)


def test_topk_matches_bruteforce_order_with_ties():
    g = np.random.default_rng(2)
    for _ in range(50):
        V = int(g.integers(1, 300))
        # coarse values force many exact ties
        l = np.round(g.standard_normal(V) * 3).astype(np.float64)
        K = int(g.integers(1, 12))
        got = O.topk_ids(l, K).tolist()
        assert got == brute_sorted_ids(l.tolist())[:min(K, V)]


def test_log_conf_is_log_softmax():
    g = np.random.default_rng(3)
    for _ in range(20):
        V = int(g.integers(2, 500))
        l = O.decode(synth.cast_row(g.standard_normal(V).astype(np.float32) * 3, "bf16"), "bf16")
        mx, _, sp = O.row_stats(l)
        ids = np.arange(V)
        lc = O.log_conf(l, ids, mx, sp)
        ref = l - special.logsumexp(l)
        np.testing.assert_allclose(lc, ref, rtol=1e-12, atol=1e-12)
        assert math.fsum(np.exp(lc).tolist()) == pytest.approx(1.0, abs=1e-12)


def test_log_conf_confident_token_keeps_relative_precision():
    # one dominant logit: log c of the top token is about -sum(exp(others - max))
    l = np.array([40.0, 0.0, -1.0, 2.0])
    mx, _, sp = O.row_stats(l)
    lc = O.log_conf(l, np.array([0]), mx, sp)[0]
    tail = math.exp(-40) + math.exp(-41) + math.exp(-38)
    assert lc == pytest.approx(-tail, rel=1e-12)


# ---------------------------------------------------------------------------
# keys
# ---------------------------------------------------------------------------

def test_key_order_is_breadth_first_then_rank_path():
    k_a = O.key_child(0, 0, 0)
    k_b = O.key_child(0, 0, 1)
    k_aa = O.key_child(k_a, 1, 0)
    k_ab = O.key_child(k_a, 1, 7)
    k_ba = O.key_child(k_b, 1, 0)
    k_r = O.key_child(0, 0, 0, src=1)          # retrieval child of the root
    k_rr = O.key_child(k_r, 1, 0)               # its retrieval child
    assert 0 < k_a < k_b < k_r < k_aa < k_ab < k_ba < k_rr
    assert O.key_depth(k_aa) == 2 and O.key_depth(k_rr) == 2
    assert k_rr >> O.KEY_SRC_SHIFT & 1 == 1
    deep = 0
    for d in range(O.MAX_DEPTH):
        deep = O.key_child(deep, d, O.MAX_RANK)
    assert deep < (1 << 63)


# ---------------------------------------------------------------------------
# P-a, P-b: path values
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_path_value_is_product_of_confidences(dtype):
    w = small_workload(V=200, B=3, D=4, K_e=3, K_n=4, dtype=dtype)
    dr, drow, _, _ = build(w)
    for b, t in enumerate(dr.trees):
        for i in range(1, t.n):
            # walk the parent chain; each edge's confidence from its own row
            terms, j = [], i
            while j > 0:
                p = t.parent[j]
                row = drow(t.depth[p] + 1, b, t.eslot[p])
                lse = special.logsumexp(row)
                terms.append(row[t.token[j]] - lse)
                j = p
            assert t.S[i] == pytest.approx(math.fsum(terms), rel=1e-11, abs=1e-12)
            assert math.exp(t.S[i]) == pytest.approx(math.prod(math.exp(x) for x in terms),
                                                     rel=1e-10)
            assert t.logc[i] == pytest.approx(terms[0], rel=1e-11, abs=1e-12)


def test_value_monotone_along_edges():
    w = small_workload(V=300, B=4, D=5, K_e=4, K_n=5, dtype="bf16")
    dr, *_ = build(w, seed=11)
    for t in dr.trees:
        for i in range(1, t.n):
            assert t.S[i] <= t.S[t.parent[i]]


def test_children_are_topk_of_their_row_in_rank_order():
    w = small_workload(V=100, B=2, D=3, K_e=2, K_n=5, dtype="bf16")
    dr, drow, _, _ = build(w, seed=5)
    for b, t in enumerate(dr.trees):
        kids = {}
        for i in range(1, t.n):
            kids.setdefault(t.parent[i], []).append(i)
        for p, ch in kids.items():
            row = drow(t.depth[p] + 1, b, t.eslot[p]).tolist()
            want = brute_sorted_ids(row)[:w.K_n]
            assert [t.token[c] for c in ch] == want
            ranks = [(t.key[c] >> (O.KEY_SRC_SHIFT - O.RANK_BITS * t.depth[c])) & O.MAX_RANK
                     for c in ch]
            assert ranks == list(range(len(ch)))


def test_frontier_is_the_best_of_its_layer():
    w = small_workload(V=120, B=3, D=4, K_e=3, K_n=4)
    dr, *_ = build(w, seed=9)
    for b, t in enumerate(dr.trees):
        for d in range(1, dr.depth_built):
            layer = [i for i in range(t.n) if t.depth[i] == d]
            fr = dr.frontiers[b][d]
            rest = [i for i in layer if i not in fr]
            assert len(fr) == min(w.K_e, len(layer))
            for x in fr:
                for y in rest:
                    assert (t.S[x], -t.key[x]) > (t.S[y], -t.key[y])
            for x, y in zip(fr, fr[1:]):
                assert (t.S[x], -t.key[x]) > (t.S[y], -t.key[y])
            # slot j of layer d+1 expanded frontier[j]
            assert [t.eslot[u] for u in fr] == list(range(len(fr)))


# ---------------------------------------------------------------------------
# P-c, P-d: rerank
# ---------------------------------------------------------------------------

def test_rerank_parent_closed_and_sized():
    w = small_workload(V=150, B=4, D=5, K_e=3, K_n=4, dtype="bf16")
    dr, *_ = build(w, seed=21)
    for t in dr.trees:
        for m in (1, 5, 17, 40, 10 ** 4):
            sel = O.rerank(t, m)
            assert len(sel) == min(m, t.n - 1)
            assert len(set(sel)) == len(sel)
            closed = set(sel) | {0}
            assert all(t.parent[i] in closed for i in sel)


def test_rerank_is_best_connected_subtree_bruteforce():
    """Top-m by value is the connected m-node subtree with the largest sum of
    path values (the expected number of accepted draft tokens under the
    confidence model), checked by enumerating every parent-closed subset."""
    checked = 0
    for seed in range(12):
        g = np.random.default_rng(seed)
        K_n = int(g.integers(2, 4))
        D = int(g.integers(2, 4))
        K_e = int(g.integers(1, 3))
        w = small_workload(V=16, B=1, D=D, K_e=K_e, K_n=K_n)
        dr, *_ = build(w, seed=100 + seed)
        t = dr.trees[0]
        nodes = list(range(1, t.n))
        if len(nodes) > 15:
            continue
        for m in range(1, min(6, len(nodes)) + 1):
            best, best_set = -1.0, None
            for sub in itertools.combinations(nodes, m):
                s = set(sub) | {0}
                if not all(t.parent[i] in s for i in sub):
                    continue
                val = math.fsum(math.exp(t.S[i]) for i in sub)
                if val > best:
                    best, best_set = val, set(sub)
            sel = O.rerank(t, m)
            assert math.fsum(math.exp(t.S[i]) for i in sel) == pytest.approx(best, rel=1e-12)
            vals = sorted(t.S[i] for i in nodes)
            if all(a != b for a, b in zip(vals, vals[1:])):
                assert set(sel) == best_set
            checked += 1
    assert checked > 20


# ---------------------------------------------------------------------------
# hand-computed worked example
# ---------------------------------------------------------------------------

def test_worked_example_golden():
    g = json.load(open(os.path.join(GOLDEN, "worked_tree.json")))
    rows = {1: np.log(np.array(g["layer1_probs"])), 2: np.log(np.array(g["layer2_probs"]))}
    dr = O.draft_phase(lambda layer, b, j: rows[layer], 1, [g["root_token"]], g["D"],
                       g["K_e"], g["K_n"])
    t = dr.trees[0]
    e = g["expect"]
    assert t.token == e["node_token"]
    assert t.parent == e["node_parent"]
    np.testing.assert_allclose(np.exp(t.S), e["node_value"], rtol=1e-12)
    sel = O.rerank(t, g["m"])
    assert sel == e["selected"]
    f = O.flatten(t, sel, g["m"] + 1, 0, g["D"])
    assert f.node == e["flat_node"] and f.token == e["flat_token"]
    assert f.parent == e["flat_parent"]
    assert f.mask[:, 0].tolist() == e["mask_rows"]
    assert f.retrieve.tolist() == e["retrieve"]


# ---------------------------------------------------------------------------
# P-e: flatten, mask, positions, paths
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("prefix", [0, 4096])
def test_flatten_mask_positions_paths(prefix):
    w = small_workload(V=100, B=3, D=4, K_e=3, K_n=4, m=20)
    dr, *_ = build(w, seed=31)
    P = 40
    for t in dr.trees:
        for m in (0, 1, 7, 20, 39):
            sel = O.rerank(t, m)
            f = O.flatten(t, sel, P, prefix, w.D)
            n = len(sel) + 1
            assert f.node[0] == 0 and f.parent[0] == -1
            keys = [t.key[v] for v in f.node[:n]]
            assert keys == sorted(keys)
            for i in range(P):
                bits = [j for j in range(P) if f.mask[i, j // 32] >> (j % 32) & 1]
                if i >= n:
                    assert f.token[i] == -1 and bits == [i] and f.pos[i] == prefix
                    continue
                # ancestors through the TREE's parent pointers, mapped to flat
                anc, v = [], f.node[i]
                while v >= 0:
                    anc.append(f.node.index(v))
                    v = t.parent[v]
                assert sorted(anc) == bits
                assert max(bits) == i                     # lower triangular
                assert len(bits) == t.depth[f.node[i]] + 1
                assert f.pos[i] - prefix == len(bits) - 1
            leaves = [i for i in range(n) if i not in f.parent[1:n]]
            assert f.n_leaves == len(leaves)
            for li, leaf in enumerate(leaves):
                path = [x for x in f.retrieve[li] if x >= 0]
                assert path[0] == 0 and path[-1] == leaf
                for a, c in zip(path, path[1:]):
                    assert f.parent[c] == a


# ---------------------------------------------------------------------------
# O7 greedy: P-f closed form and walk equivalence
# ---------------------------------------------------------------------------

def _flat_round(w, seed, m, noise_free=True):
    dr, drow, _, _ = build(w, seed=seed)
    out = []
    for b, t in enumerate(dr.trees):
        sel = O.rerank(t, m)
        f = O.flatten(t, sel, m + 1, 0, w.D)
        out.append((t, f, b))
    return dr, drow, out


def test_greedy_without_noise_follows_rank0_chain():
    w = small_workload(V=80, B=4, D=5, K_e=3, K_n=4, dtype="bf16")
    dr, drow, rows = _flat_round(w, 41, 25)
    g = np.random.default_rng(0)
    for t, f, b in rows:
        fresh = {}

        def target(i):
            v = f.node[i]
            if t.eslot[v] >= 0:
                return drow(t.depth[v] + 1, b, t.eslot[v])
            return fresh.setdefault(i, g.standard_normal(w.V))

        L, path, nxt = O.verify_greedy(f, lambda i: int(np.argmax(target(i))))
        # closed form: follow rank-0 children while they are selected
        chain, v = [0], 0
        while True:
            kids = [c for c in range(1, t.n) if t.parent[c] == v and
                    (t.key[c] >> (O.KEY_SRC_SHIFT - O.RANK_BITS * t.depth[c])) & O.MAX_RANK == 0]
            if not kids or kids[0] not in f.node:
                break
            v = kids[0]
            chain.append(f.node.index(v))
        assert L == len(chain) - 1
        assert path == chain
        assert nxt == int(np.argmax(target(chain[-1])))


def test_greedy_paths_equal_child_walk_when_siblings_distinct():
    w = small_workload(V=12, B=6, D=4, K_e=2, K_n=3)
    dr, drow, rows = _flat_round(w, 43, 12)
    g = np.random.default_rng(5)
    for t, f, b in rows:
        n = len([x for x in f.node if x >= 0])
        amax = g.integers(0, w.V, size=n)
        # bias towards matches so that walks go deep
        for i in range(1, n):
            if g.random() < 0.6:
                amax[f.parent[i]] = f.token[i]
        L, path, nxt = O.verify_greedy(f, lambda i: int(amax[i]))
        u, walk = 0, [0]
        while True:
            nxt_c = [c for c in range(1, n) if f.parent[c] == u and f.token[c] == amax[u]]
            if not nxt_c:
                break
            u = nxt_c[0]
            walk.append(u)
        assert path == walk and L == len(walk) - 1 and nxt == amax[walk[-1]]


# ---------------------------------------------------------------------------
# O8 stochastic: P-g special case, P-h textbook chain, P-i tree losslessness
# ---------------------------------------------------------------------------

def test_t1_target_equal_draft_accepts_first_child():
    w = small_workload(V=60, B=4, D=4, K_e=3, K_n=3, dtype="bf16")
    dr, drow, rows = _flat_round(w, 51, 20)
    g = np.random.default_rng(1)
    for t, f, b in rows:
        def target(i):
            v = f.node[i]
            if t.eslot[v] >= 0:
                return drow(t.depth[v] + 1, b, t.eslot[v])
            return np.zeros(w.V)

        def qrow(i):
            v = f.node[i]
            return drow(t.depth[v] + 1, b, t.eslot[v])

        for _ in range(5):
            U = g.random((len(f.node), 2))
            U[:, 0] = np.minimum(U[:, 0], 0.999999)
            L, path, _ = O.verify_stochastic(f, target, qrow, 1.0, U)
            Lg, pg, _ = O.verify_greedy(f, lambda i: int(np.argmax(target(i))))
            assert path == pg and L == Lg


def _mk_flat(tokens, parents):
    n = len(tokens)
    depth = [0] * n
    for i in range(1, n):
        depth[i] = depth[parents[i]] + 1
    return O.Flat(list(range(n)), list(tokens), list(parents), depth,
                  np.zeros((n, 1), np.uint32), np.zeros((1, 1), np.int32), 0, depth)


def _dist(g, V, floor=0.02):
    p = g.dirichlet(np.ones(V))
    p = (1 - floor * V) * p + floor
    return p / p.sum()


def test_chain_speculative_sampling_textbook():
    """One child drawn from q: P(accept) = sum min(p, q) and the first emitted
    token follows p (EAGLE-2 explainer, ledger section)."""
    V, N = 16, 60000
    g = np.random.default_rng(7)
    p, q = _dist(g, V), _dist(g, V)
    lp, lq = np.log(p), np.log(q)
    counts = np.zeros(V)
    acc = 0
    for _ in range(N):
        x = int(g.choice(V, p=q))
        f = _mk_flat([0, x], [-1, 0])
        U = g.random((2, 2))
        L, path, nxt = O.verify_stochastic(f, lambda i: lp, lambda i: lq, 1.0, U)
        first = x if L >= 1 else nxt
        acc += L
        counts[first] += 1
    assert stats.chisquare(counts, p * N).pvalue > 1e-3
    pa = np.minimum(p, q).sum()
    assert abs(acc / N - pa) < 4 * math.sqrt(pa * (1 - pa) / N)


@functools.lru_cache(maxsize=None)
def _cond(seed, ctx, V, floor):
    g = synth.keyed(991, seed, len(ctx), *ctx)
    return _dist(g, V, floor)


def _lossless_trial_counts(N, V, sampled, seed=3, proposal="draft"):
    """Joint counts of the first two emitted tokens over N verify calls on a
    depth-2 tree: 3 root children, 2 children under each.  Children are drawn
    i.i.d. from the draft distribution (sampled) or are its top-k tokens."""
    g = np.random.default_rng(seed)
    p = lambda ctx: _cond(seed, ctx, V, 0.03)
    q = lambda ctx: _cond(seed + 1000, ctx, V, 0.01)
    lp = functools.lru_cache(maxsize=None)(lambda ctx: np.log(p(ctx)))
    lq = functools.lru_cache(maxsize=None)(lambda ctx: np.log(q(ctx)))
    counts = np.zeros((V, V))
    for _ in range(N):
        tokens, parents, ctxs = [0], [-1], [()]
        lvl1 = []
        q0 = q(())
        kids = g.choice(V, size=3, p=q0) if sampled else np.argsort(-q0, kind="stable")[:3]
        for x in kids:
            tokens.append(int(x)); parents.append(0); ctxs.append((int(x),))
            lvl1.append(len(tokens) - 1)
        for u in lvl1:
            qu = q(ctxs[u])
            kk = g.choice(V, size=2, p=qu) if sampled else np.argsort(-qu, kind="stable")[:2]
            for x in kk:
                tokens.append(int(x)); parents.append(u); ctxs.append(ctxs[u] + (int(x),))
        f = _mk_flat(tokens, parents)
        U = g.random((len(tokens), 2))
        L, path, nxt = O.verify_stochastic(f, lambda i: lp(ctxs[i]), lambda i: lq(ctxs[i]), 1.0, U,
                                           proposal=proposal)
        emitted = [tokens[i] for i in path[1:]] + [nxt]
        if len(emitted) < 2:       # the next round starts from exact target sampling
            emitted.append(int(g.choice(V, p=p((emitted[0],)))))
        counts[emitted[0], emitted[1]] += 1
    expect = np.array([[p(())[a] * p((a,))[c] for c in range(V)] for a in range(V)])
    return counts, expect


def _assert_follows_target(counts, expect, N):
    assert stats.chisquare(counts.ravel(), expect.ravel() * N).pvalue > 1e-3
    assert stats.chisquare(counts.sum(1), expect.sum(1) * N).pvalue > 1e-3


@pytest.mark.slow
def test_tree_speculative_sampling_is_lossless_with_sampled_children():
    """Children drawn i.i.d. from q, no pruning, q-proposal rule: the first two
    emitted tokens follow the target's joint distribution (losslessness
    section) on a 16-token vocabulary."""
    N, V = 100000, 16
    counts, expect = _lossless_trial_counts(N, V, sampled=True, proposal="draft")
    _assert_follows_target(counts, expect, N)


@pytest.mark.slow
def test_point_mass_walk_is_lossless_on_topk_children():
    """The trees the library builds: deterministic top-k children, each
    verified as a point-mass proposal.  The first two emitted tokens follow
    the target's joint distribution (losslessness section), V = 16."""
    N, V = 100000, 16
    counts, expect = _lossless_trial_counts(N, V, sampled=False, proposal="point")
    _assert_follows_target(counts, expect, N)


@pytest.mark.slow
def test_point_mass_walk_is_lossless_with_sampled_children():
    """Point-mass verification does not depend on how the candidates were
    chosen: sampled children give the target's distribution too."""
    N, V = 50000, 16
    counts, expect = _lossless_trial_counts(N, V, sampled=True, proposal="point", seed=4)
    _assert_follows_target(counts, expect, N)


@pytest.mark.slow
def test_negative_control_topk_children_are_biased():
    """Deterministic top-k children under the q-proposal rule are not exactly
    lossless (the reason top-k trees take point-mass proposals); the bias is
    detectable on the same 16-token vocabulary."""
    N, V = 50000, 16
    counts, expect = _lossless_trial_counts(N, V, sampled=False, proposal="draft")
    assert stats.chisquare(counts.sum(1), expect.sum(1) * N).pvalue < 1e-6


def test_inverse_cdf_sampling_exact_cases():
    p = np.array([0.25, 0.0, 0.5, 0.25])
    assert O.sample_inverse_cdf(p, 0.0) == 0
    assert O.sample_inverse_cdf(p, 0.2499) == 0
    assert O.sample_inverse_cdf(p, 0.25) == 2          # strictly greater than u*sum
    assert O.sample_inverse_cdf(p, 0.7499) == 2
    assert O.sample_inverse_cdf(p, 0.75) == 3
    assert O.sample_inverse_cdf(p * 4.0, 0.99) == 3    # unnormalised input


@pytest.mark.parametrize("T", [1.0, 1.6])
def test_residual_after_rejection(T):
    """A rejected child with p = (.5,.5), q = (.9,.1): the residual puts all
    mass on token 1, so the emission is token 1 for any uniform.  Logits are
    T log p and T log q, so softmax(logits / T) gives those p and q."""
    lp, lq = T * np.log([0.5, 0.5]), T * np.log([0.9, 0.1])
    f = _mk_flat([0, 0], [-1, 0])
    for u1 in (0.0, 0.3, 0.99):
        U = np.array([[0.0, u1], [0.99, 0.0]])      # 0.99 > p/q = 0.556: reject
        L, path, nxt = O.verify_stochastic(f, lambda i: lp, lambda i: lq, T, U)
        assert L == 0 and nxt == 1
    U = np.array([[0.0, 0.0], [0.5, 0.0]])          # 0.5 < 0.556: accept
    L, path, nxt = O.verify_stochastic(f, lambda i: lp, lambda i: lq, T, U)
    assert L == 1 and path == [0, 1]


def test_graft_tail_anchor_rule():
    """Tail-only grafting hangs the template off the deepest selected node,
    ties to the higher value, then the smaller key."""
    t = O.new_tree(5)
    a = t.add(1, 0, 1, -0.1, -0.1, O.key_child(0, 0, 0))
    b = t.add(2, 0, 1, -0.5, -0.5, O.key_child(0, 0, 1))
    c = t.add(3, a, 2, -0.3, -0.2, O.key_child(t.key[a], 1, 0))
    d = t.add(4, a, 2, -0.2, -0.1, O.key_child(t.key[a], 1, 1))
    e = t.add(6, b, 2, -0.2, -0.1, O.key_child(t.key[b], 1, 0))
    assert O.graft_tail_anchor(t, [a, b, c, d, e]) == d      # d and e tie on S; d's key is smaller
    assert O.graft_tail_anchor(t, [a, b, c]) == c
    assert O.graft_tail_anchor(t, [a, b]) == a
    assert O.graft_tail_anchor(t, []) == 0


def test_graft_template_under_an_anchor():
    """Template under a depth-2 anchor: chain c starts at M[x_anchor][c] and
    continues with successor 0; depths continue from the anchor; keys carry
    the retrieval bit and sort after draft keys of the same depth; levels
    past the key's depth limit are not built."""
    V = 20
    M = (np.arange(V)[:, None] * 3 + np.arange(4)[None, :] + 1) % V
    t = O.new_tree(5)
    a = t.add(1, 0, 1, -0.1, -0.1, O.key_child(0, 0, 0))
    d = t.add(4, a, 2, -0.2, -0.1, O.key_child(t.key[a], 1, 1))
    added = O.graft_template(t, M, 5, 3, 2, anchor=d)
    assert len(added) == 5
    n1, n2, n3, n4, n5 = added
    assert [t.token[n] for n in added] == [M[4, 0], M[4, 1], M[M[4, 0], 0], M[M[4, 1], 0],
                                           M[M[M[4, 0], 0], 0]]
    assert [t.parent[n] for n in added] == [d, d, n1, n2, n3]
    assert [t.depth[n] for n in added] == [3, 3, 4, 4, 5]
    for n in added:
        assert (t.key[n] >> 58) & 1 == 1 and O.key_depth(t.key[n]) == t.depth[n]
        assert t.src[n] == 1 and t.S[n] == -math.inf
    draft3 = O.key_child(t.key[d], 2, 7)                     # a draft node at depth 3
    assert draft3 < t.key[n1] and draft3 < t.key[n2]
    # an anchor at depth 10: only one level (depth 11) fits under the key
    t2 = O.new_tree(5)
    p = 0
    for lvl in range(1, 11):
        p = t2.add(1, p, lvl, -0.1 * lvl, -0.1, O.key_child(t2.key[p], lvl - 1, 0))
    added = O.graft_template(t2, M, 8, 3, 2, anchor=p)
    assert len(added) == 2 and all(t2.depth[n] == 11 for n in added)


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("mode", ["retrieval", "point"])
def test_point_mass_children_thresholds(mode, T):
    """Point-mass proposals (Graft retrieval children, or every child in the
    "point" mode): the k-th is accepted iff
    U < p(x_k) / (1 - p(x_1) - .. - p(x_{k-1})), i.e. from p with the rejected
    tokens removed and renormalised; the emission then excludes them.  No
    draft row is read.  At temperature T the logits are T log p, so that
    softmax(logits / T) = p and the thresholds are the same."""
    p = np.array([0.1, 0.2, 0.3, 0.15, 0.25])
    lp = T * np.log(p)
    f = _mk_flat([0, 2, 4, 1], [-1, 0, 0, 0])      # root, then children with tokens 2, 4, 1
    if mode == "retrieval":
        ret, prop = [False, True, True, True], "draft"
    else:
        ret, prop = None, "point"
    no_q = lambda i: (_ for _ in ()).throw(AssertionError("no draft row is needed"))
    eps = 1e-9
    # first child: threshold p(2) = 0.3
    for u, want in ((0.3 - eps, 1), (0.3 + eps, None)):
        U = np.array([[0.0, 0.0], [u, 0.0], [0.999, 0.0], [0.999, 0.0]])
        L, path, _ = O.verify_stochastic(f, lambda i: lp, no_q, T, U, retrieval=ret, proposal=prop)
        assert (path[1] if L else None) == want
    # second child after rejecting token 2: threshold 0.25 / 0.7
    t2 = 0.25 / 0.7
    for u, want in ((t2 - eps, 2), (t2 + eps, None)):
        U = np.array([[0.0, 0.0], [0.999, 0.0], [u, 0.0], [0.999, 0.0]])
        L, path, _ = O.verify_stochastic(f, lambda i: lp, no_q, T, U, retrieval=ret, proposal=prop)
        assert (path[1] if L else None) == want
    # third child after rejecting 2 and 4: threshold 0.2 / 0.45
    t3 = 0.2 / 0.45
    for u, want in ((t3 - eps, 3), (t3 + eps, None)):
        U = np.array([[0.0, 0.0], [0.999, 0.0], [0.999, 0.0], [u, 0.0]])
        L, path, _ = O.verify_stochastic(f, lambda i: lp, no_q, T, U, retrieval=ret, proposal=prop)
        assert (path[1] if L else None) == want
    # all rejected: the emission draws from {0: 0.1, 3: 0.15} renormalised
    for u1, want in ((0.0, 0), (0.4 - eps, 0), (0.4 + eps, 3), (0.999, 3)):
        U = np.array([[0.0, u1], [0.999, 0.0], [0.999, 0.0], [0.999, 0.0]])
        L, path, nxt = O.verify_stochastic(f, lambda i: lp, no_q, T, U, retrieval=ret, proposal=prop)
        assert L == 0 and nxt == want


def test_point_mass_duplicate_siblings():
    """Point-mass children with a repeated token: once token 2 is rejected it
    has no mass left, so its duplicate is rejected for any uniform, the next
    child's threshold is p(4) / (1 - p(2)), and the emission leaves token 2
    out once (threshold 0.1 / 0.45 between tokens 0 and 1)."""
    p = np.array([0.1, 0.2, 0.3, 0.15, 0.25])
    lp = np.log(p)
    f = _mk_flat([0, 2, 2, 4], [-1, 0, 0, 0])
    no_q = lambda i: (_ for _ in ()).throw(AssertionError("no draft row is needed"))
    eps = 1e-9
    for u2 in (0.0, 0.5):
        U = np.array([[0.0, 0.0], [0.999, 0.0], [u2, 0.0], [0.999, 0.0]])
        L, path, _ = O.verify_stochastic(f, lambda i: lp, no_q, 1.0, U, proposal="point")
        assert L == 0
    t3 = 0.25 / 0.7
    for u, want in ((t3 - eps, 3), (t3 + eps, None)):
        U = np.array([[0.0, 0.0], [0.999, 0.0], [0.0, 0.0], [u, 0.0]])
        L, path, _ = O.verify_stochastic(f, lambda i: lp, no_q, 1.0, U, proposal="point")
        assert (path[1] if L else None) == want
    # emission over {0: .1, 1: .2, 3: .15} / 0.45
    for u1, want in ((0.1 / 0.45 - eps, 0), (0.1 / 0.45 + eps, 1), (0.3 / 0.45 + eps, 3)):
        U = np.array([[0.0, u1], [0.999, 0.0], [0.0, 0.0], [0.999, 0.0]])
        L, path, nxt = O.verify_stochastic(f, lambda i: lp, no_q, 1.0, U, proposal="point")
        assert L == 0 and nxt == want


def _mixed_trial_counts(N, V, seed=5):
    """Joint counts of the first two emitted tokens over N verify calls on a
    tree that mixes sampled draft children and deterministic retrieval nodes:
    2 draft children of the root drawn from q, then 2 fixed retrieval children,
    each retrieval child with one fixed retrieval child below it."""
    g = np.random.default_rng(seed)
    p = lambda ctx: _cond(seed, ctx, V, 0.03)
    q = lambda ctx: _cond(seed + 1000, ctx, V, 0.01)
    counts = np.zeros((V, V))
    for _ in range(N):
        tokens, parents, ctxs, ret = [0], [-1], [()], [False]
        for x in g.choice(V, size=2, p=q(())):
            tokens.append(int(x)); parents.append(0); ctxs.append((int(x),)); ret.append(False)
        lvl1 = []
        for x in (1, 3):                            # fixed retrieval tokens
            tokens.append(x); parents.append(0); ctxs.append((x,)); ret.append(True)
            lvl1.append(len(tokens) - 1)
        for u in lvl1:
            x = (tokens[u] + 2) % V
            tokens.append(x); parents.append(u); ctxs.append(ctxs[u] + (x,)); ret.append(True)
        f = _mk_flat(tokens, parents)
        U = g.random((len(tokens), 2))
        L, path, nxt = O.verify_stochastic(f, lambda i: np.log(p(ctxs[i])),
                                           lambda i: np.log(q(ctxs[i])), 1.0, U, retrieval=ret)
        emitted = [tokens[i] for i in path[1:]] + [nxt]
        if len(emitted) < 2:
            emitted.append(int(g.choice(V, p=p((emitted[0],)))))
        counts[emitted[0], emitted[1]] += 1
    expect = np.array([[p(())[a] * p((a,))[c] for c in range(V)] for a in range(V)])
    return counts, expect


@pytest.mark.slow
def test_point_mass_retrieval_nodes_keep_the_tree_lossless():
    """Sampled draft children plus deterministic retrieval nodes (point-mass
    proposals) under the rule: the first two emitted tokens still follow the
    target's joint distribution."""
    N, V = 60000, 16
    counts, expect = _mixed_trial_counts(N, V)
    assert stats.chisquare(counts.ravel(), expect.ravel() * N).pvalue > 1e-3
    assert stats.chisquare(counts.sum(1), expect.sum(1) * N).pvalue > 1e-3


# ---------------------------------------------------------------------------
# O9 CAST: P-j Theorem 4.1, P-k anchor scan, P-l select()
# ---------------------------------------------------------------------------

def test_select_row_hand_cases():
    L, M = 256, 16
    assert O.cast_select_row(0, L, M) == 0
    assert O.cast_select_row(255, L, M) == 0
    assert O.cast_select_row(256, L, M) == 1
    assert O.cast_select_row(3 * 256 - 1, L, M) == 2
    assert O.cast_select_row(15 * 256, L, M) == 15
    assert O.cast_select_row(10 ** 6, L, M) == 15


def test_anchor_scan_equals_first_drop_on_concave_utility():
    g = np.random.default_rng(4)
    for _ in range(200):
        k = int(g.integers(1, 20))
        marg = np.sort(g.exponential(1.0, size=k))[::-1]
        u = np.concatenate([[0.0], np.cumsum(marg)])
        c = np.concatenate([[0.0], np.cumsum(g.uniform(0.5, 1.5, size=k))])
        C = float(g.uniform(0.0, 2.0))
        # first-drop: keep item k while its own marginal per unit cost >= C
        n = 1
        while n < k and (u[n + 1] - u[n]) / (c[n + 1] - c[n]) >= C:
            n += 1
        if n < k and all((u[j + 1] - u[j]) / (c[j + 1] - c[j]) <= (u[j] - u[j - 1]) / (c[j] - c[j - 1])
                         for j in range(1, k)):
            assert O.anchor_scan(u, c, C, k) == n


def test_anchor_scan_looks_past_a_plateau():
    u = np.array([0.0, 1.0, 1.1, 1.2, 3.0])
    c = np.array([0.0, 1.0, 2.0, 3.0, 4.0])
    # marginals from anchor 1: 0.1, 0.1, (3.0-1.0)/3 = 0.667
    assert O.anchor_scan(u, c, 0.5, 4) == 4
    assert O.anchor_scan(u, c, 0.7, 4) == 1
    assert O.anchor_scan(u, c, 0.0, 4) == 4
    assert O.anchor_scan(u, c, 0.5, 0) == 0


def _cast_params(w, C1, C2, C3):
    S_T, S_D = synth.cost_tables(w)
    cs = w.cast
    return dict(S_T=S_T, S_D=S_D, L=cs.L, M=cs.M, C1=list(C1), C2=C2, C3=list(C3), R=cs.R)


def test_theorem_4_1_cast_reduces_to_fixed_topk():
    """With c_k = lam*k + delta and C1 = sum_b v_b(K)/(B*lam) the width rule keeps
    exactly K per layer (CAST notes, key design 2, Theorem 4.1); with per-row
    C3 = v_(m)/lam the verify count is m, and C2 = -inf never stops early.
    The whole round then equals fixed EAGLE-2.  The theorem's equality is taken
    with a relative slack of 1e-9 to absorb float rounding (reading)."""
    lam = 0.02
    w = small_workload(V=500, B=3, D=4, K_e=3, K_n=4, m=14, dtype="bf16",
                       cast=CastSpec(lam=lam, delta=1.0))
    dr_fixed, drow, arena, roots = build(w, seed=61)
    C1 = []
    for d in range(1, w.D + 1):
        tot = 0.0
        for t in dr_fixed.trees:
            layer = O.order_by_value(t, [i for i in range(t.n) if t.depth[i] == d])
            tot += math.exp(t.S[layer[w.K_e - 1]])
        C1.append(tot / (w.B * lam) * (1 - 1e-9))
    C3 = []
    for t in dr_fixed.trees:
        order = O.order_by_value(t, range(1, t.n))
        C3.append(math.exp(t.S[order[w.m - 1]]) / lam * (1 - 1e-9))
    cast = _cast_params(w, C1, -math.inf, C3)
    # a width cap above K: the threshold alone must stop at K
    dr_cast = O.draft_phase(drow, w.B, roots, w.D, w.K_e + 1, w.K_n, cast=cast)
    assert dr_cast.widths == [w.K_e] * w.D and dr_cast.depth_built == w.D
    for a, b_ in zip(dr_fixed.trees, dr_cast.trees):
        assert a.token == b_.token and a.parent == b_.parent and a.S == b_.S and a.key == b_.key
    cv = O.cast_verify_costs(cast["S_T"], 0, cast["L"], cast["M"], w.m + 5)
    for b, t in enumerate(dr_cast.trees):
        assert O.cast_verify_count(t, cv, C3[b], w.m + 5) == w.m
    # and one notch above the theorem's C1 drops the K-th node somewhere
    cast_hi = _cast_params(w, [c * (1 + 1e-6) for c in C1], -math.inf, C3)
    assert O.draft_phase(drow, w.B, roots, w.D, w.K_e, w.K_n, cast=cast_hi).widths[0] < w.K_e


def test_cast_depth_gate_limits():
    w = small_workload(V=300, B=2, D=5, K_e=3, K_n=3, dtype="bf16", cast=CastSpec())
    _, drow, _, roots = build(w, seed=71)
    run = lambda C2: O.draft_phase(drow, w.B, roots, w.D, w.K_e, w.K_n,
                                   cast=_cast_params(w, [0.0] * w.D, C2, [0.0] * w.B))
    assert run(0.0).depth_built == w.D          # score is never negative
    assert run(1e9).depth_built == 1            # stops after the first layer
    depths = [run(c).depth_built for c in (0.0, 0.01, 0.1, 0.5, 2.0, 1e9)]
    assert depths == sorted(depths, reverse=True)


def test_cast_depth_gate_fifo_hand_example():
    """Hand-computed gate with R = 2.  Rows are logs of exact probabilities
    with one candidate kept per layer (C1 = inf), so the kept utility of layer i
    is a product of known numbers and every gate score is exact arithmetic."""
    V = 4
    probs = {1: [0.8, 0.1, 0.06, 0.04], 2: [0.5, 0.3, 0.1, 0.1],
             3: [0.9, 0.05, 0.03, 0.02], 4: [0.7, 0.1, 0.1, 0.1]}
    drow = lambda layer, b, j: np.log(np.array(probs[layer]))
    S_T = np.zeros((1, 5), np.float32); S_T[0, 1:] = 1.0
    S_D = np.zeros((1, 5), np.float32); S_D[0, 1:] = [2.0, 3.0, 4.0, 5.0]   # c_k = k + 1
    # u1 = .8, u2 = .4, u3 = .36, u4 = .252 (products along rank-0 chain)
    # layer1: A={1}        score = 1 * .8/2 = .4
    # layer2: A={1,.5}     score = .75 * .4/2 = .15
    # layer3: A={.5,.9}    score = .7 * .36/2 = .126   (R = 2 evicts the initial 1)
    def depth(C2):
        cast = dict(S_T=S_T, S_D=S_D, L=256, M=1, C1=[math.inf] * 4, C2=C2, C3=[0.0], R=2)
        return O.draft_phase(drow, 1, [0], 4, 2, 2, cast=cast).depth_built
    assert depth(0.41) == 1
    assert depth(0.39) == 2 and depth(0.151) == 2
    assert depth(0.149) == 3 and depth(0.127) == 3
    assert depth(0.125) == 4


def cast_lookup_example():
    """The hand-worked CAST round of test_cast_cost_lookup_hand_example: inputs
    and the values worked out by hand (also run on the GPU)."""
    V, B, D, K_e, K_n, m_max, prefix = 4, 2, 4, 3, 2, 8, 4
    probs = {1: [0.5, 0.3, 0.15, 0.05], 2: [0.7, 0.2, 0.06, 0.04],
             3: [0.5, 0.3, 0.12, 0.08], 4: [0.4, 0.3, 0.2, 0.1]}
    draft = np.zeros((D, B, K_e, V), np.float32)
    for d in range(1, D + 1):
        draft[d - 1] = np.log(np.array(probs[d])).astype(np.float32)
    k = np.arange(1, 9)
    S_T = np.zeros((4, 9), np.float32)
    S_D = np.zeros((4, 9), np.float32)
    S_T[0, 1:] = 1 + 0.2 * (k - 1)
    S_T[1, 1:] = 2 * (1 + 0.25 * (k - 1))
    S_T[2, 1:] = 1 + 0.5 * (k - 1)
    S_T[3, 1:] = 1 + 1.0 * (k - 1)
    S_D[0, 1:] = [0.5, 0.5, 0.8, 1.1, 1.4, 1.7, 2.0, 2.3]
    S_D[1, 1:] = 0.2 + 0.2 * k
    S_D[2, 1:] = 0.3 * k
    S_D[3, 1:] = 0.5 * k
    cast = dict(S_T=S_T, S_D=S_D, L=2, M=4, C1=[2.0, 3.0, 0.8, 0.8], C2=1.0, C3=[0.56, 0.32], R=3)
    shape = dict(V=V, B=B, D=D, K_e=K_e, K_n=K_n, m_max=m_max, prefix=prefix)
    expect = dict(widths=[2, 1, 2], depth_built=3, m_rows=[3, 5])
    return shape, draft, cast, expect


def test_cast_cost_lookup_hand_example():
    """CAST's cost lookup worked by hand (CAST notes, key designs 1, 2 and 4).

    Draft rows are logs of exact probabilities that depend on the layer only,
    so both requests grow the same tree and every value is a product of the
    listed numbers.  K_n = 2 children per node, width cap 3, D_max = 4.
    Grid step L = 2 over M = 4 rows, so select(c) = row min(c // 2, 3); the
    context prefix is 4 tokens.

    Width costs c_k = S_D[r][k] / S_T[r][1]:
      row 0: 0.5, 0.5, 0.8, ...   (c_2 = c_1: the second node costs nothing)
      row 1: 0.2, 0.3, 0.4, ...   (S_T[1][1] = 2)
      row 2: 0.3, 0.6, 0.9, ...

    Layer 1, context 0 (tree tokens fed so far; neither the root nor the
    prompt counts) -> row 0.  Candidates 0.5, 0.3: u = 0.5, 0.8.  The cost
    does not rise from k = 1 to 2 while the utility does, so the anchor moves:
    n_1 = 2.  (Row 2, reached if the 4 prompt tokens counted, has marginal
    0.3 / 0.3 = 1.0 < C1 = 2 and gives n_1 = 1; skipping the zero-cost step
    also gives n_1 = 1.)
    Layer 2, context 2 -> row 1.  Children of 0.5 and 0.3 under row
    (0.7, 0.2): 0.35, 0.21, 0.10, 0.06; u = 0.35, 0.56, 0.66 (cap 3).
    Marginals 0.21 / 0.1 = 2.1 and 0.31 / 0.2 = 1.55 are below C1 = 3: n_2 = 1.
    Layer 3, context 3 -> row 1.  Children of 0.35 under (0.5, 0.3): 0.175,
    0.105; marginal 0.105 / 0.1 = 1.05 >= C1 = 0.8: n_3 = 2.  (Counting the
    root makes the context 4 -> row 2, marginal 0.105 / 0.3 = 0.35: n_3 = 1.)

    Depth gate (R = 3, C2 = 1): layer 1 score 1 * 0.8 / 0.5 = 1.6 (grow);
    layer 2 pushes 0.35 / 0.8 = 0.4375, score 0.71875 * 0.35 / 0.2 = 1.258
    (grow); layer 3 pushes 0.28 / 0.35 = 0.8, score
    (1 + 0.4375 + 0.8) / 3 * 0.28 / 0.3 = 0.696 < 1: stop with 3 layers of 4.

    Verify count: the cost context is the prefix, 4 -> row 2 of S_T,
    c_k = S_T[2][k] / S_T[2][1] = 1 + 0.5 (k - 1).  Node values in order:
    0.5, 0.35, 0.3, 0.21, 0.175, 0.105, 0.10, 0.06; with a linear cost the
    anchor scan keeps node k while v_(k) / 0.5 >= C3.  Request 0 (C3 = 0.56,
    keep v >= 0.28): m = 3.  Request 1 (C3 = 0.32, keep v >= 0.16): m = 5.
    (Row 0 of S_T, slope 0.2, gives 5 and 7 (keep v >= 0.112, v >= 0.064);
    S_D's row 2 read as the verify cost, slope 0.3, also gives 5 and 7.)
    """
    shape, draft, cast, expect = cast_lookup_example()
    B, m_max = shape["B"], shape["m_max"]
    out = O.run_round(B=B, V=shape["V"], dtype="f32", D=shape["D"], K_e=shape["K_e"],
                      K_n=shape["K_n"], m_max=m_max, root_tok=[0] * B, draft_raw=draft,
                      target_raw_fn=lambda dr, fl: np.zeros((B, m_max + 1, shape["V"]), np.float32),
                      temperature=np.zeros(B, np.float32), U=np.zeros((B, m_max + 1, 2), np.float32),
                      prefix=shape["prefix"], cast=cast)
    assert out["draft"].widths == expect["widths"]
    assert out["draft"].depth_built == expect["depth_built"]
    assert out["m_rows"].tolist() == expect["m_rows"]
    vals = sorted(math.exp(s) for s in out["draft"].trees[0].S[1:])[::-1]
    np.testing.assert_allclose(vals, [0.5, 0.35, 0.3, 0.21, 0.175, 0.105, 0.10, 0.06], rtol=1e-6)


def test_cast_verify_count_limits():
    w = small_workload(V=200, B=2, D=4, K_e=3, K_n=3, m=12, cast=CastSpec())
    dr, *_ = build(w, seed=81)
    S_T, _ = synth.cost_tables(w)
    cv = O.cast_verify_costs(S_T, 0, 256, 16, w.m)
    for t in dr.trees:
        assert O.cast_verify_count(t, cv, 0.0, w.m) == min(w.m, t.n - 1)
        assert O.cast_verify_count(t, cv, 1e9, w.m) == 1


# ---------------------------------------------------------------------------
# O10 Graft: P-m
# ---------------------------------------------------------------------------

def _graft_setup(seed=91, B=3, V=400):
    gs = GraftSpec()
    w = Workload("pin_graft", B=B, V=V, dtype="bf16", D=8, K_e=8, K_n=8, m=60,
                 verify="greedy", sigma=0.5, graft=gs)
    M0 = synth.succ_matrix0(w, seed)
    return w, M0


def test_succ_matrix0_rows_are_distinct_successors():
    w, M0 = _graft_setup(B=2, V=300)
    assert M0.shape == (2, 300, 8)
    assert M0.min() >= 0 and M0.max() < 300
    for b in range(2):
        assert all(len(set(r)) == 8 for r in M0[b].tolist())


def test_graft_stages_and_template_gather():
    w, M0 = _graft_setup()
    arena = synth.draft_arena(w, 5, 0)
    roots = synth.root_tokens(w, 5, 0)
    drow = lambda layer, b, j: O.decode(arena[layer - 1, b, j], w.dtype)
    base = O.draft_phase(drow, w.B, roots, w.D, w.K_e, w.K_n)
    gs = w.graft
    # c_d of each row at each checkpoint, from the unpruned tree
    cd = [[math.exp(max(t.S[i] for i in range(t.n) if t.depth[i] == d)) for d in gs.ck_depth]
          for t in base.trees]
    for stage in range(4):
        # pass the first `stage` checkpoints, fail the next one (stage 3: pass all)
        for b in range(w.B):
            tau = [cd[b][s] * (0.5 if s < stage else 2.0) for s in range(3)]
            graft = dict(ck_depth=gs.ck_depth, tau=tau, k_draft=gs.k_draft, K_max=gs.K_max)
            dr = O.draft_phase(drow, w.B, roots, w.D, w.K_e, w.K_n, graft=graft)
            want = gs.k_draft[stage] if stage < 3 else gs.K_max
            assert dr.k_draft[b] == want
            t = dr.trees[b]
            built = gs.ck_depth[stage] if stage < 3 else w.D
            assert max(t.depth) == built
            sel = O.rerank(t, dr.k_draft[b])
            M = M0[b].copy()
            added = O.graft_template(t, M, gs.K_max - len(sel), gs.tpl_depth, gs.tpl_width)
            assert len(sel) + len(added) == gs.K_max             # |T| = K_max always
            for k, u in enumerate(added):
                lvl, c = k // gs.tpl_width + 1, k % gs.tpl_width
                p = t.parent[u]
                assert t.depth[u] == lvl
                assert t.token[u] == M[t.token[p], c if lvl == 1 else 0]
                assert (p == 0) == (lvl == 1)
            f = O.flatten(t, sel + added, gs.K_max + 1, 0, 8)
            keys = [t.key[v] for v in f.node]
            assert keys == sorted(keys)


def test_graft_no_gate_equals_eagle2_top60():
    w, M0 = _graft_setup()
    arena = synth.draft_arena(w, 6, 0)
    roots = synth.root_tokens(w, 6, 0)
    drow = lambda layer, b, j: O.decode(arena[layer - 1, b, j], w.dtype)
    gs = w.graft
    graft = dict(ck_depth=gs.ck_depth, tau=[-math.inf] * 3, k_draft=gs.k_draft, K_max=gs.K_max)
    a = O.draft_phase(drow, w.B, roots, w.D, w.K_e, w.K_n, graft=graft)
    b_ = O.draft_phase(drow, w.B, roots, w.D, w.K_e, w.K_n)
    for ta, tb, kd in zip(a.trees, b_.trees, a.k_draft):
        assert kd == gs.K_max
        assert O.rerank(ta, kd) == O.rerank(tb, 60)


def test_succ_update_is_full_sort_last_writer_wins():
    V, k = 50, 8
    g = np.random.default_rng(9)
    M = g.integers(0, V, size=(V, k)).astype(np.int32)
    M_before = M.copy()
    flat_token = [7, 3, 9, 3, -1, 12]
    rows = {i: np.round(g.standard_normal(V) * 2) for i in range(6)}   # ties on purpose
    O.succ_update(M, flat_token, 6, lambda i: rows[i], k)
    assert M[3].tolist() == brute_sorted_ids(rows[3].tolist())[:k]     # position 3 wins over 1
    assert M[9].tolist() == brute_sorted_ids(rows[2].tolist())[:k]
    assert M[12].tolist() == brute_sorted_ids(rows[5].tolist())[:k]
    assert M[7].tolist() == M_before[7].tolist()                       # the root is not refreshed
    touched = {3, 9, 12}
    for v in range(V):
        if v not in touched:
            assert M[v].tolist() == M_before[v].tolist()

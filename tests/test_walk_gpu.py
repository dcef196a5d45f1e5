"""GPU tests of the T > 0 accept walk in ddt_tree_verify.

Losslessness (EAGLE-2 explainer, losslessness section: the output
distribution equals the target's, whatever the tree): on a 16-token
vocabulary, the first two emitted tokens of many verify calls are compared by
chi-square with the target's joint distribution p(a) p(c | a).  Target rows
are keyed by the token context of each flat position, so duplicate contexts
share one conditional.  The expected distribution comes from the inputs alone
(softmax of the fp32 target logits in fp64), never from the library.

  * point-mass proposals on the top-k trees the library itself builds
    (ddt_tree_expand .. ddt_tree_verify): lossless;
  * q-proposals on children drawn i.i.d. from the draft: lossless;
  * point-mass proposals on those sampled children: lossless;
  * negative control: q-proposals on deterministic top-k children are biased.

The give-up path of the walk's cross-workgroup wait: with a tiny spin limit
the waits run out, workgroup 0 finishes each request alone, every kernel
exits normally, the outcome equals the oracle's, and the wait counters are
back at 0 for the next call.
"""
import numpy as np
import pytest
import torch
from scipy import stats

from gen import configs
from oracle import ddt_oracle as O
from tests import harness as H

pytestmark = pytest.mark.gpu

V = 16


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    from dynamic_draft_tree_row_amd import _lib
    _lib.load()      # raises if the library was not built: no fallback


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# context-keyed distributions on a 16-token vocabulary
# ---------------------------------------------------------------------------

def _dist(seed, ctx, floor):
    g = np.random.default_rng([seed, len(ctx), *ctx])
    p = g.dirichlet(np.ones(V))
    p = (1 - floor * V) * p + floor
    return p / p.sum()


class Model:
    """fp32 logits log p(. | ctx) of the target and log q(. | ctx) of the draft
    for contexts of up to two tokens, and the distributions the library sees
    (softmax of those fp32 logits, in fp64)."""

    def __init__(self, seed):
        def table(s, floor):
            t0 = np.log(_dist(s, (), floor)).astype(np.float32)
            t1 = np.stack([np.log(_dist(s, (a,), floor)) for a in range(V)]).astype(np.float32)
            t2 = np.stack([[np.log(_dist(s, (a, c), floor)) for c in range(V)]
                           for a in range(V)]).astype(np.float32)
            return t0, t1, t2
        self.lp0, self.lp1, self.lp2 = table(seed, 0.03)
        self.lq0, self.lq1, self.lq2 = table(seed + 1000, 0.01)
        sm = lambda x: np.exp(x - x.max(-1, keepdims=True)) / np.exp(x - x.max(-1, keepdims=True)).sum(-1, keepdims=True)
        self.p0 = sm(self.lp0.astype(np.float64))
        self.p1 = sm(self.lp1.astype(np.float64))
        self.q0 = sm(self.lq0.astype(np.float64))
        self.q1 = sm(self.lq1.astype(np.float64))

    def joint(self):
        return self.p0[:, None] * self.p1


def _emitted(rng, model, tok, acc_len, acc_path, nxt):
    """First two emitted tokens per request: the accepted path's tokens, then
    the next token; a walk that accepted nothing is continued by exact target
    sampling, as the next round would start."""
    B = acc_len.shape[0]
    first = np.where(acc_len >= 1, tok[np.arange(B), np.maximum(acc_path[:, 1], 0)], nxt)
    second = np.where(acc_len >= 2, tok[np.arange(B), np.maximum(acc_path[:, 2], 0)], nxt)
    none = acc_len == 0
    if none.any():
        u = rng.random(int(none.sum()))
        cdf = np.cumsum(model.p1[first[none]], axis=1)
        second = second.copy()
        second[none] = np.minimum((u[:, None] >= cdf).sum(1), V - 1)
    return first, second


def _chi2_joint(counts, model):
    N = counts.sum()
    exp = model.joint() * N
    return (stats.chisquare(counts.ravel(), exp.ravel()).pvalue,
            stats.chisquare(counts.sum(1), exp.sum(1)).pvalue)


# ---------------------------------------------------------------------------
# trees the library builds (top-k children), point-mass proposals
# ---------------------------------------------------------------------------

def _library_topk_counts(model, calls, B, seed, proposal):
    from dynamic_draft_tree_row_amd import api
    w = configs.Workload("walk_chi2", B=B, V=V, dtype="f32", D=2, K_e=3, K_n=3, m=8,
                         verify="t1", sigma=0.0, proposal=proposal)
    run = H.runner_for(w)
    # draft rows: layer 1 from q(.), layer 2 slot j from q(. | token of frontier slot j)
    fr = O.topk_ids(model.lq0.astype(np.float64), 3)        # layer-1 frontier = the root's top 3
    arena = np.zeros((2, B, 3, V), np.float32)
    arena[0, :, :] = model.lq0
    for j in range(3):
        arena[1, :, j] = model.lq1[fr[j]]
    # the same tree in the oracle: flat tokens give every position's context
    rows = lambda layer, b, j: arena[layer - 1, 0, j].astype(np.float64)
    dr = O.draft_phase(rows, 1, [0], 2, 3, 3)
    t = dr.trees[0]
    sel = O.rerank(t, 8)
    f = O.flatten(t, sel, 9, 0, 2)
    n = len([x for x in f.node if x >= 0])
    ctxs = []
    for i in range(n):
        path, j = [], i
        while j > 0:
            path.append(f.token[j]); j = f.parent[j]
        ctxs.append(tuple(reversed(path)))
    target = np.zeros((B, 9, V), np.float32)
    for i, c in enumerate(ctxs):
        target[:, i] = model.lp0 if not c else (model.lp1[c[0]] if len(c) == 1 else model.lp2[c[0], c[1]])
    arena_d = torch.from_numpy(arena).cuda()
    target_d = torch.from_numpy(target).cuda()
    roots = torch.zeros(B, dtype=torch.int32, device="cuda")
    T = torch.ones(B, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(seed)
    counts = np.zeros((V, V))
    tok = np.array(f.token[:n] + [0] * (9 - n), np.int64)[None, :].repeat(B, 0)
    for call in range(calls):
        run.draft(arena_d, roots)
        U = torch.from_numpy(rng.random((B, 9, 2), dtype=np.float32)).cuda()
        run.verify(target_d, arena_d, T, U, proposal=proposal)
        torch.cuda.synchronize()
        if call == 0:
            got = run.flat.token.cpu().numpy()
            assert (got[:, :n] == np.array(f.token[:n])[None, :]).all(), "library tree differs from the oracle's"
        a, c = _emitted(rng, model, tok, run.accept_len.cpu().numpy(), run.accept_path.cpu().numpy(),
                        run.next_token.cpu().numpy())
        np.add.at(counts, (a, c), 1)
    return counts


def test_point_mass_walk_lossless_on_library_trees():
    model = Model(21)
    counts = _library_topk_counts(model, calls=25, B=4096, seed=5, proposal="point")
    pj, pm = _chi2_joint(counts, model)
    say(f"point-mass, library top-k trees: N={int(counts.sum())} p(joint)={pj:.3g} p(first)={pm:.3g}")
    assert pj > 1e-3 and pm > 1e-3


# ---------------------------------------------------------------------------
# trees written by hand into the tree state: sampled or top-k children
# ---------------------------------------------------------------------------

P_MAN = 10
PARENT = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3], np.int32)
DEPTH = np.array([0, 1, 1, 1, 2, 2, 2, 2, 2, 2], np.int32)
ESLOT = np.array([0, 0, 1, 2, -1, -1, -1, -1, -1, -1], np.int32)


class ManualTrees:
    """Depth-2 trees with 3 root children and 2 children under each, drawn
    from the draft (sampled) or its top-k, written straight into the tree and
    flat buffers in breadth-first order (flat position = node).  Node i of
    depth 1 is expanded with draft row slot i - 1 of layer 2."""

    def __init__(self, model, B, proposal):
        w = configs.Workload("walk_manual", B=B, V=V, dtype="f32", D=2, K_e=3, K_n=3, m=9,
                             verify="t1", sigma=0.0, proposal=proposal)
        self.model, self.B, self.proposal = model, B, proposal
        self.run = run = H.runner_for(w)
        tr, fl = run.tree, run.flat
        P = P_MAN
        key = (DEPTH.astype(np.int64) << 59) | np.arange(P)
        cap = tr.token.shape[1]
        self.cap = cap
        pad = lambda a, fillv: np.concatenate([a, np.full(cap - P, fillv, a.dtype)])
        tr.parent.copy_(torch.from_numpy(pad(PARENT, -1)[None].repeat(B, 0)))
        tr.depth.copy_(torch.from_numpy(pad(DEPTH, -1)[None].repeat(B, 0)))
        tr.eslot.copy_(torch.from_numpy(pad(ESLOT, -1)[None].repeat(B, 0)))
        tr.key.copy_(torch.from_numpy(pad(key, -1)[None].repeat(B, 0)))
        tr.n_nodes.fill_(P)
        fl.node.copy_(torch.arange(P, dtype=torch.int32)[None].repeat(B, 1))
        fl.parent.copy_(torch.from_numpy(PARENT[None].repeat(B, 0)))
        fl.pos.copy_(torch.from_numpy(DEPTH[None].repeat(B, 0)))
        fl.m.fill_(P - 1)
        fl.n_leaves.fill_(6)
        self.T = torch.ones(B, dtype=torch.float32, device="cuda")

    @staticmethod
    def _stats(l):
        l64 = l.astype(np.float64)
        mx = l64.max(-1)
        e = np.exp(l64 - mx[..., None])
        am = l64.argmax(-1)
        tot = e.sum(-1) - np.take_along_axis(e, am[..., None], -1)[..., 0]
        return mx.astype(np.float32), tot.astype(np.float32)

    def call(self, rng, sampled):
        """One verify call on fresh trees; returns the inputs and outputs."""
        from dynamic_draft_tree_row_amd import api
        m, B, P, run = self.model, self.B, P_MAN, self.run
        tr, fl = run.tree, run.flat
        if sampled:
            x1 = np.minimum((rng.random((B, 3))[..., None] >= np.cumsum(m.q0)).sum(-1), V - 1)
            u2 = rng.random((B, 3, 2))
            x2 = np.minimum((u2[..., None] >= np.cumsum(m.q1, axis=1)[x1][:, :, None, :]).sum(-1), V - 1)
        else:
            top0 = np.argsort(-m.q0, kind="stable")[:3]
            x1 = np.broadcast_to(top0, (B, 3)).copy()
            x2 = np.stack([np.argsort(-m.q1[a], kind="stable")[:2] for a in top0])[None].repeat(B, 0)
        tok = np.zeros((B, P), np.int64)
        tok[:, 1:4] = x1
        tok[:, 4:10] = x2.reshape(B, 6)
        arena = np.zeros((2, B, 3, V), np.float32)
        arena[0, :, 0] = m.lq0
        arena[1] = m.lq1[x1]
        rm, rs = np.zeros((B, 2, 3), np.float32), np.zeros((B, 2, 3), np.float32)
        rm[:, 0, 0], rs[:, 0, 0] = self._stats(m.lq0)
        rm[:, 1], rs[:, 1] = self._stats(m.lq1[x1])
        target = np.zeros((B, P, V), np.float32)
        target[:, 0] = m.lp0
        target[:, 1:4] = m.lp1[x1]
        target[:, 4:10] = m.lp2[np.repeat(x1, 2, axis=1), x2.reshape(B, 6)]
        tr.token.copy_(torch.from_numpy(np.concatenate([tok, np.full((B, self.cap - P), -1)], 1).astype(np.int32)))
        tr.rmax.copy_(torch.from_numpy(rm))
        tr.rsp.copy_(torch.from_numpy(rs))
        fl.token.copy_(torch.from_numpy(tok.astype(np.int32)))
        U = rng.random((B, P, 2), dtype=np.float32)
        api.tree_verify(tr, fl, torch.from_numpy(target).cuda(), torch.from_numpy(arena).cuda(), self.T,
                        torch.from_numpy(U).cuda(), run.accept_len, run.accept_path, run.next_token,
                        run.ws, proposal=self.proposal)
        torch.cuda.synchronize()
        out = (run.accept_len.cpu().numpy(), run.accept_path.cpu().numpy(), run.next_token.cpu().numpy())
        return tok, arena, target, U, out


def _manual_counts(model, calls, B, seed, sampled, proposal):
    trees = ManualTrees(model, B, proposal)
    rng = np.random.default_rng(seed)
    counts = np.zeros((V, V))
    for _ in range(calls):
        tok, _, _, _, (al, ap, nx) = trees.call(rng, sampled)
        a, c = _emitted(rng, model, tok, al, ap, nx)
        np.add.at(counts, (a, c), 1)
    return counts


@pytest.mark.parametrize("proposal", ["draft", "point"])
@pytest.mark.parametrize("sampled", [True, False])
def test_walk_on_written_trees_matches_oracle(proposal, sampled):
    # exact parity on the hand-written trees (duplicate sibling tokens are
    # frequent when children are sampled); requests with a decision inside
    # the oracle's margin floor are left out, as the round harness does
    model = Model(23)
    trees = ManualTrees(model, 512, proposal)
    rng = np.random.default_rng(31)
    tok, arena, target, U, (al, ap, nx) = trees.call(rng, sampled)
    checked = 0
    for b in range(512):
        f = O.Flat(list(range(P_MAN)), tok[b].tolist(), PARENT.tolist(), DEPTH.tolist(),
                   np.zeros((P_MAN, 1), np.uint32), np.zeros((1, 3), np.int32), 6, DEPTH.tolist())
        qrow = lambda i, b=b: arena[0, b, 0].astype(np.float64) if i == 0 else arena[1, b, i - 1].astype(np.float64)
        mg = []
        L, path, nxt = O.verify_stochastic(f, lambda i, b=b: target[b, i].astype(np.float64), qrow, 1.0,
                                           U[b], mg, proposal=proposal)
        if O.margin_failures([(k, v, b) for k, v in mg]):
            continue
        checked += 1
        assert al[b] == L and nx[b] == nxt, f"request {b}"
        assert ap[b, :L + 1].tolist() == path and (ap[b, L + 1:] == -1).all(), f"request {b}"
    say(f"written trees proposal={proposal} sampled={sampled}: {checked} of 512 compared")
    assert checked > 400


@pytest.mark.parametrize("proposal", ["draft", "point"])
def test_walk_lossless_on_sampled_children(proposal):
    model = Model(22)
    counts = _manual_counts(model, calls=25, B=4096, seed=6, sampled=True, proposal=proposal)
    pj, pm = _chi2_joint(counts, model)
    say(f"{proposal} proposals, sampled children: N={int(counts.sum())} p(joint)={pj:.3g} p(first)={pm:.3g}")
    assert pj > 1e-3 and pm > 1e-3


def test_walk_negative_control_draft_q_on_topk_children():
    model = Model(22)
    counts = _manual_counts(model, calls=13, B=4096, seed=7, sampled=False, proposal="draft")
    pj, pm = _chi2_joint(counts, model)
    say(f"draft proposals, top-k children: N={int(counts.sum())} p(first)={pm:.3g}")
    assert pm < 1e-6


# ---------------------------------------------------------------------------
# the cross-workgroup wait running out
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("proposal", ["point", "draft"])
def test_walk_wait_give_up_finishes_alone(proposal):
    """Spin limit 1: a T = 1 request's workgroups (12 per request here) give up
    waiting for each other almost at once; workgroup 0 must finish every walk
    alone with the oracle's outcome, and the counters must be back at 0 so the
    next call with the default limit is exact too."""
    from dynamic_draft_tree_row_amd import api
    base = configs.shrink(configs.C3, V=9001, B=4)
    w = configs.Workload(**{**base.__dict__, "proposal": proposal})
    case = H.oracle_case(w, 3, 0)
    run = H.runner_for(w)
    arena = H.to_dev(case.draft, w.dtype)
    run.draft(arena, torch.from_numpy(case.roots).cuda())
    target = H.to_dev(case.target, w.dtype)
    T = torch.from_numpy(case.T).cuda()
    U = torch.from_numpy(case.U).cuda()
    o = case.out
    for limit in (1, 0, 1):
        say(f"give-up test proposal={proposal} spin limit={limit or 'default'}")
        prev = api.set_walk_spin_limit(limit)
        try:
            run.verify(target, arena, T, U, proposal=proposal)
            torch.cuda.synchronize()
        finally:
            api.set_walk_spin_limit(prev)
        assert run.accept_len.cpu().tolist() == o["accept_len"].tolist()
        np.testing.assert_array_equal(run.accept_path.cpu().numpy(), o["accept_path"])
        assert run.next_token.cpu().tolist() == o["next_token"].tolist()
        assert (run.tree.walk_sync.cpu().numpy() == 0).all(), "wait counters not reset"

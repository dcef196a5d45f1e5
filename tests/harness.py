"""Parity harness: one round through the oracle and through the HIP library.

Inputs come only from gen/ (seeded); expected values only from oracle/.  A batch
row whose float-driven decisions sit closer to a threshold than the oracle's
margin floor (the generator's "score gap" guarantee) is re-keyed with an
attempt counter and regenerated before anything is compared.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from gen import synth
from gen.configs import Workload
from oracle import ddt_oracle as O


def cast_params(w: Workload, seed: int = 0) -> dict:
    S_T, S_D = synth.cost_tables(w, seed)
    cs = w.cast
    return dict(S_T=S_T, S_D=S_D, L=cs.L, M=cs.M, C1=[cs.C1] * w.D, C2=cs.C2,
                C3=[cs.C3] * w.B, R=cs.R)


def graft_params(w: Workload, tau) -> dict:
    gs = w.graft
    if gs.mode == "prune_then_graft":
        return dict(ck_depth=tuple(gs.ck_depth), tau=list(tau), k_draft=tuple(gs.k_draft),
                    K_max=gs.K_max)
    return dict(ck_depth=(), tau=[], k_draft=(), K_max=gs.K_max, draft_cap=gs.fixed_k_draft,
                anchor="tail" if gs.mode == "tail_only" else "root")


def flat_layout(trees, flats, P):
    """Per flat position: canonical key, depth, expand slot, token ([B][P])."""
    B = len(flats)
    fk = np.full((B, P), -1, np.int64)
    fd = np.zeros((B, P), np.int32)
    fs = np.full((B, P), -1, np.int32)
    ft = np.full((B, P), -1, np.int32)
    for b, (t, f) in enumerate(zip(trees, flats)):
        for i, v in enumerate(f.node):
            if v < 0:
                continue
            fk[b, i] = t.key[v]
            fd[b, i] = t.depth[v]
            fs[b, i] = t.eslot[v]
            ft[b, i] = t.token[v]
    return fk, fd, fs, ft


@dataclass
class Case:
    w: Workload
    seed: int
    rnd: int
    rows: List[int]
    attempts: np.ndarray
    draft: np.ndarray          # raw [D][nb][R][V]
    target: np.ndarray         # raw [nb][P][V]
    roots: np.ndarray
    U: np.ndarray
    T: np.ndarray
    out: dict                  # oracle outputs
    cast: Optional[dict] = None
    graft: Optional[dict] = None
    M_before: Optional[np.ndarray] = None
    M_after: Optional[np.ndarray] = None
    tries: int = 0
    shared_M: bool = False


class SharedRows:
    """Every request's view of one successor matrix [V][k]: the oracle reads and
    refreshes the same rows for all requests, in request order."""

    def __init__(self, M1):
        self.M = M1

    def __getitem__(self, b):
        return self.M


def oracle_case(w: Workload, seed: int, rnd: int, rows=None, cast=None, graft=None,
                M=None, M0=None, max_tries=60, shared_M=False) -> Case:
    """Run the oracle on batch rows `rows` of (seed, rnd), re-keying rows whose
    decisions fall inside the margin floor.  M/M0 are full-batch [B][V][k], or
    one [V][k] matrix shared by every row when shared_M."""
    rows = list(range(w.B)) if rows is None else list(rows)
    nb = len(rows)
    att = np.zeros(nb, np.int64)
    draft = None
    for tries in range(1, max_tries + 1):
        if draft is None:
            draft = synth.draft_arena(w, seed, rnd, att, rows=rows)
        roots = synth.root_tokens(w, seed, rnd, rows=rows)
        U = synth.uniforms(w, seed, rnd, att, rows=rows)
        T = synth.temperatures(w, seed, rnd, rows=rows)
        held = {}

        def tfn(dr, flats):
            fk, fd, fs, ft = flat_layout(dr.trees, flats, w.m_max + 1)
            held["t"] = synth.target_arena(w, seed, rnd, draft, fk, fd, fs, ft, att, M0r, rows=rows)
            return held["t"]

        if shared_M:
            Mc = SharedRows(M.copy())
            M0r = np.stack([M0] * w.B) if M0 is not None else None
        else:
            Mc = M[rows].copy() if M is not None else None
            M0r = M0
        cst = None
        if cast is not None:
            cst = dict(cast)
            cst["C3"] = [cast["C3"][r] for r in rows]
        gs = w.graft
        out = O.run_round(B=nb, V=w.V, dtype=w.dtype, D=w.D, K_e=w.K_e, K_n=w.K_n, m_max=w.m_max,
                          root_tok=roots, draft_raw=draft, target_raw_fn=tfn, temperature=T, U=U,
                          prefix=w.prefix, cast=cst, graft=graft, M=Mc,
                          k_succ=gs.k_succ if gs else 8,
                          tpl=(gs.tpl_depth, gs.tpl_width) if gs else (8, 8),
                          proposal=w.proposal)
        bad = O.margin_failures(out["margins"])
        if not bad:
            M_after = None
            if shared_M:
                M_after = Mc.M
            elif M is not None:
                M_after = M.copy()
                M_after[rows] = Mc
            return Case(w, seed, rnd, rows, att, draft, held["t"], roots, U, T, out, cst, graft,
                        M, M_after, tries, shared_M)
        redo = list(range(nb)) if -1 in bad else sorted(bad)
        att[redo] += 1
        synth.draft_arena(w, seed, rnd, att, rows=rows, out=draft, only=redo)
    raise RuntimeError(f"no margin-clean inputs after {max_tries} attempts")


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------

def to_dev(raw: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(raw)).to(device)
    return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(device).view(torch.bfloat16)


def runner_for(w: Workload, device="cuda", shared_M=False):
    import torch
    from dynamic_draft_tree_row_amd.round_driver import RoundRunner, RoundShape
    gs = w.graft
    shape = RoundShape(B=w.B, V=w.V, dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16,
                       D=w.D, K_e=w.K_e, K_n=w.K_n, m=w.m_max, prefix=w.prefix,
                       graft=gs is not None, tpl_depth=gs.tpl_depth if gs else 8,
                       tpl_width=gs.tpl_width if gs else 8, k_succ=gs.k_succ if gs else 8,
                       shared_M=shared_M,
                       graft_anchor=1 if gs is not None and gs.mode == "tail_only" else 0)
    return RoundRunner(shape, device)


def dev_cast(cast: dict, device="cuda", ctx_verify: int = 0):
    """CAST parameters on the device; ctx_verify is the verify-cost context
    (the oracle takes the context prefix)."""
    import torch
    from dynamic_draft_tree_row_amd.api import CastParams
    f = lambda a: torch.tensor(np.asarray(a, np.float32), device=device)
    return CastParams(S_T=f(cast["S_T"]), S_D=f(cast["S_D"]), L=cast["L"], C1=f(cast["C1"]),
                      C2=float(cast["C2"]), C3=f(cast["C3"]), R=cast["R"], ctx_verify=ctx_verify)


def dev_gate(graft: dict):
    from dynamic_draft_tree_row_amd.api import GraftGate
    return GraftGate(ck_depth=list(graft["ck_depth"]), tau=[float(x) for x in graft["tau"]],
                     k_draft=list(graft["k_draft"]), K_max=graft.get("draft_cap", graft["K_max"]))


def gpu_round(case: Case, device="cuda") -> dict:
    """The same round through the library; returns host copies of everything."""
    import torch
    w = case.w
    wb = Workload(**{**w.__dict__, "B": len(case.rows)})
    run = runner_for(wb, device, case.shared_M)
    arena = to_dev(case.draft, w.dtype, device)
    roots = torch.from_numpy(case.roots).to(device)
    cast = dev_cast(case.cast, device, w.prefix) if case.cast else None
    gate = dev_gate(case.graft) if case.graft else None
    if case.M_before is None:
        M = None
    elif case.shared_M:
        M = torch.from_numpy(np.ascontiguousarray(case.M_before)).to(device)
    else:
        M = torch.from_numpy(np.ascontiguousarray(case.M_before[case.rows])).to(device)
    run.draft(arena, roots, cast=cast, gate=gate, M=M)
    target = to_dev(case.target, w.dtype, device)
    T = torch.from_numpy(case.T).to(device)
    U = torch.from_numpy(case.U).to(device)
    run.verify(target, arena, T, U, M=M, proposal=w.proposal)
    torch.cuda.synchronize()
    t, f = run.tree, run.flat
    g = lambda x: x.cpu().numpy()
    res = dict(token=g(t.token), parent=g(t.parent), depth=g(t.depth), eslot=g(t.eslot),
               key=g(t.key), S=g(t.S), logc=g(t.logc), rmax=g(t.rmax), rsp=g(t.rsp),
               n_nodes=g(t.n_nodes), widths=g(t.widths), k_draft=g(t.k_draft),
               sel=g(run.sel), m_out=g(run.m_out), f_node=g(f.node), f_token=g(f.token),
               f_parent=g(f.parent), f_pos=g(f.pos), f_mask=g(f.mask).view(np.uint32),
               f_ret=g(f.retrieve), f_nl=g(f.n_leaves), f_m=g(f.m), accept_len=g(run.accept_len),
               accept_path=g(run.accept_path), next_token=g(run.next_token),
               argmax=g(run.row_argmax))
    if M is not None:
        res["M"] = g(M)
    return res


def compare(case: Case, r: dict) -> None:
    """Exact on every integer output, rtol 1e-5 on fp32 values."""
    o = case.out
    ot = o["tree"]
    w = case.w
    for b in range(len(case.rows)):
        n = int(ot["n_nodes"][b])
        tag = f"row {case.rows[b]} (seed {case.seed}, round {case.rnd}, attempt {case.attempts[b]})"
        assert int(r["n_nodes"][b]) == n, tag + " n_nodes"
        for k in ("token", "parent", "depth", "eslot", "key"):
            np.testing.assert_array_equal(r[k][b, :n], ot[k][b, :n], err_msg=f"{tag} {k}")
        for k in ("S", "logc"):
            a, e = r[k][b, :n], ot[k][b, :n]
            fin = np.isfinite(e)
            np.testing.assert_array_equal(np.isfinite(a), fin, err_msg=f"{tag} {k} finiteness")
            np.testing.assert_allclose(a[fin], e[fin], rtol=1e-5, atol=1e-30, err_msg=f"{tag} {k}")
        used = ot["eslot"][b, :n]
        for v in range(n):
            j = int(used[v])
            if j < 0:
                continue
            d = int(ot["depth"][b, v])
            assert r["rmax"][b, d, j] == ot["rmax"][b, d, j], f"{tag} rmax"
            np.testing.assert_allclose(r["rsp"][b, d, j], ot["rsp"][b, d, j], rtol=1e-5,
                                       err_msg=f"{tag} rsp")
        m = int(o["m_rows"][b])
        assert int(r["m_out"][b]) == m and int(r["f_m"][b]) == m, f"{tag} m"
        assert sorted(r["sel"][b, 1:m + 1].tolist()) == sorted(o["sels"][b]), f"{tag} selection"
        assert r["sel"][b, 0] == 0 and (r["sel"][b, m + 1:] == -1).all(), f"{tag} sel padding"
        f = o["flats"][b]
        np.testing.assert_array_equal(r["f_node"][b], f.node, err_msg=f"{tag} flat node")
        np.testing.assert_array_equal(r["f_token"][b], f.token, err_msg=f"{tag} flat token")
        np.testing.assert_array_equal(r["f_parent"][b], f.parent, err_msg=f"{tag} flat parent")
        np.testing.assert_array_equal(r["f_pos"][b], f.pos, err_msg=f"{tag} pos")
        np.testing.assert_array_equal(r["f_mask"][b], f.mask, err_msg=f"{tag} mask")
        assert int(r["f_nl"][b]) == f.n_leaves, f"{tag} n_leaves"
        nl = f.n_leaves
        np.testing.assert_array_equal(r["f_ret"][b, :nl], f.retrieve[:nl], err_msg=f"{tag} retrieve")
        assert (r["f_ret"][b, nl:] == -1).all(), f"{tag} retrieve padding"
        np.testing.assert_array_equal(r["argmax"][b, :m + 1], o["argmax"][b, :m + 1],
                                      err_msg=f"{tag} argmax")
        assert int(r["accept_len"][b]) == int(o["accept_len"][b]), f"{tag} accept_len"
        np.testing.assert_array_equal(r["accept_path"][b], o["accept_path"][b], err_msg=f"{tag} path")
        assert int(r["next_token"][b]) == int(o["next_token"][b]), f"{tag} next_token"
    if case.cast is not None:
        wd = o["draft"].widths
        np.testing.assert_array_equal(r["widths"][:len(wd)], wd, err_msg="CAST widths")
    if case.graft is not None:
        np.testing.assert_array_equal(r["k_draft"], o["draft"].k_draft, err_msg="Graft k_draft")
        exp_M = case.M_after if case.shared_M else case.M_after[case.rows]
        np.testing.assert_array_equal(r["M"], exp_M, err_msg="successor matrix")


def calibrate_tau(w: Workload, seed: int, rounds: int, q: float = 25.0):
    """Checkpoint thresholds from warm-up rounds of the same generator: at each
    checkpoint, the q-th percentile of c_d = exp(max S at that depth) over the
    rows still active (Graft review: thresholds calibrated on warm-up data)."""
    gs = w.graft
    cds = []
    for r in range(rounds):
        arena = synth.draft_arena(w, seed, 10_000 + r)
        roots = synth.root_tokens(w, seed, 10_000 + r)
        drow = lambda layer, b, j: O.decode(arena[layer - 1, b, j], w.dtype)
        dr = O.draft_phase(drow, w.B, roots, max(gs.ck_depth), w.K_e, w.K_n)
        for t in dr.trees:
            cds.append([math.exp(max(t.S[i] for i in range(t.n) if t.depth[i] == d))
                        for d in gs.ck_depth])
    cds = np.array(cds)
    alive = np.ones(len(cds), bool)
    tau = []
    for s in range(len(gs.ck_depth)):
        ts = float(np.percentile(cds[alive, s], q))
        tau.append(ts)
        alive &= cds[:, s] > ts
    return tau


def gpu_flat_layout(run, B):
    """Flat-position layout (key, depth, expand slot, token) read back from the
    library's own outputs: used only to lay out target rows for batch rows the
    oracle does not compute."""
    t, f = run.tree, run.flat
    node = f.node.cpu().numpy()
    key, dep = t.key.cpu().numpy(), t.depth.cpu().numpy()
    esl, tok = t.eslot.cpu().numpy(), t.token.cpu().numpy()
    P = node.shape[1]
    fk = np.full((B, P), -1, np.int64)
    fd = np.zeros((B, P), np.int32)
    fs = np.full((B, P), -1, np.int32)
    ft = np.full((B, P), -1, np.int32)
    for b in range(B):
        ok = node[b] >= 0
        nv = node[b][ok]
        fk[b, ok] = key[b, nv]; fd[b, ok] = dep[b, nv]; fs[b, ok] = esl[b, nv]; ft[b, ok] = tok[b, nv]
    return fk, fd, fs, ft


def gpu_round_full(case: Case, device="cuda") -> dict:
    """The whole batch through the library; the sampled rows carry exactly the
    oracle's inputs, the other rows are generated with attempt 0 and their
    target rows are laid out from the library's own flat layout."""
    import torch
    w = case.w
    B = w.B
    att = np.zeros(B, np.int64)
    att[case.rows] = case.attempts
    draft = synth.draft_arena(w, case.seed, case.rnd, att)
    np.testing.assert_array_equal(draft[:, case.rows], case.draft)
    run = runner_for(w, device)
    arena = to_dev(draft, w.dtype, device)
    roots = torch.from_numpy(synth.root_tokens(w, case.seed, case.rnd)).to(device)
    run.draft(arena, roots)
    torch.cuda.synchronize()
    others = [b for b in range(B) if b not in case.rows]
    fk, fd, fs, ft = gpu_flat_layout(run, B)
    target = np.empty((B, w.m_max + 1, w.V), synth.raw_dtype(w))
    target[case.rows] = case.target
    if others:
        target[others] = synth.target_arena(w, case.seed, case.rnd, draft[:, others], fk[others],
                                            fd[others], fs[others], ft[others], att[others],
                                            rows=others)
    T = torch.from_numpy(synth.temperatures(w, case.seed, case.rnd)).to(device)
    U = torch.from_numpy(synth.uniforms(w, case.seed, case.rnd, att)).to(device)
    run.verify(to_dev(target, w.dtype, device), arena, T, U, proposal=w.proposal)
    torch.cuda.synchronize()
    t, f = run.tree, run.flat
    g = lambda x: x.cpu().numpy()
    res = dict(token=g(t.token), parent=g(t.parent), depth=g(t.depth), eslot=g(t.eslot),
               key=g(t.key), S=g(t.S), logc=g(t.logc), rmax=g(t.rmax), rsp=g(t.rsp),
               n_nodes=g(t.n_nodes), widths=g(t.widths), k_draft=g(t.k_draft),
               sel=g(run.sel), m_out=g(run.m_out), f_node=g(f.node), f_token=g(f.token),
               f_parent=g(f.parent), f_pos=g(f.pos), f_mask=g(f.mask).view(np.uint32),
               f_ret=g(f.retrieve), f_nl=g(f.n_leaves), f_m=g(f.m), accept_len=g(run.accept_len),
               accept_path=g(run.accept_path), next_token=g(run.next_token),
               argmax=g(run.row_argmax), T=g(T))
    return res


def check_invariants(r: dict, w: Workload) -> None:
    """Properties that hold for every row at any size."""
    B = r["n_nodes"].shape[0]
    for b in range(B):
        n = int(r["n_nodes"][b])
        par, S = r["parent"][b, :n], r["S"][b, :n]
        assert par[0] == -1 and (par[1:] >= 0).all() and (par[1:] < np.arange(1, n)).all()
        fin = np.isfinite(S)
        assert (S[1:][fin[1:]] <= S[par[1:]][fin[1:]]).all(), f"row {b}: value not monotone"
        m = int(r["m_out"][b])
        sel = set(r["sel"][b, 1:m + 1].tolist()) | {0}
        assert all(int(par[v]) in sel for v in sel if v != 0), f"row {b}: selection not connected"
        P = r["f_node"].shape[1]
        dep = r["depth"][b]
        for i in range(m + 1):
            bits = sum(bin(int(x)).count("1") for x in r["f_mask"][b, i])
            assert bits == dep[r["f_node"][b, i]] + 1
        L = int(r["accept_len"][b])
        path = r["accept_path"][b]
        assert 0 <= L <= w.D and path[0] == 0
        for s in range(1, L + 1):
            assert r["f_parent"][b, path[s]] == path[s - 1]
            if r["T"][b] == 0:
                assert r["f_token"][b, path[s]] == r["argmax"][b, path[s - 1]]
        if r["T"][b] == 0:
            assert r["next_token"][b] == r["argmax"][b, path[L]]

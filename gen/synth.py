"""Seeded synthetic inputs for the draft-tree round.

Both the CPU oracle and the HIP path are fed from here; this module holds none
of the method's arithmetic (no softmax statistics, no selection, no tree
logic). It makes random logit rows, noise, uniforms, temperatures, root tokens,
the initial successor matrix and cost tables, and it lays rows out by index.

Every random stream is a numpy Philox generator keyed by a tuple of integers,
so any single row can be regenerated on its own, independent of the order in
which rows are produced.

Draft logits ("virtual draft model"): the draft forward for frontier slot j of
layer d of batch row b returns row (round, b, d, j). A row is t * N(0, 1)^V with
a per-row scale t ~ U(0.3, 3), plus one planted peak v* ~ U{0..V-1} whose
softmax probability is pi ~ U(0.05, 0.98), spanning the confidence range of the
EAGLE-2 explainer's calibration figure (section on why confidence approximates
acceptance). Rows are cast to the workload dtype (bf16 by round-to-nearest-even).

Target logits: the target row at a tree node is the draft row that expanded
that node (a fresh keyed row when the node was never expanded) plus
N(0, sigma) noise, cast to the dtype. For the Graft workload, a keyed half of
the rows get their peak moved onto the node token's first successor in the
initial successor matrix, so that retrieval can be accepted.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import PROXY_DRAFT, PROXY_TARGET, ProxyShape, Workload

# stream tags
S_DRAFT, S_TNOISE, S_FRESH, S_UNIF, S_TEMP, S_ROOT, S_SUCC, S_COST, S_PLANT = range(1, 10)

_M64 = (1 << 64) - 1


def _splitmix(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _M64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def keyed(*fields: int) -> np.random.Generator:
    """A Philox generator whose 128-bit key is a hash of the integer fields."""
    h1, h2 = 0x243F6A8885A308D3, 0x13198A2E03707344
    for f in fields:
        f = int(f) & _M64
        h1 = _splitmix(h1 ^ f)
        h2 = _splitmix(h2 + f + 0x5851F42D4C957F2D)
    return np.random.Generator(np.random.Philox(key=np.array([h1, h2], dtype=np.uint64)))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even. Finite inputs."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    return (r >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def raw_dtype(w: Workload):
    return np.float32 if w.dtype == "f32" else np.uint16


def cast_row(x: np.ndarray, dtype: str) -> np.ndarray:
    return np.asarray(x, np.float32) if dtype == "f32" else to_bf16_bits(x)


def as_f32(raw: np.ndarray, dtype: str) -> np.ndarray:
    return np.asarray(raw, np.float32) if dtype == "f32" else from_bf16_bits(raw)


def _lse(x64: np.ndarray) -> float:
    mx = float(np.max(x64))
    return mx + float(np.log(np.sum(np.exp(x64 - mx))))


def logit_row(gen: np.random.Generator, V: int) -> np.ndarray:
    """t * N(0,1)^V with one planted peak of softmax probability pi (float32)."""
    t = gen.uniform(0.3, 3.0)
    row = gen.standard_normal(V, dtype=np.float32)
    row *= np.float32(t)
    vstar = int(gen.integers(V))
    pi = gen.uniform(0.05, 0.98)
    rest = row.astype(np.float64)
    rest[vstar] = -np.inf
    row[vstar] = np.float32(np.log(pi / (1.0 - pi)) + _lse(rest))
    return row


# ----------------------------------------------------------------------------
# draft arena
# ----------------------------------------------------------------------------

def draft_row(w: Workload, seed: int, rnd: int, b: int, layer: int, slot: int,
              attempt: int = 0) -> np.ndarray:
    """Raw (dtype) draft row for frontier slot `slot` of layer `layer` (1-based)."""
    g = keyed(S_DRAFT, seed, rnd, b, layer, slot, attempt)
    return cast_row(logit_row(g, w.V), w.dtype)


def _rows(w: Workload, rows):
    return list(range(w.B)) if rows is None else [int(r) for r in rows]


def draft_arena(w: Workload, seed: int, rnd: int, attempts=None,
                layers=None, out: np.ndarray | None = None, rows=None,
                only=None) -> np.ndarray:
    """Raw draft arena [D][len(rows)][R_max][V]; layer d's slice is arena[d-1].

    rows: the batch rows to generate (default all); arena row i is batch row
    rows[i] and attempts[i] its re-key counter.  only: indices into rows to
    (re)fill in an existing `out`.  Layer 1 only ever reads slot 0 (the root);
    its other slots are filled too so that every slice has the same shape.
    """
    rows = _rows(w, rows)
    D, R, V = w.D, w.R_max, w.V
    att = np.zeros(len(rows), np.int64) if attempts is None else np.asarray(attempts)
    if out is None:
        out = np.empty((D, len(rows), R, V), raw_dtype(w))
    layers = range(1, D + 1) if layers is None else layers
    idx = range(len(rows)) if only is None else only
    jobs = [(d, i, j) for d in layers for i in idx for j in range(R)]

    def fill(job):
        d, i, j = job
        out[d - 1, i, j] = draft_row(w, seed, rnd, rows[i], d, j, int(att[i]))

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, jobs))
    return out


def root_tokens(w: Workload, seed: int, rnd: int, rows=None) -> np.ndarray:
    g = keyed(S_ROOT, seed, rnd)
    return g.integers(0, w.V, size=w.B).astype(np.int32)[_rows(w, rows)]


# ----------------------------------------------------------------------------
# target arena (stand-in for the target forward over the flattened tree)
# ----------------------------------------------------------------------------

def target_arena(w: Workload, seed: int, rnd: int, draft: np.ndarray,
                 flat_key: np.ndarray, flat_depth: np.ndarray, flat_slot: np.ndarray,
                 flat_token: np.ndarray, attempts=None, M0: np.ndarray | None = None,
                 out: np.ndarray | None = None, rows=None, only=None) -> np.ndarray:
    """Raw target rows [len(rows)][m_max+1][V] in flat order.

    flat_* are [len(rows)][m_max+1] arrays describing each flat position: the
    node's canonical key (int64, -1 for padding), depth, the frontier slot it
    was expanded with at layer depth+1 (-1 if never expanded) and its token.
    draft is the matching [D][len(rows)][R][V] arena; M0 is indexed by the
    original batch row.  only: indices into rows to (re)fill in `out`.
    """
    rows = _rows(w, rows)
    V = w.V
    P = flat_key.shape[1]
    att = np.zeros(len(rows), np.int64) if attempts is None else np.asarray(attempts)
    if out is None:
        out = np.empty((len(rows), P, V), raw_dtype(w))
    plant = w.graft.plant_prob if (w.graft is not None and M0 is not None) else 0.0

    def fill(job):
        ib, i = job
        b = rows[ib]
        key = int(flat_key[ib, i])
        slot = int(flat_slot[ib, i])
        depth = int(flat_depth[ib, i])
        if key < 0:                                   # padding position
            base = logit_row(keyed(S_FRESH, seed, rnd, b, 1 << 62, i, int(att[ib])), V)
        elif slot >= 0 and depth + 1 <= w.D:
            base = as_f32(draft[depth, ib, slot], w.dtype).copy()
        else:
            base = logit_row(keyed(S_FRESH, seed, rnd, b, key, int(att[ib])), V)
        gn = keyed(S_TNOISE, seed, rnd, b, key if key >= 0 else (1 << 62) + i, int(att[ib]))
        noise = gn.standard_normal(V, dtype=np.float32)
        noise *= np.float32(w.sigma)
        base += noise
        tok = int(flat_token[ib, i])
        if plant > 0.0 and key >= 0 and tok >= 0:
            gp = keyed(S_PLANT, seed, rnd, b, key, int(att[ib]))
            if gp.uniform() < plant:
                s = int(M0[b, tok, 0])
                base[s] = np.float32(float(np.max(base)) + gp.uniform(0.5, 3.0))
        out[ib, i] = cast_row(base, w.dtype)

    idx = range(len(rows)) if only is None else only
    jobs = [(ib, i) for ib in idx for i in range(P)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, jobs))
    return out


# ----------------------------------------------------------------------------
# uniforms, temperatures
# ----------------------------------------------------------------------------

def uniforms(w: Workload, seed: int, rnd: int, attempts=None, rows=None) -> np.ndarray:
    """fp32 [rows][m_max+1][2]: [..,0] accept test at flat position i, [..,1] emission there."""
    rows = _rows(w, rows)
    att = np.zeros(len(rows), np.int64) if attempts is None else np.asarray(attempts)
    out = np.empty((len(rows), w.m_max + 1, 2), np.float32)
    for i, b in enumerate(rows):
        out[i] = keyed(S_UNIF, seed, rnd, b, int(att[i])).random((w.m_max + 1, 2), dtype=np.float32)
    return out


def temperatures(w: Workload, seed: int, rnd: int, rows=None) -> np.ndarray:
    rows = _rows(w, rows)
    if w.verify == "greedy":
        return np.zeros(len(rows), np.float32)
    if w.verify == "t1":
        return np.ones(len(rows), np.float32)
    g = keyed(S_TEMP, seed, rnd)
    if w.verify == "tmix":            # greedy rows and three sampling temperatures
        return np.array([0.0, 0.7, 1.0, 1.6], np.float32)[g.integers(0, 4, w.B)][rows]
    return (g.random(w.B) < 0.5).astype(np.float32)[rows]


# ----------------------------------------------------------------------------
# Graft: initial successor matrix and checkpoint thresholds
# ----------------------------------------------------------------------------

def succ_matrix0(w: Workload, seed: int, B: int | None = None) -> np.ndarray:
    """int32 [B][V][k]: k distinct successors per token, Zipf(s) ranked.

    For request b, token v draws 32 Zipf ranks; its successors are the k
    smallest distinct ranks r (most frequent first), mapped to tokens through
    perm_b[(shift_b[v] + r) mod V] with two seeded permutations of the vocab.
    """
    gs = w.graft
    B = w.B if B is None else B
    V, k = w.V, gs.k_succ
    out = np.empty((B, V, k), np.int32)

    def one(b):
        g = keyed(S_SUCC, seed, b)
        perm = g.permutation(V)
        shift = g.permutation(V)
        draws = (g.zipf(gs.zipf_s, size=(V, 32)) - 1) % V
        draws.sort(axis=1)
        new = np.ones_like(draws, dtype=bool)
        new[:, 1:] = draws[:, 1:] != draws[:, :-1]
        order = np.argsort(~new, axis=1, kind="stable")[:, :k]
        ranks = np.take_along_axis(draws, order, axis=1)
        short = np.nonzero(new.sum(axis=1) < k)[0]
        for v in short:
            have = list(dict.fromkeys(draws[v].tolist()))
            r = 0
            while len(have) < k:
                if r not in have:
                    have.append(r)
                r += 1
            ranks[v] = sorted(have)[:k]
        out[b] = perm[(shift[:, None] + ranks) % V]

    with ThreadPoolExecutor(min(_workers(), 4)) as ex:
        list(ex.map(one, range(B)))
    return out


# ----------------------------------------------------------------------------
# CAST cost tables
# ----------------------------------------------------------------------------

def cost_tables(w: Workload, seed: int = 0):
    """(S_T, S_D) fp32 [M][N+1]; column n holds the time for n tokens (column 0 unused).

    "linear": S_T[r][n] = 1 + lam*(n-1) and S_D[r][n] = lam*n + delta, so the
    normalised width cost S_D[.][k] / S_T[.][1] is lam*k + delta and the verify
    cost S_T[.][k] / S_T[.][1] is lam*k + (1 - lam): both have slope lam.
    "seeded": per-row random positive increments (increasing in n and in r).
    "roofline": roofline_table of the proxy target and draft shapes at batch
    table_B (default: the workload's B): flat while a forward is HBM-bound,
    rising once it is MFMA-bound, so that equal neighbouring costs occur.
    """
    cs = w.cast
    M, N = cs.M, cs.N
    if cs.table == "roofline":
        Bt = cs.table_B or w.B
        return (roofline_table(PROXY_TARGET, Bt, cs.L, M, N),
                roofline_table(PROXY_DRAFT, Bt, cs.L, M, N))
    S_T = np.zeros((M, N + 1), np.float32)
    S_D = np.zeros((M, N + 1), np.float32)
    n = np.arange(1, N + 1, dtype=np.float64)
    if cs.table == "linear":
        S_T[:, 1:] = (1.0 + cs.lam * (n - 1))[None, :]
        S_D[:, 1:] = (cs.lam * n + cs.delta)[None, :]
    else:
        g = keyed(S_COST, seed)
        for r in range(M):
            base_t = 1.0 + 0.05 * r
            inc_t = g.uniform(0.005, 0.04, size=N)
            inc_t[0] = 0.0
            S_T[r, 1:] = base_t + np.cumsum(inc_t)
            inc_d = g.uniform(0.01, 0.05, size=N)
            S_D[r, 1:] = 0.8 + 0.02 * r + np.cumsum(inc_d)
    return S_T, S_D


HBM_BYTES_PER_S = 8.0e12        # MI355X HBM3E
MFMA_BF16_FLOP_PER_S = 2.5e15   # MI355X dense bf16 matrix peak


def roofline_table(shape: ProxyShape, B: int, L: int, M: int, N: int) -> np.ndarray:
    """[M][N+1] float32 microseconds: for context c = k*L (row k) and n new
    tokens (column n), the larger of HBM time and MFMA time of a bf16 forward of
    `shape` at batch B (column 0 is 0).  Bytes per layer: the projection weights
    once plus the context keys and values; flops: 2 per weight per token plus
    causal attention, 4*Hq*D per (query, key) pair with query i of the n new
    tokens seeing c + i + 1 keys.  The LM head adds its weights and 2*d*V flops
    per token."""
    d, D = shape.d_model, shape.D
    w_layer = d * (shape.Hq + 2 * shape.Hkv) * D + shape.Hq * D * d + 3 * d * shape.ffn
    n = np.arange(1, N + 1, dtype=np.float64)
    head = np.maximum(2.0 * d * shape.V / HBM_BYTES_PER_S,
                      2.0 * B * n * d * shape.V / MFMA_BF16_FLOP_PER_S)
    t = np.zeros((M, N + 1), np.float64)
    for k in range(M):
        c = k * L
        by = 2.0 * w_layer + 2.0 * 2 * B * c * shape.Hkv * D
        fl = 2.0 * B * n * w_layer + 4.0 * B * shape.Hq * D * (n * c + n * (n + 1) / 2)
        layer = np.maximum(by / HBM_BYTES_PER_S, fl / MFMA_BF16_FLOP_PER_S)
        t[k, 1:] = (shape.n_layers * layer + head) * 1e6
    return t.astype(np.float32)

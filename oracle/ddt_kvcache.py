"""CPU oracle for committing the accepted path into a block-paged KV cache.
TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the bench's CPU-baseline leg
may import or run this module.  The HIP product path never calls it, and the
two share no code: this file imports numpy only.

What it computes, from the pages:
  * EAGLE-2 explainer (pinghaoyang.com.cn, "EAGLE-2 完全拆解"), engineering
    difficulty two: candidate KV is kept apart from the committed context;
    after verification the accepted tokens' KV is committed and the rejected
    candidates' KV is dropped; with block-paged storage, allocation, reference
    counting, reclamation and copy-on-write are part of that step.  The same
    page's decode-step flow ends with "commit accepted tokens and their KV,
    discard rejected candidate KV".

Readings (the pages give no layout):
  * candidates' KV is the round's contiguous tree buffer [B][P][Hkv][D], so a
    rejected candidate costs nothing to drop;
  * the committed context of request b is a list of fixed-size blocks
    (table[b]); token t sits at slot t % block of block table[b][t // block];
  * a block shared by several requests (ref > 1) is copied before one of them
    writes into it; holder counts are read when the call starts;
  * free blocks form a stack; blocks are popped from its top and pushed back
    on it, in the orders the boundary's documentation fixes (request index
    order, table order).

The state is a dict of numpy arrays (k, v as uint16 bf16 bits so that copies
are compared bit for bit): k, v [n_blocks][block][Hkv][D]; table [B][max_blocks]
(-1 unused); len [B]; ref [n_blocks]; free_ids [n_blocks]; n_free (int).
Every function works on the dict in place, one request at a time.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np


def new_state(B: int, max_blocks: int, n_blocks: int, block: int, Hkv: int, D: int) -> Dict:
    """An empty cache: every block free, stacked so that block 0 is on top."""
    return {
        "k": np.zeros((n_blocks, block, Hkv, D), np.uint16),
        "v": np.zeros((n_blocks, block, Hkv, D), np.uint16),
        "table": np.full((B, max_blocks), -1, np.int32),
        "len": np.zeros(B, np.int32),
        "ref": np.zeros(n_blocks, np.int32),
        "free_ids": np.arange(n_blocks - 1, -1, -1, dtype=np.int32),
        "n_free": n_blocks,
        "block": block,
    }


def context(st: Dict, b: int):
    """Request b's committed keys and values in token order: ([len][Hkv][D]) x 2."""
    bs = st["block"]
    n = int(st["len"][b])
    ks = [st["k"][st["table"][b][t // bs], t % bs] for t in range(n)]
    vs = [st["v"][st["table"][b][t // bs], t % bs] for t in range(n)]
    shape = st["k"].shape[2:]
    if n == 0:
        return np.zeros((0,) + shape, np.uint16), np.zeros((0,) + shape, np.uint16)
    return np.stack(ks), np.stack(vs)


def commit(st: Dict, accept_len: np.ndarray, accept_path: np.ndarray, k_tree: np.ndarray,
           v_tree: np.ndarray) -> np.ndarray:
    """Append each request's accepted path (root first) to its context.

    k_tree, v_tree: uint16 [B][P][Hkv][D]; accept_path [B][Dp+1] flat indices.
    Returns status [B]: tokens committed, 0 (nothing accepted), -1 (context
    capacity), -2 (free stack exhausted), -3 (a path entry outside [0, P))."""
    B, max_blocks = st["table"].shape
    bs = st["block"]
    P = k_tree.shape[1]
    ref0 = st["ref"].copy()                       # holder counts at the call
    status = np.zeros(B, np.int32)
    plans = []                                    # admitted: (b, L0, n, old block or -1, first, last, off)
    nf = st["n_free"]
    used = 0
    stopped = False
    for b in range(B):
        a = int(accept_len[b])
        if a < 0:
            continue
        n = a + 1
        L0 = int(st["len"][b])
        path = [int(x) for x in accept_path[b][:n]]
        if any(p < 0 or p >= P for p in path):
            status[b] = -3
            continue
        if L0 + n > max_blocks * bs:
            status[b] = -1
            continue
        off, first, last = L0 % bs, L0 // bs, (L0 + n - 1) // bs
        old = int(st["table"][b][first]) if off > 0 else -1
        cow = off > 0 and ref0[old] > 1
        need = (last - first + 1) - (1 if off > 0 else 0) + (1 if cow else 0)
        if stopped or used + need > nf:
            stopped = True
            status[b] = -2
            continue
        used += need
        status[b] = n
        plans.append((b, L0, n, old if cow else -1, first, last, off, path))

    # allocation: pop from the top, request by request, the copy block first
    top = nf
    for (b, L0, n, old, first, last, off, path) in plans:
        if old >= 0:
            top -= 1
            nb = int(st["free_ids"][top])
            st["k"][nb, :off] = st["k"][old, :off]
            st["v"][nb, :off] = st["v"][old, :off]
            st["table"][b][first] = nb
            st["ref"][nb] = 1
        for t in range(first + (1 if off > 0 else 0), last + 1):
            top -= 1
            nb = int(st["free_ids"][top])
            st["table"][b][t] = nb
            st["ref"][nb] = 1
        for j, p in enumerate(path):
            t = L0 + j
            blk = st["table"][b][t // bs]
            st["k"][blk, t % bs] = k_tree[b, p]
            st["v"][blk, t % bs] = v_tree[b, p]
        st["len"][b] = L0 + n

    # copied blocks lose their copiers as holders; the ones left with none go
    # back on the stack, ordered by their lowest-index copier
    copiers: Dict[int, List[int]] = {}
    for (b, _L0, _n, old, *_rest) in plans:
        if old >= 0:
            copiers.setdefault(old, []).append(b)
    freed = []
    for old, bl in copiers.items():
        st["ref"][old] -= len(bl)
        if st["ref"][old] == 0:
            freed.append((min(bl), old))
    for _, old in sorted(freed):
        st["free_ids"][top] = old
        top += 1
    st["n_free"] = top
    return status


def fork(st: Dict, src: np.ndarray, dst: np.ndarray) -> np.ndarray:
    """Pairs in order: dst takes src's blocks (each gains a holder) and length.
    A pair is skipped (status -1) unless dst holds nothing and is no src."""
    B = st["table"].shape[0]
    srcs = {int(x) for x in src}
    status = np.zeros(len(src), np.int32)
    for i, (s, d) in enumerate(zip(src, dst)):
        s, d = int(s), int(d)
        ok = 0 <= s < B and 0 <= d < B and s != d and d not in srcs \
            and st["len"][d] == 0 and st["table"][d][0] == -1
        if not ok:
            status[i] = -1
            continue
        st["table"][d] = st["table"][s]
        st["len"][d] = st["len"][s]
        for x in st["table"][s]:
            if x >= 0:
                st["ref"][x] += 1
    return status


def release(st: Dict, req: np.ndarray) -> None:
    """Requests in order: each block loses a holder, blocks left with none are
    pushed in table order, and the request's row and length are cleared."""
    B = st["table"].shape[0]
    for r in req:
        r = int(r)
        if not 0 <= r < B:
            continue
        for t, x in enumerate(st["table"][r]):
            if x < 0:
                continue
            st["ref"][x] -= 1
            if st["ref"][x] == 0:
                st["free_ids"][st["n_free"]] = x
                st["n_free"] += 1
            st["table"][r][t] = -1
        st["len"][r] = 0

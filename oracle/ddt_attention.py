"""CPU oracle for tree attention in the verify forward.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the bench's CPU-baseline leg
may import or run this module.  The HIP product path never calls it, and the
two share no code: this file imports numpy only.

What it computes, from the pages:
  * EAGLE-2 explainer (pinghaoyang.com.cn, "EAGLE-2 完全拆解"): the target model
    scores the whole flattened tree in one forward; each tree token sees the
    context and its own ancestors (itself included) and never a sibling
    (reranking section and the engineering-difficulties section on the mask).
  * Graft review (paper.rainbus.top): the hybrid tree is flattened with the
    same ancestor mask before that one forward (execution-flow step 3), and
    the experiments compare against a standard scaled dot-product attention.

Attention itself is the textbook scaled dot-product form with grouped key and
value heads: query head h reads key/value head h // (Hq / Hkv) (reading: the
pages name no head layout; this is the usual grouped-query convention).  The
oracle finds each query's visible tree positions by walking the flat parent
chain, not by reading a bitmask, so that a mask built elsewhere is checked
against the tree itself.  Everything is float64.
"""
from __future__ import annotations

from typing import List

import numpy as np


def visible_positions(parent: np.ndarray, i: int) -> List[int]:
    """Flat positions tree token i attends to: i and its ancestors, root last.

    EAGLE-2 explainer, mask paragraphs: ancestors only, self included."""
    out = []
    j = i
    while j >= 0:
        out.append(j)
        j = int(parent[j])
    return out


def tree_attention(q: np.ndarray, k_pre: np.ndarray, v_pre: np.ndarray, k_tree: np.ndarray,
                   v_tree: np.ndarray, parent: np.ndarray, n: int, scale: float) -> np.ndarray:
    """Attention output of one request's flattened tree.

    q [P][Hq][D]; k_pre, v_pre [L][Hkv][D] (L may be 0); k_tree, v_tree [P][Hkv][D];
    parent [P] flat parent index (-1 at the root); n = number of verified flat
    positions (m + 1).  Query i <= n - 1 attends to every prefix position and
    to visible_positions(i); its weights are softmax(scale * q . k).  Returns
    out [P][Hq][D] in float64, zero at positions n..P-1.
    """
    q = np.asarray(q, np.float64)
    P, Hq, D = q.shape
    L = k_pre.shape[0]
    Hkv = k_tree.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.zeros((P, Hq, D))
    for i in range(n):
        vis = visible_positions(parent, i)
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([np.asarray(k_pre[:, g, :], np.float64),
                                   np.asarray(k_tree[vis, g, :], np.float64)])
            vals = np.concatenate([np.asarray(v_pre[:, g, :], np.float64),
                                   np.asarray(v_tree[vis, g, :], np.float64)])
            s = scale * (keys @ q[i, h])
            w = np.exp(s - s.max())
            out[i, h] = (w / w.sum()) @ vals
    return out

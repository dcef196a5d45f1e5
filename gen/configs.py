"""The five synthetic workloads the draft-tree round is tested and measured on.

Each workload fixes the batch, vocabulary, logit dtype, tree budgets and verify
mode. The tree budgets follow the pages: depth 6 / expand 10 / 60 draft tokens
from the EAGLE-2 explainer's "why a dynamic tree is not better when bigger"
section, the CAST cost-table and threshold knobs from the CAST notes' key
designs 1-4, and K_max = 60 with 8/24/40 stage budgets and an 8x8 retrieval
template from the Graft review's execution-flow and weaknesses paragraphs.
Vocabulary sizes are those of the model families the pages evaluate on.

This module holds workload descriptions only, no part of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class CastSpec:
    """CAST thresholds and cost-table grid (CAST notes, key designs 1-4).

    With the cost slope lam = 0.02, C1 = 1 is the break-even point (a node must
    add 0.02 expected accepted tokens to pay for 0.02 of a target forward).  On
    this synthetic draft distribution (one planted token per row over a
    128K-token Gaussian tail) break-even never pays for a second branch and the
    tree collapses to a chain, so the workload uses thresholds 20x lower, at
    which every width, depth and verify-count decision is exercised within the
    configured depth-8 / width-10 / 60-token budget.  BREAK_EVEN keeps the
    break-even setting for comparison.
    """
    C1: float = 0.05         # width threshold, same for every layer
    C2: float = 0.005        # depth threshold
    C3: float = 0.02         # verify-count threshold (per row)
    R: int = 3               # FIFO length of the depth gain buffer
    L: int = 256             # context grid step of the cost table
    M: int = 16              # context grid rows
    N: int = 128             # token-count columns (n = 1..N)
    lam: float = 0.02        # closed-form cost slope
    delta: float = 1.0       # closed-form cost intercept
    table: str = "linear"    # "linear" (c_k = lam*k + delta), "seeded" or "roofline"
    table_B: int = 0         # batch of the "roofline" table (0: the workload's B)


BREAK_EVEN = dict(C1=1.0, C2=0.1, C3=0.5)


@dataclass(frozen=True)
class ProxyShape:
    """Decoder shape behind the "roofline" cost tables: an 8B-class target
    (32 layers, 32 query / 8 key-value heads of 128, FFN 14336, vocabulary
    128256) and a one-layer draft head of the same width."""
    d_model: int
    n_layers: int
    Hq: int
    Hkv: int
    D: int
    ffn: int
    V: int


PROXY_TARGET = ProxyShape(4096, 32, 32, 8, 128, 14336, 128256)
PROXY_DRAFT = ProxyShape(4096, 1, 32, 8, 128, 14336, 128256)


@dataclass(frozen=True)
class GraftSpec:
    """Graft hybrid-tree knobs (Graft review, execution-flow paragraph)."""
    K_max: int = 60
    ck_depth: Tuple[int, ...] = (1, 2, 6)     # tree depths of checkpoints d0, d1, d5
    k_draft: Tuple[int, ...] = (8, 24, 40)    # draft nodes kept when pruned there
    tpl_depth: int = 8
    tpl_width: int = 8
    k_succ: int = 8                           # successors per row of M
    zipf_s: float = 1.1
    plant_prob: float = 0.5                   # target rows that follow M0's top successor
    # "prune_then_graft" (the method), or the two grafts it is compared with
    # (Graft review, Fig. 2): "root_only" and "tail_only" keep a fixed draft
    # budget with no checkpoints and hang the template off the root or off
    # the tail of the draft tree
    mode: str = "prune_then_graft"
    fixed_k_draft: int = 24


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    V: int
    dtype: str               # "f32" or "bf16"
    D: int                   # draft layers below the root
    K_e: int                 # expand budget (frontier size)
    K_n: int                 # children per expanded node (vocab top-k)
    m: int                   # verify budget (draft nodes, root excluded)
    verify: str              # "greedy", "t1", "mixed" (greedy or T = 1 per row) or "tmix" (T in {0, 0.7, 1, 1.6})
    sigma: float             # target = draft + N(0, sigma) noise (sigma = std dev)
    prefix: int = 0          # context prefix length in front of the tree
    cast: Optional[CastSpec] = None
    graft: Optional[GraftSpec] = None
    # T > 0 verify of draft children: "point" (point-mass proposals, for the
    # deterministic top-k children the tree builder attaches) or "draft"
    # (q = the draft row's softmax, the proposal of sampled children)
    proposal: str = "point"

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def m_max(self) -> int:
        return self.graft.K_max if self.graft else self.m

    @property
    def R_max(self) -> int:
        return self.K_e

    def nodes_cap(self) -> int:
        """Upper bound on nodes per row: root + every layer's children (+ template)."""
        n = 1 + self.K_n + (self.D - 1) * self.K_e * self.K_n
        if self.graft:
            n += self.graft.tpl_depth * self.graft.tpl_width
        return n


C1 = Workload("eagle2_b1_v32000_f32", B=1, V=32000, dtype="f32", D=6, K_e=10, K_n=10,
              m=60, verify="greedy", sigma=0.5)
C2 = Workload("cast_b8_v128256_bf16", B=8, V=128256, dtype="bf16", D=8, K_e=10, K_n=10,
              m=60, verify="greedy", sigma=0.5, cast=CastSpec())
C3 = Workload("eagle2_t1_b8_v152064_bf16", B=8, V=152064, dtype="bf16", D=6, K_e=10,
              K_n=10, m=60, verify="t1", sigma=0.7)
C4 = Workload("graft_b16_v152064_bf16", B=16, V=152064, dtype="bf16", D=8, K_e=8, K_n=8,
              m=60, verify="greedy", sigma=0.5, graft=GraftSpec())
C5 = Workload("eagle2_mixed_b64_v128256_bf16", B=64, V=128256, dtype="bf16", D=10,
              K_e=16, K_n=16, m=128, verify="mixed", sigma=0.5, prefix=4096)

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4, C5)}
ORDER = (C1, C2, C3, C4, C5)


def shrink(w: Workload, V: int, B: Optional[int] = None, **kw) -> Workload:
    """The same workload at a smaller vocabulary (and optionally batch)."""
    d = dict(w.__dict__)
    d.update(name=f"{w.name}@V{V}", V=V)
    if B is not None:
        d["B"] = B
    d.update(kw)
    return Workload(**d)

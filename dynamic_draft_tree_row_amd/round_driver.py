"""One speculative-decoding round composed from the library calls.

draft(): layers 1..D of ddt_tree_expand (EAGLE-2 expansion; CAST width/depth or
the Graft gate when given), then ddt_tree_select (rerank and flat layout in one
launch), or for Graft ddt_tree_rerank, ddt_succ_gather and ddt_tree_build_mask.  verify(): ddt_tree_verify and, for Graft,
ddt_succ_update.  Between the two a serving engine runs the target forward over
the flattened tree; here the caller supplies the target logits.

All layers are enqueued without a host synchronisation: rows that stop early
(Graft prune, CAST depth gate) carry a zero frontier width on the device and
the later layers' kernels skip them.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import api


@dataclass
class RoundShape:
    B: int
    V: int
    dtype: torch.dtype
    D: int
    K_e: int
    K_n: int
    m: int                       # verify budget (Graft: K_max)
    prefix: int = 0
    graft: bool = False
    tpl_depth: int = 8
    tpl_width: int = 8
    k_succ: int = 8
    shared_M: bool = False       # Graft: one successor matrix [V][k] for every row
    graft_anchor: int = 0        # Graft template under the root (0) or the draft tree's tail (1)

    @property
    def m_max(self) -> int:
        return self.m

    @property
    def Dp(self) -> int:
        if not self.graft:
            return self.D
        if self.graft_anchor == 1:
            return min(self.D + self.tpl_depth, 11)        # the canonical key's depth limit
        return max(self.D, self.tpl_depth)

    @property
    def cap(self) -> int:
        n = 1 + self.K_n + (self.D - 1) * self.K_e * self.K_n
        return n + (self.tpl_depth * self.tpl_width if self.graft else 0)

    @property
    def P(self) -> int:
        return self.m + 1


class RoundRunner:
    def __init__(self, shape: RoundShape, device="cuda"):
        s = self.shape = shape
        self.device = device
        self.tree = api.DeviceTree(s.B, s.cap, s.D, s.K_e, device)
        self.flat = api.DeviceFlat(s.B, s.m_max, s.Dp, device)
        i32 = dict(dtype=torch.int32, device=device)
        self.sel = torch.full((s.B, s.m_max + 1), -1, **i32)
        self.m_out = torch.zeros(s.B, **i32)
        self.accept_len = torch.zeros(s.B, **i32)
        self.accept_path = torch.full((s.B, s.Dp + 1), -1, **i32)
        self.next_token = torch.zeros(s.B, **i32)
        self.row_argmax = torch.zeros((s.B, s.P), **i32)
        self.k_top = s.k_succ if s.graft else 0
        self.row_topk = torch.zeros((s.B, s.P, self.k_top), **i32) if s.graft else None
        need = max(api.workspace_bytes(s.B * s.K_e, s.V, s.dtype, s.K_n),
                   api.workspace_bytes(s.B * s.P, s.V, s.dtype, max(1, self.k_top)))
        self.ws = torch.empty(need, dtype=torch.uint8, device=device)

    def draft(self, draft_arena: torch.Tensor, root_tok: torch.Tensor,
              cast: Optional[api.CastParams] = None, gate: Optional[api.GraftGate] = None,
              M: Optional[torch.Tensor] = None, stream=None) -> None:
        """draft_arena: [D][B][K_e][V] draft logits, layer d's slice at [d-1]."""
        s = self.shape
        for d in range(1, s.D + 1):
            api.tree_expand(self.tree, d, root_tok, draft_arena[d - 1], s.K_n, s.K_e, self.ws,
                            cast=cast, gate=gate, stream=stream)
        if not s.graft:
            api.tree_select(self.tree, s.m_max, self.sel, self.m_out, s.prefix, self.flat, cast=cast,
                            use_k_draft=gate is not None, stream=stream)
            return
        api.tree_rerank(self.tree, s.m_max, self.sel, self.m_out, cast=cast,
                        use_k_draft=gate is not None, stream=stream)
        api.succ_gather(self.tree, M, s.k_succ, s.tpl_depth, s.tpl_width, s.m_max, s.m_max,
                        self.sel, self.m_out, shared=s.shared_M, anchor=s.graft_anchor,
                        stream=stream)
        api.tree_build_mask(self.tree, self.sel, self.m_out, s.prefix, self.flat, stream=stream)

    def verify(self, target: torch.Tensor, draft_arena: Optional[torch.Tensor],
               temperature: torch.Tensor, uniforms: torch.Tensor,
               M: Optional[torch.Tensor] = None, stream=None, proposal: str = "point") -> None:
        """target: [B][m_max+1][V] in flat order.  proposal: how T > 0 rows
        verify draft children ("point": as the deterministic top-k choices
        they are; "draft": as samples of the draft row)."""
        api.tree_verify(self.tree, self.flat, target, draft_arena, temperature, uniforms,
                        self.accept_len, self.accept_path, self.next_token, self.ws,
                        k_top=self.k_top, row_topk=self.row_topk, row_argmax=self.row_argmax,
                        proposal=proposal, stream=stream)
        if self.shape.graft:
            api.succ_update(M, self.flat, self.shape.k_succ, row_topk=self.row_topk,
                            k_top=self.k_top, shared=self.shape.shared_M, stream=stream)

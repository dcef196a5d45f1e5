"""Thin torch-facing wrappers over the C ABI (include/ddt.h).

Torch only provides device memory and the stream; every step of the round runs
in the library's HIP kernels.  Names follow the C calls without the ``ddt_``
prefix.  All tensors must live on the same ROCm device.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

from . import _lib as L

_DT = {torch.float32: L.DDT_F32, torch.bfloat16: L.DDT_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None, device=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")
    return _DT[t.dtype]


def logits_desc(x: torch.Tensor) -> L.Logits:
    """Descriptor of a [n0][n1][V] logit tensor with unit stride along V."""
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("logits must be 3-D [n0][n1][V] with contiguous rows")
    return L.Logits(C.c_void_p(x.data_ptr()), dtype_code(x), x.shape[2], x.stride(0), x.stride(1))


def chunk_elems(dtype) -> int:
    return L.load().ddt_chunk_elems(_DT[dtype] if isinstance(dtype, torch.dtype) else dtype)


def workspace_bytes(rows: int, V: int, dtype, K: int) -> int:
    code = _DT[dtype] if isinstance(dtype, torch.dtype) else dtype
    return int(L.load().ddt_workspace_bytes(rows, V, code, K))


class _Carved:
    """A caller-owned device buffer carved into typed views by the library."""

    def _view(self, ptr: int, dtype, shape):
        off = ptr - self.buf.data_ptr()
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.buf[off:off + nbytes].view(dtype).view(*shape)


class DeviceTree(_Carved):
    """Tree state for B rows of at most `cap` nodes (include/ddt.h, ddt_tree)."""

    def __init__(self, B: int, cap: int, D_max: int, R_max: int, device="cuda"):
        lib = L.load()
        nbytes = int(lib.ddt_tree_bytes(B, cap, D_max, R_max))
        if nbytes == 0:
            raise ValueError("invalid tree sizes")
        self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.c = L.Tree()
        L.check("ddt_tree_bind", lib.ddt_tree_bind(C.byref(self.c), C.c_void_p(self.buf.data_ptr()),
                                                   nbytes, B, cap, D_max, R_max))
        self.B, self.cap, self.D_max, self.R_max = B, cap, D_max, R_max
        c = self.c
        v = self._view
        self.token = v(c.token, torch.int32, (B, cap))
        self.parent = v(c.parent, torch.int32, (B, cap))
        self.depth = v(c.depth, torch.int32, (B, cap))
        self.eslot = v(c.eslot, torch.int32, (B, cap))
        self.key = v(c.key, torch.int64, (B, cap))
        self.S = v(c.S, torch.float32, (B, cap))
        self.logc = v(c.logc, torch.float32, (B, cap))
        self.rmax = v(c.rmax, torch.float32, (B, D_max, R_max))
        self.rsp = v(c.rsp, torch.float32, (B, D_max, R_max))
        self.n_nodes = v(c.n_nodes, torch.int32, (B,))
        self.n_front = v(c.n_front, torch.int32, (B,))
        self.frontier = v(c.frontier, torch.int32, (B, R_max))
        self.active = v(c.active, torch.int32, (B,))
        self.k_draft = v(c.k_draft, torch.int32, (B,))
        self.cont = v(c.cont, torch.int32, (1,))
        self.widths = v(c.widths, torch.int32, (D_max,))
        self.walk_sync = v(c.walk_sync, torch.int32, (B, 2))


class DeviceFlat(_Carved):
    """Flattened tree buffers (include/ddt.h, ddt_flat)."""

    def __init__(self, B: int, m_max: int, Dp: int, device="cuda"):
        lib = L.load()
        nbytes = int(lib.ddt_flat_bytes(B, m_max, Dp))
        if nbytes == 0:
            raise ValueError("invalid flat sizes")
        self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.c = L.Flat()
        L.check("ddt_flat_bind", lib.ddt_flat_bind(C.byref(self.c), C.c_void_p(self.buf.data_ptr()),
                                                   nbytes, B, m_max, Dp))
        c = self.c
        self.B, self.P, self.W, self.Dp, self.L = c.B, c.P, c.W, c.Dp, c.L
        v = self._view
        P, W = c.P, c.W
        self.node = v(c.node, torch.int32, (B, P))
        self.token = v(c.token, torch.int32, (B, P))
        self.parent = v(c.parent, torch.int32, (B, P))
        self.pos = v(c.pos, torch.int32, (B, P))
        self.mask = v(c.mask, torch.int32, (B, P, W))
        self.retrieve = v(c.retrieve, torch.int32, (B, c.L, Dp + 1))
        self.n_leaves = v(c.n_leaves, torch.int32, (B,))
        self.m = v(c.m, torch.int32, (B,))


@dataclass
class CastParams:
    """CAST tables and thresholds on the device (include/ddt.h, ddt_cast)."""
    S_T: torch.Tensor          # fp32 [M][N+1]
    S_D: torch.Tensor          # fp32 [M][N+1]
    L: int
    C1: torch.Tensor           # fp32 [D_max]
    C2: float
    C3: torch.Tensor           # fp32 [B]
    R: int
    ctx_verify: int = 0

    def struct(self) -> L.Cast:
        M, N1 = self.S_T.shape
        return L.Cast(_ptr(self.S_T), _ptr(self.S_D), self.L, M, N1 - 1, _ptr(self.C1),
                      float(self.C2), _ptr(self.C3), self.R, self.ctx_verify)


@dataclass
class GraftGate:
    ck_depth: Sequence[int]
    tau: Sequence[float]
    k_draft: Sequence[int]
    K_max: int

    def struct(self) -> L.Gate:
        g = L.Gate()
        g.n_ck = len(self.ck_depth)
        for i, (d, t, k) in enumerate(zip(self.ck_depth, self.tau, self.k_draft)):
            g.ck_depth[i], g.tau[i], g.k_draft[i] = d, t, k
        g.K_max = self.K_max
        return g


def tree_expand(tree: DeviceTree, layer: int, root_tok: torch.Tensor, logits: torch.Tensor,
                K_n: int, K_e: int, ws: torch.Tensor, cast: Optional[CastParams] = None,
                gate: Optional[GraftGate] = None, stream=None) -> None:
    d = logits_desc(logits)
    cs = C.byref(cast.struct()) if cast is not None else None
    gs = C.byref(gate.struct()) if gate is not None else None
    L.check("ddt_tree_expand", L.load().ddt_tree_expand(
        C.byref(tree.c), layer, _ptr(root_tok), C.byref(d), K_n, K_e, cs, gs, _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream, logits.device)))


def tree_rerank(tree: DeviceTree, m_max: int, sel: torch.Tensor, m_out: torch.Tensor,
                cast: Optional[CastParams] = None, use_k_draft: bool = False, stream=None) -> None:
    cs = C.byref(cast.struct()) if cast is not None else None
    L.check("ddt_tree_rerank", L.load().ddt_tree_rerank(
        C.byref(tree.c), m_max, cs, int(use_k_draft), _ptr(sel), _ptr(m_out),
        _stream(stream, sel.device)))


def succ_gather(tree: DeviceTree, M: torch.Tensor, k_succ: int, tpl_depth: int, tpl_width: int,
                K_max: int, m_max: int, sel: torch.Tensor, m_out: torch.Tensor, shared: bool = False,
                anchor: int = 0, stream=None) -> None:
    """ddt_succ_gather (anchor 0, the root) or ddt_succ_gather_at (anchor 1:
    the tail of the selected draft tree)."""
    V = M.shape[-2]
    bstride = 0 if shared else V * k_succ
    if anchor == 0:
        L.check("ddt_succ_gather", L.load().ddt_succ_gather(
            C.byref(tree.c), _ptr(M), bstride, V, k_succ, tpl_depth, tpl_width, K_max, m_max,
            _ptr(sel), _ptr(m_out), _stream(stream, M.device)))
    else:
        L.check("ddt_succ_gather_at", L.load().ddt_succ_gather_at(
            C.byref(tree.c), _ptr(M), bstride, V, k_succ, tpl_depth, tpl_width, K_max, m_max,
            anchor, _ptr(sel), _ptr(m_out), _stream(stream, M.device)))


def tree_build_mask(tree: DeviceTree, sel: torch.Tensor, m: torch.Tensor, prefix_len: int,
                    flat: DeviceFlat, dense: Optional[torch.Tensor] = None, stream=None) -> None:
    L.check("ddt_tree_build_mask", L.load().ddt_tree_build_mask(
        C.byref(tree.c), _ptr(sel), _ptr(m), prefix_len, C.byref(flat.c), _ptr(dense),
        _stream(stream, sel.device)))


def tree_select(tree: DeviceTree, m_max: int, sel: torch.Tensor, m_out: torch.Tensor, prefix_len: int,
                flat: DeviceFlat, cast: Optional[CastParams] = None, use_k_draft: bool = False,
                dense: Optional[torch.Tensor] = None, stream=None) -> None:
    """ddt_tree_select: tree_rerank and tree_build_mask in one launch."""
    cs = C.byref(cast.struct()) if cast is not None else None
    L.check("ddt_tree_select", L.load().ddt_tree_select(
        C.byref(tree.c), m_max, cs, int(use_k_draft), _ptr(sel), _ptr(m_out), prefix_len,
        C.byref(flat.c), _ptr(dense), _stream(stream, sel.device)))


PROPOSALS = {"draft": L.DDT_PROPOSAL_DRAFT, "point": L.DDT_PROPOSAL_POINT}


def tree_verify(tree: DeviceTree, flat: DeviceFlat, target: torch.Tensor,
                draft_arena: Optional[torch.Tensor], temperature: torch.Tensor,
                uniforms: torch.Tensor, accept_len: torch.Tensor, accept_path: torch.Tensor,
                next_token: torch.Tensor, ws: torch.Tensor, k_top: int = 0,
                row_topk: Optional[torch.Tensor] = None, row_argmax: Optional[torch.Tensor] = None,
                proposal: str = "point", stream=None) -> None:
    """target: [B][P][V]; draft_arena: [D][B][R][V] (layer-major) or None;
    proposal: "point" (children verified as point-mass proposals; the draft
    arena is not read) or "draft" (q = the draft row's softmax)."""
    td = logits_desc(target)
    if draft_arena is not None:
        dd = logits_desc(draft_arena[0])
        dref, dls = C.byref(dd), draft_arena.stride(0)
    else:
        dref, dls = None, 0
    L.check("ddt_tree_verify", L.load().ddt_tree_verify(
        C.byref(tree.c), C.byref(flat.c), C.byref(td), dref, dls, _ptr(temperature),
        _ptr(uniforms), PROPOSALS[proposal], k_top, _ptr(row_topk), _ptr(row_argmax), _ptr(accept_len),
        _ptr(accept_path), _ptr(next_token), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, target.device)))


def set_walk_spin_limit(polls: int) -> int:
    """ddt_set_walk_spin_limit: polls before a T > 0 walk's cross-workgroup
    wait gives up (0 restores the default); returns the previous value."""
    return int(L.load().ddt_set_walk_spin_limit(int(polls)))


def succ_update(M: torch.Tensor, flat: DeviceFlat, k_succ: int, row_topk: Optional[torch.Tensor] = None,
                k_top: int = 0, target: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                shared: bool = False, stream=None) -> None:
    V = M.shape[-2]
    bstride = 0 if shared else V * k_succ
    td = C.byref(logits_desc(target)) if target is not None else None
    wsz = ws.numel() * ws.element_size() if ws is not None else 0
    L.check("ddt_succ_update", L.load().ddt_succ_update(
        _ptr(M), bstride, V, k_succ, C.byref(flat.c), _ptr(row_topk), k_top, td, _ptr(ws), wsz,
        _stream(stream, M.device)))


def attention_splits(B: int, P: int, Hq: int, Hkv: int, ctx: int, splits: int = 0) -> Tuple[int, int]:
    """(split count, workspace bytes) of ddt_tree_attention_split for these
    sizes (ctx: context positions)."""
    lib = L.load()
    return (int(lib.ddt_tree_attention_splits(B, P, Hq, Hkv, ctx, splits)),
            int(lib.ddt_tree_attention_ws_bytes(B, P, Hq, Hkv, ctx, splits)))


def tree_attention(flat: DeviceFlat, q: torch.Tensor, k_tree: torch.Tensor, v_tree: torch.Tensor,
                   out: torch.Tensor, k_pre: Optional[torch.Tensor] = None,
                   v_pre: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                   stream=None, splits: Optional[int] = None,
                   ws: Optional[torch.Tensor] = None) -> None:
    """ddt_tree_attention: q [B][P][Hq][D], k/v_tree [B][P][Hkv][D], k/v_pre [B][L][Hkv][D]
    (bf16, contiguous); out fp32 [B][P][Hq][D].  splits (0 = the library's
    choice) calls ddt_tree_attention_split instead, with ws (uint8, device) or
    a workspace allocated here."""
    B, P, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    Lp = 0 if k_pre is None else k_pre.shape[1]
    for t in (q, k_tree, v_tree) + ((k_pre, v_pre) if Lp else ()):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("tree_attention takes contiguous bf16 tensors")
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (B, P, Hq, D):
        raise ValueError("out must be contiguous fp32 [B][P][Hq][D]")
    a = L.Attn(_ptr(q), _ptr(k_pre) if Lp else None, _ptr(v_pre) if Lp else None, _ptr(k_tree),
               _ptr(v_tree), B, P, Hq, Hkv, D, Lp, float(scale if scale is not None else D ** -0.5))
    if splits is None:
        L.check("ddt_tree_attention", L.load().ddt_tree_attention(C.byref(flat.c), C.byref(a), _ptr(out),
                                                                    _stream(stream, q.device)))
        return
    _, need = attention_splits(B, P, Hq, Hkv, Lp, splits)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    L.check("ddt_tree_attention_split", L.load().ddt_tree_attention_split(
        C.byref(flat.c), C.byref(a), _ptr(out), splits, _ptr(ws), nbytes, _stream(stream, q.device)))


def row_topk(x: torch.Tensor, K: int, ws: torch.Tensor, ids: Optional[torch.Tensor] = None,
             logc: Optional[torch.Tensor] = None, rmax: Optional[torch.Tensor] = None,
             rsp: Optional[torch.Tensor] = None, stream=None) -> None:
    d = logits_desc(x)
    L.check("ddt_row_topk", L.load().ddt_row_topk(
        C.byref(d), x.shape[0], x.shape[1], K, _ptr(ids), _ptr(logc), _ptr(rmax), _ptr(rsp),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream, x.device)))


def row_topk_noalloc(x: torch.Tensor, K: int, ids: Optional[torch.Tensor] = None,
                     logc: Optional[torch.Tensor] = None, rmax: Optional[torch.Tensor] = None,
                     rsp: Optional[torch.Tensor] = None, stream=None) -> None:
    """ddt_row_topk_noalloc: the row reduction with its partials in the
    library's fixed per-device array (no workspace, nothing allocated)."""
    d = logits_desc(x)
    L.check("ddt_row_topk_noalloc", L.load().ddt_row_topk_noalloc(
        C.byref(d), x.shape[0], x.shape[1], K, _ptr(ids), _ptr(logc), _ptr(rmax), _ptr(rsp),
        _stream(stream, x.device)))


class PagedKV:
    """The caller-owned arrays of a block-paged KV context (ddt_kv_cache) on
    one device: k, v bf16 [n_blocks][block][Hkv][D], table [B][max_blocks],
    len [B], ref [n_blocks], a free stack with block 0 on top, and the commit's
    plan scratch.  The methods bind the three calls; all state stays on the
    device."""

    def __init__(self, B: int, max_blocks: int, n_blocks: int, block: int, Hkv: int, D: int,
                 device="cuda"):
        i32 = dict(dtype=torch.int32, device=device)
        self.k = torch.zeros(n_blocks, block, Hkv, D, dtype=torch.bfloat16, device=device)
        self.v = torch.zeros_like(self.k)
        self.table = torch.full((B, max_blocks), -1, **i32)
        self.len = torch.zeros(B, **i32)
        self.ref = torch.zeros(n_blocks, **i32)
        self.free_ids = torch.arange(n_blocks - 1, -1, -1, **i32)
        self.n_free = torch.tensor([n_blocks], **i32)
        self.plan = torch.zeros(B, 4, **i32)
        self.B, self.max_blocks, self.n_blocks, self.block, self.Hkv, self.D = \
            B, max_blocks, n_blocks, block, Hkv, D
        self.c = L.KVCache(_ptr(self.k), _ptr(self.v), _ptr(self.table), _ptr(self.len), _ptr(self.ref),
                           _ptr(self.free_ids), _ptr(self.n_free), _ptr(self.plan),
                           B, max_blocks, n_blocks, block, Hkv, D)

    def commit(self, accept_len: torch.Tensor, accept_path: torch.Tensor, k_tree: torch.Tensor,
               v_tree: torch.Tensor, status: torch.Tensor, stream=None) -> None:
        """ddt_kv_commit: accept_path [B][Dp+1] int32; k/v_tree bf16 [B][P][Hkv][D]."""
        B, P = k_tree.shape[0], k_tree.shape[1]
        if B != self.B or tuple(k_tree.shape[2:]) != (self.Hkv, self.D) or v_tree.shape != k_tree.shape:
            raise ValueError("k_tree / v_tree must be [B][P][Hkv][D] of this cache")
        for t in (k_tree, v_tree):
            if t.dtype != torch.bfloat16 or not t.is_contiguous():
                raise ValueError("k_tree / v_tree must be contiguous bf16")
        for t in (accept_len, accept_path, status):
            if t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError("accept_len, accept_path and status must be contiguous int32")
        L.check("ddt_kv_commit", L.load().ddt_kv_commit(
            C.byref(self.c), _ptr(accept_len), _ptr(accept_path), accept_path.shape[1] - 1,
            _ptr(k_tree), _ptr(v_tree), P, _ptr(status), _stream(stream, k_tree.device)))

    def fork(self, src: torch.Tensor, dst: torch.Tensor, status: torch.Tensor, stream=None) -> None:
        """ddt_kv_fork over int32 [n] device vectors."""
        L.check("ddt_kv_fork", L.load().ddt_kv_fork(C.byref(self.c), _ptr(src), _ptr(dst), src.numel(),
                                                    _ptr(status), _stream(stream, src.device)))

    def release(self, req: torch.Tensor, stream=None) -> None:
        """ddt_kv_release over an int32 [n] device vector."""
        L.check("ddt_kv_release", L.load().ddt_kv_release(C.byref(self.c), _ptr(req), req.numel(),
                                                          _stream(stream, req.device)))

"""CAST inference-cost tables measured on this GPU.

CAST (papernotes.org notes, key design 1) reads the cost of growing the tree
from a table f(B, c, n), the time of one forward with batch B, context c and n
input tokens, measured offline on the deployment GPU and kept per batch size as
S_T(B) (target model) and S_D(B) (draft model), sampled at c = k*L (rows
k = 0 .. M-1) and n = 1 .. N (columns; column 0, no tokens, costs 0).  The
notes' section on limitations adds that the table has to be measured again for
every GPU and batch size; this module is that measurement.

It times proxy forwards of named model shapes with random bf16 weights: one
decoder layer, timed and multiplied by the layer count, plus the LM head.  A
layer is the QKV projection, attention of the n new positions over the c
context positions and over their own causal prefix (this library's tree
attention with a chain-shaped tree, key-split when the batch is small), the
output projection and a gated FFN
with residual adds; the projections are library GEMMs with weights stored
[out][in] as checkpoints hold them (torch.nn.functional.linear, hipBLASLt on
this device).  Each timed unit is captured once in a HIP graph and
replayed, so host launch cost does not enter the table (serving stacks replay
their decode forwards from graphs too), and consecutive layers in the graph use
different weight and context copies, so that weights stream from HBM as they
do in a real forward instead of being served from the last-level cache.
Measured times are made non-decreasing in n (a running maximum): a longer
input never costs less than a shorter one.

The tables feed ddt_tree_expand / ddt_tree_rerank through api.CastParams
(S_T, S_D as [M][N+1] float32, grid step L); the width and verify costs are
ratios of table entries, so the unit (microseconds here) cancels.
"""
from __future__ import annotations

from dataclasses import astuple, dataclass
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class ProxyModel:
    """Shape of a decoder-only model for cost measurement (weights are random)."""
    d_model: int
    n_layers: int
    Hq: int
    Hkv: int
    D: int
    ffn: int
    V: int

    def layer_weight_bytes(self) -> int:
        """bf16 bytes of one layer's projections (QKV, output, gate+up, down)."""
        d = self.d_model
        return 2 * (d * (self.Hq + 2 * self.Hkv) * self.D + self.Hq * self.D * d + 3 * d * self.ffn)

    def head_weight_bytes(self) -> int:
        return 2 * self.d_model * self.V


# an 8B-class target with the 128256-token vocabulary of the bench workloads,
# and a one-layer draft head of the same width (EAGLE-style draft)
TARGET_8B = ProxyModel(d_model=4096, n_layers=32, Hq=32, Hkv=8, D=128, ffn=14336, V=128256)
DRAFT_HEAD = ProxyModel(d_model=4096, n_layers=1, Hq=32, Hkv=8, D=128, ffn=14336, V=128256)


def assemble(times_layer: np.ndarray, times_head: np.ndarray, n_layers: int) -> np.ndarray:
    """Cost table [M][N+1] from per-(row, n) layer times [M][N] and LM-head
    times [N] (microseconds): column n = n_layers * layer + head, column 0 = 0,
    then a running maximum along n."""
    times_layer = np.asarray(times_layer, np.float64)
    times_head = np.asarray(times_head, np.float64)
    M, N = times_layer.shape
    if times_head.shape != (N,):
        raise ValueError("times_head must have one entry per column")
    t = np.zeros((M, N + 1), np.float64)
    t[:, 1:] = n_layers * times_layer + times_head[None, :]
    t[:, 1:] = np.maximum.accumulate(t[:, 1:], axis=1)
    return t.astype(np.float32)


class _Layer:
    """Weights and context keys/values of one decoder layer on the device."""

    def __init__(self, pm: ProxyModel, B: int, c: int, device, g):
        import torch
        # [out][in], scaled by 1/sqrt(in)
        w = lambda o, i: (torch.randn(o, i, device=device, generator=g) * i ** -0.5).to(torch.bfloat16)
        d = pm.d_model
        self.Wqkv, self.Wo = w((pm.Hq + 2 * pm.Hkv) * pm.D, d), w(d, pm.Hq * pm.D)
        self.Wgu, self.Wd = w(2 * pm.ffn, d), w(d, pm.ffn)
        self.kp = self.vp = None
        if c > 0:
            shp = (B, c, pm.Hkv, pm.D)
            self.kp = torch.randn(*shp, device=device, generator=g).to(torch.bfloat16)
            self.vp = torch.randn(*shp, device=device, generator=g).to(torch.bfloat16)


class _Proxy:
    """Forward pieces of a proxy model for batch B on one device."""

    def __init__(self, pm: ProxyModel, B: int, n_max: int, device, seed: int, copies: int):
        import torch
        from . import api
        self.torch, self.api, self.pm, self.B, self.device = torch, api, pm, B, device
        self.copies = copies
        self.g = torch.Generator(device=device).manual_seed(seed)
        self.x = torch.randn(B * n_max, pm.d_model, device=device, generator=self.g).to(torch.bfloat16)
        self.Wlm = (torch.randn(pm.V, pm.d_model, device=device, generator=self.g)
                    * pm.d_model ** -0.5).to(torch.bfloat16)
        self.layers: List[_Layer] = []
        self.flats: Dict[int, object] = {}

    def set_context(self, c: int):
        self.layers = []
        self.torch.cuda.empty_cache()
        self.layers = [_Layer(self.pm, self.B, c, self.device, self.g) for _ in range(self.copies)]

    def flat(self, n: int):
        """A flat of n positions holding a chain: position i sees 0 .. i."""
        f = self.flats.get(n)
        if f is None:
            torch = self.torch
            f = self.api.DeviceFlat(self.B, n - 1, 1, self.device)
            mask = np.zeros((n, f.W), np.uint32)
            for i in range(n):
                for j in range(i + 1):
                    mask[i, j // 32] |= np.uint32(1 << (j % 32))
            f.mask.copy_(torch.from_numpy(np.broadcast_to(mask, (self.B, n, f.W)).copy().view(np.int32)))
            f.m.fill_(n - 1)
            self.flats[n] = f
        return f

    def layer(self, ly: _Layer, n: int, x):
        torch, pm, B = self.torch, self.pm, self.B
        lin = torch.nn.functional.linear
        hq, hk = pm.Hq * pm.D, pm.Hkv * pm.D
        qkv = lin(x, ly.Wqkv)
        q = qkv[:, :hq].reshape(B, n, pm.Hq, pm.D).contiguous()
        k = qkv[:, hq:hq + hk].reshape(B, n, pm.Hkv, pm.D).contiguous()
        v = qkv[:, hq + hk:].reshape(B, n, pm.Hkv, pm.D).contiguous()
        out = torch.empty(B, n, pm.Hq, pm.D, dtype=torch.float32, device=self.device)
        self.api.tree_attention(self.flat(n), q, k, v, out, k_pre=ly.kp, v_pre=ly.vp, splits=0)
        h = x + lin(out.reshape(B * n, hq).to(torch.bfloat16), ly.Wo)
        gu = lin(h, ly.Wgu)
        f = torch.nn.functional.silu(gu[:, :pm.ffn]) * gu[:, pm.ffn:]
        return h + lin(f, ly.Wd)

    def layers_fn(self, n: int) -> Callable[[], object]:
        def run():
            x = self.x[:self.B * n]
            for ly in self.layers:
                x = self.layer(ly, n, x)
            return x
        return run

    def head_fn(self, n: int) -> Callable[[], object]:
        return lambda: self.torch.nn.functional.linear(self.x[:self.B * n], self.Wlm)


def _graph_time_us(torch, fn: Callable[[], object], units: int, reps: int, pool, side) -> float:
    """Average time of one of the `units` pieces of work fn enqueues, from
    `reps` replays of a HIP graph of fn captured on stream `side`."""
    fn()                                            # library handles and workspaces
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        g.capture_begin(pool=pool)
        fn()
        g.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (reps * units)


def measure_tables(B: int, L: int, M: int, N: int, target: ProxyModel = TARGET_8B,
                   draft: ProxyModel = DRAFT_HEAD, reps: int = 4, copies: int = 2,
                   device="cuda", seed: int = 0,
                   log: Optional[Callable[[str], None]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """S_T, S_D ([M][N+1] float32, microseconds) for batch B: row k is context
    k*L, column n the forward of n new tokens.  N <= 256 (the attention's flat
    positions) and both models need heads of 128."""
    import torch
    if not 1 <= N <= 256 or M < 1 or L < 1 or B < 1 or reps < 1 or copies < 1:
        raise ValueError("need 1 <= N <= 256 and positive B, M, L, reps, copies")
    for pm in (target, draft):
        if pm.D != 128 or pm.Hq % pm.Hkv != 0 or pm.Hq // pm.Hkv > 16:
            raise ValueError("proxy models need heads of 128 and at most 16 query heads per key head")
    # one memory pool for every capture, held by a graph that lives through
    # the whole measurement (a pool whose graphs are all gone cannot be reused)
    pool = torch.cuda.graph_pool_handle()
    side = torch.cuda.Stream()
    one = torch.ones(1, device=device)
    keeper = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        keeper.capture_begin(pool=pool)
        one.add(1.0)
        keeper.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    tabs = []
    for name, pm, s in (("target", target, seed), ("draft", draft, seed + 1)):
        px = _Proxy(pm, B, N, device, s, copies)
        head = np.array([_graph_time_us(torch, px.head_fn(n), 1, reps, pool, side) for n in range(1, N + 1)])
        lay = np.zeros((M, N))
        for k in range(M):
            px.set_context(k * L)
            for n in range(1, N + 1):
                lay[k, n - 1] = _graph_time_us(torch, px.layers_fn(n), copies, reps, pool, side)
            if log:
                log(f"cost table {name} B={B} context {k * L}: n=1 {pm.n_layers * lay[k, 0] + head[0]:.1f} us, "
                    f"n={N} {pm.n_layers * lay[k, -1] + head[-1]:.1f} us")
        tabs.append(assemble(lay, head, pm.n_layers))
        del px
        torch.cuda.empty_cache()
    del keeper
    return tabs[0], tabs[1]


def save_tables(path: str, S_T: np.ndarray, S_D: np.ndarray, B: int, L: int,
                target: ProxyModel = TARGET_8B, draft: ProxyModel = DRAFT_HEAD,
                device: str = "") -> None:
    """Store measured tables with what they were measured for (batch B, grid
    step L, the proxy shapes, the device name): the tables are computed
    offline once per GPU and batch size and read back at serving time.  The
    file is written at `path` as given (through a handle, so no suffix is
    added); load_tables reads the same name."""
    S_T, S_D = np.asarray(S_T, np.float32), np.asarray(S_D, np.float32)
    if S_T.shape != S_D.shape or S_T.ndim != 2 or S_T.shape[1] < 2:
        raise ValueError("S_T and S_D must be [M][N+1] tables of the same shape")
    with open(path, "wb") as fh:
        _savez(fh, S_T, S_D, B, L, target, draft, device)


def _savez(fh, S_T, S_D, B, L, target, draft, device) -> None:
    np.savez(fh, S_T=S_T, S_D=S_D, B=np.int64(B), L=np.int64(L),
             target=np.array(astuple(target), np.int64), draft=np.array(astuple(draft), np.int64),
             device=np.array(device))


def load_tables(path: str) -> dict:
    """Tables stored by save_tables: dict(S_T, S_D, B, L, target, draft, device).
    A path without the file (as numpy's own savez would have named it
    `path`.npz) is looked up with that suffix too."""
    import os
    if not os.path.exists(path) and os.path.exists(path + ".npz"):
        path = path + ".npz"
    with np.load(path, allow_pickle=False) as z:
        return {"S_T": z["S_T"], "S_D": z["S_D"], "B": int(z["B"]), "L": int(z["L"]),
                "target": ProxyModel(*[int(x) for x in z["target"]]),
                "draft": ProxyModel(*[int(x) for x in z["draft"]]), "device": str(z["device"])}

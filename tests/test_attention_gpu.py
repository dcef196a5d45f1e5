"""GPU parity of ddt_tree_attention against the tree-attention oracle.

Random trees in flat order (every parent before its children), masks written
by the test from the parent chains, seeded bf16 queries, keys and values, and
a context prefix of 0, 50 or 300 positions (key blocks that straddle the
prefix/tree boundary).  One case takes its flat tree and mask from a real
round (expand, rerank, build_mask).

Tolerance, from the arithmetic: scores and sums accumulate in fp32 from exact
bf16 products; the attention weights enter the value product rounded to bf16
(relative error at most 2^-9 each), so each output element is off by at most
2^-9 * max|v| over its visible values, plus fp32 rounding.  The test allows
2^-8 * max|v| over the head's values + 1e-5.
"""
import numpy as np
import pytest
import torch

from gen import configs, synth
from oracle import ddt_attention as A
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    from dynamic_draft_tree_row_amd import _lib
    _lib.load()


def _bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest even) and return the float32 values."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def _to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda").to(torch.bfloat16)


def _random_tree(rng, n: int) -> np.ndarray:
    parent = np.full(n, -1, np.int32)
    for i in range(1, n):
        parent[i] = rng.integers(max(0, i - 8), i)         # parents precede children
    return parent


def _mask_rows(parent: np.ndarray, n: int, P: int, W: int) -> np.ndarray:
    rows = np.zeros((P, W), np.uint32)
    for i in range(P):
        j = i if i < n else -1
        if i >= n:
            rows[i, i // 32] |= np.uint32(1 << (i % 32))       # padding: self only
        while j >= 0:
            rows[i, j // 32] |= np.uint32(1 << (j % 32))
            j = int(parent[j])
    return rows


def _check(out, q, kp, vp, kt, vt, parents, ns, scale):
    B = q.shape[0]
    for b in range(B):
        want = A.tree_attention(q[b], kp[b], vp[b], kt[b], vt[b], parents[b], ns[b], scale)
        got = out[b]
        Hq, Hkv = q.shape[2], kt.shape[2]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            vmax = max(np.abs(vt[b, :, g]).max(), np.abs(vp[b, :, g]).max() if vp.shape[1] else 0.0)
            tol = 2.0 ** -8 * vmax + 1e-5
            err = np.abs(got[:, h] - want[:, h]).max()
            assert err <= tol, f"request {b} head {h}: max error {err} > {tol}"


@pytest.mark.parametrize("Lp", [0, 50, 300])
@pytest.mark.parametrize("P,Hq,Hkv", [(61, 8, 2), (129, 4, 4), (20, 2, 1)])
def test_tree_attention_random_trees(Lp, P, Hq, Hkv):
    _random_case(Lp, P, Hq, Hkv)


# key splits (ddt_tree_attention_split): the library's choice (0) and forced
# counts, ragged last splits, a tree-only case (one block: one split), one
# flat position (a decode step over a long context), the CAST verify shape
@pytest.mark.parametrize("Lp,P,Hq,Hkv,splits", [
    (300, 61, 8, 2, 0), (300, 61, 8, 2, 3), (50, 20, 2, 1, 2), (1000, 129, 4, 4, 5),
    (0, 61, 8, 2, 2), (700, 1, 32, 8, 0), (2000, 61, 32, 8, 0), (130, 70, 2, 2, 32)])
def test_tree_attention_key_splits(Lp, P, Hq, Hkv, splits):
    _random_case(Lp, P, Hq, Hkv, splits)


def _random_case(Lp, P, Hq, Hkv, splits=None):
    from dynamic_draft_tree_row_amd import api
    rng = np.random.default_rng(1000 * P + Lp + Hq)
    B, D = 3, 128
    flat = api.DeviceFlat(B, P - 1, 8, "cuda")
    W = flat.W
    ns = [P, max(1, P // 2), 1]                              # full, half, root only
    parents, masks = [], []
    for b in range(B):
        par = _random_tree(rng, P)
        par[ns[b]:] = -1
        parents.append(par)
        masks.append(_mask_rows(par, ns[b], P, W))
    flat.mask.copy_(torch.from_numpy(np.stack(masks).view(np.int32)).to("cuda"))
    flat.m.copy_(torch.tensor([n - 1 for n in ns], dtype=torch.int32, device="cuda"))
    q = _bf16(rng.standard_normal((B, P, Hq, D)))
    kt = _bf16(rng.standard_normal((B, P, Hkv, D)))
    vt = _bf16(rng.standard_normal((B, P, Hkv, D)))
    kp = _bf16(rng.standard_normal((B, Lp, Hkv, D)))
    vp = _bf16(rng.standard_normal((B, Lp, Hkv, D)))
    out = torch.full((B, P, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    used = None if splits is None else api.attention_splits(B, P, Hq, Hkv, Lp, splits)[0]
    print(f"tree_attention P={P} Hq={Hq} Hkv={Hkv} L={Lp} splits={splits} -> {used}", flush=True)
    scale = D ** -0.5
    api.tree_attention(flat, _to_dev(q), _to_dev(kt), _to_dev(vt), out,
                       k_pre=_to_dev(kp) if Lp else None, v_pre=_to_dev(vp) if Lp else None,
                       scale=scale, splits=splits)
    torch.cuda.synchronize()
    _check(out.cpu().numpy(), q, kp, vp, kt, vt, parents, ns, scale)


def test_tree_attention_on_a_round_flat_tree():
    # the flat tree and mask the library writes for a real draft phase
    # (expand, rerank, build_mask) of a small B = 4 mixed workload with a prefix
    from dynamic_draft_tree_row_amd import api
    w = configs.shrink(configs.C5, V=4100, B=4)
    run = H.runner_for(w, "cuda")
    arena = H.to_dev(synth.draft_arena(w, 3, 0), w.dtype)
    roots = torch.from_numpy(synth.root_tokens(w, 3, 0)).to("cuda")
    run.draft(arena, roots)
    torch.cuda.synchronize()
    flat = run.flat
    P, B = flat.P, w.B
    par = flat.parent.cpu().numpy()
    ns = (flat.m.cpu().numpy() + 1).tolist()
    rng = np.random.default_rng(7)
    Hq, Hkv, D, Lp = 8, 2, 128, w.prefix
    q = _bf16(rng.standard_normal((B, P, Hq, D)))
    kt = _bf16(rng.standard_normal((B, P, Hkv, D)))
    vt = _bf16(rng.standard_normal((B, P, Hkv, D)))
    kp = _bf16(rng.standard_normal((B, Lp, Hkv, D)))
    vp = _bf16(rng.standard_normal((B, Lp, Hkv, D)))
    out = torch.zeros((B, P, Hq, D), dtype=torch.float32, device="cuda")
    print(f"tree_attention on a round: P={P} L={Lp} n={ns}", flush=True)
    api.tree_attention(flat, _to_dev(q), _to_dev(kt), _to_dev(vt), out,
                       k_pre=_to_dev(kp) if Lp else None, v_pre=_to_dev(vp) if Lp else None)
    torch.cuda.synchronize()
    _check(out.cpu().numpy(), q, kp, vp, kt, vt, [par[b] for b in range(B)], ns, D ** -0.5)


def test_tree_attention_deterministic():
    from dynamic_draft_tree_row_amd import api
    rng = np.random.default_rng(11)
    B, P, Hq, Hkv, D, Lp = 2, 61, 8, 2, 128, 70
    flat = api.DeviceFlat(B, P - 1, 8, "cuda")
    masks = np.stack([_mask_rows(_random_tree(rng, P), P, P, flat.W) for _ in range(B)])
    flat.mask.copy_(torch.from_numpy(masks.view(np.int32)).to("cuda"))
    flat.m.fill_(P - 1)
    t = [_to_dev(_bf16(rng.standard_normal(s))) for s in
         [(B, P, Hq, D), (B, P, Hkv, D), (B, P, Hkv, D), (B, Lp, Hkv, D), (B, Lp, Hkv, D)]]
    for splits in (None, 3):
        outs = []
        for _ in range(2):
            o = torch.empty((B, P, Hq, D), dtype=torch.float32, device="cuda")
            api.tree_attention(flat, t[0], t[1], t[2], o, k_pre=t[3], v_pre=t[4], splits=splits)
            outs.append(o.cpu())
        assert torch.equal(outs[0], outs[1]), f"splits={splits}"

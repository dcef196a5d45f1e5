"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Exact on token ids, tree structure, selections, flat layout, masks, retrieve
paths, argmaxes, accept lengths/paths, next tokens and successor-matrix rows;
rtol 1e-5 on fp32 path values and log confidences.  Small cases span several
vocab chunks and a ragged tail; full-size cases run the five workloads in the
launch configuration the bench times (the B=64 workload is compared on sampled
rows, every row checked for the method's invariants).
"""
import dataclasses
import json
import os
import sys

import numpy as np
import pytest
import torch

from gen import configs, synth
from oracle import ddt_oracle as O
from tests import harness as H

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    from dynamic_draft_tree_row_amd import _lib
    _lib.load()      # raises if the library was not built: no fallback


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# row reduction alone
# ---------------------------------------------------------------------------

def _rows_with_ties(V, dtype, seed):
    g = np.random.default_rng(seed)
    rows = [(g.standard_normal(V) * g.uniform(0.3, 3)).astype(np.float32) for _ in range(3)]
    rows.append(np.round(g.standard_normal(V) * 2).astype(np.float32))      # heavy ties
    rows.append(np.full(V, 1.5, np.float32))                                 # all equal
    r = (g.standard_normal(V)).astype(np.float32)
    r[g.integers(0, V, size=min(V, 5))] = 9.0                                # repeated max
    rows.append(r)
    return np.stack([synth.cast_row(x, dtype) for x in rows])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 7, 100, 4095, 4096, 8191, 8192, 8193, 33001, 128256])
def test_row_topk_parity(dtype, V):
    from dynamic_draft_tree_row_amd import api
    raw = _rows_with_ties(V, dtype, V)
    n = raw.shape[0]
    pad = 3                                   # row stride V + 3: unaligned rows too
    host = np.zeros((2, 3, V + pad), raw.dtype)
    host.reshape(6, V + pad)[:, :V] = raw
    x = H.to_dev(host, dtype)[:, :, :V]
    for K in sorted({1, min(8, V), min(10, V), min(32, V)}):
        say(f"row_topk dtype={dtype} V={V} K={K}")
        ws = torch.empty(api.workspace_bytes(6, V, x.dtype, K), dtype=torch.uint8, device="cuda")
        ids = torch.empty((6, K), dtype=torch.int32, device="cuda")
        lc = torch.empty((6, K), dtype=torch.float32, device="cuda")
        mx = torch.empty(6, dtype=torch.float32, device="cuda")
        sp = torch.empty(6, dtype=torch.float32, device="cuda")
        api.row_topk(x, K, ws, ids, lc, mx, sp)
        torch.cuda.synchronize()
        for i in range(n):
            l = O.decode(raw[i], dtype)
            m, _, s = O.row_stats(l)
            want = O.topk_ids(l, K)
            assert ids[i].cpu().tolist() == want.tolist(), f"row {i}"
            np.testing.assert_allclose(lc[i].cpu().numpy(), O.log_conf(l, want, m, s),
                                       rtol=1e-5, atol=1e-30)
            assert float(mx[i]) == np.float32(m)
            np.testing.assert_allclose(float(sp[i]), s, rtol=1e-5, atol=1e-30)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [8193, 33001])
def test_row_topk_parity_wide_launch(dtype, V):
    # 260 rows: launches of 256 rows or more reduce chunks of twice the length
    from dynamic_draft_tree_row_amd import api
    n = 260
    base = _rows_with_ties(V, dtype, V + 1)
    g = np.random.default_rng(V)
    extra = np.stack([synth.cast_row((g.standard_normal(V) * g.uniform(0.3, 3)).astype(np.float32), dtype)
                      for _ in range(n - base.shape[0])])
    raw = np.concatenate([base, extra])
    pad = 5
    host = np.zeros((1, n, V + pad), raw.dtype)
    host[0, :, :V] = raw
    x = H.to_dev(host, dtype)[:, :, :V]
    for K in (1, 10, 32):
        say(f"row_topk wide dtype={dtype} V={V} K={K}")
        ws = torch.empty(api.workspace_bytes(n, V, x.dtype, K), dtype=torch.uint8, device="cuda")
        ids = torch.empty((n, K), dtype=torch.int32, device="cuda")
        lc = torch.empty((n, K), dtype=torch.float32, device="cuda")
        mx = torch.empty(n, dtype=torch.float32, device="cuda")
        sp = torch.empty(n, dtype=torch.float32, device="cuda")
        api.row_topk(x, K, ws, ids, lc, mx, sp)
        torch.cuda.synchronize()
        ids_h, lc_h, mx_h, sp_h = ids.cpu().numpy(), lc.cpu().numpy(), mx.cpu().numpy(), sp.cpu().numpy()
        for i in range(n):
            l = O.decode(raw[i], dtype)
            m, _, s_ = O.row_stats(l)
            want = O.topk_ids(l, K)
            assert ids_h[i].tolist() == want.tolist(), f"row {i} K={K}"
            np.testing.assert_allclose(lc_h[i], O.log_conf(l, want, m, s_), rtol=1e-5, atol=1e-30)
            assert mx_h[i] == np.float32(m)
            np.testing.assert_allclose(sp_h[i], s_, rtol=1e-5, atol=1e-30)


def _rows_special(V, dtype, seed):
    """Rows with values the packed bf16 reading of the reduction cannot order:
    masked (-inf) entries, whole masked chunks, the bf16 value -2^121 that the
    kernels use as padding (as data, and filling the ragged last chunk), and
    a value of magnitude 2^125 (read as fp16 NaN)."""
    g = np.random.default_rng(seed)
    rows = []
    r = (g.standard_normal(V) * 2).astype(np.float32)
    r[g.random(V) < 0.3] = -np.inf                                          # masked entries
    r[g.integers(0, V, size=40)] = 5.0                                       # >= 32 finite survivors
    rows.append(r)
    r = (g.standard_normal(V) * 1.5).astype(np.float32)
    r[: min(V - 40, 20000)] = -np.inf                                        # whole masked chunks
    rows.append(r)
    r = g.standard_normal(V).astype(np.float32)
    r[g.integers(0, V, size=min(V, 50))] = -(2.0 ** 121)                     # the padding value as data
    rows.append(r)
    r = g.standard_normal(V).astype(np.float32)
    r[V - min(V, 20000):] = -(2.0 ** 121)                                    # ...filling the last chunks
    r[: min(V, 40)] = 3.0
    rows.append(r)
    rows.append(np.full(V, -(2.0 ** 121), np.float32))                       # ...everywhere
    r = g.standard_normal(V).astype(np.float32)
    r[g.integers(0, V, size=3)] = 2.0 ** 125                                 # fp16 reading: NaN
    r[g.integers(0, V, size=5)] = -(2.0 ** 124)
    rows.append(r)
    return np.stack([synth.cast_row(x, dtype) for x in rows])


def _check_rows(raw, dtype, n, K, ids, lc, mx, sp):
    ids_h, lc_h, mx_h, sp_h = ids.cpu().numpy(), lc.cpu().numpy(), mx.cpu().numpy(), sp.cpu().numpy()
    for i in range(n):
        l = O.decode(raw[i], dtype)
        m, _, s_ = O.row_stats(l)
        want = O.topk_ids(l, K)
        assert ids_h[i].tolist() == want.tolist(), f"row {i} K={K}"
        np.testing.assert_allclose(lc_h[i], O.log_conf(l, want, m, s_), rtol=1e-5, atol=1e-30)
        assert mx_h[i] == np.float32(m)
        np.testing.assert_allclose(sp_h[i], s_, rtol=1e-5, atol=1e-30)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [8193, 33001, 128256])
@pytest.mark.parametrize("wide", [False, True])
def test_row_topk_parity_special_values(dtype, V, wide):
    # wide: 260 rows, so that the chunks are twice as long
    from dynamic_draft_tree_row_amd import api
    raw = _rows_special(V, dtype, V + 7)
    if wide:
        g = np.random.default_rng(V)
        extra = np.stack([synth.cast_row((g.standard_normal(V) * g.uniform(0.3, 3)).astype(np.float32), dtype)
                          for _ in range(260 - raw.shape[0])])
        raw = np.concatenate([raw, extra])
    n = raw.shape[0]
    host = np.zeros((1, n, V + 3), raw.dtype)
    host[0, :, :V] = raw
    x = H.to_dev(host, dtype)[:, :, :V]
    for K in (1, 10, 32):
        say(f"row_topk special dtype={dtype} V={V} wide={wide} K={K}")
        ws = torch.empty(api.workspace_bytes(n, V, x.dtype, K), dtype=torch.uint8, device="cuda")
        ids = torch.empty((n, K), dtype=torch.int32, device="cuda")
        lc = torch.empty((n, K), dtype=torch.float32, device="cuda")
        mx = torch.empty(n, dtype=torch.float32, device="cuda")
        sp = torch.empty(n, dtype=torch.float32, device="cuda")
        api.row_topk(x, K, ws, ids, lc, mx, sp)
        torch.cuda.synchronize()
        _check_rows(raw, dtype, min(n, 12), K, ids, lc, mx, sp)


# ---------------------------------------------------------------------------
# whole rounds, small vocabularies
# ---------------------------------------------------------------------------

def _case(w, seed, rnd, rows=None, M=None, tau=None):
    cast = H.cast_params(w) if w.cast else None
    graft = H.graft_params(w, tau) if w.graft else None
    M0 = M
    return H.oracle_case(w, seed, rnd, rows=rows, cast=cast, graft=graft, M=M, M0=M0)


SMALL = {
    "eagle2_f32": configs.shrink(configs.C1, V=5000, B=2),
    "cast": configs.shrink(configs.C2, V=17000),
    "cast_b12": configs.shrink(configs.C2, V=9000, B=12),       # more workgroups sharing the layer ticket
    "t1": configs.shrink(configs.C3, V=9001, B=4),            # odd V: unaligned bf16 rows
    "mixed_prefix": configs.shrink(configs.C5, V=4100, B=6),
    # 20 requests x 16 frontier rows: layers of 256 rows or more take the
    # plain reduction and the layer kernel's finishing form
    "mixed_wide": configs.shrink(configs.C5, V=4100, B=20),
    # T > 0 draft children verified with q = the draft row's softmax
    "t1_draft_q": configs.shrink(configs.C3, V=9001, B=4, proposal="draft"),
    "mixed_draft_q": configs.shrink(configs.C5, V=4100, B=6, proposal="draft"),
    # sampling temperatures other than 1: exact normalisers before the first test
    "tmix": configs.shrink(configs.C3, V=7001, B=8, verify="tmix"),
    "tmix_draft_q": configs.shrink(configs.C3, V=7001, B=8, verify="tmix", proposal="draft"),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_small(name, seed):
    w = SMALL[name]
    for rnd in range(2):
        case = _case(w, seed, rnd)
        say(f"round {name} seed={seed} round={rnd} B={w.B} V={w.V} tries={case.tries}")
        H.compare(case, H.gpu_round(case))


def test_cast_seeded_cost_table():
    cs = configs.CastSpec(table="seeded", C1=0.5, C2=0.05, C3=0.3)
    w = configs.Workload(**{**SMALL["cast"].__dict__, "cast": cs, "name": "cast_seeded"})
    cast = H.cast_params(w, seed=9)
    for seed in (3, 4):
        case = H.oracle_case(w, seed, 0, cast=cast)
        say(f"cast seeded table seed={seed}")
        H.compare(case, H.gpu_round(case))


@pytest.mark.parametrize("table_B,C1,C2,C3", [(64, 10.0, 0.5, 0.5), (16, 2.0, 1.0, 0.3)])
def test_cast_roofline_cost_table(table_B, C1, C2, C3):
    # MI355X-shaped costs: flat while a forward is HBM-bound (equal neighbouring
    # costs, the zero-cost-step branch of the width and verify scans), rising
    # once it is MFMA-bound
    cs = configs.CastSpec(table="roofline", table_B=table_B, C1=C1, C2=C2, C3=C3)
    w = configs.Workload(**{**SMALL["cast"].__dict__, "cast": cs, "name": f"cast_roofline_{table_B}"})
    cast = H.cast_params(w)
    for seed in (3, 4):
        case = H.oracle_case(w, seed, 0, cast=cast)
        say(f"cast roofline table B={table_B} seed={seed} m={case.out['m_rows'].tolist()}")
        H.compare(case, H.gpu_round(case))


@pytest.mark.parametrize("C2", [0.001, 0.002])
def test_cast_gain_fifo_full_length(C2):
    # R = 8, the longest gain FIFO the state holds, and 11 layers: from layer 9
    # on a push meets a full FIFO and drops the oldest ratio (CAST notes, key
    # design 3).  At these thresholds the depth gate stops the tree at layer 9
    # or 10, so the decisions read the full-length FIFO.
    cs = configs.CastSpec(C1=0.05, C2=C2, C3=0.02, R=8)
    base = configs.shrink(configs.C2, V=3000, B=3)
    w = configs.Workload(**{**base.__dict__, "D": 11, "m": 120, "cast": cs, "name": "cast_fifo8"})
    cast = H.cast_params(w)
    for seed in (1, 2, 3):
        case = H.oracle_case(w, seed, 0, cast=cast)
        say(f"cast FIFO R=8 C2={C2} seed={seed} depth={case.out['draft'].depth_built}")
        H.compare(case, H.gpu_round(case))


def test_graft_small_multi_round():
    w = configs.shrink(configs.C4, V=6000, B=5)
    tau = H.calibrate_tau(w, 77, 4)
    M = synth.succ_matrix0(w, 77)
    M0 = M.copy()
    for rnd in range(3):
        case = H.oracle_case(w, 77, rnd, cast=None, graft=H.graft_params(w, tau), M=M, M0=M0)
        say(f"graft round {rnd} k_draft={case.out['draft'].k_draft}")
        H.compare(case, H.gpu_round(case))
        M = case.M_after


def test_graft_wide_flat_rows():
    # 18 requests x 61 flat rows: launches over the flat verify rows of 512
    # rows or more reduce wide chunks, in the verify and in the successor
    # refresh alike
    w = configs.shrink(configs.C4, V=4100, B=18)
    assert w.B * (w.m_max + 1) >= 512
    tau = H.calibrate_tau(w, 79, 4)
    M = synth.succ_matrix0(w, 79)
    M0 = M.copy()
    for rnd in range(2):
        case = H.oracle_case(w, 79, rnd, cast=None, graft=H.graft_params(w, tau), M=M, M0=M0)
        say(f"graft wide flat round {rnd} k_draft={case.out['draft'].k_draft}")
        H.compare(case, H.gpu_round(case))
        M = case.M_after


@pytest.mark.parametrize("proposal", ["draft", "point"])
def test_graft_stochastic_verify_point_mass(proposal):
    # Graft with T > 0: retrieval nodes are verified with point-mass
    # proposals (accepted with probability p(x), rejected tokens leave the
    # residual), so a T = 1 request's walk can run through grafted chains;
    # draft children before them take q-proposals or point-mass proposals
    base = configs.shrink(configs.C4, V=6000, B=6)
    w = configs.Workload(**{**base.__dict__, "verify": "t1", "name": base.name + "_t1",
                            "proposal": proposal})
    tau = H.calibrate_tau(w, 83, 4)
    M = synth.succ_matrix0(w, 83)
    M0 = M.copy()
    for rnd in range(3):
        case = H.oracle_case(w, 83, rnd, cast=None, graft=H.graft_params(w, tau), M=M, M0=M0)
        say(f"graft T>0 round {rnd} k_draft={case.out['draft'].k_draft} "
            f"accept={case.out['accept_len'].tolist()}")
        H.compare(case, H.gpu_round(case))
        M = case.M_after


@pytest.mark.parametrize("verify", ["greedy", "t1"])
@pytest.mark.parametrize("mode", ["root_only", "tail_only"])
def test_graft_variants(mode, verify):
    # the two grafts prune-then-graft is compared with (Graft review, Fig. 2):
    # a fixed draft budget with no checkpoints, the template under the root or
    # under the tail of the selected draft tree
    base = configs.shrink(configs.C4, V=6000, B=5)
    gs = dataclasses.replace(base.graft, mode=mode)
    w = configs.Workload(**{**base.__dict__, "graft": gs, "verify": verify,
                            "name": f"{base.name}_{mode}_{verify}"})
    M = synth.succ_matrix0(w, 61)
    M0 = M.copy()
    for rnd in range(2):
        case = H.oracle_case(w, 61, rnd, graft=H.graft_params(w, None), M=M, M0=M0)
        say(f"graft {mode} {verify} round {rnd} m={case.out['m_rows'].tolist()} "
            f"accept={case.out['accept_len'].tolist()}")
        H.compare(case, H.gpu_round(case))
        M = case.M_after


def test_graft_shared_successor_matrix():
    # one successor matrix for the whole batch (row stride 0): every request
    # reads it in the draft phase, refreshes land in request order
    w = configs.shrink(configs.C4, V=5000, B=4)
    tau = H.calibrate_tau(w, 91, 4)
    M = synth.succ_matrix0(w, 91)[0].copy()
    M0 = M.copy()
    for rnd in range(2):
        case = H.oracle_case(w, 91, rnd, graft=H.graft_params(w, tau), M=M, M0=M0, shared_M=True)
        say(f"graft shared-M round {rnd} k_draft={case.out['draft'].k_draft}")
        H.compare(case, H.gpu_round(case))
        M = case.M_after


def test_determinism_bitwise():
    w = SMALL["mixed_prefix"]
    case = _case(w, 5, 0)
    a = H.gpu_round(case)
    b = H.gpu_round(case)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


@pytest.mark.parametrize("shape", [
    dict(V=16, D=2, K_e=2, K_n=2, m=60),        # fewer nodes than the budget
    dict(V=64, D=1, K_e=1, K_n=5, m=3),         # one layer
    dict(V=300, D=11, K_e=1, K_n=1, m=11),      # deepest chain
    dict(V=9000, D=3, K_e=32, K_n=32, m=255),   # widest frontier, largest budget
])
def test_round_edge_shapes(shape):
    w = configs.Workload("edge", B=3, dtype="bf16", verify="mixed", sigma=0.5, prefix=7, **shape)
    case = _case(w, 11, 0)
    say(f"edge {shape}")
    H.compare(case, H.gpu_round(case))


def _direct_case(w, draft, target, roots, T, U, cast=None):
    """A case from inputs given directly (no generator, no re-keying): the
    oracle's round on exactly these inputs."""
    B = w.B
    out = O.run_round(B=B, V=w.V, dtype=w.dtype, D=w.D, K_e=w.K_e, K_n=w.K_n, m_max=w.m_max,
                      root_tok=roots, draft_raw=draft, target_raw_fn=lambda dr, fl: target,
                      temperature=T, U=U, prefix=w.prefix, cast=cast, proposal=w.proposal)
    return H.Case(w, 0, 0, list(range(B)), np.zeros(B, np.int64), draft, target, roots, U, T, out,
                  cast)


def test_cast_cost_lookup_hand_example():
    # the hand-worked CAST round of the oracle pins: a 4-row cost grid of step
    # 2 that the widths move through, a zero-cost step, different S_T and S_D
    # slopes, and a 4-token prefix that picks the verify-cost row
    from tests.test_oracle_pins import cast_lookup_example
    shape, draft, cast, expect = cast_lookup_example()
    B, P, V = shape["B"], shape["m_max"] + 1, shape["V"]
    w = configs.Workload("cast_lookup", B=B, V=V, dtype="f32", D=shape["D"], K_e=shape["K_e"],
                         K_n=shape["K_n"], m=shape["m_max"], verify="greedy", sigma=0.0,
                         prefix=shape["prefix"],
                         cast=configs.CastSpec(L=cast["L"], M=cast["M"], R=cast["R"]))
    target = np.random.default_rng(3).standard_normal((B, P, V)).astype(np.float32)
    case = _direct_case(w, draft, target, np.zeros(B, np.int32), np.zeros(B, np.float32),
                        np.zeros((B, P, 2), np.float32), cast)
    assert case.out["draft"].widths == expect["widths"]
    assert case.out["m_rows"].tolist() == expect["m_rows"]
    H.compare(case, H.gpu_round(case))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rerank_exact_ties_take_the_sort_path(dtype):
    # constant draft rows: every token has confidence 1/V, so the nodes of a
    # layer tie exactly (32 + 1024 + 1024 nodes).  With m = 255 the 1024 tied
    # nodes of layer 2 straddle the cut: more candidates than the rank count
    # holds, so the rerank takes its full-sort path.  Ties go by canonical key
    # (shallower first, then the rank path), in the frontier too.
    V, B, D, K, m = 100, 2, 3, 32, 255
    w = configs.Workload("ties", B=B, V=V, dtype=dtype, D=D, K_e=K, K_n=K, m=m, verify="greedy",
                         sigma=0.0)
    row = synth.cast_row(np.full(V, 0.5, np.float32), dtype)
    draft = np.broadcast_to(row, (D, B, K, V)).copy()
    g = np.random.default_rng(4)
    target = np.stack([np.stack([synth.cast_row(g.standard_normal(V).astype(np.float32), dtype)
                                 for _ in range(m + 1)]) for _ in range(B)])
    case = _direct_case(w, draft, target, np.array([3, 5], np.int32), np.zeros(B, np.float32),
                        np.zeros((B, m + 1, 2), np.float32))
    t = case.out["draft"].trees[0]
    assert t.n == 1 + K + 2 * K * K
    say(f"ties dtype={dtype} selected={len(case.out['sels'][0])}")
    H.compare(case, H.gpu_round(case))


@pytest.mark.parametrize("name", ["cast", "mixed_prefix"])
def test_dense_mask_matches_the_bitmask_with_the_prefix(name):
    # the optional dense mask: every prefix column visible, then the ancestor
    # bits of the flat tree (padding rows see the prefix and themselves)
    from dynamic_draft_tree_row_amd import api
    w = SMALL[name]
    case = _case(w, 2, 0)
    run = H.runner_for(w)
    cast = H.dev_cast(case.cast, "cuda", w.prefix) if case.cast else None
    run.draft(H.to_dev(case.draft, w.dtype), torch.from_numpy(case.roots).cuda(), cast=cast)
    P = w.m_max + 1
    dense = torch.full((w.B, P, w.prefix + P), 7, dtype=torch.uint8, device="cuda")
    api.tree_build_mask(run.tree, run.sel, run.m_out, w.prefix, run.flat, dense=dense)
    torch.cuda.synchronize()
    d = dense.cpu().numpy()
    say(f"dense mask {name} prefix={w.prefix} P={P}")
    for b in range(w.B):
        f = case.out["flats"][b]
        bits = np.unpackbits(f.mask.view(np.uint8), axis=1, bitorder="little")[:, :P]
        want = np.concatenate([np.ones((P, w.prefix), np.uint8), bits], 1)
        np.testing.assert_array_equal(d[b], want, err_msg=f"row {b}")


@pytest.mark.parametrize("name", ["cast", "mixed_prefix", "eagle2_f32"])
def test_select_equals_rerank_then_mask(name):
    # ddt_tree_select (one launch) against ddt_tree_rerank + ddt_tree_build_mask
    # on the same drafted trees: every output equal bit for bit
    from dynamic_draft_tree_row_amd import api
    w = SMALL[name]
    case = _case(w, 3, 1)
    run = H.runner_for(w)
    cast = H.dev_cast(case.cast, "cuda", w.prefix) if case.cast else None
    run.draft(H.to_dev(case.draft, w.dtype), torch.from_numpy(case.roots).cuda(), cast=cast)
    P = w.m_max + 1
    dense = torch.full((w.B, P, w.prefix + P), 7, dtype=torch.uint8, device="cuda")
    api.tree_select(run.tree, w.m_max, run.sel, run.m_out, w.prefix, run.flat, cast=cast, dense=dense)
    sel2 = torch.full_like(run.sel, -5)
    m2 = torch.full_like(run.m_out, -5)
    flat2 = api.DeviceFlat(w.B, w.m_max, run.shape.Dp, "cuda")
    dense2 = torch.full_like(dense, 9)
    api.tree_rerank(run.tree, w.m_max, sel2, m2, cast=cast)
    api.tree_build_mask(run.tree, sel2, m2, w.prefix, flat2, dense=dense2)
    torch.cuda.synchronize()
    say(f"select vs rerank+mask {name}: m={m2.tolist()}")
    assert torch.equal(run.sel, sel2) and torch.equal(run.m_out, m2)
    assert torch.equal(dense, dense2)
    for k in ("node", "token", "parent", "pos", "mask", "retrieve", "n_leaves", "m"):
        assert torch.equal(getattr(run.flat, k), getattr(flat2, k)), k


def test_graft_successor_matrix_resume():
    # M is the only state a round leaves for the next: a snapshot taken after
    # two rounds and restored replays the next two rounds bit for bit, and
    # both replays equal the oracle's rounds
    w = configs.shrink(configs.C4, V=6000, B=5)
    tau = H.calibrate_tau(w, 79, 4)
    M = synth.succ_matrix0(w, 79)
    M0 = M.copy()
    cases = []
    for rnd in range(4):
        case = H.oracle_case(w, 79, rnd, graft=H.graft_params(w, tau), M=M, M0=M0)
        cases.append(case)
        M = case.M_after
    run = H.runner_for(w)
    gate = H.dev_gate(cases[0].graft)
    Md = torch.from_numpy(np.ascontiguousarray(M0)).cuda()

    def play(case):
        arena = H.to_dev(case.draft, w.dtype)
        run.draft(arena, torch.from_numpy(case.roots).cuda(), gate=gate, M=Md)
        run.verify(H.to_dev(case.target, w.dtype), arena, torch.from_numpy(case.T).cuda(),
                   torch.from_numpy(case.U).cuda(), M=Md)
        torch.cuda.synchronize()
        g = lambda x: x.cpu().numpy().copy()
        return dict(accept_len=g(run.accept_len), accept_path=g(run.accept_path),
                    next_token=g(run.next_token), flat_token=g(run.flat.token), M=g(Md))

    for c in cases[:2]:
        play(c)
    snap = Md.clone()
    first = [play(c) for c in cases[2:]]
    Md.copy_(snap)
    second = [play(c) for c in cases[2:]]
    for r, (a, b_, c) in enumerate(zip(first, second, cases[2:])):
        say(f"graft resume round {r + 2} accept={a['accept_len'].tolist()}")
        for k in a:
            np.testing.assert_array_equal(a[k], b_[k], err_msg=f"replay differs: {k}")
        np.testing.assert_array_equal(a["accept_len"], c.out["accept_len"])
        np.testing.assert_array_equal(a["next_token"], c.out["next_token"])
        np.testing.assert_array_equal(a["M"], c.M_after)


# ---------------------------------------------------------------------------
# full-size workloads, the bench's launch configuration
# ---------------------------------------------------------------------------

def _tau_golden():
    return json.load(open(os.path.join(GOLDEN, "graft_tau.json")))["tau"]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("cfg", [configs.C1, configs.C2, configs.C3, configs.C4],
                         ids=lambda c: c.name)
def test_round_full(cfg):
    # three seeds x two consecutive rounds (one seed for the B = 1 workload);
    # Graft carries its successor matrix from round to round
    i = configs.ORDER.index(cfg)
    seeds = [1000 + i] if cfg is configs.C1 else [1000 + i, 2000 + i, 3000 + i]
    for seed in seeds:
        M = synth.succ_matrix0(cfg, seed) if cfg.graft else None
        M0 = None if M is None else M.copy()
        for rnd in range(2):
            graft = H.graft_params(cfg, _tau_golden()) if cfg.graft else None
            cast = H.cast_params(cfg) if cfg.cast else None
            case = H.oracle_case(cfg, seed, rnd, cast=cast, graft=graft, M=M, M0=M0)
            say(f"full {cfg.name} seed={seed} round={rnd} tries={case.tries} "
                f"accept={case.out['accept_len'].tolist()}")
            H.compare(case, H.gpu_round(case))
            if cfg.graft:
                M = case.M_after


@pytest.mark.timeout(1200)
def test_round_full_b64_sampled_rows():
    # 16 of the 64 requests compared with the oracle (greedy and T = 1 rows),
    # every request checked for the method's invariants
    w = configs.C5
    rows = list(range(0, 64, 4))
    case = _case(w, 1005, 0, rows=rows)
    say(f"full {w.name} sampled rows {rows} T={case.T.tolist()} tries={case.tries}")
    assert (case.T == 0).any() and (case.T > 0).any()
    r = H.gpu_round_full(case)
    sub = {k: (v[rows] if k != "widths" else v) for k, v in r.items()}
    H.compare(case, sub)
    H.check_invariants(r, w)
